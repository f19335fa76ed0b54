"""MI355X-native sparse mixture-of-experts forward layer.

HIP kernels for gfx950 behind a C ABI (``include/moe.h``, built into
``lib/libmoe_mi355x.so``); ``api`` is the same-named Python binding and
``layer.MoELayer`` composes one forward pass.
"""
from . import api
from .api import MoEError
from .layer import MoELayer, MoEOutputs

__all__ = ["api", "MoEError", "MoELayer", "MoEOutputs"]
