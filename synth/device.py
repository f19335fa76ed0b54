"""Copy drawn inputs to torch tensors (bit-exact; bf16 patterns are viewed, not converted)."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from .gen import Inputs


def tensor(a: Optional[np.ndarray], dtype: str, device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    if a.dtype == np.uint16 and dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_torch(inp: Inputs, device="cuda") -> Dict[str, Optional[torch.Tensor]]:
    dt = inp.dtype
    out = {name: tensor(getattr(inp, name), dt, device)
           for name in ("x", "W1", "b1", "W2", "b2", "sW1", "sb1", "sW2", "sb2")}
    for name in ("W_g", "b_g", "b_sel", "noise", "gW1", "gb1", "gW2", "gb2"):
        a = getattr(inp, name)
        out[name] = None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return out
