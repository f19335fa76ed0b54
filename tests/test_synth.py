"""The seeded input draws: bit patterns, determinism and the stated recipes. CPU only."""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_rne_matches_torch():
    """fp32 -> bf16 round-to-nearest-even against torch's own conversion, including ties."""
    rng = np.random.default_rng(0)
    a = rng.normal(size=100000).astype(np.float32) * 10
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)  # exact halfway cases
    a = np.concatenate([a, ties, -ties, np.array([0.0, -0.0, 1.0, 3.0e38], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(a), ref)
    back = synth.bf16_bits_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_draw_is_deterministic_and_thread_independent():
    w = synth.FINE_SHARED.with_(T=64, d=32, F=16)
    a = synth.draw(w, threads=1)
    b = synth.draw(w, threads=8)
    for name in ("x", "W_g", "b_sel", "W1", "b1", "W2", "b2", "sW1", "sb1", "sW2", "sb2"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.x.dtype == np.uint16 and a.W_g.dtype == np.float32


def test_variance_convention():
    """N(0, v) means variance v: router N(0, 0.02) has std sqrt(0.02)."""
    inp = synth.draw(synth.DEFAULT.with_(F=8))
    assert inp.W_g.std() == pytest.approx(np.sqrt(0.02), rel=0.02)
    w1 = synth.widen(inp.W1, "bf16")
    assert w1.std() == pytest.approx(1 / np.sqrt(512), rel=0.02)


def test_zipf_router_bias_gives_zipf_popularity():
    """Switch top-1 workload: top-1 popularity follows Zipf(1.1) over the 64 experts
    (checked on the batch with the oracle's own router, after calibration on a Gaussian model)."""
    w = synth.SWITCH_ZIPF.with_(F=8)
    inp = synth.draw(w)
    h = oracle.router_logits(synth.widen(inp.x, "bf16"), inp.W_g, inp.b_g)
    counts = np.bincount(oracle.topk(h, 1)[:, 0], minlength=64)
    p = np.arange(1, 65) ** -1.1
    p /= p.sum()
    assert counts[0] / w.T == pytest.approx(p[0], rel=0.1)
    assert counts[:8].sum() / w.T == pytest.approx(p[:8].sum(), rel=0.05)
    assert (counts > 0).all()


def test_unit_row_router_gives_unit_logit_std():
    inp = synth.draw(synth.LARGE_CREDIT.with_(T=2048, F=8, E=128))
    h = oracle.router_logits(synth.widen(inp.x, "bf16"), inp.W_g, None)
    assert h.std() == pytest.approx(1.0, rel=0.03)


def test_token_losses():
    a = synth.token_losses(synth.DEFAULT)
    b = synth.token_losses(synth.DEFAULT)
    assert a.dtype == np.float32 and a.shape == (synth.DEFAULT.T,)
    assert (a == b).all() and (a >= 1.0).all()
    assert abs(float(a.mean()) - 2.0) < 0.1
