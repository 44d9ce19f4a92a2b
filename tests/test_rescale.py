"""Running-maximum paths of the kernels (GPU), against the fp64 oracles.

The online softmax takes a tile's weights against the running reference
maximum and only recomputes them after a rescale when they grow too large
("Transformer 演进与变体", section Flash Attention: the running maximum and
denominator are updated per key block and the partial output rescaled).
Random inputs settle the maximum on the first tile, so these inputs plant a
trend along the key index: scores rising by many log2 units per tile (a
rescale on almost every tile), falling (tiny weights after the first tile)
and isolated spikes far above the rest (weights that would overflow against
the old reference).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.test_parity import TOL

attn = pytest.importorskip("transformer_attention_attn_amd")

PATTERNS = ("rising", "falling", "spikes")


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,w", [("causal", 0), ("full", 0), ("causal_window", 300)])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_trend_bf16(device, pattern, mask, w, D):
    import torch

    B, Hq, Hkv, S = 1, 8, 2, 700
    print(f"rescale: bf16 {pattern} {mask} w={w} D={D}", flush=True)
    inp = workloads.make_trend_inputs(B, Hq, Hkv, S, D, "bf16", seed=90, pattern=pattern)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd(q, k, v, mask=mask, window=w)
    torch.cuda.synchronize()
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], mask, w)
    got = o.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("pattern", PATTERNS)
def test_trend_fwd_ex(device, pattern):
    """The general path (Sq != Skv, queries aligned to the end of the keys)."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = 1, 4, 1, 300, 900, 128
    inp = workloads.make_trend_inputs(B, Hq, Hkv, Skv, D, "bf16", seed=91, pattern=pattern)
    q = torch.from_numpy(inp["q_bits"][:, :, Skv - Sq:].copy().view(np.int16)).view(torch.bfloat16)
    q = q.to(device)
    _, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd_ex(q, k, v, mask="causal")
    torch.cuda.synchronize()
    ref = oracle.cross_attention(inp["q"][:, :, Skv - Sq:], inp["k"], inp["v"], "causal")
    err = float(np.max(np.abs(o.float().cpu().numpy() - ref)))
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("mask", ["causal", "full"])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_trend_fp8(device, pattern, mask):
    import torch

    B, Hq, Hkv, S, D = 1, 8, 2, 700, 128
    inp = workloads.make_trend_inputs(B, Hq, Hkv, S, D, "fp8", seed=92, pattern=pattern)
    q, k, v = workloads.to_torch(inp, "fp8", device)
    o = attn.fwd(q, k, v, mask=mask)
    torch.cuda.synchronize()
    codes = (inp["q_codes"], inp["k_codes"], inp["v_codes"])
    ref = oracle.fp8_attention(*codes, mask)
    tol = oracle.fp8_tolerance(*codes, mask, rounded_denominator=True)
    err = np.abs(o.float().cpu().numpy() - ref)
    assert np.all(err <= tol), float(np.max(err - tol))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_trend_inputs_plant_the_trend(dtype):
    """Host check of the generator: seeded, quantised like make_inputs, and the
    oracle's row maximum really moves (rising: to the last visible key;
    falling: stays at the first; spikes: to the latest spike)."""
    B, Hq, Hkv, S, D = 1, 2, 1, 300, 128
    a = workloads.make_trend_inputs(B, Hq, Hkv, S, D, dtype, seed=5, pattern="rising")
    b = workloads.make_trend_inputs(B, Hq, Hkv, S, D, dtype, seed=5, pattern="rising")
    for n in ("q", "k", "v"):
        assert a[n].shape == ((B, Hq, S, D) if n == "q" else (B, Hkv, S, D))
        assert np.array_equal(a[n], b[n])
    scale = 1.0 / np.sqrt(D)
    for pattern, where in (("rising", "last"), ("falling", "first"), ("spikes", "spike")):
        x = workloads.make_trend_inputs(B, Hq, Hkv, S, D, dtype, seed=5, pattern=pattern)
        s = (x["q"][0, 0].astype(np.float64) @ x["k"][0, 0].astype(np.float64).T) * scale
        i = S - 1
        arg = int(np.argmax(s[i, : i + 1]))
        if where == "last":
            assert arg > S - 20
        elif where == "first":
            assert arg < 20
        else:
            assert arg == int(np.argmax(x["k"][0, 0, :, 0]))
