"""Large-size cases (GPU): long sequences, long caches, wide row strides,
many sequences, a distance-bias table over 81919 distances and FP8
local+global at 32768 positions, each compared with the fp64 oracles on
sampled rows.

They exercise the index arithmetic at sizes beyond the workloads: 64-bit
element offsets of long sequences, 32-bit buffer-descriptor extents of
strided tiles near their limit, large grids.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.test_parity import TOL

attn = pytest.importorskip("transformer_attention_attn_amd")


def bf16(bits, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@pytest.mark.gpu
def test_long_sequence_causal_gqa(device):
    """S = 65536 (4.3e9 visible pairs per head group), sampled rows."""
    import torch

    B, Hq, Hkv, S, D = 1, 8, 2, 65536, 128
    print(f"large: causal GQA S={S}", flush=True)
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, "bf16", seed=70)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    rows = [0, 1, 4095, 4096, 32767, 32768, 65534, 65535]
    got = o[:, :, rows].float().cpu().numpy()
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], "causal", rows=rows)
    err = float(np.max(np.abs(got - ref)))
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
def test_long_window(device):
    """S = 131072 with a 2048-key window: every item sees 17 tiles."""
    import torch

    B, Hq, Hkv, S, D, w = 1, 4, 1, 131072, 64, 2048
    print(f"large: window S={S} w={w}", flush=True)
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, "bf16", seed=71)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd(q, k, v, mask="causal_window", window=w)
    torch.cuda.synchronize()
    rows = [0, 2047, 2048, 65536, 131071]
    got = o[:, :, rows].float().cpu().numpy()
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], "causal_window", w, rows=rows)
    assert float(np.max(np.abs(got - ref))) <= TOL["bf16"]


@pytest.mark.gpu
def test_long_decode_cache(device):
    """A 262144-position cache (multi-query), full and ragged lengths."""
    import torch

    B, Hq, Hkv, Sq, Smax, D = 2, 16, 1, 1, 262144, 128
    print(f"large: decode Smax={Smax}", flush=True)
    inp = workloads.make_decode_inputs(B, Hq, Hkv, Sq, Smax, D, seed=72)
    q, k, v = (bf16(inp[n + "_bits"], device) for n in ("q", "k", "v"))
    for lens in (None, [262144, 100003]):
        cl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=device)
        o = attn.decode(q, k, v, cache_len=cl)
        torch.cuda.synchronize()
        ref = oracle.decode_attention(inp["q"], inp["k"], inp["v"], "causal", cache_len=lens)
        assert float(np.max(np.abs(o.float().cpu().numpy() - ref))) <= TOL["bf16"], lens


@pytest.mark.gpu
def test_wide_row_strides(device):
    """attn_fwd_ex with K and V rows 2^22 elements apart (8 MiB), so a 128-key
    tile spans about 1 GiB of address space (the per-tile descriptor extent
    stays below 2^32 bytes); only the used rows are written."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = 1, 4, 1, 64, 130, 128
    stride = 1 << 22
    print(f"large: row stride {stride} elements", flush=True)
    inp = workloads.make_decode_inputs(B, Hq, Hkv, Sq, Skv, D, seed=73)
    q = bf16(inp["q_bits"], device)
    views = []
    for n in ("k", "v"):
        buf = torch.empty(Skv * stride, dtype=torch.bfloat16, device=device)
        view = buf.as_strided((B, Hkv, Skv, D), (Skv * stride, Skv * stride, stride, 1))
        view.copy_(bf16(inp[n + "_bits"], device))
        views.append((buf, view))
    o = attn.fwd_ex(q, views[0][1], views[1][1], mask="causal")
    torch.cuda.synchronize()
    ref = oracle.cross_attention(inp["q"], inp["k"], inp["v"], "causal")
    assert float(np.max(np.abs(o.float().cpu().numpy() - ref))) <= TOL["bf16"]


@pytest.mark.gpu
def test_many_sequences(device):
    """B = 512 short sequences of 32 heads (16384 work items)."""
    import torch

    B, Hq, Hkv, S, D = 512, 32, 8, 65, 64
    print(f"large: B={B}", flush=True)
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, "bf16", seed=74)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    o = attn.fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    sel = [0, 1, 255, 511]
    got = o[sel].float().cpu().numpy()
    ref = oracle.attention(inp["q"][sel], inp["k"][sel], inp["v"][sel], "causal")
    assert float(np.max(np.abs(got - ref))) <= TOL["bf16"]


@pytest.mark.gpu
def test_long_distance_bias_chunk(device):
    """A bucketed distance-bias table over Sq + Skv - 1 = 81919 distances (a
    4096-query chunk at the end of 77824 keys, causal), sampled rows of every
    head, sequence-major tensors."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = 1, 8, 2, 4096, 77824, 128
    print(f"large: distance bias Sq={Sq} Skv={Skv}", flush=True)
    inp = workloads.make_decode_inputs(B, Hq, Hkv, Sq, Skv, D, seed=75)
    q, k, v = (bf16(inp[n + "_bits"], device).transpose(1, 2).contiguous().transpose(1, 2)
               for n in ("q", "k", "v"))
    table = workloads.make_distance_bias(Hq, Sq, Skv, seed=76)
    o = attn.fwd_ex(q, k, v, mask="causal", dist_bias=torch.from_numpy(table).to(device))
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 2048, 4094, 4095]
    got = o[:, :, rows].float().cpu().numpy()
    ref = oracle.cross_attention(inp["q"], inp["k"], inp["v"], "causal", rows=rows,
                                 dist_bias=table)
    err = float(np.max(np.abs(got - ref)))
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
def test_long_fp8_local_global(device):
    """FP8 local + global at S = 32768 with 64 globals (the global rows' walks
    span 32768 keys), sampled rows including every kind of row."""
    import torch

    B, Hq, Hkv, S, D = 1, 4, 4, 32768, 64
    g = tuple(int(x) for x in np.linspace(0, S - 1, 64).astype(np.int64))
    print(f"large: FP8 local+global S={S} globals={len(g)}", flush=True)
    inp = workloads.make_inputs(B, Hq, Hkv, S, D, "fp8", seed=77)
    q, k, v = workloads.to_torch(inp, "fp8", device)
    o = attn.fwd(q, k, v, mask="local_global", window=256, global_idx=list(g))
    torch.cuda.synchronize()
    rows = sorted({0, 1, 255, 256, 257, 16383, 16384, S - 1} | set(g[1:4]))
    got = o[:, :, rows].float().cpu().numpy().astype(np.float64)
    codes = (inp["q_codes"], inp["k_codes"], inp["v_codes"])
    ref = oracle.fp8_attention(*codes, "local_global", 256, rows=rows, global_idx=g)
    tol = oracle.fp8_tolerance(*codes, "local_global", 256, rows=rows, rounded_denominator=True,
                               global_idx=g)
    err = np.abs(got - ref)
    print(f"max abs err {err.max():.3e}, worst error / tolerance {(err / tol).max():.3f}", flush=True)
    assert np.all(err <= tol), float((err - tol).max())
