"""Decode attention (attn_decode) against the fp64 decode oracle.

GPU cases compare every element of the output with oracle.decode_attention on
the same seeded inputs (bf16 tolerance 2e-2, as for the full-sequence path);
cache positions beyond a sequence's length, and under a sliding window those
before the first position any new query sees, hold NaN, so any read of them
into the result shows.  Host-only cases check the validation of the boundary.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.test_parity import TOL

attn = pytest.importorskip("transformer_attention_attn_amd")


def run_decode(device, B, Hq, Hkv, Sq, Smax, D, mask, lens=None, seed=0, scale=None,
               rows=None, window=0, ws_guard=False):
    import torch

    print(f"decode case B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Smax={Smax} D={D} {mask} w={window} "
          f"lens={None if lens is None else list(lens)[:8]} seed={seed}", flush=True)
    inp = workloads.make_decode_inputs(B, Hq, Hkv, Sq, Smax, D, seed)
    kb, vb = inp["k_bits"].copy(), inp["v_bits"].copy()
    for b, L in enumerate([Smax] * B if lens is None else lens):
        kb[b, :, L:] = 0x7FC0  # positions past the length hold NaN
        vb[b, :, L:] = 0x7FC0
        if window:  # and those before every new query's window
            cut = max(0, L - Sq - window + 1)
            kb[b, :, :cut] = 0x7FC0
            vb[b, :, :cut] = 0x7FC0
    q = torch.from_numpy(inp["q_bits"].view(np.int16)).view(torch.bfloat16).to(device)
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(device)
    v = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(device)
    cl = None if lens is None else torch.tensor(list(lens), dtype=torch.int32, device=device)
    ws = None
    if ws_guard:  # the workspace the call asks for, then a guard region it must not touch
        need = attn.decode_workspace_bytes(B, Hq, Hkv, Sq, Smax, D, mask, window)
        ws = torch.full((need + 65536,), 0x5A, dtype=torch.uint8, device=device)
    o = attn.decode(q, k, v, cache_len=cl, mask=mask, scale=scale, window=window, workspace=ws)
    torch.cuda.synchronize()
    if ws_guard:
        assert bool((ws[need:] == 0x5A).all()), "write past the workspace"
    got = o.float().cpu().numpy()
    ref = oracle.decode_attention(inp["q"], inp["k"], inp["v"], mask,
                                  cache_len=lens, scale=scale, window=window)
    if rows is not None:
        got = np.stack([got[b, a, i] for b, a, i in rows])
        ref = np.stack([ref[b, a, i] for b, a, i in rows])
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got.astype(np.float64) - ref)))


SWEEP = []
_rng = np.random.default_rng(77)
for D in (64, 128):
    for (Hq, Hkv, Sq) in ((8, 8, 1), (32, 8, 1), (32, 8, 8), (8, 1, 4), (4, 2, 3), (32, 1, 1)):
        for Smax in (1, 33, 300, 2049):
            for mask in ("causal", "full"):
                B = 1 + int(_rng.integers(3))
                lens = None
                if _rng.integers(2) and Smax > 1:
                    lens = tuple(int(x) for x in _rng.integers(0, Smax + 1, size=B))
                SWEEP.append((B, Hq, Hkv, Sq, Smax, D, mask, lens, 0))
        # sliding window: one, a part of a tile, several tiles, about the cache
        for Smax, window in ((300, 1), (300, 17), (2049, 100), (2049, 700), (2049, 2049)):
            B = 1 + int(_rng.integers(3))
            lens = None
            if _rng.integers(2):
                lens = tuple(int(x) for x in _rng.integers(0, Smax + 1, size=B))
            SWEEP.append((B, Hq, Hkv, Sq, Smax, D, "causal_window", lens, window))


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"D{c[5]}-H{c[1]}x{c[2]}-Sq{c[3]}-S{c[4]}-"
                                                      f"{c[6]}{c[8] or ''}-"
                                                      f"{'ragged' if c[7] else 'full'}")
def test_decode_sweep(device, case):
    B, Hq, Hkv, Sq, Smax, D, mask, lens, window = case
    err = run_decode(device, B, Hq, Hkv, Sq, Smax, D, mask, lens, seed=Smax + 3 * Sq + D,
                     window=window)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.2, 1.0])
def test_decode_scales(device, scale):
    err = run_decode(device, 2, 16, 4, 2, 700, 128, "causal", (700, 431), seed=9, scale=scale)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
def test_decode_edge_lengths(device):
    """Lengths 0, below Sq, exactly Sq, one tile, a tile plus one, and lengths
    ending on and around the split boundaries of the plan."""
    lens = (0, 2, 4, 32, 33, 255, 256, 257, 1023, 1024, 4096)
    err = run_decode(device, len(lens), 8, 2, 4, 4096, 128, "causal", lens, seed=10)
    assert err <= TOL["bf16"], err
    for window in (1, 3, 32, 253, 1021):
        err = run_decode(device, len(lens), 8, 2, 4, 4096, 128, "causal_window", lens, seed=11,
                         window=window)
        assert err <= TOL["bf16"], (window, err)


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["one_long", "many_short", "mqa_skew", "window_skew"])
def test_decode_split_plan(device, case):
    """Lengths that push the plan made from the device-side lengths: one long
    sequence among empty and short ones (it takes nearly all splits), many
    sequences (most take one split), a key/value head shared by 32 query
    heads, and a window over skewed lengths.  The workspace is followed by a
    guard region the call must leave alone."""
    if case == "one_long":
        args = (9, 8, 2, 1, 65536, 128, "causal", (0, 65536, 3, 100, 0, 1, 300, 2, 31), 0)
    elif case == "many_short":
        lens = tuple(int(x) for x in np.random.default_rng(3).integers(0, 4097, size=96))
        args = (96, 8, 2, 2, 4096, 64, "causal", lens, 0)
    elif case == "mqa_skew":
        args = (3, 32, 1, 1, 40000, 128, "full", (40000, 257, 9999), 0)
    else:
        args = (5, 16, 4, 2, 30000, 128, "causal_window", (30000, 5000, 4097, 4095, 17), 4096)
    B, Hq, Hkv, Sq, Smax, D, mask, lens, window = args
    err = run_decode(device, B, Hq, Hkv, Sq, Smax, D, mask, lens, seed=12, window=window,
                     ws_guard=True)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(workloads.DECODE_WORKLOADS))
def test_decode_workload_full_size(device, name):
    """The decode workloads at full size, in the launch configuration the
    benchmark times; sampled (b, head, position) rows compared element-wise."""
    w = workloads.DECODE_WORKLOADS[name]
    rng = np.random.default_rng(w.seed + 5)
    rows = {(0, 0, 0), (w.B - 1, w.Hq - 1, w.Sq - 1)}
    for _ in range(12):
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Sq))))
    lens = tuple(int(x) for x in w.cache_len()) if w.lengths != "full" else None
    err = run_decode(device, w.B, w.Hq, w.Hkv, w.Sq, w.Smax, w.D, w.mask, lens, seed=w.seed,
                     rows=sorted(rows), window=w.window)
    print(f"{name}: max abs err {err:.3e}", flush=True)
    assert err <= TOL["bf16"], err


# ----------------------------------------------------------------------------
# host-only: validation happens before any device access
# ----------------------------------------------------------------------------

FAKE = 0x100000  # an aligned non-null address; never dereferenced (validation fails first)


def decode_status(B=1, Hq=8, Hkv=2, Sq=1, Smax=1000, D=128, mask="causal", scale=0.1,
                  dtype=attn.DTYPE_BF16, ws=0, ws_bytes=0, ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE * 7),
                  cache_len=0, window=0):
    q, k, v, o = ptrs
    return attn.decode_raw(q, k, v, o, cache_len, B, Hq, Hkv, Sq, Smax, D, mask, window, scale,
                           dtype, ws, ws_bytes, 0)


def test_decode_workspace_plan():
    # key ranges of at most 256 positions (eight 32-key tiles) never split
    assert attn.decode_workspace_status(64, 32, 8, 1, 256, 128) == (0, 0)
    assert attn.decode_workspace_status(64, 32, 8, 4, 65536, 128, "causal_window",
                                        window=253) == (0, 0)
    # longer ranges: 256 partial slots of 32 rows x (D + 2) floats, then 8
    # bytes per (sequence, key/value head) pair; independent of the lengths
    for B, Hkv, D in ((1, 8, 128), (64, 8, 128), (3, 1, 64)):
        st, n = attn.decode_workspace_status(B, 4 * Hkv, Hkv, 1, 8192, D)
        assert st == 0 and n == 256 * 32 * (D + 2) * 4 + 8 * B * Hkv
    # the same for every mask kind, and for a window whose range is 257 positions
    n = attn.decode_workspace_status(1, 32, 8, 1, 8192, 128)[1]
    assert attn.decode_workspace_status(1, 32, 8, 1, 8192, 128, "full")[1] == n
    assert attn.decode_workspace_status(1, 32, 8, 1, 8192, 128, "causal_window",
                                        window=257)[1] == n


def test_decode_rejects_bad_arguments():
    ws_n = attn.decode_workspace_bytes(1, 8, 2, 1, 1000, 128)
    assert ws_n > 0
    st = lambda **kw: attn.status_string(decode_status(**kw))  # noqa: E731
    assert st(ptrs=(0, FAKE, FAKE * 3, FAKE * 5)) == "ATTN_ERR_NULL"
    assert st(Sq=0) == "ATTN_ERR_SHAPE"
    assert st(Smax=0) == "ATTN_ERR_SHAPE"
    assert st(Hq=6, Hkv=4) == "ATTN_ERR_HEADS"
    assert st(D=96) == "ATTN_ERR_UNSUPPORTED"
    assert st(dtype=attn.DTYPE_FP32) == "ATTN_ERR_UNSUPPORTED"
    assert st(mask="causal_window") == "ATTN_ERR_WINDOW"         # window 0
    assert st(mask="causal_window", window=-3) == "ATTN_ERR_WINDOW"
    assert st(mask="causal", window=5) == "ATTN_ERR_WINDOW"      # a window without its mask
    assert st(mask="full", window=5) == "ATTN_ERR_WINDOW"
    assert st(mask="local_global", window=5) == "ATTN_ERR_UNSUPPORTED"
    assert st(Hq=32, Hkv=1, Sq=2) == "ATTN_ERR_UNSUPPORTED"   # 64 query rows per key/value head
    assert st(scale=float("nan")) == "ATTN_ERR_SCALE"
    assert st(ptrs=(FAKE + 8, FAKE * 3, FAKE * 5, FAKE * 7)) == "ATTN_ERR_ALIGN"
    assert st(cache_len=FAKE + 2) == "ATTN_ERR_ALIGN"
    assert st(ptrs=(FAKE, FAKE * 3, FAKE * 5, FAKE)) == "ATTN_ERR_ALIAS"
    assert st() == "ATTN_ERR_WORKSPACE"                        # needed but not given
    assert st(ws=FAKE * 64, ws_bytes=ws_n - 16) == "ATTN_ERR_WORKSPACE"
    assert st(ws=FAKE * 64 + 4, ws_bytes=ws_n) == "ATTN_ERR_WORKSPACE"
    assert st(ws=FAKE, ws_bytes=ws_n) == "ATTN_ERR_ALIAS"       # workspace over q


def test_decode_symbols_exported():
    lib = ctypes.CDLL(attn.LIB_PATH)
    for name in ("attn_decode", "attn_decode_workspace", "attn_decode_noalloc"):
        assert hasattr(lib, name)
