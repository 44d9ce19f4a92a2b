"""Block-sparse attention (attn_fwd_ex with block_layout) and the layout
builders.

CPU: the C builders write the same bits as the oracle's pattern definitions;
argument validation.  GPU: every output element against
oracle.block_sparse_attention (fp64) at the bf16 tolerance over both head
dimensions, full and causal masks, the three patterns, random layouts (stray
bits beyond the last block included), rows that see nothing, group sizes
1/2/4/8 and both memory layouts; an all-ones layout equals the dense call bit
for bit; the two sparse workloads at full size on sampled rows.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import sparse as sp
from tests.test_parity import TOL

attn = pytest.importorskip("transformer_attention_attn_amd")


def pack(lay):
    """bool [nb][nb] -> uint32 [nb][words] with bit J % 32 of word J // 32."""
    lay = np.asarray(lay, dtype=bool)
    nb = lay.shape[0]
    out = np.zeros((nb, (nb + 31) // 32), dtype=np.uint32)
    for I in range(nb):
        for J in np.nonzero(lay[I])[0]:
            out[I, J // 32] |= np.uint32(1) << np.uint32(J % 32)
    return out


def unpack(words, nb):
    return np.array([[(int(words[I, J // 32]) >> (J % 32)) & 1 for J in range(nb)]
                     for I in range(nb)], dtype=bool)


# ----------------------------------------------------------------------------
# CPU: builders and validation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("nb", [1, 2, 7, 31, 32, 33, 64, 100, 128])
def test_builders_match_oracle(nb):
    for local, stride in ((0, 1), (1, 3), (3, 2), (7, 8), (0, 200), (200, 5)):
        assert np.array_equal(attn.layout_strided(nb, local, stride),
                              pack(sp.strided_layout(nb, local, stride))), (local, stride)
    for chunk in (1, 2, 3, 8, 200):
        assert np.array_equal(attn.layout_fixed(nb, chunk), pack(sp.fixed_layout(nb, chunk)))
    rng = np.random.default_rng(nb)
    for radius, g, r in ((0, 0, 0), (1, 2, 3), (3, 1, 1), (nb, 0, 2)):
        rand = rng.integers(0, nb, size=(nb, r))
        assert np.array_equal(attn.layout_bigbird(nb, radius, g, rand),
                              pack(sp.bigbird_layout(nb, radius, g, rand.reshape(nb, -1)))), (
            radius, g, r)


def test_builders_reject_bad_arguments():
    for call in (lambda: attn.layout_strided(0, 1, 1), lambda: attn.layout_strided(513, 1, 1),
                 lambda: attn.layout_strided(8, -1, 1), lambda: attn.layout_strided(8, 1, 0),
                 lambda: attn.layout_fixed(8, 0),
                 lambda: attn.layout_bigbird(8, 1, 1, np.full((8, 1), 8)),
                 lambda: attn.layout_bigbird(8, -1, 1, np.zeros((8, 0)))):
        with pytest.raises(attn.AttnError) as e:
            call()
        assert attn.status_string(e.value.status) == "ATTN_ERR_SHAPE"


def sparse_status(**kw):
    a = attn.FwdArgs()
    base = 0x1000000
    a.q, a.k, a.v, a.o = base, base * 3, base * 5, base * 7
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = 1, 8, 2, 1000, 1000, 128
    a.q_stride[:] = [8 * 1000 * 128, 1000 * 128, 128]
    a.k_stride[:] = [2 * 1000 * 128, 1000 * 128, 128]
    a.v_stride[:] = [2 * 1000 * 128, 1000 * 128, 128]
    a.o_stride[:] = [8 * 1000 * 128, 1000 * 128, 128]
    a.mask_kind, a.window, a.scale, a.dtype = 1, 0, 0.1, attn.DTYPE_BF16
    a.alibi_slopes, a.q_len, a.kv_len, a.block_layout = None, None, None, base * 9
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return attn.status_string(attn.fwd_ex_raw(a, 0))


def test_block_layout_validation():
    assert sparse_status(Skv=1001, k_stride=[2 * 1001 * 128, 1001 * 128, 128],
                         v_stride=[2 * 1001 * 128, 1001 * 128, 128]) == "ATTN_ERR_UNSUPPORTED"
    assert sparse_status(mask_kind=2, window=10) == "ATTN_ERR_UNSUPPORTED"
    assert sparse_status(alibi_slopes=0x2000000) == "ATTN_ERR_UNSUPPORTED"
    assert sparse_status(q_len=0x2000000) == "ATTN_ERR_UNSUPPORTED"
    S = 32768 + 64  # one block past the longest layout
    assert sparse_status(Sq=S, Skv=S, q_stride=[8 * S * 128, S * 128, 128],
                         k_stride=[2 * S * 128, S * 128, 128], v_stride=[2 * S * 128, S * 128, 128],
                         o_stride=[8 * S * 128, S * 128, 128]) == "ATTN_ERR_UNSUPPORTED"
    assert sparse_status(block_layout=0x9000002) == "ATTN_ERR_ALIGN"
    assert sparse_status(block_layout=0x7000000 + 4096) == "ATTN_ERR_ALIAS"   # inside o


# ----------------------------------------------------------------------------
# GPU parity
# ----------------------------------------------------------------------------

def run_sparse(device, B, Hq, Hkv, S, D, mask, lay_bool, words=None, layout="bhsd", seed=0,
               rows=None):
    """Max abs error of block-sparse attn_fwd_ex against the oracle.  `words`
    (the device layout) defaults to the packed `lay_bool`."""
    import torch

    from tests.test_fwd_ex import empty_out, place

    print(f"sparse case B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {mask} {layout} seed={seed} "
          f"density={np.mean(lay_bool):.3f}", flush=True)
    inp = workloads.make_decode_inputs(B, Hq, Hkv, S, S, D, seed)
    q, k, v = (place(inp[n + "_bits"], layout, device) for n in ("q", "k", "v"))
    o = empty_out(B, Hq, S, D, layout, device)
    if words is None:
        words = pack(lay_bool)
    lay_d = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)
    attn.fwd_ex(q, k, v, mask=mask, out=o, block_layout=lay_d)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ref = oracle.block_sparse_attention(inp["q"], inp["k"], inp["v"], lay_bool, 64,
                                        mask == "causal", rows=rows)
    if rows is not None:
        got = got[:, :, rows]
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got.astype(np.float64) - ref)))


def random_layout(rng, nb, density, causal):
    lay = rng.random((nb, nb)) < density
    return np.tril(lay) if causal else lay


SWEEP = []
_rng = np.random.default_rng(93)
for D in (64, 128):
    for S in (64, 100, 257, 1000, 2049):
        for mask in ("full", "causal"):
            for pat in ("strided", "fixed", "bigbird", "random"):
                Hq, Hkv = [(8, 2), (4, 4), (8, 1), (4, 2)][int(_rng.integers(4))]
                layout = ["bhsd", "bshd"][int(_rng.integers(2))]
                SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, S, D, mask, pat, layout,
                              int(_rng.integers(1 << 30))))


def sweep_layout(pat, nb, causal, seed):
    rng = np.random.default_rng(seed)
    if pat == "strided":
        return sp.strided_layout(nb, int(rng.integers(0, 3)), int(rng.integers(1, 5)))
    if pat == "fixed":
        return sp.fixed_layout(nb, int(rng.integers(1, 5)))
    if pat == "bigbird":
        lay = sp.bigbird_layout(nb, int(rng.integers(0, 2)), int(rng.integers(0, 2)),
                                rng.integers(0, nb, size=(nb, 2)))
        return np.tril(lay) if causal else lay
    return random_layout(rng, nb, 0.3, causal)


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"D{c[4]}-S{c[3]}-{c[5]}-{c[6]}-{c[7]}")
def test_sparse_sweep(device, case):
    B, Hq, Hkv, S, D, mask, pat, layout, seed = case
    nb = sp.n_blocks(S, 64)
    lay = sweep_layout(pat, nb, mask == "causal", seed)
    err = run_sparse(device, B, Hq, Hkv, S, D, mask, lay, layout=layout, seed=seed % 1000)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_sparse_edge_layouts(device, D):
    """Rows that see nothing (zeros), single 64-key halves of 128-key tiles,
    stray bits past the last block, upper-triangle bits under a causal mask."""
    S = 1000
    nb = sp.n_blocks(S, 64)
    rng = np.random.default_rng(40 + D)
    lay = random_layout(rng, nb, 0.25, False)
    lay[3] = False                          # query block 3 sees nothing
    lay[5] = False
    lay[5, 2] = True                        # first half of tile 1 (D = 128) only
    lay[6] = False
    lay[6, 3] = True                        # second half of tile 1 only
    words = pack(lay)
    words[:, -1] |= np.uint32(0xFFFFFFFF) << np.uint32(nb % 32)  # blocks >= nb: no keys
    for mask in ("full", "causal"):
        err = run_sparse(device, 2, 8, 2, S, D, mask, lay, words=words, seed=7)
        assert err <= TOL["bf16"], (mask, err)


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_all_ones_layout_equals_dense(device, D):
    import torch

    inp = workloads.make_decode_inputs(2, 8, 2, 777, 777, D, seed=24)
    q, k, v = (torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16)
               .to(device).contiguous() for n in ("q", "k", "v"))
    nb = sp.n_blocks(777, 64)
    ones = torch.from_numpy(pack(np.ones((nb, nb), dtype=bool)).view(np.int32)).to(device)
    for mask in ("causal", "full"):
        a = attn.fwd_ex(q, k, v, mask=mask)
        b = attn.fwd_ex(q, k, v, mask=mask, block_layout=ones)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), mask


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S,mask,density", [(32768, "full", 0.45), (32768, "causal", 0.9),
                                            (20001, "full", 0.8), (12345, "causal", 0.35)])
def test_sparse_long_sequences(device, D, S, mask, density):
    """Layouts up to the 512-block limit (32768 positions), dense enough that
    an item's tile list fills several list registers (up to 256 tiles of 128
    keys, 512 of 64); sampled rows of every head against the oracle,
    including the first and last rows of blocks and the ragged tail."""
    nb = sp.n_blocks(S, 64)
    rng = np.random.default_rng(S + D)
    lay = random_layout(rng, nb, density, mask == "causal")
    lay[np.arange(nb), np.arange(nb)] = True  # every row sees its own block
    rows = sorted({0, 63, 64, 4095, 8192, S // 2, S - 65, S - 64, S - 1}
                  | {int(x) for x in rng.integers(S, size=6)})
    err = run_sparse(device, 1, 8, 2, S, D, mask, lay, seed=S % 997, rows=rows)
    assert err <= TOL["bf16"], err


def workload_layout_bool(w):
    nb = w.n_blocks()
    if w.pattern == "strided":
        return sp.strided_layout(nb, *w.pattern_args)
    if w.pattern == "fixed":
        return sp.fixed_layout(nb, *w.pattern_args)
    radius, g, _ = w.pattern_args
    return sp.bigbird_layout(nb, radius, g, w.rand_blocks())


def workload_layout_words(w):
    nb = w.n_blocks()
    if w.pattern == "strided":
        return attn.layout_strided(nb, *w.pattern_args)
    if w.pattern == "fixed":
        return attn.layout_fixed(nb, *w.pattern_args)
    radius, g, _ = w.pattern_args
    return attn.layout_bigbird(nb, radius, g, w.rand_blocks())


SPARSE_WORKLOADS = [n for n, w in workloads.EX_WORKLOADS.items() if w.pattern]


@pytest.mark.parametrize("name", SPARSE_WORKLOADS)
def test_workload_layouts_match_oracle(name):
    w = workloads.EX_WORKLOADS[name]
    assert np.array_equal(workload_layout_words(w), pack(workload_layout_bool(w)))


@pytest.mark.gpu
@pytest.mark.parametrize("name", SPARSE_WORKLOADS)
def test_sparse_workload_full_size(device, name):
    """The block-sparse workloads at full size with the layout the benchmark
    builds (C builder); sampled rows of batch 0 and the last batch, all heads,
    against the oracle's own layout."""
    import torch

    w = workloads.EX_WORKLOADS[name]
    print(f"sparse workload {name}", flush=True)
    inp = workloads.ex_workload_inputs(w)
    q, k, v = (torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16)
               .to(device).contiguous() for n in ("q", "k", "v"))
    lay_d = torch.from_numpy(workload_layout_words(w).view(np.int32)).to(device)
    o = attn.fwd_ex(q, k, v, mask=w.mask, scale=w.scale, block_layout=lay_d)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    rng = np.random.default_rng(w.seed + 5)
    rows = sorted({0, 1, 63, 64, 127, 128, w.Sq // 2, w.Sq - 1}
                  | {int(x) for x in rng.integers(w.Sq, size=8)})
    lay = workload_layout_bool(w)
    for b in sorted({0, w.B - 1}):
        ref = oracle.block_sparse_attention(inp["q"][b:b + 1], inp["k"][b:b + 1],
                                            inp["v"][b:b + 1], lay, 64, w.mask == "causal",
                                            scale=w.scale, rows=rows)
        err = float(np.max(np.abs(got[b:b + 1, :, rows].astype(np.float64) - ref)))
        print(f"{name} b={b}: max abs err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], (b, err)
