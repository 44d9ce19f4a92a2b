"""attn_fwd_ex (Sq != Skv, strided layouts, ALiBi, padded batches, local +
global tokens) against the fp64 oracle.

GPU cases compare every output element with oracle.cross_attention (queries
aligned to the end of the keys) at the bf16 tolerance, over head-major,
sequence-major and padded-row layouts for inputs and output, with and
without ALiBi slopes and per-sequence lengths (NaN in every padded position);
with Sq == Skv and dense layouts the result must equal attn_fwd's bit for
bit.  Host-only cases check the validation.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.test_parity import TOL

attn = pytest.importorskip("transformer_attention_attn_amd")


def place(bits, layout, device):
    """A [B, H, S, D] bf16 view of the bit array in the given memory layout."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    B, H, S, D = t.shape
    if layout == "bhsd":
        return t.to(device).contiguous()
    if layout == "bshd":
        return t.transpose(1, 2).contiguous().to(device).transpose(1, 2)
    if layout == "padded":
        buf = torch.zeros((B, H, S, D + 24), dtype=torch.bfloat16)
        buf[..., :D] = t
        return buf.to(device)[..., :D]
    raise ValueError(layout)


def empty_out(B, H, S, D, layout, device):
    import torch

    if layout == "bhsd":
        return torch.empty((B, H, S, D), dtype=torch.bfloat16, device=device)
    if layout == "bshd":
        return torch.empty((B, S, H, D), dtype=torch.bfloat16, device=device).transpose(1, 2)
    return torch.empty((B, H, S, D + 8), dtype=torch.bfloat16, device=device)[..., :D]


def run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window=0, layout="bhsd", out_layout="bhsd",
           seed=0, scale=None, slopes=None, q_len=None, kv_len=None, global_idx=(),
           dist_bias=None, rel=0.0):
    """Max abs error of attn_fwd_ex against the oracle, less rel * |oracle| per
    element.  With lengths, the padded query rows, keys and values hold NaN
    (bf16 0x7FC0)."""
    import torch

    print(f"fwd_ex case B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} {mask} w={window} "
          f"{layout}->{out_layout} seed={seed} scale={scale} alibi={slopes is not None} "
          f"q_len={q_len} kv_len={kv_len} globals={list(global_idx)} "
          f"dist_bias={dist_bias is not None}", flush=True)
    rng = np.random.default_rng(seed)
    bits = {}
    vals = {}
    for name, shape in (("q", (B, Hq, Sq, D)), ("k", (B, Hkv, Skv, D)), ("v", (B, Hkv, Skv, D))):
        bits[name] = workloads.bf16_round_bits(workloads.draw(shape, rng))
        vals[name] = workloads.bf16_bits_to_float(bits[name])
    for b in range(B):
        if q_len is not None:
            bits["q"][b, :, q_len[b]:] = 0x7FC0
        if kv_len is not None:
            bits["k"][b, :, kv_len[b]:] = 0x7FC0
            bits["v"][b, :, kv_len[b]:] = 0x7FC0
    q, k, v = (place(bits[n], layout, device) for n in ("q", "k", "v"))
    o = empty_out(B, Hq, Sq, D, out_layout, device)
    dev_arr = lambda x, dt: None if x is None else torch.tensor(list(x), dtype=dt, device=device)  # noqa: E731
    attn.fwd_ex(q, k, v, mask=mask, window=window, scale=scale, out=o,
                alibi_slopes=dev_arr(slopes, torch.float32), q_len=dev_arr(q_len, torch.int32),
                kv_len=dev_arr(kv_len, torch.int32), global_idx=list(global_idx) or None,
                dist_bias=None if dist_bias is None else torch.from_numpy(dist_bias).to(device))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ref = oracle.cross_attention(vals["q"], vals["k"], vals["v"], mask, window, scale=scale,
                                 alibi_slopes=slopes, q_len=q_len, kv_len=kv_len,
                                 global_idx=global_idx, dist_bias=dist_bias)
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got.astype(np.float64) - ref) - rel * np.abs(ref)))


SWEEP = []
_rng = np.random.default_rng(91)
for D in (64, 128):
    for (Sq, Skv) in ((100, 300), (300, 100), (257, 257), (1, 500), (64, 1000), (513, 2049),
                      (129, 128)):
        for mask in ("full", "causal", "causal_window"):
            Hq, Hkv = [(8, 2), (4, 4), (8, 1)][int(_rng.integers(3))]
            window = int(_rng.choice([1, 63, 200])) if mask == "causal_window" else 0
            layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            out_layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, Sq, Skv, D, mask, window, layout,
                          out_layout))


@pytest.mark.gpu
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-{c[6]}-"
                                                      f"{c[8]}-{c[9]}")
def test_fwd_ex_sweep(device, case):
    B, Hq, Hkv, Sq, Skv, D, mask, window, layout, out_layout = case
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window, layout, out_layout,
                 seed=Sq * 3 + Skv + D)
    assert err <= TOL["bf16"], err


ALIBI_SWEEP = []
_rng = np.random.default_rng(92)
for D in (64, 128):
    for (Sq, Skv) in ((100, 300), (300, 100), (257, 257), (1, 500), (513, 2049)):
        for mask in ("full", "causal", "causal_window"):
            Hq, Hkv = [(8, 2), (4, 4), (8, 1)][int(_rng.integers(3))]
            window = int(_rng.choice([1, 63, 200])) if mask == "causal_window" else 0
            layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            ALIBI_SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, Sq, Skv, D, mask, window,
                                layout))


@pytest.mark.gpu
@pytest.mark.parametrize("case", ALIBI_SWEEP, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-{c[6]}-"
                                                            f"{c[8]}")
def test_fwd_ex_alibi_sweep(device, case):
    """ALiBi with distinct slopes per query head (also inside one group)."""
    B, Hq, Hkv, Sq, Skv, D, mask, window, layout = case
    slopes = [float(x) for x in workloads.make_alibi_slopes(Hq)]
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window, layout, layout,
                 seed=Sq + 7 * Skv + D, slopes=slopes)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.1, 0.5])
@pytest.mark.parametrize("mask", ["full", "causal"])
def test_fwd_ex_alibi_scales(device, scale, mask):
    """Zero and negative scales, and steep slopes (weights decay within a
    few keys), on both ALiBi forms."""
    slopes = [0.02, 0.5, 2.0, 8.0]
    err = run_ex(device, 1, 4, 2, 130, 700, 128, mask, seed=31, scale=scale, slopes=slopes)
    assert err <= TOL["bf16"], err


DIST_SWEEP = []
_rng = np.random.default_rng(93)
for D in (64, 128):
    for (Sq, Skv) in ((100, 300), (300, 100), (257, 257), (1, 500), (513, 2049), (129, 128)):
        for mask in ("full", "causal", "causal_window"):
            Hq, Hkv = [(8, 2), (4, 4), (8, 1)][int(_rng.integers(3))]
            window = int(_rng.choice([1, 63, 200])) if mask == "causal_window" else 0
            layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            DIST_SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, Sq, Skv, D, mask, window,
                               layout))


@pytest.mark.gpu
@pytest.mark.parametrize("case", DIST_SWEEP, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-{c[6]}-"
                                                           f"{c[8]}")
def test_fwd_ex_distance_bias_sweep(device, case):
    """A bucketed distance-bias table (distinct per query head, also inside
    one group), every element against the oracle."""
    B, Hq, Hkv, Sq, Skv, D, mask, window, layout = case
    table = workloads.make_distance_bias(Hq, Sq, Skv, seed=Sq + Skv + D)
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window, layout, layout,
                 seed=Sq + 5 * Skv + D, dist_bias=table)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.1, 0.5])
@pytest.mark.parametrize("D", [64, 128])
def test_fwd_ex_distance_bias_scales_and_steep(device, scale, D):
    """Zero and negative scales, and a steep table (a row's weight sits on a
    few distances, -30 elsewhere), so the bias alone picks the keys.  Outputs
    are then close to single value rows (|O| up to about 4.5), where rounding
    O to bf16 alone (P rounded to bf16, O rounded once, to nearest even) may
    be off by half a unit in the last place, 2^-8 |O|: the check allows that
    on top of the bf16 tolerance."""
    rng = np.random.default_rng(41)
    Sq, Skv = 130, 700
    table = (rng.standard_normal((4, Sq + Skv - 1)) * 4.0).astype(np.float32)
    table[:, rng.random(Sq + Skv - 1) < 0.8] = -30.0
    for mask in ("full", "causal"):
        err = run_ex(device, 1, 4, 2, Sq, Skv, D, mask, seed=37, scale=scale, dist_bias=table,
                     rel=2.0 ** -8)
        assert err <= TOL["bf16"], (mask, err)


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_fwd_ex_distance_bias_as_alibi(device, D):
    """The table -m_a |d| gives ALiBi's result (two kernels, same inputs)."""
    import torch

    B, Hq, Hkv, Sq, Skv = 2, 8, 2, 200, 333
    slopes = workloads.make_alibi_slopes(Hq)
    d = np.arange(Sq + Skv - 1) - (Skv - 1)
    table = (-slopes[:, None].astype(np.float64) * np.abs(d)[None, :]).astype(np.float32)
    rng = np.random.default_rng(42)
    q = torch.from_numpy(workloads.draw((B, Hq, Sq, D), rng)).to(torch.bfloat16).to(device)
    k = torch.from_numpy(workloads.draw((B, Hkv, Skv, D), rng)).to(torch.bfloat16).to(device)
    v = torch.from_numpy(workloads.draw((B, Hkv, Skv, D), rng)).to(torch.bfloat16).to(device)
    for mask in ("full", "causal", "causal_window"):
        a = attn.fwd_ex(q, k, v, mask=mask, window=77,
                        alibi_slopes=torch.from_numpy(slopes).to(device))
        b = attn.fwd_ex(q, k, v, mask=mask, window=77, dist_bias=torch.from_numpy(table).to(device))
        torch.cuda.synchronize()
        err = (a.float() - b.float()).abs().max().item()
        assert err <= TOL["bf16"], (mask, err)


RAGGED = [
    # (B, Hq, Hkv, Sq, Skv, D, mask, window, q_len, kv_len, alibi)
    (4, 8, 2, 300, 300, 128, "causal", 0, (300, 1, 129, 0), (300, 1, 129, 0), False),
    (3, 4, 4, 257, 257, 64, "full", 0, (257, 100, 64), (257, 100, 64), True),
    (3, 8, 1, 200, 600, 128, "causal", 0, (200, 17, 0), (600, 300, 5), True),
    (2, 8, 2, 130, 400, 64, "causal_window", 50, (130, 64), (130, 399), False),
    (3, 4, 2, 400, 150, 128, "causal", 0, (400, 33, 150), (150, 150, 0), True),
    (2, 4, 4, 64, 1000, 128, "full", 0, (64, 30), (1000, 999), False),
    (4, 8, 8, 513, 513, 64, "causal_window", 128, (513, 256, 255, 129), (513, 256, 255, 129), True),
    # windows near INT_MAX with queries ahead of their keys (position - window
    # must not wrap in 32 bits)
    (3, 8, 2, 300, 200, 128, "causal_window", 2**31 - 1, (300, 100, 50), (200, 40, 50), False),
    (2, 4, 4, 257, 129, 64, "causal_window", 2**31 - 2, (257, 200), (129, 1), True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-{c[6]}-"
                                                      f"{'alibi' if c[10] else 'plain'}")
def test_fwd_ex_padded_batches(device, case):
    """Per-sequence lengths (right padding, NaN in every padded position),
    including empty sequences, single rows, q_len > kv_len and lengths on
    and beside tile edges."""
    B, Hq, Hkv, Sq, Skv, D, mask, window, q_len, kv_len, alibi = case
    slopes = [float(x) for x in workloads.make_alibi_slopes(Hq)] if alibi else None
    for layout in ("bhsd", "bshd"):
        err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window, layout, layout,
                     seed=Sq + Skv + B, slopes=slopes, q_len=q_len, kv_len=kv_len)
        assert err <= TOL["bf16"], (layout, err)


@pytest.mark.gpu
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-{c[6]}")
def test_fwd_ex_distance_bias_padded_batches(device, case):
    """The distance bias on the same padded batches (each sequence's own
    positions index the table)."""
    B, Hq, Hkv, Sq, Skv, D, mask, window, q_len, kv_len, _ = case
    table = workloads.make_distance_bias(Hq, Sq, Skv, seed=B + D)
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, mask, window, "bshd", "bhsd",
                 seed=Sq + Skv + B + 1, q_len=q_len, kv_len=kv_len, dist_bias=table)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_fwd_ex_huge_window_sq_gt_skv(device, D):
    """Sq > Skv (the first queries see no key) with windows near INT_MAX: the
    same result as the causal mask."""
    for w in (2**31 - 1, 2**30 + 5):
        err = run_ex(device, 1, 8, 2, 333, 130, D, "causal_window", w, seed=D + 3)
        assert err <= TOL["bf16"], (w, err)


@pytest.mark.gpu
def test_fwd_ex_full_lengths_equal_no_lengths(device):
    """Lengths equal to Sq and Skv give the same bits as no lengths."""
    import torch

    inp = workloads.make_decode_inputs(2, 8, 2, 300, 700, 128, seed=23)
    q, k, v = (torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16)
               .to(device).contiguous() for n in ("q", "k", "v"))
    ql = torch.tensor([300, 300], dtype=torch.int32, device=device)
    kl = torch.tensor([700, 700], dtype=torch.int32, device=device)
    for mask in ("causal", "full"):
        a = attn.fwd_ex(q, k, v, mask=mask)
        b = attn.fwd_ex(q, k, v, mask=mask, q_len=ql, kv_len=kl)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), mask


LG_SWEEP = []
_rng = np.random.default_rng(93)
for D in (64, 128):
    for (Sq, Skv) in ((257, 257), (100, 300), (300, 100), (1, 500), (64, 1000), (513, 2049)):
        for window in (0, 3, 200):
            g = sorted({int(x) for x in _rng.integers(0, Skv, size=int(_rng.integers(0, 5)))}
                       | ({Skv - 1} if _rng.integers(2) else set()))
            Hq, Hkv = [(8, 2), (4, 4), (8, 1)][int(_rng.integers(3))]
            layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            out_layout = ["bhsd", "bshd", "padded"][int(_rng.integers(3))]
            LG_SWEEP.append((1 + int(_rng.integers(2)), Hq, Hkv, Sq, Skv, D, window, tuple(g),
                             layout, out_layout))


@pytest.mark.gpu
@pytest.mark.parametrize("case", LG_SWEEP, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-w{c[6]}-"
                                                         f"g{len(c[7])}-{c[8]}-{c[9]}")
def test_fwd_ex_local_global_sweep(device, case):
    """Local + global tokens with the queries at the end of the keys (global
    indices are key positions), every layout, windows 0 to 200."""
    B, Hq, Hkv, Sq, Skv, D, window, g, layout, out_layout = case
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, "local_global", window, layout, out_layout,
                 seed=Sq + 7 * Skv + D + window, global_idx=g)
    assert err <= TOL["bf16"], err


LG_PADDED = [
    # (B, Hq, Hkv, Sq, Skv, D, window, globals, q_len, kv_len)
    (3, 8, 2, 600, 600, 64, 64, (0, 100, 450, 599), (600, 300, 0), (600, 300, 0)),
    (3, 4, 4, 700, 700, 128, 32, (3, 650), (700, 500, 650), (700, 500, 651)),
    (2, 8, 1, 256, 900, 128, 100, (0, 700, 899), (256, 100), (900, 750)),
    (2, 12, 12, 1100, 1100, 64, 512, (0, 1000), (1100, 999), (1100, 999)),
    # more queries than keys, a window wider than the keys, huge window
    (2, 8, 2, 300, 100, 128, 200, (13, 99), (300, 120), (100, 40)),
    (1, 4, 1, 400, 150, 64, 2 ** 31 - 1, (7,), (400,), (150,)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", LG_PADDED, ids=lambda c: f"D{c[5]}-Sq{c[3]}-Skv{c[4]}-w{c[6]}")
def test_fwd_ex_local_global_padded(device, case):
    """Padded Longformer batches: per-sequence lengths with global positions
    past a sequence's end, on a padded query row's position, and in empty
    sequences; padded positions hold NaN and padded rows must come out zero."""
    B, Hq, Hkv, Sq, Skv, D, window, g, q_len, kv_len = case
    err = run_ex(device, B, Hq, Hkv, Sq, Skv, D, "local_global", window, "bshd", "bhsd",
                 seed=Sq + D + window, q_len=q_len, kv_len=kv_len, global_idx=g)
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
def test_fwd_ex_square_dense_equals_fwd(device, D):
    """Sq == Skv with dense layouts computes exactly what attn_fwd computes."""
    import torch

    inp = workloads.make_inputs(2, 8, 2, 700, D, "bf16", seed=21)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    for mask, w, g in (("causal", 0, None), ("causal_window", 100, None), ("full", 0, None),
                       ("local_global", 64, [0, 333, 699])):
        a = attn.fwd(q, k, v, mask=mask, window=w, global_idx=g)
        b = attn.fwd_ex(q, k, v, mask=mask, window=w, global_idx=g)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), mask


@pytest.mark.gpu
def test_fwd_ex_chunked_prefill_matches_full_prefill(device):
    """Prefilling the last 512 positions as one chunk against the 1536-key
    prefix gives the last 512 rows of the full causal prefill (same key order
    and tiles, so the rows agree to the bf16 tolerance)."""
    import torch

    inp = workloads.make_inputs(1, 8, 2, 1536, 128, "bf16", seed=22)
    q, k, v = workloads.to_torch(inp, "bf16", device)
    full = attn.fwd(q, k, v, mask="causal")
    chunk = attn.fwd_ex(q[:, :, 1024:], k, v, mask="causal")
    torch.cuda.synchronize()
    err = float((full[:, :, 1024:].float() - chunk.float()).abs().max())
    assert err <= TOL["bf16"], err


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(workloads.EX_WORKLOADS))
def test_fwd_ex_workload_full_size(device, name):
    """The workloads with separate query and key lengths at full size, in the
    layout and launch configuration the benchmark times; sampled (b, head)
    pairs, sampled rows compared element-wise."""
    import torch

    w = workloads.EX_WORKLOADS[name]
    print(f"fwd_ex workload {name}", flush=True)
    inp = workloads.ex_workload_inputs(w)
    q, k, v = (place(inp[n + "_bits"], w.layout, device) for n in ("q", "k", "v"))
    o = empty_out(w.B, w.Hq, w.Sq, w.D, w.layout, device)
    slopes = w.alibi_slopes()
    table = w.distance_bias()
    q_len, kv_len = w.lengths_qkv()
    dev = lambda x: None if x is None else torch.from_numpy(x).to(device)  # noqa: E731
    attn.fwd_ex(q, k, v, mask=w.mask, window=w.window, scale=w.scale, out=o,
                alibi_slopes=dev(slopes), q_len=dev(q_len), kv_len=dev(kv_len),
                global_idx=list(w.global_idx) or None, dist_bias=dev(table))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    rng = np.random.default_rng(w.seed + 5)
    rows = sorted({0, 1, 127, 128, w.Sq // 2, w.Sq - 1}
                  | {int(x) for x in rng.integers(w.Sq, size=10)}
                  | {int(g) for g in w.global_idx if g < w.Sq})
    G = w.Hq // w.Hkv
    for b, a in {(0, 0), (w.B - 1, w.Hq - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hq)))}:
        h = a // G
        ref = oracle.cross_attention(
            inp["q"][b:b + 1, a:a + 1], inp["k"][b:b + 1, h:h + 1], inp["v"][b:b + 1, h:h + 1],
            w.mask, w.window, scale=w.scale, rows=rows,
            alibi_slopes=None if slopes is None else slopes[a:a + 1].astype(np.float64),
            q_len=None if q_len is None else q_len[b:b + 1],
            kv_len=None if kv_len is None else kv_len[b:b + 1], global_idx=w.global_idx,
            dist_bias=None if table is None else table[a:a + 1])
        err = float(np.max(np.abs(got[b, a, rows].astype(np.float64) - ref[0, 0])))
        print(f"{name} b={b} a={a}: max abs err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], (b, a, err)


# ----------------------------------------------------------------------------
# host-only validation (fake aligned addresses, never dereferenced)
# ----------------------------------------------------------------------------

def ex_status(**kw):
    a = attn.FwdArgs()
    a.alibi_slopes, a.q_len, a.kv_len, a.global_idx, a.n_global = None, None, None, None, 0
    a.dist_bias = None
    base = 0x1000000
    a.q, a.k, a.v, a.o = base, base * 3, base * 5, base * 7
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = 1, 8, 2, 100, 300, 128
    dense = lambda H, S: [H * S * 128, S * 128, 128]  # noqa: E731
    a.q_stride[:] = dense(8, 100)
    a.k_stride[:] = dense(2, 300)
    a.v_stride[:] = dense(2, 300)
    a.o_stride[:] = dense(8, 100)
    a.mask_kind, a.window, a.scale, a.dtype = 1, 0, 0.1, attn.DTYPE_BF16
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return attn.status_string(attn.fwd_ex_raw(a, 0))


def test_fwd_ex_rejects_bad_arguments():
    assert ex_status(q=0) == "ATTN_ERR_NULL"
    assert ex_status(Sq=0) == "ATTN_ERR_SHAPE"
    assert ex_status(Skv=0) == "ATTN_ERR_SHAPE"
    assert ex_status(Hq=6, Hkv=4) == "ATTN_ERR_HEADS"
    assert ex_status(D=96) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(dtype=attn.DTYPE_FP32) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(mask_kind=4) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(mask_kind=3, alibi_slopes=0x2000000) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(mask_kind=3, block_layout=0x2000000) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(mask_kind=3, window=-1) == "ATTN_ERR_WINDOW"
    assert ex_status(mask_kind=3, Sq=1 << 29, Skv=1 << 29) == "ATTN_ERR_SHAPE"
    g = (ctypes.c_int * 65)(*range(65))
    gp = ctypes.cast(g, ctypes.c_void_p).value
    assert ex_status(mask_kind=1, global_idx=gp, n_global=1) == "ATTN_ERR_GLOBAL"
    assert ex_status(mask_kind=3, global_idx=None, n_global=1) == "ATTN_ERR_GLOBAL"
    assert ex_status(mask_kind=3, global_idx=gp, n_global=65) == "ATTN_ERR_GLOBAL"
    assert ex_status(mask_kind=3, global_idx=gp, n_global=-1) == "ATTN_ERR_GLOBAL"
    big = (ctypes.c_int * 2)(5, 300)  # 300 is not a key position when Skv = 300
    assert ex_status(mask_kind=3, global_idx=ctypes.cast(big, ctypes.c_void_p).value,
                     n_global=2) == "ATTN_ERR_GLOBAL"
    assert ex_status(mask_kind=2, window=0) == "ATTN_ERR_WINDOW"
    assert ex_status(scale=float("inf")) == "ATTN_ERR_SCALE"
    assert ex_status(q=0x1000008) == "ATTN_ERR_ALIGN"
    assert ex_status(k_stride=[2 * 300 * 128, 300 * 128, 132]) == "ATTN_ERR_ALIGN"
    assert ex_status(k_stride=[2 * 300 * 128, 300 * 128, -128]) == "ATTN_ERR_ALIGN"
    assert ex_status(v_stride=[0, 0, (1 << 23) + 8]) == "ATTN_ERR_SHAPE"
    assert ex_status(o=0x1000000) == "ATTN_ERR_ALIAS"                  # o over q
    assert ex_status(o_stride=[8 * 100 * 128, 100 * 128, 64]) == "ATTN_ERR_ALIAS"  # rows overlap
    assert ex_status(alibi_slopes=0x2000002) == "ATTN_ERR_ALIGN"
    assert ex_status(q_len=0x2000001) == "ATTN_ERR_ALIGN"
    assert ex_status(kv_len=0x2000003) == "ATTN_ERR_ALIGN"
    assert ex_status(alibi_slopes=0x2000000, scale=1e-30) == "ATTN_ERR_SCALE"
    assert ex_status(alibi_slopes=0x7000000 + 64) == "ATTN_ERR_ALIAS"  # slopes inside o
    assert ex_status(kv_len=0x7000000) == "ATTN_ERR_ALIAS"             # lengths inside o
    # distance bias: general masks only, not with ALiBi or a layout
    assert ex_status(dist_bias=0x2000000, mask_kind=3) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(dist_bias=0x2000000, alibi_slopes=0x3000000) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(dist_bias=0x2000000, block_layout=0x3000000) == "ATTN_ERR_UNSUPPORTED"
    assert ex_status(dist_bias=0x2000002) == "ATTN_ERR_ALIGN"
    assert ex_status(dist_bias=0x2000000, scale=1e-30) == "ATTN_ERR_SCALE"
    assert ex_status(dist_bias=0x7000000 + 4096) == "ATTN_ERR_ALIAS"  # table inside o
    assert ex_status(dist_bias=0x6FFFF00) == "ATTN_ERR_ALIAS"         # table runs into o
    assert ex_status(dist_bias=0x2000000, Sq=1 << 28, Skv=(1 << 28) + 1,
                     q_stride=[0, 0, 128], o_stride=[0, 0, 128]) == "ATTN_ERR_SHAPE"
