"""Host logic of the benchmark (CPU only): its FLOP and byte counts agree with
the oracle's independent counts, and it refuses more than one GPU."""
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workloads
from oracle import cross as cr


@pytest.mark.parametrize("name", list(workloads.DECODE_WORKLOADS))
def test_decode_counts_match_oracle(name):
    w = workloads.DECODE_WORKLOADS[name]
    lens = w.cache_len()
    nbytes, flops = bench.decode_counts(w, lens)
    assert nbytes == oracle.decode_cache_bytes(w.B, w.Hkv, w.D, lens, 2, Sq=w.Sq, kind=w.mask,
                                               window=w.window)
    assert flops == oracle.decode_effective_flops(w.Hq, w.Sq, w.D, lens, w.mask, w.window)


@pytest.mark.parametrize("mask,window", [("causal", 0), ("full", 0), ("causal_window", 1),
                                         ("causal_window", 3), ("causal_window", 50)])
def test_decode_counts_short_caches(mask, window):
    """Lengths of zero, below the number of new positions, and below and
    above the window."""
    w = workloads.DecodeWorkload("t", 7, 8, 2, 4, 64, 64, mask, "full", window=window)
    lens = [0, 1, 3, 4, 6, 52, 64]
    nbytes, flops = bench.decode_counts(w, lens)
    assert flops == oracle.decode_effective_flops(w.Hq, w.Sq, w.D, lens, mask, window)
    assert nbytes == oracle.decode_cache_bytes(w.B, w.Hkv, w.D, lens, 2, Sq=w.Sq, kind=mask,
                                               window=window)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (5, 3), (3, 5), (64, 1000), (300, 100)])
@pytest.mark.parametrize("mask,window", [("full", 0), ("causal", 0), ("causal_window", 1),
                                         ("causal_window", 37)])
def test_ex_pairs_match_oracle(Sq, Skv, mask, window):
    assert bench.ex_visible_pairs(Sq, Skv, mask, window) == cr.cross_visible_pairs(
        Sq, Skv, mask, window)


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (5, 3), (3, 5), (64, 1000), (300, 100), (700, 700)])
@pytest.mark.parametrize("window,g", [(0, ()), (2, (0,)), (37, (1, 2, 60, 299, 699)),
                                      (1000, (5,))])
def test_ex_local_global_pairs_match_oracle(Sq, Skv, window, g):
    assert bench.ex_visible_pairs(Sq, Skv, "local_global", window, g) == cr.cross_visible_pairs(
        Sq, Skv, "local_global", window, g)


@pytest.mark.parametrize("name", list(workloads.EX_WORKLOADS))
def test_ex_workload_flops(name):
    w = workloads.EX_WORKLOADS[name]
    if w.pattern:
        from oracle import sparse as sp

        nb = w.n_blocks()
        lay = (sp.strided_layout(nb, *w.pattern_args) if w.pattern == "strided" else
               sp.fixed_layout(nb, *w.pattern_args) if w.pattern == "fixed" else
               sp.bigbird_layout(nb, w.pattern_args[0], w.pattern_args[1], w.rand_blocks()))
        pairs = sp.block_sparse_pairs(w.Sq, lay, 64, w.mask == "causal") * w.B
        assert bench.ex_effective_flops(w) == 4.0 * w.D * pairs * w.Hq
        return
    q_len, kv_len = w.lengths_qkv()
    pairs = 0
    for b in range(w.B):
        pairs += cr.cross_visible_pairs(w.Sq if q_len is None else int(q_len[b]),
                                        w.Skv if kv_len is None else int(kv_len[b]),
                                        w.mask, w.window, w.global_idx)
    assert bench.ex_effective_flops(w) == 4.0 * w.D * pairs * w.Hq


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_max_abs_err():
    assert bench.max_abs_err(np.array([1.0, 2.0]), np.array([1.5, 2.0])) == 0.5


@pytest.mark.parametrize("S", [64, 100, 1000, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_layout_pairs_match_oracle(S, causal):
    """The bench's pair count of a block-sparse layout equals the oracle's."""
    from oracle import sparse as sp

    nb = sp.n_blocks(S, 64)
    rng = np.random.default_rng(S)
    lay = rng.random((nb, nb)) < 0.3
    words = np.zeros((nb, (nb + 31) // 32), dtype=np.uint32)
    for I in range(nb):
        for J in np.nonzero(lay[I])[0]:
            words[I, J // 32] |= np.uint32(1) << np.uint32(J % 32)
    assert bench.layout_pairs(words, S, causal) == sp.block_sparse_pairs(S, lay, 64, causal)


def test_distance_bias_recipe():
    """The bucketed distance-bias input: per-head rows over d = -(Skv-1) ..
    Sq-1, one value per distance below 8 on each side, shared log buckets
    further out, a single value past the maximum distance on each side."""
    import numpy as np

    Sq, Skv, Hq = 300, 700, 3
    t = workloads.make_distance_bias(Hq, Sq, Skv, seed=4)
    assert t.shape == (Hq, Sq + Skv - 1) and t.dtype == np.float32 and t.flags["C_CONTIGUOUS"]
    at = lambda d: t[:, d + Skv - 1]  # noqa: E731
    near = [tuple(at(d)) for d in range(-7, 8)]
    assert len(set(near)) == 15  # distinct buckets for |d| < 8 on either side (and 0)
    assert np.array_equal(at(200), at(Sq - 1)) and np.array_equal(at(-200), at(-(Skv - 1)))
    assert not np.array_equal(at(200), at(-200))
    assert np.array_equal(workloads.make_distance_bias(Hq, Sq, Skv, seed=4), t)
