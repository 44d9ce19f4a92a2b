"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic.  It is the one piece shared by the fp64 oracle's tests,
the GPU parity tests and the benchmark, so that both sides see identical
inputs.

Workloads (shapes follow the examples on the pages):

* ``causal_mha_fp32_s256``   -- causal multi-head, fp32, B=1 H=4 S=256 D=64,
  scale 1/8.
* ``causal_mha_bf16_s2048``  -- causal multi-head, bf16, B=4 H=32 S=2048 D=128.
* ``causal_gqa_bf16_s8192``  -- causal grouped-query (32 query heads over 8
  key/value heads), bf16, B=1 S=8192 D=128.
* ``window_gqa_bf16_s16384`` -- causal sliding window of 4096 keys (key j is
  visible from query i when i-4096 < j <= i), grouped-query, bf16,
  B=1 S=16384 D=128; window and length follow the Mistral and Longformer
  figures on "Transformer 演进与变体", section 稀疏注意力.
* ``local_global_bf16_s8192`` -- bidirectional band |i-j| <= 512 plus global
  tokens {0, 1000, 3000, 6000}, 12 heads, B=1 S=8192 D=64: the document example
  of "Transformer 演进与变体", section 稀疏注意力 (Longformer paragraph).
* ``causal_gqa_fp8_s8192`` -- the grouped-query workload with E4M3 inputs
  (the FP8 forward of "Transformer 演进与变体", section Flash Attention), bf16
  output.  The N(0, 1) draws are rounded to E4M3 (nearest even).
* ``causal_mha_fp8_d64_s8192`` -- E4M3 inputs at head width 64: 12 heads of
  the local+global workload's shape, B=1 S=8192, causal mask.
* ``local_global_fp8_s8192`` -- the local+global workload (window 512,
  globals {0, 1000, 3000, 6000}) with E4M3 inputs.

Decode workloads (the Sq newest positions of each sequence against its
key/value cache, "Transformer 架构及其变体", section 预填充创建缓存，解码复用缓存):

* ``decode_gqa_bf16_b16_l8192``  -- one new position per sequence, 16
  sequences with full 8192-position caches, 32 query heads over 8 key/value
  heads, D=128 (the head shapes of the grouped-query workload above).
* ``decode_gqa_bf16_b8_sq4_l16384`` -- four new positions per sequence (a
  chunk or draft tokens, causal among themselves), 8 sequences with ragged
  cache lengths drawn uniformly from [Smax/4, Smax], Smax=16384.
* ``decode_mqa_bf16_b4_l65536`` -- multi-query (one key/value head for 32
  query heads), one new position, 4 sequences with full 65536-position caches.

Workloads with separate query and key lengths (queries aligned to the end of
the keys):

* ``chunk_prefill_gqa_bf16_q2048_kv8192`` -- the last 2048 positions of an
  8192-token prompt prefilled as one chunk against the whole prefix, causal,
  the grouped-query head shapes above ("Transformer 架构及其变体", section
  预填充创建缓存，解码复用缓存).
* ``cross_mha_bf16_q1024_kv4096_bshd`` -- cross attention, 1024 decoder
  queries against 4096 encoder keys, every key visible, 16 heads of D=64, B=4,
  all tensors sequence-major ([B][S][H][D]) ("Trasformer 浅析", section
  交叉注意力; heads of 64 as in the original model's head width,
  "Transformer 演进与变体", section MHA：多头注意力).
* ``alibi_padded_mha_bf16_b8_s4096`` -- causal prefill of 8 right-padded
  sequences (valid lengths uniform in [1024, 4096]) with the ALiBi distance
  bias, 32 heads of D=128 ("Transformer 演进与变体", section 线性偏置注意力;
  "Trasformer 浅析", section 填充掩码与因果掩码).  Slopes 2^(-8 (a+1) / 32).

* ``bigbird_bf16_b4_h12_s4096`` -- Big Bird over 64-position blocks: window
  radius 1 block, 2 global blocks, 3 random blocks per query block, every
  direction visible; B=4, 12 heads of D=64, S=4096 ("第 8 章 AI 算法
  Transformer大模型", section 8.3.3 with the block-sparse form of 8.3.4).
* ``strided_causal_gqa_bf16_s8192`` -- Sparse Transformer strided pattern
  over 64-position blocks (the own block and 7 before it, plus every 8th
  block back), causal, the grouped-query head shapes above (section 8.3.1).

Values are iid N(0, 1) from ``numpy.random.default_rng(seed)``, drawn as
float32 in the order Q, K, V, each shaped [B][H][S][D].  bf16 workloads round
those draws to nearest-even bf16; the rounded values are what every consumer
(kernel and oracle) sees.
"""
from __future__ import annotations

import dataclasses
from typing import Tuple

import numpy as np

MASK_FULL = "full"
MASK_CAUSAL = "causal"
MASK_CAUSAL_WINDOW = "causal_window"
MASK_LOCAL_GLOBAL = "local_global"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    dtype: str  # "fp32", "bf16" or "fp8" (E4M3 inputs, bf16 output)
    mask: str
    window: int = 0
    global_idx: Tuple[int, ...] = ()
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["global_idx"] = list(self.global_idx)
        return d


WORKLOADS = {
    w.name: w
    for w in (
        Workload("causal_mha_fp32_s256", 1, 4, 4, 256, 64, "fp32", MASK_CAUSAL, seed=1),
        Workload("causal_mha_bf16_s2048", 4, 32, 32, 2048, 128, "bf16", MASK_CAUSAL, seed=2),
        Workload("causal_gqa_bf16_s8192", 1, 32, 8, 8192, 128, "bf16", MASK_CAUSAL, seed=3),
        Workload("window_gqa_bf16_s16384", 1, 32, 8, 16384, 128, "bf16", MASK_CAUSAL_WINDOW,
                 window=4096, seed=4),
        Workload("local_global_bf16_s8192", 1, 12, 12, 8192, 64, "bf16", MASK_LOCAL_GLOBAL,
                 window=512, global_idx=(0, 1000, 3000, 6000), seed=5),
        Workload("causal_gqa_fp8_s8192", 1, 32, 8, 8192, 128, "fp8", MASK_CAUSAL, seed=14),
        # FP8 at head width 64 (the local+global workload's heads, causal mask)
        Workload("causal_mha_fp8_d64_s8192", 1, 12, 12, 8192, 64, "fp8", MASK_CAUSAL, seed=17),
        # the local+global workload with E4M3 inputs
        Workload("local_global_fp8_s8192", 1, 12, 12, 8192, 64, "fp8", MASK_LOCAL_GLOBAL,
                 window=512, global_idx=(0, 1000, 3000, 6000), seed=18),
    )
}

# The workload the headline throughput is quoted on.
HEADLINE = "causal_gqa_bf16_s8192"


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Smax: int
    D: int
    mask: str      # "causal", "full" or "causal_window"
    lengths: str   # "full": every cache holds Smax positions; "ragged": seeded in [Smax/4, Smax]
    seed: int = 0
    dtype: str = "bf16"
    window: int = 0  # the w of "causal_window"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def cache_len(self) -> np.ndarray:
        if self.lengths == "full":
            return np.full(self.B, self.Smax, dtype=np.int32)
        rng = np.random.default_rng(self.seed + 1000)
        return rng.integers(self.Smax // 4, self.Smax + 1, size=self.B).astype(np.int32)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["cache_len"] = [int(x) for x in self.cache_len()]
        return d


DECODE_WORKLOADS = {
    w.name: w
    for w in (
        DecodeWorkload("decode_gqa_bf16_b16_l8192", 16, 32, 8, 1, 8192, 128, MASK_CAUSAL, "full",
                       seed=6),
        DecodeWorkload("decode_gqa_bf16_b8_sq4_l16384", 8, 32, 8, 4, 16384, 128, MASK_CAUSAL,
                       "ragged", seed=7),
        DecodeWorkload("decode_mqa_bf16_b4_l65536", 4, 32, 1, 1, 65536, 128, MASK_CAUSAL, "full",
                       seed=8),
        # a 4096-position sliding window (Mistral's, "Transformer 演进与变体", section
        # 稀疏注意力) over caches of 8192 to 32768 positions
        DecodeWorkload("decode_window_gqa_bf16_b16_w4096_l32768", 16, 32, 8, 1, 32768, 128,
                       MASK_CAUSAL_WINDOW, "ragged", seed=9, window=4096),
    )
}
DECODE_HEADLINE = "decode_gqa_bf16_b16_l8192"


@dataclasses.dataclass(frozen=True)
class ExWorkload:
    """A call of the entry point with separate query and key lengths and
    strided layouts: Sq queries aligned to the end of Skv keys."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    mask: str      # "full", "causal" or "causal_window"
    layout: str    # "bhsd" (head-major) or "bshd" (sequence-major) for q, k, v and o
    window: int = 0
    seed: int = 0
    dtype: str = "bf16"
    alibi: bool = False   # ALiBi with the slopes of alibi_slopes()
    lengths: str = "full"  # "full", or "ragged": per-sequence lengths of lengths()
    # block-sparse pattern over 64-position blocks: "" (none), "strided" (args:
    # local, stride), "fixed" (chunk) or "bigbird" (radius, n_global, n_random)
    pattern: str = ""
    pattern_args: Tuple[int, ...] = ()
    global_idx: Tuple[int, ...] = ()  # local_global: global key positions
    dist_bias: bool = False  # a distance-bias table, that of distance_bias()

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def alibi_slopes(self):
        """Hq slopes (float32) when alibi is set, else None."""
        return make_alibi_slopes(self.Hq) if self.alibi else None

    def distance_bias(self):
        """The [Hq][Sq + Skv - 1] float32 distance-bias table when dist_bias is
        set, else None."""
        return make_distance_bias(self.Hq, self.Sq, self.Skv, self.seed) if self.dist_bias else None

    def n_blocks(self) -> int:
        return -(-self.Sq // SPARSE_BLOCK)

    def rand_blocks(self) -> np.ndarray:
        """Big Bird's random key blocks, [nb][n_random] (an input of the pattern)."""
        if self.pattern != "bigbird":
            raise ValueError("only the bigbird pattern draws random blocks")
        return make_rand_blocks(self.n_blocks(), self.pattern_args[2], self.seed)

    def lengths_qkv(self):
        """(q_len, kv_len) int32 arrays of B valid lengths, or (None, None)."""
        if self.lengths == "full":
            return None, None
        return make_ragged_lengths(self.B, self.Sq, self.Skv, self.seed)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["pattern_args"] = list(self.pattern_args)
        d["global_idx"] = list(self.global_idx)
        ql, kl = self.lengths_qkv()
        if ql is not None:
            d["q_len"], d["kv_len"] = [int(x) for x in ql], [int(x) for x in kl]
        return d


EX_WORKLOADS = {
    w.name: w
    for w in (
        # the last 2048 positions of an 8192-token prompt prefilled as one chunk
        ExWorkload("chunk_prefill_gqa_bf16_q2048_kv8192", 1, 32, 8, 2048, 8192, 128, MASK_CAUSAL,
                   "bhsd", seed=9),
        # decoder queries against a longer encoder sequence, sequence-major tensors
        ExWorkload("cross_mha_bf16_q1024_kv4096_bshd", 4, 16, 16, 1024, 4096, 64, MASK_FULL,
                   "bshd", seed=10),
        # causal prefill of a right-padded batch with ALiBi instead of positions in q/k
        ExWorkload("alibi_padded_mha_bf16_b8_s4096", 8, 32, 32, 4096, 4096, 128, MASK_CAUSAL,
                   "bhsd", seed=11, alibi=True, lengths="ragged"),
        # the same padded causal prefill with a bucketed relative-position bias
        # per head (one learned value per distance bucket) instead of ALiBi
        ExWorkload("relbias_padded_mha_bf16_b8_s4096", 8, 32, 32, 4096, 4096, 128, MASK_CAUSAL,
                   "bhsd", seed=15, lengths="ragged", dist_bias=True),
        # Big Bird: window of 3 blocks, 2 global blocks, 3 random blocks per row
        ExWorkload("bigbird_bf16_b4_h12_s4096", 4, 12, 12, 4096, 4096, 64, MASK_FULL, "bhsd",
                   seed=12, pattern="bigbird", pattern_args=(1, 2, 3)),
        # Sparse Transformer strided pattern on the grouped-query head shapes
        ExWorkload("strided_causal_gqa_bf16_s8192", 1, 32, 8, 8192, 8192, 128, MASK_CAUSAL,
                   "bhsd", seed=13, pattern="strided", pattern_args=(7, 8)),
        # Longformer ("Transformer 演进与变体", section 稀疏注意力: 8192 tokens, a
        # 512-position window, globals at 0, 1000, 3000, 6000) over a right-padded
        # batch of four sequences, sequence-major tensors
        ExWorkload("longformer_padded_bf16_b4_s8192_bshd", 4, 12, 12, 8192, 8192, 64,
                   MASK_LOCAL_GLOBAL, "bshd", window=512, seed=14, lengths="ragged",
                   global_idx=(0, 1000, 3000, 6000)),
    )
}

SPARSE_BLOCK = 64  # positions per block of the block-sparse patterns


def make_rand_blocks(nb: int, r: int, seed: int) -> np.ndarray:
    """r random key blocks per query block, uniform over [0, nb), drawn with
    default_rng(seed + 3000) (Big Bird's random connections; the pages fix no
    generator, so the draw is an input shared by both sides)."""
    rng = np.random.default_rng(seed + 3000)
    return rng.integers(0, nb, size=(nb, r)).astype(np.int32)


def make_alibi_slopes(H: int) -> np.ndarray:
    """Synthetic per-head ALiBi slopes: the geometric sequence 2^(-8 (a+1) / H),
    a = 0..H-1 (the pages fix no slope values; this is an input recipe)."""
    return np.exp2(-8.0 * (np.arange(H, dtype=np.float64) + 1.0) / H).astype(np.float32)


def make_distance_bias(Hq: int, Sq: int, Skv: int, seed: int, buckets: int = 32,
                       max_distance: int = 128) -> np.ndarray:
    """Synthetic distance-bias table, float32 [Hq][Sq + Skv - 1]: entry
    d + Skv - 1 of row a holds the value of the bucket of the signed distance
    d, as a learned relative-position bias would (the pages fix no values;
    this is an input recipe).  Half the buckets serve d < 0, half d >= 0;
    within each half, |d| < 8 get a bucket each, longer distances share
    log-spaced buckets up to max_distance, beyond which all share the last.
    Bucket values are N(0, 1.5^2) from default_rng(seed + 3000)."""
    rng = np.random.default_rng(seed + 3000)
    vals = rng.standard_normal((Hq, buckets)) * 1.5
    half = buckets // 2
    exact = half // 2
    d = np.arange(Sq + Skv - 1, dtype=np.int64) - (Skv - 1)
    n = np.abs(d)
    logb = exact + np.floor(np.log(np.maximum(n, 1) / exact) / np.log(max_distance / exact)
                            * (half - exact)).astype(np.int64)
    b = np.where(n < exact, n, np.minimum(logb, half - 1)) + np.where(d >= 0, half, 0)
    return np.ascontiguousarray(vals[:, b], dtype=np.float32)


def make_ragged_lengths(B: int, Sq: int, Skv: int, seed: int):
    """Per-sequence valid lengths of a right-padded batch, drawn uniformly from
    [Skv/4, Skv] for the keys with default_rng(seed + 2000); the query count is
    the same number shifted by Sq - Skv (clamped to [0, Sq]), so a square batch
    (Sq == Skv) has q_len == kv_len."""
    rng = np.random.default_rng(seed + 2000)
    kv = rng.integers(Skv // 4, Skv + 1, size=B)
    q = np.clip(kv - (Skv - Sq), 0, Sq)
    return q.astype(np.int32), kv.astype(np.int32)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bit patterns.

    Inputs are finite normal draws, so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw(shape, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _fp8_torch_dtype(dtype: str):
    import torch

    return {"fp8": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2}[dtype]


def e4m3_codes(x: np.ndarray, dtype: str = "fp8") -> np.ndarray:
    """Round float32 values to the nearest E4M3 value (ties to even, OCP
    format; or E5M2 for dtype "fp8_e5m2") with torch's own conversion; return
    the uint8 codes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_fp8_torch_dtype(dtype)).view(torch.uint8).numpy().copy()


def make_inputs(B, Hq, Hkv, S, D, dtype, seed):
    """Return dict with float32 arrays 'q','k','v' holding the values the kernel sees,
    plus (for bf16) the uint16 bit patterns under 'q_bits','k_bits','v_bits' or
    (for fp8, fp8_e5m2) the E4M3 / E5M2 codes under 'q_codes','k_codes','v_codes'."""
    rng = np.random.default_rng(seed)
    q = draw((B, Hq, S, D), rng)
    k = draw((B, Hkv, S, D), rng)
    v = draw((B, Hkv, S, D), rng)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        if dtype == "bf16":
            bits = bf16_round_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_float(bits)
        elif dtype in ("fp8", "fp8_e5m2"):
            codes = e4m3_codes(x, dtype)
            out[name + "_codes"] = codes
            out[name] = codes_to_float(codes, dtype)
        elif dtype == "fp32":
            out[name] = x
        else:
            raise ValueError(f"unknown dtype {dtype!r}")
    return out


def make_trend_inputs(B, Hq, Hkv, S, D, dtype, seed, pattern, amp=16.0):
    """make_inputs with a planted trend in the scores along the key index, for
    the running-maximum paths of the kernels: every query gets +amp in
    dimension 0, and dimension 0 of the keys is amp * t for t rising or
    falling linearly over [-1, 1] ('rising', 'falling'), or amp * (1 + 4 r) at
    the r-th of a few random positions ('spikes', each far above the last).
    Quantised like make_inputs."""
    rng = np.random.default_rng(seed)
    q = draw((B, Hq, S, D), rng)
    k = draw((B, Hkv, S, D), rng)
    v = draw((B, Hkv, S, D), rng)
    q[..., 0] += np.float32(amp)
    t = np.linspace(-1.0, 1.0, S, dtype=np.float32)
    if pattern == "rising":
        k[..., 0] = np.float32(amp) * t
    elif pattern == "falling":
        k[..., 0] = -np.float32(amp) * t
    elif pattern == "spikes":
        pos = np.sort(rng.choice(S, size=max(1, S // 97), replace=False))
        k[..., pos, 0] = np.float32(amp) * (1 + 4 * np.arange(len(pos), dtype=np.float32))
    else:
        raise ValueError(f"unknown pattern {pattern!r}")
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        if dtype == "bf16":
            bits = bf16_round_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_float(bits)
        elif dtype in ("fp8", "fp8_e5m2"):
            codes = e4m3_codes(x, dtype)
            out[name + "_codes"] = codes
            out[name] = codes_to_float(codes, dtype)
        else:
            raise ValueError(f"unknown dtype {dtype!r}")
    return out


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.Hq, w.Hkv, w.S, w.D, w.dtype, w.seed)


def make_decode_inputs(B, Hq, Hkv, Sq, Smax, D, seed):
    """bf16 decode inputs: q [B][Hq][Sq][D] and caches [B][Hkv][Smax][D], drawn in
    the order Q, K, V; same dict layout as make_inputs."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (B, Hq, Sq, D)), ("k", (B, Hkv, Smax, D)), ("v", (B, Hkv, Smax, D))):
        bits = bf16_round_bits(draw(shape, rng))
        out[name + "_bits"] = bits
        out[name] = bf16_bits_to_float(bits)
    return out


def decode_workload_inputs(w: DecodeWorkload):
    return make_decode_inputs(w.B, w.Hq, w.Hkv, w.Sq, w.Smax, w.D, w.seed)


def ex_workload_inputs(w: ExWorkload):
    """q [B][Hq][Sq][D], k and v [B][Hkv][Skv][D]: the decode generator with the
    cache capacity set to Skv (same draw order)."""
    return make_decode_inputs(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.seed)


def codes_to_float(codes: np.ndarray, dtype: str = "fp8") -> np.ndarray:
    """E4M3 (or, for "fp8_e5m2", E5M2) codes widened exactly to float32
    (torch's decoding)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes)).view(_fp8_torch_dtype(dtype)).float() \
        .numpy()


def to_torch(inputs: dict, dtype: str, device):
    """Move generated inputs into torch tensors of the kernel dtype (no arithmetic)."""
    import torch

    res = []
    for name in ("q", "k", "v"):
        if dtype == "bf16":
            t = torch.from_numpy(inputs[name + "_bits"].view(np.int16)).view(torch.bfloat16)
        elif dtype in ("fp8", "fp8_e5m2"):
            t = torch.from_numpy(inputs[name + "_codes"]).view(_fp8_torch_dtype(dtype))
        else:
            t = torch.from_numpy(inputs[name])
        res.append(t.to(device).contiguous())
    return tuple(res)
