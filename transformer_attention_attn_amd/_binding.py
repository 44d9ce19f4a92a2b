"""ctypes binding of libattn.so (argument marshalling only).

Every step of the attention forward runs inside the library's HIP kernels;
torch only provides device memory and the stream.  If the library is missing
this module raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

MASK_FULL, MASK_CAUSAL, MASK_CAUSAL_WINDOW, MASK_LOCAL_GLOBAL = 0, 1, 2, 3
DTYPE_FP32, DTYPE_BF16, DTYPE_FP8, DTYPE_FP8_E5M2 = 0, 1, 2, 3
MAX_GLOBAL = 64

MASKS = {
    "full": MASK_FULL,
    "causal": MASK_CAUSAL,
    "causal_window": MASK_CAUSAL_WINDOW,
    "local_global": MASK_LOCAL_GLOBAL,
}

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_HEADS",
    4: "ATTN_ERR_UNSUPPORTED", 5: "ATTN_ERR_WINDOW", 6: "ATTN_ERR_GLOBAL",
    7: "ATTN_ERR_ALIGN", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_ALIAS", 10: "ATTN_ERR_SCALE",
    11: "ATTN_ERR_WORKSPACE",
    12: "ATTN_ERR_SCRATCH",
}

EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_plan", "attn_decode", "attn_decode_workspace",
           "attn_decode_noalloc",
           "attn_layout_strided", "attn_layout_fixed", "attn_layout_bigbird",
           "attn_status_string", "attn_version")

SPARSE_BLOCK = 64          # positions per block of a block-sparse layout
SPARSE_MAX_BLOCKS = 512    # longest block-sparse sequence: 32768 positions


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"attn call failed: {STATUS.get(status, status)}")


class FwdArgs(ctypes.Structure):
    """attn_fwd_args of include/attn.h."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int),
        ("Sq", ctypes.c_int), ("Skv", ctypes.c_int), ("D", ctypes.c_int),
        ("q_stride", ctypes.c_longlong * 3), ("k_stride", ctypes.c_longlong * 3),
        ("v_stride", ctypes.c_longlong * 3), ("o_stride", ctypes.c_longlong * 3),
        ("mask_kind", ctypes.c_int), ("window", ctypes.c_int),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
        ("alibi_slopes", ctypes.c_void_p), ("q_len", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p), ("block_layout", ctypes.c_void_p),
        ("global_idx", ctypes.c_void_p), ("n_global", ctypes.c_int),
        ("dist_bias", ctypes.c_void_p),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("work_items", ctypes.c_longlong),
        ("tile_visits", ctypes.c_longlong),
        ("partial_tiles", ctypes.c_longlong),
        ("visible_pairs", ctypes.c_longlong),
        ("effective_flops", ctypes.c_double),
        ("rows_per_item", ctypes.c_int),
        ("heads_per_item", ctypes.c_int),
        ("keys_per_tile", ctypes.c_int),
        ("kernel", ctypes.c_int),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (built by transformer_attention_attn_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m transformer_attention_attn_amd.build`")
    lib = ctypes.CDLL(path)
    i, p, f = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.attn_fwd.argtypes = [p, p, p, p, i, i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int), i,
                             f, i, p]
    lib.attn_fwd.restype = i
    lib.attn_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int), i, i,
                              ctypes.POINTER(PlanInfo)]
    lib.attn_plan.restype = i
    lib.attn_fwd_ex.argtypes = [ctypes.POINTER(FwdArgs), p]
    lib.attn_fwd_ex.restype = i
    lib.attn_decode.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p, ctypes.c_size_t, p]
    lib.attn_decode.restype = i
    lib.attn_decode_workspace.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_decode_workspace.restype = i
    lib.attn_decode_noalloc.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p]
    lib.attn_decode_noalloc.restype = i
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.attn_layout_strided.argtypes = [i, i, i, u32p]
    lib.attn_layout_strided.restype = i
    lib.attn_layout_fixed.argtypes = [i, i, u32p]
    lib.attn_layout_fixed.restype = i
    lib.attn_layout_bigbird.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_int), i, u32p]
    lib.attn_layout_bigbird.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i
    _lib = lib
    return lib


def check_devices(q, **tensors) -> None:
    """Raise ValueError unless q and every given tensor (None entries are
    skipped) is a GPU tensor on q's device.  Runs before every launch: a host
    pointer, or one on another GPU, must never reach a kernel."""
    if not getattr(q, "is_cuda", False):
        raise ValueError("q must be a GPU tensor")
    for name, t in tensors.items():
        if t is None:
            continue
        if not getattr(t, "is_cuda", False) or t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on q's device ({q.device})")


def _mask_id(mask) -> int:
    if isinstance(mask, str):
        return MASKS[mask]
    return int(mask)


def _globals(global_idx: Optional[Sequence[int]]):
    if global_idx is None:
        return None, 0
    vals = [int(x) for x in global_idx]
    arr = (ctypes.c_int * max(1, len(vals)))(*vals)
    return arr, len(vals)


def fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, Hq: int, Hkv: int, S: int,
            D: int, mask, window: int, global_idx, scale: float, dtype: int, stream: int) -> int:
    """Direct call of attn_fwd with raw device addresses; returns the status."""
    lib = load()
    garr, ng = _globals(global_idx)
    return lib.attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, S, D, _mask_id(mask), window,
                        garr, ng, float(scale), dtype, stream)


def fwd(q, k, v, mask="causal", window: int = 0, global_idx=None, scale: Optional[float] = None,
        out=None, stream=None):
    """Attention forward on torch device tensors.

    q: [B, Hq, S, D], k, v: [B, Hkv, S, D], contiguous, bf16, fp32 or FP8
    (torch.float8_e4m3fn or torch.float8_e5m2 codes; the output is then
    bf16), on the GPU.
    Returns o shaped like q (allocated with torch unless `out` is given).
    The kernel runs on `stream` (default: torch's current stream).
    """
    import torch

    if q.dtype == torch.bfloat16:
        dt, odt = DTYPE_BF16, torch.bfloat16
    elif q.dtype == torch.float32:
        dt, odt = DTYPE_FP32, torch.float32
    elif q.dtype == torch.float8_e4m3fn:
        dt, odt = DTYPE_FP8, torch.bfloat16
    elif q.dtype == torch.float8_e5m2:
        dt, odt = DTYPE_FP8_E5M2, torch.bfloat16
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors of one dtype")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(v.shape) != (B, Hkv, S, D):
        raise ValueError("k, v must be [B, Hkv, S, D] matching q")
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    elif out.shape != q.shape or out.dtype != odt or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {odt} tensor shaped like q")
    check_devices(q, k=k, v=v, out=out)
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, D,
                     mask, window, global_idx, scale, dt, handle)
    if st != 0:
        raise AttnError(st)
    return out


def fwd_ex_raw(args: FwdArgs, stream: int) -> int:
    """Direct call of attn_fwd_ex; returns the status."""
    return load().attn_fwd_ex(ctypes.byref(args), stream)


def layout_words(nb: int) -> int:
    return (nb + 31) // 32


def _layout_call(fn, nb, *args):
    import numpy as np

    out = np.zeros((max(nb, 0), layout_words(max(nb, 0))), dtype=np.uint32)
    st = fn(nb, *args, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
    if st != 0:
        raise AttnError(st)
    return out


def layout_strided(nb: int, local_blocks: int, stride_blocks: int):
    """attn_layout_strided: [nb, words] uint32 bitmask of the strided pattern."""
    return _layout_call(load().attn_layout_strided, nb, local_blocks, stride_blocks)


def layout_fixed(nb: int, chunk_blocks: int):
    """attn_layout_fixed: [nb, words] uint32 bitmask of the fixed pattern."""
    return _layout_call(load().attn_layout_fixed, nb, chunk_blocks)


def layout_bigbird(nb: int, radius_blocks: int, n_global_blocks: int, rand_blocks):
    """attn_layout_bigbird: rand_blocks is an [nb, r] integer array (r may be 0)."""
    import numpy as np

    rb = np.ascontiguousarray(np.asarray(rand_blocks, dtype=np.int32).reshape(max(nb, 0), -1))
    return _layout_call(load().attn_layout_bigbird, nb, radius_blocks, n_global_blocks,
                        rb.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), rb.shape[1])


def fwd_ex(q, k, v, mask="causal", window: int = 0, scale: Optional[float] = None, out=None,
           stream=None, alibi_slopes=None, q_len=None, kv_len=None, block_layout=None,
           global_idx=None, dist_bias=None):
    """Forward pass with Sq != Skv and strided layouts (bf16).

    q: [B, Hq, Sq, D], k, v: [B, Hkv, Skv, D] as torch views of any strides
    whose last dimension is contiguous (e.g. a [B, S, H, D] tensor passed as
    x.transpose(1, 2)).  Queries are aligned to the end of the keys (query i at
    key position i + Skv - Sq).  Returns o shaped like q (a dense tensor unless
    `out` is given, which may be strided too).  Optional GPU tensors:
    alibi_slopes float32 [Hq] (ALiBi), q_len and kv_len int32 [B] (valid rows
    and keys per sequence of a right-padded batch; padded rows come out zero),
    block_layout int32 [nb, words] (a layout_* bitmask on the GPU: block-sparse
    attention over blocks of 64 positions), dist_bias float32 [Hq, Sq + Skv - 1]
    (entry d + Skv - 1 of row a is added to head a's scaled scores at signed
    distance d = key position - query position).  global_idx: host sequence of
    global key positions for mask "local_global".
    """
    import torch

    if q.dtype != torch.bfloat16:
        raise TypeError("fwd_ex takes bf16 tensors")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_cuda or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("q, k, v must be 4-D bf16 GPU tensors with a contiguous last dim")
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Skv, D) or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError("k, v must be [B, Hkv, Skv, D] matching q")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (B, Hq, Sq, D) or out.dtype != q.dtype or out.stride(3) != 1:
        raise ValueError("out must be shaped like q with a contiguous last dim")
    check_devices(q, k=k, v=v, out=out, alibi_slopes=alibi_slopes, q_len=q_len,
                  kv_len=kv_len, block_layout=block_layout, dist_bias=dist_bias)
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    a = FwdArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    a.mask_kind, a.window, a.scale, a.dtype = _mask_id(mask), int(window), float(scale), DTYPE_BF16
    nb = (Sq + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    for name, t, dt, shape in (("alibi_slopes", alibi_slopes, torch.float32, (Hq,)),
                               ("q_len", q_len, torch.int32, (B,)),
                               ("kv_len", kv_len, torch.int32, (B,)),
                               ("block_layout", block_layout, torch.int32,
                                (nb, layout_words(nb))),
                               ("dist_bias", dist_bias, torch.float32, (Hq, Sq + Skv - 1))):
        if t is None:
            setattr(a, name, None)
            continue
        if t.dtype != dt or t.device != q.device or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape} on "
                             "q's device")
        setattr(a, name, t.data_ptr())
    garr, a.n_global = _globals(global_idx)  # garr stays referenced until the call returns
    a.global_idx = ctypes.cast(garr, ctypes.c_void_p) if garr is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = fwd_ex_raw(a, handle)
    if st != 0:
        raise AttnError(st)
    return out


def plan(B: int, Hq: int, Hkv: int, S: int, D: int, mask="causal", window: int = 0,
         global_idx=None, dtype: str = "bf16") -> dict:
    """Host-only work plan of attn_fwd for these arguments (no GPU needed)."""
    lib = load()
    garr, ng = _globals(global_idx)
    info = PlanInfo()
    dt = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32, "fp8": DTYPE_FP8,
          "fp8_e5m2": DTYPE_FP8_E5M2}[dtype]
    st = lib.attn_plan(B, Hq, Hkv, S, D, _mask_id(mask), window, garr, ng, dt, ctypes.byref(info))
    if st != 0:
        raise AttnError(st)
    return info.as_dict()


def plan_status(B, Hq, Hkv, S, D, mask, window=0, global_idx=None, dtype=DTYPE_BF16) -> int:
    """Status attn_plan returns for these arguments (validation only)."""
    lib = load()
    garr, ng = _globals(global_idx)
    info = PlanInfo()
    return lib.attn_plan(B, Hq, Hkv, S, D, _mask_id(mask), window, garr, ng, dtype,
                         ctypes.byref(info))


def decode_workspace_status(B, Hq, Hkv, Sq, Smax, D, mask="causal", dtype=DTYPE_BF16, window=0):
    """(status, bytes) of attn_decode_workspace for these arguments (host only)."""
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.attn_decode_workspace(B, Hq, Hkv, Sq, Smax, D, _mask_id(mask), window, dtype,
                                   ctypes.byref(n))
    return st, int(n.value)


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Smax: int, D: int,
                           mask="causal", window: int = 0) -> int:
    """Device workspace bytes attn_decode needs (0 when it needs none)."""
    st, n = decode_workspace_status(B, Hq, Hkv, Sq, Smax, D, mask, window=window)
    if st != 0:
        raise AttnError(st)
    return n


def decode_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, len_ptr: int, B: int, Hq: int,
               Hkv: int, Sq: int, Smax: int, D: int, mask, window: int, scale: float, dtype: int,
               ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """Direct call of attn_decode with raw device addresses; returns the status."""
    return load().attn_decode(q_ptr, k_ptr, v_ptr, o_ptr, len_ptr, B, Hq, Hkv, Sq, Smax, D,
                              _mask_id(mask), window, float(scale), dtype, ws_ptr, ws_bytes,
                              stream)


def decode(q, k_cache, v_cache, cache_len=None, mask="causal", scale: Optional[float] = None,
           out=None, workspace=None, stream=None, window: int = 0):
    """Decode attention of the Sq newest positions against key/value caches.

    q: [B, Hq, Sq, D] bf16; k_cache, v_cache: [B, Hkv, Smax, D] bf16, contiguous,
    on the GPU.  cache_len: int32 GPU tensor of B lengths (None: all Smax).
    window: the w of mask "causal_window" (0 with the other masks).
    The workspace (a GPU tensor of at least decode_workspace_bytes bytes) is
    allocated with torch when not given.  Returns o shaped like q.
    """
    import torch

    if q.dtype != torch.bfloat16:
        raise TypeError("decode takes bf16 tensors")
    for t in (q, k_cache, v_cache):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q and the caches must be contiguous 4-D bf16 GPU tensors")
    B, Hq, Sq, D = q.shape
    Hkv, Smax = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Smax, D) or tuple(v_cache.shape) != (B, Hkv, Smax, D):
        raise ValueError("caches must be [B, Hkv, Smax, D] matching q")
    if cache_len is not None:
        if cache_len.dtype != torch.int32 or not cache_len.is_cuda or cache_len.numel() != B:
            raise ValueError("cache_len must be an int32 GPU tensor of B lengths")
        cache_len = cache_len.contiguous()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    need = decode_workspace_bytes(B, Hq, Hkv, Sq, Smax, D, mask, window)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    check_devices(q, k_cache=k_cache, v_cache=v_cache, out=out, cache_len=cache_len,
                  workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = decode_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                        cache_len.data_ptr() if cache_len is not None else 0, B, Hq, Hkv, Sq,
                        Smax, D, mask, window, scale, DTYPE_BF16, ws_ptr, ws_bytes, handle)
    if st != 0:
        raise AttnError(st)
    return out


def decode_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, len_ptr: int, B: int,
                       Hq: int, Hkv: int, Sq: int, Smax: int, D: int, mask, window: int,
                       scale: float, dtype: int, stream: int) -> int:
    """Direct call of attn_decode_noalloc with raw device addresses; returns the status."""
    return load().attn_decode_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, len_ptr, B, Hq, Hkv, Sq, Smax,
                                      D, _mask_id(mask), window, float(scale), dtype, stream)


def decode_noalloc(q, k_cache, v_cache, cache_len=None, mask="causal",
                   scale: Optional[float] = None, out=None, stream=None, window: int = 0):
    """decode() through attn_decode_noalloc: no workspace, the library's static
    device scratch instead (calls that may overlap on one GPU race).  `out`
    is allocated with torch when not given; pass it to allocate nothing."""
    import torch

    if q.dtype != torch.bfloat16:
        raise TypeError("decode_noalloc takes bf16 tensors")
    for t in (q, k_cache, v_cache):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q and the caches must be contiguous 4-D bf16 GPU tensors")
    B, Hq, Sq, D = q.shape
    Hkv, Smax = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Smax, D) or tuple(v_cache.shape) != (B, Hkv, Smax, D):
        raise ValueError("caches must be [B, Hkv, Smax, D] matching q")
    if cache_len is not None:
        if (cache_len.dtype != torch.int32 or not cache_len.is_cuda or cache_len.numel() != B
                or not cache_len.is_contiguous()):
            raise ValueError("cache_len must be a contiguous int32 GPU tensor of B lengths")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    check_devices(q, k_cache=k_cache, v_cache=v_cache, out=out, cache_len=cache_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = decode_noalloc_raw(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                out.data_ptr(), cache_len.data_ptr() if cache_len is not None else 0,
                                B, Hq, Hkv, Sq, Smax, D, mask, window, scale, DTYPE_BF16,
                                handle)
    if st != 0:
        raise AttnError(st)
    return out


def status_string(status: int) -> str:
    return load().attn_status_string(status).decode()


def version() -> int:
    return load().attn_version()
