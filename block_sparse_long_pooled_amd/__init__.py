"""MI355X (gfx950) FlashPrefill V2 block-sparse prefill attention.

A thin ctypes binding over libbslp.so with the same entry points as the C ABI
in include/bslp.h.  It only marshals arguments (tensor pointers, the problem
descriptor, the current HIP stream); every step of the path runs in the HIP
kernels of the library.  If the library is missing the calls raise; there is
no fallback.

    problem = make_problem("bf16", hq=32, hkv=8, head_dim=128, block_size=128,
                           seqlens=[16384])
    out, lse, sel = prefill(problem, params, q, k, v)

torch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbslp.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error"}


class BslpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("num_seqs", ctypes.c_int32),
        ("seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("kv_splits", ctypes.c_int32),
        ("scales_dev", ctypes.c_void_p),
        ("kv_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("v_layout", ctypes.c_int32),
    ]


class SelectParams(ctypes.Structure):
    _fields_ = [
        ("alpha", ctypes.c_float),
        ("sink_blocks", ctypes.c_int32),
        ("window_blocks", ctypes.c_int32),
        ("recent_blocks", ctypes.c_int32),
        ("mean_correction", ctypes.c_int32),
    ]


class Sizes(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("pooled_rows", ctypes.c_int64),
        ("score_elems", ctypes.c_int64),
        ("num_segments", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("kv_tokens", ctypes.c_int64),
    ]


EXPORTS = ("bslp_get_sizes", "bslp_workspace_bytes", "bslp_block_scores", "bslp_pool_kv", "bslp_score_blocks",
           "bslp_select_blocks",
           "bslp_sparse_prefill_attn", "bslp_sparse_prefill_attn_noalloc",
           "bslp_dense_prefill_attn", "bslp_quantize_e4m3", "bslp_status_string",
           "bslp_last_error")
NOALLOC_SCRATCH_BYTES = 32 << 20  # BSLP_NOALLOC_SCRATCH_BYTES

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libbslp.so (built by `python -m block_sparse_long_pooled_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_long_pooled_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.bslp_get_sizes.argtypes = [P(Problem), P(Sizes)]
    lib.bslp_workspace_bytes.argtypes = [P(Problem)]
    lib.bslp_workspace_bytes.restype = ctypes.c_size_t
    lib.bslp_block_scores.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, vp]
    lib.bslp_pool_kv.argtypes = [P(Problem), vp, vp, vp, vp, vp]
    lib.bslp_score_blocks.argtypes = [P(Problem), vp, vp, vp, vp]
    lib.bslp_select_blocks.argtypes = [P(Problem), P(SelectParams), vp, vp, vp, vp, vp, vp, vp]
    lib.bslp_sparse_prefill_attn.argtypes = [P(Problem), P(SelectParams), vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bslp_sparse_prefill_attn_noalloc.argtypes = [P(Problem), P(SelectParams), vp, vp, vp,
                                                     vp, vp, vp, vp, vp, vp, vp]
    lib.bslp_dense_prefill_attn.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp]
    lib.bslp_quantize_e4m3.argtypes = [ctypes.c_int32, vp, ctypes.c_int64, vp, vp, vp]
    for name in ("bslp_get_sizes", "bslp_block_scores", "bslp_pool_kv", "bslp_score_blocks",
                 "bslp_select_blocks",
                 "bslp_sparse_prefill_attn", "bslp_sparse_prefill_attn_noalloc",
                 "bslp_dense_prefill_attn", "bslp_quantize_e4m3"):
        getattr(lib, name).restype = ctypes.c_int
    lib.bslp_status_string.argtypes = [ctypes.c_int]
    lib.bslp_status_string.restype = ctypes.c_char_p
    lib.bslp_last_error.argtypes = []
    lib.bslp_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise BslpError(status, load_library().bslp_last_error().decode())


def make_problem(dtype: str, hq: int, hkv: int, head_dim: int, block_size: int, seqlens,
                 softmax_scale: float | None = None, q_scale: float = 1.0, k_scale: float = 1.0,
                 v_scale: float = 1.0, page_table=None, page_size: int = 0,
                 kv_splits: int = 0, scales_dev=None, kv_seqlens=None,
                 v_dmajor: bool = False) -> Problem:
    """Fills the problem descriptor.  `page_table` is a device int32 tensor
    [num_seqs, max_pages] (or None for contiguous K/V); `kv_splits` 0 lets the
    library choose the attention's KV splits, 1 turns them off; `scales_dev`
    (fp8) is a device float32 tensor of (q, k, v) scales that replaces the
    host scales, e.g. filled by quantize_e4m3.  `kv_seqlens` gives each
    request's key count when its queries are only the last `seqlens[b]`
    positions (a chunk of a chunked prefill).  `v_dmajor` (fp8): V is given
    as [Hkv, d, kv tokens] (or [pages, Hkv, d, page_size] when paged)."""
    lens = (ctypes.c_int32 * len(seqlens))(*[int(x) for x in seqlens])
    p = Problem()
    p.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    p.num_heads_q, p.num_heads_kv = hq, hkv
    p.head_dim, p.block_size = head_dim, block_size
    p.softmax_scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_dim)
    p.q_scale, p.k_scale, p.v_scale = q_scale, k_scale, v_scale
    p.num_seqs = len(seqlens)
    p.kv_splits = kv_splits
    p.v_layout = 1 if v_dmajor else 0
    if scales_dev is not None:
        p.scales_dev = scales_dev.data_ptr()
    p.seqlens = lens
    kvl = None
    if kv_seqlens is not None:
        kvl = (ctypes.c_int32 * len(kv_seqlens))(*[int(x) for x in kv_seqlens])
        p.kv_seqlens = kvl
    p._keep = [lens, page_table, scales_dev, kvl]
    if page_table is not None:
        p.page_table = page_table.data_ptr()
        p.page_size = page_size
        p.max_pages_per_seq = page_table.shape[1]
    return p


def make_params(alpha: float, sink: int = 1, window: int = 2, recent: int = 1,
                correction: bool = True) -> SelectParams:
    return SelectParams(alpha, sink, window, recent, 1 if correction else 0)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libbslp must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def get_sizes(problem: Problem) -> Sizes:
    s = Sizes()
    _check(load_library().bslp_get_sizes(ctypes.byref(problem), ctypes.byref(s)))
    return s


def workspace_bytes(problem) -> int:
    """Bytes of workspace bslp_sparse_prefill_attn needs (0: invalid problem)."""
    return int(load_library().bslp_workspace_bytes(ctypes.byref(problem)))


def block_scores(problem, q, k, v, kbar, vbar, scores, stream=None):
    _check(load_library().bslp_block_scores(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(kbar), _ptr(vbar), _ptr(scores),
                                            _stream(stream)))


def pool_kv(problem, k, v, kbar, vbar, stream=None):
    """The pooling half of block_scores."""
    _check(load_library().bslp_pool_kv(ctypes.byref(problem), _ptr(k), _ptr(v), _ptr(kbar),
                                       _ptr(vbar), _stream(stream)))


def score_blocks(problem, q, kbar, scores, stream=None):
    """The scoring half of block_scores (kbar from pool_kv)."""
    _check(load_library().bslp_score_blocks(ctypes.byref(problem), _ptr(q), _ptr(kbar),
                                            _ptr(scores), _stream(stream)))


def select_blocks(problem, params, q, kbar, scores, counts, cu, idx, stream=None):
    """Selection from the score rows; q and kbar serve the exact re-decision
    of blocks near the threshold."""
    _check(load_library().bslp_select_blocks(ctypes.byref(problem), ctypes.byref(params),
                                             _ptr(q), _ptr(kbar), _ptr(scores), _ptr(counts),
                                             _ptr(cu), _ptr(idx), _stream(stream)))


def sparse_prefill_attn(problem, params, q, k, v, kbar, vbar, cu, idx, out, lse=None,
                        workspace=None, stream=None):
    """`workspace`: a device tensor of at least get_sizes(problem).workspace_bytes
    bytes (None passes a NULL pointer and size 0)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().bslp_sparse_prefill_attn(ctypes.byref(problem), ctypes.byref(params),
                                                   _ptr(q), _ptr(k), _ptr(v), _ptr(kbar),
                                                   _ptr(vbar), _ptr(cu), _ptr(idx), _ptr(out),
                                                   _ptr(lse), _ptr(workspace), nbytes,
                                                   _stream(stream)))


def sparse_prefill_attn_noalloc(problem, params, q, k, v, kbar, vbar, cu, idx, out, lse=None,
                                stream=None):
    """sparse_prefill_attn without a workspace: the library's own device
    scratch array (NOALLOC_SCRATCH_BYTES per GPU) takes its place."""
    _check(load_library().bslp_sparse_prefill_attn_noalloc(
        ctypes.byref(problem), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(kbar),
        _ptr(vbar), _ptr(cu), _ptr(idx), _ptr(out), _ptr(lse), _stream(stream)))


def quantize_e4m3(x, codes, scale, stream=None):
    """Online per-tensor e4m3 quantisation of the bf16 or float32 device
    tensor x into the uint8 tensor codes; scale (a one-element device float32
    tensor, or a view of one) receives amax / 448."""
    dt = {"torch.bfloat16": BF16, "torch.float32": F32}[str(x.dtype)]
    _check(load_library().bslp_quantize_e4m3(dt, _ptr(x), x.numel(), _ptr(codes), _ptr(scale),
                                             _stream(stream)))


def dense_prefill_attn(problem, q, k, v, out, lse=None, stream=None):
    """Dense causal attention over every key j <= i (no index stage)."""
    _check(load_library().bslp_dense_prefill_attn(ctypes.byref(problem), _ptr(q), _ptr(k),
                                                  _ptr(v), _ptr(out), _ptr(lse),
                                                  _stream(stream)))


class Buffers:
    """Device buffers of one prefill call, allocated with torch."""

    def __init__(self, problem: Problem, device="cuda"):
        import torch
        s = get_sizes(problem)
        d, hkv, hq = problem.head_dim, problem.num_heads_kv, problem.num_heads_q
        T = s.total_tokens
        f32 = torch.float32
        self.sizes = s
        self.kbar = torch.empty((s.pooled_rows, hkv, d), dtype=f32, device=device)
        self.vbar = torch.empty((s.pooled_rows, hkv, d), dtype=f32, device=device)
        self.scores = torch.empty(max(1, s.score_elems), dtype=f32, device=device)
        self.counts = torch.empty(max(1, s.num_segments), dtype=torch.int32, device=device)
        self.cu = torch.empty(s.num_segments + 1, dtype=torch.int32, device=device)
        self.idx = torch.empty(max(1, s.score_elems), dtype=torch.int32, device=device)
        odt = f32 if problem.dtype == F32 else torch.bfloat16
        self.out = torch.empty((T, hq, d), dtype=odt, device=device)
        self.lse = torch.empty((hq, T), dtype=f32, device=device)
        self.workspace = torch.empty(max(16, s.workspace_bytes), dtype=torch.uint8, device=device)


def prefill(problem, params, q, k, v, bufs: Buffers | None = None, stream=None) -> Buffers:
    """The three stages back to back on one stream."""
    bufs = bufs or Buffers(problem, q.device)
    block_scores(problem, q, k, v, bufs.kbar, bufs.vbar, bufs.scores, stream)
    select_blocks(problem, params, q, bufs.kbar, bufs.scores, bufs.counts, bufs.cu, bufs.idx,
                  stream)
    sparse_prefill_attn(problem, params, q, k, v, bufs.kbar, bufs.vbar, bufs.cu, bufs.idx,
                        bufs.out, bufs.lse, bufs.workspace, stream)
    return bufs


__all__ = ["BF16", "F32", "FP8_E4M3", "BslpError", "Buffers", "EXPORTS", "LIB_PATH", "Problem",
           "SelectParams", "Sizes", "block_scores", "dense_prefill_attn", "get_sizes",
           "load_library", "make_params",
           "make_problem", "pool_kv", "prefill", "quantize_e4m3", "score_blocks", "select_blocks", "sparse_prefill_attn", "sparse_prefill_attn_noalloc"]
