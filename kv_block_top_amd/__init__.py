"""MI355X-native top-k KV-block selector and page-16 sparse block table.

Thin binding over the C ABI of ``libkvbt.so`` (declared in ``include/kvbt.h``):
it checks tensors, allocates outputs when none are given, and passes device
pointers and the current HIP stream. Every step of the computation runs in the
library's HIP kernels; there is no other implementation to fall back to, and
calling any entry point without the built library raises.

Layouts (token-major, contiguous):
    scores [T, H, max_k_tiles] float32 or bfloat16
    idx    [T, H, topk] int32        table [T, H, topk * 8] int32     ctx [T, H] int32
    block_table [B, max_blocks] int32; seq_lens [B]; row_req, row_pos, num_valid_pages [T]

The decode index-score producer that fills the score buffer (``include/kvbt_index.h``):
    q_idx [B*q, H, 128] bfloat16; k_cache [num_pages, H, 16, 16, 8] bfloat16 (16-token
    pages, block p in pages 8p..8p+7); scores [B*q, H, max_k_tiles] float32 or bfloat16,
    written in place for causally valid blocks only

The sparse-attention decode that consumes the table (``include/kvbt_attn.h``):
    q [T, H*G, 128] bfloat16; k_cache [P, H, 16, 16, 8] bfloat16 (8 consecutive
    dimensions of a token together); v_cache [P, H, 128, 16] bfloat16 (16 tokens of a
    dimension together); out [T, H*G, 128] float32 or bfloat16
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "select_topk_blocks", "build_sparse_block_table", "select_topk_and_build_table",
    "launch_policy", "status_string", "version", "library_path", "KvbtError",
    "F32", "BF16", "PAGES_PER_BLOCK", "MAX_TOPK", "MAX_K_TILES", "FAST_K_TILES",
    "sparse_attn_decode", "sparse_attn_waves", "ATTN_HEAD_DIM", "ATTN_MAX_GROUP",
    "index_decode_scores", "REDUCE_LSE", "REDUCE_MAX", "FP8_E4M3",
    "select_workspace_bytes", "SPLIT_AUTO", "SPLIT_ALWAYS", "SPLIT_NEVER",
    "select_topk_and_build_table_noalloc", "NOALLOC_SCRATCH_BYTES",
    "sparse_attn_splits", "sparse_attn_workspace_bytes", "ATTN_MAX_SPLITS",
]

F32 = 0
BF16 = 1
PAGES_PER_BLOCK = 8
MAX_TOPK = 64
FAST_TOPK = 16      # largest topk of the launch paths other than the topk-above-16 one
MAX_K_TILES = 1 << 24
FAST_K_TILES = 8192
ATTN_HEAD_DIM = 128
ATTN_MAX_GROUP = 16
ATTN_MAX_SPLITS = 8
REDUCE_LSE = 0
REDUCE_MAX = 1
FP8_E4M3 = 2
SPLIT_AUTO = 0      # cross-workgroup split: the library's choice (with a workspace)
SPLIT_ALWAYS = 1    # whenever the rows can take it
SPLIT_NEVER = 2
NOALLOC_SCRATCH_BYTES = 1 << 20   # the allocation-free call's scratch, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvbt.so")
_lib = None
_lock = threading.Lock()


class KvbtError(ValueError):
    """A negative status from the library (validation or launch failure)."""

    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))
        self.status = status


class _Policy(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("threads_per_block", ctypes.c_int),
                ("row_heads_per_block", ctypes.c_int), ("grid", ctypes.c_int64),
                ("vec", ctypes.c_int), ("chunks", ctypes.c_int), ("slices", ctypes.c_int),
                ("workspace_bytes", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded ``libkvbt.so`` (ctypes handle with typed entry points)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "libkvbt.so is not built (%s). Build it with "
                "`python -m kv_block_top_amd.build`." % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.kvbt_launch_policy.argtypes = [i32, i32, i32, i64, i32, i32, ctypes.POINTER(_Policy)]
        L.kvbt_select_topk_blocks.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, i32, i32,
                                              i64, vp, vp]
        L.kvbt_build_sparse_block_table.argtypes = [vp, i64, i32, i32, vp, i32, i32, vp, i32,
                                                    vp, vp, vp, vp, vp]
        L.kvbt_select_topk_and_build_table.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32,
                                                       vp, i32, vp, vp, i32, i32, i32, i32,
                                                       i64, vp, vp, vp, vp]
        L.kvbt_launch_policy_ws.argtypes = [i32, i32, i32, i64, i32, i32, i32, i64,
                                            ctypes.POINTER(_Policy)]
        L.kvbt_select_workspace_bytes.argtypes = [i32, i32, i32, i64, i32, i32, i32]
        L.kvbt_select_workspace_bytes.restype = i64
        L.kvbt_select_topk_blocks_ws.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, i32, i32,
                                                 i64, vp, i32, vp, i64, vp]
        L.kvbt_select_topk_and_build_table_ws.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32,
                                                          vp, i32, vp, vp, i32, i32, i32, i32,
                                                          i64, vp, vp, vp, i32, vp, i64, vp]
        L.kvbt_select_topk_and_build_table_noalloc.argtypes = [
            vp, i32, i64, i32, i32, vp, i32, i32, vp, i32, vp, vp, i32, i32, i32, i32, i64, vp,
            vp, vp, i32, vp]
        L.kvbt_status_string.argtypes = [i32]
        L.kvbt_status_string.restype = ctypes.c_char_p
        L.kvbt_version.argtypes = []
        L.kvbt_version.restype = ctypes.c_char_p
        L.kvbt_sparse_attn_decode.argtypes = [vp, i64, i32, i32, i32, vp, vp, i64, vp, i32,
                                              vp, i32, ctypes.c_float, vp, i32, i32, vp]
        L.kvbt_sparse_attn_decode_ws.argtypes = [vp, i64, i32, i32, i32, vp, vp, i64, vp, i32,
                                                 vp, i32, ctypes.c_float, vp, i32, i32, i32,
                                                 vp, i64, vp]
        L.kvbt_sparse_attn_splits.argtypes = [i64, i32, i32, i64]
        L.kvbt_sparse_attn_workspace_bytes.argtypes = [i64, i32, i32]
        L.kvbt_sparse_attn_workspace_bytes.restype = i64
        L.kvbt_sparse_attn_waves.argtypes = [i64, i32, i32]
        L.kvbt_sparse_attn_grouped.argtypes = [i64, i32, i32, i32]
        L.kvbt_index_decode_scores.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, i64, vp,
                                               i32, vp, ctypes.c_float, i32, vp, i32, i32, vp]
        L.kvbt_bench_empty.argtypes = [i32, vp]
        L.kvbt_bench_copy.argtypes = [vp, vp, i64, vp]
        L.kvbt_bench_read.argtypes = [vp, i64, vp, vp]
        for f in ("kvbt_launch_policy", "kvbt_launch_policy_ws", "kvbt_select_topk_blocks",
                  "kvbt_select_topk_blocks_ws", "kvbt_select_topk_and_build_table_ws",
                  "kvbt_select_topk_and_build_table_noalloc",
                  "kvbt_build_sparse_block_table", "kvbt_select_topk_and_build_table",
                  "kvbt_bench_empty", "kvbt_bench_copy", "kvbt_bench_read",
                  "kvbt_sparse_attn_decode", "kvbt_sparse_attn_waves", "kvbt_sparse_attn_grouped",
                  "kvbt_sparse_attn_decode_ws", "kvbt_sparse_attn_splits",
                  "kvbt_index_decode_scores"):
            getattr(L, f).restype = i32
        _lib = L
        return L


def status_string(status: int) -> str:
    return lib().kvbt_status_string(int(status)).decode()


def version() -> str:
    return lib().kvbt_version().decode()


def launch_policy(max_block: int, max_k_tiles: int, score_dtype: int, T: int, H: int,
                  topk: int = 16, split=None, workspace_bytes: int = 0) -> dict:
    """The launch geometry the library would use (pure host computation): of the calls
    without a workspace, or, with ``split`` given, of the *_ws calls with a workspace of
    ``workspace_bytes`` bytes."""
    p = _Policy()
    if split is None:
        st = lib().kvbt_launch_policy(max_block, max_k_tiles, score_dtype, T, H, topk,
                                      ctypes.byref(p))
    else:
        st = lib().kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk,
                                         int(split), int(workspace_bytes), ctypes.byref(p))
    if st != 0:
        raise KvbtError(st, "kvbt_launch_policy")
    return {f: getattr(p, f) for f, _ in _Policy._fields_}


def select_workspace_bytes(max_block: int, max_k_tiles: int, score_dtype: int, T: int, H: int,
                           topk: int = 16, split: int = SPLIT_AUTO) -> int:
    """Workspace bytes a *_ws call of this shape uses under ``split`` (0: none)."""
    n = lib().kvbt_select_workspace_bytes(max_block, max_k_tiles, score_dtype, T, H, topk,
                                          int(split))
    if n < 0:
        raise KvbtError(int(n), "kvbt_select_workspace_bytes")
    return int(n)


def _workspace(workspace):
    """(pointer, bytes) of a workspace tensor (any dtype), or (NULL, 0)."""
    if workspace is None:
        return ctypes.c_void_p(0), 0
    _dev_ptr(workspace, "workspace")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(x, name, dtype=None, ndim=None, shape=None, optional=False):
    if x is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, x.device))
    if dtype is not None and x.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s must have dtype %s (got %s)" % (name, dtype, x.dtype))
    if ndim is not None and x.dim() != ndim:
        raise ValueError("%s must have %d dimensions (got %d)" % (name, ndim, x.dim()))
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(x.shape)))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(x.data_ptr()) if x.numel() else ctypes.c_void_p(0)


def _score_dtype(scores):
    torch = _torch()
    if scores.dtype == torch.float32:
        return F32
    if scores.dtype == torch.bfloat16:
        return BF16
    raise ValueError("scores must be float32 or bfloat16 (got %s)" % scores.dtype)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _rows(T, device, seq_lens, decode_query_len, row_req, row_pos):
    """Row description pointers: (seq_lens, q, row_req, row_pos)."""
    torch = _torch()
    if row_req is not None:
        if row_pos is None:
            raise ValueError("row_pos is required with row_req")
        rr = _dev_ptr(row_req, "row_req", torch.int32, 1, (T,))
        rp = _dev_ptr(row_pos, "row_pos", torch.int32, 1, (T,))
        return ctypes.c_void_p(0), 1, rr, rp
    if seq_lens is None:
        raise ValueError("give seq_lens (decode form) or row_req/row_pos (explicit form)")
    sl = _dev_ptr(seq_lens, "seq_lens", torch.int32, 1)
    return sl, int(decode_query_len), ctypes.c_void_p(0), ctypes.c_void_p(0)


def _out(x, name, shape, device):
    torch = _torch()
    if x is None:
        return torch.empty(shape, dtype=torch.int32, device=device)
    _dev_ptr(x, name, torch.int32, len(shape), shape)
    return x


def select_topk_blocks(scores, num_valid_pages, topk: int = 16, num_init: int = 1,
                       num_local: int = 2, max_block: int = 0, num_decode_rows: int = 0,
                       out=None, stream=None, workspace=None, split=None):
    """Top-k KV blocks per (row, head): int32 ``[T, H, topk]``, rank order, -1 padded.

    ``max_block`` and ``num_decode_rows`` are launch hints (see include/kvbt.h); they
    never change the result. With ``workspace`` (a zero-initialised device tensor, kept
    by the caller between calls) or ``split``, the call goes through
    kvbt_select_topk_blocks_ws and may split rows across workgroups (include/kvbt.h).
    """
    torch = _torch()
    T, H, M = _shape3(scores)
    sp = _dev_ptr(scores, "scores", (torch.float32, torch.bfloat16), 3)
    nvp = _dev_ptr(num_valid_pages, "num_valid_pages", torch.int32, 1, (T,))
    out = _out(out, "out", (T, H, topk), scores.device)
    if workspace is not None or split is not None:
        wp, wn = _workspace(workspace)
        st = lib().kvbt_select_topk_blocks_ws(
            sp, _score_dtype(scores), T, H, M, nvp, topk, num_init, num_local, max_block,
            int(num_decode_rows), _dev_ptr(out, "out"),
            SPLIT_AUTO if split is None else int(split), wp, wn, _stream(stream))
    else:
        st = lib().kvbt_select_topk_blocks(sp, _score_dtype(scores), T, H, M, nvp, topk,
                                           num_init, num_local, max_block,
                                           int(num_decode_rows), _dev_ptr(out, "out"),
                                           _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_select_topk_blocks")
    return out


def build_sparse_block_table(idx, block_table, seq_lens=None, decode_query_len: int = 1,
                             row_req=None, row_pos=None, out_table=None, out_ctx=None,
                             stream=None):
    """Page-16 sparse block table ``[T, H, topk*8]`` and context lengths ``[T, H]``."""
    torch = _torch()
    T, H, K = _shape3(idx)
    ip = _dev_ptr(idx, "idx", torch.int32, 3)
    bt = _dev_ptr(block_table, "block_table", torch.int32, 2)
    B, max_blocks = block_table.shape
    sl, q, rr, rp = _rows(T, idx.device, seq_lens, decode_query_len, row_req, row_pos)
    if row_req is None and seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have one entry per block_table row")
    out_table = _out(out_table, "out_table", (T, H, K * PAGES_PER_BLOCK), idx.device)
    out_ctx = _out(out_ctx, "out_ctx", (T, H), idx.device)
    st = lib().kvbt_build_sparse_block_table(ip, T, H, K, bt, B, max_blocks, sl, q, rr, rp,
                                             _dev_ptr(out_table, "out_table"),
                                             _dev_ptr(out_ctx, "out_ctx"), _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_build_sparse_block_table")
    return out_table, out_ctx


def select_topk_and_build_table(scores, block_table, seq_lens=None, decode_query_len: int = 1,
                                row_req=None, row_pos=None, topk: int = 16, num_init: int = 1,
                                num_local: int = 2, max_block: int = 0, num_decode_rows: int = 0,
                                out=None, stream=None, workspace=None, split=None):
    """Fused selector + table in one launch: ``(idx, table, ctx)``.

    ``out`` may be a tuple of three preallocated int32 tensors of the output shapes.
    ``max_block`` and ``num_decode_rows`` are launch hints (see include/kvbt.h); they
    never change the result. ``workspace`` and ``split`` as in select_topk_blocks
    (kvbt_select_topk_and_build_table_ws).
    """
    torch = _torch()
    T, H, M = _shape3(scores)
    sp = _dev_ptr(scores, "scores", (torch.float32, torch.bfloat16), 3)
    bt = _dev_ptr(block_table, "block_table", torch.int32, 2)
    B, max_blocks = block_table.shape
    sl, q, rr, rp = _rows(T, scores.device, seq_lens, decode_query_len, row_req, row_pos)
    if row_req is None and seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have one entry per block_table row")
    o_idx, o_tab, o_ctx = out if out is not None else (None, None, None)
    o_idx = _out(o_idx, "out idx", (T, H, topk), scores.device)
    o_tab = _out(o_tab, "out table", (T, H, topk * PAGES_PER_BLOCK), scores.device)
    o_ctx = _out(o_ctx, "out ctx", (T, H), scores.device)
    if workspace is not None or split is not None:
        wp, wn = _workspace(workspace)
        st = lib().kvbt_select_topk_and_build_table_ws(
            sp, _score_dtype(scores), T, H, M, bt, B, max_blocks, sl, q, rr, rp, topk,
            num_init, num_local, max_block, int(num_decode_rows), _dev_ptr(o_idx, "out idx"),
            _dev_ptr(o_tab, "out table"), _dev_ptr(o_ctx, "out ctx"),
            SPLIT_AUTO if split is None else int(split), wp, wn, _stream(stream))
    else:
        st = lib().kvbt_select_topk_and_build_table(
            sp, _score_dtype(scores), T, H, M, bt, B, max_blocks, sl, q, rr, rp, topk,
            num_init, num_local, max_block, int(num_decode_rows), _dev_ptr(o_idx, "out idx"),
            _dev_ptr(o_tab, "out table"), _dev_ptr(o_ctx, "out ctx"), _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_select_topk_and_build_table")
    return o_idx, o_tab, o_ctx


def select_topk_and_build_table_noalloc(scores, block_table, seq_lens=None,
                                        decode_query_len: int = 1, row_req=None, row_pos=None,
                                        topk: int = 16, num_init: int = 1, num_local: int = 2,
                                        max_block: int = 0, num_decode_rows: int = 0,
                                        out=None, stream=None, split: int = SPLIT_AUTO):
    """The fused call through kvbt_select_topk_and_build_table_noalloc: the library
    allocates nothing and uses its own per-GPU scratch where the call splits rows across
    workgroups (include/kvbt.h). Pass ``out`` (three int32 tensors) to allocate nothing
    here either."""
    torch = _torch()
    T, H, M = _shape3(scores)
    sp = _dev_ptr(scores, "scores", (torch.float32, torch.bfloat16), 3)
    bt = _dev_ptr(block_table, "block_table", torch.int32, 2)
    B, max_blocks = block_table.shape
    sl, q, rr, rp = _rows(T, scores.device, seq_lens, decode_query_len, row_req, row_pos)
    if row_req is None and seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have one entry per block_table row")
    o_idx, o_tab, o_ctx = out if out is not None else (None, None, None)
    o_idx = _out(o_idx, "out idx", (T, H, topk), scores.device)
    o_tab = _out(o_tab, "out table", (T, H, topk * PAGES_PER_BLOCK), scores.device)
    o_ctx = _out(o_ctx, "out ctx", (T, H), scores.device)
    st = lib().kvbt_select_topk_and_build_table_noalloc(
        sp, _score_dtype(scores), T, H, M, bt, B, max_blocks, sl, q, rr, rp, topk, num_init,
        num_local, max_block, int(num_decode_rows), _dev_ptr(o_idx, "out idx"),
        _dev_ptr(o_tab, "out table"), _dev_ptr(o_ctx, "out ctx"), int(split), _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_select_topk_and_build_table_noalloc")
    return o_idx, o_tab, o_ctx


def sparse_attn_decode(q, k_cache, v_cache, table, ctx, scale: float, out=None,
                       out_dtype=None, waves: int = 0, decode_query_len: int = 1,
                       stream=None, workspace=None, splits=None):
    """Sparse paged-attention decode over the page-16 table: ``[T, H*G, 128]``.

    ``out_dtype`` is torch.float32 (default) or torch.bfloat16; ``waves`` picks the
    wavefronts per (row, index head) (0: the library's choice); ``decode_query_len`` is
    the rows per request (which kernel runs: see include/kvbt_attn.h). With
    ``workspace`` (a zero-initialised device tensor, kept between calls) or ``splits``
    given, kvbt_sparse_attn_decode_ws runs: ``splits`` 0 (default) lets the library
    split small batches across workgroups, 1 never splits, 2..8 asks for that many
    workgroups per (row, index head).
    """
    torch = _torch()
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [P, H, 16, 16, 8] and v_cache [P, H, 128, 16]")
    P, H = int(k_cache.shape[0]), int(k_cache.shape[1])
    kp = _dev_ptr(k_cache, "k_cache", torch.bfloat16, 5, (P, H, ATTN_HEAD_DIM // 8, 16, 8))
    vp_ = _dev_ptr(v_cache, "v_cache", torch.bfloat16, 4, (P, H, ATTN_HEAD_DIM, 16))
    T, HG, D = _shape3(q)
    if HG % H != 0:
        raise ValueError("q has %d heads, not a multiple of the cache's %d KV heads" % (HG, H))
    qp = _dev_ptr(q, "q", torch.bfloat16, 3)
    W = int(table.shape[2]) if table.dim() == 3 else 0
    tp = _dev_ptr(table, "table", torch.int32, 3, (T, H, W))
    cp = _dev_ptr(ctx, "ctx", torch.int32, 2, (T, H))
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((T, HG, D), dtype=out_dtype, device=q.device)
    op = _dev_ptr(out, "out", out_dtype, 3, (T, HG, D))
    od = F32 if out_dtype == torch.float32 else BF16
    if workspace is not None or splits is not None:
        wp, wn = _workspace(workspace)
        st = lib().kvbt_sparse_attn_decode_ws(qp, T, H, HG // H, D, kp, vp_, P, tp, W, cp,
                                              int(decode_query_len), float(scale), op, od,
                                              int(waves), int(splits or 0), wp, wn,
                                              _stream(stream))
        if st != 0:
            raise KvbtError(st, "kvbt_sparse_attn_decode_ws")
        return out
    st = lib().kvbt_sparse_attn_decode(qp, T, H, HG // H, D, kp, vp_, P, tp, W, cp,
                                       int(decode_query_len), float(scale), op, od,
                                       int(waves), _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_sparse_attn_decode")
    return out


def sparse_attn_waves(T: int, H: int, decode_query_len: int = 1) -> int:
    """Wavefronts per (row, index head) the library picks for ``waves=0``."""
    return int(lib().kvbt_sparse_attn_waves(int(T), int(H), int(decode_query_len)))


def sparse_attn_splits(T: int, H: int, splits: int = 0, workspace_bytes: int = 1 << 62) -> int:
    """Workgroups per (row, index head) ``sparse_attn_decode`` with a workspace of
    ``workspace_bytes`` splits over (0: no split)."""
    return int(lib().kvbt_sparse_attn_splits(int(T), int(H), int(splits), int(workspace_bytes)))


def sparse_attn_workspace_bytes(T: int, H: int, splits: int = 0) -> int:
    """Workspace bytes ``sparse_attn_decode`` uses with ``splits`` for T rows and H index
    heads (0 when it does not split)."""
    n = lib().kvbt_sparse_attn_workspace_bytes(int(T), int(H), int(splits))
    if n < 0:
        raise KvbtError(int(n), "kvbt_sparse_attn_workspace_bytes")
    return int(n)


def sparse_attn_grouped(T: int, H: int, G: int, decode_query_len: int) -> bool:
    """Whether ``sparse_attn_decode`` attends the rows of each request together for
    this batch shape (see include/kvbt_attn.h)."""
    return bool(lib().kvbt_sparse_attn_grouped(int(T), int(H), int(G), int(decode_query_len)))


def index_decode_scores(q_idx, k_cache, block_table, seq_lens, scores, scale: float,
                        decode_query_len: int = 1, reduce: str = "lse", k_scale=None,
                        stream=None):
    """Decode index scores written in place into ``scores`` [B*q, H, max_k_tiles]
    (float32 or bfloat16) for the causally valid blocks; returns ``scores``.

    ``reduce`` is "lse" (log-sum-exp of the block's token scores) or "max". Keys are
    bfloat16 ``[num_pages, H, 16, 16, 8]``, or FP8 E4M3 codes ``[num_pages, H, 8, 16, 16]``
    (torch.uint8 or torch.float8_e4m3fn) with ``k_scale`` float32 ``[num_pages, H, 16]``.
    """
    torch = _torch()
    if reduce not in ("lse", "max"):
        raise ValueError('reduce must be "lse" or "max"')
    if k_cache.dim() != 5:
        raise ValueError("k_cache must be 5-d")
    P, H = int(k_cache.shape[0]), int(k_cache.shape[1])
    if k_scale is None:
        kp = _dev_ptr(k_cache, "k_cache", torch.bfloat16, 5, (P, H, ATTN_HEAD_DIM // 8, 16, 8))
        kd, sp_ = BF16, ctypes.c_void_p(0)
    else:
        kp = _dev_ptr(k_cache, "k_cache", (torch.uint8, torch.float8_e4m3fn), 5,
                      (P, H, ATTN_HEAD_DIM // 16, 16, 16))
        sp_ = _dev_ptr(k_scale, "k_scale", torch.float32, 3, (P, H, 16))
        kd = FP8_E4M3
    bt = _dev_ptr(block_table, "block_table", torch.int32, 2)
    B, max_blocks = int(block_table.shape[0]), int(block_table.shape[1])
    q = int(decode_query_len)
    qp = _dev_ptr(q_idx, "q_idx", torch.bfloat16, 3, (B * q, H, ATTN_HEAD_DIM))
    sl = _dev_ptr(seq_lens, "seq_lens", torch.int32, 1, (B,))
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (B * q, H):
        raise ValueError("scores must be [B*q, H, max_k_tiles]")
    sp = _dev_ptr(scores, "scores", (torch.float32, torch.bfloat16), 3)
    st = lib().kvbt_index_decode_scores(qp, B, q, H, ATTN_HEAD_DIM, kp, kd, sp_, P, bt,
                                        max_blocks, sl, float(scale),
                                        REDUCE_LSE if reduce == "lse" else REDUCE_MAX,
                                        sp, _score_dtype(scores), int(scores.shape[2]),
                                        _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_index_decode_scores")
    return scores


def _shape3(x):
    if x.dim() != 3:
        raise ValueError("expected a 3-d tensor [T, H, *], got shape %s" % (tuple(x.shape),))
    return int(x.shape[0]), int(x.shape[1]), int(x.shape[2])


# ---------------------------------------------------------------------------
# measurement helpers (include/kvbt_bench.h)
# ---------------------------------------------------------------------------

def bench_empty(blocks: int = 1, stream=None) -> None:
    st = lib().kvbt_bench_empty(blocks, _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_bench_empty")


def bench_copy(dst, src, nbytes: int, stream=None) -> None:
    st = lib().kvbt_bench_copy(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), int(nbytes),
                               _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_bench_copy")


def bench_read(src, nbytes: int, sink, stream=None) -> None:
    st = lib().kvbt_bench_read(_dev_ptr(src, "src"), int(nbytes), _dev_ptr(sink, "sink"),
                               _stream(stream))
    if st != 0:
        raise KvbtError(st, "kvbt_bench_read")
