"""CPU oracle for the top-k KV-block selector and the page-16 sparse block table.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the
HIP library under ``kv_block_top_amd``) never calls it, shares no source with it,
and fails loudly when its own extension is missing instead of falling back here.

The arithmetic lives in ``kvbt_oracle.c`` (plain C, one full sort per row and
head); this module only builds it with gcc, marshals numpy arrays, and splits
rows over host threads (each thread runs the same sequential C code on its own
row range; ctypes releases the GIL during the call).

Score arrays are numpy ``float32`` (fp32 scores) or ``uint16`` holding bf16 bit
patterns. All index arrays are ``int32``. Shapes follow the token-major layout:
scores ``[T, H, max_k_tiles]``, idx ``[T, H, topk]``, table ``[T, H, topk*8]``,
ctx ``[T, H]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvbt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvbt_oracle.so")

F32 = 0
BF16 = 1
PAGES_PER_BLOCK = 8

_default = None
_default_lock = threading.Lock()


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library with gcc."""
    global _default
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == _LIB_PATH:
        _default = None
    return out


def _bind(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.kvbt_oracle_total_order_cmp.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    lib.kvbt_oracle_total_order_cmp.restype = i32
    lib.kvbt_oracle_select_topk_blocks.argtypes = [
        vp, i32, i64, i32, i32, vp, i32, i32, i32, vp, i64, i64]
    lib.kvbt_oracle_select_topk_blocks.restype = i32
    lib.kvbt_oracle_build_sparse_block_table.argtypes = [
        vp, i64, i32, i32, vp, i32, i32, vp, i32, vp, vp, vp, vp, i64, i64]
    lib.kvbt_oracle_build_sparse_block_table.restype = i32
    lib.kvbt_oracle_select_topk_and_build_table.argtypes = [
        vp, i32, i64, i32, i32, vp, i32, i32, vp, i32, vp, vp,
        i32, i32, i32, vp, vp, vp, i64, i64]
    lib.kvbt_oracle_select_topk_and_build_table.restype = i32
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(scores: np.ndarray) -> int:
    if scores.dtype == np.float32:
        return F32
    if scores.dtype == np.uint16:
        return BF16
    raise TypeError("scores must be float32 or uint16 (bf16 bits), got %s" % scores.dtype)


def _run_rows(fn, T: int, threads: int, rows=None):
    """Call ``fn(t0, t1)`` over [0, T) (or over each listed row), split over threads."""
    if rows is not None:
        ranges = [(int(t), int(t) + 1) for t in rows]
    else:
        threads = max(1, min(int(threads), T if T > 0 else 1))
        step = (T + threads - 1) // threads if T > 0 else 0
        ranges = [(s, min(T, s + step)) for s in range(0, T, step)] if T > 0 else []
    if not ranges:
        return
    if threads <= 1 or len(ranges) == 1:
        for t0, t1 in ranges:
            if fn(t0, t1) != 0:
                raise RuntimeError("oracle call failed")
        return
    errors = []
    lock = threading.Lock()
    it = iter(ranges)

    def worker():
        while True:
            with lock:
                nxt = next(it, None)
            if nxt is None:
                return
            if fn(*nxt) != 0:
                errors.append(nxt)

    pool = [threading.Thread(target=worker) for _ in range(min(threads, len(ranges)))]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    if errors:
        raise RuntimeError("oracle call failed on rows %r" % errors[:4])


def _row_description(T, seq_lens, decode_query_len, row_req, row_pos):
    if row_req is not None:
        row_req = np.ascontiguousarray(row_req, dtype=np.int32)
        row_pos = np.ascontiguousarray(row_pos, dtype=np.int32)
        assert row_req.shape == (T,) and row_pos.shape == (T,)
        return None, 1, row_req, row_pos
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    q = int(decode_query_len)
    assert q >= 1 and T == seq_lens.shape[0] * q, "decode form needs T == B * q"
    return seq_lens, q, None, None


class Oracle:
    """numpy front end over one loaded build of the oracle C code."""

    def __init__(self, lib_path: str = _LIB_PATH):
        self.path = lib_path
        self.lib = _bind(ctypes.CDLL(lib_path))

    def total_order_cmp(self, x_bits: int, y_bits: int) -> int:
        """IEEE 754 totalOrder on two binary32 bit patterns: -1, 0 or +1."""
        return int(self.lib.kvbt_oracle_total_order_cmp(int(x_bits) & 0xFFFFFFFF,
                                                        int(y_bits) & 0xFFFFFFFF))

    def select_topk_blocks(self, scores, num_valid_pages, topk=16, num_init=1,
                           num_local=2, threads=1, rows=None):
        """Top-k block ids per (row, head): ``[T, H, topk]`` int32, -1 padded.

        With ``rows`` only the listed rows are computed; the others hold -7.
        """
        scores = np.ascontiguousarray(scores)
        T, H, M = scores.shape
        nvp = np.ascontiguousarray(num_valid_pages, dtype=np.int32)
        assert nvp.shape == (T,)
        out = np.full((T, H, topk), -7, dtype=np.int32)
        lib, code = self.lib, _dtype_code(scores)
        _run_rows(lambda t0, t1: lib.kvbt_oracle_select_topk_blocks(
            _ptr(scores), code, T, H, M, _ptr(nvp), topk, num_init, num_local,
            _ptr(out), t0, t1), T, threads, rows)
        return out

    def build_sparse_block_table(self, idx, block_table, seq_lens=None,
                                 decode_query_len=1, row_req=None, row_pos=None,
                                 threads=1, rows=None):
        """Page-16 table ``[T, H, topk*8]`` and context lengths ``[T, H]`` (int32)."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, H, topk = idx.shape
        assert topk <= 64
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        B, max_blocks = bt.shape
        seq_lens, q, row_req, row_pos = _row_description(T, seq_lens, decode_query_len,
                                                         row_req, row_pos)
        table = np.full((T, H, topk * PAGES_PER_BLOCK), -7, dtype=np.int32)
        ctx = np.full((T, H), -7, dtype=np.int32)
        lib = self.lib
        _run_rows(lambda t0, t1: lib.kvbt_oracle_build_sparse_block_table(
            _ptr(idx), T, H, topk, _ptr(bt), B, max_blocks, _ptr(seq_lens), q,
            _ptr(row_req), _ptr(row_pos), _ptr(table), _ptr(ctx), t0, t1),
            T, threads, rows)
        return table, ctx

    def select_topk_and_build_table(self, scores, block_table, seq_lens=None,
                                    decode_query_len=1, row_req=None, row_pos=None,
                                    topk=16, num_init=1, num_local=2, threads=1,
                                    rows=None):
        """Selector then table build: ``(idx, table, ctx)``.

        With ``rows`` only the listed rows are computed; the others hold -7.
        """
        scores = np.ascontiguousarray(scores)
        T, H, M = scores.shape
        assert topk <= 64
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        B, max_blocks = bt.shape
        seq_lens, q, row_req, row_pos = _row_description(T, seq_lens, decode_query_len,
                                                         row_req, row_pos)
        idx = np.full((T, H, topk), -7, dtype=np.int32)
        table = np.full((T, H, topk * PAGES_PER_BLOCK), -7, dtype=np.int32)
        ctx = np.full((T, H), -7, dtype=np.int32)
        lib, code = self.lib, _dtype_code(scores)
        _run_rows(lambda t0, t1: lib.kvbt_oracle_select_topk_and_build_table(
            _ptr(scores), code, T, H, M, _ptr(bt), B, max_blocks, _ptr(seq_lens), q,
            _ptr(row_req), _ptr(row_pos), topk, num_init, num_local,
            _ptr(idx), _ptr(table), _ptr(ctx), t0, t1), T, threads, rows)
        return idx, table, ctx


def default() -> Oracle:
    """The oracle built from ``kvbt_oracle.c`` (built with gcc on first use)."""
    global _default
    with _default_lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _default = Oracle(_LIB_PATH)
        return _default


def total_order_cmp(x_bits: int, y_bits: int) -> int:
    return default().total_order_cmp(x_bits, y_bits)


def select_topk_blocks(*args, **kwargs):
    return default().select_topk_blocks(*args, **kwargs)


def build_sparse_block_table(*args, **kwargs):
    return default().build_sparse_block_table(*args, **kwargs)


def select_topk_and_build_table(*args, **kwargs):
    return default().select_topk_and_build_table(*args, **kwargs)
