"""Checks shared by the CPU and GPU tests: an independent rank key, brute force,
and the invariants every selector / table output must satisfy.

The rank key here is the integer image of IEEE 754 totalOrder on binary32 (flip
all bits of a negative pattern, set the sign bit of a positive one). The oracle
implements totalOrder from the standard's clauses instead, so agreement between
the two is evidence for both.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

BLOCK = 128
PAGE = 16
PAGES_PER_BLOCK = 8


def random_seeds(base: int, n: int) -> list:
    """Seeds of a randomized test: the n fixed seeds base, base + 1, ..., plus as many
    more as the environment variable KVBT_EXTRA_SEEDS says (default 0), taken from
    base * 1000 onwards so that longer campaigns of different tests stay disjoint."""
    extra = int(os.environ.get("KVBT_EXTRA_SEEDS", "0") or 0)
    return list(range(base, base + n)) + list(range(base * 1000, base * 1000 + extra))


def order_key_bits(bits32: np.ndarray) -> np.ndarray:
    """uint64 key whose integer order is the totalOrder of the binary32 patterns."""
    u = np.asarray(bits32, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    neg = (u >> np.uint64(31)) == 1
    return np.where(neg, (~u) & np.uint64(0xFFFFFFFF), u | np.uint64(0x80000000))


def row_bits(scores: np.ndarray) -> np.ndarray:
    """binary32 bit patterns of a float32 array or of a uint16 bf16-bits array."""
    if scores.dtype == np.uint16:
        return scores.astype(np.uint32) << 16
    return np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)


def forced_set(nvp: int, num_init: int, num_local: int) -> set:
    return set(range(min(num_init, nvp))) | set(range(max(0, nvp - num_local), nvp))


def brute_force_set(bits: np.ndarray, nvp: int, topk: int, num_init: int,
                    num_local: int) -> set:
    """The unique subset of size min(topk, nvp) that holds the forced blocks and whose
    scored members all outrank every block left out (rank: key desc, id asc)."""
    F = forced_set(nvp, num_init, num_local)
    size = min(topk, nvp)
    keys = order_key_bits(bits[:nvp])
    rank = {b: (int(keys[b]), -b) for b in range(nvp)}
    hits = []
    for S in itertools.combinations(range(nvp), size):
        S = set(S)
        if not F <= S:
            continue
        out = set(range(nvp)) - S
        if all(rank[s] > rank[o] for s in S - F for o in out):
            hits.append(S)
    assert len(hits) == 1, "brute force found %d upward-closed subsets" % len(hits)
    return hits[0]


def decode_rows(seq_lens, q):
    """(req, causal length c) per row of a request-major decode batch."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    T = seq_lens.shape[0] * q
    req = np.arange(T) // q
    pos = seq_lens[req] - q + (np.arange(T) - req * q)
    return req, np.maximum(pos + 1, 0)


def workload_rows(w):
    """(req, c) per row of a workload, with req = -1 for rows naming no request."""
    if w.explicit:
        req = w.row_req.astype(np.int64).copy()
        c = np.maximum(w.row_pos.astype(np.int64) + 1, 0)
        bad = (req < 0) | (req >= w.B)
        req[bad] = -1
        c[bad] = 0
        return req, c
    return decode_rows(w.seq_lens, w.decode_query_len)


def check_selector(scores, nvp_rows, idx, topk, num_init, num_local, rows=None):
    """Invariants of the selector output, row by row. Returns the number checked."""
    T, H, M = scores.shape
    nvp_rows = np.clip(np.asarray(nvp_rows, dtype=np.int64), 0, M)
    rows = range(T) if rows is None else rows
    n = 0
    for t in rows:
        nvp = int(nvp_rows[t])
        F = forced_set(nvp, num_init, num_local)
        for h in range(H):
            r = idx[t, h]
            nv = min(topk, nvp)
            assert (r[:nv] >= 0).all() and (r[nv:] == -1).all(), (t, h, r, nvp)
            sel = r[:nv]
            assert len(set(sel.tolist())) == nv, (t, h, r)
            assert (sel < nvp).all(), (t, h, r, nvp)
            assert F <= set(sel.tolist()), (t, h, r, F)
            # forced first, by ascending id
            nf = len(F)
            assert sel[:nf].tolist() == sorted(F), (t, h, r, F)
            keys = order_key_bits(row_bits(scores[t, h, :nvp]))
            scored_sel = sel[nf:]
            if len(scored_sel):
                rk = [(int(keys[b]), -int(b)) for b in scored_sel]
                assert all(rk[i] > rk[i + 1] for i in range(len(rk) - 1)), (t, h, r)
                worst = rk[-1]
                left = np.ones(nvp, dtype=bool)
                left[sel] = False
                for b in F:
                    left[b] = False
                lb = np.nonzero(left)[0]
                if len(lb):
                    lk = keys[lb]
                    # no left-out block outranks the weakest selected one
                    better = (lk > worst[0]) | ((lk == worst[0]) & (-lb > worst[1]))
                    assert not better.any(), (t, h, r)
            n += 1
    return n


def dense_pages(bt_row, c):
    """Page-16 ids of the first c tokens of a sequence stored in 128-token blocks."""
    n_pages = min(-(-int(c) // PAGE), len(bt_row) * PAGES_PER_BLOCK)
    out = []
    for p in range(n_pages):
        v = (int(bt_row[p // PAGES_PER_BLOCK]) * PAGES_PER_BLOCK + p % PAGES_PER_BLOCK) \
            & 0xFFFFFFFF
        out.append(v - (1 << 32) if v >= (1 << 31) else v)
    return out


def check_table(idx, block_table, req_rows, c_rows, table, ctx, rows=None):
    """Invariants of the table output. Returns the number of row-heads checked."""
    T, H, K = idx.shape
    max_blocks = block_table.shape[1]
    rows = range(T) if rows is None else rows
    n = 0
    for t in rows:
        req, c = int(req_rows[t]), int(c_rows[t])
        nvp = -(-c // BLOCK)
        for h in range(H):
            row, cx = table[t, h], int(ctx[t, h])
            assert row.shape == (K * PAGES_PER_BLOCK,)
            if c == 0 or req < 0:
                assert cx == 0 and (row == 0).all(), (t, h, cx, row)
                n += 1
                continue
            S = sorted({int(b) for b in idx[t, h] if 0 <= b < min(nvp, max_blocks)})
            assert 0 <= cx <= min(c, BLOCK * K), (t, h, cx)
            # a sparse row is the dense page list of the request restricted to S
            dense = dense_pages(block_table[req], c)
            want = []
            for b in S:
                want += dense[b * PAGES_PER_BLOCK:(b + 1) * PAGES_PER_BLOCK]
            assert row[:len(want)].tolist() == want, (t, h, S)
            assert (row[len(want):] == 0).all(), (t, h)
            # visible tokens: full blocks count 128, the last causal block c - 128(nvp-1)
            want_ctx = sum(BLOCK if b < nvp - 1 else c - BLOCK * (nvp - 1) for b in S)
            assert cx == want_ctx, (t, h, cx, want_ctx)
            n += 1
    return n
