"""Pins of the CPU oracle against facts other than itself (CPU only).

- IEEE 754 totalOrder: a list of binary32 patterns in known ascending order
  (tests/golden/total_order_binary32.json) and numpy's numeric order.
- Brute force over every candidate subset on tiny rows, using an integer rank key
  written independently of the oracle's clause-based comparator.
- A library special case: with no forced blocks and finite, nonzero scores the
  selector is numpy's stable argsort of the negated scores.
- Closed forms: rows with at most num_init + num_local causal blocks select all of
  them in id order; rows with at most topk causal blocks give ctx == c and the
  request's dense page list; valid count == min(topk, cdiv(c, 128)).
- The worked spec-decode example of the PR #47984 page (tests/golden).
- Invariants on the five workloads and on random cases with special values.
"""
import json
import os

import numpy as np
import pytest

import kvbt_checks as ck
from kv_block_top_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_list(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# totalOrder
# ---------------------------------------------------------------------------

def test_total_order_standard_list(orc):
    g = _bits_list("total_order_binary32.json")
    vals = [int(x, 16) for x in g["ascending_bits"]]
    for i, a in enumerate(vals):
        for j, b in enumerate(vals):
            assert orc.total_order_cmp(a, b) == (i > j) - (i < j), (hex(a), hex(b))


def test_total_order_matches_numeric_order(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal(400).astype(np.float32) * np.float32(1e3)
    x[:50] = np.float32(0.5)            # numerically equal pairs
    bits = x.view(np.uint32)
    for i in range(0, 400, 7):
        for j in range(0, 400, 5):
            want = int(np.sign(np.float64(x[i]) - np.float64(x[j])))
            assert orc.total_order_cmp(int(bits[i]), int(bits[j])) == want


def test_total_order_matches_integer_key(orc):
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=3000, dtype=np.uint64).astype(np.uint32)
    keys = ck.order_key_bits(bits)
    for i in range(0, 3000, 3):
        j = (i * 7 + 1) % 3000
        want = (keys[i] > keys[j]) * 1 - (keys[i] < keys[j]) * 1
        assert orc.total_order_cmp(int(bits[i]), int(bits[j])) == want


# ---------------------------------------------------------------------------
# brute force on tiny rows
# ---------------------------------------------------------------------------

SPECIAL32 = np.array([0x7FC00000, 0x7F800000, 0xFF800000, 0x0, 0x80000000,
                      0xFFC00000, 0x7F800001, 0x3F800000], dtype=np.uint32)


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(100 + seed)
    M = 12
    T, H = 6, 2
    x = rng.standard_normal((T, H, M)).astype(np.float32)
    bits = x.view(np.uint32)
    # specials and ties
    u = rng.random((T, H, M))
    bits[u < 0.3] = SPECIAL32[rng.integers(0, len(SPECIAL32), size=(u < 0.3).sum())]
    tie = (u >= 0.3) & (u < 0.45)
    bits[tie] = bits.reshape(-1)[rng.integers(0, bits.size, size=tie.sum())]
    nvp = rng.integers(0, M + 1, size=T).astype(np.int32)
    topk = int(rng.integers(1, 6))
    ni = int(rng.integers(0, 2))
    nl = int(rng.integers(0, 3))
    if ni + nl > topk:
        nl = max(0, topk - ni)
    idx = orc.select_topk_blocks(x, nvp, topk=topk, num_init=ni, num_local=nl)
    for t in range(T):
        for h in range(H):
            S = ck.brute_force_set(bits[t, h], int(nvp[t]), topk, ni, nl)
            got = idx[t, h]
            nv = min(topk, int(nvp[t]))
            assert set(got[:nv].tolist()) == S
            assert (got[nv:] == -1).all()
    ck.check_selector(x, nvp, idx, topk, ni, nl)


# ---------------------------------------------------------------------------
# library special case: stable argsort
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("topk", [16, 17, 32, 64])
@pytest.mark.parametrize("seed", range(6))
def test_argsort_special_case(orc, seed, topk):
    rng = np.random.default_rng(200 + seed)
    T, H, M = 16, 3, 300
    x = rng.standard_normal((T, H, M)).astype(np.float32)
    # ties: copy a random earlier element into 10% of the slots; no zeros
    for t in range(T):
        for h in range(H):
            for b in rng.integers(1, M, size=30):
                x[t, h, b] = x[t, h, rng.integers(0, b)]
    x[x == 0] = np.float32(1e-3)
    nvp = rng.integers(0, M + 1, size=T).astype(np.int32)
    nvp[:4] = [topk - 1, topk, topk + 1, 0]
    idx = orc.select_topk_blocks(x, nvp, topk=topk, num_init=0, num_local=0)
    for t in range(T):
        n = int(nvp[t])
        for h in range(H):
            want = np.argsort(-x[t, h, :n], kind="stable")[:topk]
            want = np.concatenate([want, -np.ones(topk - len(want), dtype=np.int64)])
            assert idx[t, h].tolist() == want.tolist()


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_all_forced_rows(orc):
    rng = np.random.default_rng(7)
    T, H, M = 40, 2, 8
    x = rng.standard_normal((T, H, M)).astype(np.float32)
    x.view(np.uint32)[:, :, 0] = 0xFF800000          # -inf at the init block
    x.view(np.uint32)[:, 0, 1] = 0xFFC00000          # -NaN inside the window
    nvp = np.arange(T, dtype=np.int32) % 4           # 0..3 blocks
    idx = orc.select_topk_blocks(x, nvp, topk=16, num_init=1, num_local=2)
    for t in range(T):
        n = int(nvp[t])
        for h in range(H):
            assert idx[t, h].tolist() == list(range(n)) + [-1] * (16 - n)


def test_dense_table_when_everything_fits(orc):
    """Config 1: every row has at most 16 causal blocks, so all of them are kept and the
    sparse row is the request's dense page-16 list with ctx equal to the causal length."""
    w = wl.config(1)
    idx, table, ctx = orc.select_topk_and_build_table(
        w.scores, w.block_table, topk=16, **w.row_kwargs())
    req, c = ck.workload_rows(w)
    for t in range(w.T):
        dense = ck.dense_pages(w.block_table[req[t]], c[t])
        for h in range(w.H):
            assert int(ctx[t, h]) == c[t]
            assert table[t, h, :len(dense)].tolist() == dense
            assert (table[t, h, len(dense):] == 0).all()


@pytest.mark.parametrize("topk", [17, 32, 64])
def test_dense_table_and_order_when_everything_fits_wide_topk(orc, topk):
    """topk above 16: rows of at most topk causal blocks keep all of them (ctx equals
    the causal length, the table is the dense page list); the order is the forced blocks
    in ascending id, then the rest by score descending (checked against numpy's stable
    argsort of the negated scores)."""
    rng = np.random.default_rng(900 + topk)
    T, H, M = 24, 2, topk + 8
    lens = np.concatenate([[1, 128, 129, 128 * (topk - 1) + 5, 128 * topk, 128 * topk + 1],
                           rng.integers(1, 128 * M + 1, size=T - 6)])
    w = wl.rows_case(901 + topk, lens, H=H, M=M, kind="normal", topk=topk)
    idx, table, ctx = orc.select_topk_and_build_table(
        w.scores, w.block_table, topk=topk, num_init=1, num_local=2, **w.row_kwargs())
    req, c = ck.workload_rows(w)
    nvp = np.minimum(-(-c // 128), M)
    for t in range(T):
        n = int(nvp[t])
        dense = ck.dense_pages(w.block_table[req[t]], c[t])
        for h in range(H):
            forced = sorted({0} & set(range(n)) | set(range(max(0, n - 2), n)))
            rest = [b for b in np.argsort(-w.scores[t, h, :n], kind="stable") if b not in forced]
            want = (forced + rest)[:topk]
            assert idx[t, h].tolist() == want + [-1] * (topk - len(want))
            if n <= topk:
                assert int(ctx[t, h]) == c[t]
                assert table[t, h, :len(dense)].tolist() == dense
                assert (table[t, h, len(dense):] == 0).all()
    ck.check_selector(w.scores, nvp, idx, topk, 1, 2)
    ck.check_table(idx, w.block_table, req, c, table, ctx)


def test_partial_block_pages(orc):
    """c = 128 n gives n full blocks; c = 128 n + 1 adds one page holding one token."""
    bt = np.array([[3, 9, 4, 6]], dtype=np.int32)
    for c, want_ctx, want in [
        (256, 256, [24 + j for j in range(8)] + [72 + j for j in range(8)]),
        (257, 257, [24 + j for j in range(8)] + [72 + j for j in range(8)] + [32]),
        (1, 1, [24]),
        (17, 17, [24, 25]),
    ]:
        idx = np.array([[[0, 1, 2, 3]]], dtype=np.int32)
        table, ctx = orc.build_sparse_block_table(idx, bt, row_req=np.array([0]),
                                                  row_pos=np.array([c - 1]))
        assert int(ctx[0, 0]) == want_ctx
        assert table[0, 0, :len(want)].tolist() == want
        assert (table[0, 0, len(want):] == 0).all()


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_valid_count_is_min_topk_cdiv(orc, n):
    """The valid count equals min(topk, cdiv(kv_len, 128)) on every row."""
    w = wl.config(n)
    idx, _, _ = orc.select_topk_and_build_table(w.scores, w.block_table, topk=w.topk,
                                                **w.row_kwargs())
    _, c = ck.workload_rows(w)
    nvp = np.minimum(-(-c // 128), w.M)
    valid = (idx >= 0).sum(axis=2)
    assert (valid == np.minimum(w.topk, nvp)[:, None]).all()


# ---------------------------------------------------------------------------
# the worked example of the spec-decode page
# ---------------------------------------------------------------------------

def test_spec_decode_worked_example(orc):
    g = _bits_list("spec_decode_table_example.json")
    q = g["decode_query_len"]
    idx = np.array(g["topk_idx"], dtype=np.int32)[:, None, :]
    table, ctx = orc.build_sparse_block_table(idx, np.array(g["block_table"]),
                                              seq_lens=np.array(g["seq_lens"]),
                                              decode_query_len=q)
    K = idx.shape[2]
    for part in ("pinned_by_page", "by_reading"):
        p = g[part]
        for r, want_ctx, prefix in zip(p["rows"], p["ctx"], p["table_prefix"]):
            assert int(ctx[r, 0]) == want_ctx, (part, r)
            want = prefix + [0] * (K * 8 - len(prefix))
            assert table[r, 0].tolist() == want, (part, r)


def test_decode_form_equals_explicit_form(orc):
    w = wl.random_case(5, T=24, H=2, M=30, q=4, seq_lo=0, seq_hi=30 * 128)
    a = orc.select_topk_and_build_table(w.scores, w.block_table, **w.row_kwargs())
    req, c = ck.decode_rows(w.seq_lens, 4)
    b = orc.select_topk_and_build_table(w.scores, w.block_table,
                                        row_req=req.astype(np.int32),
                                        row_pos=(c - 1).astype(np.int32))
    for x, y in zip(a, b):
        assert (x == y).all()


# ---------------------------------------------------------------------------
# special values and ties
# ---------------------------------------------------------------------------

def _sel(orc, bits32, nvp, topk=16, ni=1, nl=2):
    x = np.asarray(bits32, dtype=np.uint32).view(np.float32)[None, None, :]
    return orc.select_topk_blocks(x, np.array([nvp], dtype=np.int32), topk=topk,
                                  num_init=ni, num_local=nl)[0, 0].tolist()


def test_signed_zero_rows(orc):
    bits = [0x80000000, 0x0, 0x80000000, 0x0, 0x0, 0x80000000, 0x0, 0x80000000, 0x0, 0x0]
    # forced 0, 8, 9; then +0 at 1, 3, 4, 6; then -0 at 2, 5, 7
    assert _sel(orc, bits, 10, topk=10) == [0, 8, 9, 1, 3, 4, 6, 2, 5, 7]


def test_nan_above_inf(orc):
    bits = [0x3F800000, 0x7F800000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0x0, 0x0, 0x0]
    assert _sel(orc, bits, 8, topk=6, ni=0, nl=0) == [2, 4, 1, 0, 5, 6]


def test_nan_at_forced_tile(orc):
    bits = [0xFFC00000, 0x40000000, 0x7FC00000, 0x3F800000, 0xFFC00000, 0xFF800000]
    assert _sel(orc, bits, 6, topk=4) == [0, 4, 5, 2]


def test_ties_break_to_lower_id(orc):
    bits = np.full(200, 0x3F000000, dtype=np.uint32)
    bits[64] = bits[128] = 0x40000000
    bits[100] = 0x40000000
    got = _sel(orc, bits, 200, topk=8, ni=0, nl=0)
    assert got == [64, 100, 128, 0, 1, 2, 3, 4]


def test_bf16_equals_widened_fp32(orc):
    w = wl.random_case(21, T=16, H=2, M=70, bf16=True, special_frac=0.1, tie_frac=0.1)
    widened = wl.bf16_bits_to_f32(w.scores)
    a = orc.select_topk_blocks(w.scores, w.num_valid_pages)
    b = orc.select_topk_blocks(widened, w.num_valid_pages)
    assert (a == b).all()


@pytest.mark.parametrize("bf16", [False, True])
def test_tail_content_is_never_read(orc, bf16):
    outs = []
    for tail in ("neginf", "nan", "random"):
        w = wl.random_case(31, T=12, H=2, M=50, bf16=bf16, tail=tail, special_frac=0.05)
        outs.append(orc.select_topk_and_build_table(w.scores, w.block_table,
                                                    **w.row_kwargs()))
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            assert (x == y).all()


def test_threads_and_row_subsets_agree(orc):
    w = wl.config(3)
    a = orc.select_topk_and_build_table(w.scores, w.block_table, **w.row_kwargs())
    b = orc.select_topk_and_build_table(w.scores, w.block_table, threads=4,
                                        **w.row_kwargs())
    rows = [0, 5, 17, 255]
    c = orc.select_topk_and_build_table(w.scores, w.block_table, rows=rows,
                                        **w.row_kwargs())
    for x, y, z in zip(a, b, c):
        assert (x == y).all()
        assert (x[rows] == z[rows]).all()


def test_out_of_range_request_is_padded(orc):
    bt = np.array([[1, 2], [3, 4]], dtype=np.int32)
    idx = np.array([[[0, 1]], [[0, 1]], [[0, 1]]], dtype=np.int32)
    table, ctx = orc.build_sparse_block_table(idx, bt, row_req=np.array([0, 2, -1]),
                                              row_pos=np.array([200, 200, 200]))
    assert ctx[:, 0].tolist() == [201, 0, 0]
    assert (table[1:] == 0).all()


# ---------------------------------------------------------------------------
# invariants on the workloads and random cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_invariants(orc, n):
    w = wl.config(n)
    idx, table, ctx = orc.select_topk_and_build_table(
        w.scores, w.block_table, topk=w.topk, num_init=w.num_init,
        num_local=w.num_local, threads=4, **w.row_kwargs())
    req, c = ck.workload_rows(w)
    nvp = np.minimum(-(-c // 128), w.M)
    rows = range(w.T) if n != 4 else range(0, w.T, 3)
    ck.check_selector(w.scores, nvp, idx, w.topk, w.num_init, w.num_local, rows=rows)
    ck.check_table(idx, w.block_table, req, c, table, ctx, rows=rows)
    # the standalone selector on the generator's page counts gives the same idx
    idx2 = orc.select_topk_blocks(w.scores, w.num_valid_pages, topk=w.topk, threads=4)
    assert (idx2 == idx).all()
    t2, c2 = orc.build_sparse_block_table(idx, w.block_table, threads=4, **w.row_kwargs())
    assert (t2 == table).all() and (c2 == ctx).all()


@pytest.mark.parametrize("seed", range(8))
def test_random_invariants(orc, seed):
    rng = np.random.default_rng(seed)
    q = int(rng.choice([1, 2, 4]))
    M = int(rng.choice([5, 17, 64, 65, 129, 300]))
    w = wl.random_case(1000 + seed, T=8 * q, H=int(rng.integers(1, 4)), M=M,
                       bf16=bool(seed % 2), q=q, special_frac=0.05, tie_frac=0.05,
                       topk=int(rng.choice([1, 3, 16])), num_init=1,
                       num_local=int(rng.integers(0, 3)) if seed % 3 else 0,
                       max_blocks=int(rng.integers(1, M + 3)),
                       explicit=bool(seed % 4 == 3))
    if w.num_init + w.num_local > w.topk:
        w.num_local = w.topk - w.num_init
    idx, table, ctx = orc.select_topk_and_build_table(
        w.scores, w.block_table, topk=w.topk, num_init=w.num_init,
        num_local=w.num_local, **w.row_kwargs())
    req, c = ck.workload_rows(w)
    nvp = np.minimum(-(-c // 128), w.M)
    ck.check_selector(w.scores, nvp, idx, w.topk, w.num_init, w.num_local)
    ck.check_table(idx, w.block_table, req, c, table, ctx)


def test_builder_input_hygiene(orc):
    """-1 anywhere, ids past the causal count or the block table, and repeats are
    dropped; what remains is a set, listed as the request's dense pages."""
    rng = np.random.default_rng(77)
    B, max_blocks, K = 5, 6, 8
    bt = rng.permutation(1000)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    seq_lens = np.array([900, 129, 0, 5, 768], dtype=np.int32)
    T = B
    idx = rng.integers(-3, 9, size=(T, 2, K)).astype(np.int32)
    idx[:, :, 1] = idx[:, :, 0]                     # repeats
    idx[:, :, 3] = -1                               # -1 in the middle
    table, ctx = orc.build_sparse_block_table(idx, bt, seq_lens=seq_lens, decode_query_len=1)
    req, c = ck.decode_rows(seq_lens, 1)
    ck.check_table(idx, bt, req, c, table, ctx)
    # row 0: c = 900 -> 8 causal blocks, but the table has only 6 columns
    S = sorted({int(b) for b in idx[0, 0] if 0 <= b < 6})
    assert int(ctx[0, 0]) == 128 * len(S)
