"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every comparison is bit-exact (idx, table and ctx are integers). Outputs are
pre-filled with 0x7F7F7F7F so an unwritten entry cannot pass. Every launch path is
forced onto the same inputs and results must not depend on it:
  policy  whatever the launch policy picks for the batch;
  short   the max_block hint 1: short-row wavefronts only (longer rows loop);
  stream  one streaming wavefront per (row, head): the rows are repeated until the
          batch has more (row, head) pairs than the split path takes, and the first
          copy is compared;
  split   the max_block hint 129: where the policy takes the split path (few pairs,
          16-byte rows) that is a workgroup of one wavefront, so rows longer than
          one chunk go through the split kernel's whole-row branch ("policy" covers
          its several-wavefront branch on the same batches).
"""
import dataclasses

import numpy as np
import pytest

import kvbt_checks as ck
from kv_block_top_amd import workloads as wl

pytestmark = pytest.mark.gpu

POISON = 0x7F7F7F7F
PATHS = ("policy", "short", "stream", "split")
SPLIT_MAX_ROW_HEADS = 256     # no batch with more (row, head) pairs takes the split path


def tile_rows(w, k):
    """The workload with its rows (and, in decode form, its requests) repeated k times."""
    if k == 1:
        return w
    rep = dict(scores=np.tile(w.scores, (k, 1, 1)),
               num_valid_pages=np.tile(w.num_valid_pages, k), name=w.name + "_x%d" % k)
    if w.explicit:
        rep.update(row_req=np.tile(w.row_req, k), row_pos=np.tile(w.row_pos, k))
    else:
        rep.update(seq_lens=np.tile(w.seq_lens, k), block_table=np.tile(w.block_table, (k, 1)))
    return dataclasses.replace(w, **rep)


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_block_top_amd as kvbt
    kvbt.lib()
    return torch, kvbt, torch.device("cuda:0")


def _dev(torch, a, d):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(d).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def _poisoned(torch, shape, d):
    return torch.full(shape, POISON, dtype=torch.int32, device=d)


def gpu_fused(env, w, path="policy", scores_dev=None):
    """Fused call on the launch path named by `path` (see the module docstring)."""
    torch, kvbt, d = env
    if path == "stream" and w.T * w.H <= SPLIT_MAX_ROW_HEADS and scores_dev is None:
        k = SPLIT_MAX_ROW_HEADS // (w.T * w.H) + 1
        out = _gpu_fused(env, tile_rows(w, k), 0)
        return tuple(o[: w.T] for o in out)
    return _gpu_fused(env, w, path_hint(w, path), scores_dev)


def path_hint(w, path):
    """The max_block hint that forces `path` (at most max_k_tiles, as the API requires)."""
    return min({"short": 1, "split": 129}.get(path, 0), w.M)


def _gpu_fused(env, w, max_block, scores_dev=None, num_decode_rows=None):
    torch, kvbt, d = env
    s = scores_dev if scores_dev is not None else _dev(torch, w.scores, d)
    out = (_poisoned(torch, (w.T, w.H, w.topk), d),
           _poisoned(torch, (w.T, w.H, w.topk * 8), d),
           _poisoned(torch, (w.T, w.H), d))
    kw = (dict(row_req=_dev(torch, w.row_req, d), row_pos=_dev(torch, w.row_pos, d))
          if w.explicit else dict(seq_lens=_dev(torch, w.seq_lens, d),
                                  decode_query_len=w.decode_query_len))
    kvbt.select_topk_and_build_table(s, _dev(torch, w.block_table, d), topk=w.topk,
                                     num_init=w.num_init, num_local=w.num_local,
                                     max_block=max_block, out=out,
                                     num_decode_rows=(w.num_decode_rows if num_decode_rows is None
                                                      else num_decode_rows), **kw)
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in out)


def gpu_select_path(env, w, path="policy"):
    """Standalone selector on the launch path named by `path` (as gpu_fused)."""
    if path == "stream" and w.T * w.H <= SPLIT_MAX_ROW_HEADS:
        k = SPLIT_MAX_ROW_HEADS // (w.T * w.H) + 1
        return gpu_select(env, tile_rows(w, k))[: w.T]
    return gpu_select(env, w, path_hint(w, path))


def gpu_select(env, w, max_block=0, num_decode_rows=None):
    torch, kvbt, d = env
    out = _poisoned(torch, (w.T, w.H, w.topk), d)
    nd = w.num_decode_rows if num_decode_rows is None else num_decode_rows
    kvbt.select_topk_blocks(_dev(torch, w.scores, d), _dev(torch, w.num_valid_pages, d),
                            topk=w.topk, num_init=w.num_init, num_local=w.num_local,
                            max_block=max_block, num_decode_rows=nd, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_table(env, w, idx):
    torch, kvbt, d = env
    T, H, K = idx.shape
    ot = _poisoned(torch, (T, H, K * 8), d)
    oc = _poisoned(torch, (T, H), d)
    kw = (dict(row_req=_dev(torch, w.row_req, d), row_pos=_dev(torch, w.row_pos, d))
          if w.explicit else dict(seq_lens=_dev(torch, w.seq_lens, d),
                                  decode_query_len=w.decode_query_len))
    kvbt.build_sparse_block_table(_dev(torch, idx, d), _dev(torch, w.block_table, d),
                                  out_table=ot, out_ctx=oc, **kw)
    torch.cuda.synchronize()
    return ot.cpu().numpy(), oc.cpu().numpy()


def oracle_fused(orc, w, threads=8, rows=None):
    return orc.select_topk_and_build_table(w.scores, w.block_table, topk=w.topk,
                                           num_init=w.num_init, num_local=w.num_local,
                                           threads=threads, rows=rows, **w.row_kwargs())


def assert_same(got, want, what, rows=None):
    names = ("idx", "table", "ctx")
    for name, g, e in zip(names, got, want):
        if rows is not None:
            g, e = g[rows], e[rows]
        if not np.array_equal(g, e):
            bad = np.argwhere(g != e)
            r = tuple(bad[0])
            raise AssertionError("%s %s differs at %d places, first %s: gpu %s oracle %s" % (
                what, name, len(bad), r, g[r[:2]], e[r[:2]]))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_fused(env, orc, n, path):
    w = wl.config(n)
    print("config", n, w.name, "path", path, flush=True)
    got = gpu_fused(env, w, path)
    assert_same(got, oracle_fused(orc, w), "config %d %s" % (n, path))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_standalone(env, orc, n):
    w = wl.config(n)
    idx = gpu_select(env, w)
    want = orc.select_topk_blocks(w.scores, w.num_valid_pages, topk=w.topk, threads=8)
    assert np.array_equal(idx, want)
    table, ctx = gpu_table(env, w, idx)
    ot, oc = orc.build_sparse_block_table(want, w.block_table, threads=8, **w.row_kwargs())
    assert np.array_equal(table, ot) and np.array_equal(ctx, oc)
    fused = gpu_fused(env, w)
    assert_same(fused, (idx, table, ctx), "fused vs standalone config %d" % n)


def test_workload5_full(env, orc):
    """The long-context mixed buffer at full size (8320 rows x 4 heads x 8192 tiles), in
    the launch configuration the benchmark times; every row checked against the oracle."""
    w = wl.config(5)
    print("config 5", w.name, flush=True)
    got = gpu_fused(env, w)
    print("gpu done", flush=True)
    want = oracle_fused(orc, w, threads=16)
    print("oracle done", flush=True)
    assert_same(got, want, "config 5")
    idx = gpu_select(env, w)
    assert np.array_equal(idx, got[0])


@pytest.mark.parametrize("bf16", [False, True])
def test_decode_rows_hint_changes_only_the_order(env, orc, bf16):
    """num_decode_rows reorders the streaming launch's visit (the leading rows first,
    the rest from the last to the first); the outputs must not depend on it: the mixed
    buffer's layout (128 decode rows, 32 requests x 4, then four prefill requests) at
    600 tiles and 160-token prefills."""
    w = wl.config5(max_k_tiles=600, prefill_len=160)
    assert w.num_decode_rows == 128 and w.T == 128 + 4 * 160
    if bf16:
        w = dataclasses.replace(w, scores=wl.f32_to_bf16_bits(w.scores))
    want = oracle_fused(orc, w)
    for nd in (0, 1, 5, 127, 128, 129, w.T // 2, w.T - 1, w.T):
        print("num_decode_rows", nd, flush=True)
        assert_same(_gpu_fused(env, w, 0, num_decode_rows=nd), want, "nd %d" % nd)
        assert np.array_equal(gpu_select(env, w, num_decode_rows=nd), want[0]), "nd %d" % nd


# ---------------------------------------------------------------------------
# randomized cases: every parameter drawn from a seed
# ---------------------------------------------------------------------------

RANDOM_MS = list(range(1, 300, 7)) + [511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2048,
                                      2049, 4096, 4100, 8191, 8192]


def random_parity_case(seed):
    """A workload with every parameter drawn from `seed`: capacity (a few past 8192
    tiles), rows, heads, dtype, top-k and forced counts, value kind, row lengths (empty,
    full, beyond the capacity), block-table width, tail content, visiting-order hint; and a
    launch path."""
    rng = np.random.default_rng(seed)
    M = int(rng.choice(RANDOM_MS)) if rng.random() > 0.05 else int(rng.choice([8193, 12000, 16384]))
    T, H = int(rng.integers(1, 65)), int(rng.integers(1, 5))
    bf16 = bool(rng.integers(0, 2))
    topk = int(rng.integers(1, 17))
    ni = int(rng.integers(0, topk + 1))
    nl = int(rng.integers(0, topk - ni + 1))
    kind = str(rng.choice(KINDS))
    full = rng.random() < 0.3
    lens = np.where(rng.random(T) < 0.1, rng.integers(0, 3, T),
                    rng.integers(1, M * 128 + 300, T)).tolist()
    if full:
        lens = [M * 128] * T
    mb = None if rng.random() < 0.7 else int(rng.integers(1, M + 50))
    w = wl.rows_case(seed, lens, H=H, M=M, bf16=bf16, kind=kind, topk=topk, num_init=ni,
                     num_local=nl, max_blocks=mb,
                     tail=str(rng.choice(["neginf", "nan", "random"])))
    w = dataclasses.replace(w, num_decode_rows=int(rng.integers(0, T + 1)))
    return w, str(rng.choice(PATHS))


@pytest.mark.parametrize("seed", ck.random_seeds(9000, 64))
def test_randomized_cases(env, orc, seed):
    w, path = random_parity_case(seed)
    print("seed", seed, w.name, w.T, w.H, w.M, w.topk, w.num_init, w.num_local, path,
          w.num_decode_rows, flush=True)
    want = oracle_fused(orc, w)
    assert_same(gpu_fused(env, w, path), want, "seed %d %s" % (seed, path))
    assert np.array_equal(gpu_select_path(env, w, path), want[0]), "standalone seed %d" % seed


# ---------------------------------------------------------------------------
# edge sweeps
# ---------------------------------------------------------------------------

EDGE_BLOCKS = [1, 2, 3, 4, 15, 16, 17, 63, 64, 65, 73, 74, 127, 128, 129, 130, 255, 256,
               257, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8192]


def _edge_lens(M):
    lens = [0, 1, 2]
    for b in EDGE_BLOCKS:
        if b <= M:
            lens += [128 * (b - 1) + 1, 128 * b - 1, 128 * b]
    lens.append(128 * M + 5000)     # longer than the capacity: clamped to M blocks
    return lens


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [74, 129, 512, 1000, 8192])
@pytest.mark.parametrize("path", PATHS)
def test_edge_block_counts(env, orc, M, bf16, path):
    w = wl.rows_case(10 + M, _edge_lens(M), H=2, M=M, bf16=bf16, kind="specials")
    print(w.name, M, bf16, path, flush=True)
    assert_same(gpu_fused(env, w, path), oracle_fused(orc, w), "edge %d" % M)


KINDS = ["normal", "specials", "ties", "negative", "neginf", "nan", "increasing", "two_level"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [300, 2048, 8192])
def test_degenerate_rows(env, orc, M, bf16, kind):
    lens = [128 * M, 128 * (M // 2) + 7, 128 * 129, 128 * 200 - 3, 128 * 16, 100]
    w = wl.rows_case(20 + M, lens, H=3, M=M, bf16=bf16, kind=kind)
    print(w.name, M, bf16, flush=True)
    want = oracle_fused(orc, w)
    for path in PATHS:
        assert_same(gpu_fused(env, w, path), want, "%s %d %s" % (kind, M, path))
        got = gpu_select_path(env, w, path)
        assert np.array_equal(got, want[0]), "standalone %s %d %s" % (kind, M, path)


WIDE_KINDS = ["normal", "specials", "ties", "increasing", "two_level", "neginf"]


@pytest.mark.parametrize("kind", WIDE_KINDS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [8193, 16384, 65536])
def test_beyond_fast_path(env, orc, M, bf16, kind):
    """max_k_tiles over 8192: 24-bit block ids in the keys, one wavefront per 8192-tile
    segment; segment boundaries, short rows and full rows. The hints 1 and 129 give a
    workgroup of one wavefront, so longer rows take wavefront 0's segment loop."""
    lens = [0, 1, 100 * 128, 128 * 128, 128 * 129, 128 * 8191 + 5, 128 * 8192,
            128 * 8192 + 1, 128 * 8193, 128 * (M // 2) + 77, 128 * M]
    w = wl.rows_case(90 + M % 97, lens, H=2, M=M, bf16=bf16, kind=kind)
    print(w.name, M, bf16, kind, flush=True)
    want = oracle_fused(orc, w)
    for path in ("policy", "short", "split"):
        assert_same(gpu_fused(env, w, path), want, "wide %s %d %s" % (kind, M, path))
    assert np.array_equal(gpu_select(env, w), want[0])


@pytest.mark.parametrize("kind", ["normal", "specials", "ties"])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [65537, 200003, 1 << 20])
def test_past_65536_tiles(env, orc, M, bf16, kind):
    """max_k_tiles past 65536: at most 8 wavefronts per (row, head), wavefront w taking
    segments w, w + 8, ...; block ids past 16 bits in the keys and the table. The hints
    1 and 129 leave one wavefront to take every segment, 8193 two. 200003 tiles are not
    16-byte rows (single-element loads)."""
    lens = [0, 1, 128 * 8192 + 1, 128 * 65536, 128 * 65536 + 1, 128 * (M // 2) + 77,
            128 * M - 5, 128 * M]
    w = wl.rows_case(95 + M % 89, lens, H=2, M=M, bf16=bf16, kind=kind)
    print(w.name, M, bf16, kind, flush=True)
    want = oracle_fused(orc, w)
    for path in ("policy", "short", "split"):
        assert_same(gpu_fused(env, w, path), want, "past 65536 %s %d %s" % (kind, M, path))
    assert_same(_gpu_fused(env, w, 8193), want, "past 65536 %s %d hint 8193" % (kind, M))
    assert np.array_equal(gpu_select(env, w), want[0])


@pytest.mark.parametrize("bf16", [False, True])
def test_largest_capacity(env, orc, bf16):
    """max_k_tiles = 2^24: a row reaching the last block an int32 token position can
    (position 2^31 - 1), one ending just inside its last block, one much shorter."""
    M = env[1].MAX_K_TILES
    assert M == 1 << 24
    lens = [128 * M, 128 * (M - 1) + 1, 128 * 70001 + 3]
    w = wl.rows_case(97, lens, H=1, M=M, bf16=bf16, kind="normal")
    print(w.name, M, bf16, flush=True)
    want = oracle_fused(orc, w)
    for path in ("policy", "split"):
        assert_same(gpu_fused(env, w, path), want, "largest %s" % path)
    assert np.array_equal(gpu_select(env, w), want[0])


@pytest.mark.parametrize("topk,ni,nl", [(1, 0, 0), (1, 1, 0), (1, 0, 1), (2, 1, 1), (3, 1, 2),
                                        (5, 0, 0), (8, 2, 3), (16, 0, 0), (16, 8, 8),
                                        (16, 1, 2), (13, 4, 0)])
@pytest.mark.parametrize("M", [96, 700, 4100])
@pytest.mark.parametrize("bf16", [False, True])
def test_topk_and_forced_counts(env, orc, topk, ni, nl, M, bf16):
    # lengths of 1 to 3 and 17 to 300 blocks: bf16 rows of 129..512 blocks take the
    # preloaded-chunks code on the streaming launch path
    lens = [1, 129, 128 * 3, 128 * 17 + 1, 128 * min(M, 300), 128 * 129 + 1, 128 * 255 + 3,
            128 * 256, 128 * 257, 128 * 511 + 9, 128 * M]
    w = wl.rows_case(30 + topk + M, lens, H=2, M=M, kind="specials", topk=topk,
                     num_init=ni, num_local=nl, bf16=bf16)
    want = oracle_fused(orc, w)
    for path in PATHS:
        assert_same(gpu_fused(env, w, path), want, "topk %d %s" % (topk, path))
        got = gpu_select_path(env, w, path)
        assert np.array_equal(got, want[0]), "standalone topk %d %s" % (topk, path)


@pytest.mark.parametrize("tail", ["nan", "random"])
@pytest.mark.parametrize("bf16", [False, True])
def test_tail_content_is_ignored(env, orc, tail, bf16):
    lens = _edge_lens(1024)
    base = wl.rows_case(40, lens, H=2, M=1024, bf16=bf16, kind="normal", tail="neginf")
    other = wl.rows_case(40, lens, H=2, M=1024, bf16=bf16, kind="normal", tail=tail)
    want = oracle_fused(orc, base)
    for path in PATHS:
        assert_same(gpu_fused(env, other, path), want, "tail %s %s" % (tail, path))


@pytest.mark.parametrize("q", [1, 2, 4, 8])
@pytest.mark.parametrize("bf16", [False, True])
def test_decode_forms(env, orc, q, bf16):
    w = wl.random_case(50 + q, T=16 * q, H=2, M=150, bf16=bf16, q=q, seq_lo=0,
                       seq_hi=150 * 128, special_frac=0.05, tie_frac=0.05)
    want = oracle_fused(orc, w)
    for path in PATHS:
        assert_same(gpu_fused(env, w, path), want, "q %d %s" % (q, path))


@pytest.mark.parametrize("seed", range(6))
def test_explicit_rows_and_small_block_tables(env, orc, seed):
    rng = np.random.default_rng(seed)
    M = int(rng.choice([40, 129, 600]))
    w = wl.random_case(60 + seed, T=40, H=int(rng.integers(1, 5)), M=M, bf16=bool(seed % 2),
                       explicit=True, max_blocks=int(rng.integers(1, M + 1)),
                       special_frac=0.05)
    w.row_req[::7] = -1                  # rows naming no request
    w.row_req[3::11] = w.B + 2
    want = oracle_fused(orc, w)
    for path in PATHS:
        assert_same(gpu_fused(env, w, path), want, "explicit seed %d %s" % (seed, path))


@pytest.mark.parametrize("seed", range(4))
def test_table_builder_on_arbitrary_idx(env, orc, seed):
    """Repeats, -1 anywhere, ids past the causal count or the block table."""
    rng = np.random.default_rng(70 + seed)
    w = wl.random_case(70 + seed, T=64, H=3, M=200, q=4, max_blocks=int(rng.integers(1, 210)))
    K = int(rng.choice([1, 4, 16]))
    idx = rng.integers(-3, 210, size=(w.T, w.H, K)).astype(np.int32)
    if K > 1:
        idx[:, :, 1] = idx[:, :, 0]
    table, ctx = gpu_table(env, w, idx)
    ot, oc = orc.build_sparse_block_table(idx, w.block_table, **w.row_kwargs())
    assert np.array_equal(table, ot) and np.array_equal(ctx, oc)


def test_spec_decode_worked_example(env, orc):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "spec_decode_table_example.json")))
    w = wl.Workload(name="example", scores=np.zeros((12, 1, 3), np.float32),
                    block_table=np.array(g["block_table"], np.int32),
                    num_valid_pages=np.zeros(12, np.int32),
                    seq_lens=np.array(g["seq_lens"], np.int32), decode_query_len=4, topk=4)
    idx = np.array(g["topk_idx"], np.int32)[:, None, :]
    table, ctx = gpu_table(env, w, idx)
    for part in ("pinned_by_page", "by_reading"):
        p = g[part]
        for r, c, prefix in zip(p["rows"], p["ctx"], p["table_prefix"]):
            assert int(ctx[r, 0]) == c
            assert table[r, 0].tolist() == prefix + [0] * (32 - len(prefix))


# ---------------------------------------------------------------------------
# launch properties
# ---------------------------------------------------------------------------

def test_misaligned_scores_pointer(env, orc):
    torch, kvbt, d = env
    w = wl.rows_case(80, _edge_lens(1024), H=2, M=1024, kind="specials")
    flat = torch.empty(w.scores.size + 1, dtype=torch.float32, device=d)
    s = flat[1:].view(w.T, w.H, w.M)
    s.copy_(torch.from_numpy(w.scores).to(d))
    assert s.data_ptr() % 16 != 0
    assert_same(gpu_fused(env, w, "policy", scores_dev=s), oracle_fused(orc, w), "misaligned")


def test_empty_batch(env):
    torch, kvbt, d = env
    s = torch.empty(0, 2, 74, dtype=torch.bfloat16, device=d)
    bt = torch.zeros(0, 74, dtype=torch.int32, device=d)
    sl = torch.zeros(0, dtype=torch.int32, device=d)
    idx, table, ctx = kvbt.select_topk_and_build_table(s, bt, seq_lens=sl, decode_query_len=4)
    torch.cuda.synchronize()
    assert idx.shape == (0, 2, 16) and table.shape == (0, 2, 128) and ctx.shape == (0, 2)


def _replay_check(env, w, want, what):
    """Repeated eager calls, then four replays of a captured graph with the outputs
    poisoned before each: every result must equal the oracle's."""
    torch, kvbt, d = env
    s = _dev(torch, w.scores, d)
    bt = _dev(torch, w.block_table, d)
    kw = (dict(row_req=_dev(torch, w.row_req, d), row_pos=_dev(torch, w.row_pos, d))
          if w.explicit else dict(seq_lens=_dev(torch, w.seq_lens, d),
                                  decode_query_len=w.decode_query_len))
    out = (torch.empty(w.T, w.H, w.topk, dtype=torch.int32, device=d),
           torch.empty(w.T, w.H, w.topk * 8, dtype=torch.int32, device=d),
           torch.empty(w.T, w.H, dtype=torch.int32, device=d))

    def call():
        kvbt.select_topk_and_build_table(s, bt, topk=w.topk, num_init=w.num_init,
                                         num_local=w.num_local, out=out, **kw)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert_same(tuple(o.cpu().numpy() for o in out), want, "repeat " + what)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for o in out:
            o.fill_(POISON)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(tuple(o.cpu().numpy() for o in out), want, "replay %d of %s" % (rep, what))


def test_repeat_and_graph_replay(env, orc):
    """Repeated calls give identical bytes; so does every replay of a captured graph
    (the library keeps no state between calls and uses no memset), on each launch
    path: short rows, one streaming wavefront per row, and the split path."""
    torch, kvbt, d = env
    for n in (2, 3):
        w = wl.config(n)
        _replay_check(env, w, oracle_fused(orc, w), "config %d" % n)
    lens = [128 * 8192, 128 * 5000 + 3, 128 * 1500, 128 * 300 + 1, 128 * 129, 100]
    few = wl.rows_case(80, lens, H=2, M=8192, kind="normal")
    assert kvbt.launch_policy(0, 8192, kvbt.F32, few.T, few.H)["path"] == 2
    _replay_check(env, few, oracle_fused(orc, few), "split")
    many = tile_rows(few, 30)
    assert kvbt.launch_policy(0, 8192, kvbt.F32, many.T, many.H)["path"] == 1
    _replay_check(env, many, oracle_fused(orc, many), "stream")


def test_invariants_on_random_long_rows(env):
    """Invariants at a size the test does not oracle row by row."""
    w = wl.rows_case(90, list(np.random.default_rng(9).integers(1, 128 * 8192, size=300)),
                     H=4, M=8192, kind="normal")
    idx, table, ctx = gpu_fused(env, w)
    req, c = ck.workload_rows(w)
    nvp = np.minimum(-(-c // 128), w.M)
    ck.check_selector(w.scores, nvp, idx, 16, 1, 2, rows=range(0, w.T, 5))
    ck.check_table(idx, w.block_table, req, c, table, ctx, rows=range(0, w.T, 5))


def test_bench_helpers_run(env):
    """The measurement helpers launch and finish on a ragged size (copy checked)."""
    torch, kvbt, d = env
    n = 100000 * 16 + 48
    src = torch.arange(n // 4, dtype=torch.int32, device=d)
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=d)
    kvbt.bench_copy(dst, src, n)
    kvbt.bench_read(src, n, sink)
    kvbt.bench_empty(3)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
