"""GPU parity of the decode index-score producer against the CPU oracle.

The HIP kernel (through the C ABI) and oracle/index_scores.py take the same seeded
inputs. Which entries are written must match exactly (the others keep a NaN
sentinel); the written values are floating point and must lie within a bound derived
from the kernel's arithmetic (the oracle is float64 on the same bf16 inputs):

  |gpu - oracle| <= 2^-16 * bound + 2^-14 + 2^-20 * |oracle|   (+ 2^-8 * |oracle| for bf16)

bound = scale * max over the block's tokens of sum_d |q_d k_d|: the kernel sums 128
exact products in fp32 (error at most 128 * 2^-24 of that sum, i.e. 2^-17), and the max
or log-sum-exp of the sums carries at most that error; the hardware exp2/log2 and the
fp32 sum of at most 128 terms add a few 2^-20 in the log domain (2^-14 is a margin of
several times that), the final scaling a relative 2^-22. A bf16 output adds its rounding.
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl
from kvbt_checks import random_seeds

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_block_top_amd as kvbt
    kvbt.lib()
    return torch, kvbt, torch.device("cuda:0")


def _bf16(torch, a, d):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)


def gpu_scores(env, x, reduce, out_bf16=False, block_table=None):
    torch, kvbt, d = env
    bt = x.block_table if block_table is None else block_table
    if x.k_scale is not None:
        kc = torch.from_numpy(x.k_cache).to(d)
        ks = torch.from_numpy(x.k_scale).to(d)
    else:
        kc, ks = _bf16(torch, x.k_cache, d), None
    T, H, M = x.T, x.H, x.max_k_tiles
    if out_bf16:
        s = torch.full((T, H, M), BF16_NAN, dtype=torch.int16, device=d).view(torch.bfloat16)
    else:
        s = torch.full((T, H, M), float("nan"), dtype=torch.float32, device=d)
    kvbt.index_decode_scores(_bf16(torch, x.q_idx, d), kc,
                             torch.from_numpy(np.ascontiguousarray(bt)).to(d),
                             torch.from_numpy(x.seq_lens).to(d), s, x.scale,
                             decode_query_len=x.decode_query_len, reduce=reduce, k_scale=ks)
    torch.cuda.synchronize()
    return s.float().cpu().numpy().astype(np.float64)


def expected(index_oracle, x, reduce, block_table=None):
    bt = x.block_table if block_table is None else block_table
    init = np.full((x.T, x.H, x.max_k_tiles), np.nan)
    return index_oracle.index_decode_scores(x.q_idx, x.k_cache, bt, x.seq_lens,
                                            x.decode_query_len, x.scale, reduce, init,
                                            with_bound=True, k_scale=x.k_scale)


def assert_close(got, want, bound, out_bf16=False, label=""):
    wrote_g, wrote_w = ~np.isnan(got), ~np.isnan(want)
    if not np.array_equal(wrote_g, wrote_w):
        t, h, b = np.argwhere(wrote_g != wrote_w)[0]
        raise AssertionError("%s: written entries differ first at row %d head %d block %d "
                             "(gpu wrote %s)" % (label, t, h, b, wrote_g[t, h, b]))
    g, w, bd = got[wrote_w], want[wrote_w], bound[wrote_w]
    tol = 2.0 ** -16 * bd + 2.0 ** -14 + 2.0 ** -20 * np.abs(w)
    if out_bf16:
        tol = tol + 2.0 ** -8 * np.abs(w)
    bad = np.abs(g - w) > tol
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError("%s: %d of %d scores out of bound; e.g. gpu %r oracle %r tol %r"
                             % (label, int(bad.sum()), bad.size, g[i], w[i], tol[i]))


SEQS = [0, 1, 2, 3, 4, 5, 16, 127, 128, 129, 130, 131, 255, 256, 257, 258, 1000, 2047, 2048,
        2049]


@pytest.mark.parametrize("reduce", ["lse", "max"])
@pytest.mark.parametrize("q,H", [(1, 1), (2, 3), (4, 2), (16, 1)])
def test_seq_lengths_and_query_lengths(env, index_oracle, reduce, q, H):
    x = wl.index_inputs("idx_q%d_h%d" % (q, H), SEQS, q, H, max_k_tiles=17, seed=10 + q + H,
                        spare_blocks=5)
    want, bound = expected(index_oracle, x, reduce)
    got = gpu_scores(env, x, reduce)
    assert_close(got, want, bound, label="%s q %d H %d" % (reduce, q, H))


@pytest.mark.parametrize("reduce", ["lse", "max"])
def test_bf16_output(env, index_oracle, reduce):
    x = wl.index_inputs("idx_bf16", SEQS, 4, 2, max_k_tiles=17, seed=31)
    want, bound = expected(index_oracle, x, reduce)
    assert_close(gpu_scores(env, x, reduce, out_bf16=True), want, bound, True, reduce)


@pytest.mark.parametrize("M,max_blocks", [(3, 17), (17, 3), (17, 17), (40, 40)])
def test_capacity_limits(env, index_oracle, M, max_blocks):
    x = wl.index_inputs("idx_cap", SEQS, 2, 2, max_k_tiles=M, seed=40 + M,
                        max_blocks=max_blocks)
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce)
        assert_close(gpu_scores(env, x, reduce), want, bound,
                     label="%s M %d max_blocks %d" % (reduce, M, max_blocks))


def test_invalid_block_ids_read_as_zero_keys(env, index_oracle):
    x = wl.index_inputs("idx_bad", [1000, 300, 2049, 129], 4, 2, max_k_tiles=17, seed=50)
    bt = x.block_table.copy()
    bt[0, 1] = -1
    bt[1, 0] = x.num_blocks
    bt[2, 5] = x.num_blocks + 1000
    bt[3, 1] = -(1 << 30)
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce, block_table=bt)
        assert_close(gpu_scores(env, x, reduce, block_table=bt), want, bound, label=reduce)


@pytest.mark.parametrize("fp8", [False, True])
def test_empty_key_cache(env, index_oracle, fp8):
    # num_pages 0 (null cache pointers): every block reads as zero keys, so each written
    # score is the reduction of zero products (ln of the token count for LSE, 0 for max)
    import dataclasses
    x = wl.index_inputs("idx_empty", [1000, 300, 2049, 129], 4, 2, max_k_tiles=17, seed=51,
                        fp8=fp8)
    y = dataclasses.replace(x, k_cache=x.k_cache[:0],
                            k_scale=None if x.k_scale is None else x.k_scale[:0])
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, y, reduce)
        got = gpu_scores(env, y, reduce)
        assert_close(got, want, bound, label="%s fp8 %s" % (reduce, fp8))
        if reduce == "max":
            assert not got[~np.isnan(got)].any()


@pytest.mark.parametrize("n", [1, 2])
def test_decode_workload_shapes(env, index_oracle, n):
    # the tiny decode batch and the 74-block spec-decode batch, their seq_lens and shapes
    w = wl.config(n)
    x = wl.index_inputs("idx_" + w.name, w.seq_lens, w.decode_query_len, w.H, w.M,
                        seed=60 + n, max_blocks=w.max_blocks)
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce)
        assert_close(gpu_scores(env, x, reduce), want, bound, label="%s %s" % (w.name, reduce))
        assert_close(gpu_scores(env, x, reduce, out_bf16=True), want, bound, True,
                     label="%s %s bf16" % (w.name, reduce))


def test_boundary_and_long_context_requests(env, index_oracle):
    # the first 16 requests of the 129-block boundary batch (126..129 blocks, 1/128/129
    # tokens) and 3 requests of the 512-block long-context batch
    w3, w4 = wl.config(3), wl.config(4)
    for w, k in ((w3, 16), (w4, 3)):
        x = wl.index_inputs("idx_" + w.name, w.seq_lens[:k], 1, w.H, w.M, seed=70 + k,
                            max_blocks=w.max_blocks)
        for reduce in ("lse", "max"):
            want, bound = expected(index_oracle, x, reduce)
            assert_close(gpu_scores(env, x, reduce), want, bound, label="%s %s" % (w.name, reduce))


def test_repeat_and_graph_replay_are_identical(env):
    torch, kvbt, d = env
    x = wl.index_inputs("idx_graph", SEQS * 3, 4, 2, max_k_tiles=17, seed=80)
    args = (_bf16(torch, x.q_idx, d), _bf16(torch, x.k_cache, d),
            torch.from_numpy(x.block_table).to(d), torch.from_numpy(x.seq_lens).to(d))
    s = torch.full((x.T, x.H, x.max_k_tiles), float("-inf"), device=d)
    kvbt.index_decode_scores(*args, s, x.scale, decode_query_len=4)
    torch.cuda.synchronize()
    first = s.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        s.fill_(float("-inf"))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            kvbt.index_decode_scores(*args, s, x.scale, decode_query_len=4)
    for r in range(3):
        s.fill_(float("-inf"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(s, first), "replay %d differs from the eager call" % r


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) index keys; the bound is the same (the codes convert exactly to bf16,
# the per-token scale multiplies each exact-product sum: one more fp32 rounding, 2^-24)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("reduce", ["lse", "max"])
@pytest.mark.parametrize("q,H", [(1, 1), (4, 2), (16, 1)])
def test_fp8_keys(env, index_oracle, reduce, q, H):
    x = wl.index_inputs("idx8_q%d_h%d" % (q, H), SEQS, q, H, max_k_tiles=17,
                        seed=110 + q + H, spare_blocks=3, fp8=True)
    want, bound = expected(index_oracle, x, reduce)
    assert_close(gpu_scores(env, x, reduce), want, bound, label="fp8 %s q %d H %d" % (reduce, q, H))
    assert_close(gpu_scores(env, x, reduce, out_bf16=True), want, bound, True,
                 label="fp8 %s bf16" % reduce)


def test_fp8_every_code_and_invalid_blocks(env, index_oracle):
    # keys cycling through all finite E4M3 codes (NaN codes left out), random scales
    x = wl.index_inputs("idx8_codes", [1000, 129, 2049, 16], 4, 2, max_k_tiles=17, seed=120,
                        fp8=True)
    codes = np.arange(x.k_cache.size, dtype=np.int64) % 254
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)   # skip 0x7F
    x.k_cache[...] = codes.reshape(x.k_cache.shape)
    x.k_scale[...] = np.random.Generator(np.random.PCG64(121)).uniform(
        1e-3, 2.0, size=x.k_scale.shape).astype(np.float32)
    bt = x.block_table.copy()
    bt[0, 2] = -1
    bt[2, 7] = x.num_blocks + 5
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce, block_table=bt)
        assert_close(gpu_scores(env, x, reduce, block_table=bt), want, bound, label=reduce)


def test_fp8_spec_decode_shape(env, index_oracle):
    w = wl.config(2)
    x = wl.index_inputs("idx8_" + w.name, w.seq_lens, w.decode_query_len, w.H, w.M, seed=130,
                        max_blocks=w.max_blocks, fp8=True)
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce)
        assert_close(gpu_scores(env, x, reduce), want, bound, label="fp8 %s %s" % (w.name, reduce))


def test_long_requests_wide_grid(env, index_oracle):
    # thousands of blocks per request and a wide score buffer: most of the grid's
    # wavefronts (blocks past a request's length) end at once
    x = wl.index_inputs("idx_long", [300000, 1, 131072, 5000], 2, 1, max_k_tiles=8192, seed=140)
    for reduce in ("lse", "max"):
        want, bound = expected(index_oracle, x, reduce)
        assert_close(gpu_scores(env, x, reduce), want, bound, label="long %s" % reduce)


# ---------------------------------------------------------------------------
# randomized cases: every parameter drawn from a seed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", random_seeds(8000, 32))
def test_randomized_cases(env, index_oracle, seed):
    """Requests, query length, heads, score-buffer width, block-table width, sequence
    lengths (empty, short, past the capacity), key dtype, reduction, output dtype and
    invalid block ids, all drawn from the seed."""
    rng = np.random.default_rng(seed)
    B, q, H = int(rng.integers(1, 25)), int(rng.integers(1, 17)), int(rng.integers(1, 5))
    M = int(rng.choice([1, 2, 7, 16, 17, 74, 129, 300, 600]))
    q = max(1, min(q, 8000 // (H * M)))            # the oracle scores block by block
    B = max(1, min(B, 16000 // (q * H * M)))
    mb = None if rng.random() < 0.6 else int(rng.integers(1, M + 20))
    cap = 128 * (M if mb is None else min(M, mb))
    seqs = np.where(rng.random(B) < 0.15, rng.integers(0, 4, B),
                    rng.integers(1, cap + 700, B)).tolist()
    fp8 = bool(rng.integers(0, 2))
    reduce = str(rng.choice(["lse", "max"]))
    out_bf16 = bool(rng.integers(0, 2))
    x = wl.index_inputs("idx_rand_%d" % seed, seqs, q, H, max_k_tiles=M, seed=seed,
                        max_blocks=mb, spare_blocks=int(rng.integers(0, 4)), fp8=fp8)
    bt = x.block_table.copy()
    bad = rng.random(bt.shape) < 0.03
    bt[bad] = np.where(rng.random(bt.shape) < 0.5, -1, x.num_blocks + 7)[bad]
    print("seed", seed, "B", B, "q", q, "H", H, "M", M, "mb", mb, "fp8", fp8, reduce,
          "bf16 out", out_bf16, flush=True)
    want, bound = expected(index_oracle, x, reduce, block_table=bt)
    got = gpu_scores(env, x, reduce, out_bf16=out_bf16, block_table=bt)
    assert_close(got, want, bound, out_bf16, "seed %d" % seed)
