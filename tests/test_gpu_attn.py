"""GPU parity of the sparse paged-attention decode against the CPU oracle.

The HIP kernel (through the C ABI) and oracle/sparse_attn.py take the same seeded
inputs. Outputs are floating point, so each element must lie within a bound derived
from the kernel's arithmetic (the oracle is float64 on the same bf16 inputs):

  |gpu - oracle| <= 2^-7 * spread + 2^-12 * vmax   (+ 2^-8 * |oracle| for bf16 output)

spread = sum_i w_i |V_i[d] - out[d]| is how far relative changes of the softmax
weights can move the output; rounding each probability to bf16 (relative 2^-9), the
fp32 score sum over 128 exact products and the hardware exp2 change every weight by
a relative amount well under 2^-8, which moves the output by at most about twice that
times the spread. vmax = max |V| over the row's tokens bounds the fp32 accumulation
over up to 2048 tokens (at most ~2^-12 relative in the worst case). A bf16 output adds
its own rounding. Outputs are pre-filled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl
from kvbt_checks import random_seeds

pytestmark = pytest.mark.gpu

WAVES = (1, 2, 4, 8)


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


def to_device(env, a):
    torch, _, d = env
    return dict(q=_bf16(torch, a.q, d), k_cache=_bf16(torch, a.k_cache, d),
                v_cache=_bf16(torch, a.v_cache, d),
                table=torch.from_numpy(np.ascontiguousarray(a.table)).to(d),
                ctx=torch.from_numpy(np.ascontiguousarray(a.ctx)).to(d))


def gpu_attn(env, a, waves=0, out_bf16=False, dev=None, scale=None, ql=None):
    torch, kvbt, d = env
    dev = dev or to_device(env, a)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full(a.q.shape, float("nan"), dtype=dt, device=d)
    kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"],
                            dev["ctx"], a.scale if scale is None else scale, out=out,
                            waves=waves,
                            decode_query_len=a.decode_query_len if ql is None else ql)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def expected(attn_oracle, a, scale=None):
    return attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, a.ctx,
                                          a.scale if scale is None else scale, with_spread=True)


def assert_close(got, want, spread, vmax, G, out_bf16=False, label=""):
    vrow = np.repeat(vmax, G, axis=1)[:, :, None]            # [T, H*G, 1]
    tol = 2.0 ** -7 * spread + 2.0 ** -12 * vrow
    if out_bf16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    assert np.isfinite(got).all(), "%s: non-finite output (unwritten element?)" % label
    err = np.abs(got - want)
    bad = err > tol
    if bad.any():
        t, j, dd = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of bound; first at row %d head %d dim %d: "
                             "gpu %r oracle %r tol %r" % (label, int(bad.sum()), t, j, dd,
                                                          got[t, j, dd], want[t, j, dd],
                                                          tol[t, j, dd]))


@pytest.mark.parametrize("ctx", [1, 2, 15, 16, 17, 31, 33, 100, 1000, 2047, 2048])
@pytest.mark.parametrize("waves", WAVES)
def test_fixed_context_lengths(env, attn_oracle, ctx, waves):
    a = wl.attention_case(100 + ctx, T=3, H=2, G=8, W=128, P=300, ctx=ctx)
    want, spread, vmax = expected(attn_oracle, a)
    got = gpu_attn(env, a, waves=waves)
    assert_close(got, want, spread, vmax, a.G, label="ctx %d waves %d" % (ctx, waves))


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8, 12, 16])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_group_sizes_and_output_dtypes(env, attn_oracle, G, out_bf16):
    a = wl.attention_case(200 + G, T=5, H=3, G=G, W=64, P=200)
    want, spread, vmax = expected(attn_oracle, a)
    for waves in (0, 1, 4):
        got = gpu_attn(env, a, waves=waves, out_bf16=out_bf16)
        assert_close(got, want, spread, vmax, a.G, out_bf16, "G %d waves %d" % (G, waves))


@pytest.mark.parametrize("W", [1, 3, 8, 64, 127, 128])
def test_table_widths_and_ragged_rows(env, attn_oracle, W):
    a = wl.attention_case(300 + W, T=17, H=2, G=8, W=W, P=500)
    a.ctx[0, 0] = 0
    a.ctx[1, 1] = -7
    a.ctx[2, 0] = 16 * W + 5          # clamped to the table width
    a.ctx[3, 1] = 1 << 30
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        got = gpu_attn(env, a, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="W %d waves %d" % (W, waves))
    assert not got[0, :8].any() and not got[1, 8:].any()       # empty rows give zeros


def test_pages_outside_the_cache_read_as_zero(env, attn_oracle):
    a = wl.attention_case(401, T=8, H=2, G=4, W=128, P=64, bad_page_frac=0.25)
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        assert_close(gpu_attn(env, a, waves=waves), want, spread, vmax, a.G,
                     label="waves %d" % waves)
    a.table[:] = -1                                   # every page invalid: zero K and V
    assert not gpu_attn(env, a).any()


def test_empty_cache_gives_zeros(env, attn_oracle):
    # num_pages 0 (null cache pointers): every page reads as zeros, on the per-row kernel,
    # the request-grouped kernel and the split across workgroups
    import dataclasses
    torch, kvbt, d = env
    a = shared_page_case(3200, T=512, H=2, G=8, q=4, W=16, P=400)
    b = dataclasses.replace(a, k_cache=a.k_cache[:0], v_cache=a.v_cache[:0])
    assert b.P == 0 and kvbt.sparse_attn_grouped(b.T, b.H, b.G, 4)
    want, spread, vmax = expected(attn_oracle, b)
    assert not want.any()
    dev = to_device(env, b)
    for ql in (1, 4):
        for waves in (0, 1, 8):
            got = gpu_attn(env, b, waves=waves, dev=dev, ql=ql)
            assert not got.any(), "q %d waves %d" % (ql, waves)
    ws = torch.zeros(kvbt.sparse_attn_workspace_bytes(b.T, b.H, 4), dtype=torch.uint8, device=d)
    out = torch.full(b.q.shape, float("nan"), dtype=torch.float32, device=d)
    kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"], dev["ctx"],
                            b.scale, out=out, decode_query_len=4, workspace=ws, splits=4)
    torch.cuda.synchronize()
    assert not out.any()


@pytest.mark.parametrize("scale", [0.0, 1e-3, 1.0, 4.0])
def test_flat_and_peaked_softmax(env, attn_oracle, scale):
    # scale 0: plain mean of the listed values; 4: nearly one-hot weights
    a = wl.attention_case(500, T=6, H=2, G=8, W=32, P=100, ctx_hi=16 * 32)
    want, spread, vmax = expected(attn_oracle, a, scale=scale)
    for waves in (1, 4):
        got = gpu_attn(env, a, waves=waves, scale=scale)
        assert_close(got, want, spread, vmax, a.G, label="scale %g waves %d" % (scale, waves))


def test_empty_batch(env):
    torch, kvbt, d = env
    a = wl.attention_case(600, T=1, H=2, G=8, W=8, P=4)
    dev = to_device(env, a)
    out = kvbt.sparse_attn_decode(dev["q"][:0], dev["k_cache"], dev["v_cache"],
                                  dev["table"][:0], dev["ctx"][:0], a.scale)
    assert tuple(out.shape) == (0, 16, 128)


# rows of each decode workload whose selections feed the attention (the cache holds
# every page a kept row names, for all KV heads: about 620 MB for all 256 spec-decode
# rows; the boundary and long-context workloads keep their first rows, which include
# the 126..129-block and 1/128/129-token boundary rows)
SELECTOR_ROWS = {1: 4, 2: 256, 3: 24, 4: 16}


@pytest.fixture(scope="module")
def selector_tables(orc):
    """(name, table, ctx) from the oracle's select + table on the decode workloads."""
    out = []
    for n, rows in SELECTOR_ROWS.items():
        w = wl.config(n)
        _, table, ctx = orc.select_topk_and_build_table(
            w.scores, w.block_table, topk=w.topk, num_init=w.num_init, num_local=w.num_local,
            **w.row_kwargs())
        out.append((w.name, table[:rows], ctx[:rows], w.decode_query_len))
    return out


@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_over_selector_tables(env, attn_oracle, selector_tables, i):
    name, table, ctx, q = selector_tables[i]
    a = wl.attention_inputs("attn_" + name, table, ctx, G=8, seed=700 + i, decode_query_len=q)
    want, spread, vmax = expected(attn_oracle, a)
    for waves in (0, 1, 2, 4, 8):
        got = gpu_attn(env, a, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="%s waves %d" % (name, waves))
        # the other kernel (rows one by one, or a request's rows side by side): the same
        # bound, another rounding order
        other = gpu_attn(env, a, waves=waves, ql=1 if q > 1 else 4)
        assert_close(other, want, spread, vmax, a.G, label="%s waves %d other q" % (name, waves))
    got = gpu_attn(env, a, out_bf16=True)
    assert_close(got, want, spread, vmax, a.G, True, label="%s bf16" % name)


@pytest.mark.parametrize("ql", [1, 4])
def test_repeat_and_graph_replay_are_identical(env, attn_oracle, ql):
    torch, kvbt, d = env
    a = shared_page_case(800, T=512, H=2, G=8, q=ql, W=64, P=4000) if ql > 1 else \
        wl.attention_case(800, T=64, H=2, G=8, W=128, P=2000)
    dev = to_device(env, a)
    out = torch.empty(a.q.shape, dtype=torch.float32, device=d)
    kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"], dev["ctx"],
                            a.scale, out=out, decode_query_len=ql)
    torch.cuda.synchronize()
    first = out.clone()
    want, spread, vmax = expected(attn_oracle, a)
    assert_close(first.cpu().numpy().astype(np.float64), want, spread, vmax, a.G, label="eager")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"],
                                    dev["ctx"], a.scale, out=out, decode_query_len=ql)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "replay %d differs from the eager call" % r


# ---------------------------------------------------------------------------
# several rows per request: the request-grouped kernel
# ---------------------------------------------------------------------------

def shared_page_case(seed, *, T, H, G, q, W=128, P=3000, dup_frac=0.0, bad_frac=0.0):
    """Consecutive groups of q rows (one request each; the last may be cut short by T)
    whose page lists share most pages, at shifted positions, next to pages of their own;
    contexts differ by a few tokens between the rows (partial last pages differ).
    dup_frac of the rows list one of their pages twice, bad_frac of the entries are ids
    outside the cache."""
    import dataclasses
    rng = np.random.default_rng(seed)
    a = wl.attention_case(seed, T=T, H=H, G=G, W=W, P=P)
    table = np.empty((T, H, W), dtype=np.int32)
    ctx = np.empty((T, H), dtype=np.int32)
    for r0 in range(0, T, q):
        for h in range(H):
            base = rng.choice(P // 2, size=W, replace=False)          # shared pages
            c0 = int(rng.integers(0, 16 * W - 8))
            for t in range(r0, min(r0 + q, T)):
                own = P // 2 + rng.choice(P - P // 2, size=W, replace=False)   # its own
                lst = np.where(rng.random(W) < 0.7, base, own)
                shift = int(rng.integers(0, 3))
                lst = np.roll(lst, shift)
                if rng.random() < dup_frac:
                    lst[int(rng.integers(0, W))] = lst[0]
                bad = rng.random(W) < bad_frac
                lst[bad] = np.where(rng.random(W) < 0.5, -1, P + 5)[bad]
                table[t, h] = lst
                ctx[t, h] = min(16 * W, c0 + (t - r0) + int(rng.integers(0, 3)))
    return dataclasses.replace(a, table=table, ctx=ctx, decode_query_len=q)


# (G, q, T) with H = 2: at least 256 (request, KV head) workgroups, so the rows of each
# request are attended together (one or two column tiles, requests cut short by T, more
# rows per request than a workgroup holds)
GROUPED = [(8, 4, 512), (8, 2, 256), (8, 3, 383), (8, 8, 1024), (1, 4, 512), (3, 4, 510),
           (5, 3, 383), (9, 2, 256), (16, 4, 1024), (16, 2, 256), (4, 5, 640), (2, 16, 512)]
# smaller batches with several rows per request: every row alone, pages cacheable
ROWS_ALONE = [(8, 4, 64), (8, 3, 31), (16, 2, 9)]


@pytest.mark.parametrize("G,q,T", GROUPED + ROWS_ALONE)
def test_request_rows(env, attn_oracle, G, q, T):
    torch, kvbt, d = env
    a = shared_page_case(1000 + 31 * G + q, T=T, H=2, G=G, q=q, W=24 if T > 64 else 16 + 7 * q)
    assert kvbt.sparse_attn_grouped(T, 2, G, q) == ((G, q, T) in GROUPED)
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        got = gpu_attn(env, a, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="G %d q %d waves %d" % (G, q, waves))
    got = gpu_attn(env, a, out_bf16=True)
    assert_close(got, want, spread, vmax, a.G, True, label="G %d q %d bf16" % (G, q))


@pytest.mark.parametrize("dup,bad", [(0.3, 0.0), (0.0, 0.1), (1.0, 0.2)])
def test_request_rows_with_repeated_and_invalid_pages(env, attn_oracle, dup, bad):
    # a row listing one page twice counts it twice; invalid ids read as zero keys/values
    torch, kvbt, d = env
    a = shared_page_case(1100 + int(10 * dup + 100 * bad), T=512, H=2, G=8, q=4, W=32,
                         dup_frac=dup, bad_frac=bad)
    assert kvbt.sparse_attn_grouped(a.T, 2, 8, 4)
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        assert_close(gpu_attn(env, a, waves=waves), want, spread, vmax, a.G,
                     label="dup %g bad %g waves %d" % (dup, bad, waves))


def test_request_rows_empty_and_full_contexts(env, attn_oracle):
    torch, kvbt, d = env
    a = shared_page_case(1200, T=512, H=2, G=8, q=4, W=128)
    assert kvbt.sparse_attn_grouped(a.T, 2, 8, 4)
    a.ctx[0, :] = 0
    a.ctx[1, 0] = -3
    a.ctx[5, 1] = 1 << 30              # clamped to the width
    a.ctx[8:12, :] = 0                 # a whole request without tokens
    a.ctx[100:104, :] = 16 * 128       # a whole request at the full width
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        got = gpu_attn(env, a, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="waves %d" % waves)
    assert not got[0].any() and not got[8:12].any()


@pytest.mark.parametrize("seed", random_seeds(7100, 16))
def test_randomized_grouped_cases(env, attn_oracle, seed):
    """Several rows per request at batch sizes on both sides of the grouping threshold,
    with group size, rows per request, table width, repeats and invalid ids per seed."""
    torch, kvbt, d = env
    rng = np.random.default_rng(seed)
    q = int(rng.choice([2, 3, 4, 5, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 9, 16]))
    H = int(rng.integers(1, 4))
    T = int(rng.integers(8, 700))
    a = shared_page_case(seed, T=T, H=H, G=G, q=q, W=int(rng.integers(8, 40)),
                         dup_frac=float(rng.choice([0.0, 0.0, 0.2])),
                         bad_frac=float(rng.choice([0.0, 0.05])))
    waves = int(rng.choice([0, 1, 2, 4, 8]))
    print("seed", seed, "T", T, "H", H, "G", G, "q", q, "waves", waves, "grouped",
          kvbt.sparse_attn_grouped(T, H, G, q), flush=True)
    want, spread, vmax = expected(attn_oracle, a)
    assert_close(gpu_attn(env, a, waves=waves), want, spread, vmax, a.G, label="seed %d" % seed)


def test_many_pairs_take_the_library_wave_choice(env, attn_oracle):
    # 1040 (row, index head) pairs: eight wavefronts per workgroup for single rows; with
    # q 2 the 260 requests x 2 heads take the request-grouped kernel, four wavefronts each
    torch, kvbt, d = env
    a = wl.attention_case(900, T=520, H=2, G=4, W=16, P=400, ctx_hi=16 * 16)
    assert kvbt.sparse_attn_waves(a.T, a.H, 1) == 8
    assert kvbt.sparse_attn_waves(a.T, a.H, 2) == 4
    assert kvbt.sparse_attn_grouped(a.T, a.H, a.G, 2)
    want, spread, vmax = expected(attn_oracle, a)
    assert_close(gpu_attn(env, a), want, spread, vmax, a.G, label="auto waves, 1040 pairs, q 1")
    assert_close(gpu_attn(env, a, ql=2), want, spread, vmax, a.G, label="auto waves, q 2")


# ---------------------------------------------------------------------------
# randomized cases: every parameter drawn from a seed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", random_seeds(7000, 32))
def test_randomized_cases(env, attn_oracle, seed):
    """Rows, heads, group size, table width, cache size, context lengths (with empty,
    negative and over-wide ones), invalid page ids, scale, wavefront count, output dtype
    and rows per request, all drawn from the seed."""
    rng = np.random.default_rng(seed)
    T, H = int(rng.integers(1, 41)), int(rng.integers(1, 5))
    G, W = int(rng.integers(1, 17)), int(rng.integers(1, 129))
    P = int(rng.integers(1, 601))
    a = wl.attention_case(seed, T=T, H=H, G=G, W=W, P=P,
                          bad_page_frac=float(rng.choice([0.0, 0.0, 0.1])))
    odd = rng.random((T, H))
    a.ctx[odd < 0.05] = 0
    a.ctx[(odd >= 0.05) & (odd < 0.08)] = -int(rng.integers(1, 100))
    a.ctx[(odd >= 0.08) & (odd < 0.11)] = 16 * W + int(rng.integers(1, 1000))
    scale = a.scale * float(rng.uniform(0.25, 2.0))
    waves = int(rng.choice([0, 1, 2, 4, 8]))
    out_bf16 = bool(rng.integers(0, 2))
    ql = int(rng.choice([1, 2, 4]))
    print("seed", seed, "T", T, "H", H, "G", G, "W", W, "P", P, "waves", waves, "bf16", out_bf16,
          "q", ql, flush=True)
    want, spread, vmax = expected(attn_oracle, a, scale=scale)
    got = gpu_attn(env, a, waves=waves, out_bf16=out_bf16, scale=scale, ql=ql)
    assert_close(got, want, spread, vmax, a.G, out_bf16, "seed %d" % seed)
