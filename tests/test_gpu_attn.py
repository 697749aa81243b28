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
        # the rows-per-request hint changes the cache policy only: identical bits
        assert np.array_equal(gpu_attn(env, a, waves=waves, ql=1 if q > 1 else 4), got)
    got = gpu_attn(env, a, out_bf16=True)
    assert_close(got, want, spread, vmax, a.G, True, label="%s bf16" % name)


def test_repeat_and_graph_replay_are_identical(env, attn_oracle):
    torch, kvbt, d = env
    a = wl.attention_case(800, T=64, H=2, G=8, W=128, P=2000)
    dev = to_device(env, a)
    out = torch.empty(a.q.shape, dtype=torch.float32, device=d)
    kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"], dev["ctx"],
                            a.scale, out=out)
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
                                    dev["ctx"], a.scale, out=out)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "replay %d differs from the eager call" % r


def test_many_pairs_take_four_wavefronts(env, attn_oracle):
    # more than 1024 (row, index head) pairs: the library's choice is four wavefronts
    torch, kvbt, d = env
    a = wl.attention_case(900, T=520, H=2, G=4, W=16, P=400, ctx_hi=16 * 16)
    assert kvbt.sparse_attn_waves(a.T, a.H) == 4
    want, spread, vmax = expected(attn_oracle, a)
    assert_close(gpu_attn(env, a), want, spread, vmax, a.G, label="auto waves, 1040 pairs")


# ---------------------------------------------------------------------------
# randomized cases: every parameter drawn from a seed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(7000, 7032))
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
