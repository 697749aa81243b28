"""GPU parity of the sparse-attention decode with each (row, index head) split across
workgroups (the call with a workspace, kvbt_sparse_attn_decode_ws) against the CPU
oracle, within the bound derived in test_gpu_attn.py; and the workspace's contract:
the first 16 bytes of every 256-byte line (the arrival counters) are zero again after
every call, one workspace serves batch shapes one after another without clearing, and
the results do not depend on which workgroup of a pair finishes last (repeated calls
and graph replays are identical).
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl
from kvbt_checks import random_seeds
from test_gpu_attn import WAVES, assert_close, env, expected, shared_page_case, to_device  # noqa: F401

pytestmark = pytest.mark.gpu


def workspace(env, nbytes):
    torch, _, d = env
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=d)


def counters_are_zero(ws):
    n = ws.numel() // 256 * 256
    return not ws[:n].view(-1, 256)[:, :16].any().item()


def gpu_attn_ws(env, a, ws, splits=0, waves=0, out_bf16=False, dev=None):
    torch, kvbt, d = env
    dev = dev or to_device(env, a)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full(a.q.shape, float("nan"), dtype=dt, device=d)
    kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"],
                            dev["ctx"], a.scale, out=out, waves=waves,
                            decode_query_len=a.decode_query_len, workspace=ws, splits=splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def split_of(env, a, splits=0, nbytes=1 << 62):
    _, kvbt, _ = env
    return kvbt.sparse_attn_splits(a.T, a.H, splits, nbytes)


# (G, q, T) with H = 2: fewer than 160 (row, index head) pairs, so the library splits
# each over 2 or 4 workgroups (speculative rows, requests cut short by T, single rows)
SPLIT_AUTO = [(8, 4, 60), (8, 4, 16), (8, 2, 40), (8, 3, 31), (16, 2, 9), (1, 4, 20),
              (3, 4, 30), (5, 3, 19), (9, 2, 14), (4, 5, 50), (2, 16, 32), (16, 4, 12),
              (8, 1, 8), (8, 1, 79), (12, 1, 1), (8, 4, 77)]


@pytest.mark.parametrize("G,q,T", SPLIT_AUTO)
def test_split_rows(env, attn_oracle, G, q, T):
    torch, kvbt, d = env
    a = shared_page_case(2000 + 31 * G + q + T, T=T, H=2, G=G, q=q, W=16 + 7 * q)
    S = split_of(env, a)
    assert 2 <= S <= 4
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(T, 2))
    want, spread, vmax = expected(attn_oracle, a)
    dev = to_device(env, a)
    for waves in WAVES:
        got = gpu_attn_ws(env, a, ws, waves=waves, dev=dev)
        assert_close(got, want, spread, vmax, a.G, label="G %d q %d S %d waves %d" % (G, q, S, waves))
        assert counters_are_zero(ws)
    got = gpu_attn_ws(env, a, ws, out_bf16=True, dev=dev)
    assert_close(got, want, spread, vmax, a.G, True, label="G %d q %d bf16" % (G, q))
    # every explicit split count on the same workspace (sized for the largest)
    big = workspace(env, kvbt.sparse_attn_workspace_bytes(T, 2, 8))
    for s in (2, 3, 5, 8):
        got = gpu_attn_ws(env, a, big, splits=s, dev=dev)
        assert_close(got, want, spread, vmax, a.G, label="G %d q %d splits %d" % (G, q, s))
        assert counters_are_zero(big)


@pytest.mark.parametrize("T,q,splits", [(512, 4, 2), (1024, 8, 3), (256, 4, 8), (80, 1, 4),
                                        (200, 1, 2)])
def test_explicit_splits_beyond_the_auto_choice(env, attn_oracle, T, q, splits):
    # batches the library would not split: the grouped kernel's size, 160 or more pairs
    torch, kvbt, d = env
    if q > 1:
        a = shared_page_case(2100 + T + q, T=T, H=2, G=8, q=q, W=24)
    else:
        a = wl.attention_case(2100 + T, T=T, H=2, G=8, W=64, P=3000)
    assert split_of(env, a) == 0
    assert split_of(env, a, splits) == splits
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(T, 2, splits))
    want, spread, vmax = expected(attn_oracle, a)
    for waves in (1, 4, 8):
        got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="T %d q %d waves %d" % (T, q, waves))
    assert counters_are_zero(ws)


@pytest.mark.parametrize("dup,bad", [(0.3, 0.0), (0.0, 0.1), (1.0, 0.2)])
def test_split_with_repeated_and_invalid_pages(env, attn_oracle, dup, bad):
    torch, kvbt, d = env
    a = shared_page_case(2200 + int(10 * dup + 100 * bad), T=40, H=2, G=8, q=4, W=32,
                         dup_frac=dup, bad_frac=bad)
    assert split_of(env, a) >= 2
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, 2, 8))
    want, spread, vmax = expected(attn_oracle, a)
    for splits in (0, 2, 8):
        for waves in (1, 4):
            got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves)
            assert_close(got, want, spread, vmax, a.G,
                         label="dup %g bad %g splits %d waves %d" % (dup, bad, splits, waves))


def test_split_empty_and_full_contexts(env, attn_oracle):
    torch, kvbt, d = env
    a = shared_page_case(2300, T=48, H=2, G=8, q=4, W=128)
    assert split_of(env, a) == 2
    a.ctx[0, :] = 0                    # rows without tokens: every split empty
    a.ctx[1, 0] = -3
    a.ctx[5, 1] = 1 << 30              # clamped to the width
    a.ctx[8:12, :] = 0
    a.ctx[40:44, :] = 16 * 128         # a whole request at the full width
    a.ctx[20, 0] = 1                   # one token: one split holds it, the others none
    a.ctx[21, 1] = 17                  # two pages over the splits
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, 2, 8))
    want, spread, vmax = expected(attn_oracle, a)
    for splits in (0, 8):
        for waves in WAVES:
            got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves)
            assert_close(got, want, spread, vmax, a.G, label="splits %d waves %d" % (splits, waves))
        assert not got[0].any() and not got[8:12].any()


def test_split_at_full_width_and_largest_group(env, attn_oracle):
    # 16 query heads per index head, 128-page rows full to the last token, every split
    # count and wavefront count, both output types
    torch, kvbt, d = env
    a = wl.attention_case(2450, T=6, H=3, G=16, W=128, P=3000, ctx=16 * 128)
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, a.H, 8))
    want, spread, vmax = expected(attn_oracle, a)
    dev = to_device(env, a)
    for splits in range(2, kvbt.ATTN_MAX_SPLITS + 1):
        for waves in (1, 8):
            for out_bf16 in (False, True):
                got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves, out_bf16=out_bf16,
                                  dev=dev)
                assert_close(got, want, spread, vmax, a.G, out_bf16,
                             label="splits %d waves %d bf16 %s" % (splits, waves, out_bf16))
    assert counters_are_zero(ws)


def test_more_splits_than_pages(env, attn_oracle):
    # one or two pages per row: most of the 8 workgroups of a pair have nothing to
    # stream and publish empty partial results
    torch, kvbt, d = env
    a = shared_page_case(2400, T=40, H=2, G=8, q=4, W=2, P=64)
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, 2, 8))
    want, spread, vmax = expected(attn_oracle, a)
    for waves in WAVES:
        got = gpu_attn_ws(env, a, ws, splits=8, waves=waves)
        assert_close(got, want, spread, vmax, a.G, label="waves %d" % waves)


def test_repeats_and_graph_replays_are_identical(env, attn_oracle):
    # the merge is in split order whichever workgroup arrives last: bit-identical outputs
    torch, kvbt, d = env
    a = shared_page_case(2500, T=24, H=2, G=8, q=4, W=64, P=4000)
    assert split_of(env, a) == 4
    dev = to_device(env, a)
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, 2))
    out = torch.empty(a.q.shape, dtype=torch.float32, device=d)

    def call():
        kvbt.sparse_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["table"],
                                dev["ctx"], a.scale, out=out, decode_query_len=4, workspace=ws)

    call()
    torch.cuda.synchronize()
    first = out.clone()
    want, spread, vmax = expected(attn_oracle, a)
    assert_close(first.cpu().numpy().astype(np.float64), want, spread, vmax, a.G, label="eager")
    for r in range(5):
        out.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "repeat %d differs" % r
    assert counters_are_zero(ws)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), "replay %d differs from the eager call" % r
        assert counters_are_zero(ws)


def test_one_workspace_serves_batch_shapes_in_turn(env, attn_oracle):
    # partial results left by one shape lie where another shape's counters are not:
    # no clearing between calls of different shapes
    torch, kvbt, d = env
    cases = [shared_page_case(2600, T=64, H=2, G=8, q=4, W=40),
             shared_page_case(2601, T=200, H=2, G=8, q=4, W=24),
             shared_page_case(2602, T=30, H=3, G=16, q=2, W=32),
             shared_page_case(2603, T=96, H=1, G=4, q=3, W=48)]
    need = max(kvbt.sparse_attn_workspace_bytes(c.T, c.H, 8) for c in cases)
    ws = workspace(env, need)
    for rep in range(2):
        for i, c in enumerate(cases):
            splits = (0, 8)[(i + rep) % 2]
            want, spread, vmax = expected(attn_oracle, c)
            got = gpu_attn_ws(env, c, ws, splits=splits)
            assert_close(got, want, spread, vmax, c.G, label="case %d rep %d" % (i, rep))
            assert counters_are_zero(ws)


def test_over_the_spec_decode_selector_table(env, attn_oracle, orc):
    # the 64-request spec-decode workload's own selection (2 heads, q 4): its first 16
    # and 48 rows (the library splits them) and all 256 rows (explicit splits)
    torch, kvbt, d = env
    w = wl.config(2)
    _, table, ctx = orc.select_topk_and_build_table(
        w.scores, w.block_table, topk=w.topk, num_init=w.num_init, num_local=w.num_local,
        **w.row_kwargs())
    for rows, auto in ((16, 4), (48, 2), (256, 0)):
        a = wl.attention_inputs("attn_%s_r%d" % (w.name, rows), table[:rows], ctx[:rows], G=8,
                                seed=2700 + rows, decode_query_len=w.decode_query_len)
        assert split_of(env, a) == auto
        ws = workspace(env, kvbt.sparse_attn_workspace_bytes(a.T, a.H, 8))
        want, spread, vmax = expected(attn_oracle, a)
        dev = to_device(env, a)
        for splits in ((0, 2, 3, 8) if auto else (2, 8)):
            for waves in (0, 4, 8):
                got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves, dev=dev)
                assert_close(got, want, spread, vmax, a.G,
                             label="rows %d splits %d waves %d" % (rows, splits, waves))
        got = gpu_attn_ws(env, a, ws, splits=2, out_bf16=True, dev=dev)
        assert_close(got, want, spread, vmax, a.G, True, label="rows %d bf16" % rows)
        del dev


@pytest.mark.parametrize("seed", random_seeds(7200, 16))
def test_randomized_split_cases(env, attn_oracle, seed):
    """Rows per request (1 included), group size, heads, batch size (on both sides of
    the split threshold), table width, repeats, invalid ids, split count and wavefronts
    drawn from the seed."""
    torch, kvbt, d = env
    rng = np.random.default_rng(seed)
    q = int(rng.choice([1, 2, 3, 4, 5, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 9, 16]))
    H = int(rng.integers(1, 4))
    T = int(rng.integers(1, 300))
    a = shared_page_case(seed, T=T, H=H, G=G, q=q, W=int(rng.integers(1, 40)),
                         dup_frac=float(rng.choice([0.0, 0.0, 0.2])),
                         bad_frac=float(rng.choice([0.0, 0.05])))
    splits = int(rng.choice([0, 2, 3, 4, 6, 8]))
    waves = int(rng.choice([0, 1, 2, 4, 8]))
    out_bf16 = bool(rng.random() < 0.3)
    S = split_of(env, a, splits)
    print("seed", seed, "T", T, "H", H, "G", G, "q", q, "splits", splits, "->", S,
          "waves", waves, "bf16 out", out_bf16, flush=True)
    ws = workspace(env, kvbt.sparse_attn_workspace_bytes(T, H, splits))
    want, spread, vmax = expected(attn_oracle, a)
    got = gpu_attn_ws(env, a, ws, splits=splits, waves=waves, out_bf16=out_bf16)
    assert_close(got, want, spread, vmax, a.G, out_bf16, label="seed %d" % seed)
    assert counters_are_zero(ws)
