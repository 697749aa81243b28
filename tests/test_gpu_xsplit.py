"""GPU parity of the cross-workgroup split (launch path 4), through the C ABI.

A row is cut into slices of 1024 fp32 / 2048 bf16 tiles, each taken by its own
workgroup, which writes its top-16 to the caller's workspace; the last slice of a
(row, head) to arrive merges the lists and writes the outputs, and sets its arrival
counter back to zero. Every result must equal the oracle's bit for bit (outputs are
poisoned before each call), and the workspace's counters must read zero after every
call and every graph replay (counters and lists alike), so that the next call, of any
batch shape, needs no clearing.
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl
from test_gpu_parity import POISON, _dev, _poisoned, assert_same, oracle_fused

pytestmark = pytest.mark.gpu

KINDS = ["normal", "specials", "ties", "increasing", "two_level", "neginf", "nan"]


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_block_top_amd as kvbt
    kvbt.lib()
    return torch, kvbt, torch.device("cuda:0")


def _counter_bytes(pairs):
    return pairs * 256        # one 32-bit counter at the start of each 256-byte line


def _workspace(env, w, hint, split):
    torch, kvbt, d = env
    dtype = kvbt.BF16 if w.is_bf16 else kvbt.F32
    n = kvbt.select_workspace_bytes(hint, w.M, dtype, w.T, w.H, w.topk, split)
    p = kvbt.launch_policy(hint, w.M, dtype, w.T, w.H, w.topk, split=split, workspace_bytes=n)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=d), p


def _kw(env, w):
    torch, kvbt, d = env
    if w.explicit:
        return dict(row_req=_dev(torch, w.row_req, d), row_pos=_dev(torch, w.row_pos, d))
    return dict(seq_lens=_dev(torch, w.seq_lens, d), decode_query_len=w.decode_query_len)


def xsplit_fused(env, w, hint=0, ws=None, split=None, scores_dev=None):
    """Fused call through kvbt_select_topk_and_build_table_ws; returns outputs and the
    workspace used."""
    torch, kvbt, d = env
    if split is None:
        split = kvbt.SPLIT_ALWAYS
    if ws is None:
        ws, _ = _workspace(env, w, hint, split)
    s = scores_dev if scores_dev is not None else _dev(torch, w.scores, d)
    out = (_poisoned(torch, (w.T, w.H, w.topk), d), _poisoned(torch, (w.T, w.H, w.topk * 8), d),
           _poisoned(torch, (w.T, w.H), d))
    kvbt.select_topk_and_build_table(s, _dev(torch, w.block_table, d), topk=w.topk,
                                     num_init=w.num_init, num_local=w.num_local,
                                     max_block=hint, out=out, workspace=ws, split=split,
                                     num_decode_rows=w.num_decode_rows, **_kw(env, w))
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in out), ws


def xsplit_select(env, w, hint=0, ws=None, split=None):
    torch, kvbt, d = env
    if split is None:
        split = kvbt.SPLIT_ALWAYS
    if ws is None:
        ws, _ = _workspace(env, w, hint, split)
    out = _poisoned(torch, (w.T, w.H, w.topk), d)
    kvbt.select_topk_blocks(_dev(torch, w.scores, d), _dev(torch, w.num_valid_pages, d),
                            topk=w.topk, num_init=w.num_init, num_local=w.num_local,
                            max_block=hint, num_decode_rows=w.num_decode_rows, out=out,
                            workspace=ws, split=split)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def counters_zero(w, ws):
    """The whole workspace reads zero again: counters and lists alike."""
    return not ws.cpu().numpy().any()


def _lens(M):
    return [0, 1, 100 * 128, 128 * 128, 128 * 129, 128 * 1024 + 5, 128 * 2048 + 77,
            128 * (M // 2) + 77, 128 * M - 3, 128 * M]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [1000, 8192, 16384, 65536, (1 << 19) + 1024])
def test_xsplit_rows(env, orc, M, bf16, kind):
    """Short rows (slice 0 alone), rows ending inside a slice, full rows, specials and
    mass ties; the hint 0 gives every slice, 129 one slice (the last to arrive streams
    the rest), M // 3 a part of the rows."""
    torch, kvbt, d = env
    w = wl.rows_case(300 + M % 101 + (7 if bf16 else 0), _lens(M), H=2, M=M, bf16=bf16,
                     kind=kind)
    print(w.name, M, bf16, kind, flush=True)
    want = oracle_fused(orc, w)
    for hint in (0, 129, max(129, M // 3)):
        ws, p = _workspace(env, w, hint, kvbt.SPLIT_ALWAYS)
        assert p["path"] == 4
        got, ws = xsplit_fused(env, w, hint, ws)
        assert_same(got, want, "xsplit %s %d hint %d" % (kind, M, hint))
        assert counters_zero(w, ws), "counters left non-zero"
        idx, ws = xsplit_select(env, w, hint, ws)
        assert np.array_equal(idx, want[0]), "standalone xsplit %s %d hint %d" % (kind, M, hint)
        assert counters_zero(w, ws)


@pytest.mark.parametrize("topk,ni,nl", [(1, 0, 0), (1, 1, 0), (3, 1, 2), (5, 0, 0), (13, 4, 0),
                                        (16, 0, 0), (16, 1, 2), (16, 8, 8)])
@pytest.mark.parametrize("bf16", [False, True])
def test_xsplit_topk_and_forced_counts(env, orc, topk, ni, nl, bf16):
    torch, kvbt, d = env
    M = 4104 if bf16 else 4096          # 16-byte rows either way
    lens = [1, 129, 128 * 3, 128 * 17 + 1, 128 * 129 + 1, 128 * 1025, 128 * 3000 + 9, 128 * M]
    w = wl.rows_case(400 + topk + ni, lens, H=3, M=M, kind="specials", topk=topk,
                     num_init=ni, num_local=nl, bf16=bf16)
    want = oracle_fused(orc, w)
    assert _workspace(env, w, 0, kvbt.SPLIT_ALWAYS)[1]["path"] == 4
    got, ws = xsplit_fused(env, w)
    assert_same(got, want, "xsplit topk %d ni %d nl %d" % (topk, ni, nl))
    assert counters_zero(w, ws)
    idx, _ = xsplit_select(env, w, ws=ws)
    assert np.array_equal(idx, want[0])


def test_xsplit_workloads(env, orc):
    """The few-row batches the split is for, and workloads 3-5 forced onto it (workload
    5 on sampled rows); decode rows with their block tables."""
    torch, kvbt, d = env
    for w in (wl.few_rows(1, 8192), wl.few_rows(8, 8192), wl.few_rows(8, 8192, bf16=True),
              wl.few_rows(8, 65536), wl.config(3), wl.config(4)):
        want = oracle_fused(orc, w)
        got, ws = xsplit_fused(env, w)
        assert_same(got, want, "xsplit " + w.name)
        assert counters_zero(w, ws)
    w = wl.config(5)
    rows = np.unique(np.concatenate([np.arange(0, 128), np.arange(128, w.T, 37),
                                     np.arange(w.T - 40, w.T)]))
    want = oracle_fused(orc, w, threads=16, rows=rows)
    got, ws = xsplit_fused(env, w)
    assert_same(got, want, "xsplit " + w.name, rows=rows)
    assert counters_zero(w, ws)


def test_xsplit_auto_policy(env, orc):
    """SPLIT_AUTO takes the split on a few long rows when the workspace suffices, and the
    plain launch paths otherwise; the results are the same either way."""
    torch, kvbt, d = env
    w = wl.few_rows(8, 16384)
    want = oracle_fused(orc, w)
    ws, p = _workspace(env, w, 0, kvbt.SPLIT_AUTO)
    assert p["path"] == 4
    got, _ = xsplit_fused(env, w, ws=ws, split=kvbt.SPLIT_AUTO)
    assert_same(got, want, "auto")
    small = torch.zeros(16, dtype=torch.uint8, device=d)      # too small: not split
    got, _ = xsplit_fused(env, w, ws=small, split=kvbt.SPLIT_AUTO)
    assert_same(got, want, "auto, small workspace")
    assert not small.cpu().numpy().any()
    got, _ = xsplit_fused(env, w, ws=small, split=kvbt.SPLIT_NEVER)
    assert_same(got, want, "never")


def test_xsplit_workspace_reuse_across_shapes(env, orc):
    """One workspace serves calls of different shapes in turn (the larger first)."""
    torch, kvbt, d = env
    big = wl.rows_case(501, [128 * 8192, 128 * 5000 + 1, 128 * 300, 129, 128 * 8000] * 3,
                       H=4, M=8192, kind="normal")
    small = wl.rows_case(502, [128 * 4000 + 3, 128 * 8192], H=2, M=8192, kind="specials",
                         bf16=True)
    ws, _ = _workspace(env, big, 0, kvbt.SPLIT_ALWAYS)
    for w in (big, small, big, small):
        got, ws = xsplit_fused(env, w, ws=ws)
        assert_same(got, oracle_fused(orc, w), "reuse " + w.name)
        assert counters_zero(w, ws)


def test_xsplit_graph_replay(env, orc):
    """Four replays of a captured graph (outputs poisoned before each, eager work in
    between): identical results, counters back at zero after every replay."""
    torch, kvbt, d = env
    w = wl.rows_case(503, [128 * 8192, 128 * 6000 + 5, 128 * 1500, 128 * 129, 100], H=2,
                     M=8192, kind="specials")
    want = oracle_fused(orc, w)
    ws, p = _workspace(env, w, 0, kvbt.SPLIT_ALWAYS)
    assert p["path"] == 4
    s = _dev(torch, w.scores, d)
    bt = _dev(torch, w.block_table, d)
    kw = _kw(env, w)
    out = (torch.empty(w.T, w.H, w.topk, dtype=torch.int32, device=d),
           torch.empty(w.T, w.H, w.topk * 8, dtype=torch.int32, device=d),
           torch.empty(w.T, w.H, dtype=torch.int32, device=d))

    def call():
        kvbt.select_topk_and_build_table(s, bt, topk=w.topk, num_init=w.num_init,
                                         num_local=w.num_local, out=out, workspace=ws,
                                         split=kvbt.SPLIT_ALWAYS, **kw)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert_same(tuple(o.cpu().numpy() for o in out), want, "repeat")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
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
        assert_same(tuple(o.cpu().numpy() for o in out), want, "replay %d" % rep)
        assert counters_zero(w, ws), "replay %d left a counter" % rep


def test_xsplit_misaligned_scores_fall_back(env, orc):
    """A score buffer that is not 16-byte aligned never takes the split (it reads 16-byte
    vectors); the call still gives the oracle's results."""
    torch, kvbt, d = env
    w = wl.rows_case(504, [128 * 4096, 128 * 2000 + 1, 300], H=2, M=4096, kind="normal",
                     bf16=True)
    flat = torch.empty(w.scores.size + 1, dtype=torch.bfloat16, device=d)
    flat[1:] = _dev(torch, w.scores.reshape(-1), d)
    s = flat[1:].view(w.T, w.H, w.M)
    assert s.data_ptr() % 16 != 0
    got, ws = xsplit_fused(env, w, scores_dev=s)
    assert_same(got, oracle_fused(orc, w), "misaligned")
    assert not ws.cpu().numpy().any()
