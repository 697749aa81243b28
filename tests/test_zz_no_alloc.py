"""GPU check of the allocation-free fused call (kvbt_select_topk_and_build_table_noalloc),
through the C ABI: its outputs must equal, bit for bit, those of the call with a caller's
workspace (kvbt_select_topk_and_build_table_ws) on the same inputs, for two calls in a row
on the library's scratch, the second with a smaller batch, under the library's choice and
with the split forced; and batches that take no scratch at all.
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl

pytestmark = pytest.mark.gpu

POISON = 0x7F7F7F7F


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_block_top_amd as kvbt
    kvbt.lib()
    return torch, kvbt, torch.device("cuda:0")


def _dev(torch, a, d):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(d).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def _call(env, w, split, noalloc):
    torch, kvbt, d = env
    out = tuple(torch.full(shape, POISON, dtype=torch.int32, device=d)
                for shape in ((w.T, w.H, w.topk), (w.T, w.H, w.topk * 8), (w.T, w.H)))
    kw = (dict(row_req=_dev(torch, w.row_req, d), row_pos=_dev(torch, w.row_pos, d))
          if w.explicit else dict(seq_lens=_dev(torch, w.seq_lens, d),
                                  decode_query_len=w.decode_query_len))
    args = dict(topk=w.topk, num_init=w.num_init, num_local=w.num_local,
                num_decode_rows=w.num_decode_rows, out=out, split=split, **kw)
    s, bt = _dev(torch, w.scores, d), _dev(torch, w.block_table, d)
    if noalloc:
        kvbt.select_topk_and_build_table_noalloc(s, bt, **args)
    else:
        n = kvbt.select_workspace_bytes(0, w.M, kvbt.BF16 if w.is_bf16 else kvbt.F32, w.T, w.H,
                                        w.topk, split)
        ws = torch.zeros(max(n, 16), dtype=torch.uint8, device=d)
        kvbt.select_topk_and_build_table(s, bt, workspace=ws, **args)
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in out)


def _same(a, b, what):
    for name, x, y in zip(("idx", "table", "ctx"), a, b):
        assert np.array_equal(x, y), "%s: %s differs" % (what, name)


@pytest.mark.parametrize("split", ["auto", "always"])
def test_noalloc_equals_workspace_call_twice(env, split):
    torch, kvbt, d = env
    sp = kvbt.SPLIT_AUTO if split == "auto" else kvbt.SPLIT_ALWAYS
    first = wl.few_rows(8, 16384)
    second = wl.rows_case(950, [128 * 9000 + 3, 128 * 16384, 128 * 200, 60], H=2, M=16384,
                          kind="specials", bf16=True)
    for w in (first, second):
        dtype = kvbt.BF16 if w.is_bf16 else kvbt.F32
        p = kvbt.launch_policy(0, w.M, dtype, w.T, w.H, w.topk, split=sp,
                               workspace_bytes=kvbt.NOALLOC_SCRATCH_BYTES)
        assert p["path"] == 4 and p["workspace_bytes"] <= kvbt.NOALLOC_SCRATCH_BYTES
    assert second.T * second.H < first.T * first.H
    for w in (first, second):
        _same(_call(env, w, sp, True), _call(env, w, sp, False), "%s %s" % (w.name, split))


def test_noalloc_without_split(env):
    """Batches that take no scratch (short rows, the split refused) give the same results."""
    torch, kvbt, d = env
    for w in (wl.config(2), wl.config(1), wl.few_rows(2, 8192)):
        for sp in (kvbt.SPLIT_AUTO, kvbt.SPLIT_NEVER):
            _same(_call(env, w, sp, True), _call(env, w, sp, False), w.name)
