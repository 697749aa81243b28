"""GPU parity of topk above 16 (launch path 5, up to 64), through the C ABI.

One wavefront per (row, head) keeps a running top-64 and builds the table of up to 64
blocks. Every result must equal the oracle's bit for bit (outputs poisoned before each
call), for fp32 and bf16 scores, 16-byte and unaligned rows, special values and mass
ties, every row length around the topk and the wavefront width, decode and explicit
rows, the fused call, the standalone selector and the standalone table builder.
"""
import numpy as np
import pytest

from kv_block_top_amd import workloads as wl
from test_gpu_parity import gpu_fused, gpu_select, gpu_table, oracle_fused

pytestmark = pytest.mark.gpu

TOPKS = [17, 31, 32, 48, 64]


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_block_top_amd as kvbt
    kvbt.lib()
    return torch, kvbt, torch.device("cuda:0")


def _check(env, orc, w, what):
    torch, kvbt, d = env
    dtype = kvbt.BF16 if w.is_bf16 else kvbt.F32
    assert kvbt.launch_policy(0, w.M, dtype, w.T, w.H, w.topk)["path"] == 5
    want = oracle_fused(orc, w)
    got = gpu_fused(env, w, "policy")
    for name, g, e in zip(("idx", "table", "ctx"), got, want):
        assert np.array_equal(g, e), "%s: %s differs" % (what, name)
    got = gpu_fused(env, w, "short")     # the hint changes nothing above topk 16
    assert all(np.array_equal(g, e) for g, e in zip(got, want)), what + " (hint 1)"
    assert np.array_equal(gpu_select(env, w), want[0]), what + " (standalone)"
    table, ctx = gpu_table(env, w, want[0])
    assert np.array_equal(table, want[1]) and np.array_equal(ctx, want[2]), what + " (table)"


@pytest.mark.parametrize("topk", TOPKS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [74, 129, 512, 1003, 8192])
def test_wide_topk_rows(env, orc, topk, bf16, M):
    lens = [0, 1, 128 * 3, 128 * (topk - 1) + 7, 128 * topk, 128 * topk + 1, 128 * 63 + 1,
            128 * 64, 128 * 65, 128 * 127 + 3, 128 * 128, 128 * 129, 128 * (M // 2) + 9, 128 * M]
    w = wl.rows_case(600 + topk + M % 97, lens, H=2, M=M, bf16=bf16, kind="specials", topk=topk)
    _check(env, orc, w, "topk %d M %d bf16 %s" % (topk, M, bf16))


@pytest.mark.parametrize("kind", ["normal", "ties", "increasing", "two_level", "neginf", "nan"])
@pytest.mark.parametrize("topk,ni,nl", [(17, 1, 2), (32, 0, 0), (64, 1, 2), (64, 32, 32),
                                        (40, 7, 0), (20, 0, 5)])
def test_wide_topk_kinds_and_forced(env, orc, kind, topk, ni, nl):
    lens = [1, 128 * 2, 128 * 40 + 1, 128 * 64, 128 * 100 + 3, 128 * 700, 128 * 2048]
    w = wl.rows_case(700 + topk + ni, lens, H=3, M=2048, kind=kind, topk=topk, num_init=ni,
                     num_local=nl)
    _check(env, orc, w, "%s topk %d ni %d nl %d" % (kind, topk, ni, nl))


@pytest.mark.parametrize("M", [8193, 65536, 200003])
def test_wide_topk_beyond_fast_path(env, orc, M):
    lens = [0, 1, 128 * 100, 128 * 8192, 128 * 8193 + 1, 128 * M]
    for bf16 in (False, True):
        w = wl.rows_case(800 + M % 91, lens, H=2, M=M, bf16=bf16, kind="normal", topk=64)
        _check(env, orc, w, "M %d bf16 %s" % (M, bf16))


@pytest.mark.parametrize("seed", range(4))
def test_wide_topk_decode_rows(env, orc, seed):
    """Decode-form rows (spec decode q 4, padded requests, seq_len < q) and explicit rows
    with out-of-range requests and max_blocks below the capacity."""
    rng = np.random.default_rng(850 + seed)
    topk = int(rng.choice(TOPKS))
    w = wl.random_case(850 + seed, T=64, H=2, M=300, q=4, topk=topk, special_frac=0.05,
                       tie_frac=0.05, max_blocks=int(rng.integers(topk, 301)))
    _check(env, orc, w, "decode seed %d topk %d" % (seed, topk))
    w = wl.random_case(860 + seed, T=40, H=2, M=600, explicit=True, topk=topk,
                       max_blocks=int(rng.integers(1, 601)), bf16=True)
    _check(env, orc, w, "explicit seed %d topk %d" % (seed, topk))


@pytest.mark.parametrize("seed", range(4))
def test_wide_topk_table_on_arbitrary_idx(env, orc, seed):
    """The standalone builder above topk 16: repeats, -1 anywhere, ids past the causal
    count or the block table."""
    rng = np.random.default_rng(870 + seed)
    w = wl.random_case(870 + seed, T=64, H=3, M=200, q=4, max_blocks=int(rng.integers(1, 210)))
    K = int(rng.choice([17, 33, 64]))
    idx = rng.integers(-3, 210, size=(w.T, w.H, K)).astype(np.int32)
    idx[:, :, 1] = idx[:, :, 0]
    idx[:, :, 10:14] = idx[:, :, 2:6]
    table, ctx = gpu_table(env, w, idx)
    ot, oc = orc.build_sparse_block_table(idx, w.block_table, **w.row_kwargs())
    assert np.array_equal(table, ot) and np.array_equal(ctx, oc)
