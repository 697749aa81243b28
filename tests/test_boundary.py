"""The C-ABI library on the CPU: it loads, exports what include/*.h declares, its
launch policy keeps the 128/129 boundary, and validation rejects bad arguments
before any HIP call (no GPU is touched by any test here)."""
import ctypes
import glob
import os
import re

import pytest

import kv_block_top_amd as kvbt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

F32, BF16 = kvbt.F32, kvbt.BF16
E_NULL, E_SHAPE, E_RANGE, E_DTYPE = -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(kvbt_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = kvbt.lib()
    names = _declared_functions()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert re.match(r"^\d+\.\d+\.\d+$", kvbt.version())
    for st in (0, E_NULL, E_SHAPE, E_RANGE, E_DTYPE, -5, -6):
        assert kvbt.status_string(st) and kvbt.status_string(st) != "unknown status"
    assert kvbt.status_string(-99) == "unknown status"


@pytest.mark.parametrize("max_block,path", [
    (1, 0), (15, 0), (16, 0), (17, 0), (64, 0), (65, 0), (74, 0), (127, 0), (128, 0),
    (129, 1), (512, 1), (4096, 1), (8192, 1)])
def test_policy_boundary(max_block, path):
    p = kvbt.launch_policy(max_block, 8192, BF16, 256, 2, 16)
    assert p["path"] == path


def test_policy_zero_means_capacity():
    assert kvbt.launch_policy(0, 74, BF16, 256, 2)["path"] == 0
    assert kvbt.launch_policy(0, 128, BF16, 256, 2)["path"] == 0
    assert kvbt.launch_policy(0, 129, BF16, 256, 2)["path"] == 1


def test_policy_geometry():
    # wave path: pack up to four (row, head) per workgroup once the grid has >= 256 of them
    p = kvbt.launch_policy(74, 74, BF16, 256, 2)
    assert p["row_heads_per_block"] == 2 and p["grid"] == 256 and p["threads_per_block"] == 128
    p = kvbt.launch_policy(16, 16, F32, 4, 1)
    assert p["row_heads_per_block"] == 1 and p["grid"] == 4
    p = kvbt.launch_policy(100, 100, F32, 4096, 4)
    assert p["row_heads_per_block"] == 4 and p["grid"] == 4096
    # long-row path: four wavefronts per workgroup, rows streamed in chunks of
    # 64 lanes x 4 loads of 16 bytes when rows are 16-byte multiples, else 64 x 16 single loads
    p = kvbt.launch_policy(0, 8192, F32, 8320, 4)
    assert (p["path"], p["vec"], p["chunks"], p["grid"]) == (1, 4, 8, 8320)
    assert (p["threads_per_block"], p["row_heads_per_block"]) == (256, 4)
    p = kvbt.launch_policy(0, 8192, BF16, 65, 4)
    assert (p["path"], p["vec"], p["chunks"], p["grid"]) == (1, 8, 4, 65)
    p = kvbt.launch_policy(0, 512, BF16, 128, 4)
    assert (p["vec"], p["chunks"]) == (8, 1)
    p = kvbt.launch_policy(0, 129, BF16, 256, 4)
    assert (p["vec"], p["chunks"]) == (1, 1)
    p = kvbt.launch_policy(0, 1000, F32, 100, 4)
    assert (p["path"], p["vec"], p["chunks"]) == (1, 4, 1)
    p = kvbt.launch_policy(0, 1025, F32, 1, 1)
    assert (p["vec"], p["chunks"]) == (1, 2)
    p = kvbt.launch_policy(0, 8191, F32, 1, 1)
    assert (p["vec"], p["chunks"]) == (1, 8)


def test_policy_split_path():
    # rows over 128 blocks, 16-byte rows, and (row, head) pairs x wavefronts per pair at
    # most 256: a workgroup per pair, one wavefront per chunk of 1024 fp32 / 2048 bf16
    # tiles up to max_block (0 = max_k_tiles), at most 8
    p = kvbt.launch_policy(0, 8192, F32, 1, 4)
    assert (p["path"], p["threads_per_block"], p["row_heads_per_block"], p["grid"],
            p["vec"], p["chunks"]) == (2, 512, 1, 4, 4, 8)
    p = kvbt.launch_policy(0, 8192, BF16, 3, 1)
    assert (p["path"], p["threads_per_block"], p["grid"], p["vec"], p["chunks"]) == (2, 256, 3, 8, 4)
    p = kvbt.launch_policy(129, 8192, F32, 64, 4)
    assert (p["path"], p["threads_per_block"], p["chunks"]) == (2, 64, 1)
    p = kvbt.launch_policy(3000, 8192, F32, 8, 4)
    assert (p["path"], p["chunks"]) == (2, 3)
    p = kvbt.launch_policy(0, 1000, F32, 1, 1)
    assert (p["path"], p["vec"], p["chunks"]) == (2, 4, 1)
    assert kvbt.launch_policy(0, 8192, F32, 8, 4)["path"] == 2        # 32 x 8 waves
    assert kvbt.launch_policy(0, 8192, F32, 9, 4)["path"] == 1        # 36 x 8 > 256
    assert kvbt.launch_policy(0, 8192, BF16, 16, 4)["path"] == 2      # 64 x 4 waves
    assert kvbt.launch_policy(0, 2048, F32, 32, 4)["path"] == 2       # 128 x 2 waves
    # more pairs, unaligned rows or short rows: not the split path
    assert kvbt.launch_policy(0, 8192, F32, 65, 4)["path"] == 1
    assert kvbt.launch_policy(0, 8191, F32, 1, 1)["path"] == 1
    assert kvbt.launch_policy(128, 8192, F32, 1, 1)["path"] == 0


def test_policy_beyond_fast_path():
    # max_k_tiles over 8192: a workgroup per (row, head), one wavefront per 8192-tile
    # segment up to max_block tiles, whatever the batch size; chunks counts chunks per
    # segment
    for max_block, waves in ((0, 8), (1, 1), (128, 1), (8192, 1), (8193, 2), (65536, 8)):
        for T, H in ((1, 1), (4, 4), (1000, 4)):
            p = kvbt.launch_policy(max_block, 65536, F32, T, H)
            assert (p["path"], p["row_heads_per_block"], p["threads_per_block"], p["grid"],
                    p["vec"], p["chunks"]) == (3, 1, 64 * waves, T * H, 4, 8)
    p = kvbt.launch_policy(0, 16384, BF16, 3, 2)
    assert (p["path"], p["threads_per_block"], p["vec"], p["chunks"], p["grid"]) == (3, 128, 8, 4, 6)
    p = kvbt.launch_policy(0, 8193, F32, 1, 1)          # 32772-byte rows: single loads
    assert (p["path"], p["threads_per_block"], p["vec"], p["chunks"]) == (3, 128, 1, 8)
    assert kvbt.launch_policy(0, 8192, F32, 1, 1)["path"] == 2
    # longer rows: at most 8 wavefronts, each taking every 8th segment
    for M, max_block, waves in ((65537, 0, 8), (1 << 24, 0, 8), (1 << 24, 16384, 2),
                                (1 << 20, 1 << 20, 8), (200000, 8193, 2)):
        p = kvbt.launch_policy(max_block, M, F32, 2, 4)
        assert (p["path"], p["threads_per_block"], p["grid"]) == (3, 64 * waves, 8), (M, p)
    assert kvbt.FAST_K_TILES == 8192 and kvbt.MAX_K_TILES == 1 << 24


@pytest.mark.parametrize("args", [
    (65537, 8192, F32, 1, 1, 16), (-1, 8192, F32, 1, 1, 16), (0, 0, F32, 1, 1, 16),
    (0, (1 << 24) + 1, F32, 1, 1, 16), (0, 16, F32, -1, 1, 16), (0, 16, F32, 1, 0, 16),
    (0, 16, F32, 1, 1, 0), (0, 16, F32, 1, 1, 65), (0, 16, F32, 1 << 30, 4, 16),
    (75, 74, BF16, 1, 1, 16), (8193, 8192, F32, 1, 1, 16), (17, 16, F32, 4, 1, 16)])
def test_policy_rejects(args):
    with pytest.raises(kvbt.KvbtError) as e:
        kvbt.launch_policy(*args)
    assert e.value.status == E_RANGE


def test_policy_rejects_dtype():
    with pytest.raises(kvbt.KvbtError) as e:
        kvbt.launch_policy(0, 16, 7, 1, 1, 16)
    assert e.value.status == E_DTYPE


def _select(**kw):
    a = dict(scores=FAKE, dtype=F32, T=4, H=1, M=16, nvp=FAKE, topk=16, ni=1, nl=2,
             max_block=0, nd=0, out=FAKE)
    a.update(kw)
    return kvbt.lib().kvbt_select_topk_blocks(a["scores"], a["dtype"], a["T"], a["H"], a["M"],
                                              a["nvp"], a["topk"], a["ni"], a["nl"],
                                              a["max_block"], a["nd"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), E_DTYPE), (dict(T=-1), E_RANGE), (dict(H=0), E_RANGE),
    (dict(M=0), E_RANGE), (dict(M=(1 << 24) + 1), E_RANGE), (dict(topk=0), E_RANGE),
    (dict(topk=65), E_RANGE), (dict(ni=-1), E_RANGE), (dict(nl=-1), E_RANGE),
    (dict(ni=10, nl=7), E_RANGE), (dict(max_block=-1), E_RANGE),
    (dict(max_block=65537), E_RANGE), (dict(max_block=17), E_RANGE),
    (dict(T=1 << 29, H=8), E_RANGE),
    (dict(nd=-1), E_RANGE), (dict(nd=5), E_RANGE), (dict(T=0, nd=1), E_RANGE),
    (dict(scores=None), E_NULL), (dict(nvp=None), E_NULL), (dict(out=None), E_NULL)])
def test_select_validation(kw, status):
    assert _select(**kw) == status


def test_select_empty_batch_is_ok():
    assert _select(T=0, scores=None, nvp=None, out=None) == 0
    assert _select(T=0, scores=None, nvp=None, out=None, nd=0) == 0


def _table(**kw):
    a = dict(idx=FAKE, T=8, H=1, topk=4, bt=FAKE, B=2, mb=3, sl=FAKE, q=4, rr=None, rp=None,
             ot=FAKE, oc=FAKE)
    a.update(kw)
    return kvbt.lib().kvbt_build_sparse_block_table(a["idx"], a["T"], a["H"], a["topk"], a["bt"],
                                                    a["B"], a["mb"], a["sl"], a["q"], a["rr"],
                                                    a["rp"], a["ot"], a["oc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=7), E_SHAPE), (dict(q=3), E_SHAPE), (dict(q=0), E_RANGE), (dict(B=-1), E_RANGE),
    (dict(mb=0), E_RANGE), (dict(topk=0), E_RANGE), (dict(topk=65), E_RANGE),
    (dict(H=0), E_RANGE), (dict(sl=None), E_NULL), (dict(bt=None), E_NULL),
    (dict(idx=None), E_NULL), (dict(ot=None), E_NULL), (dict(oc=None), E_NULL),
    (dict(rr=FAKE, rp=None, T=5), E_NULL)])
def test_table_validation(kw, status):
    assert _table(**kw) == status


def test_table_empty_batch_is_ok():
    assert _table(T=0, B=0, idx=None, ot=None, oc=None) == 0


def _fused(**kw):
    a = dict(scores=FAKE, dtype=BF16, T=8, H=2, M=74, bt=FAKE, B=2, mb=74, sl=FAKE, q=4,
             rr=None, rp=None, topk=16, ni=1, nl=2, max_block=0, nd=0, oi=FAKE, ot=FAKE,
             oc=FAKE)
    a.update(kw)
    return kvbt.lib().kvbt_select_topk_and_build_table(
        a["scores"], a["dtype"], a["T"], a["H"], a["M"], a["bt"], a["B"], a["mb"], a["sl"],
        a["q"], a["rr"], a["rp"], a["topk"], a["ni"], a["nl"], a["max_block"], a["nd"],
        a["oi"], a["ot"], a["oc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=-1), E_DTYPE), (dict(T=9), E_SHAPE), (dict(M=0), E_RANGE),
    (dict(topk=3, ni=2, nl=2), E_RANGE), (dict(mb=0), E_RANGE), (dict(oi=None), E_NULL),
    (dict(ot=None), E_NULL), (dict(oc=None), E_NULL), (dict(scores=None), E_NULL),
    (dict(rr=FAKE, rp=None, T=3), E_NULL), (dict(nd=-1), E_RANGE), (dict(nd=9), E_RANGE),
    (dict(max_block=75), E_RANGE), (dict(max_block=-1), E_RANGE)])
def test_fused_validation(kw, status):
    assert _fused(**kw) == status


def test_max_block_up_to_capacity_is_accepted():
    # the hint may equal max_k_tiles (and 0 means max_k_tiles); only larger values fail
    for M in (16, 74, 128, 129, 8192, 65536):
        assert kvbt.launch_policy(M, M, F32, 4, 1)["path"] in (0, 1, 2, 3)
        with pytest.raises(kvbt.KvbtError):
            kvbt.launch_policy(M + 1, M, F32, 4, 1)


def test_dispatch_work_item_limit():
    # a dispatch counts its grid in work-items in 32 bits: workgroups x threads per
    # workgroup must stay below 2^32, or the call fails validation before any HIP call
    def total(p):
        return p["grid"] * p["threads_per_block"]
    for M, dtype, rows_ok in ((74, BF16, (1 << 26) - 4), (8192, F32, (1 << 26) - 4),
                              (65536, F32, (1 << 23) - 1)):
        p = kvbt.launch_policy(0, M, dtype, rows_ok, 1)
        assert total(p) < 1 << 32
        with pytest.raises(kvbt.KvbtError) as e:
            kvbt.launch_policy(0, M, dtype, rows_ok + 4, 1)
        assert e.value.status == E_RANGE
    assert _select(T=1 << 24, H=4) == E_RANGE
    assert _fused(T=1 << 25, B=1 << 23, H=2) == E_RANGE
    assert _table(T=1 << 28, B=1 << 26, H=1) == E_RANGE
    assert _attn(T=1 << 22, H=2, waves=8) == E_RANGE
    assert _attn(T=1 << 23, H=2, waves=0) == E_RANGE
    assert _index(B=1 << 10, ql=1, H=64, M=1024, max_blocks=1024) == E_RANGE


def test_python_layer_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    s = torch.zeros(4, 1, 16)
    with pytest.raises(ValueError):
        kvbt.select_topk_blocks(s, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        kvbt.build_sparse_block_table(torch.zeros(4, 1, 16, dtype=torch.int32),
                                      torch.zeros(4, 16, dtype=torch.int32),
                                      seq_lens=torch.zeros(4, dtype=torch.int32))


def test_bench_helpers_validate():
    L = kvbt.lib()
    assert L.kvbt_bench_empty(0, None) == E_RANGE
    assert L.kvbt_bench_copy(FAKE, FAKE, 15, None) == E_RANGE
    assert L.kvbt_bench_copy(None, FAKE, 16, None) == E_NULL
    assert L.kvbt_bench_read(FAKE, 15, FAKE, None) == E_RANGE
    assert L.kvbt_bench_read(FAKE, 0, FAKE, None) == E_RANGE
    assert L.kvbt_bench_read(None, 16, FAKE, None) == E_NULL
    assert L.kvbt_bench_read(FAKE, 16, None, None) == E_NULL


# ---------------------------------------------------------------------------
# sparse-attention decode (include/kvbt_attn.h)
# ---------------------------------------------------------------------------

def _attn(**kw):
    a = dict(q=FAKE, T=4, H=2, G=8, head_dim=128, k=FAKE, v=FAKE, P=64, table=FAKE,
             width=128, ctx=FAKE, ql=1, scale=0.088, out=FAKE, out_dtype=F32, waves=0)
    a.update(kw)
    return kvbt.lib().kvbt_sparse_attn_decode(
        a["q"], a["T"], a["H"], a["G"], a["head_dim"], a["k"], a["v"], a["P"], a["table"],
        a["width"], a["ctx"], a["ql"], ctypes.c_float(a["scale"]), a["out"], a["out_dtype"],
        a["waves"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out_dtype=7), E_DTYPE), (dict(T=-1), E_RANGE), (dict(H=0), E_RANGE),
    (dict(G=0), E_RANGE), (dict(G=17), E_RANGE), (dict(head_dim=64), E_RANGE),
    (dict(head_dim=256), E_RANGE), (dict(P=-1), E_RANGE), (dict(width=0), E_RANGE),
    (dict(width=129), E_RANGE), (dict(scale=float("nan")), E_RANGE),
    (dict(scale=float("inf")), E_RANGE), (dict(waves=3), E_RANGE), (dict(waves=16), E_RANGE),
    (dict(ql=0), E_RANGE), (dict(ql=-4), E_RANGE),
    (dict(T=1 << 30, H=2), E_RANGE), (dict(q=None), E_NULL), (dict(table=None), E_NULL),
    (dict(ctx=None), E_NULL), (dict(out=None), E_NULL), (dict(k=None), E_NULL),
    (dict(v=None), E_NULL)])
def test_attn_validation(kw, status):
    assert _attn(**kw) == status


def test_attn_empty_batch_and_empty_cache_need_no_pointers():
    assert _attn(T=0, q=None, k=None, v=None, table=None, ctx=None, out=None) == 0


def test_attn_wave_choice():
    # speculative rows: 8 below 128 pairs, else 4
    assert kvbt.sparse_attn_waves(256, 2, 4) == 4
    assert kvbt.sparse_attn_waves(63, 2, 4) == 8
    assert kvbt.sparse_attn_waves(64, 2, 4) == 4
    assert kvbt.sparse_attn_waves(4, 1, 2) == 8
    assert kvbt.sparse_attn_waves(8320, 4, 8) == 4
    # one row per request: 8 at any size
    for T, H in ((4, 1), (64, 2), (256, 2), (8320, 4)):
        assert kvbt.sparse_attn_waves(T, H, 1) == 8
        assert kvbt.sparse_attn_waves(T, H) == 8
    for T, H in ((1, 1), (128, 2), (129, 2), (8320, 4)):
        assert kvbt.sparse_attn_waves(T, H, 4) in (1, 2, 4, 8)


@pytest.mark.parametrize("T,H,G,q,grouped", [
    (256, 2, 8, 4, False),      # the 64-request spec-decode batch: 128 groups
    (512, 2, 8, 4, True),       # 128 requests: 256 groups, one per compute unit
    (510, 2, 8, 4, True),       # a request cut short by T still counts
    (508, 2, 8, 4, False),
    (4096, 2, 8, 1, False),     # one row per request: rows alone
    (1024, 2, 8, 8, True),      # 8 rows per request: two groups of 4
    (256, 2, 16, 2, True),      # 16 heads: one row per column tile
    (4096, 4, 17, 4, False),    # more heads than the columns hold
    (0, 2, 8, 4, False)])
def test_attn_grouping_choice(T, H, G, q, grouped):
    assert kvbt.sparse_attn_grouped(T, H, G, q) is grouped


def _attn_ws(**kw):
    a = dict(q=FAKE, T=4, H=2, G=8, head_dim=128, k=FAKE, v=FAKE, P=64, table=FAKE,
             width=128, ctx=FAKE, ql=4, scale=0.088, out=FAKE, out_dtype=F32, waves=0,
             splits=0, ws=FAKE, wsn=1 << 20)
    a.update(kw)
    return kvbt.lib().kvbt_sparse_attn_decode_ws(
        a["q"], a["T"], a["H"], a["G"], a["head_dim"], a["k"], a["v"], a["P"], a["table"],
        a["width"], a["ctx"], a["ql"], ctypes.c_float(a["scale"]), a["out"], a["out_dtype"],
        a["waves"], a["splits"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out_dtype=7), E_DTYPE), (dict(T=-1), E_RANGE), (dict(G=17), E_RANGE),
    (dict(width=129), E_RANGE), (dict(waves=3), E_RANGE), (dict(ql=0), E_RANGE),
    (dict(splits=-1), E_RANGE), (dict(splits=9), E_RANGE),
    (dict(wsn=-1), E_RANGE), (dict(ws=None), E_NULL), (dict(ws=ctypes.c_void_p(0x10008)), E_RANGE),
    (dict(splits=4, wsn=1024), E_RANGE),          # a split the workspace cannot hold
    (dict(splits=2, G=17), E_RANGE), (dict(q=None), E_NULL), (dict(out=None), E_NULL)])
def test_attn_ws_validation(kw, status):
    assert _attn_ws(**kw) == status


def test_attn_ws_empty_batch_needs_no_pointers():
    assert _attn_ws(T=0, q=None, k=None, v=None, table=None, ctx=None, out=None, ws=None,
                    wsn=0, splits=4) == 0


@pytest.mark.parametrize("T,H,splits", [
    (256, 2, 0),                # the 64-request spec-decode batch: 512 pairs, never split
    (80, 2, 0),                 # 160 pairs: the per-row kernel alone
    (40, 4, 0),
    (159, 1, 2),                # below 160 pairs: 2 workgroups each
    (64, 2, 2),
    (33, 2, 2),                 # 66 pairs
    (32, 2, 4),                 # up to 64 pairs: 4 each
    (16, 2, 4),
    (8, 1, 4),
    (1, 1, 4)])
def test_attn_split_choice(T, H, splits):
    assert kvbt.sparse_attn_splits(T, H) == splits
    n = kvbt.sparse_attn_workspace_bytes(T, H)
    assert (n > 0) == (splits > 0)
    if splits:
        # the workspace it asks for is exactly enough
        assert kvbt.sparse_attn_splits(T, H, 0, n) == splits
        assert kvbt.sparse_attn_splits(T, H, 0, n - 1) == 0
        assert n % 256 == 0


def test_attn_split_workspace_layout():
    # 256-byte lines: 16 bytes of counter, 15 slots of 16 bytes of partial results; one
    # partial result is 520 slots (O, then (m, l)); 32 pairs x 4 splits = 66,560 slots =
    # 4,438 lines (rounded up)
    assert kvbt.sparse_attn_workspace_bytes(16, 2) == -(-32 * 4 * 520 // 15) * 256 == 4438 * 256
    assert kvbt.sparse_attn_workspace_bytes(1, 1, 8) == -(-8 * 520 // 15) * 256
    # explicit splits for any batch; 1 never splits
    for S in range(2, kvbt.ATTN_MAX_SPLITS + 1):
        assert kvbt.sparse_attn_splits(8, 1, S) == S
        assert kvbt.sparse_attn_splits(1024, 2, S) == S
        assert kvbt.sparse_attn_workspace_bytes(1024, 2, S) == -(-2048 * S * 520 // 15) * 256
    assert kvbt.sparse_attn_splits(16, 2, 1) == 0
    assert kvbt.sparse_attn_workspace_bytes(16, 2, 1) == 0
    assert kvbt.sparse_attn_splits(0, 2, 4) == 0
    assert kvbt.sparse_attn_workspace_bytes(0, 2, 4) == 0
    # partial results past a 32-bit slot index: no split
    assert kvbt.sparse_attn_splits(1 << 19, 1, 8) == 0
    with pytest.raises(kvbt.KvbtError):
        kvbt.sparse_attn_workspace_bytes(1 << 19, 1, 8)
    with pytest.raises(kvbt.KvbtError):
        kvbt.sparse_attn_workspace_bytes(16, 2, 9)
    with pytest.raises(kvbt.KvbtError):
        kvbt.sparse_attn_workspace_bytes(1 << 30, 4, 0)


# ---------------------------------------------------------------------------
# decode index scores (include/kvbt_index.h)
# ---------------------------------------------------------------------------

def _index(**kw):
    a = dict(q=FAKE, B=4, ql=4, H=2, head_dim=128, k=FAKE, kd=BF16, ks=None, P=64, bt=FAKE,
             max_blocks=74, seq=FAKE, scale=0.088, reduce=0, scores=FAKE, dtype=F32, M=74)
    a.update(kw)
    return kvbt.lib().kvbt_index_decode_scores(
        a["q"], a["B"], a["ql"], a["H"], a["head_dim"], a["k"], a["kd"], a["ks"], a["P"],
        a["bt"], a["max_blocks"], a["seq"], ctypes.c_float(a["scale"]), a["reduce"],
        a["scores"], a["dtype"], a["M"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), E_DTYPE), (dict(reduce=2), E_RANGE), (dict(B=-1), E_RANGE),
    (dict(H=0), E_RANGE), (dict(ql=0), E_RANGE), (dict(ql=17), E_RANGE),
    (dict(head_dim=64), E_RANGE), (dict(P=-1), E_RANGE), (dict(max_blocks=0), E_RANGE),
    (dict(M=0), E_RANGE), (dict(M=(1 << 24) + 1), E_RANGE), (dict(scale=float("nan")), E_RANGE),
    (dict(B=1 << 28, ql=16, H=1), E_RANGE), (dict(q=None), E_NULL), (dict(bt=None), E_NULL),
    (dict(seq=None), E_NULL), (dict(scores=None), E_NULL), (dict(k=None), E_NULL),
    (dict(kd=F32), E_DTYPE), (dict(kd=7), E_DTYPE), (dict(kd=kvbt.FP8_E4M3), E_NULL)])
def test_index_validation(kw, status):
    assert _index(**kw) == status


def test_index_empty_batch_needs_no_pointers():
    assert _index(B=0, q=None, k=None, bt=None, seq=None, scores=None) == 0


# ---------------------------------------------------------------------------
# cross-workgroup split (path 4) with a caller's workspace
# ---------------------------------------------------------------------------

AUTO, ALWAYS, NEVER = kvbt.SPLIT_AUTO, kvbt.SPLIT_ALWAYS, kvbt.SPLIT_NEVER


def _ws_bytes(pairs, slices):
    return pairs * 256 + pairs * slices * 128


@pytest.mark.parametrize("M,dtype,T,H,max_block,waves,slices", [
    (8192, F32, 8, 4, 0, 1, 8), (8192, BF16, 8, 4, 0, 1, 4), (65536, F32, 8, 4, 0, 8, 8),
    (65536, BF16, 1, 4, 0, 4, 8), (65536, F32, 2, 1, 5000, 1, 5), (8192, F32, 1, 1, 129, 1, 1),
    (1000, F32, 3, 2, 0, 1, 1), (8192, F32, 8320, 4, 0, 1, 8), (32768, F32, 4, 1, 0, 4, 8),
    (20000, F32, 4, 1, 0, 4, 5), (16384, F32, 4, 1, 0, 2, 8)])
def test_policy_split_always_geometry(M, dtype, T, H, max_block, waves, slices):
    # chunks of 1024 fp32 / 2048 bf16 tiles up to max_block tiles, one per wavefront; a
    # slice workgroup takes the fewest (a power of two, up to 8) that leave at most 8
    # slices per (row, head); the workspace: a 256-byte line per counter, then 16
    # 64-bit keys per (row, head) and slice
    need = kvbt.select_workspace_bytes(max_block, M, dtype, T, H, 16, ALWAYS)
    assert need == _ws_bytes(T * H, slices)
    p = kvbt.launch_policy(max_block, M, dtype, T, H, 16, split=ALWAYS, workspace_bytes=need)
    assert (p["path"], p["threads_per_block"], p["grid"], p["slices"], p["chunks"],
            p["workspace_bytes"]) == (4, 64 * waves, T * H * slices, slices, waves, need)
    with pytest.raises(kvbt.KvbtError) as e:
        kvbt.launch_policy(max_block, M, dtype, T, H, 16, split=ALWAYS, workspace_bytes=need - 1)
    assert e.value.status == E_RANGE


def test_policy_split_auto_and_never():
    # the library's choice: at most 128 (row, head) pairs whose hinted rows span at
    # least four chunks, where the launch without a workspace would stream them (path 1
    # or 3), with enough workspace; otherwise the paths without a workspace
    big = 1 << 40
    for M, dtype, T, H, path in ((8192, F32, 8, 4, 2), (8192, F32, 32, 4, 4),
                                 (8192, F32, 33, 4, 1), (65536, F32, 8, 4, 4),
                                 (65536, BF16, 1, 1, 4), (16384, F32, 2, 4, 4),
                                 (16384, F32, 64, 4, 3), (8192, BF16, 16, 4, 2),
                                 (8192, BF16, 64, 4, 1), (4096, F32, 32, 4, 4),
                                 (3072, F32, 8, 4, 2), (512, BF16, 128, 4, 1),
                                 (74, BF16, 256, 2, 0), (8192, F32, 8320, 4, 1)):
        p = kvbt.launch_policy(0, M, dtype, T, H, 16, split=AUTO, workspace_bytes=big)
        assert p["path"] == path, (M, T, H, p)
        assert (p["workspace_bytes"] > 0) == (path == 4)
        assert kvbt.select_workspace_bytes(0, M, dtype, T, H) == p["workspace_bytes"]
        q = kvbt.launch_policy(0, M, dtype, T, H, 16, split=NEVER, workspace_bytes=big)
        assert q == kvbt.launch_policy(0, M, dtype, T, H, 16)
    # too small a workspace: not split, no error
    p = kvbt.launch_policy(0, 65536, F32, 8, 4, 16, split=AUTO, workspace_bytes=1000)
    assert p["path"] == 3 and p["workspace_bytes"] == 0
    # the library splits only rows its slices cover (64 slices x 8 wavefronts x 1024 fp32
    # or 2048 bf16 tiles); forced, longer rows finish in the last slice
    for M, dtype, path in (((1 << 19), F32, 4), ((1 << 19) + 1024, F32, 3), ((1 << 20), BF16, 4),
                           ((1 << 20) + 8, BF16, 3), ((1 << 24), F32, 3)):
        p = kvbt.launch_policy(0, M, dtype, 1, 4, 16, split=AUTO, workspace_bytes=big)
        assert p["path"] == path, (M, dtype, p)
        p = kvbt.launch_policy(0, M, dtype, 1, 4, 16, split=ALWAYS, workspace_bytes=big)
        assert (p["path"], p["slices"], p["threads_per_block"]) == (4, 64, 512), (M, p)
    # rows that are not 16-byte multiples, or hints of at most 128 blocks: never split
    assert kvbt.launch_policy(0, 8191, F32, 1, 1, 16, split=ALWAYS, workspace_bytes=big)["path"] == 1
    assert kvbt.launch_policy(128, 8192, F32, 1, 1, 16, split=ALWAYS,
                              workspace_bytes=big)["path"] == 0
    assert kvbt.select_workspace_bytes(128, 8192, F32, 1, 1, 16, ALWAYS) == 0


def test_policy_split_rejects():
    for split, wsb in ((3, 0), (-1, 0), (AUTO, -1)):
        with pytest.raises(kvbt.KvbtError) as e:
            kvbt.launch_policy(0, 8192, F32, 8, 4, 16, split=split, workspace_bytes=wsb)
        assert e.value.status == E_RANGE
    assert kvbt.lib().kvbt_select_workspace_bytes(0, 8192, 7, 8, 4, 16, AUTO) == E_DTYPE
    assert kvbt.lib().kvbt_launch_policy_ws(0, 8192, F32, 8, 4, 16, AUTO, 0, None) == E_NULL


def _select_ws(**kw):
    a = dict(scores=FAKE, dtype=F32, T=8, H=4, M=8192, nvp=FAKE, topk=16, ni=1, nl=2,
             max_block=0, nd=0, out=FAKE, split=ALWAYS, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return kvbt.lib().kvbt_select_topk_blocks_ws(
        a["scores"], a["dtype"], a["T"], a["H"], a["M"], a["nvp"], a["topk"], a["ni"], a["nl"],
        a["max_block"], a["nd"], a["out"], a["split"], a["ws"], a["wsb"], None)


def _fused_ws(**kw):
    a = dict(scores=FAKE, dtype=F32, T=8, H=4, M=8192, bt=FAKE, B=8, mb=8192, sl=FAKE, q=1,
             rr=None, rp=None, topk=16, ni=1, nl=2, max_block=0, nd=0, oi=FAKE, ot=FAKE,
             oc=FAKE, split=ALWAYS, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return kvbt.lib().kvbt_select_topk_and_build_table_ws(
        a["scores"], a["dtype"], a["T"], a["H"], a["M"], a["bt"], a["B"], a["mb"], a["sl"],
        a["q"], a["rr"], a["rp"], a["topk"], a["ni"], a["nl"], a["max_block"], a["nd"],
        a["oi"], a["ot"], a["oc"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), E_NULL), (dict(wsb=-1), E_RANGE), (dict(ws=ctypes.c_void_p(0x10008)), E_RANGE),
    (dict(split=5), E_RANGE), (dict(wsb=1000), E_RANGE), (dict(max_block=8193), E_RANGE),
    (dict(topk=65), E_RANGE), (dict(scores=None), E_NULL), (dict(dtype=3), E_DTYPE)])
def test_ws_entry_points_validate(kw, status):
    assert _select_ws(**kw) == status
    assert _fused_ws(**kw) == status


def test_ws_entry_points_empty_batch():
    assert _select_ws(T=0, scores=None, nvp=None, out=None, ws=None, wsb=0) == 0
    assert _fused_ws(T=0, B=0, scores=None, oi=None, ot=None, oc=None, ws=None, wsb=0) == 0


@pytest.mark.parametrize("M,dtype,vec", [(74, BF16, 1), (128, BF16, 8), (129, F32, 1),
                                         (8192, F32, 4), (65536, BF16, 8), (8193, F32, 1)])
@pytest.mark.parametrize("topk", [17, 32, 64])
def test_policy_topk_above_16(M, dtype, vec, topk):
    # topk above 16: path 5 whatever the hint and batch (a wavefront per (row, head), four
    # per workgroup), 16-byte loads on 16-byte rows; never the cross-workgroup split
    for max_block, T, H in ((0, 4, 1), (1, 256, 2), (M, 8320, 4)):
        for split in (None, ALWAYS):
            p = kvbt.launch_policy(max_block, M, dtype, T, H, topk, split=split,
                                   workspace_bytes=1 << 40)
            assert (p["path"], p["threads_per_block"], p["row_heads_per_block"], p["grid"],
                    p["vec"], p["workspace_bytes"]) == (5, 256, 4, (T * H + 3) // 4, vec, 0)
    assert kvbt.launch_policy(0, M, dtype, 4, 1, 16)["path"] != 5
    assert kvbt.MAX_TOPK == 64 and kvbt.FAST_TOPK == 16


# ---------------------------------------------------------------------------
# the allocation-free fused call
# ---------------------------------------------------------------------------

E_SCRATCH = -6


def _noalloc(**kw):
    a = dict(scores=FAKE, dtype=F32, T=8, H=4, M=8192, bt=FAKE, B=8, mb=8192, sl=FAKE, q=1,
             rr=None, rp=None, topk=16, ni=1, nl=2, max_block=0, nd=0, oi=FAKE, ot=FAKE,
             oc=FAKE, split=AUTO)
    a.update(kw)
    return kvbt.lib().kvbt_select_topk_and_build_table_noalloc(
        a["scores"], a["dtype"], a["T"], a["H"], a["M"], a["bt"], a["B"], a["mb"], a["sl"],
        a["q"], a["rr"], a["rp"], a["topk"], a["ni"], a["nl"], a["max_block"], a["nd"],
        a["oi"], a["ot"], a["oc"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(split=4), E_RANGE), (dict(topk=65), E_RANGE), (dict(max_block=8193), E_RANGE),
    (dict(T=9), E_SHAPE), (dict(scores=None), E_NULL), (dict(oc=None), E_NULL),
    (dict(dtype=5), E_DTYPE),
    # the split forced on a batch whose lists exceed the scratch: refused, nothing launched
    (dict(T=8320, B=8320, split=ALWAYS), E_SCRATCH),
    (dict(T=1024, B=1024, H=4, M=65536, mb=65536, split=ALWAYS), E_SCRATCH)])
def test_noalloc_validation(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_covers_the_library_choice():
    # every batch the library would split on its own fits the scratch
    assert kvbt.NOALLOC_SCRATCH_BYTES == 1 << 20
    for M in (4096, 8192, 16384, 65536):
        for dtype in (F32, BF16):
            n = kvbt.select_workspace_bytes(0, M, dtype, 128, 1, 16, AUTO)
            assert 0 <= n <= kvbt.NOALLOC_SCRATCH_BYTES
    assert kvbt.select_workspace_bytes(0, 65536, F32, 128, 1, 16, AUTO) > 0
