"""Benchmark of the fused top-k block selector + page-16 sparse block table.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--no-long]
                    [--no-cpu] [--profile-only]

A step is one fused call (select + table, one launch) over one batch of the
workload, with inputs resident in HBM. The K timed steps are captured in one HIP
graph and replayed once between two events on the launch stream, so host launch
overhead is excluded; ms_per_step = elapsed / K.

Workloads (seeded, synthetic; kv_block_top_amd.workloads):
    2 (default): 64 spec-decode requests x query length 4, 2 index heads, capacity
                 74 blocks, bf16 scores -- the short-context production shape;
    "configs" times all five workloads the same way, each with its own record (µs per
                 call warm and cold, the launch floor and the time above it, rows/s,
                 algorithmic bytes, roofline object, launch policy, and the oracle's rate
                 on all host threads and on one): 1 tiny decode (4 rows, 16 tiles, fp32),
                 2 as above, 3 boundary + special values (256 rows x 4 heads, 129 tiles,
                 bf16), 4 long-context decode (128 rows x 4 heads, 512 tiles, bf16), 5 the
                 8320-row mixed decode + prefill buffer, 4 heads, 8192 tiles (1M tokens),
                 fp32 (also reported under "long_context");
    "few_rows": 1 or 8 decode rows x 4 heads at the full capacity of 8192 or 65536
                 tiles (fp32), far fewer (row, head) pairs than compute units.
The primary figure is warm (the same
inputs every call, as a serving step reads scores just written); "cold" repeats the
call over > 512 MB of distinct input copies so that every call reads from HBM.

Algorithmic bytes per call (the roofline numerator): the scores of every causal
tile, sum over (row, head) of nvp * sizeof(score); the idx, table and ctx writes,
T*H*(topk + 8*topk + 1)*4; one 4-byte block-table read per valid selected block,
sum of min(topk, nvp)*4; the row metadata (seq_lens B*4, or row_req/row_pos T*8).

"sparse_attention" times the consumer of the table: the sparse paged-attention decode
over the default workload's own page-16 table and ctx (8 query heads per index head,
head dimension 128, bf16 cache of the pages the table names, fp32 output).
"sparse_attention_large_batch" repeats that table 4 times as further requests with
pages of their own (256 requests): large enough that the rows of each request are
attended together. Its
algorithmic bytes are the minimum any kernel must move: each distinct (page, KV head)
the rows name, 4 KB of keys plus 4 KB of values, read once; the queries; the output;
the table entries used and ctx. "sparse_attention_long" does the same over the first
64 rows of the 64k-token long-context decode workload's table (one row per request, so
no page is shared and the pages stream past the caches). "sparse_attention_few_rows"
times the first 16 and 64 rows of the default workload's table (32 and 128 (row, head)
pairs, which leave most compute units idle) with a workspace, where every (row, head)
is split across workgroups, next to the same call without one.

"index_scores" times the step before the selector: the decode index-score producer
over the default workload's requests (their seq_lens, query length and heads; seeded
index queries and a compact paged index-K cache, head dimension 128, log-sum-exp
reduction), writing the decode rows of a score buffer shaped like the workload's.
Its algorithmic bytes: the index keys of every causal token of every request and head,
read once (256 bytes each), the queries, the scores written and the block-table
entries; "index_scores_long" does the same for the first 8 requests of the 64k-token
long-context decode workload, and "index_scores_long_fp8" for the same requests with
the keys in the FP8 (E4M3) cache (128 bytes of codes + a 4-byte scale per key).

"decode_step" times the three calls of one decode step in one graph (index scores ->
fused select + table -> sparse attention) on the default workload's requests, the
index-K and KV caches paged by one shared block table; "decode_step_fp8_index" the same
with the optional FP8 (E4M3) index cache in place of the bf16 one.

The attention, index-score and decode-step legs cycle through several device copies of
their caches ("input_copies"), so that between two uses of one copy at least 512 MB of
others is read: in serving, each layer reads its own caches, so a call never finds them
in the chip's 256 MB memory-side cache. Replaying one copy would let that cache serve
much of the attention's 300 MB KV cache (41 instead of 55 us per call on the
spec-decode table).

The CPU oracle is used only by the cpu-baseline leg (skipped with --no-cpu): it times
the oracle, and checks the GPU results it saw against the oracle's on the same inputs
(all rows of workload 2, sampled rows of workload 5 and of the attention).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD published peak
MALL_BYTES = 256 << 20   # MI355X Infinity Cache: memory-side, in front of HBM

# HBM traffic per launch from rocprofv3 counter runs of `bench.py --profile-only`
# (summaries under profiles/): FETCH_SIZE and WRITE_SIZE in KiB per dispatch of the
# measured kernel, averaged over the dispatches. A plain 256 MiB copy reads FETCH_SIZE
# 131083 KiB and WRITE_SIZE 262144 KiB on the same box, so FETCH_SIZE counts half the
# bytes read: fetched bytes = 2.0 x FETCH_SIZE, written bytes = 1.0 x WRITE_SIZE. A
# reading holds only for the sources of its kernel it was taken on (their SHA-256);
# after any change to them the traffic is reported as null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
KERNEL_SOURCES = {
    "select": ("kv_block_top_amd/csrc/kvbt_kernels.hip", "kv_block_top_amd/csrc/kvbt_device.h",
               "kv_block_top_amd/csrc/kvbt_divide.h", "kv_block_top_amd/csrc/kvbt_launch.h",
               "kv_block_top_amd/csrc/kvbt_api.cpp", "include/kvbt.h"),
    "attn": ("kv_block_top_amd/csrc/kvbt_attn.hip", "kv_block_top_amd/csrc/kvbt_device.h",
             "kv_block_top_amd/csrc/kvbt_divide.h", "kv_block_top_amd/csrc/kvbt_attn_launch.h",
             "kv_block_top_amd/csrc/kvbt_api.cpp", "include/kvbt_attn.h"),
    "index": ("kv_block_top_amd/csrc/kvbt_index.hip", "kv_block_top_amd/csrc/kvbt_device.h",
              "kv_block_top_amd/csrc/kvbt_divide.h", "kv_block_top_amd/csrc/kvbt_index_launch.h",
              "kv_block_top_amd/csrc/kvbt_api.cpp", "include/kvbt_index.h"),
}
SELECT_SOURCES_SHA256 = "b3dedf16c179ae2942a8fd250142895ab3178d137675b5dd0d8a08e6a00ea281"
ATTN_SOURCES_SHA256 = "9dd50f3bb02f97b5ce0520a89c15858bdad3c7e0ea2c48b47fa4dbb75800ca38"
INDEX_SOURCES_SHA256 = "dfe4c6fcb18d723654aa9722ccd463079810aa07177b1cfd59c9eeb6790381fb"
COUNTERS = {   # workload -> (kernel, sources SHA-256, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "tiny_decode_b4_t16_h1_f32": ("select", SELECT_SOURCES_SHA256, 23.50, 2.38),
    "spec_decode_b64_q4_t74_h2_bf16": ("select", SELECT_SOURCES_SHA256, 125.75, 296.00),
    "boundary_specials_b256_t129_h4_bf16": ("select", SELECT_SOURCES_SHA256, 240.25, 584.00),
    "long_decode_b128_t512_h4_bf16": ("select", SELECT_SOURCES_SHA256, 382.56, 292.00),
    "mixed_unified_t8320_h4_tiles8192_f32": ("select", SELECT_SOURCES_SHA256,
                                             294470.10, 18990.84),
    # few rows: the call with a workspace, the library's choice (path 2 at 8192 tiles,
    # the cross-workgroup split at 65536)
    "few_rows_r1_h4_tiles8192_f32": ("select", SELECT_SOURCES_SHA256, 116.69, 2.38),
    "few_rows_r8_h4_tiles8192_f32": ("select", SELECT_SOURCES_SHA256, 644.06, 19.00),
    "few_rows_r8_h4_tiles65536_f32": ("select", SELECT_SOURCES_SHA256, 4297.58, 91.30),
    "sparse_attn_spec_decode_b64_q4_t74_h2_bf16_g8_d128": ("attn", ATTN_SOURCES_SHA256,
                                                           133016.02, 2048.43),
    "sparse_attn_spec_decode_b64_q4_t74_h2_bf16_x4_g8_d128": ("attn", ATTN_SOURCES_SHA256,
                                                              482706.95, 8192.73),
    "sparse_attn_long_decode_b128_t512_h4_bf16_r64_g8_d128": ("attn", ATTN_SOURCES_SHA256,
                                                              127780.50, 1024.00),
    # few rows with a workspace: each (row, head) split across workgroups
    "sparse_attn_spec_decode_b64_q4_t74_h2_bf16_r16_g8_d128_split": ("attn",
                                                                     ATTN_SOURCES_SHA256,
                                                                     9981.76, 1354.38),
    "sparse_attn_spec_decode_b64_q4_t74_h2_bf16_r64_g8_d128_split": ("attn",
                                                                     ATTN_SOURCES_SHA256,
                                                                     31040.08, 2966.66),
    "index_scores_spec_decode_b64_q4_t74_h2_bf16_d128_lse": ("index", INDEX_SOURCES_SHA256,
                                                             83537.02, 172.39),
    "index_scores_long_decode_b128_t512_h4_bf16_r8_d128_lse": ("index", INDEX_SOURCES_SHA256,
                                                               230151.44, 113.05),
    "index_scores_long_decode_b128_t512_h4_bf16_r8_d128_fp8_lse": ("index",
                                                                   INDEX_SOURCES_SHA256,
                                                                   120063.11, 112.95),
}


def _nvp(w):
    if w.explicit:
        c = np.maximum(w.row_pos.astype(np.int64) + 1, 0)
        bad = (w.row_req < 0) | (w.row_req >= w.B)
        c[bad] = 0
    else:
        q = w.decode_query_len
        t = np.arange(w.T)
        req = t // q
        c = np.maximum(w.seq_lens.astype(np.int64)[req] - q + (t - req * q) + 1, 0)
    return np.minimum((c + 127) // 128, w.M)


def kernel_sources_sha256(kernel: str) -> str:
    """SHA-256 over the sources a kernel's code comes from (paths and contents)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(name: str):
    """HBM bytes per launch from the recorded counters, or None if not measured on
    the current sources of the kernel."""
    rec = COUNTERS.get(name)
    if rec is None or kernel_sources_sha256(rec[0]) != rec[1]:
        return None
    return int(round((rec[2] * FETCH_SCALE + rec[3] * WRITE_SCALE) * 1024))


def inputs_sha256(w) -> str:
    """SHA-256 over every input array of the workload (scores, block table, row
    description), in a fixed order: identifies the exact inputs a result was measured on."""
    import hashlib
    h = hashlib.sha256()
    for arr in (w.scores, w.block_table, w.num_valid_pages, w.seq_lens, w.row_req, w.row_pos):
        if arr is not None:
            h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()


def algorithmic_bytes(w) -> int:
    nvp = _nvp(w)
    s = 2 if w.is_bf16 else 4
    scores = int(nvp.sum()) * w.H * s
    outputs = w.T * w.H * (w.topk + 8 * w.topk + 1) * 4
    gathers = int(np.minimum(w.topk, nvp).sum()) * w.H * 4
    meta = w.T * 8 if w.explicit else w.B * 4
    return scores + outputs + gathers + meta


def _to_dev(torch, a, d):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(d).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


class FusedCall:
    """Device-resident inputs and outputs of one workload, and the call itself; with
    `split` given, through the workspace entry point with a workspace of its own."""

    def __init__(self, torch, kvbt, w, d, split=None):
        self.w = w
        self.kvbt = kvbt
        self.split = split
        self.ws = None
        if split is not None:
            n = kvbt.select_workspace_bytes(w.max_block, w.M, kvbt.BF16 if w.is_bf16 else kvbt.F32,
                                            w.T, w.H, w.topk, split)
            self.ws = torch.zeros(max(n, 16), dtype=torch.uint8, device=d)
        self.s = _to_dev(torch, w.scores, d)
        self.bt = _to_dev(torch, w.block_table, d)
        if w.explicit:
            self.kw = dict(row_req=_to_dev(torch, w.row_req, d),
                           row_pos=_to_dev(torch, w.row_pos, d))
        else:
            self.kw = dict(seq_lens=_to_dev(torch, w.seq_lens, d),
                           decode_query_len=w.decode_query_len)
        self.out = (torch.empty(w.T, w.H, w.topk, dtype=torch.int32, device=d),
                    torch.empty(w.T, w.H, w.topk * 8, dtype=torch.int32, device=d),
                    torch.empty(w.T, w.H, dtype=torch.int32, device=d))

    def __call__(self):
        self.kvbt.select_topk_and_build_table(self.s, self.bt, topk=self.w.topk,
                                              num_init=self.w.num_init,
                                              num_local=self.w.num_local,
                                              num_decode_rows=self.w.num_decode_rows,
                                              out=self.out, workspace=self.ws,
                                              split=self.split, **self.kw)

    def outputs(self):
        return tuple(o.cpu().numpy() for o in self.out)


def rotation_copies(footprint: int) -> int:
    """Input copies a timed loop cycles through so that no call finds its inputs in the
    memory-side cache: between two uses of one copy, at least twice that cache's size
    of other copies is read."""
    return 1 + max(1, -(-2 * MALL_BYTES // max(int(footprint), 1)))


class Rotation:
    """Calls its callables in turn (one per call), each bound to its own input copy."""

    def __init__(self, calls):
        self.calls, self.k = list(calls), 0

    def __call__(self):
        self.calls[self.k % len(self.calls)]()
        self.k += 1


def time_graph(torch, fn, steps: int, warmup: int) -> float:
    """Seconds per call: `steps` calls captured in one graph, replayed once."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    g.replay()                       # untimed: pages the graph in
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e-3 / steps


def measure(torch, kvbt, w, d, steps, warmup, copies=1, split=None):
    """Times the fused call on `w`; with copies > 1 the calls cycle through that many
    device copies of the inputs; `split` as in FusedCall."""
    call = FusedCall(torch, kvbt, w, d, split)
    call()
    torch.cuda.synchronize()
    outputs = call.outputs()
    if copies > 1:
        calls = [call] + [FusedCall(torch, kvbt, w, d, split) for _ in range(copies - 1)]
        sec = time_graph(torch, Rotation(calls), steps, warmup)
        del calls
    else:
        sec = time_graph(torch, call, steps, warmup)
    ab = algorithmic_bytes(w)
    achieved = ab / sec / 1e9
    policy = kvbt.launch_policy(w.max_block, w.M, kvbt.BF16 if w.is_bf16 else kvbt.F32,
                                w.T, w.H, w.topk, split=split,
                                workspace_bytes=0 if call.ws is None else call.ws.numel())
    return {
        "sec": sec, "rows_per_s": w.T / sec, "us_per_call": sec * 1e6,
        "algorithmic_bytes": ab, "policy": policy, "outputs": outputs,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 5),
                     "traffic": measured_traffic(w.name)},
    }, call


def workload_leg(torch, kvbt, w, d, steps, warmup, floor_us, cold=True, split=None):
    """One workload's record: µs per call (graph-replayed; inputs cycled through copies
    when they exceed the memory-side cache), the same with every call on its own input
    copy (`cold`), the launch floor beside both, rows/s and the roofline object. `split`
    as in FusedCall."""
    ab = algorithmic_bytes(w)
    copies = rotation_copies(ab) if ab > MALL_BYTES else 1
    res, _ = measure(torch, kvbt, w, d, steps, warmup, copies=copies, split=split)
    us = res["us_per_call"]
    leg = {"workload": w.name, "rows": w.T, "index_heads": w.H, "max_k_tiles": w.M,
           "topk": w.topk, "score_dtype": "bf16" if w.is_bf16 else "fp32",
           "inputs_sha256": inputs_sha256(w), "input_copies": copies, "steps": steps,
           "us_per_call": round(us, 3), "launch_floor_us": round(floor_us, 3),
           "us_over_floor": round(us - floor_us, 3),
           "rows_per_s": round(res["rows_per_s"], 1),
           "row_heads_per_s": round(res["rows_per_s"] * w.H, 1),
           "algorithmic_bytes_per_call": res["algorithmic_bytes"],
           "roofline": res["roofline"], "policy": res["policy"]}
    if cold and copies == 1:
        sec, n = cold_seconds(torch, kvbt, w, d, split=split)
        leg["cold"] = {"us_per_call": round(sec * 1e6, 3),
                       "us_over_floor": round(sec * 1e6 - floor_us, 3), "copies": n,
                       "achieved_GBps": round(ab / sec / 1e9, 3),
                       "frac": round(ab / sec / 1e9 / HBM_PEAK_GBPS, 5),
                       "note": "each call on its own copy of the inputs (> 512 MB in all)"}
    return leg, res["outputs"]


# ---------------------------------------------------------------------------
# the table's consumer: sparse paged-attention decode
# ---------------------------------------------------------------------------

# few-row batches timed beside the five workloads: (rows, max_k_tiles), 4 heads, fp32,
# every row at full capacity
FEW_ROWS = ((1, 8192), (8, 8192), (8, 65536))

ATTN_GROUP = 8      # query heads per index (KV) head
ATTN_SEED = 902


ATTN_LONG_ROWS = 64  # rows of the long-context decode workload the second attention run keeps
ATTN_REPLICAS = 4    # copies of the spec-decode table in the large-batch attention run
ATTN_FEW_ROWS = (16, 64)   # rows of the spec-decode table the few-rows attention runs keep


def attention_workload(wl, w, table, ctx, rows=None, replicas=1):
    """Attention inputs over a selector's table: its first `rows` rows, or the table
    repeated `replicas` times as further requests with pages of their own (page ids
    offset by one more than the largest id per copy)."""
    tag = "" if rows is None else "_r%d" % rows
    if rows is not None:
        table, ctx = table[:rows], ctx[:rows]
    if replicas > 1:
        tag += "_x%d" % replicas
        span = int(table.max()) + 1
        table = np.concatenate([table + c * span for c in range(replicas)]).astype(np.int32)
        ctx = np.concatenate([ctx] * replicas).astype(np.int32)
    return wl.attention_inputs("sparse_attn_%s%s_g%d_d128" % (w.name, tag, ATTN_GROUP), table,
                               ctx, G=ATTN_GROUP, seed=ATTN_SEED,
                               decode_query_len=w.decode_query_len)


def attn_inputs_sha256(a) -> str:
    import hashlib
    h = hashlib.sha256()
    for arr in (a.q, a.k_cache, a.v_cache, a.table, a.ctx):
        h.update(np.ascontiguousarray(arr).tobytes())
    h.update(np.float64(a.scale).tobytes())
    return h.hexdigest()


def attn_bytes(a):
    """(algorithmic, gathered) bytes of one attention call: distinct (page, KV head)
    slabs named within ctx read once, versus every row reading its own pages."""
    W = a.table.shape[2]
    c = np.clip(a.ctx.astype(np.int64), 0, 16 * W)
    npg = (c + 15) // 16                                          # [T, H]
    used = np.arange(W)[None, None, :] < npg[:, :, None]          # [T, H, W]
    pages = a.table.astype(np.int64)
    valid = used & (pages >= 0) & (pages < a.P)
    heads = np.broadcast_to(np.arange(a.H)[None, :, None], pages.shape)
    slabs = np.unique(pages[valid] * a.H + heads[valid]).shape[0]
    kv = 2 * 16 * 128 * 2                                         # K + V of one page, one head
    q_out = a.T * a.H * a.G * 128 * (2 + 4)
    meta = int(npg.sum()) * 4 + a.T * a.H * 4
    return slabs * kv + q_out + meta, int(valid.sum()) * kv + q_out + meta


class AttnCall:
    """One attention call over device copies of `a`; with `workspace`, the call with a
    zero-initialised workspace of its own (the library's split choice)."""

    def __init__(self, torch, kvbt, a, d, workspace=False):
        def bf16(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(d).view(
                torch.bfloat16)
        self.kvbt, self.a = kvbt, a
        self.q, self.k, self.v = bf16(a.q), bf16(a.k_cache), bf16(a.v_cache)
        self.table = torch.from_numpy(a.table).to(d)
        self.ctx = torch.from_numpy(a.ctx).to(d)
        self.out = torch.empty(a.q.shape, dtype=torch.float32, device=d)
        self.ws = None
        if workspace:
            n = kvbt.sparse_attn_workspace_bytes(a.T, a.H)
            self.ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=d)

    def __call__(self):
        kw = {} if self.ws is None else {"workspace": self.ws}
        self.kvbt.sparse_attn_decode(self.q, self.k, self.v, self.table, self.ctx, self.a.scale,
                                     out=self.out, decode_query_len=self.a.decode_query_len,
                                     **kw)


def measure_attention(torch, kvbt, a, d, steps, warmup, workspace=False):
    call = AttnCall(torch, kvbt, a, d, workspace)
    call()
    torch.cuda.synchronize()
    out = call.out.cpu().numpy()
    footprint = sum(t.numel() * t.element_size() for t in (call.k, call.v))
    copies = rotation_copies(footprint)
    calls = [call] + [AttnCall(torch, kvbt, a, d, workspace) for _ in range(copies - 1)]
    sec = time_graph(torch, Rotation(calls), steps, warmup)
    del calls
    ab, gathered = attn_bytes(a)
    achieved = ab / sec / 1e9
    name = a.name + ("_split" if workspace else "")
    return {
        "workload": name, "rows": a.T, "index_heads": a.H, "query_heads_per_index_head": a.G,
        "head_dim": 128, "cache_pages": a.P, "mean_ctx": round(float(a.ctx.mean()), 1),
        "decode_query_len": a.decode_query_len,
        "requests_together": kvbt.sparse_attn_grouped(a.T, a.H, a.G, a.decode_query_len),
        "splits_per_row_head": kvbt.sparse_attn_splits(a.T, a.H) if workspace else 0,
        "inputs_sha256": attn_inputs_sha256(a), "steps": steps, "input_copies": copies,
        "us_per_call": round(sec * 1e6, 3), "rows_per_s": round(a.T / sec, 1),
        "waves_per_row_head": (4 if workspace and kvbt.sparse_attn_splits(a.T, a.H)
                               else kvbt.sparse_attn_waves(a.T, a.H, a.decode_query_len)),
        "algorithmic_bytes_per_call": ab, "gathered_bytes_per_call": gathered,
        "gathered_GBps": round(gathered / sec / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 5),
                     "traffic": measured_traffic(name)},
    }, out


# ---------------------------------------------------------------------------
# the step before the selector: decode index scores
# ---------------------------------------------------------------------------

INDEX_SEED = 903


def index_workload(wl, w, requests=None, tag="", fp8=False):
    seq = w.seq_lens if requests is None else w.seq_lens[:requests]
    return wl.index_inputs("index_scores_%s%s_d128_%slse" % (w.name, tag, "fp8_" if fp8 else ""),
                           seq, w.decode_query_len, w.H, w.M, seed=INDEX_SEED,
                           max_blocks=w.max_blocks, fp8=fp8)


def index_inputs_sha256(x) -> str:
    import hashlib
    h = hashlib.sha256()
    for arr in (x.q_idx, x.k_cache, x.block_table, x.seq_lens, x.k_scale):
        if arr is not None:
            h.update(np.ascontiguousarray(arr).tobytes())
    h.update(np.array([x.decode_query_len, x.max_k_tiles], np.int64).tobytes())
    h.update(np.float64(x.scale).tobytes())
    return h.hexdigest()


def index_bytes(x) -> int:
    q = x.decode_query_len
    seq = x.seq_lens.astype(np.int64)
    mb = min(x.block_table.shape[1], x.max_k_tiles)
    tokens = np.minimum(np.maximum(seq, 0), mb * 128)
    per_key = 128 + 4 if x.k_scale is not None else 256     # FP8 codes + scale, or bf16
    keys = int(tokens.sum()) * x.H * per_key
    rows = np.arange(x.T)
    c = np.maximum(seq[rows // q] - q + rows % q + 1, 0)
    nvp = np.minimum((c + 127) // 128, mb)
    scores = int(nvp.sum()) * x.H * 4
    bt = int(((tokens + 127) // 128).sum()) * 4
    return keys + x.T * x.H * 256 + scores + bt + x.B * 4


class IndexCall:
    def __init__(self, torch, kvbt, x, d):
        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(
                torch.bfloat16)
        self.kvbt, self.x = kvbt, x
        self.q = bf16(x.q_idx)
        if x.k_scale is not None:
            self.k = torch.from_numpy(x.k_cache).to(d)
            self.ks = torch.from_numpy(x.k_scale).to(d)
        else:
            self.k, self.ks = bf16(x.k_cache), None
        self.bt = torch.from_numpy(x.block_table).to(d)
        self.seq = torch.from_numpy(x.seq_lens).to(d)
        self.scores = torch.full((x.T, x.H, x.max_k_tiles), float("-inf"), device=d)

    def __call__(self):
        self.kvbt.index_decode_scores(self.q, self.k, self.bt, self.seq, self.scores,
                                      self.x.scale, decode_query_len=self.x.decode_query_len,
                                      reduce="lse", k_scale=self.ks)


def measure_index(torch, kvbt, x, d, steps, warmup):
    call = IndexCall(torch, kvbt, x, d)
    call()
    torch.cuda.synchronize()
    out = call.scores.cpu().numpy()
    copies = rotation_copies(call.k.numel() * call.k.element_size())
    calls = [call] + [IndexCall(torch, kvbt, x, d) for _ in range(copies - 1)]
    sec = time_graph(torch, Rotation(calls), steps, warmup)
    del calls
    ab = index_bytes(x)
    achieved = ab / sec / 1e9
    return {
        "workload": x.name, "requests": x.B, "rows": x.T, "index_heads": x.H,
        "head_dim": 128, "reduce": "lse", "max_k_tiles": x.max_k_tiles,
        "key_dtype": "fp8_e4m3" if x.k_scale is not None else "bf16",
        "causal_tokens": int(np.maximum(x.seq_lens.astype(np.int64), 0).sum()),
        "inputs_sha256": index_inputs_sha256(x), "steps": steps, "input_copies": copies,
        "us_per_call": round(sec * 1e6, 3), "rows_per_s": round(x.T / sec, 1),
        "algorithmic_bytes_per_call": ab,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 5),
                     "traffic": measured_traffic(x.name)},
    }, out


# ---------------------------------------------------------------------------
# one whole decode step: index scores -> select + table -> sparse attention
# ---------------------------------------------------------------------------

class DecodeStep:
    """The three calls of a decode step on one stream, sharing one block table: the
    index-K cache and the KV cache are paged by the same 128-token physical blocks. With
    `fp8`, the index keys are FP8 E4M3 codes with per-token scales (the optional FP8
    index cache) instead of bf16."""

    def __init__(self, torch, kvbt, wl, w, d, fp8=False):
        x = index_workload(wl, w, fp8=fp8)
        self.kvbt, self.x, self.w = kvbt, x, w
        rng = np.random.Generator(np.random.PCG64(ATTN_SEED + 1))

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(
                torch.bfloat16)
        self.q_idx = bf16(x.q_idx)
        if fp8:
            self.k_idx = torch.from_numpy(x.k_cache).to(d)
            self.k_scale = torch.from_numpy(x.k_scale).to(d)
        else:
            self.k_idx, self.k_scale = bf16(x.k_cache), None
        self.bt = torch.from_numpy(x.block_table).to(d)
        self.seq = torch.from_numpy(x.seq_lens).to(d)
        self.scores = torch.full((x.T, x.H, x.max_k_tiles), float("-inf"), device=d,
                                 dtype=torch.bfloat16)
        pages = x.num_blocks * 8
        kv = wl.f32_to_bf16_bits(rng.standard_normal((2, pages, x.H, 128 * 16),
                                                     dtype=np.float32))
        self.k = bf16(kv[0]).view(pages, x.H, 16, 16, 8)
        self.v = bf16(kv[1]).view(pages, x.H, 128, 16)
        self.q = bf16(wl.f32_to_bf16_bits(rng.standard_normal((x.T, x.H * ATTN_GROUP, 128),
                                                              dtype=np.float32)))
        self.out = (torch.empty(x.T, x.H, w.topk, dtype=torch.int32, device=d),
                    torch.empty(x.T, x.H, w.topk * 8, dtype=torch.int32, device=d),
                    torch.empty(x.T, x.H, dtype=torch.int32, device=d))
        self.o = torch.empty(x.T, x.H * ATTN_GROUP, 128, dtype=torch.float32, device=d)

    def __call__(self):
        x, w, kvbt = self.x, self.w, self.kvbt
        kvbt.index_decode_scores(self.q_idx, self.k_idx, self.bt, self.seq, self.scores,
                                 x.scale, decode_query_len=x.decode_query_len, reduce="lse",
                                 k_scale=self.k_scale)
        kvbt.select_topk_and_build_table(self.scores, self.bt, seq_lens=self.seq,
                                         decode_query_len=x.decode_query_len, topk=w.topk,
                                         num_init=w.num_init, num_local=w.num_local,
                                         out=self.out)
        kvbt.sparse_attn_decode(self.q, self.k, self.v, self.out[1], self.out[2],
                                1.0 / np.sqrt(128.0), out=self.o,
                                decode_query_len=x.decode_query_len)


def measure_decode_step(torch, kvbt, wl, w, d, steps, fp8=False):
    step = DecodeStep(torch, kvbt, wl, w, d, fp8)
    step()
    torch.cuda.synchronize()
    ctx = step.out[2].cpu().numpy()
    footprint = sum(t.numel() * t.element_size() for t in (step.k_idx, step.k, step.v))
    copies = rotation_copies(footprint)
    steps_list = [step] + [DecodeStep(torch, kvbt, wl, w, d, fp8) for _ in range(copies - 1)]
    sec = time_graph(torch, Rotation(steps_list), steps, 5)
    del steps_list
    return {
        "workload": "decode_step_%s%s_g%d_d128" % (w.name, "_fp8_index" if fp8 else "",
                                                   ATTN_GROUP),
        "calls": ["index_decode_scores (lse, %s keys, bf16 scores)"
                  % ("FP8 E4M3" if fp8 else "bf16"), "select_topk_and_build_table",
                  "sparse_attn_decode (fp32 out)"],
        "rows": step.x.T, "index_heads": step.x.H, "steps": steps, "input_copies": copies,
        "us_per_step": round(sec * 1e6, 3), "rows_per_s": round(step.x.T / sec, 1),
        "mean_sparse_ctx": round(float(ctx.mean()), 1),
        "note": "one graph of the three calls per step; each call is checked against its "
                "oracle by the tests and the other legs, the chain is not (the selection "
                "depends on the scores' last bits)",
    }


# ---------------------------------------------------------------------------
# the cpu-baseline leg: the only user of the oracle here
# ---------------------------------------------------------------------------

def host_cpu():
    """The host's CPU model and counts (logical CPUs, and those this process may use)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count() or 1,
            "usable_cpus": usable}


def oracle_rate(orc, w, threads, budget_s, rows=None):
    """Rows per second of the oracle's fused call on `w` (or on the listed rows), repeated
    for about `budget_s` seconds with `threads` host threads."""
    reps, t0 = 0, time.perf_counter()
    n = w.T if rows is None else len(rows)
    while True:
        orc.select_topk_and_build_table(w.scores, w.block_table, topk=w.topk,
                                        num_init=w.num_init, num_local=w.num_local,
                                        threads=threads, rows=rows, **w.row_kwargs())
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    what = "%d rows" % n if rows is None else "%d sampled rows" % n
    return {"value": round(n * reps / el, 1), "unit": "rows/s", "threads": threads,
            "sample": "%s: %s x %d heads, %d passes in %.2f s" % (w.name, what, w.H, reps, el)}


def cpu_leg(w, gpu_outputs, threads, budget_s, long_check=None, attn_check=None,
            index_checks=(), legs=(), leg_seconds=1.5):
    """Times the oracle on a bounded sample and checks the GPU results seen against it.

    long_check: (workload, gpu outputs, rows) of the long-context run. attn_check: a list
    of (SHA-256 of the attention inputs the GPU ran on, gpu output, rows, replicas, rows
    kept or None) over the default workload's table; the oracle rebuilds those inputs
    from its own sparse table and must arrive at the same bytes.
    index_checks: (inputs, gpu scores, requests to check) of the index-score runs.
    Returns (cpu_baseline, checks)."""
    import oracle
    from kv_block_top_amd import workloads as wl
    from oracle import index_scores, sparse_attn
    orc = oracle.default()
    checks = {}

    def compare(wk, got, rows):
        want = orc.select_topk_and_build_table(wk.scores, wk.block_table, topk=wk.topk,
                                               num_init=wk.num_init, num_local=wk.num_local,
                                               threads=threads, rows=rows, **wk.row_kwargs())
        sel = slice(None) if rows is None else np.asarray(rows)
        for name, g, e in zip(("idx", "table", "ctx"), got, want):
            if not np.array_equal(g[sel], e[sel]):
                raise SystemExit("bench: GPU %s differs from the oracle on %s" % (name, wk.name))
        return want

    _, table, ctx = compare(w, gpu_outputs, None)
    checks["verified_rows"] = w.T
    if long_check is not None:
        compare(*long_check)
        checks["long_context_verified_rows"] = len(long_check[2])
    # every other timed workload: its GPU outputs against the oracle's (all rows, or a
    # sample of a large one), then the oracle's own rate on all threads and on one
    for wk, got, rows, leg in legs:
        if wk.name != w.name and (long_check is None or wk.name != long_check[0].name):
            compare(wk, got, rows)
        checks[wk.name + "_verified_rows"] = wk.T if rows is None else len(rows)
        leg["cpu_oracle"] = {"all_threads": oracle_rate(orc, wk, threads, leg_seconds, rows),
                             "one_thread": oracle_rate(orc, wk, 1, leg_seconds, rows)}
    for sha, got, rows, replicas, kept in attn_check or ():
        a = attention_workload(wl, w, table, ctx, rows=kept, replicas=replicas)
        if attn_inputs_sha256(a) != sha:
            raise SystemExit("bench: attention inputs rebuilt from the oracle's table differ")
        rows = np.asarray(rows)
        want, spread, vmax = sparse_attn.sparse_attn_decode(
            a.q[rows], a.k_cache, a.v_cache, a.table[rows], a.ctx[rows], a.scale,
            with_spread=True)
        tol = 2.0 ** -7 * spread + 2.0 ** -12 * np.repeat(vmax, a.G, axis=1)[:, :, None]
        err = np.abs(got[rows].astype(np.float64) - want)
        if not (err <= tol).all():
            raise SystemExit("bench: GPU attention outside the error bound on %s" % a.name)
        key = "attention" if replicas == 1 else "attention_x%d" % replicas
        key += "" if kept is None else "_r%d_split" % kept
        checks[key + "_verified_rows"] = int(len(rows))
        checks[key + "_max_err_over_bound"] = round(
            float((err / np.maximum(tol, 1e-300)).max()), 4)
        del a
    for x, got, reqs in index_checks:
        q = x.decode_query_len
        worst = 0.0
        for r in reqs:
            rows = slice(r * q, (r + 1) * q)
            init = np.full((q, x.H, x.max_k_tiles), -np.inf)
            want, bound = index_scores.index_decode_scores(
                x.q_idx[rows], x.k_cache, x.block_table[r: r + 1], x.seq_lens[r: r + 1], q,
                x.scale, "lse", init, with_bound=True, k_scale=x.k_scale)
            g = got[rows].astype(np.float64)
            wrote = np.isfinite(want)
            if not np.array_equal(np.isfinite(g), wrote):
                raise SystemExit("bench: index scores written to other entries on %s" % x.name)
            tol = 2.0 ** -16 * bound[wrote] + 2.0 ** -14 + 2.0 ** -20 * np.abs(want[wrote])
            err = np.abs(g[wrote] - want[wrote])
            if not (err <= tol).all():
                raise SystemExit("bench: index scores outside the error bound on %s" % x.name)
            worst = max(worst, float((err / tol).max()) if err.size else 0.0)
        checks[x.name + "_verified_requests"] = len(reqs)
        checks[x.name + "_max_err_over_bound"] = round(worst, 4)

    main = oracle_rate(orc, w, threads, budget_s)
    one = oracle_rate(orc, w, 1, max(1.0, budget_s / 4))
    base = {"value": main["value"], "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": main["sample"], "one_core": {"value": one["value"],
                                                   "sample": one["sample"]}}
    base.update(host_cpu())
    base["note"] = ("cores = host threads the oracle ran on: all usable CPUs, at most 16 "
                    "(one GPU's share of its host)")
    return base, checks


def cold_seconds(torch, kvbt, w, d, total_bytes=640 << 20, max_copies=2048, split=None):
    """Seconds per call when every call reads inputs no earlier call touched: one graph
    replay over enough independent copies of the workload (inputs and outputs) to
    exceed the 256 MB MALL and every L2, so each call's inputs come from HBM."""
    per = w.scores.nbytes + w.block_table.nbytes + w.T * w.H * (w.topk * 9 + 1) * 4 + 4096
    n = int(min(max_copies, max(2, total_bytes // per)))
    calls = [FusedCall(torch, kvbt, w, d, split) for _ in range(n)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls[0]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    sec = start.elapsed_time(stop) * 1e-3 / n
    del g, calls
    return sec, n


def launch_floor(torch, kvbt, steps):
    return time_graph(torch, lambda: kvbt.bench_empty(1), steps, 5) * 1e6


def read_bandwidth(torch, kvbt, d, nbytes=1 << 30, reps=10):
    """GB/s of the library's read-only stream over `nbytes` (no writes)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=d)
    sink = torch.zeros(4, dtype=torch.int32, device=d)
    for _ in range(2):
        kvbt.bench_read(src, nbytes, sink)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        kvbt.bench_read(src, nbytes, sink)
    stop.record()
    torch.cuda.synchronize()
    sec = start.elapsed_time(stop) * 1e-3 / reps
    del src
    return nbytes / sec / 1e9


def copy_bandwidth(torch, kvbt, d, nbytes=1 << 30):
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=d).fill_(1.0)
    dst = torch.empty_like(src)
    sec = time_graph(torch, lambda: kvbt.bench_copy(dst, src, nbytes), 10, 3)
    return 2 * nbytes / sec / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--long-steps", type=int, default=50)
    ap.add_argument("--attn-steps", type=int, default=50)
    ap.add_argument("--no-long", action="store_true",
                    help="skip the per-workload legs (configs 1-5 and the few-row batches)")
    ap.add_argument("--no-attn", action="store_true", help="skip the sparse-attention leg")
    ap.add_argument("--no-index", action="store_true", help="skip the index-score legs")
    ap.add_argument("--index-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the cpu-baseline leg (oracle timing and result checks)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="only run the timed calls (for profilers); print nothing else")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported "
              "(every (row, head) is independent, so more GPUs would each run their own "
              "share with no exchange)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_block_top_amd as kvbt
    from kv_block_top_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    kvbt.lib()
    d = torch.device("cuda:0")
    # the oracle's host threads: every usable CPU, at most one GPU's share of the host (16)
    threads = max(1, min(16, host_cpu()["usable_cpus"]))

    w = wl.config(args.workload)
    if args.profile_only:
        # eager calls only (profilers see one dispatch per call), then a 256 MiB copy
        # whose HBM counter readings scale the kernels'
        work = [(w, args.steps)]
        if not args.no_long:
            work += [(wl.config(n), args.long_steps if n == 5 else args.steps)
                     for n in (1, 2, 3, 4, 5) if n != args.workload]
            work += [(wl.few_rows(n_rows, M), args.steps) for n_rows, M in FEW_ROWS]
            work += [((wl.few_rows(n_rows, M), kvbt.SPLIT_AUTO), args.steps)
                     for n_rows, M in FEW_ROWS]
        for wk, n in work:
            wk, split = wk if isinstance(wk, tuple) else (wk, None)
            call = FusedCall(torch, kvbt, wk, d, split)
            for _ in range(n):
                call()
            torch.cuda.synchronize()
            print("profiled %s x %d" % (wk.name, n), flush=True)
            if wk is w and not args.no_attn:
                _, table, ctx = call.outputs()
                for reps in (1, ATTN_REPLICAS):
                    a = attention_workload(wl, w, table, ctx, replicas=reps)
                    acall = AttnCall(torch, kvbt, a, d)
                    for _ in range(args.attn_steps):
                        acall()
                    torch.cuda.synchronize()
                    print("profiled %s x %d" % (a.name, args.attn_steps), flush=True)
                    del acall, a
            if wk is w and not args.no_attn:
                w4 = wl.config(4)
                c4 = FusedCall(torch, kvbt, w4, d)
                c4()
                torch.cuda.synchronize()
                _, t4, x4 = c4.outputs()
                del c4
                a = attention_workload(wl, w4, t4, x4, ATTN_LONG_ROWS)
                acall = AttnCall(torch, kvbt, a, d)
                for _ in range(args.attn_steps):
                    acall()
                torch.cuda.synchronize()
                print("profiled %s x %d" % (a.name, args.attn_steps), flush=True)
                del acall, a, w4
                for rows in ATTN_FEW_ROWS:
                    a = attention_workload(wl, w, table, ctx, rows=rows)
                    for ws in (False, True):
                        acall = AttnCall(torch, kvbt, a, d, ws)
                        for _ in range(args.attn_steps):
                            acall()
                        torch.cuda.synchronize()
                        print("profiled %s%s x %d" % (a.name, "_split" if ws else "",
                                                      args.attn_steps), flush=True)
                        del acall
                    del a
            if wk is w and not args.no_index:
                for x in (index_workload(wl, w), index_workload(wl, wl.config(4), 8, "_r8"),
                          index_workload(wl, wl.config(4), 8, "_r8", fp8=True)):
                    icall = IndexCall(torch, kvbt, x, d)
                    for _ in range(args.index_steps):
                        icall()
                    torch.cuda.synchronize()
                    print("profiled %s x %d" % (x.name, args.index_steps), flush=True)
                    del icall, x
            del call
        nb = 256 << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=d)
        dst = torch.empty_like(src)
        for _ in range(3):
            kvbt.bench_copy(dst, src, nb)
        torch.cuda.synchronize()
        print("profiled copy 256 MiB x 3", flush=True)
        return
    # a workload larger than the memory-side cache cycles through input copies (see the
    # long-context leg); the small ones are timed warm, as a serving step reads scores
    # just written, and cold below
    floor_us = launch_floor(torch, kvbt, args.steps)
    ab_main = algorithmic_bytes(w)
    res, _ = measure(torch, kvbt, w, d, args.steps, args.warmup,
                     copies=rotation_copies(ab_main) if ab_main > MALL_BYTES else 1)

    line = {
        "metric": "selector+table rows/s, us/call at 74 blocks, achieved HBM GB/s vs peak",
        "value": round(res["rows_per_s"], 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["sec"] * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32" if w.is_bf16 else "u64",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.T, "index_heads": w.H, "max_k_tiles": w.M,
                   "topk": w.topk, "query_len": w.decode_query_len,
                   "score_dtype": "bf16" if w.is_bf16 else "fp32", "call": "fused",
                   "inputs_sha256": inputs_sha256(w)},
        "us_per_call": round(res["us_per_call"], 3),
        "roofline": res["roofline"],
        "algorithmic_bytes_per_call": res["algorithmic_bytes"],
        "policy": res["policy"],
    }
    line["launch_floor_us"] = round(floor_us, 3)
    line["us_over_floor"] = round(res["us_per_call"] - floor_us, 3)
    cold, ncopies = cold_seconds(torch, kvbt, w, d)
    line["cold"] = {"us_per_call": round(cold * 1e6, 3),
                    "us_over_floor": round(cold * 1e6 - floor_us, 3), "copies": ncopies,
                    "note": "each call on its own copy of the inputs (> 512 MB in all)"}

    # every workload on its own: configs 1-5 (the default one is re-timed inside its leg
    # with the same method) and a handful of rows at the fast path's and the largest
    # capacity, each with the launch floor beside its time
    legs = []            # (workload, gpu outputs, rows checked (None = all), leg dict)
    line["configs"] = {}
    outputs4 = None
    if not args.no_long:
        for n in (1, 2, 3, 4, 5):
            wk = wl.config(n)
            steps_n = args.long_steps if n == 5 else args.steps
            leg, out = workload_leg(torch, kvbt, wk, d, steps_n, 3 if n == 5 else args.warmup,
                                    floor_us)
            line["configs"][wk.name] = leg
            _progress("%s %.3f us per call" % (wk.name, leg["us_per_call"]))
            legs.append((wk, out, _sample_rows(wk) if n == 5 else None, leg))
            if n == 4:
                outputs4 = (wk, out)
            del wk
        # few rows: the library's choice with a workspace (the cross-workgroup split
        # where it takes it), without one (the paths that need no workspace), and the
        # split forced
        line["few_rows"] = {}
        for n_rows, M in FEW_ROWS:
            wk = wl.few_rows(n_rows, M)
            leg, out = workload_leg(torch, kvbt, wk, d, args.steps, args.warmup, floor_us,
                                    split=kvbt.SPLIT_AUTO)
            plain, out_plain = workload_leg(torch, kvbt, wk, d, args.steps, args.warmup,
                                            floor_us)
            forced, out_forced = workload_leg(torch, kvbt, wk, d, args.steps, args.warmup,
                                              floor_us, split=kvbt.SPLIT_ALWAYS)
            for o in (out_plain, out_forced):
                if not all(np.array_equal(a, b) for a, b in zip(out, o)):
                    raise SystemExit("bench: %s differs between launch paths" % wk.name)
            keep = ("us_per_call", "us_over_floor", "cold", "policy")
            leg["without_workspace"] = {k: plain[k] for k in keep}
            leg["split_across_workgroups"] = {k: forced[k] for k in keep}
            line["few_rows"][wk.name] = leg
            _progress("%s %.3f us per call (%.3f without a workspace, %.3f split across "
                      "workgroups)" % (wk.name, leg["us_per_call"], plain["us_per_call"],
                                       forced["us_per_call"]))
            legs.append((wk, out, None, leg))
            del wk
    long_check = None
    if legs:
        w5, out5, rows5, leg5 = legs[4]
        line["long_context"] = dict(leg5, num_decode_rows=w5.num_decode_rows)
        long_check = (w5, out5, rows5)
    attn_check = []
    if not args.no_attn:
        _, table, ctx = res["outputs"]
        a = attention_workload(wl, w, table, ctx)
        ra, out_a = measure_attention(torch, kvbt, a, d, args.attn_steps, 5)
        line["sparse_attention"] = ra
        attn_check.append((ra["inputs_sha256"], out_a, _sample_rows(a, 32), 1, None))
        del a
        a = attention_workload(wl, w, table, ctx, replicas=ATTN_REPLICAS)
        ra, out_a = measure_attention(torch, kvbt, a, d, args.attn_steps, 5)
        line["sparse_attention_large_batch"] = ra
        attn_check.append((ra["inputs_sha256"], out_a, _sample_rows(a, 32), ATTN_REPLICAS, None))
        del a
        if outputs4 is None:
            w4 = wl.config(4)
            r4, _ = measure(torch, kvbt, w4, d, 20, 3)
            outputs4 = (w4, r4["outputs"])
            del r4
        w4, (_, t4, x4) = outputs4
        a4 = attention_workload(wl, w4, t4, x4, ATTN_LONG_ROWS)
        ra4, _ = measure_attention(torch, kvbt, a4, d, args.attn_steps, 5)
        line["sparse_attention_long"] = ra4
        del a4, w4
        few = []
        for rows in ATTN_FEW_ROWS:
            a = attention_workload(wl, w, table, ctx, rows=rows)
            plain, _ = measure_attention(torch, kvbt, a, d, args.attn_steps, 5)
            rs, out_s = measure_attention(torch, kvbt, a, d, args.attn_steps, 5, workspace=True)
            rs["without_workspace_us_per_call"] = plain["us_per_call"]
            rs["without_workspace_roofline_frac"] = plain["roofline"]["frac"]
            few.append(rs)
            attn_check.append((rs["inputs_sha256"], out_s, _sample_rows(a, 16), 1, rows))
            _progress("%s %.3f us per call with a workspace (%d workgroups per row and head), "
                      "%.3f without" % (a.name, rs["us_per_call"], rs["splits_per_row_head"],
                                        plain["us_per_call"]))
            del a
        line["sparse_attention_few_rows"] = few
        _progress("sparse attention legs done")
    index_checks = []
    if not args.no_index:
        for key, x in (("index_scores", index_workload(wl, w)),
                       ("index_scores_long", index_workload(wl, wl.config(4), 8, "_r8")),
                       ("index_scores_long_fp8",
                        index_workload(wl, wl.config(4), 8, "_r8", fp8=True))):
            ri, out_i = measure_index(torch, kvbt, x, d, args.index_steps, 5)
            line[key] = ri
            reqs = sorted(set(np.linspace(0, x.B - 1, min(x.B, 6)).astype(int).tolist()))
            index_checks.append((x, out_i, reqs))
            del x
        _progress("index-score legs done")
    if not (args.no_index or args.no_attn):
        line["decode_step"] = measure_decode_step(torch, kvbt, wl, w, d, args.attn_steps)
        line["decode_step_fp8_index"] = measure_decode_step(torch, kvbt, wl, w, d,
                                                            args.attn_steps, fp8=True)
    line["copy_GBps"] = round(copy_bandwidth(torch, kvbt, d), 1)
    line["read_stream_GBps"] = round(read_bandwidth(torch, kvbt, d), 1)
    if not args.no_cpu:
        _progress("cpu baseline and oracle checks")
        base, checks = cpu_leg(w, res["outputs"], threads, args.cpu_seconds, long_check,
                               attn_check, index_checks, legs)
        line["cpu_baseline"] = base
        line["checked_against_oracle"] = checks
    print(json.dumps(line))


def _progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the JSON line)."""
    print("bench: " + msg, file=sys.stderr, flush=True)


def _sample_rows(w, n=512):
    rng = np.random.default_rng(123)
    rows = set(rng.choice(w.T, size=min(n, w.T), replace=False).tolist())
    rows |= {0, 1, 2, 3, w.T - 1, w.T - 2}
    return sorted(rows)


if __name__ == "__main__":
    main()
