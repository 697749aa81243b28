"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no part of the selector or the table build. It draws scores,
sequence lengths and block tables, and fills in the per-row metadata a serving
engine's metadata builder would hand to the selector (causal page counts, row
request ids and positions, the ``-inf`` fill of unwritten tiles). Both the HIP
path and the CPU oracle take their inputs from here, so neither can feed the
other.

Score arrays are numpy ``float32`` or ``uint16`` bf16 bit patterns (rounded to
nearest-even from fp32 once), shape ``[T, H, max_k_tiles]``, token-major.

The five named workloads (``config(1)`` .. ``config(5)``) follow these recipes:

1. tiny: 4 decode requests (query length 1), seq_lens U[1, 2048], 16 tiles, 1 head,
   fp32 N(0, 1); block table [4, 16] of distinct ids in [0, 4096).
2. short-context spec decode: 64 requests x query length 4 (256 rows), 2 heads,
   74 tiles, bf16 N(0, 1). Requests 0-7 hold exactly 15/16/17/63/64/65/73/74 full
   blocks, request 8 has seq_len 0 (padded rows), the rest U[1, 9472].
3. boundary and special values: 256 decode rows, 4 heads, 129 tiles, bf16.
   Rows 0-11 sit at the 126..129-block boundaries and at 1/128/129 tokens.
   Each in-range tile is independently NaN, +Inf, -Inf, +0 or -0 with 1% each,
   or (5%) a copy of another in-range tile of the same row and head; tiles 64 and
   128 always hold a special value, cycling row by row.
4. long-context decode: 128 rows, 4 heads, 512 tiles, seq_lens U[32768, 65536],
   bf16 of N(0, 1) plus a per-request sum of three sinusoids over the block id
   (periods U[64, 1024] blocks, phases U[0, 2pi), amplitude 2/3 each).
5. mixed unified buffer: 32 decode requests x query length 4 (rows 0-127), then
   4 prefill requests of 2048 tokens with prefixes 0, 262144, 786432 and 1046528
   (rows 128-8319); 4 heads; 8192 tiles (1M tokens); fp32 N(0, 1).

Randomness: ``numpy.random.Generator(PCG64(seed))`` with the config number as the
seed, drawn in a fixed order.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK_TOKENS = 128

# bf16 bit patterns of the special values the boundary workload injects
BF16_QNAN = 0x7FC0
BF16_PINF = 0x7F80
BF16_NINF = 0xFF80
BF16_PZERO = 0x0000
BF16_NZERO = 0x8000
F32_NINF_BITS = 0xFF800000


@dataclasses.dataclass
class Workload:
    name: str
    scores: np.ndarray                  # [T, H, M] float32, or uint16 bf16 bits
    block_table: np.ndarray             # [B, max_blocks] int32
    num_valid_pages: np.ndarray         # [T] int32, input of the standalone selector
    seq_lens: Optional[np.ndarray]      # [B] int32 (decode form) or None
    decode_query_len: int               # q of the decode form (1 when explicit)
    row_req: Optional[np.ndarray] = None   # [T] int32 (explicit form) or None
    row_pos: Optional[np.ndarray] = None   # [T] int32 (explicit form) or None
    topk: int = 16
    num_init: int = 1
    num_local: int = 2
    max_block: int = 0                  # launch hint; 0 means max_k_tiles
    num_decode_rows: int = 0            # launch hint: decode rows at the head of the buffer

    @property
    def T(self) -> int:
        return int(self.scores.shape[0])

    @property
    def H(self) -> int:
        return int(self.scores.shape[1])

    @property
    def M(self) -> int:
        return int(self.scores.shape[2])

    @property
    def B(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def is_bf16(self) -> bool:
        return self.scores.dtype == np.uint16

    @property
    def explicit(self) -> bool:
        return self.row_req is not None

    def row_kwargs(self) -> dict:
        """Row description in the keyword form both the oracle and the binding take."""
        if self.explicit:
            return dict(row_req=self.row_req, row_pos=self.row_pos)
        return dict(seq_lens=self.seq_lens, decode_query_len=self.decode_query_len)


# ---------------------------------------------------------------------------
# helpers (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # no finite pattern carries past bit 31 (NaNs, which may, are set below)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def decode_positions(seq_lens: np.ndarray, q: int) -> tuple[np.ndarray, np.ndarray]:
    """Request id and absolute position of every row of a request-major decode batch."""
    B = seq_lens.shape[0]
    rows = np.arange(B * q, dtype=np.int64)
    req = rows // q
    pos = seq_lens.astype(np.int64)[req] - q + (rows - req * q)
    return req, pos


def causal_pages(pos: np.ndarray) -> np.ndarray:
    """Causal page count a metadata builder stores per row: cdiv(pos + 1, 128), >= 0."""
    c = np.maximum(pos.astype(np.int64) + 1, 0)
    return (c + BLOCK_TOKENS - 1) // BLOCK_TOKENS


def _fill_tail(scores: np.ndarray, written: np.ndarray) -> None:
    """Set tiles at or past each row's written count to -inf (the unwritten tail)."""
    M = scores.shape[2]
    tail = np.arange(M)[None, :] >= np.minimum(written, M)[:, None]   # [T, M]
    if scores.dtype == np.uint16:
        scores[np.broadcast_to(tail[:, None, :], scores.shape)] = BF16_NINF
    else:
        scores[np.broadcast_to(tail[:, None, :], scores.shape)] = -np.inf


def _block_table(rng, B: int, max_blocks: int, id_space: int, used: np.ndarray) -> np.ndarray:
    """Distinct physical ids from a seeded permutation; entries past ``used`` are 0."""
    ids = rng.permutation(id_space)[: B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    cols = np.arange(max_blocks)[None, :]
    ids[cols >= np.minimum(used, max_blocks)[:, None]] = 0
    return ids


def _normal_scores(rng, T: int, H: int, M: int) -> np.ndarray:
    return rng.standard_normal((T, H, M), dtype=np.float32)


def _decode_workload(name, rng, seq_lens, q, H, M, max_blocks, id_space, bf16,
                     scores_f32=None, topk=16) -> Workload:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    T = B * q
    _, pos = decode_positions(seq_lens, q)
    nvp = causal_pages(pos)
    used = (seq_lens.astype(np.int64) + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    bt = _block_table(rng, B, max_blocks, id_space, used)
    if scores_f32 is None:
        scores_f32 = _normal_scores(rng, T, H, M)
    scores = f32_to_bf16_bits(scores_f32) if bf16 else scores_f32
    _fill_tail(scores, nvp)
    return Workload(name=name, scores=scores, block_table=bt,
                    num_valid_pages=nvp.astype(np.int32), seq_lens=seq_lens,
                    decode_query_len=q, topk=topk, max_block=0)


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def config1() -> Workload:
    rng = np.random.Generator(np.random.PCG64(1))
    seq_lens = rng.integers(1, 2048, size=4, endpoint=True)
    return _decode_workload("tiny_decode_b4_t16_h1_f32", rng, seq_lens, q=1, H=1, M=16,
                            max_blocks=16, id_space=4096, bf16=False)


def config2() -> Workload:
    rng = np.random.Generator(np.random.PCG64(2))
    B, q = 64, 4
    seq_lens = np.empty(B, dtype=np.int64)
    seq_lens[:8] = BLOCK_TOKENS * np.array([15, 16, 17, 63, 64, 65, 73, 74])
    seq_lens[8] = 0
    seq_lens[9:] = rng.integers(1, 9472, size=B - 9, endpoint=True)
    return _decode_workload("spec_decode_b64_q4_t74_h2_bf16", rng, seq_lens, q=q, H=2,
                            M=74, max_blocks=74, id_space=1 << 16, bf16=True)


def _inject_specials(rng, scores: np.ndarray, written: np.ndarray) -> None:
    """Boundary-workload specials on bf16 bits, in place (see the module docstring)."""
    T, H, M = scores.shape
    specials = np.array([BF16_QNAN, BF16_PINF, BF16_NINF, BF16_PZERO, BF16_NZERO],
                        dtype=np.uint16)
    u = rng.random((T, H, M))
    src = rng.random((T, H, M))
    for t in range(T):
        nw = int(min(written[t], M))
        if nw == 0:
            continue
        for h in range(H):
            row = scores[t, h]
            for b in range(nw):
                x = u[t, h, b]
                if x < 0.05:
                    row[b] = specials[int(x / 0.01)]
                elif x < 0.10:
                    row[b] = row[int(src[t, h, b] * nw)]
            for j, b in enumerate((64, 128)):
                if b < nw:
                    k = (t + j) % 6
                    row[b] = specials[k] if k < 5 else row[0]


def config3() -> Workload:
    rng = np.random.Generator(np.random.PCG64(3))
    B = 256
    fixed = [128 * 126 + 1, 128 * 127 - 1, 128 * 127, 128 * 127 + 1, 128 * 128 - 1,
             128 * 128, 128 * 128 + 1, 128 * 129 - 1, 128 * 129, 1, 128, 129]
    seq_lens = np.empty(B, dtype=np.int64)
    seq_lens[: len(fixed)] = fixed
    seq_lens[len(fixed):] = rng.integers(1, 128 * 129, size=B - len(fixed), endpoint=True)
    w = _decode_workload("boundary_specials_b256_t129_h4_bf16", rng, seq_lens, q=1, H=4,
                         M=129, max_blocks=129, id_space=1 << 17, bf16=True)
    _inject_specials(rng, w.scores, w.num_valid_pages)
    return w


def config4() -> Workload:
    rng = np.random.Generator(np.random.PCG64(4))
    B, H, M = 128, 4, 512
    seq_lens = rng.integers(32768, 65536, size=B, endpoint=True)
    periods = rng.uniform(64.0, 1024.0, size=(B, 3))
    phases = rng.uniform(0.0, 2.0 * np.pi, size=(B, 3))
    blocks = np.arange(M, dtype=np.float64)
    bias = ((2.0 / 3.0) * np.sin(2.0 * np.pi * blocks[None, None, :] / periods[:, :, None]
                                 + phases[:, :, None])).sum(axis=1)        # [B, M]
    noise = _normal_scores(rng, B, H, M)
    scores = (noise.astype(np.float64) + bias[:, None, :]).astype(np.float32)
    return _decode_workload("long_decode_b128_t512_h4_bf16", rng, seq_lens, q=1, H=H, M=M,
                            max_blocks=M, id_space=1 << 17, bf16=True, scores_f32=scores)


def config5(max_k_tiles: int = 8192, prefill_len: int = 2048) -> Workload:
    rng = np.random.Generator(np.random.PCG64(5))
    H, M = 4, max_k_tiles
    full = M * BLOCK_TOKENS
    nd_req, q = 32, 4
    dec_seq = np.empty(nd_req, dtype=np.int64)
    dec_seq[0] = full
    dec_seq[1] = 1
    dec_seq[2:] = rng.integers(1, full, size=nd_req - 2, endpoint=True)
    prefix = np.array([0, full // 4, 3 * full // 4, full - prefill_len], dtype=np.int64)
    n_pre = prefix.shape[0]
    dec_req, dec_pos = decode_positions(dec_seq, q)
    pre_rows = np.arange(prefill_len, dtype=np.int64)
    pre_req = np.repeat(np.arange(n_pre, dtype=np.int64) + nd_req, prefill_len)
    pre_pos = (prefix[:, None] + pre_rows[None, :]).reshape(-1)
    row_req = np.concatenate([dec_req, pre_req]).astype(np.int32)
    row_pos = np.concatenate([dec_pos, pre_pos]).astype(np.int32)
    T = row_req.shape[0]
    nvp = causal_pages(row_pos)
    req_len = np.concatenate([dec_seq, prefix + prefill_len])
    used = (req_len + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    bt = _block_table(rng, nd_req + n_pre, M, 1 << 19, used)
    scores = _normal_scores(rng, T, H, M)
    _fill_tail(scores, nvp)
    return Workload(name="mixed_unified_t%d_h4_tiles%d_f32" % (T, M), scores=scores,
                    block_table=bt, num_valid_pages=nvp.astype(np.int32), seq_lens=None,
                    decode_query_len=1, row_req=row_req, row_pos=row_pos, max_block=0,
                    num_decode_rows=nd_req * q)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def few_rows(n_rows: int, M: int, *, H: int = 4, bf16: bool = False, seed: int = 6) -> Workload:
    """A handful of decode rows (q = 1) at the full capacity of M tiles each (128 M
    tokens of context): the batch shape where (row, head) pairs are far fewer than the
    chip's 256 compute units. fp32 (or bf16) N(0, 1) scores; distinct physical ids."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.full(n_rows, BLOCK_TOKENS * M, dtype=np.int64)
    return _decode_workload("few_rows_r%d_h%d_tiles%d_%s" % (n_rows, H, M,
                                                             "bf16" if bf16 else "f32"),
                            rng, seq_lens, q=1, H=H, M=M, max_blocks=M,
                            id_space=max(1 << 16, 2 * n_rows * M), bf16=bf16)


def config(n: int) -> Workload:
    return CONFIGS[n]()


# ---------------------------------------------------------------------------
# small random cases for the edge sweeps
# ---------------------------------------------------------------------------

def random_case(seed: int, *, T: int = 8, H: int = 2, M: int = 40, bf16: bool = False,
                q: int = 1, seq_lo: int = 0, seq_hi: Optional[int] = None,
                special_frac: float = 0.0, tie_frac: float = 0.0, topk: int = 16,
                num_init: int = 1, num_local: int = 2, max_blocks: Optional[int] = None,
                explicit: bool = False, tail: str = "neginf") -> Workload:
    """A small seeded workload; T must be a multiple of q in decode form.

    ``tail`` chooses the content of tiles past each row's causal count: "neginf"
    (the engine's fill), "nan" or "random" (results must not depend on it).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if seq_hi is None:
        seq_hi = M * BLOCK_TOKENS
    if max_blocks is None:
        max_blocks = M
    if explicit:
        B = max(1, T // 2)
        row_req = rng.integers(0, B, size=T).astype(np.int32)
        row_pos = rng.integers(seq_lo - 1, seq_hi, size=T).astype(np.int32)
        pos = row_pos.astype(np.int64)
        req_len = np.zeros(B, dtype=np.int64)
        np.maximum.at(req_len, row_req, pos + 1)
        seq_lens = None
    else:
        assert T % q == 0
        B = T // q
        seq_lens = rng.integers(seq_lo, seq_hi, size=B, endpoint=True).astype(np.int32)
        _, pos = decode_positions(seq_lens, q)
        req_len = seq_lens.astype(np.int64)
        row_req = row_pos = None
    nvp = causal_pages(pos)
    used = (req_len + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    bt = _block_table(rng, B, max_blocks, max(1 << 16, 2 * B * max_blocks), used)
    f = rng.standard_normal((T, H, M), dtype=np.float32)
    scores = f32_to_bf16_bits(f) if bf16 else f
    if special_frac > 0 or tie_frac > 0:
        u = rng.random((T, H, M))
        src = rng.integers(0, M, size=(T, H, M))
        if bf16:
            sp = np.array([BF16_QNAN, BF16_PINF, BF16_NINF, BF16_PZERO, BF16_NZERO,
                           0xFFC0, 0x7F81], dtype=np.uint16)
            flat = scores
        else:
            sp = np.array([0x7FC00000, 0x7F800000, 0xFF800000, 0x0, 0x80000000,
                           0xFFC00000, 0x7F800001], dtype=np.uint32)
            flat = scores.view(np.uint32)
        kind = np.minimum((u / max(special_frac, 1e-12) * len(sp)).astype(np.int64),
                          len(sp) - 1)
        is_sp = u < special_frac
        flat[is_sp] = sp[kind[is_sp]]
        is_tie = (u >= special_frac) & (u < special_frac + tie_frac)
        tt, hh, bb = np.nonzero(is_tie)
        flat[tt, hh, bb] = flat[tt, hh, np.minimum(src[tt, hh, bb], bb)]
    if tail == "neginf":
        _fill_tail(scores, nvp)
    elif tail == "nan":
        M_ = scores.shape[2]
        mask = np.arange(M_)[None, :] >= np.minimum(nvp, M_)[:, None]
        m3 = np.broadcast_to(mask[:, None, :], scores.shape)
        if bf16:
            scores[m3] = BF16_QNAN
        else:
            scores.view(np.uint32)[m3] = 0x7FC00000
    elif tail != "random":
        raise ValueError(tail)
    return Workload(name="random_%d" % seed, scores=scores, block_table=bt,
                    num_valid_pages=nvp.astype(np.int32), seq_lens=seq_lens,
                    decode_query_len=q if not explicit else 1, row_req=row_req,
                    row_pos=row_pos, topk=topk, num_init=num_init, num_local=num_local)


def rows_case(seed: int, causal_lens, *, H: int = 2, M: int = 8192, bf16: bool = False,
              kind: str = "normal", topk: int = 16, num_init: int = 1, num_local: int = 2,
              max_blocks: Optional[int] = None, tail: str = "neginf") -> Workload:
    """One request per row with the given causal lengths (explicit row form).

    ``kind`` shapes the in-range scores: "normal" N(0, 1); "specials" N(0, 1) with 5%
    each of the special values and 10% copies of other tiles; "ties" one value;
    "negative" -|N(0, 1)|; "neginf" all -inf; "nan" all +NaN; "increasing" sorted
    ascending along the row; "two_level" mostly one value with 0.5% larger ones.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    c = np.asarray(causal_lens, dtype=np.int64)
    T = c.shape[0]
    if max_blocks is None:
        max_blocks = M
    row_req = np.arange(T, dtype=np.int32)
    row_pos = (c - 1).astype(np.int32)
    nvp = causal_pages(c - 1)
    used = nvp
    bt = _block_table(rng, T, max_blocks, max(1 << 16, 2 * T * max_blocks), used)
    x = rng.standard_normal((T, H, M), dtype=np.float32)
    if kind == "negative":
        x = -np.abs(x)
    elif kind == "ties":
        x[:] = np.float32(0.75)
    elif kind == "neginf":
        x[:] = -np.inf
    elif kind == "nan":
        x[:] = np.nan
    elif kind == "increasing":
        x = np.sort(x, axis=2)
    elif kind == "two_level":
        x[:] = np.float32(1.0)
        x[rng.random(x.shape) < 0.005] = np.float32(3.0)
    scores = f32_to_bf16_bits(x) if bf16 else x
    if kind == "specials":
        flat = scores if bf16 else scores.view(np.uint32)
        sp = (np.array([BF16_QNAN, BF16_PINF, BF16_NINF, BF16_PZERO, BF16_NZERO, 0xFFC0, 0x7F81],
                       dtype=np.uint16) if bf16 else
              np.array([0x7FC00000, 0x7F800000, 0xFF800000, 0, 0x80000000, 0xFFC00000,
                        0x7F800001], dtype=np.uint32))
        u = rng.random(scores.shape)
        is_sp = u < 0.35
        flat[is_sp] = sp[rng.integers(0, len(sp), size=int(is_sp.sum()))]
        tie = (u >= 0.35) & (u < 0.45)
        tt, hh, bb = np.nonzero(tie)
        flat[tt, hh, bb] = flat[tt, hh, rng.integers(0, M, size=len(bb))]
    if tail == "neginf":
        _fill_tail(scores, nvp)
    elif tail == "nan":
        mask = np.arange(M)[None, :] >= np.minimum(nvp, M)[:, None]
        m3 = np.broadcast_to(mask[:, None, :], scores.shape)
        if bf16:
            scores[m3] = BF16_QNAN
        else:
            scores.view(np.uint32)[m3] = 0x7FC00000
    return Workload(name="rows_%d_%s" % (seed, kind), scores=scores, block_table=bt,
                    num_valid_pages=nvp.astype(np.int32), seq_lens=None, decode_query_len=1,
                    row_req=row_req, row_pos=row_pos, topk=topk, num_init=num_init,
                    num_local=num_local)


# ---------------------------------------------------------------------------
# inputs of the sparse paged-attention decode (the consumer of the sparse table)
# ---------------------------------------------------------------------------

HEAD_DIM = 128
PAGE_TOKENS = 16


@dataclasses.dataclass
class AttnInputs:
    """Inputs of one sparse-attention decode call (bf16 arrays as uint16 bits).

    q [T, H*G, D]; k_cache [P, H, D/8, 16, 8]; v_cache [P, H, D, 16];
    table [T, H, W] int32 page ids; ctx [T, H] int32; scale = 1/sqrt(D).
    """
    name: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    table: np.ndarray
    ctx: np.ndarray
    scale: float
    decode_query_len: int = 1       # rows per request (the rows' grouping, not the data)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def G(self) -> int:
        return int(self.q.shape[1]) // self.H

    @property
    def P(self) -> int:
        return int(self.k_cache.shape[0])


def _bf16_normal(rng, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _kv_pages(rng, P: int, H: int, D: int) -> tuple[np.ndarray, np.ndarray]:
    k = _bf16_normal(rng, (P, H, D // 8, PAGE_TOKENS, 8))
    v = _bf16_normal(rng, (P, H, D, PAGE_TOKENS))
    return k, v


def attention_inputs(name: str, table: np.ndarray, ctx: np.ndarray, G: int, seed: int,
                     D: int = HEAD_DIM, decode_query_len: int = 1) -> AttnInputs:
    """Attention inputs over a given sparse table (for example a select + table result).

    The page ids the table holds are renamed to a compact, seeded random order
    (storage names only: every row keeps its pages and their order), so the cache
    holds just the pages the table names, each with N(0, 1) bf16 keys and values
    for every KV head; q is N(0, 1) bf16.
    """
    table = np.ascontiguousarray(table, dtype=np.int32)
    T, H, _ = table.shape
    rng = np.random.Generator(np.random.PCG64(seed))
    uniq, inverse = np.unique(table, return_inverse=True)
    perm = rng.permutation(uniq.shape[0]).astype(np.int32)
    compact = perm[inverse.reshape(-1)].reshape(table.shape).astype(np.int32)
    q = _bf16_normal(rng, (T, H * G, D))
    k, v = _kv_pages(rng, uniq.shape[0], H, D)
    return AttnInputs(name=name, q=q, k_cache=k, v_cache=v, table=compact,
                      ctx=np.ascontiguousarray(ctx, dtype=np.int32),
                      scale=float(1.0 / np.sqrt(D)), decode_query_len=decode_query_len)


def attention_case(seed: int, *, T: int = 4, H: int = 2, G: int = 8, W: int = 128,
                   P: int = 64, ctx=None, ctx_hi: Optional[int] = None,
                   bad_page_frac: float = 0.0, D: int = HEAD_DIM) -> AttnInputs:
    """A small seeded attention case with random page lists.

    ``ctx`` fixes every row's context length (an int, or an array [T, H]); otherwise it
    is uniform in [0, ctx_hi] (default 16 * W). ``bad_page_frac`` of the table entries
    are replaced by ids outside [0, P) (negative or >= P).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    table = rng.integers(0, P, size=(T, H, W)).astype(np.int32)
    if bad_page_frac > 0:
        bad = rng.random((T, H, W)) < bad_page_frac
        alt = np.where(rng.random((T, H, W)) < 0.5, -1 - rng.integers(0, 1 << 20, size=(T, H, W)),
                       P + rng.integers(0, 1 << 20, size=(T, H, W)))
        table[bad] = alt[bad].astype(np.int32)
    if ctx is None:
        hi = PAGE_TOKENS * W if ctx_hi is None else ctx_hi
        ctx_arr = rng.integers(0, hi, size=(T, H), endpoint=True).astype(np.int32)
    else:
        ctx_arr = np.broadcast_to(np.asarray(ctx, dtype=np.int32), (T, H)).copy()
    q = _bf16_normal(rng, (T, H * G, D))
    k, v = _kv_pages(rng, P, H, D)
    return AttnInputs(name="attn_case_%d" % seed, q=q, k_cache=k, v_cache=v, table=table,
                      ctx=ctx_arr, scale=float(1.0 / np.sqrt(D)))


# ---------------------------------------------------------------------------
# inputs of the decode index-score producer (the step before the selector)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class IndexInputs:
    """Inputs of one decode index-score call (bf16 arrays as uint16 bits).

    q_idx [T, H, D]; k_cache [8 * num_blocks, H, D/8, 16, 8] (16-token pages, block p in
    pages 8p .. 8p + 7); block_table [B, max_blocks]; seq_lens [B]; T = B * q;
    max_k_tiles M; scale = 1/sqrt(D). With FP8 keys, k_cache holds E4M3 codes (uint8)
    [8 * num_blocks, H, D/16, 16, 16] and k_scale [8 * num_blocks, H, 16] float32.
    """
    name: str
    q_idx: np.ndarray
    k_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    decode_query_len: int
    max_k_tiles: int
    scale: float
    k_scale: Optional[np.ndarray] = None

    @property
    def T(self) -> int:
        return int(self.q_idx.shape[0])

    @property
    def H(self) -> int:
        return int(self.q_idx.shape[1])

    @property
    def B(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0]) // 8


def fp8_e4m3_quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """E4M3 codes [..., n] (uint8, torch's round-to-nearest conversion) and float32 scales
    [...] with scale = max|x| / 448 over the last axis (input preparation only)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    sc = (np.maximum(np.abs(x).max(axis=-1), np.float32(1e-30)) / np.float32(448.0)).astype(np.float32)
    q8 = torch.from_numpy(x / sc[..., None]).to(torch.float8_e4m3fn)
    return q8.view(torch.uint8).numpy().copy(), sc


def index_inputs(name: str, seq_lens, q: int, H: int, max_k_tiles: int, seed: int,
                 max_blocks: Optional[int] = None, D: int = HEAD_DIM,
                 spare_blocks: int = 0, fp8: bool = False) -> IndexInputs:
    """Seeded index queries, a compact paged index-K cache and its block table.

    Every request's used blocks (cdiv(seq_len, 128), at most max_blocks) get distinct
    physical ids from a seeded permutation of the cache's blocks (entries past them are
    0); keys and queries are N(0, 1) bf16. `spare_blocks` adds unreferenced blocks.
    With `fp8`, the same N(0, 1) keys are stored as E4M3 codes with one scale per
    (page, head, token) (max |key| / 448).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    if max_blocks is None:
        max_blocks = max_k_tiles
    rng = np.random.Generator(np.random.PCG64(seed))
    used = np.minimum((seq_lens.astype(np.int64) + BLOCK_TOKENS - 1) // BLOCK_TOKENS, max_blocks)
    nb = int(used.sum()) + spare_blocks
    ids = rng.permutation(max(nb, 1)).astype(np.int32)
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    at = 0
    for r in range(B):
        bt[r, : used[r]] = ids[at: at + used[r]]
        at += int(used[r])
    ksc = None
    if fp8:
        kf = rng.standard_normal((max(nb, 1) * 8, H, PAGE_TOKENS, D), dtype=np.float32)
        codes, ksc = fp8_e4m3_quantize(kf)                       # [P, H, 16, D], [P, H, 16]
        P_ = codes.shape[0]
        k = np.ascontiguousarray(
            codes.reshape(P_, H, PAGE_TOKENS, D // 16, 16).transpose(0, 1, 3, 2, 4))
    else:
        k = _bf16_normal(rng, (max(nb, 1) * 8, H, D // 8, PAGE_TOKENS, 8))
    qi = _bf16_normal(rng, (B * q, H, D))
    return IndexInputs(name=name, q_idx=qi, k_cache=k, block_table=bt, seq_lens=seq_lens,
                       decode_query_len=q, max_k_tiles=max_k_tiles,
                       scale=float(1.0 / np.sqrt(D)), k_scale=ksc)
