"""CPU oracle for the decode index-score producer (the step before the selector).

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The HIP library never calls
it and shares no source with it.

What the pages fix (vLLM PR #47502 report, "[Minimax-M3] Using tok_sparse_select from
MSA instead of triton kernels": Implementation breakdown items 1-2 and the
indexer_msa.py module docstring and constants in Key source snippets): the decode
score kernel writes only block scores, one per (decode row, index head, 128-token
block), into the decode rows [:nd] of the unified buffer [total_q, H, max_k_tiles];
it writes causally valid blocks only (the rest of the buffer keeps its -inf fill);
the index-K cache is paged in blocks of the same 128 tokens as the sparse blocks.
What they leave open, and the readings taken here (each is stated in the design
notes too):
  - a token's index score is scale * <q_idx[t, h], k_idx[token, h]> (one index key per
    token and index head, like a KV head);
  - a block's score reduces its causal tokens' index scores by log-sum-exp ("lse",
    the log of the block's share of the query's softmax mass) or by max ("max"); the
    caller picks one;
  - decode rows: row t is request t // q at position seq_lens[req] - q + t % q; its
    causal length is c = max(position + 1, 0), it scores blocks b < min(cdiv(c, 128),
    max_blocks, max_k_tiles), and block b holds its tokens 128 b .. min(128 (b + 1), c) - 1;
  - index-K cache layout (bf16): [num_pages, H, D/8, 16, 8] with 16-token pages, the
    tokens of physical 128-token block p in pages 8p .. 8p + 7 (the page-16 mapping of
    the sparse table); element (page, h, d // 8, slot, d % 8) is dimension d of token
    slot; a physical block id outside [0, num_pages / 8) reads as zero keys;
  - FP8 index keys (optional): OCP FP8 E4M3 codes in [num_pages, H, D/16, 16, 16]
    (element (page, h, d // 16, slot, d % 16)) with one float32 scale per (page, h, slot):
    the key is scale * e4m3(code);
  - arithmetic in float64 on the exact values of the bf16 / fp8 inputs.

Arrays: q_idx [T, H, D] and k_cache uint16 bf16 bit patterns (or k_cache uint8 FP8
codes with k_scale [num_pages, H, 16] float32); block_table [B, max_blocks], seq_lens
[B] int32; scores [T, H, max_k_tiles] float64 (a copy of the given initial buffer with
the scored entries replaced). Pins: tests/test_oracle_index.py.
"""
from __future__ import annotations

import numpy as np

BLOCK_TOKENS = 128
PAGE_TOKENS = 16
PAGES_PER_BLOCK = 8


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """float64 value of OCP FP8 E4M3 codes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def block_keys(k_cache: np.ndarray, phys: int, h: int, n: int,
               k_scale: np.ndarray | None = None) -> np.ndarray:
    """Keys [n, D] (float64) of the first n tokens of physical block `phys`, head h.

    bf16 cache (uint16, [P, H, D/8, 16, 8]) or, with `k_scale` [P, H, 16], an FP8 E4M3
    cache (uint8, [P, H, D/16, 16, 16]) whose keys are scale * e4m3(code)."""
    P = k_cache.shape[0]
    fp8 = k_scale is not None
    D = k_cache.shape[2] * (16 if fp8 else 8)
    if phys < 0 or (phys + 1) * PAGES_PER_BLOCK > P:
        return np.zeros((n, D))
    tok = np.arange(n)
    page = phys * PAGES_PER_BLOCK + tok // PAGE_TOKENS
    slot = tok % PAGE_TOKENS
    d = np.arange(D)
    if fp8:
        codes = k_cache[page[:, None], h, d[None, :] // 16, slot[:, None], d[None, :] % 16]
        return e4m3_value(codes) * k_scale[page, h, slot].astype(np.float64)[:, None]
    return bf16_value(k_cache[page[:, None], h, d[None, :] // 8, slot[:, None], d[None, :] % 8])


def reduce_scores(s: np.ndarray, reduce: str) -> float:
    if reduce == "max":
        return float(s.max())
    if reduce == "lse":
        m = s.max()
        return float(m + np.log(np.exp(s - m).sum()))
    raise ValueError(reduce)


def index_decode_scores(q_idx: np.ndarray, k_cache: np.ndarray, block_table: np.ndarray,
                        seq_lens: np.ndarray, decode_query_len: int, scale: float,
                        reduce: str, scores_in: np.ndarray, with_bound: bool = False,
                        k_scale: np.ndarray | None = None):
    """Block scores of the decode rows (see the module docstring).

    Returns a float64 copy of `scores_in` [T, H, M] with every scored entry replaced.
    With `with_bound` it also returns, per entry, scale * max over the block's tokens
    of sum_d |q_d k_d| (0 where not scored), the size of the products the kernel sums,
    from which the parity tests derive their tolerance. `k_scale` selects FP8 keys.
    """
    T, H, D = q_idx.shape
    B, max_blocks = block_table.shape
    q = decode_query_len
    M = scores_in.shape[2]
    if T != B * q:
        raise ValueError("T must equal B * decode_query_len")
    out = np.array(scores_in, dtype=np.float64, copy=True)
    bound = np.zeros((T, H, M))
    qf = bf16_value(q_idx)
    for t in range(T):
        req = t // q
        c = max(int(seq_lens[req]) - q + (t - req * q) + 1, 0)
        nvp = min(-(-c // BLOCK_TOKENS), max_blocks, M)
        for h in range(H):
            for b in range(nvp):
                n = min(BLOCK_TOKENS, c - BLOCK_TOKENS * b)
                keys = block_keys(k_cache, int(block_table[req, b]), h, n, k_scale)
                s = scale * (keys @ qf[t, h])
                out[t, h, b] = reduce_scores(s, reduce)
                if with_bound:
                    bound[t, h, b] = abs(scale) * (np.abs(keys) @ np.abs(qf[t, h])).max()
    if with_bound:
        return out, bound
    return out
