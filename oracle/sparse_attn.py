"""CPU oracle for sparse paged-attention decode over the page-16 sparse block table.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The HIP library never calls
it and shares no source with it.

What it computes (vLLM PR #47984 report, "[ROCm][MiniMax-M3][Spec Decode] Support
speculative decode with AITER sparse PA": Summary and Implementation breakdown items
1-3 describe the sparse paged attention that consumes the page-16 sparse block table
and the per-row sparse context length; the attention itself is not printed there, so
this is ordinary scaled dot-product attention restricted to the listed tokens):

    for each row t, index head h and query head j of h's group (j in [h*G, (h+1)*G)):
        c = min(max(ctx[t, h], 0), 16 * W)           W = table width (topk * 8)
        token i (0 <= i < c) lives in page table[t, h, i // 16], slot i % 16
        s_i = scale * <q[t, j], K_i>                 over the head dimension D
        out[t, j] = sum_i softmax(s)_i * V_i         (all zeros when c == 0)

Readings where the pages are silent (each is stated in the design notes too):
  - KV head h of the cache pairs with index head h, and its group of G consecutive
    query heads attends over h's sparse row.
  - Cache layouts (bf16): K [P, H, D/8, 16, 8], i.e. K_i[d] = k[page, h, d // 8, slot,
    d % 8]; V [P, H, D, 16], i.e. V_i[d] = v[page, h, d, slot].
  - A page id outside [0, P) stands for a page of zero keys and zero values.
  - Arithmetic in float64 on the exact values of the bf16 inputs.

Arrays: q [T, H*G, D], k_cache and v_cache as above, all numpy uint16 bf16 bit
patterns; table [T, H, W] and ctx [T, H] int32. The pins that tie this code to the
mathematics (closed forms, a library attention routine on dense arrays, invariances)
are in tests/test_oracle_attn.py.
"""
from __future__ import annotations

import numpy as np

TOKENS_PER_PAGE = 16


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (bf16 is the top half of a binary32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gather_tokens(k_cache: np.ndarray, v_cache: np.ndarray, pages: np.ndarray,
                  slots: np.ndarray, h: int) -> tuple[np.ndarray, np.ndarray]:
    """Keys and values [n, D] (float64) of the tokens (pages[i], slots[i]) of KV head h.

    Pages outside [0, P) give zero rows.
    """
    P = k_cache.shape[0]
    D = v_cache.shape[2]
    if P == 0:                      # an empty cache: every page is outside it
        return np.zeros((len(pages), D)), np.zeros((len(pages), D))
    ok = (pages >= 0) & (pages < P)
    pg = np.where(ok, pages, 0).astype(np.int64)
    d = np.arange(D)
    keys = bf16_value(k_cache[pg[:, None], h, d[None, :] // 8, slots[:, None], d[None, :] % 8])
    vals = bf16_value(v_cache[pg[:, None], h, d[None, :], slots[:, None]])
    keys[~ok] = 0.0
    vals[~ok] = 0.0
    return keys, vals


def sparse_attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                       table: np.ndarray, ctx: np.ndarray, scale: float,
                       with_spread: bool = False):
    """Attention output [T, H*G, D] float64 (see the module docstring).

    With ``with_spread`` it also returns, per output element, the weighted spread
    sum_i w_i |V_i[d] - out[d]| (how far a relative change of the weights can move
    the result) and, per (row, index head), the largest |V_i[d]| over the listed
    tokens; the parity tests derive their tolerance from these.
    """
    T, HG, D = q.shape
    H = k_cache.shape[1]
    W = table.shape[2]
    if HG % H != 0:
        raise ValueError("query heads (%d) must be a multiple of KV heads (%d)" % (HG, H))
    G = HG // H
    qf = bf16_value(q)
    out = np.zeros((T, HG, D), dtype=np.float64)
    spread = np.zeros((T, HG, D), dtype=np.float64)
    vmax = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for h in range(H):
            c = min(max(int(ctx[t, h]), 0), TOKENS_PER_PAGE * W)
            if c == 0:
                continue
            i = np.arange(c)
            pages = table[t, h, i // TOKENS_PER_PAGE].astype(np.int64)
            keys, vals = gather_tokens(k_cache, v_cache, pages, i % TOKENS_PER_PAGE, h)
            vmax[t, h] = np.abs(vals).max()
            for j in range(h * G, (h + 1) * G):
                s = scale * (keys @ qf[t, j])            # [c]
                e = np.exp(s - s.max())
                w = e / e.sum()
                o = w @ vals                              # [D]
                out[t, j] = o
                if with_spread:
                    spread[t, j] = w @ np.abs(vals - o[None, :])
    if with_spread:
        return out, spread, vmax
    return out
