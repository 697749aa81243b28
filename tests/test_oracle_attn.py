"""Pins of the sparse-attention oracle (CPU only).

The oracle (oracle/sparse_attn.py) reads tokens out of the paged cache through index
formulas. These tests tie it to things other than itself:
  - a library routine: torch's scaled_dot_product_attention (float64, CPU) on dense
    per-row key/value arrays, which the tests scatter into pages with reshapes and
    transposes of their own;
  - closed forms: one token, equal keys (plain mean), one dominant key, two tokens
    (a logistic weight), constant values per KV head (query-head grouping), zero
    pages, empty rows;
  - invariances: reordering whole pages, clamping ctx to the table width.
"""
import math

import numpy as np
import pytest
import torch

from kv_block_top_amd import workloads as wl

D = 128


def to_bf16(x):
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def from_bf16(b):
    return wl.bf16_bits_to_f32(b).astype(np.float64)


def paged_cache(dense_k, dense_v, P, rng):
    """Scatter dense [H][n_h, D] keys/values (bf16 bits) into a paged cache.

    Returns (k_cache, v_cache, pages) where pages[h] lists the page ids holding head
    h's tokens in order. Built with reshapes and transposes only (no index formula).
    """
    H = len(dense_k)
    k_cache = to_bf16(rng.standard_normal((P, H, D // 8, 16, 8)))
    v_cache = to_bf16(rng.standard_normal((P, H, D, 16)))
    free = rng.permutation(P)
    pages, at = [], 0
    for h in range(H):
        n = dense_k[h].shape[0]
        npg = -(-n // 16)
        ids = free[at: at + npg]
        at += npg
        pad = npg * 16 - n
        kk = np.concatenate([dense_k[h], to_bf16(np.zeros((pad, D)))]) if pad else dense_k[h]
        vv = np.concatenate([dense_v[h], to_bf16(np.zeros((pad, D)))]) if pad else dense_v[h]
        # token-major [npg, 16, D] -> K [npg, D/8, 16, 8] and V [npg, D, 16]
        k_cache[ids, h] = kk.reshape(npg, 16, D // 8, 8).transpose(0, 2, 1, 3)
        v_cache[ids, h] = vv.reshape(npg, 16, D).transpose(0, 2, 1)
        pages.append(ids)
    return k_cache, v_cache, pages


def single_row(dense_k, dense_v, q_bits, W, rng, P=None):
    """One row (T = 1): table and ctx listing each head's dense tokens in order."""
    H = len(dense_k)
    need = sum(-(-k.shape[0] // 16) for k in dense_k)
    P = P or need + 5
    k_cache, v_cache, pages = paged_cache(dense_k, dense_v, P, rng)
    table = rng.integers(0, P, size=(1, H, W)).astype(np.int32)    # junk past the row
    ctx = np.zeros((1, H), dtype=np.int32)
    for h in range(H):
        table[0, h, :len(pages[h])] = pages[h]
        ctx[0, h] = dense_k[h].shape[0]
    return q_bits[None], k_cache, v_cache, table, ctx


def sdpa(q, k, v, scale):
    """torch's attention for one query vector over [n, D] keys/values (float64)."""
    qt = torch.from_numpy(q).reshape(1, 1, 1, D)
    kt = torch.from_numpy(k).reshape(1, 1, -1, D)
    vt = torch.from_numpy(v).reshape(1, 1, -1, D)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale).reshape(D).numpy()


@pytest.mark.parametrize("lengths,G,scale", [
    ((1, 16), 1, 0.088), ((17, 2047), 2, 0.088), ((15, 33), 3, 0.5), ((2048,), 8, 0.088),
    ((129, 64, 250), 1, 0.02)])
def test_matches_library_attention_on_dense_pages(attn_oracle, lengths, G, scale):
    rng = np.random.Generator(np.random.PCG64(sum(lengths) + G))
    dk = [to_bf16(rng.standard_normal((n, D))) for n in lengths]
    dv = [to_bf16(rng.standard_normal((n, D))) for n in lengths]
    H = len(lengths)
    q = to_bf16(rng.standard_normal((H * G, D)))
    args = single_row(dk, dv, q, 128, rng)
    out = attn_oracle.sparse_attn_decode(*args, scale)
    for h in range(H):
        for g in range(G):
            j = h * G + g
            want = sdpa(from_bf16(q[j]), from_bf16(dk[h]), from_bf16(dv[h]), scale)
            np.testing.assert_allclose(out[0, j], want, rtol=0, atol=1e-12)


def test_single_token_returns_its_value(attn_oracle):
    rng = np.random.Generator(np.random.PCG64(11))
    dk = [to_bf16(rng.standard_normal((1, D))) for _ in range(2)]
    dv = [to_bf16(rng.standard_normal((1, D))) for _ in range(2)]
    q = to_bf16(rng.standard_normal((2 * 4, D)))
    out = attn_oracle.sparse_attn_decode(*single_row(dk, dv, q, 8, rng), 3.0)
    for j in range(8):
        assert np.array_equal(out[0, j], from_bf16(dv[j // 4][0]))


def test_equal_keys_give_the_mean_of_values(attn_oracle):
    rng = np.random.Generator(np.random.PCG64(12))
    n = 37
    dk = [to_bf16(np.full((n, D), 0.25))]
    dv = [to_bf16(rng.standard_normal((n, D)))]
    q = to_bf16(rng.standard_normal((3, D)))
    out = attn_oracle.sparse_attn_decode(*single_row(dk, dv, q, 8, rng), 0.7)
    mean = from_bf16(dv[0]).sum(axis=0) / n
    for j in range(3):
        np.testing.assert_allclose(out[0, j], mean, rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value(attn_oracle):
    # one key scores 1000 above all others: every other weight is below e^-1000
    rng = np.random.Generator(np.random.PCG64(13))
    n, m = 100, 58
    k = np.zeros((n, D))
    k[m, 5] = 1.0
    q = np.zeros((1, D))
    q[0, 5] = 1000.0
    dv = [to_bf16(rng.standard_normal((n, D)))]
    out = attn_oracle.sparse_attn_decode(*single_row([to_bf16(k)], dv, to_bf16(q), 8, rng), 1.0)
    assert np.array_equal(out[0, 0], from_bf16(dv[0][m]))


def test_two_tokens_logistic_weight(attn_oracle):
    # w_b = 1 / (1 + exp(s_a - s_b)) for two tokens with scores s_a = 0.5 * 2, s_b = 0
    rng = np.random.Generator(np.random.PCG64(14))
    k = np.zeros((2, D))
    k[0, 0] = 2.0
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    v = np.zeros((2, D))
    v[0, :] = 3.0
    v[1, :] = -1.0
    out = attn_oracle.sparse_attn_decode(
        *single_row([to_bf16(k)], [to_bf16(v)], to_bf16(q), 8, rng), 0.5)
    wb = 1.0 / (1.0 + math.exp(1.0))
    np.testing.assert_allclose(out[0, 0], np.full(D, 3.0 * (1 - wb) - 1.0 * wb), rtol=1e-15)


def test_query_heads_group_onto_their_kv_head(attn_oracle):
    # H = 3 KV heads with constant values h + 1; G = 2 query heads each
    rng = np.random.Generator(np.random.PCG64(15))
    H, G = 3, 2
    dk = [to_bf16(rng.standard_normal((40 + h, D))) for h in range(H)]
    dv = [to_bf16(np.full((40 + h, D), h + 1.0)) for h in range(H)]
    q = to_bf16(rng.standard_normal((H * G, D)))
    out = attn_oracle.sparse_attn_decode(*single_row(dk, dv, q, 8, rng), 0.3)
    for j in range(H * G):
        np.testing.assert_allclose(out[0, j], np.full(D, j // G + 1.0), rtol=1e-14)


def test_empty_and_negative_ctx_give_zeros(attn_oracle):
    a = wl.attention_case(21, T=3, H=2, G=2, W=4, P=8, ctx=0)
    out = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, a.ctx, a.scale)
    assert not out.any()
    ctx = np.array([[-5, 0], [0, -1], [-1 << 30, 0]], dtype=np.int32)
    out = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, ctx, a.scale)
    assert not out.any()


def test_ctx_beyond_the_table_is_clamped(attn_oracle):
    a = wl.attention_case(22, T=2, H=2, G=2, W=3, P=10, ctx=48)
    want = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, a.ctx, a.scale)
    big = np.full_like(a.ctx, 1 << 30)
    got = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, big, a.scale)
    assert np.array_equal(got, want)


def test_pages_outside_the_cache_are_zero_pages(attn_oracle):
    rng = np.random.Generator(np.random.PCG64(23))
    n = 64                                    # 4 pages; pages 1 and 3 will be invalid
    dk = rng.standard_normal((n, D))
    dv = rng.standard_normal((n, D))
    q = to_bf16(rng.standard_normal((1, D)))
    args = list(single_row([to_bf16(dk)], [to_bf16(dv)], q, 8, rng))
    P = args[1].shape[0]
    args[3][0, 0, 1] = -1
    args[3][0, 0, 3] = P + 7
    out = attn_oracle.sparse_attn_decode(*args, 0.2)
    zk, zv = from_bf16(to_bf16(dk)), from_bf16(to_bf16(dv))
    for p in (1, 3):
        zk[16 * p: 16 * p + 16] = 0.0
        zv[16 * p: 16 * p + 16] = 0.0
    want = sdpa(from_bf16(q[0]), zk, zv, 0.2)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-12)
    args[3][0, 0, :4] = [-1, -2, P, P + 1]
    assert not attn_oracle.sparse_attn_decode(*args, 0.2).any()


def test_empty_cache_gives_zeros(attn_oracle):
    # with no page in the cache every listed page lies outside it: zero keys and values,
    # so every output is a convex combination of zero vectors
    import dataclasses
    a = wl.attention_case(25, T=5, H=2, G=4, W=8, P=40)
    b = dataclasses.replace(a, k_cache=a.k_cache[:0], v_cache=a.v_cache[:0])
    assert b.P == 0 and (b.ctx > 0).any()
    out, spread, vmax = attn_oracle.sparse_attn_decode(b.q, b.k_cache, b.v_cache, b.table,
                                                       b.ctx, b.scale, with_spread=True)
    assert out.shape == (5, 8, 128)
    assert not out.any() and not spread.any() and not vmax.any()


def test_reordering_whole_pages_changes_nothing(attn_oracle):
    a = wl.attention_case(24, T=3, H=2, G=3, W=16, P=300, ctx=16 * 9 + 5)
    want = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, a.table, a.ctx, a.scale)
    rng = np.random.Generator(np.random.PCG64(25))
    table = a.table.copy()
    for t in range(a.T):
        for h in range(a.H):
            table[t, h, :9] = table[t, h, rng.permutation(9)]      # the partial 10th stays
    got = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, table, a.ctx, a.scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    table[:, :, [8, 9]] = table[:, :, [9, 8]]                     # moving the partial page does
    got = attn_oracle.sparse_attn_decode(a.q, a.k_cache, a.v_cache, table, a.ctx, a.scale)
    assert np.abs(got - want).max() > 1e-6


def test_spread_and_value_bound(attn_oracle):
    rng = np.random.Generator(np.random.PCG64(26))
    dv = [to_bf16(np.full((20, D), 1.5)), to_bf16(rng.standard_normal((30, D)))]
    dk = [to_bf16(rng.standard_normal((20, D))), to_bf16(rng.standard_normal((30, D)))]
    q = to_bf16(rng.standard_normal((2, D)))
    out, spread, vmax = attn_oracle.sparse_attn_decode(*single_row(dk, dv, q, 8, rng), 0.1,
                                                       with_spread=True)
    assert not spread[0, 0].any()                       # equal values: no spread
    assert vmax[0, 0] == 1.5
    assert vmax[0, 1] == np.abs(from_bf16(dv[1])).max()
    assert (spread[0, 1] > 0).all() and (spread[0, 1] <= 2 * vmax[0, 1]).all()
