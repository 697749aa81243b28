"""Pins of the decode index-score oracle (CPU only).

oracle/index_scores.py reads index keys out of the paged cache through index formulas
and reduces each causal block by log-sum-exp or max. These tests tie it to things
other than itself: torch's logsumexp / amax (float64) on dense per-request key arrays
that the tests scatter into pages with reshapes and transposes of their own; closed
forms (constant keys, a zero query, a one-token last block, a dominant key, zero keys
for invalid blocks); and the causal and capacity structure (which entries are
written, for every spec-decode row).
"""
import math

import numpy as np
import pytest
import torch

from kv_block_top_amd import workloads as wl

D = 128
NEG = -np.inf


def to_bf16(x):
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def from_bf16(b):
    return wl.bf16_bits_to_f32(b).astype(np.float64)


def build(dense, H, rng, spare=3):
    """Paged cache + block table for dense per-request keys: dense[r][h] is [n_r, D].

    Blocks get random physical ids; a request's keys are split into 128-token blocks,
    each block into 8 pages of 16 tokens stored as [D/8, 16, 8] (reshapes only)."""
    B = len(dense)
    used = [-(-dense[r][0].shape[0] // 128) for r in range(B)]
    nb = sum(used) + spare
    perm = rng.permutation(nb)
    k_cache = to_bf16(rng.standard_normal((nb * 8, H, D // 8, 16, 8)))
    bt = np.zeros((B, max(max(used), 1)), dtype=np.int32)
    at = 0
    for r in range(B):
        ids = perm[at: at + used[r]]
        at += used[r]
        bt[r, : used[r]] = ids
        for h in range(H):
            x = dense[r][h]
            pad = used[r] * 128 - x.shape[0]
            if pad:
                x = np.concatenate([x, to_bf16(np.zeros((pad, D)))])
            blocks = x.reshape(used[r], 8, 16, D // 8, 8).transpose(0, 1, 3, 2, 4)
            for j, p in enumerate(ids):
                k_cache[p * 8: p * 8 + 8, h] = blocks[j]
    return k_cache, bt


def run(index_oracle, q_idx, k_cache, bt, seq_lens, q, scale, reduce, M=None, fill=NEG):
    T, H, _ = q_idx.shape
    M = M or bt.shape[1]
    init = np.full((T, H, M), fill)
    return index_oracle.index_decode_scores(q_idx, k_cache, bt, np.asarray(seq_lens, np.int32),
                                            q, scale, reduce, init)


@pytest.mark.parametrize("reduce", ["lse", "max"])
@pytest.mark.parametrize("lens,q,H", [((1, 128, 129), 1, 1), ((300, 1000), 4, 2),
                                      ((2048, 17), 2, 3), ((5, 4, 3), 4, 1)])
def test_matches_library_reductions(index_oracle, reduce, lens, q, H):
    rng = np.random.Generator(np.random.PCG64(sum(lens) + q + H))
    dense = [[to_bf16(rng.standard_normal((n, D))) for _ in range(H)] for n in lens]
    k_cache, bt = build(dense, H, rng)
    q_idx = to_bf16(rng.standard_normal((len(lens) * q, H, D)))
    scale = 0.0884
    got = run(index_oracle, q_idx, k_cache, bt, lens, q, scale, reduce)
    for t in range(len(lens) * q):
        r, lq = divmod(t, q)
        c = max(lens[r] - q + lq + 1, 0)
        nvp = -(-c // 128)
        for h in range(H):
            keys = torch.from_numpy(from_bf16(dense[r][h][:c]))
            s = scale * (keys @ torch.from_numpy(from_bf16(q_idx[t, h])))
            for b in range(nvp):
                part = s[128 * b: min(128 * (b + 1), c)]
                want = torch.logsumexp(part, 0) if reduce == "lse" else torch.amax(part)
                assert abs(got[t, h, b] - float(want)) <= 1e-12 * max(1.0, abs(float(want)))
            assert np.all(got[t, h, nvp:] == NEG)


def test_constant_keys_and_zero_query(index_oracle):
    rng = np.random.Generator(np.random.PCG64(3))
    lens = (300,)
    dense = [[to_bf16(np.full((300, D), 0.5))]]
    k_cache, bt = build(dense, 1, rng)
    q_idx = to_bf16(np.full((1, 1, D), 0.25))
    s = 0.1 * D * 0.5 * 0.25
    lse = run(index_oracle, q_idx, k_cache, bt, lens, 1, 0.1, "lse")
    mx = run(index_oracle, q_idx, k_cache, bt, lens, 1, 0.1, "max")
    for b, n in enumerate((128, 128, 44)):
        assert abs(lse[0, 0, b] - (s + math.log(n))) < 1e-12
        assert mx[0, 0, b] == s
    zero = run(index_oracle, to_bf16(np.zeros((1, 1, D))), k_cache, bt, lens, 1, 0.1, "lse")
    np.testing.assert_allclose(zero[0, 0, :3], [math.log(128), math.log(128), math.log(44)],
                               rtol=0, atol=1e-14)


def test_one_token_last_block_is_its_logit(index_oracle):
    rng = np.random.Generator(np.random.PCG64(4))
    n = 128 * 3 + 1
    dense = [[to_bf16(rng.standard_normal((n, D)))]]
    k_cache, bt = build(dense, 1, rng)
    q_idx = to_bf16(rng.standard_normal((1, 1, D)))
    logit = 0.3 * float(from_bf16(dense[0][0][n - 1]) @ from_bf16(q_idx[0, 0]))
    for reduce in ("lse", "max"):
        got = run(index_oracle, q_idx, k_cache, bt, (n,), 1, 0.3, reduce)
        assert abs(got[0, 0, 3] - logit) < 1e-12


def test_dominant_key_lse_equals_its_logit(index_oracle):
    # one key scores 1000 above the rest of its block: lse = 1000 + log(1 + ~e^-1000)
    rng = np.random.Generator(np.random.PCG64(5))
    keys = np.zeros((200, D))
    keys[150, 7] = 1.0
    dense = [[to_bf16(keys)]]
    k_cache, bt = build(dense, 1, rng)
    q = np.zeros((1, 1, D))
    q[0, 0, 7] = 1000.0
    got = run(index_oracle, to_bf16(q), k_cache, bt, (200,), 1, 1.0, "lse")
    assert got[0, 0, 1] == 1000.0
    assert abs(got[0, 0, 0] - math.log(128)) < 1e-14


def test_spec_rows_write_only_their_causal_blocks(index_oracle):
    # q = 4 rows at positions seq_len - 4 .. seq_len - 1 (causal lengths seq_len - 3 ..
    # seq_len): 258 puts the first two rows' last token in block 1 and the last two rows'
    # in block 2; 3 leaves the first row empty; 0 leaves all four empty
    rng = np.random.Generator(np.random.PCG64(6))
    lens = (258, 3, 0, 130)
    dense = [[to_bf16(rng.standard_normal((max(n, 1), D)))] for n in lens]
    k_cache, bt = build(dense, 1, rng)
    q_idx = to_bf16(rng.standard_normal((16, 1, D)))
    q_idx[1:4] = q_idx[0]                     # one query for the four rows of request 0
    got = run(index_oracle, q_idx, k_cache, bt, lens, 4, 0.1, "lse", M=4, fill=np.nan)
    written = ~np.isnan(got[:, 0, :])
    want = np.zeros((16, 4), dtype=bool)
    for t, nv in enumerate([2, 2, 3, 3, 0, 1, 1, 1, 0, 0, 0, 0, 1, 1, 2, 2]):
        want[t, :nv] = True
    assert np.array_equal(written, want)
    # with one query, request 0's rows agree where they see the same tokens: block 0
    # for all four, block 1 for the last three (the first sees 127 of its tokens)
    assert np.all(got[1:4, 0, 0] == got[0, 0, 0])
    assert np.all(got[2:4, 0, 1] == got[1, 0, 1]) and got[0, 0, 1] != got[1, 0, 1]


def test_capacity_limits(index_oracle):
    rng = np.random.Generator(np.random.PCG64(7))
    dense = [[to_bf16(rng.standard_normal((1000, D)))]]
    k_cache, bt = build(dense, 1, rng)
    q_idx = to_bf16(rng.standard_normal((1, 1, D)))
    full = run(index_oracle, q_idx, k_cache, bt, (1000,), 1, 0.1, "max")
    assert np.isfinite(full[0, 0, :8]).all()
    short = run(index_oracle, q_idx, k_cache, bt, (1000,), 1, 0.1, "max", M=5)
    assert np.array_equal(short[0, 0], full[0, 0, :5])
    narrow = index_oracle.index_decode_scores(q_idx, k_cache, bt[:, :3], np.array([1000], np.int32),
                                              1, 0.1, "max", np.full((1, 1, 8), NEG))
    assert np.array_equal(narrow[0, 0, :3], full[0, 0, :3]) and np.all(narrow[0, 0, 3:] == NEG)


def test_invalid_physical_blocks_read_as_zero_keys(index_oracle):
    rng = np.random.Generator(np.random.PCG64(8))
    dense = [[to_bf16(rng.standard_normal((400, D)))]]
    k_cache, bt = build(dense, 1, rng, spare=0)
    q_idx = to_bf16(rng.standard_normal((1, 1, D)))
    good = run(index_oracle, q_idx, k_cache, bt, (400,), 1, 0.1, "lse")
    nb = k_cache.shape[0] // 8
    bt2 = bt.copy()
    bt2[0, 1] = -3
    bt2[0, 3] = nb
    got = run(index_oracle, q_idx, k_cache, bt2, (400,), 1, 0.1, "lse")
    assert got[0, 0, 0] == good[0, 0, 0] and got[0, 0, 2] == good[0, 0, 2]
    assert abs(got[0, 0, 1] - math.log(128)) < 1e-14 and abs(got[0, 0, 3] - math.log(16)) < 1e-14
    mx = run(index_oracle, q_idx, k_cache, bt2, (400,), 1, 0.1, "max")
    assert mx[0, 0, 1] == 0.0 and mx[0, 0, 3] == 0.0


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) index keys with one scale per (page, head, slot)
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_for_every_code(index_oracle):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = index_oracle.e4m3_value(codes)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), np.nonzero(~same)[0][:8]


def test_e4m3_hand_values(index_oracle):
    v = index_oracle.e4m3_value(np.array([0x7E, 0x01, 0x08, 0x38, 0x80, 0x7F, 0xFE, 0x3C],
                                         dtype=np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -9 and v[2] == 2.0 ** -6 and v[3] == 1.0
    assert v[4] == 0.0 and np.signbit(v[4]) and np.isnan(v[5])
    assert v[6] == -448.0 and v[7] == 1.5


def build_fp8(dense, H, rng, spare=2):
    """FP8 paged cache + scales + block table for dense per-request fp32 keys: each
    token's keys are quantized with scale = max|k| / 448 (torch's e4m3 conversion);
    pages stored as [D/16, 16, 16] by reshapes. Returns the dequantized dense keys too."""
    B = len(dense)
    used = [-(-dense[r][0].shape[0] // 128) for r in range(B)]
    nb = sum(used) + spare
    perm = rng.permutation(nb)
    k_cache = rng.integers(0, 0x7E, size=(nb * 8, H, D // 16, 16, 16)).astype(np.uint8)
    k_scale = rng.random((nb * 8, H, 16)).astype(np.float32)
    bt = np.zeros((B, max(max(used), 1)), dtype=np.int32)
    deq = []
    at = 0
    for r in range(B):
        ids = perm[at: at + used[r]]
        at += used[r]
        bt[r, : used[r]] = ids
        deq.append([])
        for h in range(H):
            x = dense[r][h].astype(np.float32)
            n = x.shape[0]
            sc = np.maximum(np.abs(x).max(axis=1), 1e-30).astype(np.float32) / np.float32(448.0)
            q8 = torch.from_numpy(x / sc[:, None]).to(torch.float8_e4m3fn)
            deq[r].append(q8.double().numpy() * sc[:, None].astype(np.float64))
            codes = q8.view(torch.uint8).numpy()
            pad = used[r] * 128 - n
            codes = np.concatenate([codes, np.zeros((pad, D), np.uint8)]) if pad else codes
            scp = np.concatenate([sc, np.ones(pad, np.float32)]) if pad else sc
            blocks = codes.reshape(used[r], 8, 16, D // 16, 16).transpose(0, 1, 3, 2, 4)
            sblocks = scp.reshape(used[r], 8, 16)
            for j, p in enumerate(ids):
                k_cache[p * 8: p * 8 + 8, h] = blocks[j]
                k_scale[p * 8: p * 8 + 8, h] = sblocks[j]
    return k_cache, k_scale, bt, deq


@pytest.mark.parametrize("reduce", ["lse", "max"])
@pytest.mark.parametrize("lens,q,H", [((1, 128, 129), 1, 2), ((300, 1000), 4, 1)])
def test_fp8_keys_match_library_reductions(index_oracle, reduce, lens, q, H):
    rng = np.random.Generator(np.random.PCG64(97 + sum(lens)))
    dense = [[rng.standard_normal((n, D)) * rng.uniform(0.1, 4.0) for _ in range(H)]
             for n in lens]
    k_cache, k_scale, bt, deq = build_fp8(dense, H, rng)
    q_idx = to_bf16(rng.standard_normal((len(lens) * q, H, D)))
    scale = 0.0884
    init = np.full((len(lens) * q, H, bt.shape[1]), NEG)
    got = index_oracle.index_decode_scores(q_idx, k_cache, bt, np.asarray(lens, np.int32), q,
                                           scale, reduce, init, k_scale=k_scale)
    for t in range(len(lens) * q):
        r, lq = divmod(t, q)
        c = max(lens[r] - q + lq + 1, 0)
        for h in range(H):
            s = scale * (torch.from_numpy(deq[r][h][:c]) @ torch.from_numpy(from_bf16(q_idx[t, h])))
            for b in range(-(-c // 128)):
                part = s[128 * b: min(128 * (b + 1), c)]
                want = torch.logsumexp(part, 0) if reduce == "lse" else torch.amax(part)
                assert abs(got[t, h, b] - float(want)) <= 1e-12 * max(1.0, abs(float(want)))


def test_fp8_zero_query_and_scale_linearity(index_oracle):
    rng = np.random.Generator(np.random.PCG64(98))
    dense = [[rng.standard_normal((200, D))]]
    k_cache, k_scale, bt, _ = build_fp8(dense, 1, rng)
    init = np.full((1, 1, 2), NEG)
    zero = index_oracle.index_decode_scores(to_bf16(np.zeros((1, 1, D))), k_cache, bt,
                                            np.array([200], np.int32), 1, 0.1, "lse", init,
                                            k_scale=k_scale)
    np.testing.assert_allclose(zero[0, 0], [math.log(128), math.log(72)], rtol=0, atol=1e-14)
    q_idx = to_bf16(rng.standard_normal((1, 1, D)))
    one = index_oracle.index_decode_scores(q_idx, k_cache, bt, np.array([200], np.int32), 1,
                                           0.1, "max", init, k_scale=k_scale)
    two = index_oracle.index_decode_scores(q_idx, k_cache, bt, np.array([200], np.int32), 1,
                                           0.1, "max", init, k_scale=k_scale * 2)
    np.testing.assert_allclose(two[0, 0], 2 * one[0, 0], rtol=1e-14)
