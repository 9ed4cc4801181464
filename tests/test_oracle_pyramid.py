"""Pins for the oracle's pyramid attention (CPU only).

Pyramid Sparse Attention page: key/value blocks at several resolutions, each
level the average of the finer one; every (query block, key block) pair
attends at the level its importance earns, by thresholds; probabilities stay
consistent across levels. Pinned by: level 0 everywhere equals binary block
attention; keys and values that are constant inside every group of tokens
give the same output at any mix of levels (this fixes the +level*ln 2 weight
of a pooled key); constant V is reproduced; the level mask relates exactly
to the per-row cumulative-mass mask at each threshold; the tile lists are
checked by decoding them back into (level, block) pairs.
"""
import numpy as np
import pytest

import oracle


def rand_qkv(B, N, H, D, seed):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((B, N, H, D)) for _ in range(3))


def full_rows(o, B, H, N, bq):
    nQ = -(-N // bq)
    return o.reshape(B, H, nQ * bq, -1)[:, :, :N]


def test_level_zero_everywhere_is_block_attention(oracle_lib):
    B, N, H, D, bq, bk = 1, 200, 2, 16, 32, 16
    q, k, v = rand_qkv(B, N, H, D, 1)
    nQ, nK = -(-N // bq), -(-N // bk)
    m = (np.random.default_rng(2).random((B, H, nQ, nK)) < 0.5).astype(np.uint8)
    o1, l1 = oracle.pyramid_attention(q, k, v, bq, bk, 0.4, m, nQ * nK)
    o2, l2, _ = oracle.attention(q, k, v, bq, bk, 0.4, m, nQ * nK)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12, equal_nan=True)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12, equal_nan=True)


@pytest.mark.parametrize("levels", [(1, 2), (1, 3), (1, 2, 3)])
def test_group_constant_keys_and_values_give_level_zero_output(oracle_lib, levels):
    """If every group of 4 consecutive tokens shares one key and one value, a
    pooled key equals each of its tokens, and with weight 2^l it carries the
    same probability mass: any mix of levels gives the level-0 output."""
    B, N, H, D, bq, bk = 1, 256, 2, 8, 32, 64
    r = np.random.default_rng(3)
    base = r.standard_normal((B, N // 4, H, D, 3))
    q = r.standard_normal((B, N, H, D))
    k = np.repeat(base[..., 0], 4, axis=1)
    v = np.repeat(base[..., 1], 4, axis=1)
    nQ, nK = N // bq, N // bk
    mix = r.choice(np.array(levels, np.uint8), size=(B, H, nQ, nK))
    ones = np.ones_like(mix)
    o_mix, l_mix = oracle.pyramid_attention(q, k, v, bq, bk, 0.7, mix, nQ * nK)
    o_ref, l_ref = oracle.pyramid_attention(q, k, v, bq, bk, 0.7, ones, nQ * nK)
    np.testing.assert_allclose(o_mix, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_mix, l_ref, rtol=0, atol=1e-12)
    # without the per-key weight the mix would differ
    k2 = k.copy()
    k2[:, 1::4] += 1.0                       # break the groups
    o_brk, _ = oracle.pyramid_attention(q, k2, v, bq, bk, 0.7, mix, nQ * nK)
    assert np.abs(o_brk - o_ref).max() > 1e-3


def test_constant_values_are_reproduced_at_every_level(oracle_lib):
    B, N, H, D, bq, bk = 1, 128, 1, 8, 16, 64
    q, k, _ = rand_qkv(B, N, H, D, 4)
    c = np.random.default_rng(5).standard_normal(D)
    v = np.broadcast_to(c, (B, N, H, D)).copy()
    m = np.random.default_rng(6).integers(0, 4, size=(B, H, 8, 2)).astype(np.uint8)
    m[..., 0] = np.maximum(m[..., 0], 1)     # no empty row
    o, _ = oracle.pyramid_attention(q, k, v, bq, bk, 0.5, m, 16)
    np.testing.assert_allclose(o.reshape(-1, D), np.broadcast_to(c, (o.size // D, D)),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("taus", [(0.3, 0.6, 0.9), (0.5, 0.5, 0.8), (0.2, 0.95), (0.7,)])
def test_level_mask_matches_cumulative_mass_at_each_threshold(oracle_lib, taus):
    r = np.random.default_rng(7)
    base = r.standard_normal((300, 8))
    q = r.standard_normal((1, 300, 3, 8)) + base[None, :, None, :]
    k = r.standard_normal((1, 300, 3, 8)) + base[None, :, None, :]
    lv, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.6, 4, 0, levels_tau=list(taus))
    for l, t in enumerate(taus):
        m1, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.6, 1, t)
        np.testing.assert_array_equal((lv >= 1) & (lv <= l + 1), m1.astype(bool))
    assert lv.max() <= len(taus)
    assert np.all((lv == 1).sum(-1) >= 1)      # every row's best block at full resolution


def test_regions_by_hand(oracle_lib):
    # N = 256: levels hold 256, 128, 64 rows -> 4, 2, 1 blocks of 64
    rb, rr = oracle.pyramid_regions(256, 64, 3)
    assert rb.tolist() == [0, 4, 6, 7] and rr.tolist() == [256, 128, 64]
    # N = 296: 296, 148, 74 rows -> 5, 3, 2 blocks
    rb, rr = oracle.pyramid_regions(296, 64, 3)
    assert rb.tolist() == [0, 5, 8, 10] and rr.tolist() == [296, 148, 74]


@pytest.mark.parametrize("N", [256, 296, 1000])
def test_pyramid_lists_decode_to_the_mask(oracle_lib, N):
    B, H, bq, bk, L = 2, 2, 64, 64, 3
    nQ, nK = -(-N // bq), -(-N // bk)
    r = np.random.default_rng(N)
    m = r.integers(0, 4, size=(B, H, nQ, nK)).astype(np.uint8)
    rp, kv, qm = oracle.compact_pyramid(m, B, H, nQ, nK, N, bk, L, nQ * nK)
    rb, _ = oracle.pyramid_regions(N, bk, L)
    assert rp[-1] == kv.size == qm.size
    for row in range(B * H * nQ):
        e0, e1 = rp[row], rp[row + 1]
        assert np.all(np.diff(kv[e0:e1]) > 0) and np.all(qm[e0:e1] > 0)
        got = {(int(a), q_) for a, qq in zip(kv[e0:e1], qm[e0:e1]) for q_ in range(4)
               if qq >> q_ & 1}
        want = set()
        mrow = m.reshape(-1, nK)[row]
        for c in np.nonzero(mrow)[0]:
            l = int(mrow[c]) - 1
            per = bk >> l                                # pooled rows of a block
            for row0 in range(c * per, (c + 1) * per, bk // 4):
                want.add((int(rb[l] + row0 // bk), (row0 % bk) // (bk // 4)))
        assert got == want
    # all level 0: the plain ascending lists with whole tiles
    ones = (m > 0).astype(np.uint8)
    rp1, kv1, qm1 = oracle.compact_pyramid(ones, B, H, nQ, nK, N, bk, L, nQ * nK)
    rp0, kv0 = oracle.compact(ones, B, H, nQ, nK, nQ * nK)
    np.testing.assert_array_equal(rp1, rp0)
    np.testing.assert_array_equal(kv1, kv0)
    assert np.all(qm1 == 15)
