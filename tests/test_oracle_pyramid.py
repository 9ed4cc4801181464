"""Pins for the oracle's pyramid attention (CPU only).

Pyramid Sparse Attention page: key/value blocks at several resolutions, each
level the average of the finer one; every (query block, key block) pair
attends at the level its importance earns, by thresholds; probabilities stay
consistent across levels. Pinned by: level 0 everywhere equals binary block
attention; keys and values that are constant inside every group of tokens
give the same output at any mix of levels (this fixes the +level*ln 2 weight
of a pooled key); constant V is reproduced; the level mask relates exactly
to the per-row cumulative-mass mask at each threshold; the tile lists match
layouts worked out by hand for three and four levels
(tests/golden/pyramid_lists_296*.txt), and, decoded into pooled key rows
with numpy alone, give the attention the oracle computes from the level
mask.
"""
import os

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


@pytest.mark.parametrize("levels", [(1, 2), (1, 3), (1, 2, 3), (1, 4), (1, 2, 3, 4)])
def test_group_constant_keys_and_values_give_level_zero_output(oracle_lib, levels):
    """If every group of 8 consecutive tokens shares one key and one value, a
    pooled key equals each of its tokens, and with weight 2^l it carries the
    same probability mass: any mix of levels gives the level-0 output."""
    B, N, H, D, bq, bk = 1, 256, 2, 8, 32, 64
    r = np.random.default_rng(3)
    base = r.standard_normal((B, N // 8, H, D, 3))
    q = r.standard_normal((B, N, H, D))
    k = np.repeat(base[..., 0], 8, axis=1)
    v = np.repeat(base[..., 1], 8, axis=1)
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
    m = np.random.default_rng(6).integers(0, 5, size=(B, H, 8, 2)).astype(np.uint8)
    m[..., 0] = np.maximum(m[..., 0], 1)     # no empty row
    o, _ = oracle.pyramid_attention(q, k, v, bq, bk, 0.5, m, 16)
    np.testing.assert_allclose(o.reshape(-1, D), np.broadcast_to(c, (o.size // D, D)),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("taus", [(0.3, 0.6, 0.9), (0.5, 0.5, 0.8), (0.2, 0.95), (0.7,),
                                  (0.2, 0.4, 0.6, 0.8)])
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
    # four levels: 296, 148, 74, 37 rows -> 5, 3, 2, 1 blocks
    rb, rr = oracle.pyramid_regions(296, 64, 4)
    assert rb.tolist() == [0, 5, 8, 10, 11] and rr.tolist() == [296, 148, 74, 37]


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pyramid_lists_296.txt")
GOLDEN4 = os.path.join(os.path.dirname(__file__), "golden", "pyramid_lists_296_four_levels.txt")


def golden_rows(path=GOLDEN):
    rows = []
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            m, want = line.split("|")
            pairs = [tuple(int(x) for x in t.split(":")) for t in want.split()]
            rows.append(([int(x) for x in m.split()], pairs))
    return rows


@pytest.mark.parametrize("path,L", [(GOLDEN, 3), (GOLDEN4, 4)])
def test_pyramid_lists_golden_by_hand(oracle_lib, path, L):
    """N = 296, three or four levels, ragged last block: lists worked out by
    hand from the level layout (tests/golden/pyramid_lists_296*.txt)."""
    rows = golden_rows(path)
    N, bk = 296, 64
    nQ, nK = len(rows), 5
    m = np.array([r[0] for r in rows], np.uint8).reshape(1, 1, nQ, nK)
    rp, kv, qm = oracle.compact_pyramid(m, 1, 1, nQ, nK, N, bk, L, nQ * nK)
    want_rp = np.cumsum([0] + [len(r[1]) for r in rows])
    np.testing.assert_array_equal(rp, want_rp)
    for a, (_, pairs) in enumerate(rows):
        got = list(zip(kv[rp[a]:rp[a + 1]].tolist(), qm[rp[a]:rp[a + 1]].tolist()))
        assert got == pairs, (a, got, pairs)


def decode_and_attend(q, k, v, bq, bk, scale, n_levels, rp, kv, qm, rows):
    """Attention of the given list rows evaluated from the lists alone: each
    entry (augmented block, eighth bits) names pooled key rows of one level
    (level l region = augmented blocks [rb_l, rb_l+1), N >> l valid rows);
    pooled row g of level l is the mean of tokens g*2^l .. g*2^l + 2^l - 1 of
    K and of V, and its score carries + l ln 2 (it stands for 2^l tokens)."""
    B, N, H, D = q.shape
    nQ = -(-N // bq)
    starts, valid = [0], []
    for l in range(n_levels):
        valid.append(N >> l)
        starts.append(starts[-1] + -(-(N >> l) // bk))
    outs = []
    for row in rows:
        bh, a = divmod(int(row), nQ)
        b, h = divmod(bh, H)
        keys, vals, bias = [], [], []
        for ab, bits in zip(kv[rp[row]:rp[row + 1]], qm[rp[row]:rp[row + 1]]):
            l = max(i for i in range(n_levels) if starts[i] <= ab)
            g = 1 << l
            for eighth in range(8):
                if not (bits >> eighth) & 1:
                    continue
                for pr in range((ab - starts[l]) * bk + eighth * (bk // 8),
                                (ab - starts[l]) * bk + (eighth + 1) * (bk // 8)):
                    if pr >= valid[l]:
                        continue
                    keys.append(k[b, pr * g:(pr + 1) * g, h].mean(axis=0))
                    vals.append(v[b, pr * g:(pr + 1) * g, h].mean(axis=0))
                    bias.append(l * np.log(2.0))
        qi = q[b, a * bq:min(N, (a + 1) * bq), h]
        if not keys:
            outs.append((np.zeros_like(qi), np.full(len(qi), -np.inf)))
            continue
        s = scale * qi @ np.array(keys).T + np.array(bias)[None, :]
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        outs.append((p @ np.array(vals) / p.sum(axis=1, keepdims=True),
                     mx[:, 0] + np.log(p.sum(axis=1))))
    return outs


@pytest.mark.parametrize("L", [3, 4])
@pytest.mark.parametrize("N", [256, 296, 1000])
def test_pyramid_lists_decode_to_the_mask(oracle_lib, N, L):
    """The lists, decoded into pooled key rows with no help from the oracle,
    give the attention the oracle computes from the level mask itself."""
    B, H, D, bq, bk = 1, 2, 8, 64, 64
    nQ, nK = -(-N // bq), -(-N // bk)
    r = np.random.default_rng(N + L)
    q, k, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    m = r.integers(0, L + 1, size=(B, H, nQ, nK)).astype(np.uint8)
    m[..., 0, :] = 0                                 # one empty row per head
    rp, kv, qm = oracle.compact_pyramid(m, B, H, nQ, nK, N, bk, L, nQ * nK)
    assert rp[-1] == kv.size == qm.size
    for row in range(B * H * nQ):
        e0, e1 = rp[row], rp[row + 1]
        assert np.all(np.diff(kv[e0:e1]) > 0) and np.all(qm[e0:e1] > 0)
    o_ref, l_ref = oracle.pyramid_attention(q, k, v, bq, bk, 0.5, m, nQ * nK)
    rows = np.arange(B * H * nQ)
    for row, (o, lse) in zip(rows, decode_and_attend(q, k, v, bq, bk, 0.5, L, rp, kv, qm, rows)):
        n = len(o)
        np.testing.assert_allclose(o, o_ref[row, :n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref[row, :n], rtol=0, atol=1e-12)
    # all level 0: the plain ascending lists with whole tiles
    ones = (m > 0).astype(np.uint8)
    rp1, kv1, qm1 = oracle.compact_pyramid(ones, B, H, nQ, nK, N, bk, L, nQ * nK)
    rp0, kv0 = oracle.compact(ones, B, H, nQ, nK, nQ * nK)
    np.testing.assert_array_equal(rp1, rp0)
    np.testing.assert_array_equal(kv1, kv0)
    assert np.all(qm1 == 255)


def test_decode_catches_a_shifted_eighth(oracle_lib):
    """The decode check is sharp: moving the selected eighths of one entry by
    two eighths changes the decoded attention."""
    N, B, H, D, bq, bk, L = 296, 1, 1, 8, 64, 64, 3
    rows = golden_rows()
    nQ, nK = len(rows), 5
    m = np.array([r[0] for r in rows], np.uint8).reshape(1, 1, nQ, nK)
    rp, kv, qm = oracle.compact_pyramid(m, B, H, nQ, nK, N, bk, L, nQ * nK)
    r = np.random.default_rng(11)
    q, k, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    o_ref, _ = oracle.pyramid_attention(q, k, v, bq, bk, 0.5, m, nQ * nK)
    bad = qm.copy()
    bad[1] = 60                                      # row 0, block 5: eighths 2-5, not 4-7
    (o_bad, _), = decode_and_attend(q, k, v, bq, bk, 0.5, L, rp, kv, bad, [0])
    assert np.abs(o_bad - o_ref[0, :len(o_bad)]).max() > 1e-3


def test_compaction_rejects_levels_above_the_pyramid(oracle_lib):
    m = np.array([[[[1, 4, 0, 0, 0]]]], np.uint8)      # level 3 in a three-level pyramid
    with pytest.raises(ValueError):
        oracle.compact_pyramid(m, 1, 1, 1, 5, 296, 64, 3, 5)
