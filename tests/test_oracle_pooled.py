"""Pins for the oracle's pooled-score mask and list compaction (CPU only).

Pooled scores are checked against an independent numpy evaluation (pairwise
summed means and a matrix product); selection against numpy argmax / stable
argsort and, for the cumulative-mass rule, against exhaustive enumeration of
every subset of key blocks on small rows. Compaction is checked against a
numpy nonzero scan.
"""
import itertools

import numpy as np
import pytest

import oracle


def rand_qk(B, N, H, D, seed):
    r = np.random.default_rng(seed)
    base = r.standard_normal((N, D))  # shared structure so scores spread out
    q = r.standard_normal((B, N, H, D)) + base[None, :, None, :]
    k = r.standard_normal((B, N, H, D)) + base[None, :, None, :]
    return q, k


def numpy_scores(q, k, bq, bk, scale):
    B, N, H, D = q.shape
    nQ, nK = -(-N // bq), -(-N // bk)
    S = np.zeros((B, H, nQ, nK))
    for b in range(B):
        for h in range(H):
            qb = np.stack([q[b, a * bq:min(N, (a + 1) * bq), h].mean(axis=0) for a in range(nQ)])
            kb = np.stack([k[b, c * bk:min(N, (c + 1) * bk), h].mean(axis=0) for c in range(nK)])
            S[b, h] = scale * (qb @ kb.T)
    return S


@pytest.mark.parametrize("N,bq,bk", [(200, 32, 16), (130, 16, 16)])
def test_scores_match_numpy(oracle_lib, N, bq, bk):
    q, k = rand_qk(1, N, 3, 16, seed=N)
    _, S, _ = oracle.build_mask_pooled(q, k, bq, bk, 0.25, 0, 1, want_scores=True)
    ref = numpy_scores(q, k, bq, bk, 0.25)
    np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-14)


def test_full_budget_keeps_everything(oracle_lib):
    q, k = rand_qk(1, 150, 2, 8, seed=2)
    nK = -(-150 // 16)
    m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 0, nK)
    assert np.all(m == 1)
    m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 0, nK + 5)
    assert np.all(m == 1)
    m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 1, 1.0)
    assert np.all(m == 1)


def test_top1_is_argmax_and_topk_is_stable_sort_prefix(oracle_lib):
    q, k = rand_qk(2, 190, 2, 8, seed=3)
    S = numpy_scores(q, k, 16, 16, 0.5)
    m1, _, _ = oracle.build_mask_pooled(q, k, 16, 16, 0.5, 0, 1)
    assert np.all(m1.sum(axis=-1) == 1)
    np.testing.assert_array_equal(m1.argmax(axis=-1), S.argmax(axis=-1))
    for kk in (3, 5):
        mk, _, _ = oracle.build_mask_pooled(q, k, 16, 16, 0.5, 0, kk)
        order = np.argsort(-S, axis=-1, kind="stable")[..., :kk]
        ref = np.zeros_like(mk)
        np.put_along_axis(ref, order, 1, axis=-1)
        np.testing.assert_array_equal(mk, ref)


def test_ties_break_to_lower_block(oracle_lib):
    # identical key blocks give exactly equal pooled scores
    B, N, H, D = 1, 64, 1, 4
    r = np.random.default_rng(4)
    q = r.standard_normal((B, N, H, D))
    blk = r.standard_normal((16, D))
    k = np.tile(blk, (4, 1))[None, :, None, :].copy()
    m, S, _ = oracle.build_mask_pooled(q, k, 16, 16, 1.0, 0, 2, want_scores=True)
    assert np.all(S[..., 0:1] == S)
    assert np.all(m[..., :2] == 1) and np.all(m[..., 2:] == 0)


@pytest.mark.parametrize("tau", [0.3, 0.5, 0.8, 0.95])
def test_cumulative_mass_is_minimal_subset(oracle_lib, tau):
    """Exhaustive check on nK = 7: the kept set is a smallest subset of key
    blocks whose softmax mass reaches tau, and it has the largest mass among
    subsets of that size."""
    B, N, H, D, bq, bk = 1, 7 * 8, 2, 6, 8, 8
    q, k = rand_qk(B, N, H, D, seed=int(tau * 100))
    m, S, _ = oracle.build_mask_pooled(q, k, bq, bk, 1.5, 1, tau, want_scores=True)
    nK = 7
    for h in range(H):
        for a in range(7):
            s = S[0, h, a]
            p = np.exp(s - s.max())
            p /= p.sum()
            best = None
            for size in range(1, nK + 1):
                masses = [(p[list(c)].sum(), c) for c in itertools.combinations(range(nK), size)]
                ok = [x for x in masses if x[0] >= tau]
                if ok:
                    best = (size, max(x[0] for x in masses))
                    break
            kept = np.nonzero(m[0, h, a])[0]
            assert len(kept) == best[0]
            assert abs(p[kept].sum() - best[1]) < 1e-12


def test_cumulative_mass_keeps_argmax_and_rows_nonempty(oracle_lib):
    q, k = rand_qk(1, 300, 3, 8, seed=9)
    S = numpy_scores(q, k, 32, 16, 0.4)
    m, _, margin = oracle.build_mask_pooled(q, k, 32, 16, 0.4, 1, 0.6)
    assert np.all(m.sum(axis=-1) >= 1)
    am = S.argmax(axis=-1)
    assert np.all(np.take_along_axis(m, am[..., None], axis=-1) == 1)
    assert np.all(margin >= 0)


# ------------------------------------------------------------- compaction
@pytest.mark.parametrize("shared", [False, True])
def test_compaction_matches_nonzero_scan(oracle_lib, shared):
    B, H, nQ, nK = 2, 3, 5, 11
    r = np.random.default_rng(6)
    if shared:
        mask = (r.random((nQ, nK)) < 0.4).astype(np.uint8)
        full = np.broadcast_to(mask, (B, H, nQ, nK))
        hs = 0
    else:
        mask = (r.random((B, H, nQ, nK)) < 0.4).astype(np.uint8)
        mask[0, 1, 2] = 0  # an empty row
        full = mask
        hs = nQ * nK
    skip = (r.random((B, H, nQ, nK)) < 0.3).astype(np.uint8)
    for sk in (None, skip):
        row_ptr, kv_idx = oracle.compact(mask, B, H, nQ, nK, hs, sk)
        eff = full.astype(bool) & (True if sk is None else ~sk.astype(bool))
        eff = eff.reshape(-1, nK)
        assert row_ptr[-1] == eff.sum() == kv_idx.size
        for row in range(B * H * nQ):
            np.testing.assert_array_equal(kv_idx[row_ptr[row]:row_ptr[row + 1]],
                                          np.nonzero(eff[row])[0])


# ------------------------------------------------------ global selection
def _row_argmax_mask(S):
    m = np.zeros(S.shape, np.uint8)
    np.put_along_axis(m, S.argmax(axis=-1)[..., None], 1, axis=-1)
    return m


def test_global_topk_full_budget_and_top1(oracle_lib):
    q, k = rand_qk(1, 150, 2, 8, seed=12)
    nQ, nK = -(-150 // 32), -(-150 // 16)
    m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 2, nQ * nK)
    assert np.all(m == 1)
    # one pair per head plus every row's best block is the per-row top-1 mask
    # (the head's best pair is its row's best block)
    m1, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 2, 1)
    r1, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.3, 0, 1)
    np.testing.assert_array_equal(m1, r1)


@pytest.mark.parametrize("kk", [3, 17, 40])
def test_global_topk_is_head_wide_stable_sort_prefix_plus_row_best(oracle_lib, kk):
    q, k = rand_qk(2, 190, 2, 8, seed=13 + kk)
    S = numpy_scores(q, k, 32, 16, 0.5)
    B, H, nQ, nK = S.shape
    m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.5, 2, kk)
    flat = S.reshape(B, H, nQ * nK)
    order = np.argsort(-flat, axis=-1, kind="stable")[..., :kk]
    ref = np.zeros(flat.shape, np.uint8)
    np.put_along_axis(ref, order, 1, axis=-1)
    ref = ref.reshape(S.shape) | _row_argmax_mask(S)
    np.testing.assert_array_equal(m, ref)


def test_global_topk_ties_break_to_lower_pair_index(oracle_lib):
    # identical key blocks: every pair of a row scores the same
    B, N, H, D = 1, 64, 1, 4
    r = np.random.default_rng(14)
    q = np.tile(r.standard_normal((1, D)), (N, 1))[None, :, None, :].copy()
    k = np.tile(r.standard_normal((16, D)), (4, 1))[None, :, None, :].copy()
    m, S, _ = oracle.build_mask_pooled(q, k, 16, 16, 1.0, 2, 6, want_scores=True)
    assert np.all(S == S.flat[0])
    # pairs 0..5 in row-major order, plus block 0 of every row
    ref = np.zeros(16, np.uint8)
    ref[:6] = 1
    ref = ref.reshape(4, 4)
    ref[:, 0] = 1
    np.testing.assert_array_equal(m[0, 0], ref)


@pytest.mark.parametrize("tau", [0.2, 0.45, 0.7, 0.9])
def test_global_cumulative_mass_is_minimal_pair_set(oracle_lib, tau):
    """Exhaustive over all 12 pairs of a 3x4 head: the kept pairs minus the
    rows' best blocks form a smallest set of pairs whose mass (each row's
    softmax over its blocks) reaches tau * nQ, with the largest mass among
    sets of that size; the rows' best blocks are added on top."""
    B, N, H, D, bq, bk = 1, 48, 2, 6, 16, 12
    q, k = rand_qk(B, N, H, D, seed=int(tau * 1000))
    m, S, margin = oracle.build_mask_pooled(q, k, bq, bk, 2.0, 3, tau, want_scores=True)
    nQ, nK = 3, 4
    for h in range(H):
        s = S[0, h]
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = (p / p.sum(axis=1, keepdims=True)).ravel()
        best = None
        for size in range(1, nQ * nK + 1):
            cands = [(p[list(c)].sum(), c) for c in itertools.combinations(range(nQ * nK), size)]
            ok = [x for x in cands if x[0] >= tau * nQ]
            if ok:
                best = max(ok)
                break
        ref = np.zeros(nQ * nK, np.uint8)
        if best is None:
            ref[:] = 1
        else:
            ref[list(best[1])] = 1
        ref = ref.reshape(nQ, nK) | _row_argmax_mask(s)
        np.testing.assert_array_equal(m[0, h], ref)
        assert margin[0, h, 0] >= 0


def test_global_cumulative_mass_monotone_in_tau_and_rows_nonempty(oracle_lib):
    q, k = rand_qk(1, 300, 3, 8, seed=15)
    prev = None
    for tau in (0.05, 0.2, 0.5, 0.8, 0.95, 1.0):
        m, _, _ = oracle.build_mask_pooled(q, k, 32, 16, 0.4, 3, tau)
        assert np.all(m.sum(axis=-1) >= 1)
        if prev is not None:
            assert np.all(m >= prev)          # larger tau keeps a superset
        prev = m
    assert prev.mean() > 0.9
