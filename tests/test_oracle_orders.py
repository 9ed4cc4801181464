"""Pins for the oracle's per-head choice of token order (PAROAttention
summary page, section 二: each head takes the axis order under which its
attention is most sparsity-friendly; reading: fewest tiles kept by the
pooled per-row selection, ties to the lower order).

Each check ties the composition to something outside it: permutations built
here by numpy transposes, the already pinned pooled mask, and inputs whose
best order follows from their construction."""
import numpy as np
import pytest

import oracle

ORDERS = ((0, 1, 2), (0, 2, 1), (1, 0, 2), (1, 2, 0), (2, 0, 1), (2, 1, 0))


def _perm_numpy(T, Hs, Ws, axes):
    """perm[i'] = original token at new position i': the (t, y, x) index grid
    transposed so that axes[0] varies slowest and axes[2] fastest."""
    return np.arange(T * Hs * Ws).reshape(T, Hs, Ws).transpose(axes).ravel()


def _inputs(B, H, T, Hs, Ws, d, seed):
    r = np.random.default_rng(seed)
    shape = (B, T * Hs * Ws, H, d)
    return (r.standard_normal(shape).astype(np.float32),
            r.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("mode,param", [(0, 3.0), (1, 0.5)])
def test_counts_equal_masks_of_gathered_inputs(mode, param):
    """Every order's count is the kept-tile count of the pooled mask of Q
    and K gathered by a numpy transpose of the token grid; order 0 is the
    identity."""
    B, H, T, Hs, Ws, d, bq, bk = 2, 3, 4, 6, 8, 16, 16, 16
    q, k = _inputs(B, H, T, Hs, Ws, d, 3)
    orders, counts = oracle.choose_token_orders(q, k, T, Hs, Ws, bq, bk, 0.25, mode, param)
    assert np.array_equal(_perm_numpy(T, Hs, Ws, (0, 1, 2)), np.arange(T * Hs * Ws))
    for o, axes in enumerate(ORDERS):
        p = _perm_numpy(T, Hs, Ws, axes)
        assert np.array_equal(oracle.make_permutation(T, Hs, Ws, oracle.PERM_AXES, axes), p)
        m, _, _ = oracle.build_mask_pooled(np.ascontiguousarray(q[:, p]),
                                           np.ascontiguousarray(k[:, p]), bq, bk, 0.25, mode,
                                           param)
        assert np.array_equal(counts[:, o], m.astype(np.int64).sum(axis=(0, 2, 3)))
    best = np.argmin(counts, axis=1)      # numpy's argmin takes the first minimum
    assert np.array_equal(orders, best)


def test_constant_inputs_tie_to_identity():
    """Identical tokens: every order gives the same mask, so every head keeps
    the identity (ties go to the lower order)."""
    B, H, T, Hs, Ws, d = 1, 2, 3, 4, 8, 16
    q = np.full((B, T * Hs * Ws, H, d), 0.5, np.float32)
    orders, counts = oracle.choose_token_orders(q, q.copy(), T, Hs, Ws, 16, 16, 0.3, 1, 0.4)
    assert np.all(counts == counts[:, :1])
    assert np.all(orders == 0)


def test_tokens_keyed_by_position_prefer_frames_fastest():
    """Q = K = a random vector per (row, column) position, the same in every
    frame, plus small noise: with the frame axis fastest (orders 3 and 5) a
    block of 16 tokens holds one position over the 16 frames, its pooled
    query matches exactly one pooled key block, and the cumulative mass is
    reached with one block per row; every other order mixes positions inside
    a block and spreads the mass. Orders 3 and 5 tie; the lower one wins."""
    B, H, T, Hs, Ws, d = 1, 2, 16, 4, 8, 64
    r = np.random.default_rng(7)
    pos = r.standard_normal((Hs, Ws, H, d)) * 3.0
    x = np.broadcast_to(pos[None], (T, Hs, Ws, H, d)).reshape(1, T * Hs * Ws, H, d)
    x = (x + 0.01 * r.standard_normal(x.shape)).astype(np.float32)
    orders, counts = oracle.choose_token_orders(x, x.copy(), T, Hs, Ws, 16, 16, 0.125, 1, 0.9)
    nQ = T * Hs * Ws // 16
    assert np.all(counts[:, 3] == nQ) and np.all(counts[:, 5] == nQ)
    assert np.all(counts[:, [0, 1, 2, 4]] > nQ)
    assert np.all(orders == 3)


def test_rejects_other_modes():
    q, k = _inputs(1, 1, 2, 4, 8, 16, 1)
    with pytest.raises(ValueError):
        oracle.choose_token_orders(q, k, 2, 4, 8, 16, 16, 0.25, 3, 0.5)
