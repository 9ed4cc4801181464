"""Pins for the oracle's token orders before blocking (CPU only).

PAROAttention summary page, section 二 (six axis orders, one per head) and
VMoBA summary page, section 三 (temporal chunks, spatial patches and cubes).
Pinned by hand-worked orders, by the bijection and locality properties every
such order has, by the orders that must reduce to the identity, and by the
permutation equivariance of dense attention (gather, attend, scatter back).
"""
import itertools
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_orders.txt")


def golden_cases():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        head, perm = line.split("|")
        T, Hs, Ws, kind, a0, a1, a2 = (int(x) for x in head.split())
        out.append(((T, Hs, Ws, kind, (a0, a1, a2)), [int(x) for x in perm.split()]))
    return out


@pytest.mark.parametrize("case", golden_cases())
def test_golden_token_orders(oracle_lib, case):
    (T, Hs, Ws, kind, axes), want = case
    assert oracle.make_permutation(T, Hs, Ws, kind, axes).tolist() == want


def coords(perm, Hs, Ws):
    p = np.asarray(perm, dtype=np.int64)
    return p // (Hs * Ws), (p // Ws) % Hs, p % Ws


@pytest.mark.parametrize("axes", list(itertools.permutations(range(3))))
def test_axis_orders_are_bijections_with_the_named_fastest_axis(oracle_lib, axes):
    T, Hs, Ws = 3, 4, 5
    perm = oracle.make_permutation(T, Hs, Ws, oracle.PERM_AXES, axes)
    assert sorted(perm.tolist()) == list(range(T * Hs * Ws))
    co = np.stack(coords(perm, Hs, Ws))          # [3][N]
    ext = (T, Hs, Ws)
    fast, mid, slow = axes[2], axes[1], axes[0]
    # the fastest axis counts up and wraps; the slowest changes least often
    assert np.array_equal(co[fast], np.tile(np.arange(ext[fast]), T * Hs * Ws // ext[fast]))
    assert np.array_equal(co[slow], np.repeat(np.arange(ext[slow]), T * Hs * Ws // ext[slow]))
    if axes == (0, 1, 2):
        np.testing.assert_array_equal(perm, np.arange(T * Hs * Ws))


@pytest.mark.parametrize("box", [(1, 2, 2), (2, 3, 2), (3, 4, 5), (2, 1, 5), (1, 4, 5),
                                 (4, 7, 9), (2, 3, 4)])
def test_box_partitions_are_bijections_of_contiguous_boxes(oracle_lib, box):
    T, Hs, Ws = 5, 7, 9
    perm = oracle.make_permutation(T, Hs, Ws, oracle.PERM_BOXES, box)
    assert sorted(perm.tolist()) == list(range(T * Hs * Ws))
    t, y, x = coords(perm, Hs, Ws)
    bid = ((t // box[0]) * -(-Hs // box[1]) + y // box[1]) * -(-Ws // box[2]) + x // box[2]
    # every box is one contiguous run, boxes in (t, y, x) order
    assert np.all(np.diff(bid) >= 0)
    for b in np.unique(bid):
        run = np.nonzero(bid == b)[0]
        assert run[-1] - run[0] + 1 == run.size
        # inside a box, tokens keep (t, y, x) order
        assert np.all(np.diff(perm[run]) > 0)
    if box[1] >= Hs and box[2] >= Ws:              # whole-frame chunks: identity
        np.testing.assert_array_equal(perm, np.arange(T * Hs * Ws))


def test_gather_then_scatter_restores(oracle_lib):
    r = np.random.default_rng(3)
    x = r.standard_normal((2, 60, 3, 8))
    perms = np.stack([oracle.make_permutation(3, 4, 5, 0, ax) for ax in
                      [(2, 1, 0), (1, 0, 2), (0, 2, 1)]])
    for P in (perms[0], perms):
        g = oracle.permute_tokens(x, P)
        np.testing.assert_array_equal(oracle.permute_tokens(g, P, scatter=True), x)
        if P.ndim == 1:
            np.testing.assert_array_equal(g[:, 1], x[:, P[1]])


def test_dense_attention_is_equivariant_under_token_orders(oracle_lib):
    """Attention over all tiles in a permuted order, scattered back, equals
    attention in the original order (softmax is a sum over all keys)."""
    B, T, Hs, Ws, H, D = 1, 3, 4, 6, 2, 16
    N = T * Hs * Ws
    r = np.random.default_rng(4)
    q, k, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    bq = bk = 16
    nQ = nK = -(-N // 16)
    ones = np.ones((nQ, nK), np.uint8)
    o, lse, _ = oracle.attention(q, k, v, bq, bk, 0.3, ones, 0)
    P = np.stack([oracle.make_permutation(T, Hs, Ws, 0, (2, 0, 1)),
                  oracle.make_permutation(T, Hs, Ws, 1, (2, 2, 3))])
    qp, kp, vp = (oracle.permute_tokens(a, P) for a in (q, k, v))
    op, lsep, _ = oracle.attention(qp, kp, vp, bq, bk, 0.3, ones, 0)
    op = op.reshape(B, H, nQ * bq, D)[:, :, :N].transpose(0, 2, 1, 3)
    back = oracle.permute_tokens(np.ascontiguousarray(op), P, scatter=True)
    want = o.reshape(B, H, nQ * bq, D)[:, :, :N].transpose(0, 2, 1, 3)
    np.testing.assert_allclose(back, want, rtol=0, atol=1e-12)
