"""Pins for the oracle's visiting order of kept key blocks (CPU only).

LiteAttention summary page, section 五: visiting the key blocks of a row
radial-centrically reaches the row maximum sooner, so the running-maximum
test skips more. The order is pinned by hand-worked cases (tie-breaking
included), by the centre-out property that any such order has (every prefix
of the visit is a contiguous run of the ascending list), and by its effect on
a constructed input whose row maxima sit on the diagonal blocks.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "radial_order_cases.txt")


def golden_cases():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        head, kept, want = (part.split() for part in line.split("|"))
        out.append((tuple(int(x) for x in head), [int(x) for x in kept], [int(x) for x in want]))
    return out


@pytest.mark.parametrize("case", golden_cases())
def test_golden_radial_orders(oracle_lib, case):
    (N, bq, bk, a), kept, want = case
    nQ = -(-N // bq)
    # one list row per row block; only row a holds the case
    lens = np.zeros(nQ, np.int32)
    lens[a] = len(kept)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = oracle.order_lists(row_ptr, np.array(kept, np.int32), N, bq, bk, oracle.ORDER_RADIAL)
    assert got.tolist() == want


def random_lists(rng, R, nK, density):
    mask = rng.random((R, nK)) < density
    lens = mask.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kv = np.concatenate([np.nonzero(m)[0] for m in mask]).astype(np.int32)
    return row_ptr, kv


@pytest.mark.parametrize("N,bq,bk", [(1000, 64, 64), (1000, 128, 64), (777, 128, 64)])
def test_ascending_order_is_identity(oracle_lib, N, bq, bk):
    rng = np.random.default_rng(N + bq)
    nQ, nK = -(-N // bq), -(-N // bk)
    row_ptr, kv = random_lists(rng, 3 * nQ, nK, 0.4)
    got = oracle.order_lists(row_ptr, kv, N, bq, bk, oracle.ORDER_ASCENDING)
    np.testing.assert_array_equal(got, kv)


@pytest.mark.parametrize("N,bq,bk,density", [(1000, 64, 64, 0.5), (1000, 128, 64, 0.3),
                                               (777, 128, 64, 1.0), (4099, 64, 64, 0.05)])
def test_radial_order_is_a_centre_out_permutation(oracle_lib, N, bq, bk, density):
    rng = np.random.default_rng(N + bq + int(100 * density))
    nQ, nK = -(-N // bq), -(-N // bk)
    R = 2 * nQ
    row_ptr, kv = random_lists(rng, R, nK, density)
    got = oracle.order_lists(row_ptr, kv, N, bq, bk, oracle.ORDER_RADIAL)
    for r in range(R):
        e0, e1 = row_ptr[r], row_ptr[r + 1]
        asc, vis = kv[e0:e1], got[e0:e1]
        assert sorted(vis.tolist()) == asc.tolist()            # a permutation
        pos = np.searchsorted(asc, vis)                        # list index of each visit
        lo = hi = None
        for p in pos:                                          # every prefix is contiguous
            if lo is None:
                lo = hi = p
            else:
                assert p == lo - 1 or p == hi + 1
                lo, hi = min(lo, p), max(hi, p)
        a = r % nQ
        if bq == bk and vis.size and a in asc:                 # the diagonal block first
            assert vis[0] == a


def test_gaps_in_radial_order_match_brute_force(oracle_lib):
    """Gaps recomputed from the full score matrix, visiting each row's kept
    blocks in the order the (separately pinned) list ordering gives."""
    B, N, H, D, bq, bk = 1, 200, 2, 16, 32, 16
    r = np.random.default_rng(5)
    q, k, v = (r.standard_normal((B, N, H, D)) for _ in range(3))
    nQ, nK = -(-N // bq), -(-N // bk)
    mask = (r.random((B, H, nQ, nK)) < 0.6).astype(np.uint8)
    _, _, gap = oracle.attention(q, k, v, bq, bk, 0.9, mask, nQ * nK, want_gap=True,
                                 order=oracle.ORDER_RADIAL)
    flat = mask.reshape(B * H * nQ, nK)
    row_ptr = np.concatenate([[0], np.cumsum(flat.sum(axis=1))]).astype(np.int32)
    kv = np.concatenate([np.nonzero(m)[0] for m in flat]).astype(np.int32)
    order = oracle.order_lists(row_ptr, kv, N, bq, bk, oracle.ORDER_RADIAL)
    for row in range(B * H * nQ):
        bh, a = divmod(row, nQ)
        s = 0.9 * (q[0, a * bq:min(N, (a + 1) * bq), bh] @ k[0, :, bh].T)
        cols = order[row_ptr[row]:row_ptr[row + 1]]
        run = np.full(s.shape[0], -np.inf)
        for c in cols:
            loc = s[:, c * bk:min(N, (c + 1) * bk)].max(axis=1)
            want = (loc - run).max()
            assert gap[row, c] == want or abs(gap[row, c] - want) <= 1e-12
            run = np.maximum(run, loc)
        assert np.all(np.isnan(gap[row, np.setdiff1d(np.arange(nK), cols)]))


def diagonal_peak_inputs(n_blocks=4, blk=16, A=20.0):
    """Scores scale*q.k = A inside the diagonal blocks and 0 elsewhere (exact:
    q = 8 e_blk, k = 10 e_blk, scale 1/4, so 0.25 * 80 = 20)."""
    N, D = n_blocks * blk, 16
    q = np.zeros((1, N, 1, D), np.float32)
    k = np.zeros((1, N, 1, D), np.float32)
    for i in range(N):
        q[0, i, 0, i // blk] = 8.0
        k[0, i, 0, i // blk] = 10.0
    v = np.random.default_rng(1).standard_normal((1, N, 1, D)).astype(np.float32)
    return q, k, v, 0.25


def test_radial_order_marks_every_off_diagonal_tile_on_diagonal_peaks(oracle_lib):
    """Worked by hand: with tau = 10, radial order visits the diagonal block
    (score 20) first, so every later tile (score 0, gap -20) is marked: 4 rows
    x 3 = 12 tiles. Ascending order only marks the tiles after the diagonal:
    3 + 2 + 1 + 0 = 6."""
    q, k, v, scale = diagonal_peak_inputs()
    skip0 = np.zeros((1, 1, 4, 4), np.uint8)
    _, _, gap_r, new_r = oracle.skip_step(q, k, v, 16, 16, scale, skip0, 10.0,
                                          order=oracle.ORDER_RADIAL)
    _, _, gap_a, new_a = oracle.skip_step(q, k, v, 16, 16, scale, skip0, 10.0,
                                          order=oracle.ORDER_ASCENDING)
    assert int(new_r.sum()) == 12 and int(new_a.sum()) == 6
    np.testing.assert_array_equal(new_r[0, 0], 1 - np.eye(4, dtype=np.uint8))
    np.testing.assert_array_equal(new_a[0, 0], np.triu(np.ones((4, 4), np.uint8), 1))
    off = ~np.eye(4, dtype=bool)
    assert np.all(gap_r[off] == -20.0) and np.all(gap_r[~off] == np.inf)


def test_marked_tiles_obey_the_suppression_bound_in_radial_order(oracle_lib):
    """The exp(-tau) bound at the marking step holds for any visiting order."""
    B, N, H, D, bq, bk = 1, 128, 2, 16, 16, 16
    r = np.random.default_rng(32)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    q = 4.0 * u + 0.3 * r.standard_normal((B, N, H, D))
    k = 0.3 * r.standard_normal((B, N, H, D))
    k[:, 48:64] += 4.0 * u          # the peak block sits mid-sequence
    v = r.standard_normal((B, N, H, D))
    tau = 3.0
    ones = np.ones((8, 8), np.uint8)
    _, _, gap = oracle.attention(q, k, v, bq, bk, 0.5, ones, 0, want_gap=True,
                                 order=oracle.ORDER_RADIAL)
    marked = gap <= -tau
    assert marked.any()
    for row in range(B * H * 8):
        bh, a = divmod(row, 8)
        s = 0.5 * (q[0, a * bq:(a + 1) * bq, bh] @ k[0, :, bh].T)
        m = s.max(axis=1, keepdims=True)
        for c in np.nonzero(marked[row])[0]:
            assert np.all(np.exp(s[:, c * bk:(c + 1) * bk] - m) <= np.exp(-tau) * (1 + 1e-12))
