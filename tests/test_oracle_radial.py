"""Pins for the oracle's radial mask (CPU only).

The window rule is pinned to a hand-derived table and the hand-worked tiny
workload (tests/golden); the token-level predicate to the closed-form count
of kept pairs; the tile lift to a brute-force OR over token pairs and, on
block-aligned grids, to a closed-form tile count; plus symmetry, monotonicity
in the window and n log n growth of the kept-tile count.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_window_table_matches_hand_derivation(oracle_lib):
    for h0, beta, bk, d, kept, h in (map(int, r) for r in _read_rows("radial_windows.txt")):
        got_kept, got_h = oracle.radial_window(d, h0, beta, bk)
        assert got_kept == bool(kept), (h0, beta, bk, d)
        if kept:
            assert got_h == h, (h0, beta, bk, d)


def test_tiny_workload_by_hand(oracle_lib):
    rows = _read_rows("radial_tiny_mask.txt")
    pairs = int(rows[0][0])
    mask = np.array([[int(ch) for ch in r[0]] for r in rows[1:]], dtype=np.uint8)
    assert oracle.radial_count_pairs(4, 8, 8, 64, 2, 64) == pairs
    np.testing.assert_array_equal(oracle.build_mask_radial(4, 8, 8, 64, 64, 64, 2), mask)


def band(F, h):
    """Ordered pairs (u, w) in [0, F)^2 with |u - w| < h (h <= F)."""
    return F * (2 * h - 1) - h * (h - 1)


def closed_form_pairs(T, F, h0, beta, bk):
    tot = 0
    for d in range(T):
        kept, h = oracle.radial_window(d, h0, beta, bk)
        if kept:
            tot += (T if d == 0 else 2 * (T - d)) * band(F, min(F, h))
    return tot


@pytest.mark.parametrize("T,Hs,Ws,h0,beta,bk", [
    (6, 3, 5, 12, 2, 8), (9, 4, 4, 8, 2, 16), (11, 2, 7, 9, 3, 4), (5, 6, 6, 40, 2, 8),
    (17, 1, 9, 6, 2, 4),
])
def test_pair_count_closed_form(oracle_lib, T, Hs, Ws, h0, beta, bk):
    assert oracle.radial_count_pairs(T, Hs, Ws, h0, beta, bk) == \
        closed_form_pairs(T, Hs * Ws, h0, beta, bk)


def brute_tile_mask(T, Hs, Ws, bq, bk, h0, beta):
    F = Hs * Ws
    N = T * F
    i = np.arange(N)
    t, s = i // F, i % F
    kept = np.zeros(T, bool)
    hw = np.zeros(T, np.int64)
    for d in range(T):
        kept[d], hw[d] = oracle.radial_window(d, h0, beta, bk)
    d = np.abs(t[:, None] - t[None, :])
    pair = kept[d] & (np.abs(s[:, None] - s[None, :]) < hw[d])
    nQ, nK = -(-N // bq), -(-N // bk)
    pad = np.zeros((nQ * bq, nK * bk), bool)
    pad[:N, :N] = pair
    return pad.reshape(nQ, bq, nK, bk).any(axis=(1, 3)).astype(np.uint8)


@pytest.mark.parametrize("T,Hs,Ws,bq,bk,h0,beta", [
    (7, 5, 9, 16, 8, 12, 2), (7, 5, 9, 32, 16, 8, 2), (10, 3, 7, 16, 16, 20, 3),
    (13, 4, 5, 8, 8, 4, 2), (5, 8, 8, 64, 64, 64, 2), (9, 7, 7, 32, 8, 30, 2),
])
def test_tile_lift_equals_bruteforce_or(oracle_lib, T, Hs, Ws, bq, bk, h0, beta):
    np.testing.assert_array_equal(
        oracle.build_mask_radial(T, Hs, Ws, bq, bk, h0, beta),
        brute_tile_mask(T, Hs, Ws, bq, bk, h0, beta))


@pytest.mark.parametrize("T,m,B,h0", [(8, 4, 16, 40), (20, 5, 8, 30), (33, 3, 16, 8), (16, 6, 4, 13)])
def test_aligned_tile_count_closed_form(oracle_lib, T, m, B, h0):
    """F = m*B, Bq = Bk = B: each kept frame pair contributes m(2w-1) - w(w-1)
    tiles with w = min(m, ceil((h-1)/B) + 1)."""
    F = m * B
    mask = oracle.build_mask_radial(T, 1, F, B, B, h0, 2)
    expect = 0
    for d in range(T):
        kept, h = oracle.radial_window(d, h0, 2, B)
        if kept:
            w = min(m, -(-(h - 1) // B) + 1)
            expect += (T if d == 0 else 2 * (T - d)) * (m * (2 * w - 1) - w * (w - 1))
    assert int(mask.sum()) == expect


def test_symmetric_when_blocks_equal_and_monotone_in_window(oracle_lib):
    prev = None
    for h0 in (8, 12, 16, 24, 40, 64):
        m = oracle.build_mask_radial(9, 5, 11, 16, 16, h0, 2)
        np.testing.assert_array_equal(m, m.T)
        if prev is not None:
            assert np.all(m >= prev)
        prev = m


def test_tile_count_grows_as_n_log_n(oracle_lib):
    """Kept distances grow logarithmically in T, so kept tiles / (T log T) stays
    bounded while kept tiles / T keeps growing (unlike a fixed band)."""
    F, B, h0 = 64, 16, 32
    counts = {}
    for T in (32, 64, 128, 256, 512):
        counts[T] = int(oracle.build_mask_radial(T, 1, F, B, B, h0, 2).sum())
        nd = sum(oracle.radial_window(d, h0, 2, B)[0] for d in range(T))
        assert nd <= 4 * math.log2(T)
    per_t = [counts[T] / T for T in sorted(counts)]
    per_tlogt = [counts[T] / (T * math.log2(T)) for T in sorted(counts)]
    assert all(b > a for a, b in zip(per_t, per_t[1:]))
    assert max(per_tlogt) / min(per_tlogt) < 1.5
    # dense work grows 4x per doubling of T; here the ratio stays near
    # 2 (1 + 1/log2 T) and falls toward 2 as T grows
    ratios = [counts[2 * T] / counts[T] for T in (32, 64, 128, 256)]
    assert all(r < 2.6 for r in ratios)
    assert all(b < a for a, b in zip(ratios, ratios[1:]))
