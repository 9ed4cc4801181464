"""Pins for the oracle's masked attention and tile gaps (CPU only).

Each check ties the oracle to something other than itself: textbook dense
attention evaluated with matrix products and a library routine, closed forms
(constant V, identity V, zero scale), block-diagonal independence, and a
brute-force recomputation of the tile gaps from the full score matrix.
"""
import numpy as np
import pytest
import torch

import oracle


def rand_qkv(B, N, H, D, seed, dtype=np.float64):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, N, H, D)).astype(dtype)
    k = r.standard_normal((B, N, H, D)).astype(dtype)
    v = r.standard_normal((B, N, H, D)).astype(dtype)
    return q, k, v


def dense_ref(q, k, v, scale, keep=None):
    """Textbook softmax(scale Q K^T) V per (b, h) with numpy matrix products.

    keep: optional boolean [B][H][N][N] token mask. Returns o [B][H][N][D], lse [B][H][N]."""
    B, N, H, D = q.shape
    o = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, :, h, :] @ k[b, :, h, :].T)
            if keep is not None:
                s = np.where(keep[b, h], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            e = np.where(ok[:, None], np.exp(s - np.where(ok[:, None], m, 0.0)), 0.0)
            l = e.sum(axis=1)
            o[b, h, ok] = (e[ok] @ v[b, :, h, :]) / l[ok, None]
            lse[b, h, ok] = m[ok, 0] + np.log(l[ok])
    return o, lse


def oracle_full(q, k, v, bq, bk, scale, mask, head_stride):
    B, N, H, D = q.shape
    nQ = -(-N // bq)
    o, lse, _ = oracle.attention(q, k, v, bq, bk, scale, mask, head_stride)
    o = o.reshape(B, H, nQ * bq, D)[:, :, :N]
    lse = lse.reshape(B, H, nQ * bq)[:, :, :N]
    return o, lse


def token_keep(mask, B, H, N, bq, bk):
    """Expand a [B][H][nQ][nK] tile mask to a boolean [B][H][N][N] token mask."""
    rows = np.arange(N) // bq
    cols = np.arange(N) // bk
    return mask[:, :, rows][:, :, :, cols].astype(bool)


@pytest.mark.parametrize("N,bq,bk", [(64, 16, 16), (100, 32, 16), (77, 16, 32)])
def test_all_ones_equals_dense(oracle_lib, N, bq, bk):
    B, H, D = 2, 2, 8
    q, k, v = rand_qkv(B, N, H, D, seed=N)
    scale = 1 / np.sqrt(D)
    nQ, nK = -(-N // bq), -(-N // bk)
    ones = np.ones((nQ, nK), np.uint8)
    o, lse = oracle_full(q, k, v, bq, bk, scale, ones, 0)
    o_ref, lse_ref = dense_ref(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
    # library routine: torch SDPA in float64 on the CPU
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3).contiguous()
    o_t = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,bq,bk", [(96, 32, 16), (70, 16, 16)])
def test_random_mask_matches_token_masked_softmax(oracle_lib, N, bq, bk):
    B, H, D = 1, 3, 16
    q, k, v = rand_qkv(B, N, H, D, seed=7 + N)
    scale = 0.3
    nQ, nK = -(-N // bq), -(-N // bk)
    r = np.random.default_rng(5)
    mask = (r.random((B, H, nQ, nK)) < 0.4).astype(np.uint8)
    mask[0, 0, 1, :] = 0  # one empty row block
    o, lse = oracle_full(q, k, v, bq, bk, scale, mask, nQ * nK)
    o_ref, lse_ref = dense_ref(q, k, v, scale, token_keep(mask, B, H, N, bq, bk))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lse_ref))
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
    # empty row block: O = 0, LSE = -inf
    assert np.all(o[0, 0, bq:2 * bq] == 0.0)
    assert np.all(lse[0, 0, bq:2 * bq] == -np.inf)


def test_constant_v_rows_reproduce_constant(oracle_lib):
    B, N, H, D, bq, bk = 1, 80, 2, 8, 16, 16
    q, k, _ = rand_qkv(B, N, H, D, seed=3)
    c = np.linspace(-1, 2, D)
    v = np.broadcast_to(c, (B, N, H, D)).copy()
    nQ, nK = 5, 5
    mask = (np.random.default_rng(1).random((B, H, nQ, nK)) < 0.5).astype(np.uint8)
    mask[..., 0] = 1
    o, _ = oracle_full(q, k, v, bq, bk, 0.7, mask, nQ * nK)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)


def test_identity_v_gives_probabilities(oracle_lib):
    """N = D = 64, V = I: o_i is row i of the attention matrix."""
    B, N, H, D, bq, bk = 1, 64, 1, 64, 16, 16
    q, k, _ = rand_qkv(B, N, H, D, seed=11)
    v = np.eye(N)[None, :, None, :].copy()
    mask = (np.random.default_rng(2).random((B, H, 4, 4)) < 0.5).astype(np.uint8)
    mask[..., 2] = 1
    o, _ = oracle_full(q, k, v, bq, bk, 0.2, mask, 16)
    keep = token_keep(mask, B, H, N, bq, bk)[0, 0]
    P = o[0, 0]
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(P[~keep] == 0.0)
    assert np.all(P[keep] > 0.0)


def test_zero_scale_is_mean_over_kept_keys(oracle_lib):
    B, N, H, D, bq, bk = 1, 72, 2, 4, 16, 16
    q, k, v = rand_qkv(B, N, H, D, seed=4)
    nQ, nK = 5, 5
    mask = (np.random.default_rng(9).random((B, H, nQ, nK)) < 0.5).astype(np.uint8)
    mask[..., 4] = 1  # ragged last key block (8 keys) always kept
    o, lse = oracle_full(q, k, v, bq, bk, 0.0, mask, nQ * nK)
    keep = token_keep(mask, B, H, N, bq, bk)
    for h in range(H):
        for i in range(N):
            J = np.nonzero(keep[0, h, i])[0]
            np.testing.assert_allclose(o[0, h, i], v[0, J, h].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[0, h, i], np.log(len(J)), rtol=0, atol=1e-13)


def test_block_diagonal_is_independent_dense_per_block(oracle_lib):
    B, N, H, D, bq, bk = 1, 64, 2, 8, 16, 16
    q, k, v = rand_qkv(B, N, H, D, seed=8)
    mask = np.eye(4, dtype=np.uint8)
    o, lse = oracle_full(q, k, v, bq, bk, 0.5, mask, 0)
    for blk in range(4):
        sl = slice(16 * blk, 16 * blk + 16)
        o_b, lse_b = dense_ref(q[:, sl], k[:, sl], v[:, sl], 0.5)
        np.testing.assert_allclose(o[:, :, sl], o_b, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, sl], lse_b, rtol=0, atol=1e-12)


def test_single_valid_key_returns_its_value(oracle_lib):
    """Only the ragged last key block (one key) is kept: o_i = v_{N-1}."""
    B, N, H, D, bq, bk = 1, 49, 1, 8, 16, 16
    q, k, v = rand_qkv(B, N, H, D, seed=12)
    mask = np.zeros((4, 4), np.uint8)
    mask[:, 3] = 1
    o, lse = oracle_full(q, k, v, bq, bk, 0.4, mask, 0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, N - 1, 0], (N, D)), rtol=0, atol=1e-14)
    s = 0.4 * (q[0, :, 0] @ k[0, N - 1, 0])
    np.testing.assert_allclose(lse[0, 0], s, rtol=0, atol=1e-13)


def test_bf16_and_f32_inputs_widen_exactly(oracle_lib):
    from synth import f32_to_bf16_bits, bf16_bits_to_f32
    B, N, H, D, bq, bk = 1, 40, 2, 8, 16, 16
    q, k, v = rand_qkv(B, N, H, D, seed=13)
    qb, kb, vb = (f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    ones = np.ones((3, 3), np.uint8)
    o_b, _ = oracle_full(qb, kb, vb, bq, bk, 0.3, ones, 0)
    up = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    o_d, _ = oracle_full(up(qb), up(kb), up(vb), bq, bk, 0.3, ones, 0)
    np.testing.assert_array_equal(o_b, o_d)
    q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
    o_f, _ = oracle_full(q32, k32, v32, bq, bk, 0.3, ones, 0)
    o_d, _ = oracle_full(*(x.astype(np.float64) for x in (q32, k32, v32)), bq, bk, 0.3, ones, 0)
    np.testing.assert_array_equal(o_f, o_d)


# ------------------------------------------------------------------ tile gaps
def brute_gaps(q, k, scale, mask, bq, bk):
    """Gaps from the full score matrix: per-tile row maxima, running max by
    cumulative maximum over the kept tiles in ascending order."""
    B, N, H, D = q.shape
    nQ, nK = mask.shape[-2:]
    g = np.full((B, H, nQ, nK), np.nan)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, :, h, :] @ k[b, :, h, :].T)
            pad = np.full((nQ * bq, nK * bk), -np.inf)
            pad[:N, :N] = s
            tmax = pad.reshape(nQ, bq, nK, bk).max(axis=3)  # [nQ][bq][nK]
            for a in range(nQ):
                cols = np.nonzero(mask[b, h, a])[0]
                if cols.size == 0:
                    continue
                valid = min(N, (a + 1) * bq) - a * bq
                loc = tmax[a, :valid][:, cols]               # [rows][kept]
                run = np.maximum.accumulate(loc, axis=1)
                prev = np.concatenate([np.full((valid, 1), -np.inf), run[:, :-1]], axis=1)
                g[b, h, a, cols] = (loc - prev).max(axis=0)
    return g


@pytest.mark.parametrize("N,bq,bk", [(96, 32, 16), (75, 16, 16)])
def test_gaps_match_brute_force(oracle_lib, N, bq, bk):
    B, H, D = 1, 2, 16
    q, k, v = rand_qkv(B, N, H, D, seed=21 + N)
    nQ, nK = -(-N // bq), -(-N // bk)
    mask = (np.random.default_rng(N).random((B, H, nQ, nK)) < 0.6).astype(np.uint8)
    _, _, gap = oracle.attention(q, k, v, bq, bk, 0.9, mask, nQ * nK, want_gap=True)
    ref = brute_gaps(q, k, 0.9, mask, bq, bk).reshape(B * H * nQ, nK)
    np.testing.assert_array_equal(np.isnan(gap), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(gap[ok], ref[ok], rtol=0, atol=1e-12)
    # the first visited tile of every non-empty row is +inf (never marked)
    for r in range(B * H * nQ):
        cols = np.nonzero(~np.isnan(ref[r]))[0]
        if cols.size:
            assert gap[r, cols[0]] == np.inf
            assert np.all(np.isfinite(gap[r, cols[1:]]))


def test_marked_tiles_obey_the_suppression_bound(oracle_lib):
    """Every score of a tile with gap <= -tau lies at least tau below its row max."""
    B, N, H, D, bq, bk = 1, 128, 2, 16, 16, 16
    r = np.random.default_rng(31)
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    # queries aligned with u; only the first key block carries u, so later
    # tiles sit far below the running maximum set by the first one
    q = 4.0 * u + 0.3 * r.standard_normal((B, N, H, D))
    k = 0.3 * r.standard_normal((B, N, H, D))
    k[:, :bk] += 4.0 * u
    v = r.standard_normal((B, N, H, D))
    tau = 3.0
    ones = np.ones((8, 8), np.uint8)
    _, lse, gap = oracle.attention(q, k, v, bq, bk, 0.5, ones, 0, want_gap=True)
    marked = gap <= -tau
    assert marked.any()
    for row in range(B * H * 8):
        bh, a = divmod(row, 8)
        s = 0.5 * (q[0, a * bq:(a + 1) * bq, bh] @ k[0, :, bh].T)
        m = s.max(axis=1, keepdims=True)
        l = np.exp(s - m).sum(axis=1)
        for c in np.nonzero(marked[row])[0]:
            blk = s[:, c * bk:(c + 1) * bk]
            assert np.all(np.exp(blk - m) <= np.exp(-tau) * (1 + 1e-12))
            # dropping the tile moves each normalised output by <= 2|C| e^-tau max|v|
            w_drop = np.exp(blk - m).sum(axis=1) / l
            assert np.all(w_drop <= bk * np.exp(-tau))
