"""Whole GPU paths shared by several parity tests: the pyramid pipeline
(levels, level mask, lists, forward) and the carried skip set over denoising
steps, each checked against the oracle as it runs. No attention arithmetic
lives here; the oracle supplies every expected value."""
import math

import numpy as np
import torch

import block_sparse_attention_flashattention_amd as bsa
import oracle
import synth
from _gpu_util import (DEV, GAP_ABS, assert_all_written, compare, dev, gather_rows, host, note,
                       shape_of)

LOG2E = 1.4426950408889634


def run_pyramid(w, x, taus, rows=None):
    """GPU pipeline: levels of K/V, level mask, lists, forward."""
    s = shape_of(w)
    L = len(taus)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    prow = bsa.bsa_pyramid_rows(s, L)
    kp = torch.zeros((w.B, max(prow, 1), w.H, w.d), dtype=q.dtype, device=DEV)
    vp = torch.zeros_like(kp)
    bsa.bsa_build_kv_pyramid(s, L, k, v, kp, vp)
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    R = w.B * w.H * w.nQ
    mask = torch.empty(R * w.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pyramid(s, q, k, w.scale, taus, mask, ws)
    rb, _ = oracle.pyramid_regions(w.N, w.Bk, L)
    cap = R * int(rb[-1])
    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(cap, dtype=torch.int32, device=DEV)
    qm = torch.empty(cap, dtype=torch.int32, device=DEV)
    nnz = bsa.bsa_compact_pyramid_lists(s, L, mask, w.nQ * w.nK, rp, kv, qm, want_nnz=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((R * w.Bq,), float("nan"), dtype=torch.float32, device=DEV)[: w.B * w.H * w.N]
    bsa.bsa_pyramid_attn_fwd(s, q, k, v, kp, vp, L, o, lse, rp, kv, qm, w.scale)
    torch.cuda.synchronize()
    assert_all_written(s, o, lse, rp, 0, f"pyramid {w.name} {L} levels")
    return dict(kp=kp, vp=vp, mask=host(mask).reshape(w.B, w.H, w.nQ, w.nK), rp=host(rp),
                kv=host(kv)[:nnz], qm=host(qm)[:nnz], o=o, lse=lse, nnz=nnz, prow=prow)


def gap_matrix(gap_list, rp, kv, R, nK):
    """List-ordered gaps -> [R][nK] (NaN where no tile was listed)."""
    out = np.full((R, nK), np.nan)
    for r in range(R):
        e0, e1 = rp[r], rp[r + 1]
        out[r, kv[e0:e1]] = gap_list[e0:e1]
    return out


def skip_carry(w, steps, tau, rows=None, order=bsa.ORDER_ASCENDING, freeze_after=None):
    """Run `steps` denoising steps of the carried skip mask on the GPU and check
    each against the oracle. `tau` is one threshold or one per step; `order`
    the visiting order of each row's list; from step `freeze_after` on, the
    skip set is shared unchanged (no gaps, no update)."""
    s = shape_of(w)
    R = w.B * w.H * w.nQ
    nK = w.nK
    x0 = synth.make_qkv(w, step=0)
    v_np = x0["v"]
    v = dev(v_np)
    ones = torch.ones(w.nQ * nK, dtype=torch.uint8, device=DEV)
    skip = torch.zeros(R * nK, dtype=torch.uint8, device=DEV)
    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv_asc = torch.empty(R * nK, dtype=torch.int32, device=DEV)
    kv = torch.empty(R * nK, dtype=torch.int32, device=DEV)
    gap = torch.empty(R * nK, dtype=torch.float32, device=DEV)
    taus = list(tau) if isinstance(tau, (list, tuple)) else [tau] * steps
    for st in range(steps):
        frozen = freeze_after is not None and st >= freeze_after
        tau_s = taus[st]
        tau2 = np.float32(np.float64(tau_s) * LOG2E)
        x = x0 if st == 0 else synth.make_step_qk(w, st)
        q, k = dev(x["q"]), dev(x["k"])
        skip_prev = host(skip).reshape(R, nK).copy()
        nnz = bsa.bsa_compact_block_lists(s, ones, 0, skip, rp, kv_asc, want_nnz=True)
        bsa.bsa_order_block_lists(s, order, rp, 0, kv_asc, kv)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.B * w.H * w.N,), float("nan"), dtype=torch.float32, device=DEV)
        bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, rp, kv, 0, w.scale, None if frozen else gap)
        if not frozen:
            bsa.bsa_update_skip_mask(s, rp, kv, gap, tau_s, skip)
        torch.cuda.synchronize()
        assert_all_written(s, o, lse, rp, 0, f"{w.name} step {st}")
        rp_h, kv_h = host(rp).astype(np.int64), host(kv)[:nnz]
        skip_new = host(skip).reshape(R, nK)
        # lists are the complement of the carried set, in the requested order
        rp_ref, kv_ref = oracle.compact(np.ones((w.nQ, nK), np.uint8), w.B, w.H, w.nQ, nK, 0,
                                        skip_prev.reshape(w.B, w.H, w.nQ, nK))
        np.testing.assert_array_equal(rp_h, rp_ref)
        np.testing.assert_array_equal(kv_h, oracle.order_lists(rp_ref, kv_ref, w.N, w.Bq, w.Bk,
                                                               order))
        sel = np.arange(R) if rows is None else rows
        if frozen:
            np.testing.assert_array_equal(skip_new, skip_prev)
            eff = (1 - skip_prev).reshape(w.B, w.H, w.nQ, nK)
            o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], v_np, w.Bq, w.Bk, w.scale, eff,
                                                 w.nQ * nK, rows=sel)
            og, lg = gather_rows(host(o), host(lse), sel, w.B, w.H, w.N, w.Bq)
            compare(og, lg, o_ref, lse_ref, f"{w.name} step {st} (shared mask)")
            continue
        gap_h = host(gap)[:nnz].astype(np.float32)
        # update rule, bit-exact on the GPU's own gaps in fp32 / log2 units
        gm = gap_matrix(gap_h, rp_h, kv_h, R, nK)
        expect = skip_prev | (np.nan_to_num(gm, nan=np.inf) <= -tau2).astype(np.uint8)
        np.testing.assert_array_equal(skip_new, expect)
        assert np.all(skip_new >= skip_prev), "skip set must only grow"
        # against the oracle (fp64): outputs, gaps, decisions
        o_ref, lse_ref, gap_ref, skip_ref = oracle.skip_step(
            x["q"], x["k"], v_np, w.Bq, w.Bk, w.scale, skip_prev.reshape(w.B, w.H, w.nQ, nK),
            tau_s, rows=sel, order=order)
        og, lg = gather_rows(host(o), host(lse), sel, w.B, w.H, w.N, w.Bq)
        compare(og, lg, o_ref, lse_ref, f"{w.name} step {st}")
        g_gpu = gm[sel] * math.log(2.0)
        fin = np.isfinite(gap_ref) & np.isfinite(g_gpu)
        assert np.array_equal(np.isnan(gap_ref), np.isnan(gm[sel])), "visited tiles differ"
        assert np.array_equal(np.isposinf(gap_ref), np.isposinf(g_gpu)), "first-tile pattern"
        gerr = float(np.abs(g_gpu[fin] - gap_ref[fin]).max()) if fin.any() else 0.0
        dec_gpu = skip_new[sel]
        dec_ref = skip_ref.reshape(R, nK)[sel]
        flips = np.argwhere(dec_gpu != dec_ref)
        for r_, c_ in flips:
            assert abs(gap_ref[r_, c_] + tau_s) <= GAP_ABS, \
                "decision differs away from the threshold"
        note(f"{w.name} step {st} (order {order}, tau {tau_s}): {nnz} tiles, "
             f"{int(skip_new.sum())} skipped, gap max err {gerr:.2e}, "
             f"{len(flips)} threshold-edge flips")
        assert gerr <= GAP_ABS
    return int(skip_new.sum())
