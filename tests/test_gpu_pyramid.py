"""GPU parity for pyramid attention, through the C ABI.

Pyramid Sparse Attention page: pooled key/value levels, a level per block
pair by thresholds, consistent probabilities, logical blocks decoupled from
hardware tiles. Level masks and tile lists are integer decisions on fp64
scores computed in the same order on both sides and must match bit for bit;
pooled keys/values are the fp32 mean rounded to bf16 (checked against the
oracle's fp64 mean within one bf16 step); outputs within the attention bounds
of the oracle, whose pooled keys are exact fp64 means.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
import oracle
import synth
from _gpu_util import DEV, compare, dev, gather_rows, host, note, sample_rows, shape_of

pytestmark = pytest.mark.gpu


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even."""
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


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
    o = torch.empty_like(q)
    lse = torch.empty(R * w.Bq, dtype=torch.float32, device=DEV)[: w.B * w.H * w.N]
    bsa.bsa_pyramid_attn_fwd(s, q, k, v, kp, vp, L, o, lse, rp, kv, qm, w.scale)
    torch.cuda.synchronize()
    return dict(kp=kp, vp=vp, mask=host(mask).reshape(w.B, w.H, w.nQ, w.nK), rp=host(rp),
                kv=host(kv)[:nnz], qm=host(qm)[:nnz], o=o, lse=lse, nnz=nnz, prow=prow)


@pytest.mark.parametrize("L", [2, 3])
def test_kv_pyramid_levels(L):
    w = synth.Workload("pyr_small", 2, 3, 128, 4, 7, 12, 64, 64, "bf16", "pooled", 640, True)
    x = synth.make_qkv(w)
    out = run_pyramid(w, x, [0.3, 0.6, 0.9][:L])
    rb, rr = oracle.pyramid_regions(w.N, w.Bk, L)
    for name, t in (("k", out["kp"]), ("v", out["vp"])):
        src = x[name].view(np.uint16).astype(np.uint32) << 16
        src = src.view(np.float32).astype(np.float64)       # exact bf16 values
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
        for l in range(1, L):
            g = w.N >> l
            mean = src.reshape(w.B, g, 1 << l, w.H, w.d).mean(axis=2)
            want = bf16_bits(mean.astype(np.float32))
            row0 = (rb[l] - rb[1]) * w.Bk
            diff = np.abs(got[:, row0:row0 + g].astype(np.int32) - want.astype(np.int32))
            assert diff.max() <= 1, f"{name} level {l}: {diff.max()} bf16 steps"
            note(f"{name} level {l}: {int((diff == 0).mean() * 100)}% exact, "
                 f"max {diff.max()} bf16 step")


@pytest.mark.parametrize("Bq", [64, 128])
@pytest.mark.parametrize("taus", [(0.4,), (0.3, 0.7), (0.2, 0.5, 0.9), (0.5, 0.5, 0.95)])
def test_pyramid_small_against_oracle(Bq, taus):
    w = synth.Workload("pyr_small", 2, 3, 128, 5, 12, 16, Bq, 64, "bf16", "pooled", 641, True)
    x = synth.make_qkv(w)
    note(f"pyramid small Bq={Bq} taus={taus} N={w.N}")
    out = run_pyramid(w, x, list(taus))
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=list(taus))
    np.testing.assert_array_equal(out["mask"], mref)
    rp, kv, qm = oracle.compact_pyramid(mref, w.B, w.H, w.nQ, w.nK, w.N, w.Bk, len(taus),
                                        w.nQ * w.nK)
    np.testing.assert_array_equal(out["rp"], rp)
    np.testing.assert_array_equal(out["kv"], kv)
    np.testing.assert_array_equal(out["qm"], qm)
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK)
    rows = np.arange(w.B * w.H * w.nQ)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"pyramid small Bq={Bq} {taus}")


def test_pyramid_group_constant_inputs_match_level_zero():
    """Keys and values constant inside groups of 4 tokens: any level mix gives
    the level-0 output (consistent probabilities), on the GPU too."""
    w = synth.Workload("pyr_const", 1, 2, 128, 4, 8, 16, 128, 64, "bf16", "pooled", 642, True)
    x = synth.make_qkv(w)
    for name in ("k", "v"):
        a = x[name].reshape(w.B, w.N // 4, 4, w.H, w.d)
        x[name] = np.ascontiguousarray(np.repeat(a[:, :, :1], 4, axis=2).reshape(x[name].shape))
    mixed = run_pyramid(w, x, [0.2, 0.5, 1.0])
    level0 = run_pyramid(w, x, [1.0])
    assert (mixed["mask"] > 1).any()
    d = (mixed["o"].float() - level0["o"].float()).abs()
    note(f"group-constant inputs: level mix vs level 0, max {d.max().item():.3e}")
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


def test_pyramid_wan13b_480p_sampled():
    w = synth.workload("wan13b_480p")
    x = synth.make_qkv(w)
    taus = [0.3048, 0.6, 0.9]
    out = run_pyramid(w, x, taus)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=taus)
    np.testing.assert_array_equal(out["mask"], mref)
    counts = [int((mref == v).sum()) for v in range(4)]
    note(f"480p levels (dropped, l0, l1, l2): {counts}; {out['nnz']} augmented tiles")
    rows = sample_rows(w.B, w.H, w.nQ, 3, 41, heads=[0, 6, w.H - 1])
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK, rows=rows)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, "480p pyramid")


def test_pyramid_head_dim_64_against_oracle():
    w = synth.Workload("pyr_d64", 1, 2, 64, 4, 9, 16, 64, 64, "bf16", "pooled", 643, True)
    x = synth.make_qkv(w)
    taus = [0.3, 0.6, 0.9]
    out = run_pyramid(w, x, taus)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=taus)
    np.testing.assert_array_equal(out["mask"], mref)
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK)
    rows = np.arange(w.B * w.H * w.nQ)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, "pyramid d=64")


@pytest.mark.parametrize("taus", [(1.0,), (0.3, 0.6, 0.9)])
def test_pyramid_long_rows_sampled(taus):
    """720p grid, one head at d = 64, row blocks of 64: with tau = 1 every row
    lists all 1,182 key blocks, more than the forward's list of non-empty half
    steps holds, so it steps through every half; with three levels the rows
    are shorter and the empty halves are left out. Sampled rows."""
    w = synth.Workload("pyr_long", 1, 1, 64, 21, 45, 80, 64, 64, "bf16", "pooled", 644, True)
    x = synth.make_qkv(w)
    out = run_pyramid(w, x, list(taus))
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=list(taus))
    np.testing.assert_array_equal(out["mask"], mref)
    lens = np.diff(out["rp"])
    note(f"pyramid long rows {taus}: entries per row {lens.min()}..{lens.max()}")
    if taus == (1.0,):
        assert lens.min() > 1023
    rows = sample_rows(w.B, w.H, w.nQ, 6, 45)
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK, rows=rows)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"pyramid long rows {taus}")
