"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Masks and lists must match bit for bit; attention outputs within max-abs 2e-2
and mean-abs 2e-3 of the oracle (bf16 inputs), LSE within 1e-2. Small shapes
are compared in full (several tiles, ragged tails, empty rows); the
video-sized workloads at their full size on stratified row samples, which
are exact for the sampled rows.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
import oracle
import synth
from _gpu_util import (DEV, GAP_ABS, assert_all_written, compare, dev, gather_rows, host, note,
                       radial_lists, run_fwd, sample_rows, shape_of)

pytestmark = pytest.mark.gpu


def small(d, Bq, T=3, Hs=7, Ws=9, B=2, H=3, dtype="bf16", seed=500):
    return synth.Workload(f"small_d{d}_q{Bq}", B, H, d, T, Hs, Ws, Bq, 64, dtype, "ones", seed,
                          True)


# ------------------------------------------------------------------ masks
@pytest.mark.parametrize("T,Hs,Ws,Bq,h0,beta", [
    (4, 8, 8, 64, 64, 2), (7, 5, 9, 64, 40, 2), (9, 13, 11, 128, 100, 3), (30, 3, 5, 128, 32, 2),
    (21, 45, 80, 128, 512, 2), (132, 45, 80, 128, 480, 2), (21, 30, 52, 64, 256, 2),
])
def test_radial_mask_bit_exact(T, Hs, Ws, Bq, h0, beta):
    note(f"radial T={T} Hs={Hs} Ws={Ws} Bq={Bq} h0={h0} beta={beta}")
    s = bsa.shape(1, 1, 128, T, Hs, Ws, Bq)
    mask = torch.empty(s.nQ * s.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_radial(s, h0, beta, mask)
    torch.cuda.synchronize()
    ref = oracle.build_mask_radial(T, Hs, Ws, Bq, 64, h0, beta)
    np.testing.assert_array_equal(host(mask).reshape(s.nQ, s.nK), ref)


@pytest.mark.parametrize("per_head,with_skip", [(True, True), (True, False), (False, False),
                                                (False, True)])
def test_compaction_bit_exact(per_head, with_skip):
    B, H, T, Hs, Ws, Bq = 2, 3, 11, 13, 17, 64
    s = bsa.shape(B, H, 128, T, Hs, Ws, Bq)
    nQ, nK = s.nQ, s.nK
    r = np.random.default_rng(17)
    mask = (r.random((B, H, nQ, nK) if per_head else (nQ, nK)) < 0.3).astype(np.uint8)
    if per_head:
        mask[1, 2, 5] = 0
    skip = (r.random((B, H, nQ, nK)) < 0.2).astype(np.uint8) if with_skip else None
    mhs = nQ * nK if per_head else 0
    R = nQ if (not per_head and skip is None) else B * H * nQ
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv_idx = torch.empty(R * nK, dtype=torch.int32, device=DEV)
    nnz = bsa.bsa_compact_block_lists(s, dev(mask), mhs, dev(skip) if skip is not None else None,
                                      row_ptr, kv_idx, want_nnz=True)
    torch.cuda.synchronize()
    Bo, Ho = (B, H) if R != nQ else (1, 1)
    rp_ref, kv_ref = oracle.compact(mask, Bo, Ho, nQ, nK, mhs if R != nQ else 0, skip)
    np.testing.assert_array_equal(host(row_ptr), rp_ref)
    assert nnz == kv_ref.size
    np.testing.assert_array_equal(host(kv_idx)[:nnz], kv_ref)
    # capacity error reports the needed size and leaves kv_idx alone
    with pytest.raises(bsa.BsaError) as ei:
        bsa.bsa_compact_block_lists(s, dev(mask), mhs, dev(skip) if skip is not None else None,
                                    row_ptr, kv_idx, kv_capacity=nnz - 1, want_nnz=True)
    assert ei.value.status == 3


# -------------------------------------------------------------- attention
def _random_lists(w, seed, density=0.35, empty_row=True):
    r = np.random.default_rng(seed)
    mask = (r.random((w.B, w.H, w.nQ, w.nK)) < density).astype(np.uint8)
    if empty_row:
        mask[0, 1, w.nQ // 2] = 0
    mask[..., w.nK - 1] |= (r.random((w.B, w.H, w.nQ)) < 0.5).astype(np.uint8)  # ragged key block
    return mask


@pytest.mark.parametrize("d,Bq", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("mode", ["per_head", "shared", "dense"])
def test_fwd_bf16_small_full_compare(d, Bq, mode):
    w = small(d, Bq)
    note(f"fwd bf16 d={d} Bq={Bq} mode={mode} N={w.N}")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    if mode == "dense":
        mask_np, mhs, rp, kv, shared = np.ones((w.nQ, w.nK), np.uint8), 0, None, None, 0
    elif mode == "shared":
        mask_np = _random_lists(w, 3)[0, 0]
        mhs, shared = 0, 1
    else:
        mask_np, mhs, shared = _random_lists(w, 4), w.nQ * w.nK, 0
    if mode != "dense":
        R = w.nQ if shared else w.B * w.H * w.nQ
        rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
        kv = torch.empty(R * w.nK, dtype=torch.int32, device=DEV)
        bsa.bsa_compact_block_lists(s, dev(mask_np), mhs, None, rp, kv)
    o, lse, _ = run_fwd(s, q, k, v, rp, kv, shared, w.scale)
    assert_all_written(s, o, lse, rp, shared, f"d={d} Bq={Bq} {mode}")
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mask_np, mhs)
    rows = np.arange(w.B * w.H * w.nQ)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"d={d} Bq={Bq} {mode}")


def test_fwd_bf16_deterministic_run_twice():
    w = small(128, 128, T=5, Hs=9, Ws=13)
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    _, rp, kv = radial_lists(s, 48)
    o1, l1, _ = run_fwd(s, q, k, v, rp, kv, 1, w.scale)
    o2, l2, _ = run_fwd(s, q, k, v, rp, kv, 1, w.scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_fwd_f32_tiny_radial_and_dense():
    w = synth.workload("tiny")
    note(f"tiny fp32 workload N={w.N}")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    mask, rp, kv = radial_lists(s, w.h0, w.beta)
    ref_mask = oracle.build_mask_radial(w.T, w.Hs, w.Ws, w.Bq, w.Bk, w.h0, w.beta)
    np.testing.assert_array_equal(host(mask).reshape(w.nQ, w.nK), ref_mask)
    rows = np.arange(w.B * w.H * w.nQ)
    for label, m, r_, k_, sh in (("radial", ref_mask, rp, kv, 1),
                                 ("dense", np.ones_like(ref_mask), None, None, 0)):
        o, lse, _ = run_fwd(s, q, k, v, r_, k_, sh, w.scale)
        o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, m, 0)
        og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
        _, mean_abs, _ = compare(og, lg, o_ref, lse_ref, f"tiny fp32 {label}")
        assert mean_abs < 1e-5  # fp32 path: far inside the bf16 bound


def test_fwd_f32_small_ragged():
    w = small(128, 64, dtype="f32", T=2, Hs=9, Ws=11, H=2)
    x = synth.make_qkv(w)
    s = shape_of(w)
    mask_np = _random_lists(w, 8)
    rp = torch.empty(w.B * w.H * w.nQ + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, dev(mask_np), w.nQ * w.nK, None, rp, kv)
    o, lse, _ = run_fwd(s, dev(x["q"]), dev(x["k"]), dev(x["v"]), rp, kv, 0, w.scale)
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mask_np,
                                         w.nQ * w.nK)
    og, lg = gather_rows(host(o), host(lse), np.arange(w.B * w.H * w.nQ), w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, "small fp32 per-head")


# ---------------------------------------------------------- full workloads
def _full_radial(name, per_head, seed):
    w = synth.workload(name)
    note(f"{name}: generating {w.B}x{w.N}x{w.H}x{w.d} bf16 inputs")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    mask, rp, kv = radial_lists(s, w.h0, w.beta)
    ref_mask = oracle.build_mask_radial(w.T, w.Hs, w.Ws, w.Bq, w.Bk, w.h0, w.beta)
    np.testing.assert_array_equal(host(mask).reshape(w.nQ, w.nK), ref_mask)
    rp_ref, kv_ref = oracle.compact(ref_mask, 1, 1, w.nQ, w.nK, 0)
    np.testing.assert_array_equal(host(rp), rp_ref)
    np.testing.assert_array_equal(host(kv)[:kv_ref.size], kv_ref)
    note(f"{name}: masks and lists bit-exact ({kv_ref.size} tiles per head)")
    o, lse, _ = run_fwd(s, q, k, v, rp, kv, 1, w.scale)
    # the position-major workgroup order covers every row block of every head
    assert_all_written(s, o, lse, rp, 1, name)
    heads = sorted({0, w.H - 1, w.H // 2})
    F_blocks = [a for a in range(1, w.nQ) if (a * w.Bq) // w.F != ((a + 1) * w.Bq - 1) // w.F]
    rows = sample_rows(w.B, w.H, w.nQ, per_head, seed, heads=heads, extra=F_blocks[:2])
    note(f"{name}: oracle on {len(rows)} sampled row blocks")
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, ref_mask,
                                         0, rows=rows)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"{name} sampled")


def test_fwd_wan14b_720p_radial_sampled():
    _full_radial("wan14b_720p", per_head=4, seed=3)


def test_fwd_all_rows_empty():
    """Every list empty: O = 0 and LSE = -inf everywhere, for both row-block sizes."""
    for Bq in (64, 128):
        w = small(128, Bq, T=2, Hs=5, Ws=7, B=1, H=2)
        x = synth.make_qkv(w)
        s = shape_of(w)
        R = w.B * w.H * w.nQ
        rp = torch.zeros(R + 1, dtype=torch.int32, device=DEV)
        kv = torch.zeros(1, dtype=torch.int32, device=DEV)
        o, lse, gap = run_fwd(s, dev(x["q"]), dev(x["k"]), dev(x["v"]), rp, kv, 0, w.scale,
                              gap_len=1)
        assert torch.count_nonzero(o.float()).item() == 0
        assert bool(torch.all(torch.isneginf(lse)))


@pytest.mark.parametrize("Bq", [64, 128])
def test_fwd_zero_scale_ragged(Bq):
    """scale = 0: uniform weights over each row's listed keys, ragged last block included."""
    w = small(128, Bq, T=3, Hs=7, Ws=9, B=1, H=2)
    x = synth.make_qkv(w)
    s = shape_of(w)
    mask_np = _random_lists(w, 11)
    mask_np[..., w.nK - 1] = 1
    rp = torch.empty(w.B * w.H * w.nQ + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, dev(mask_np), w.nQ * w.nK, None, rp, kv)
    o, lse, _ = run_fwd(s, dev(x["q"]), dev(x["k"]), dev(x["v"]), rp, kv, 0, 0.0)
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, 0.0, mask_np,
                                         w.nQ * w.nK)
    og, lg = gather_rows(host(o), host(lse), np.arange(w.B * w.H * w.nQ), w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"zero scale Bq={Bq}")
