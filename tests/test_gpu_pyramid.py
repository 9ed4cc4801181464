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
from _gpu_paths import run_pyramid
from _gpu_util import DEV, compare, dev, gather_rows, host, note, sample_rows, shape_of

pytestmark = pytest.mark.gpu


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even."""
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@pytest.mark.parametrize("L", [2, 3, 4])
def test_kv_pyramid_levels(L):
    w = synth.Workload("pyr_small", 2, 3, 128, 4, 7, 12, 64, 64, "bf16", "pooled", 640, True)
    x = synth.make_qkv(w)
    out = run_pyramid(w, x, [0.3, 0.6, 0.9, 0.95][:L])
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
@pytest.mark.parametrize("taus", [(0.4,), (0.3, 0.7), (0.2, 0.5, 0.9), (0.5, 0.5, 0.95),
                                  (0.2, 0.4, 0.7, 0.95), (0.3, 0.3, 0.6, 1.0)])
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


@pytest.mark.parametrize("group,taus", [(4, [0.2, 0.5, 1.0]), (8, [0.2, 0.4, 0.6, 1.0])])
def test_pyramid_group_constant_inputs_match_level_zero(group, taus):
    """Keys and values constant inside groups of `group` tokens: any level mix
    gives the level-0 output (consistent probabilities), on the GPU too."""
    w = synth.Workload("pyr_const", 1, 2, 128, 4, 8, 16, 128, 64, "bf16", "pooled", 642, True)
    x = synth.make_qkv(w)
    for name in ("k", "v"):
        a = x[name].reshape(w.B, w.N // group, group, w.H, w.d)
        x[name] = np.ascontiguousarray(np.repeat(a[:, :, :1], group, axis=2)
                                       .reshape(x[name].shape))
    mixed = run_pyramid(w, x, taus)
    level0 = run_pyramid(w, x, [1.0])
    assert (mixed["mask"] == len(taus)).any()        # the coarsest level is used
    d = (mixed["o"].float() - level0["o"].float()).abs()
    note(f"group-constant inputs ({group}): level mix vs level 0, max {d.max().item():.3e}")
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


@pytest.mark.parametrize("taus", [(0.3048, 0.6, 0.9), (0.25, 0.5, 0.75, 0.9)])
def test_pyramid_wan13b_480p_sampled(taus):
    w = synth.workload("wan13b_480p")
    x = synth.make_qkv(w)
    taus = list(taus)
    out = run_pyramid(w, x, taus)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=taus)
    np.testing.assert_array_equal(out["mask"], mref)
    counts = [int((mref == v).sum()) for v in range(len(taus) + 1)]
    note(f"480p tiles per mask value (dropped, level 0, 1, ...): {counts}; "
         f"{out['nnz']} augmented tiles")
    rows = sample_rows(w.B, w.H, w.nQ, 3, 41, heads=[0, 6, w.H - 1])
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK, rows=rows)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"480p pyramid {taus}")


@pytest.mark.parametrize("taus", [(0.3, 0.6, 0.9), (0.2, 0.4, 0.6, 0.9)])
def test_pyramid_head_dim_64_against_oracle(taus):
    w = synth.Workload("pyr_d64", 1, 2, 64, 4, 9, 16, 64, 64, "bf16", "pooled", 643, True)
    x = synth.make_qkv(w)
    taus = list(taus)
    out = run_pyramid(w, x, taus)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=taus)
    np.testing.assert_array_equal(out["mask"], mref)
    o_ref, lse_ref = oracle.pyramid_attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mref,
                                              w.nQ * w.nK)
    rows = np.arange(w.B * w.H * w.nQ)
    og, lg = gather_rows(host(out["o"]), host(out["lse"]), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"pyramid d=64 {taus}")


@pytest.mark.parametrize("taus", [(1.0,), (0.3, 0.6, 0.9), (0.2, 0.4, 0.6, 0.9)])
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


@pytest.mark.parametrize("taus", [(1.0,), (0.3, 0.6, 0.9), (0.2, 0.4, 0.6, 0.9)])
def test_pyramid_mask_rows_over_2048_blocks(taus):
    """Level masks over rows of 2,560 key blocks (one workgroup per row, the
    sorted walk in steps of 512), bit-exact against the oracle."""
    w = synth.Workload("pyr_very_long", 1, 1, 64, 40, 32, 128, 128, 64, "bf16", "pooled", 645,
                       True)
    assert w.nK > 2048
    x = synth.make_qkv(w)
    s = shape_of(w)
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    mask = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pyramid(s, dev(x["q"]), dev(x["k"]), w.scale, list(taus), mask, ws)
    torch.cuda.synchronize()
    got = host(mask).reshape(w.B, w.H, w.nQ, w.nK)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=list(taus))
    note(f"pyramid level mask rows of {w.nK} blocks {taus}: "
         f"{[int((mref == l).sum()) for l in range(len(taus) + 1)]} per level")
    np.testing.assert_array_equal(got, mref)


def _level_mask_gpu(w, x, taus):
    s = shape_of(w)
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    mask = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pyramid(s, dev(x["q"]), dev(x["k"]), w.scale, list(taus), mask, ws)
    torch.cuda.synchronize()
    return host(mask).reshape(w.B, w.H, w.nQ, w.nK)


@pytest.mark.parametrize("grid,Bq", [((8, 40, 40), 64), ((15, 50, 80), 128)])
@pytest.mark.parametrize("taus", [(1.0,), (0.3, 0.6, 0.9), (0.2, 0.4, 0.6, 0.9)])
def test_pyramid_mask_one_wave_rows_bit_exact(grid, Bq, taus):
    """Level masks of rows of 200 and of 938 key blocks (the last one ragged),
    where one wave sorts a whole row in registers, bit-exact against the
    oracle."""
    w = synth.Workload("pyr_wave_rows", 1, 2, 64, *grid, Bq, 64, "bf16", "pooled", 646, True)
    assert 128 < w.nK <= 1024
    x = synth.make_qkv(w)
    got = _level_mask_gpu(w, x, taus)
    ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                         levels_tau=list(taus))
    note(f"pyramid level mask, rows of {w.nK} blocks {taus}: "
         f"{[int((ref == l).sum()) for l in range(len(taus) + 1)]} per level")
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("period", [3, 7])
@pytest.mark.parametrize("taus", [(0.3, 0.6, 0.9), (0.2, 0.4, 0.6, 0.9)])
def test_pyramid_mask_tied_rows_bit_exact(period, taus):
    """Rows of 400 key blocks whose keys repeat every `period` blocks, so every
    score comes in a tie group of 57 or more blocks: tied blocks take their
    levels in ascending block order."""
    w = synth.Workload("pyr_ties", 1, 2, 64, 25, 32, 32, 128, 64, "bf16", "pooled", 647, True)
    x = synth.make_qkv(w)
    k = x["k"].reshape(w.B, w.nK, w.Bk, w.H, w.d)
    x["k"] = np.ascontiguousarray(k[:, np.arange(w.nK) % period].reshape(x["k"].shape))
    got = _level_mask_gpu(w, x, taus)
    ref, S, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                         levels_tau=list(taus), want_scores=True)
    assert np.all(S[..., period:] == S[..., :-period])   # scores repeat with the keys
    np.testing.assert_array_equal(got, ref)


def test_pyramid_forward_deterministic_run_twice():
    """Packed 16-row groups from several levels: the same inputs give the same
    O and LSE bit for bit (no float atomics on this path)."""
    w = synth.Workload("pyr_twice", 1, 2, 128, 5, 12, 16, 64, 64, "bf16", "pooled", 648, True)
    x = synth.make_qkv(w)
    taus = [0.2, 0.4, 0.7, 0.95]
    a = run_pyramid(w, x, taus)
    b = run_pyramid(w, x, taus)
    assert (a["mask"] == 4).any()
    assert torch.equal(a["o"].view(torch.int16), b["o"].view(torch.int16))
    assert torch.equal(a["lse"], b["lse"])
