"""GPU parity for the dynamic mask builders and the step carry, through the C ABI.

Pooled masks are decided by comparisons on fp64 pooled scores that both sides
compute in the same fixed order, so the masks must match bit for bit. The
skip carry is checked per denoising step: outputs within the attention bounds,
tile gaps within 1e-3 of the oracle's, the update's decisions bit-exact
against the rule applied to the GPU's own gaps in the kernel's precision
(fp32, log2 units), and the skip set only grows. Where the oracle's fp64
decision differs, the gap must sit within the gap tolerance of the threshold.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
import oracle
import synth
from _gpu_paths import skip_carry as _skip_carry
from _gpu_util import (DEV, assert_all_written, compare, dev, gather_rows, host, note,
                       radial_lists, run_fwd, sample_rows, shape_of)

pytestmark = pytest.mark.gpu



def _pooled_gpu(w, x, mode, param):
    s = shape_of(w)
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    mask = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pooled(s, dev(x["q"]), dev(x["k"]), w.scale, mode, param, mask, ws)
    torch.cuda.synchronize()
    return host(mask).reshape(w.B, w.H, w.nQ, w.nK)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Bq", [64, 128])
@pytest.mark.parametrize("mode,param", [(0, 1.0), (0, 4.0), (1, 0.5), (1, 0.9), (1, 1.0)])
def test_pooled_mask_small_bit_exact(dtype, Bq, mode, param):
    w = synth.Workload("pooled_small", 2, 3, 128, 5, 12, 17, Bq, 64, dtype, "pooled", 610, True)
    note(f"pooled small {dtype} Bq={Bq} mode={mode} param={param} N={w.N}")
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    np.testing.assert_array_equal(got, ref)
    if mode == 0:
        assert np.all(got.sum(-1) == min(int(param), w.nK))


def test_pooled_mask_d64_bit_exact():
    w = synth.Workload("pooled_d64", 1, 2, 64, 4, 9, 14, 64, 64, "bf16", "pooled", 611, True)
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, 1, 0.7)
    ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 1, 0.7)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("mode,param", [(0, 300.0), (1, 0.5), (1, 0.95)])
def test_pooled_mask_long_rows_bit_exact(mode, param):
    """720p grid, one head at d = 64: rows of 1,182 key blocks, so the row
    sort runs 2,048 keys over four waves, several pairs per lane."""
    w = synth.Workload("pooled_long", 1, 1, 64, 21, 45, 80, 128, 64, "bf16", "pooled", 612, True)
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    note(f"pooled long rows mode={mode} param={param}: {int(ref.sum())} kept of {ref.size}")
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("period,mode,param", [(7, 0, 77.0), (7, 0, 300.0), (7, 1, 0.3),
                                               (7, 1, 0.95), (3, 0, 77.0), (3, 1, 0.3)])
def test_pooled_mask_long_rows_ties_bit_exact(period, mode, param):
    """Rows of 400 key blocks in which the keys repeat every `period` blocks,
    so every score comes in a tie group of 57 or 58 blocks (period 7) or of
    133 or 134 (period 3, more than one wave of candidates with the cut key):
    the k-th or 128th pair of a row falls inside a tie group, the radix
    select ends with equal keys among its last candidates, and the long-row
    paths must take tied blocks in ascending order (top-k directly,
    cumulative mass through the full sort)."""
    w = synth.Workload("pooled_ties_long", 1, 2, 64, 25, 32, 32, 128, 64, "bf16", "pooled", 614,
                       True)
    x = synth.make_qkv(w)
    k = x["k"].reshape(w.B, w.nK, w.Bk, w.H, w.d)
    x["k"] = np.ascontiguousarray(k[:, np.arange(w.nK) % period].reshape(x["k"].shape))
    got = _pooled_gpu(w, x, mode, param)
    ref, S, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param,
                                         want_scores=True)
    assert np.all(S[..., period:] == S[..., :-period])   # scores repeat with the keys
    note(f"pooled tied long rows period={period} mode={mode} param={param}: "
         f"{int(ref.sum())} kept")
    np.testing.assert_array_equal(got, ref)


# Rows longer than the in-LDS select holds (nK > 2048) take one workgroup
# per row: N = 163,840 tokens, 1,280 row blocks of 2,560 key blocks.
def _very_long():
    return synth.Workload("pooled_very_long", 1, 1, 64, 40, 32, 128, 128, 64, "bf16", "pooled",
                          615, True)


@pytest.mark.parametrize("mode,param", [(0, 300.0), (0, 2000.0), (1, 0.3), (1, 0.95), (1, 1.0)])
def test_pooled_mask_rows_over_2048_blocks_bit_exact(mode, param):
    """Top-k and cumulative mass over rows of 2,560 key blocks; the mass walk
    takes the sorted pairs in steps of 512 (tau 0.95 and 1.0 need several)."""
    w = _very_long()
    assert w.nK > 2048
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    note(f"pooled rows of {w.nK} blocks mode={mode} param={param}: {int(ref.sum())} kept")
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("period,mode,param", [(2, 0, 77.0), (2, 1, 0.3), (3, 1, 0.6)])
def test_pooled_mask_rows_over_2048_blocks_ties_bit_exact(period, mode, param):
    """Rows of 2,560 key blocks whose keys repeat every 2 or 3 blocks: tie
    groups of 1,280 or 853-854 blocks, longer than one LDS step of the walk
    for period 2, taken in ascending block order."""
    w = _very_long()
    x = synth.make_qkv(w)
    k = x["k"].reshape(w.B, w.nK, w.Bk, w.H, w.d)
    x["k"] = np.ascontiguousarray(k[:, np.arange(w.nK) % period].reshape(x["k"].shape))
    got = _pooled_gpu(w, x, mode, param)
    ref, S, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param,
                                         want_scores=True)
    assert np.all(S[..., period:] == S[..., :-period])
    note(f"pooled tied rows of {w.nK} blocks period={period} mode={mode}: {int(ref.sum())} kept")
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("mode,param", [(2, 40000.0), (3, 0.3)])
def test_pooled_global_rows_over_2048_blocks(mode, param):
    """Head-wide selection over rows of 2,560 key blocks (row statistics one
    lane per row, probabilities elementwise)."""
    w = _very_long()
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    note(f"head-wide rows of {w.nK} blocks mode={mode}: {int(ref.sum())} kept, "
         f"{int(np.sum(got != ref))} differ, head margin {margin[:, :, 0].min():.3e}")
    _check_global(got, ref, margin, mode, "rows over 2048 blocks")


def test_pooled_mask_wan13b_480p_full():
    w = synth.workload("wan13b_480p")
    note(f"{w.name}: generating inputs")
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, w.pooled_mode, w.pooled_param)
    ref, _, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale,
                                              w.pooled_mode, w.pooled_param)
    diff = int(np.sum(got != ref))
    note(f"{w.name}: {ref.sum()} kept tiles ({100 * (1 - ref.mean()):.1f}% sparse), "
         f"{diff} differ; smallest selection margin {margin.min():.3e}")
    np.testing.assert_array_equal(got, ref)
    assert 0.80 < 1 - ref.mean() < 0.90


def test_pooled_then_forward_wan13b_480p_sampled():
    """The pooled builder feeding compaction and the Bq = 64 forward, end to end."""
    w = synth.workload("wan13b_480p")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    R = w.B * w.H * w.nQ
    mask = torch.empty(R * w.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pooled(s, q, k, w.scale, w.pooled_mode, w.pooled_param, mask, ws)
    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(R * w.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, mask, w.nQ * w.nK, None, rp, kv)
    o, lse, _ = run_fwd(s, q, k, v, rp, kv, 0, w.scale)
    assert_all_written(s, o, lse, rp, 0, "480p pooled")
    mask_h = host(mask).reshape(w.B, w.H, w.nQ, w.nK)
    rows = sample_rows(w.B, w.H, w.nQ, 3, 21, heads=[0, 5, w.H - 1])
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mask_h,
                                         w.nQ * w.nK, rows=rows)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"{w.name} pooled sampled")


# ----------------------------------------------------- head-wide selection
def _check_global(got, ref, margin, mode, label):
    """Top-k (mode 2) decides on exact integers and must match bit for bit; the
    mass rule (mode 3) may differ only in a head whose prefix sum lies within
    rounding of its target (the GPU sums the mass in a fixed parallel order)."""
    B, H = ref.shape[:2]
    for b in range(B):
        for h in range(H):
            if np.array_equal(got[b, h], ref[b, h]):
                continue
            assert mode == 3 and margin[b, h, 0] < 1e-9, \
                f"{label}: head ({b}, {h}) differs, margin {margin[b, h, 0]:.3e}"
    assert np.all(got.sum(-1) >= 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Bq", [64, 128])
@pytest.mark.parametrize("mode,param", [(2, 1.0), (2, 37.0), (2, 10 ** 6), (3, 0.05), (3, 0.3),
                                        (3, 0.8), (3, 1.0)])
def test_pooled_global_small_bit_exact(dtype, Bq, mode, param):
    w = synth.Workload("pooled_small", 2, 3, 128, 5, 12, 17, Bq, 64, dtype, "pooled", 612, True)
    note(f"pooled head-wide {dtype} Bq={Bq} mode={mode} param={param} N={w.N}")
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    _check_global(got, ref, margin, mode, "small")
    np.testing.assert_array_equal(got, ref)


def test_pooled_global_ties_bit_exact():
    """Equal key blocks give equal scores across whole rows: the cut falls
    inside a tie group and must take the lower pair indices first."""
    w = synth.Workload("pooled_ties", 1, 2, 64, 2, 8, 16, 64, 64, "f32", "pooled", 613, True)
    x = synth.make_qkv(w)
    k = x["k"].copy()
    k[:, 64:] = np.tile(k[:, :64], (1, (w.N - 64) // 64 + 1, 1, 1))[:, :w.N - 64]
    x = dict(x, k=np.ascontiguousarray(k))
    for mode, param in ((2, 5.0), (2, 3.0), (3, 0.4)):
        got = _pooled_gpu(w, x, mode, param)
        ref, S, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode,
                                                  param, want_scores=True)
        assert np.all(S[..., :1] == S)          # every block of a row ties
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("mode,param", [(2, 39322.0), (3, 0.5)])
def test_pooled_global_wan13b_480p_full(mode, param):
    w = synth.workload("wan13b_480p")
    x = synth.make_qkv(w)
    got = _pooled_gpu(w, x, mode, param)
    ref, _, margin = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
    diff = int(np.sum(got != ref))
    note(f"{w.name} head-wide mode {mode} param {param}: {int(ref.sum())} kept "
         f"({100 * (1 - ref.mean()):.1f}% sparse), {diff} differ; smallest head margin "
         f"{margin[:, :, 0].min():.3e}; kept per head {ref.sum(axis=(2, 3)).ravel().tolist()}")
    _check_global(got, ref, margin, mode, w.name)


# ---------------------------------------------------------------- skip carry
# Thresholds here are set from these inputs' gap distribution (most gaps lie
# in [-4, 0] natural-log units) so that tiles are actually marked and carried;
# at the workload's own tau = 10 nothing is marked (checked last).
def test_skip_carry_small_steps():
    w = synth.Workload("skip_small", 1, 3, 128, 6, 10, 14, 64, 64, "bf16", "skip", 620, True,
                       tau=1.0, steps=5)
    _skip_carry(w, w.steps, w.tau)


def test_skip_carry_small_bq128_ragged():
    w = synth.Workload("skip_small128", 2, 2, 64, 5, 9, 13, 128, 64, "bf16", "skip", 621, True,
                       tau=0.25, steps=4)
    _skip_carry(w, w.steps, w.tau)


@pytest.mark.parametrize("Bq", [64, 128])
def test_skip_carry_gap_batches_with_remainder(Bq):
    """Lists of 71 entries (a ragged 20-key last block): the kernel folds the
    gaps of 64 consecutive entries per atomic, so every row has one full batch
    and a 7-entry remainder; all rows are checked."""
    w = synth.Workload("skip_batches", 1, 1, 64, 5, 30, 30, Bq, 64, "bf16", "skip", 623, True,
                       tau=1.0, steps=2)
    assert w.nK == 71 and w.N % 64 == 20
    _skip_carry(w, w.steps, w.tau)


def test_skip_carry_480p_sampled():
    """All ten denoising steps of the 480p carry (sigma 0.5 -> 0.05), each
    checked against the oracle from the GPU's previous skip set."""
    w = synth.workload("skip_carry_480p")
    rows = sample_rows(w.B, w.H, w.nQ, 2, 23, heads=[0, w.H - 1])
    _skip_carry(w, w.steps, 2.0, rows=rows)


def test_skip_carry_480p_workload_tau_marks_nothing():
    w = synth.workload("skip_carry_480p")
    rows = sample_rows(w.B, w.H, w.nQ, 1, 24, heads=[3])
    marked = _skip_carry(w, 2, w.tau, rows=rows)
    assert marked == 0


# ------------------------------------------- visiting order and schedules
def test_skip_carry_small_radial_order():
    w = synth.Workload("skip_small", 1, 3, 128, 6, 10, 14, 64, 64, "bf16", "skip", 620, True,
                       tau=1.0, steps=5)
    _skip_carry(w, w.steps, w.tau, order=bsa.ORDER_RADIAL)


def test_skip_carry_small_bq128_ragged_radial_order():
    w = synth.Workload("skip_small128", 2, 2, 64, 5, 9, 13, 128, 64, "bf16", "skip", 621, True,
                       tau=0.25, steps=4)
    _skip_carry(w, w.steps, w.tau, order=bsa.ORDER_RADIAL)


def test_skip_carry_480p_sampled_radial_order():
    w = synth.workload("skip_carry_480p")
    rows = sample_rows(w.B, w.H, w.nQ, 2, 25, heads=[0, w.H - 1])
    _skip_carry(w, w.steps, 2.0, rows=rows, order=bsa.ORDER_RADIAL)


def _gpu_steps(w, s, v, skip, steps, order, tau):
    """Carry on the GPU over the given steps (no oracle); returns each step's
    O and LSE and leaves the carried set in `skip`."""
    R, nK = w.B * w.H * w.nQ, w.nK
    ones = torch.ones(w.nQ * nK, dtype=torch.uint8, device=DEV)
    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv_asc = torch.empty(R * nK, dtype=torch.int32, device=DEV)
    kv = torch.empty(R * nK, dtype=torch.int32, device=DEV)
    gap = torch.empty(R * nK, dtype=torch.float32, device=DEV)
    outs = []
    for st in steps:
        x = synth.make_step_qk(w, st)
        q, k = dev(x["q"]), dev(x["k"])
        bsa.bsa_compact_block_lists(s, ones, 0, skip, rp, kv_asc)
        bsa.bsa_order_block_lists(s, order, rp, 0, kv_asc, kv)
        o = torch.empty_like(q)
        lse = torch.empty(w.B * w.H * w.N, dtype=torch.float32, device=DEV)
        bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, rp, kv, 0, w.scale, gap)
        bsa.bsa_update_skip_mask(s, rp, kv, gap, tau, skip)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    return outs


def test_skip_carry_save_and_restore_resumes_bit_exactly(tmp_path):
    """LiteAttention summary page, section 六: the skip mask persists across
    steps. Ten steps in one run equal five steps, the carried set saved to a
    file and loaded into a fresh buffer, then the other five: same skip sets,
    same O and LSE bit for bit (the kernels are deterministic)."""
    w = synth.Workload("skip_resume", 1, 3, 128, 6, 10, 14, 64, 64, "bf16", "skip", 624, True,
                       tau=1.0, steps=10)
    s = shape_of(w)
    v = dev(synth.make_qkv(w, step=0, want=("v",))["v"])
    R = w.B * w.H * w.nQ * w.nK
    full = torch.zeros(R, dtype=torch.uint8, device=DEV)
    outs_full = _gpu_steps(w, s, v, full, range(10), bsa.ORDER_RADIAL, w.tau)
    half = torch.zeros(R, dtype=torch.uint8, device=DEV)
    outs_a = _gpu_steps(w, s, v, half, range(5), bsa.ORDER_RADIAL, w.tau)
    np.save(tmp_path / "skip.npy", half.cpu().numpy())
    resumed = dev(np.load(tmp_path / "skip.npy"))
    del half
    outs_b = _gpu_steps(w, s, v, resumed, range(5, 10), bsa.ORDER_RADIAL, w.tau)
    assert torch.equal(resumed, full)
    for i, ((o1, l1), (o2, l2)) in enumerate(zip(outs_full, outs_a + outs_b)):
        np.testing.assert_array_equal(o1, o2, err_msg=f"step {i}")
        np.testing.assert_array_equal(l1, l2, err_msg=f"step {i}")
    note(f"resumed carry: {int(full.sum())} tiles skipped after 10 steps, identical")


def test_skip_carry_tau_schedule_then_shared_mask():
    """Stricter threshold early (larger tau), looser later; the second half of
    the steps shares the skip set reached at the half-way point."""
    w = synth.Workload("skip_sched", 1, 2, 128, 6, 10, 14, 64, 64, "bf16", "skip", 622, True,
                       tau=1.0, steps=6)
    taus = [2.0, 1.5, 1.0, 1.0, 1.0, 1.0]
    _skip_carry(w, w.steps, taus, order=bsa.ORDER_RADIAL, freeze_after=3)


def test_order_lists_bit_exact():
    # shared radial lists of the 720p shape, and per-head ragged lists
    w = synth.workload("wan14b_720p")
    s = shape_of(w)
    mask, rp, kv = radial_lists(s, w.h0, w.beta)
    nnz = int(host(rp)[-1])
    out = torch.empty_like(kv)
    for order in (bsa.ORDER_ASCENDING, bsa.ORDER_RADIAL):
        bsa.bsa_order_block_lists(s, order, rp, 1, kv, out)
        torch.cuda.synchronize()
        ref = oracle.order_lists(host(rp), host(kv)[:nnz], w.N, w.Bq, w.Bk, order)
        np.testing.assert_array_equal(host(out)[:nnz], ref)
        note(f"720p shared lists, order {order}: {nnz} entries bit-exact")
    r = np.random.default_rng(7)
    for (T, Hs, Ws, bq) in ((5, 9, 13, 128), (7, 11, 17, 64)):
        s2 = bsa.shape(2, 3, 128, T, Hs, Ws, bq)
        R = 6 * s2.nQ
        m = (r.random((R, s2.nK)) < 0.3).astype(np.uint8)
        m[:, 0] = 0
        m[::7] = 0                                   # some empty rows
        rp_ref, kv_ref = oracle.compact(m.reshape(2, 3, s2.nQ, s2.nK), 2, 3, s2.nQ, s2.nK,
                                        s2.nQ * s2.nK)
        rp_d, kv_d = dev(rp_ref), dev(kv_ref.astype(np.int32))
        out = torch.full_like(kv_d, -1)
        bsa.bsa_order_block_lists(s2, bsa.ORDER_RADIAL, rp_d, 0, kv_d, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(
            host(out), oracle.order_lists(rp_ref, kv_ref, s2.N, bq, 64, bsa.ORDER_RADIAL))


def test_fwd_wan14b_720p_radial_order_sampled():
    """Forward over radially ordered lists: the visiting order changes only
    rounding, so the outputs stay within the bounds of the oracle."""
    w = synth.workload("wan14b_720p")
    s = shape_of(w)
    x = synth.make_qkv(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    mask, rp, kv = radial_lists(s, w.h0, w.beta)
    kv2 = torch.empty_like(kv)
    bsa.bsa_order_block_lists(s, bsa.ORDER_RADIAL, rp, 1, kv, kv2)
    o, lse, _ = run_fwd(s, q, k, v, rp, kv2, 1, w.scale)
    rows = sample_rows(w.B, w.H, w.nQ, 2, 26, heads=[0, 17, w.H - 1])
    mask_h = host(mask).reshape(w.nQ, w.nK)
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, mask_h, 0,
                                         rows=rows)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, "720p radial order")


# ------------------------------------------------------------ long video
def test_fwd_hunyuan_4x_radial_sampled():
    w = synth.workload("hunyuan_4x")
    note(f"{w.name}: generating {w.B}x{w.N}x{w.H}x{w.d} bf16 inputs")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    mask = torch.empty(s.nQ * s.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_radial(s, w.h0, w.beta, mask)
    rp = torch.empty(s.nQ + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(s.nQ * s.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, mask, 0, None, rp, kv)
    o, lse, _ = run_fwd(s, q, k, v, rp, kv, 1, w.scale)
    assert_all_written(s, o, lse, rp, 1, w.name)
    ref_mask = oracle.build_mask_radial(w.T, w.Hs, w.Ws, w.Bq, w.Bk, w.h0, w.beta)
    np.testing.assert_array_equal(host(mask).reshape(w.nQ, w.nK), ref_mask)
    heads = [0, w.H - 1]
    F_blocks = [a for a in range(1, w.nQ) if (a * w.Bq) // w.F != ((a + 1) * w.Bq - 1) // w.F]
    rows = sample_rows(w.B, w.H, w.nQ, 3, 9, heads=heads, extra=F_blocks[:1])
    note(f"{w.name}: oracle on {len(rows)} sampled row blocks")
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, ref_mask,
                                         0, rows=rows)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, f"{w.name} sampled")


def test_fwd_with_tile_gaps_deterministic_run_twice():
    """Per-head lists with tile gaps (the skip carry's forward): O, LSE and the
    gaps, folded in with a float atomic max, are the same bit for bit on a
    second run."""
    w = synth.Workload("gap_twice", 1, 3, 128, 6, 10, 14, 64, 64, "bf16", "skip", 649, True,
                       tau=1.0, steps=1)
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    R = w.B * w.H * w.nQ
    ones = torch.ones(R * w.nK, dtype=torch.uint8, device=DEV)   # one mask per head
    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(R * w.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, ones, w.nQ * w.nK, None, rp, kv)   # per-head lists
    assert int(rp[-1]) == R * w.nK
    nnz = R * w.nK
    o1, l1, g1 = run_fwd(s, q, k, v, rp, kv, 0, w.scale, gap_len=nnz)
    o2, l2, g2 = run_fwd(s, q, k, v, rp, kv, 0, w.scale, gap_len=nnz)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert not torch.isnan(g1).any()
    assert torch.equal(g1, g2)
