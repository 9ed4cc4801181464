"""GPU parity over seeded random small shapes, the whole path end to end.

Each case draws batch, heads, head dim, frames, frame height and width, row
block, input type (bf16, or fp32 for the fp32 forward) and mask rule from a
fixed seed, so that grids with ragged last row and key blocks, a single
partial block, one frame or many small frames all occur.
Masks and block lists must match the oracle bit for bit; every output row is
compared with the oracle's masked attention within the attention bounds, and
every element of O and LSE must be written.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
import oracle
import synth
from _gpu_paths import run_pyramid, skip_carry
from _gpu_util import (DEV, assert_all_written, compare, dev, gather_rows, host, note, run_fwd,
                       shape_of)

pytestmark = pytest.mark.gpu

RULES = ["radial", "topk", "mass", "headwide_topk", "headwide_mass"]


def _draw(case: int):
    r = np.random.default_rng(9000 + case)
    B = int(r.integers(1, 3))
    H = int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    T = int(r.integers(1, 7))
    Hs = int(r.integers(3, 25))
    Ws = int(r.integers(3, 33))
    Bq = int(r.choice([64, 128]))
    rule = RULES[case % len(RULES)]
    h0 = int(r.choice([16, 32, 64, 128]))
    dtype = "f32" if case % 4 == 3 else "bf16"
    w = synth.Workload(f"rand{case}", B, H, d, T, Hs, Ws, Bq, 64, dtype,
                       "radial" if rule == "radial" else "pooled", 9100 + case, True,
                       h0=h0, beta=2)
    param = {"radial": 0.0, "topk": float(r.integers(1, 6)), "mass": float(r.uniform(0.2, 0.95)),
             "headwide_topk": float(r.integers(1, 4 * w.nQ + 1)),
             "headwide_mass": float(r.uniform(0.2, 0.95))}[rule]
    return w, rule, param


@pytest.mark.parametrize("case", range(20))
def test_random_shape_path_matches_oracle(case):
    w, rule, param = _draw(case)
    note(f"random case {case}: {w.dtype} B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} "
         f"(N={w.N}) Bq={w.Bq} rule={rule} param={param:g}")
    x = synth.make_qkv(w)
    s = shape_of(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    if rule == "radial":
        mask = torch.empty(w.nQ * w.nK, dtype=torch.uint8, device=DEV)
        bsa.bsa_build_mask_radial(s, w.h0, w.beta, mask)
        ref = oracle.build_mask_radial(w.T, w.Hs, w.Ws, w.Bq, w.Bk, w.h0, w.beta)
        got = host(mask).reshape(w.nQ, w.nK)
        shared, mhs, R = 1, 0, w.nQ
    else:
        mode = {"topk": 0, "mass": 1, "headwide_topk": 2, "headwide_mass": 3}[rule]
        ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
        mask = torch.empty(w.B * w.H * w.nQ * w.nK, dtype=torch.uint8, device=DEV)
        bsa.bsa_build_mask_pooled(s, q, k, w.scale, mode, param, mask, ws)
        ref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, mode, param)
        got = host(mask).reshape(w.B, w.H, w.nQ, w.nK)
        shared, mhs, R = 0, w.nQ * w.nK, w.B * w.H * w.nQ
    np.testing.assert_array_equal(got, ref)

    rp = torch.empty(R + 1, dtype=torch.int32, device=DEV)
    kv = torch.empty(R * w.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, mask, mhs, None, rp, kv)
    rp_ref, kv_ref = oracle.compact(ref.reshape(-1) if shared else ref,
                                    1 if shared else w.B, 1 if shared else w.H, w.nQ, w.nK, mhs)
    rp_h = host(rp)
    np.testing.assert_array_equal(rp_h, rp_ref)
    np.testing.assert_array_equal(host(kv)[:rp_h[-1]], kv_ref)

    o, lse, _ = run_fwd(s, q, k, v, rp, kv, shared, w.scale)
    label = f"random case {case} ({rule})"
    assert_all_written(s, o, lse, rp, shared, label)
    o_ref, lse_ref, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, ref, mhs)
    rows = np.arange(w.B * w.H * w.nQ)
    og, lg = gather_rows(host(o), host(lse), rows, w.B, w.H, w.N, w.Bq)
    compare(og, lg, o_ref, lse_ref, label)


def _draw_pyramid(case: int):
    r = np.random.default_rng(9500 + case)
    L = 1 + case % 4
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    T, Hs = int(r.integers(1, 7)), int(r.integers(3, 25))
    Ws = 8 * int(r.integers(1, 5))          # N a multiple of 8: every level pools whole groups
    Bq = int(r.choice([64, 128]))
    taus = sorted(float(t) for t in r.uniform(0.1, 1.0, size=L))
    w = synth.Workload(f"rand_pyr{case}", B, H, d, T, Hs, Ws, Bq, 64, "bf16", "pooled",
                       9600 + case, True)
    return w, taus


@pytest.mark.parametrize("case", range(12))
def test_random_shape_pyramid_matches_oracle(case):
    w, taus = _draw_pyramid(case)
    note(f"random pyramid case {case}: B={w.B} H={w.H} d={w.d} grid {w.T}x{w.Hs}x{w.Ws} "
         f"(N={w.N}) Bq={w.Bq} taus={[round(t, 3) for t in taus]}")
    x = synth.make_qkv(w)
    out = run_pyramid(w, x, taus)
    mref, _, _ = oracle.build_mask_pooled(x["q"], x["k"], w.Bq, w.Bk, w.scale, 4, 0,
                                          levels_tau=taus)
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
    compare(og, lg, o_ref, lse_ref, f"random pyramid case {case}")


@pytest.mark.parametrize("case", range(8))
def test_random_shape_skip_carry_matches_oracle(case):
    """Three denoising steps of the carried skip set: lists, outputs, tile
    gaps and update decisions against the oracle at every step."""
    r = np.random.default_rng(9800 + case)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    T, Hs, Ws = int(r.integers(1, 7)), int(r.integers(3, 25)), int(r.integers(3, 33))
    Bq = int(r.choice([64, 128]))
    tau = float(r.uniform(0.5, 3.0))
    order = bsa.ORDER_RADIAL if case % 2 else bsa.ORDER_ASCENDING
    w = synth.Workload(f"rand_skip{case}", B, H, d, T, Hs, Ws, Bq, 64, "bf16", "skip",
                       9900 + case, True, tau=tau, steps=3)
    note(f"random skip case {case}: B={B} H={H} d={d} grid {T}x{Hs}x{Ws} (N={w.N}) Bq={Bq} "
         f"tau={tau:.3f} order={order}")
    skip_carry(w, 3, tau, order=order)
