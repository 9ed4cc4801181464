"""Helpers shared by the GPU parity tests: moving the generator's bytes to the
device, calling the library through its binding, and comparing with the
oracle row by row. No attention arithmetic lives here."""
import sys

import numpy as np
import torch

import block_sparse_attention_flashattention_amd as bsa

DEV = "cuda:0"

# acceptance bounds for attention outputs against the fp64 oracle
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_ABS = 1e-2
GAP_ABS = 1e-3


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """Same bytes on the GPU: uint16 -> bf16, float32 -> float32, uint8/int32 as is."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def shape_of(w, heads=None):
    H = w.H if heads is None else heads
    return bsa.shape(w.B, H, w.d, w.T, w.Hs, w.Ws, w.Bq, w.Bk)


def radial_lists(s, h0, beta=2):
    """GPU radial mask + shared lists."""
    mask = torch.empty(s.nQ * s.nK, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_radial(s, h0, beta, mask)
    row_ptr = torch.empty(s.nQ + 1, dtype=torch.int32, device=DEV)
    kv_idx = torch.empty(s.nQ * s.nK, dtype=torch.int32, device=DEV)
    bsa.bsa_compact_block_lists(s, mask, 0, None, row_ptr, kv_idx)
    return mask, row_ptr, kv_idx


def run_fwd(s, q, k, v, row_ptr=None, kv_idx=None, shared=0, scale=None, gap_len=0):
    # NaN-filled outputs: a row block the kernel never writes stays NaN
    o = torch.full_like(q, float("nan"))
    lse = torch.full((s.batch * s.heads * s.N,), float("nan"), dtype=torch.float32, device=DEV)
    gap = torch.full((gap_len,), float("nan"), dtype=torch.float32, device=DEV) if gap_len else None
    bsa.bsa_sparse_attn_fwd(s, q, k, v, o, lse, row_ptr, kv_idx, shared, scale, gap)
    torch.cuda.synchronize()
    return o, lse, gap


def gather_rows(o_gpu: np.ndarray, lse_gpu: np.ndarray, rows, B, H, N, bq):
    """GPU outputs of the given list rows as [n][bq][D] / [n][bq] (NaN padding)."""
    nQ = -(-N // bq)
    D = o_gpu.shape[-1]
    o = np.full((len(rows), bq, D), np.nan)
    lse = np.full((len(rows), bq), np.nan)
    lse_g = lse_gpu.reshape(B, H, N)
    for t, r in enumerate(rows):
        bh, a = divmod(int(r), nQ)
        b, h = divmod(bh, H)
        i0, i1 = a * bq, min(N, (a + 1) * bq)
        o[t, :i1 - i0] = o_gpu[b, i0:i1, h, :]
        lse[t, :i1 - i0] = lse_g[b, h, i0:i1]
    return o, lse


def compare(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    """Assert the acceptance bounds on valid rows; returns (max_abs, mean_abs, lse_max)."""
    valid = ~np.isnan(lse_ref)
    d = np.abs(o_gpu[valid] - o_ref[valid])
    assert not np.isnan(d).any(), f"{label}: NaN in GPU output"
    max_abs, mean_abs = float(d.max()), float(d.mean())
    fin = valid & np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu[valid]), np.isneginf(lse_ref[valid])), \
        f"{label}: empty-row pattern differs"
    lse_err = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    note(f"{label}: O max-abs {max_abs:.3e} mean-abs {mean_abs:.3e}; LSE max {lse_err:.3e}")
    assert max_abs <= O_MAX_ABS, f"{label}: max-abs {max_abs}"
    assert mean_abs <= O_MEAN_ABS, f"{label}: mean-abs {mean_abs}"
    assert lse_err <= LSE_ABS, f"{label}: lse {lse_err}"
    return max_abs, mean_abs, lse_err


def sample_rows(B, H, nQ, per_head, seed, heads=None, extra=()):
    """Stratified row sample: first, last (ragged), and uniform row blocks per head."""
    r = np.random.default_rng(seed)
    hs = range(H) if heads is None else heads
    rows = []
    for b in range(B):
        for h in hs:
            base = (b * H + h) * nQ
            pick = {0, nQ - 1, *extra}
            pick |= set(r.choice(nQ, size=min(nQ, per_head), replace=False).tolist())
            rows += [base + a for a in sorted(pick) if 0 <= a < nQ]
    return np.array(rows, dtype=np.int64)


def assert_all_written(s, o, lse, row_ptr=None, shared=0, label=""):
    """Every element of O is written (no NaN left from the fill) and every
    query of a row block with a non-empty list has a finite LSE; rows with an
    empty list have LSE = -inf. Checked on the device over the whole tensors."""
    assert not bool(torch.isnan(o).any()), f"{label}: O has unwritten (NaN) elements"
    B, H, N, bq = s.batch, s.heads, s.N, s.block_q
    nQ = -(-N // bq)
    if row_ptr is None:
        nonempty = torch.ones(B * H * nQ, dtype=torch.bool, device=DEV)
    else:
        rp = row_ptr[: (nQ if shared else B * H * nQ) + 1].long()
        nonempty = (rp[1:] > rp[:-1])
        if shared:
            nonempty = nonempty.repeat(B * H)
    tok = nonempty.view(B * H, nQ).repeat_interleave(bq, dim=1)[:, :N].reshape(-1)
    lse_ok = torch.where(tok, torch.isfinite(lse), torch.isneginf(lse))
    assert bool(lse_ok.all()), f"{label}: {int((~lse_ok).sum())} LSE values wrong or unwritten"
    note(f"{label}: all {o.numel()} O values and {lse.numel()} LSE values written")
