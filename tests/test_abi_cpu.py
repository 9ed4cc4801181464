"""C-ABI checks that need no GPU: the library loads, exports every function
include/bsa.h declares, and rejects bad arguments with the documented status
before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import block_sparse_attention_flashattention_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

INVALID, UNSUPPORTED, CAPACITY = 1, 2, 3
P = 0x10000  # a 16-byte aligned stand-in address; validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"BSA_API\s+[\w\s\*]+?\b(bsa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        from block_sparse_attention_flashattention_amd import build
        build.build()
    return bsa.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 20
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)", out))
    assert set(names) <= exported
    for n in names:
        getattr(L, n)


def T(ptr=P, sb=0, sn=128, sh=128):
    return bsa.Tensor(ptr, sb, sn, sh)


def S(**kw):
    base = dict(batch=1, heads=2, head_dim=128, frames=3, height=5, width=7, block_q=128,
                block_k=64)
    base.update(kw)
    return bsa.Shape(*[base[k] for k in ("batch", "heads", "head_dim", "frames", "height",
                                          "width", "block_q", "block_k")])


def fwd(L, s, q=None, k=None, v=None, o=None, dt=0, row_ptr=None, kv_idx=None, shared=0,
        scale=0.1, gap=None):
    return L.bsa_sparse_attn_fwd(C.byref(s), dt, q or T(), k or T(P + 256), v or T(P + 512),
                                 o or T(P + 1024), None, row_ptr, kv_idx, shared, scale, gap,
                                 None)


def test_status_strings(L):
    for st in range(5):
        assert bsa.bsa_status_string(st)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), UNSUPPORTED), (dict(head_dim=0), INVALID), (dict(block_q=32), UNSUPPORTED),
    (dict(block_k=128), UNSUPPORTED), (dict(batch=-1), INVALID), (dict(frames=-2), INVALID),
    (dict(frames=100000, height=200, width=200), INVALID),
])
def test_shape_validation(L, kw, status):
    assert fwd(L, S(**kw)) == status
    assert bsa.bsa_last_error()


def test_fwd_argument_validation(L):
    s = S()
    assert fwd(L, s, q=T(ptr=None)) == INVALID
    assert fwd(L, s, q=T(ptr=P + 8)) == INVALID                 # misaligned
    assert fwd(L, s, k=T(P + 256, sn=100)) == INVALID           # stride not a multiple of 8
    assert fwd(L, s, v=T(P + 512, sh=-8)) == INVALID            # negative stride
    assert fwd(L, s, o=T(P)) == INVALID                         # o aliases q
    assert fwd(L, s, k=T(P + 256, sn=64)) == INVALID            # rows overlap
    assert fwd(L, s, v=T(P + 512, sn=1 << 24)) == UNSUPPORTED   # tile span too large
    assert fwd(L, s, dt=7) == UNSUPPORTED
    assert fwd(L, s, scale=-1.0) == INVALID
    assert fwd(L, s, scale=float("nan")) == INVALID
    assert fwd(L, s, row_ptr=P) == INVALID                      # lists half given
    assert fwd(L, s, shared=2, row_ptr=P, kv_idx=P) == INVALID
    assert fwd(L, s, gap=P) == INVALID                          # gaps need lists
    # gaps feed the skip update, which reads per-head lists only
    assert fwd(L, s, shared=1, row_ptr=P, kv_idx=P, gap=P) == UNSUPPORTED
    assert "per-head" in bsa.bsa_last_error()
    # fp32: strides must be multiples of 4 elements
    assert fwd(L, s, dt=1, q=T(sn=130)) == INVALID


def test_empty_shapes_are_noops(L):
    for kw in (dict(batch=0), dict(heads=0), dict(frames=0)):
        assert fwd(L, S(**kw), q=T(ptr=None)) == 0


def test_radial_validation(L):
    s = S()
    assert L.bsa_build_mask_radial(C.byref(s), 31, 2, P, None) == INVALID   # h0 < Bk/2
    assert L.bsa_build_mask_radial(C.byref(s), 64, 1, P, None) == INVALID   # base < 2
    assert L.bsa_build_mask_radial(C.byref(s), 64, 2, None, None) == INVALID
    assert L.bsa_build_mask_radial(C.byref(S(head_dim=80)), 64, 2, P, None) == UNSUPPORTED


def test_pooled_validation(L):
    s = S()
    need = L.bsa_pooled_workspace_bytes(C.byref(s))
    B, H, D, nQ, nK = 1, 2, 128, 1, 2
    # pooled means and scores, plus the head-wide modes' probabilities
    assert need >= 8 * (B * H * (nQ + nK) * D + 2 * B * H * nQ * nK)
    assert need % 256 == 0

    def call(mode=1, param=0.5, ws=P, wsb=need, mask=P, dt=0, shape=s, scale=0.1):
        return L.bsa_build_mask_pooled(C.byref(shape), dt, T(), T(P + 256), scale, mode, param,
                                       mask, ws, wsb, None)
    assert call(mode=4) == INVALID
    assert call(mode=-1) == INVALID
    assert call(mode=2, param=0.5) == INVALID     # head-wide top-k needs an integer k
    assert call(mode=3, param=0.0) == INVALID
    assert call(mode=3, param=1.01) == INVALID
    assert call(mode=1, param=0.0) == INVALID
    assert call(mode=1, param=1.5) == INVALID
    assert call(mode=0, param=0.0) == INVALID
    assert call(mode=0, param=2.5) == INVALID
    assert call(wsb=need - 8) == INVALID
    assert call(ws=None) == INVALID
    assert call(ws=P + 64) == INVALID          # workspace alignment
    assert call(mask=None) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(dt=3) == UNSUPPORTED
    long_rows = S(frames=33, height=100, width=100)   # 330,000 tokens -> 5,157 key blocks
    assert call(shape=long_rows) == INVALID              # supported; the workspace is short
    assert "workspace" in bsa.bsa_last_error()
    big = S(frames=60, height=100, width=100)   # 600,000 tokens -> 9,375 key blocks
    assert call(shape=big) == UNSUPPORTED


def test_compaction_validation(L):
    s = S()
    nQ, nK = 1, 2
    def call(mhs=0, skip=None, row_ptr=P, kv_idx=P, cap=4, nnz=None):
        return L.bsa_compact_block_lists(C.byref(s), P, mhs, skip, row_ptr, kv_idx, cap, nnz, None)
    assert call(mhs=1) == INVALID                 # 0 < stride < nQ*nK
    assert call(row_ptr=None) == INVALID
    assert call(cap=-1) == INVALID
    assert call(cap=nQ * nK - 1) == CAPACITY      # shared list, worst case not covered
    assert call(mhs=nQ * nK, skip=P, cap=2 * nQ * nK - 1) == CAPACITY


def test_skip_update_validation(L):
    s = S()
    assert L.bsa_update_skip_mask(C.byref(s), P, P, P, 0.0, P, None) == INVALID
    assert L.bsa_update_skip_mask(C.byref(s), P, P, P, float("nan"), P, None) == INVALID
    assert L.bsa_update_skip_mask(C.byref(s), None, P, P, 10.0, P, None) == INVALID
    assert L.bsa_update_skip_mask(C.byref(s), P, P, P, 10.0, None, None) == INVALID


def test_order_lists_validation(L):
    s = S()
    def call(order=1, row_ptr=P, shared=1, kv_in=P, kv_out=P + 4096):
        return L.bsa_order_block_lists(C.byref(s), order, row_ptr, shared, kv_in, kv_out, None)
    assert call(order=2) == INVALID
    assert call(order=-1) == INVALID
    assert call(shared=2) == INVALID
    assert call(row_ptr=None) == INVALID
    assert call(kv_in=None) == INVALID
    assert call(kv_out=None) == INVALID
    assert call(kv_out=P) == INVALID                  # in place is refused
    assert L.bsa_order_block_lists(C.byref(S(head_dim=96)), 1, P, 1, P, P + 64, None) == UNSUPPORTED
    # empty shapes enqueue nothing and need no pointers
    assert L.bsa_order_block_lists(C.byref(S(frames=0)), 1, None, 1, None, None, None) == 0


def test_permutation_validation(L):
    s = S()
    def mk(kind, axes, perm=P):
        return L.bsa_make_token_permutation(C.byref(s), kind, (C.c_int32 * 3)(*axes), perm, None)
    assert mk(0, (0, 1, 1)) == INVALID               # not a permutation of the axes
    assert mk(0, (0, 1, 3)) == INVALID
    assert mk(1, (1, 0, 2)) == INVALID               # empty box
    assert mk(2, (1, 1, 1)) == INVALID
    assert mk(0, (2, 0, 1), perm=None) == INVALID
    assert L.bsa_make_token_permutation(C.byref(s), 0, None, P, None) == INVALID
    N = 3 * 5 * 7
    def pt(perm=P, phs=0, scatter=0, x=None, out=None, dt=0):
        return L.bsa_permute_tokens(C.byref(s), dt, perm, phs, scatter, x or T(), out or T(P + 4096),
                                    None)
    assert pt(phs=N - 1) == INVALID
    assert pt(scatter=2) == INVALID
    assert pt(perm=None) == INVALID
    assert pt(out=T()) == INVALID                    # in place is refused
    assert pt(x=T(P + 8)) == INVALID                 # misaligned
    assert pt(dt=5) == UNSUPPORTED


def test_pyramid_validation(L):
    s = S()                                          # N = 105 tokens: odd
    s4 = S(frames=4, height=5, width=8)              # N = 160 tokens
    assert L.bsa_pyramid_rows(C.byref(s4), 1) == 0
    assert L.bsa_pyramid_rows(C.byref(s4), 2) == 64 * 2      # 80 rows -> 2 blocks
    assert L.bsa_pyramid_rows(C.byref(s4), 3) == 64 * 3      # + 40 rows -> 1 block
    assert L.bsa_pyramid_rows(C.byref(s4), 4) == 64 * 4      # + 20 rows -> 1 block
    assert L.bsa_pyramid_rows(C.byref(s4), 5) == -1
    kvp = lambda shape, nl: L.bsa_build_kv_pyramid(C.byref(shape), 0, nl, T(), T(P + 256),
                                                   T(P + 512), T(P + 768), None)
    assert kvp(s4, 0) == INVALID
    assert kvp(s, 2) == UNSUPPORTED                  # N not a multiple of 2
    assert kvp(S(frames=1, height=4, width=5), 4) == UNSUPPORTED   # N = 20: not of 8
    assert kvp(s4, 5) == INVALID
    taus = (C.c_double * 3)(0.5, 0.4, 0.9)
    def mk(nl=3, t=taus, ws=P, wsb=1 << 30):
        return L.bsa_build_mask_pyramid(C.byref(s4), 0, T(), T(P + 256), 0.1, nl, t, P, ws, wsb,
                                        None)
    assert mk() == INVALID                           # thresholds must not decrease
    assert mk(t=(C.c_double * 3)(0.0, 0.5, 0.9)) == INVALID
    assert mk(nl=5, t=(C.c_double * 5)(0.1, 0.2, 0.3, 0.4, 0.5)) == INVALID
    assert mk(nl=4, t=(C.c_double * 4)(0.1, 0.2, 0.5, 0.4)) == INVALID
    assert mk(t=None) == INVALID
    lists = lambda nl=3, cap=0, rp=P: L.bsa_compact_pyramid_lists(C.byref(s4), nl, P, 0, rp, P,
                                                                  P + 64, cap, None, None)
    assert lists(rp=None) == INVALID
    assert lists(cap=1) == CAPACITY
    assert lists(nl=5) == INVALID
    fwd = lambda dt=0, nl=3, kp=None, qm=P: L.bsa_pyramid_attn_fwd(
        C.byref(s4), dt, T(), T(P + 256), T(P + 512), kp or T(P + 768), T(P + 1024), nl,
        T(P + 2048), None, P, P, qm, 0.1, None)
    assert fwd(dt=1) == UNSUPPORTED                  # bf16 only
    assert fwd(qm=None) == INVALID
    assert fwd(kp=T(P + 768, sn=64)) == INVALID      # k_pyr row stride differs from k


# ------------------------------------------------ debug check of block lists
def lists_of(rows):
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    kv = np.array([c for r in rows for c in r], dtype=np.int32)
    return rp, kv


def check(s, rp, kv, shared=1, n_blocks=0, ascending=False, kv_len=None):
    try:
        bsa.bsa_check_block_lists(s, shared, rp, kv, n_blocks, ascending, kv_len)
        return 0, ""
    except bsa.BsaError as e:
        return e.status, e.detail


# S(): N = 105 tokens, Bq = 128 -> nQ = 1, nK = 2; per-head lists: B*H*nQ = 2 rows
@pytest.mark.parametrize("rows,shared,asc,expect", [
    ([[0, 1]], 1, True, (0, None, None)),
    ([[1, 0]], 1, False, (0, None, None)),             # any order when ascending is not asked
    ([[1, 0]], 1, True, (INVALID, 0, 6)),
    ([[0, 0]], 1, False, (INVALID, 0, 5)),
    ([[0, 0]], 1, True, (INVALID, 0, 5)),
    ([[0, 2]], 1, False, (INVALID, 0, 4)),              # key block 2 does not exist
    ([[-1]], 1, False, (INVALID, 0, 4)),
    ([[], [1]], 0, True, (0, None, None)),              # empty rows are fine
    ([[1], [1, 5, 1]], 0, False, (INVALID, 1, 4)),      # rule 4 before rule 5 in one row
])
def test_list_check_rules_on_host(L, rows, shared, asc, expect):
    s = S()
    rp, kv = lists_of(rows)
    status, detail = check(s, rp, kv, shared=shared, ascending=asc)
    assert status == expect[0]
    if status:
        assert f"row {expect[1]}: rule {expect[2]}" in detail


def test_list_check_row_pointer_rules_on_host(L):
    s = S()
    kv = np.array([0, 1, 0], np.int32)
    assert check(s, np.array([1, 2, 3], np.int32), kv, shared=0)[1].startswith(
        "block lists, row 0: rule 1")
    assert "row 1: rule 2" in check(s, np.array([0, 2, 1], np.int32), kv, shared=0)[1]
    assert "row 1: rule 3" in check(s, np.array([0, 1, 3], np.int32), kv, shared=0, kv_len=2)[1]
    # a pointer past kv_len is reported at its row; nothing past kv_len is read
    assert "row 0: rule 3" in check(s, np.array([0, 9, 3], np.int32), kv, shared=0)[1]
    # pyramid-style lists name augmented blocks: n_blocks widens the range
    assert check(s, np.array([0, 1], np.int32), np.array([3], np.int32), n_blocks=4)[0] == 0
    assert check(s, np.array([0, 1], np.int32), np.array([3], np.int32))[0] == INVALID


def test_list_check_matches_brute_force_on_random_lists(L):
    """The host check against a direct restatement of the list contract on
    random, partly corrupted lists: valid iff every row holds distinct blocks
    in range (and ascending when asked)."""
    r = np.random.default_rng(5)
    s = S(batch=2, heads=3, frames=4, height=8, width=8, block_q=64)   # nQ = nK = 4
    R, nK = 2 * 3 * 4, 4
    for trial in range(300):
        rows = [sorted(r.choice(nK, size=r.integers(0, nK + 1), replace=False).tolist())
                for _ in range(R)]
        if trial % 3 == 1:
            rows[r.integers(R)] = r.integers(-1, nK + 1, size=r.integers(1, 5)).tolist()
        elif trial % 3 == 2:
            rr = rows[r.integers(R)]
            r.shuffle(rr)
        rp, kv = lists_of(rows)
        for asc in (False, True):
            ok = all(len(set(x)) == len(x) and all(0 <= c < nK for c in x)
                     and (not asc or x == sorted(x)) for x in rows)
            assert (check(s, rp, kv, shared=0, ascending=asc)[0] == 0) == ok, (rows, asc)


def test_list_check_argument_validation(L):
    s = S()
    call = lambda **kw: L.bsa_check_block_lists(
        C.byref(s), kw.get("shared", 1), kw.get("rp", P), kw.get("kv", P), kw.get("n", 4),
        kw.get("nb", 0), 0, kw.get("dev", 0), None)
    assert call(shared=2) == INVALID
    assert call(dev=2) == INVALID
    assert call(n=-1) == INVALID
    assert call(nb=-1) == INVALID
    assert call(rp=None) == INVALID
    assert call(kv=None) == INVALID


def test_pooled_noalloc_validation(L):
    """Same argument checks as the workspace form; shapes whose scratch would
    exceed the static 64 MiB are refused before anything is enqueued."""
    def call(shape=S(), mode=1, param=0.5, mask=P, dt=0):
        return L.bsa_build_mask_pooled_noalloc(C.byref(shape), dt, T(), T(P + 256), 0.1, mode,
                                               param, mask, None)
    assert call(mode=5) == INVALID
    assert call(param=0.0) == INVALID
    assert call(mask=None) == INVALID
    assert call(dt=3) == UNSUPPORTED
    assert call(shape=S(frames=60, height=100, width=100)) == UNSUPPORTED   # > 8192 key blocks
    # 480p layer, 12 heads: per-row modes fit (37.7 MB) -- not launched here;
    # head-wide modes need 108 MiB and are refused with CAPACITY
    big = S(heads=12, frames=21, height=30, width=52, block_q=64)
    assert call(shape=big, mode=3, param=0.5) == CAPACITY
    assert call(shape=big, mode=2, param=4) == CAPACITY
    assert "static scratch" in bsa.bsa_last_error()
    # 720p shape at 40 heads: even the per-row modes exceed it
    assert call(shape=S(heads=40, frames=21, height=45, width=80)) == CAPACITY
