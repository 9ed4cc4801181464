"""fp64 CPU oracle for block-sparse video attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path. The arithmetic
lives in bsa_oracle.c (plain fp64 loops); this file only marshals arrays.
It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsa_oracle.c")
_LIB = os.path.join(_HERE, "libbsa_oracle.so")

DT_BF16, DT_F32, DT_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        i64, p, d = C.c_int64, C.c_void_p, C.c_double
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = C.c_int
        L.oracle_radial_window.argtypes = [i64, i64, i64, i64, C.POINTER(i64)]
        L.oracle_radial_window.restype = C.c_int
        L.oracle_radial_count_pairs.argtypes = [i64] * 6
        L.oracle_radial_count_pairs.restype = i64
        L.oracle_build_mask_radial.argtypes = [i64] * 7 + [p]
        L.oracle_build_mask_radial.restype = None
        L.oracle_build_mask_pooled.argtypes = ([i64] * 6 + [C.c_int] + [p, i64, i64, i64] * 2
                                               + [d, C.c_int, d, p, p, p, p, i64])
        L.oracle_build_mask_pooled.restype = C.c_int
        L.oracle_compact.argtypes = [i64] * 4 + [p, i64, p, p, p]
        L.oracle_compact.restype = i64
        L.oracle_attention.argtypes = ([i64] * 6 + [C.c_int] + [p, i64, i64, i64] * 3
                                       + [d, p, i64, i64, p, p, p, p, C.c_int])
        L.oracle_attention.restype = C.c_int
        L.oracle_order_lists.argtypes = [i64] * 5 + [C.c_int, p, p, p]
        L.oracle_order_lists.restype = None
        L.oracle_make_permutation.argtypes = [i64, i64, i64, C.c_int, p, p]
        L.oracle_make_permutation.restype = None
        L.oracle_pyramid_attention.argtypes = ([i64] * 6 + [C.c_int] + [p, i64, i64, i64] * 3
                                               + [d, p, i64, i64, p, p, p])
        L.oracle_pyramid_attention.restype = C.c_int
        L.oracle_pyramid_regions.argtypes = [i64, i64, i64, p, p]
        L.oracle_pyramid_regions.restype = None
        L.oracle_compact_pyramid.argtypes = [i64] * 7 + [p, i64, p, p, p]
        L.oracle_compact_pyramid.restype = i64
        L.oracle_choose_token_orders.argtypes = ([i64] * 8 + [C.c_int, p, p, d, C.c_int, d, p,
                                                                p])
        L.oracle_choose_token_orders.restype = C.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _strides(a: np.ndarray):
    """Element strides of a [B][N][H][d] array with d contiguous."""
    if a.ndim != 4 or a.strides[3] != a.itemsize:
        raise ValueError("expected [B][N][H][d] with contiguous head_dim")
    return tuple(s // a.itemsize for s in a.strides[:3])


# ------------------------------------------------------------------- radial
def radial_window(d: int, h0: int, beta: int, bk: int):
    h = C.c_int64(0)
    kept = lib().oracle_radial_window(d, h0, beta, bk, C.byref(h))
    return bool(kept), int(h.value)


def radial_count_pairs(T, Hs, Ws, h0, beta, bk) -> int:
    return int(lib().oracle_radial_count_pairs(T, Hs, Ws, h0, beta, bk))


def build_mask_radial(T, Hs, Ws, bq, bk, h0, beta) -> np.ndarray:
    if h0 < bk // 2:
        raise ValueError("radial window must be at least half a key block")
    N = T * Hs * Ws
    nQ, nK = -(-N // bq), -(-N // bk)
    m = np.zeros((nQ, nK), dtype=np.uint8)
    lib().oracle_build_mask_radial(T, Hs, Ws, bq, bk, h0, beta, _ptr(m))
    return m


# ------------------------------------------------------------------- pooled
def build_mask_pooled(q: np.ndarray, k: np.ndarray, bq: int, bk: int, scale: float,
                      mode: int, param: float, want_scores=False, levels_tau=None):
    """Returns (mask [B][H][nQ][nK] uint8, scores or None, margin [B][H][nQ]).

    mode 0: per-row top-k (param = k); 1: per-row cumulative mass (param =
    tau_p); 2: head-wide top-k over all (row, block) pairs (param = k);
    3: head-wide cumulative mass reaching tau_p * nQ (param = tau_p). In the
    head-wide modes every row also keeps its best block. 4: pyramid levels
    (Pyramid Sparse Attention page): mask = 1 + level by the thresholds
    levels_tau (non-decreasing), 0 = dropped."""
    B, N, H, D = q.shape
    nQ, nK = -(-N // bq), -(-N // bk)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and k.shape == q.shape
    mask = np.zeros((B, H, nQ, nK), dtype=np.uint8)
    scores = np.zeros((B, H, nQ, nK), dtype=np.float64) if want_scores else None
    margin = np.zeros((B, H, nQ), dtype=np.float64)
    lt = np.ascontiguousarray(levels_tau if levels_tau is not None else [], dtype=np.float64)
    if mode == 4 and not (1 <= lt.size <= 4 and np.all(np.diff(lt) >= 0)):
        raise ValueError("pyramid levels need 1..4 non-decreasing thresholds")
    rc = lib().oracle_build_mask_pooled(
        B, H, N, D, bq, bk, dt, _ptr(q), *_strides(q), _ptr(k), *_strides(k),
        float(scale), int(mode), float(param), _ptr(mask),
        _ptr(scores) if scores is not None else None, _ptr(margin),
        _ptr(lt) if lt.size else None, int(lt.size))
    if rc != 0:
        raise MemoryError("oracle_build_mask_pooled failed to allocate")
    return mask, scores, margin


# --------------------------------------------------------------- compaction
def compact(mask: np.ndarray, B: int, H: int, nQ: int, nK: int,
            mask_head_stride: int, skip: np.ndarray | None = None):
    """CSR lists (row_ptr int32 [B*H*nQ+1], kv_idx int32 [nnz])."""
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    if skip is not None:
        skip = np.ascontiguousarray(skip, dtype=np.uint8)
    L = lib()
    sp = _ptr(skip) if skip is not None else None
    nnz = L.oracle_compact(B, H, nQ, nK, _ptr(mask), mask_head_stride, sp, None, None)
    row_ptr = np.zeros(B * H * nQ + 1, dtype=np.int32)
    kv_idx = np.zeros(max(nnz, 1), dtype=np.int32)
    L.oracle_compact(B, H, nQ, nK, _ptr(mask), mask_head_stride, sp,
                     _ptr(row_ptr), _ptr(kv_idx))
    return row_ptr, kv_idx[:nnz]


ORDER_ASCENDING, ORDER_RADIAL = 0, 1


def order_lists(row_ptr: np.ndarray, kv_idx: np.ndarray, N: int, bq: int, bk: int,
                order: int) -> np.ndarray:
    """Each CSR row's key blocks in visiting order (LiteAttention summary page,
    section 五: radial-centric order; see oracle_order_lists)."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    kv_in = np.ascontiguousarray(kv_idx, dtype=np.int32)
    nQ = -(-N // bq)
    out = np.empty_like(kv_in)
    if kv_in.size:
        lib().oracle_order_lists(N, bq, bk, nQ, row_ptr.size - 1, int(order), _ptr(row_ptr),
                                 _ptr(kv_in), _ptr(out))
    return out


# ------------------------------------------------------- token permutation
PERM_AXES, PERM_BOXES = 0, 1


def make_permutation(T: int, Hs: int, Ws: int, kind: int, axes) -> np.ndarray:
    """perm[i'] = original token of new position i' (PAROAttention summary page,
    section 二: one of the six axis orders; VMoBA summary page, section 三:
    temporal chunks, spatial patches or cubes). kind 0: axes = (slowest,
    middle, fastest) axis ids (0 frame, 1 row, 2 column); kind 1: axes =
    box extent (frames, rows, columns)."""
    if kind == PERM_AXES and sorted(axes) != [0, 1, 2]:
        raise ValueError("axis order must be a permutation of (0, 1, 2)")
    if kind == PERM_BOXES and min(axes) < 1:
        raise ValueError("box extents must be >= 1")
    ax = np.ascontiguousarray(axes, dtype=np.int64)
    perm = np.empty(T * Hs * Ws, dtype=np.int32)
    lib().oracle_make_permutation(T, Hs, Ws, int(kind), _ptr(ax), _ptr(perm))
    return perm


def choose_token_orders(q: np.ndarray, k: np.ndarray, T: int, Hs: int, Ws: int, bq: int,
                        bk: int, scale: float, mode: int, param: float):
    """Per-head token order ([PARO] section 二, reading in bsa_oracle.c):
    (order per head [H], kept tiles per head and order [H][6]). q, k are
    [B][N][H][d] bf16 bits (uint16) or float32."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    B, N, H, D = q.shape
    assert N == T * Hs * Ws and k.shape == q.shape and k.dtype == q.dtype
    orders = np.empty(H, dtype=np.int32)
    counts = np.empty((H, 6), dtype=np.int64)
    rc = lib().oracle_choose_token_orders(B, H, T, Hs, Ws, D, bq, bk, _dtype_code(q), _ptr(q),
                                          _ptr(k), float(scale), int(mode), float(param),
                                          _ptr(orders), _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_choose_token_orders: bad arguments")
    return orders, counts


def permute_tokens(x: np.ndarray, perm: np.ndarray, scatter: bool = False) -> np.ndarray:
    """Gather (out[:, i'] = x[:, perm[i']]) or scatter (out[:, perm[i']] = x[:, i'])
    of the token axis of a [B][N][H][d] array; perm is [N] (every head) or
    [H][N] (one per head)."""
    out = np.empty_like(x)
    P = np.asarray(perm)
    for h in range(x.shape[2]):
        ph = P if P.ndim == 1 else P[h]
        if scatter:
            out[:, ph, h, :] = x[:, :, h, :]
        else:
            out[:, :, h, :] = x[:, ph, h, :]
    return out


# ------------------------------------------------------------------ pyramid
def pyramid_regions(N: int, bk: int, n_levels: int):
    """(first augmented block of each level's region + total, rows per level)."""
    rb = np.zeros(n_levels + 1, np.int64)
    rr = np.zeros(n_levels + 1, np.int64)
    lib().oracle_pyramid_regions(N, bk, n_levels, _ptr(rb), _ptr(rr))
    return rb, rr[:n_levels]


def compact_pyramid(mask: np.ndarray, B: int, H: int, nQ: int, nK: int, N: int, bk: int,
                    n_levels: int, mask_head_stride: int):
    """Augmented-tile lists of a pyramid mask (1 to 4 levels): (row_ptr, kv_idx, kv_eighths),
    bit i of an entry's eighths = pooled rows i*bk/8 .. (i+1)*bk/8 - 1 of the block."""
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    L = lib()
    nnz = L.oracle_compact_pyramid(B, H, nQ, nK, N, bk, n_levels, _ptr(mask), mask_head_stride,
                                   None, None, None)
    if nnz < 0:
        raise ValueError("compact_pyramid: n_levels outside 1..4 or a mask value above it")
    row_ptr = np.zeros(B * H * nQ + 1, np.int32)
    kv = np.zeros(max(nnz, 1), np.int32)
    qm = np.zeros(max(nnz, 1), np.uint8)
    L.oracle_compact_pyramid(B, H, nQ, nK, N, bk, n_levels, _ptr(mask), mask_head_stride,
                             _ptr(row_ptr), _ptr(kv), _ptr(qm))
    return row_ptr, kv[:nnz], qm[:nnz]


def pyramid_attention(q, k, v, bq: int, bk: int, scale: float, mask: np.ndarray,
                      mask_head_stride: int, rows=None):
    """Attention where key block c attends at level mask-1 (Pyramid Sparse
    Attention page): pooled keys/values of 2^level tokens with score +
    level*ln 2. Returns (o [n][bq][D], lse [n][bq])."""
    B, N, H, D = q.shape
    nQ = -(-N // bq)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    top = int(mask.max()) - 1 if mask.size else 0
    if top >= 1 and N % (1 << top):
        raise ValueError(f"level {top} needs N divisible by {1 << top}")
    dt = _dtype_code(q)
    if rows is None:
        rows = np.arange(B * H * nQ, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, bq, D), np.float64)
    lse = np.empty((rows.size, bq), np.float64)
    rc = lib().oracle_pyramid_attention(
        B, H, N, D, bq, bk, dt, _ptr(q), *_strides(q), _ptr(k), *_strides(k), _ptr(v),
        *_strides(v), float(scale), _ptr(mask), mask_head_stride, rows.size, _ptr(rows),
        _ptr(o), _ptr(lse))
    if rc != 0:
        raise MemoryError("oracle_pyramid_attention failed to allocate")
    return o, lse


# ---------------------------------------------------------------- attention
def attention(q, k, v, bq: int, bk: int, scale: float, mask: np.ndarray,
              mask_head_stride: int, rows=None, want_gap=False, order: int = ORDER_ASCENDING):
    """Masked attention for the given rows ((b*H + h)*nQ + a); all rows if None.

    Tile gaps visit each row's kept blocks in `order` (ascending or radial).
    Returns (o [n][bq][D] fp64, lse [n][bq] fp64, gap [n][nK] fp64 or None).
    """
    B, N, H, D = q.shape
    nQ, nK = -(-N // bq), -(-N // bk)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    if rows is None:
        rows = np.arange(B * H * nQ, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    o = np.empty((n, bq, D), dtype=np.float64)
    lse = np.empty((n, bq), dtype=np.float64)
    gap = np.empty((n, nK), dtype=np.float64) if want_gap else None
    rc = lib().oracle_attention(
        B, H, N, D, bq, bk, dt, _ptr(q), *_strides(q), _ptr(k), *_strides(k),
        _ptr(v), *_strides(v), float(scale), _ptr(mask), mask_head_stride,
        n, _ptr(rows), _ptr(o), _ptr(lse), _ptr(gap) if gap is not None else None, int(order))
    if rc != 0:
        raise MemoryError("oracle_attention failed to allocate")
    return o, lse, gap


# ---------------------------------------------------------------- skip carry
def skip_step(q, k, v, bq: int, bk: int, scale: float, skip_prev: np.ndarray,
              tau: float, rows=None, order: int = ORDER_ASCENDING):
    """One denoising step of the carried skip mask, decided in fp64.

    LiteAttention summary page, sections 二, 三, 五 and 六: the effective mask of
    step s is (all tiles) minus the tiles skipped so far; attention runs over it
    while each visited tile's gap (local max minus running max, in ascending
    key-block order, or radial-centric order as in section 五) is measured;
    tiles with gap <= -tau (natural-log units) join the skip set, which only
    grows. Tiles marked at step s are still computed at step s.

    Returns (o, lse, gap, skip_new) with o/lse/gap as in attention() for the
    given rows (all rows if None) and skip_new [B][H][nQ][nK].
    """
    B, N, H, D = q.shape
    nQ, nK = -(-N // bq), -(-N // bk)
    eff = (1 - np.asarray(skip_prev, dtype=np.uint8)).reshape(B, H, nQ, nK)
    o, lse, gap = attention(q, k, v, bq, bk, scale, eff, nQ * nK, rows=rows, want_gap=True,
                            order=order)
    if rows is None:
        rows = np.arange(B * H * nQ)
    new = np.array(skip_prev, dtype=np.uint8).reshape(B * H * nQ, nK).copy()
    marked = np.nan_to_num(gap, nan=np.inf) <= -tau
    new[np.asarray(rows)] |= marked.astype(np.uint8)
    return o, lse, gap, new.reshape(B, H, nQ, nK)
