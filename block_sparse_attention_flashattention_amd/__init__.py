"""Python binding of libbsa: block-sparse video attention on MI355X (gfx950).

A thin ctypes layer over the C ABI in include/bsa.h. Every function here only
marshals arguments (torch device tensors -> pointers, strides and the current
HIP stream); all computation runs in the HIP kernels of libbsa.so. There is
no fallback: if the library is missing or fails to load, the calls raise.

Tensors: q, k, v, o are [B][N][H][d] views with d contiguous (bf16 or fp32);
masks are uint8; lists are int32; lse and tile_gap are fp32.
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = [
    "BsaError", "Shape", "shape", "lib", "BSA_BF16", "BSA_F32",
    "bsa_build_mask_radial", "bsa_pooled_workspace_bytes", "bsa_build_mask_pooled",
    "bsa_build_mask_pooled_noalloc",
    "bsa_compact_block_lists", "bsa_order_block_lists", "bsa_sparse_attn_fwd",
    "bsa_update_skip_mask", "ORDER_ASCENDING", "ORDER_RADIAL",
    "bsa_make_token_permutation", "bsa_permute_tokens", "PERM_AXES", "PERM_BOXES",
    "bsa_token_orders_workspace_bytes", "bsa_choose_token_orders", "AXIS_ORDERS",
    "bsa_pyramid_rows", "bsa_build_kv_pyramid", "bsa_build_mask_pyramid",
    "bsa_compact_pyramid_lists", "bsa_pyramid_attn_fwd", "bsa_check_block_lists",
    "bsa_status_string", "bsa_last_error",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED, BSA_ERR_CAPACITY, BSA_ERR_DEVICE = range(5)
BSA_BF16, BSA_F32 = 0, 1
ORDER_ASCENDING, ORDER_RADIAL = 0, 1
PERM_AXES, PERM_BOXES = 0, 1


class BsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{fn}: status {status} ({bsa_status_string(status)}): {detail}")


class Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "heads", "head_dim", "frames", "height", "width", "block_q", "block_k")]

    @property
    def N(self):
        return self.frames * self.height * self.width

    @property
    def nQ(self):
        return -(-self.N // self.block_q)

    @property
    def nK(self):
        return -(-self.N // self.block_k)


class Tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("stride_b", C.c_int64), ("stride_n", C.c_int64),
                ("stride_h", C.c_int64)]


def shape(B, H, d, T, Hs, Ws, Bq, Bk=64) -> Shape:
    return Shape(B, H, d, T, Hs, Ws, Bq, Bk)


_lib = None


def lib() -> C.CDLL:
    """Load libbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_flashattention_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, f32, f64, sz = (C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double,
                                     C.c_size_t)
        SP = C.POINTER(Shape)
        sig = {
            "bsa_build_mask_radial": (i32, [SP, i32, i32, p, p]),
            "bsa_pooled_workspace_bytes": (sz, [SP]),
            "bsa_build_mask_pooled": (i32, [SP, i32, Tensor, Tensor, f64, i32, f64, p, p, sz, p]),
            "bsa_build_mask_pooled_noalloc": (i32, [SP, i32, Tensor, Tensor, f64, i32, f64, p, p]),
            "bsa_compact_block_lists": (i32, [SP, p, i64, p, p, p, i64, C.POINTER(i64), p]),
            "bsa_order_block_lists": (i32, [SP, i32, p, i32, p, p, p]),
            "bsa_make_token_permutation": (i32, [SP, i32, C.POINTER(i32), p, p]),
            "bsa_permute_tokens": (i32, [SP, i32, p, i64, i32, Tensor, Tensor, p]),
            "bsa_token_orders_workspace_bytes": (sz, [SP, i32]),
            "bsa_choose_token_orders": (i32, [SP, i32, Tensor, Tensor, f64, i32, f64, p, p, p, sz,
                                              p]),
            "bsa_pyramid_rows": (i64, [SP, i32]),
            "bsa_build_kv_pyramid": (i32, [SP, i32, i32, Tensor, Tensor, Tensor, Tensor, p]),
            "bsa_build_mask_pyramid": (i32, [SP, i32, Tensor, Tensor, f64, i32,
                                             C.POINTER(f64), p, p, sz, p]),
            "bsa_compact_pyramid_lists": (i32, [SP, i32, p, i64, p, p, p, i64, C.POINTER(i64),
                                                p]),
            "bsa_pyramid_attn_fwd": (i32, [SP, i32, Tensor, Tensor, Tensor, Tensor, Tensor, i32,
                                           Tensor, p, p, p, p, f32, p]),
            "bsa_sparse_attn_fwd": (i32, [SP, i32, Tensor, Tensor, Tensor, Tensor, p, p, p, i32,
                                          f32, p, p]),
            "bsa_update_skip_mask": (i32, [SP, p, p, p, f32, p, p]),
            "bsa_check_block_lists": (i32, [SP, i32, p, p, i64, i64, i32, i32, p]),
            "bsa_status_string": (C.c_char_p, [i32]),
            "bsa_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def bsa_status_string(status: int) -> str:
    return lib().bsa_status_string(status).decode()


def bsa_last_error() -> str:
    return lib().bsa_last_error().decode()


def _check(fn: str, status: int):
    if status != BSA_OK:
        raise BsaError(fn, status, bsa_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _tensor(t) -> Tensor:
    if t is None:
        return Tensor(None, 0, 0, 0)
    if t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1):
        raise ValueError("expected a [B][N][H][d] tensor with contiguous head_dim")
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def bsa_build_mask_radial(s: Shape, h0: int, decay_base: int, mask, stream=None):
    _check("bsa_build_mask_radial",
           lib().bsa_build_mask_radial(C.byref(s), h0, decay_base, _ptr(mask), _stream(stream)))


def bsa_pooled_workspace_bytes(s: Shape) -> int:
    return int(lib().bsa_pooled_workspace_bytes(C.byref(s)))


def bsa_build_mask_pooled(s: Shape, q, k, scale: float, mode: int, param: float, mask,
                          workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bsa_build_mask_pooled",
           lib().bsa_build_mask_pooled(C.byref(s), _dtype(q), _tensor(q), _tensor(k), scale,
                                       mode, param, _ptr(mask), _ptr(workspace), nbytes,
                                       _stream(stream)))


def bsa_build_mask_pooled_noalloc(s: Shape, q, k, scale: float, mode: int, param: float, mask,
                                  stream=None):
    _check("bsa_build_mask_pooled_noalloc",
           lib().bsa_build_mask_pooled_noalloc(C.byref(s), _dtype(q), _tensor(q), _tensor(k),
                                               scale, mode, param, _ptr(mask), _stream(stream)))


def bsa_compact_block_lists(s: Shape, mask, mask_head_stride: int, skip, row_ptr, kv_idx,
                            kv_capacity: int | None = None, want_nnz: bool = False,
                            stream=None):
    """Returns the number of listed tiles when want_nnz (the call then syncs)."""
    if kv_capacity is None:
        kv_capacity = kv_idx.numel() if kv_idx is not None else 0
    nnz = C.c_int64(-1)
    _check("bsa_compact_block_lists",
           lib().bsa_compact_block_lists(C.byref(s), _ptr(mask), mask_head_stride, _ptr(skip),
                                         _ptr(row_ptr), _ptr(kv_idx), kv_capacity,
                                         C.byref(nnz) if want_nnz else None, _stream(stream)))
    return int(nnz.value) if want_nnz else None


def bsa_order_block_lists(s: Shape, order: int, row_ptr, lists_shared: int, kv_in, kv_out,
                          stream=None):
    _check("bsa_order_block_lists",
           lib().bsa_order_block_lists(C.byref(s), order, _ptr(row_ptr), lists_shared,
                                       _ptr(kv_in), _ptr(kv_out), _stream(stream)))


def bsa_make_token_permutation(s: Shape, kind: int, axes, perm, stream=None):
    ax = (C.c_int32 * 3)(*[int(a) for a in axes])
    _check("bsa_make_token_permutation",
           lib().bsa_make_token_permutation(C.byref(s), kind, ax, _ptr(perm), _stream(stream)))


# the six axis orders in the numbering of bsa_choose_token_orders
AXIS_ORDERS = ((0, 1, 2), (0, 2, 1), (1, 0, 2), (1, 2, 0), (2, 0, 1), (2, 1, 0))


def bsa_token_orders_workspace_bytes(s: Shape, dtype_code: int) -> int:
    return int(lib().bsa_token_orders_workspace_bytes(C.byref(s), dtype_code))


def bsa_choose_token_orders(s: Shape, q, k, scale: float, mode: int, param: float, order_out,
                            counts_out, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bsa_choose_token_orders",
           lib().bsa_choose_token_orders(C.byref(s), _dtype(q), _tensor(q), _tensor(k), scale,
                                         mode, param, _ptr(order_out), _ptr(counts_out),
                                         _ptr(workspace), nbytes, _stream(stream)))


def bsa_permute_tokens(s: Shape, perm, perm_head_stride: int, scatter: int, x, out,
                       stream=None):
    _check("bsa_permute_tokens",
           lib().bsa_permute_tokens(C.byref(s), _dtype(x), _ptr(perm), perm_head_stride, scatter,
                                    _tensor(x), _tensor(out), _stream(stream)))


def bsa_pyramid_rows(s: Shape, n_levels: int) -> int:
    return int(lib().bsa_pyramid_rows(C.byref(s), n_levels))


def bsa_build_kv_pyramid(s: Shape, n_levels: int, k, v, k_pyr, v_pyr, stream=None):
    _check("bsa_build_kv_pyramid",
           lib().bsa_build_kv_pyramid(C.byref(s), _dtype(k), n_levels, _tensor(k), _tensor(v),
                                      _tensor(k_pyr), _tensor(v_pyr), _stream(stream)))


def bsa_build_mask_pyramid(s: Shape, q, k, scale: float, levels_tau, mask, workspace,
                           stream=None):
    taus = (C.c_double * len(levels_tau))(*[float(t) for t in levels_tau])
    nbytes = workspace.numel() * workspace.element_size()
    _check("bsa_build_mask_pyramid",
           lib().bsa_build_mask_pyramid(C.byref(s), _dtype(q), _tensor(q), _tensor(k), scale,
                                        len(levels_tau), taus, _ptr(mask), _ptr(workspace),
                                        nbytes, _stream(stream)))


def bsa_compact_pyramid_lists(s: Shape, n_levels: int, mask, mask_head_stride: int, row_ptr,
                              kv_idx, kv_eighths, kv_capacity: int | None = None,
                              want_nnz: bool = False, stream=None):
    if kv_capacity is None:
        kv_capacity = kv_idx.numel() if kv_idx is not None else 0
    nnz = C.c_int64(-1)
    _check("bsa_compact_pyramid_lists",
           lib().bsa_compact_pyramid_lists(C.byref(s), n_levels, _ptr(mask), mask_head_stride,
                                           _ptr(row_ptr), _ptr(kv_idx), _ptr(kv_eighths),
                                           kv_capacity, C.byref(nnz) if want_nnz else None,
                                           _stream(stream)))
    return int(nnz.value) if want_nnz else None


def bsa_pyramid_attn_fwd(s: Shape, q, k, v, k_pyr, v_pyr, n_levels: int, o, lse, row_ptr,
                         kv_idx, kv_eighths, scale: float | None = None, stream=None):
    if scale is None:
        scale = 1.0 / float(s.head_dim) ** 0.5
    _check("bsa_pyramid_attn_fwd",
           lib().bsa_pyramid_attn_fwd(C.byref(s), _dtype(q), _tensor(q), _tensor(k), _tensor(v),
                                      _tensor(k_pyr), _tensor(v_pyr), n_levels, _tensor(o),
                                      _ptr(lse), _ptr(row_ptr), _ptr(kv_idx), _ptr(kv_eighths),
                                      scale, _stream(stream)))


def bsa_sparse_attn_fwd(s: Shape, q, k, v, o, lse=None, row_ptr=None, kv_idx=None,
                        lists_shared: int = 0, scale: float | None = None, tile_gap=None,
                        stream=None):
    if scale is None:
        scale = 1.0 / float(s.head_dim) ** 0.5
    _check("bsa_sparse_attn_fwd",
           lib().bsa_sparse_attn_fwd(C.byref(s), _dtype(q), _tensor(q), _tensor(k), _tensor(v),
                                     _tensor(o), _ptr(lse), _ptr(row_ptr), _ptr(kv_idx),
                                     lists_shared, scale, _ptr(tile_gap), _stream(stream)))


def bsa_update_skip_mask(s: Shape, row_ptr, kv_idx, tile_gap, tau: float, skip, stream=None):
    _check("bsa_update_skip_mask",
           lib().bsa_update_skip_mask(C.byref(s), _ptr(row_ptr), _ptr(kv_idx), _ptr(tile_gap),
                                      tau, _ptr(skip), _stream(stream)))


def bsa_check_block_lists(s: Shape, lists_shared: int, row_ptr, kv_idx, n_blocks: int = 0,
                          ascending: bool = False, kv_len: int | None = None, stream=None):
    """Debug check of block lists. numpy int32 arrays are checked on the host,
    torch tensors on the device they live on (the call then synchronises)."""
    import numpy as np
    on_device = not isinstance(row_ptr, np.ndarray)
    if on_device:
        rp, kv = _ptr(row_ptr), _ptr(kv_idx)
        n = kv_idx.numel() if kv_idx is not None else 0
        st = _stream(stream)
    else:
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        kv_idx = np.ascontiguousarray(kv_idx if kv_idx is not None else [], dtype=np.int32)
        rp, kv = row_ptr.ctypes.data, kv_idx.ctypes.data
        n, st = kv_idx.size, None
    _check("bsa_check_block_lists",
           lib().bsa_check_block_lists(C.byref(s), lists_shared, rp, kv,
                                       n if kv_len is None else kv_len, n_blocks,
                                       1 if ascending else 0, 1 if on_device else 0, st))
