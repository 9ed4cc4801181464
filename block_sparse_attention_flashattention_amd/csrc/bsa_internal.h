// bsa_internal.h -- declarations shared by the C-ABI host layer and the HIP
// kernel launchers of libbsa. Not installed; the public interface is bsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// Geometry derived once on the host from bsa_shape (all validated).
struct Geom {
  int32_t B, H, D, T, Hs, Ws, Bq, Bk;
  int64_t N, F, nQ, nK;
};

struct TensorArg {
  const void* ptr;
  int64_t sb, sn, sh;  // element strides
};

// ---- masks and lists (mask_kernels.hip)
hipError_t launch_radial_mask(const Geom& g, int32_t h0, int32_t beta, uint8_t* mask,
                              hipStream_t st);

size_t pooled_workspace_bytes(const Geom& g);
// Scratch bytes the pooled builder uses in `mode` (at most the workspace size),
// and the device address of the library's static scratch on the current
// device (kStaticScratchBytes; shared by every call on that device).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
size_t pooled_scratch_need(const Geom& g, int32_t mode);
hipError_t static_scratch(void** ptr);
hipError_t launch_pooled_mask(const Geom& g, int dtype, TensorArg q, TensorArg k, double scale,
                              int32_t mode, double param, uint8_t* mask, void* ws,
                              hipStream_t st, const double* levels = nullptr,
                              int32_t n_levels = 0);
hipError_t launch_pooled_global(const Geom& g, int32_t mode, double param, uint8_t* mask,
                                void* ws, hipStream_t st);

// Counts kept tiles per list row into row_ptr[1..R] and row_ptr[0] = 0, then
// turns row_ptr into its inclusive prefix sum.
hipError_t launch_compact_count_scan(const Geom& g, int64_t R, const uint8_t* mask,
                                     int64_t mask_head_stride, const uint8_t* skip,
                                     int32_t* row_ptr, hipStream_t st);
hipError_t launch_compact_scatter(const Geom& g, int64_t R, const uint8_t* mask,
                                  int64_t mask_head_stride, const uint8_t* skip,
                                  const int32_t* row_ptr, int32_t* kv_idx, hipStream_t st);
hipError_t launch_zero_row_ptr(int32_t* row_ptr, hipStream_t st);
// Pyramid lists: count + scan into row_ptr (count_only), or scatter.
// rb[0..n_levels] = first augmented block of each level region, then the end.
hipError_t launch_pyramid_lists(const Geom& g, int32_t n_levels, const int64_t* rb,
                                const uint8_t* mask, int64_t mhs, int32_t* row_ptr,
                                int32_t* kv_idx, int32_t* kv_eighths, bool count_only,
                                hipStream_t st);
// Pooled key/value levels 1..n_levels-1 (means of 2^l tokens) into k_pyr/v_pyr.
hipError_t launch_kv_pyramid(const Geom& g, int elem_bytes, int32_t n_levels, const int64_t* rb,
                             TensorArg k, TensorArg v, TensorArg kp, TensorArg vp,
                             hipStream_t st);
hipError_t launch_order_lists(const Geom& g, int64_t R, int32_t order, const int32_t* row_ptr,
                              const int32_t* kv_in, int32_t* kv_out, hipStream_t st);

hipError_t launch_skip_update(const Geom& g, const int32_t* row_ptr, const int32_t* kv_idx,
                              const float* tile_gap, float tau2, uint8_t* skip,
                              hipStream_t st);

// ---- debug checks of block lists (list_check.hip). Both return the first
// failing row (or -1) and its rule in *rule (0 = none). kv_len < 0 on the
// device takes row_ptr[R] as the length of kv.
int64_t check_lists_host(const int32_t* row_ptr, const int32_t* kv, int64_t R, int64_t kv_len,
                         int64_t n_blocks, bool ascending, int* rule);
hipError_t check_lists_device(const int32_t* row_ptr, const int32_t* kv, int64_t R,
                              int64_t kv_len, int64_t n_blocks, bool ascending, int* rule,
                              int64_t* row, hipStream_t st);

// ---- token orders (permute_kernels.hip)
hipError_t launch_make_permutation(const Geom& g, int32_t kind, const int32_t* axes,
                                   int32_t* perm, hipStream_t st);
hipError_t launch_permute_tokens(const Geom& g, int elem_bytes, const int32_t* perm,
                                 int64_t perm_head_stride, int32_t scatter, TensorArg in,
                                 TensorArg out, hipStream_t st);
hipError_t launch_zero_counts(unsigned long long* counts, int64_t n, hipStream_t st);
hipError_t launch_count_kept(const Geom& g, int32_t order, const uint8_t* mask,
                             unsigned long long* counts, hipStream_t st);
hipError_t launch_choose_order(int32_t H, const unsigned long long* counts, int32_t* order_out,
                               hipStream_t st);

// ---- attention forward
struct AttnArgs {
  TensorArg q, k, v;
  void* o;
  int64_t osb, osn, osh;
  float* lse;
  const int32_t* row_ptr;  // NULL = dense
  const int32_t* kv_idx;
  int32_t lists_shared;
  float scale;
  float* tile_gap;
  // pyramid attention (kv_eighths non-NULL): pooled levels and region starts
  TensorArg kp{}, vp{};
  const int32_t* kv_eighths = nullptr;
  int64_t pyr_rb[5] = {0, 0, 0, 0, 0};
};

hipError_t launch_attn_bf16(const Geom& g, const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_f32(const Geom& g, const AttnArgs& a, hipStream_t st);

}  // namespace bsa
