// pyramid_kernels.hip -- pooled key/value levels for pyramid attention (gfx950).
//
// Page: [PSA] "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍": key/value
// blocks kept at several resolutions, each coarser level the average of the
// finer one. Level l row g is the mean of tokens [g*2^l, (g+1)*2^l) of K (and
// of V), summed in fp32 in ascending token order, divided by 2^l and rounded
// to the tensor's type (nearest even). Levels 1.. are stored one after the
// other in k_pyr / v_pyr, each level starting at a multiple of 64 rows; the
// padding rows are not written. HBM-bound data movement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

struct Orows {
  int64_t r[4];  // r[l] = first row of level l in the pooled tensor (l = 1..3)
};

// Levels 1 .. LV of one tensor in one pass: one thread per (b, group g of
// 2^LV tokens, h, 16-byte chunk) reads tokens g*2^LV .. (g+1)*2^LV - 1 once
// and writes the 2^(LV-l) level-l rows of the group for every l. Each sum is
// formed exactly as a separate pass per level would (from zero, one token at
// a time in ascending order): the level-(l+1) sum of a group continues the
// level-l sum of its first half, so the rows are the same bits. The token
// count is a multiple of 2^LV, so every group is whole.
template <typename V, int LV>
__device__ inline void pool_group(const char* src, int64_t isn, char* dst, int64_t osn,
                                  int64_t g, const int64_t (&orow)[4]) {
  constexpr int NT = 1 << LV;
  V x[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) x[i] = V::load(src + i * isn);
  // sums[i] = sum of the first 2^l tokens of sub-group i, level by level
  typename V::acc sums[NT / 2];
#pragma unroll
  for (int i = 0; i < NT / 2; ++i) {
    typename V::acc a = {};
    a = a + V::widen(x[2 * i]);
    a = a + V::widen(x[2 * i + 1]);
    sums[i] = a;
    V::store(dst + (orow[1] + g * (NT / 2) + i) * osn, a * 0.5f);
  }
#pragma unroll
  for (int l = 2; l <= LV; ++l) {
    const int per = 1 << l, cnt = NT >> l;
#pragma unroll
    for (int i = 0; i < cnt; ++i) {
      typename V::acc a = sums[2 * i];  // level l-1 sum of the first half
#pragma unroll
      for (int t = per / 2; t < per; ++t) a = a + V::widen(x[i * per + t]);
      sums[i] = a;
      V::store(dst + (orow[l] + g * cnt + i) * osn, a * (1.0f / per));
    }
  }
}

struct Bf16Chunk {  // 8 bf16 values, summed in fp32, rounded to nearest even
  using acc = f32x8;
  u32x4 raw;
  __device__ static Bf16Chunk load(const char* p) { return {*(const u32x4*)p}; }
  __device__ static acc widen(Bf16Chunk c) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, c.raw), f32x8);
  }
  __device__ static void store(char* p, acc v) {
    *(u32x4*)p = __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));
  }
};

struct F32Chunk {  // 4 fp32 values
  using acc = f32x4;
  f32x4 raw;
  __device__ static F32Chunk load(const char* p) { return {*(const f32x4*)p}; }
  __device__ static acc widen(F32Chunk c) { return c.raw; }
  __device__ static void store(char* p, acc v) { *(f32x4*)p = v; }
};

template <typename V, int LV>
__global__ void kv_pool_kernel(int64_t B, int64_t H, int64_t NG, int64_t cpr,
                               const char* __restrict__ in, int64_t isb, int64_t isn,
                               int64_t ish, char* __restrict__ out, int64_t osb, int64_t osn,
                               int64_t osh, Orows orows) {
  const int64_t total = B * NG * H * cpr;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % cpr;
    const int64_t r = t / cpr;
    const int64_t h = r % H;
    const int64_t bg = r / H;
    const int64_t g = bg % NG, b = bg / NG;
    const char* src = in + b * isb + (g << LV) * isn + h * ish + c * 16;
    char* dst = out + b * osb + h * osh + c * 16;
    pool_group<V, LV>(src, isn, dst, osn, g, orows.r);
  }
}

inline unsigned grid_for(int64_t work, int threads, int64_t cap = 1 << 20) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

template <typename V, int LV>
hipError_t launch_levels(const Geom& g, int64_t eb, const TensorArg& in, const TensorArg& out,
                         const Orows& orows, hipStream_t st) {
  const int64_t cpr = (int64_t)g.D * eb / 16;
  const int64_t NG = g.N >> LV;
  const int64_t work = (int64_t)g.B * NG * g.H * cpr;
  if (work == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_pool_kernel<V, LV>), dim3(grid_for(work, 256)), dim3(256), 0, st,
                     (int64_t)g.B, (int64_t)g.H, NG, cpr, (const char*)in.ptr, in.sb * eb,
                     in.sn * eb, in.sh * eb, (char*)out.ptr, out.sb * eb, out.sn * eb,
                     out.sh * eb, orows);
  return hipGetLastError();
}

template <typename V>
hipError_t launch_levels(const Geom& g, int64_t eb, int32_t n_levels, const TensorArg& in,
                         const TensorArg& out, const Orows& orows, hipStream_t st) {
  if (n_levels == 2) return launch_levels<V, 1>(g, eb, in, out, orows, st);
  if (n_levels == 3) return launch_levels<V, 2>(g, eb, in, out, orows, st);
  return launch_levels<V, 3>(g, eb, in, out, orows, st);
}

}  // namespace

hipError_t launch_kv_pyramid(const Geom& g, int elem_bytes, int32_t n_levels, const int64_t* rb,
                             TensorArg k, TensorArg v, TensorArg kp, TensorArg vp,
                             hipStream_t st) {
  if (n_levels < 2) return hipSuccess;
  if (n_levels > 4) return hipErrorInvalidValue;  // levels 1 to 3 at most
  if (g.N % (int64_t(1) << (n_levels - 1))) return hipErrorInvalidValue;  // whole groups
  Orows orows{};  // first row of each pooled level in k_pyr / v_pyr
  for (int l = 1; l < n_levels; ++l) orows.r[l] = (rb[l] - rb[1]) * 64;
  for (int kvsel = 0; kvsel < 2; ++kvsel) {
    const TensorArg& in = kvsel ? v : k;
    const TensorArg& out = kvsel ? vp : kp;
    const hipError_t err =
        elem_bytes == 2 ? launch_levels<Bf16Chunk>(g, 2, n_levels, in, out, orows, st)
                        : launch_levels<F32Chunk>(g, 4, n_levels, in, out, orows, st);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace bsa
