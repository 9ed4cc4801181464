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

// One thread per (b, pooled row g, h, 16-byte chunk) of one level.
template <bool BF16>
__global__ void kv_pool_kernel(int64_t B, int64_t H, int64_t G, int32_t l, int64_t cpr,
                               const char* __restrict__ in, int64_t isb, int64_t isn,
                               int64_t ish, char* __restrict__ out, int64_t osb, int64_t osn,
                               int64_t osh, int64_t orow0) {
  const int64_t total = B * G * H * cpr;
  const int n = 1 << l;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % cpr;
    const int64_t r = t / cpr;
    const int64_t h = r % H;
    const int64_t bg = r / H;
    const int64_t g = bg % G, b = bg / G;
    const char* src = in + b * isb + (g * n) * isn + h * ish + c * 16;
    char* dst = out + b * osb + (orow0 + g) * osn + h * osh + c * 16;
    if constexpr (BF16) {
      f32x8 acc = {};
      for (int i = 0; i < n; ++i) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + i * isn));
        acc = acc + __builtin_convertvector(x, f32x8);
      }
      acc = acc * (1.0f / (float)n);
      *(u32x4*)dst = __builtin_bit_cast(u32x4, __builtin_convertvector(acc, bf16x8));
    } else {
      f32x4 acc = {};
      for (int i = 0; i < n; ++i) acc = acc + *(const f32x4*)(src + i * isn);
      *(f32x4*)dst = acc * (1.0f / (float)n);
    }
  }
}

inline unsigned grid_for(int64_t work, int threads, int64_t cap = 1 << 20) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_kv_pyramid(const Geom& g, int elem_bytes, int32_t n_levels, const int64_t* rb,
                             TensorArg k, TensorArg v, TensorArg kp, TensorArg vp,
                             hipStream_t st) {
  const int64_t cpr = (int64_t)g.D * elem_bytes / 16;
  const int64_t eb = elem_bytes;
  for (int32_t l = 1; l < n_levels; ++l) {
    const int64_t G = g.N >> l;
    const int64_t work = (int64_t)g.B * G * g.H * cpr;
    if (work == 0) continue;
    const int64_t orow0 = (rb[l] - rb[1]) * 64;
    for (int kvsel = 0; kvsel < 2; ++kvsel) {
      const TensorArg& in = kvsel ? v : k;
      const TensorArg& out = kvsel ? vp : kp;
      if (elem_bytes == 2)
        hipLaunchKernelGGL(kv_pool_kernel<true>, dim3(grid_for(work, 256)), dim3(256), 0, st,
                           (int64_t)g.B, (int64_t)g.H, G, l, cpr, (const char*)in.ptr,
                           in.sb * eb, in.sn * eb, in.sh * eb, (char*)out.ptr, out.sb * eb,
                           out.sn * eb, out.sh * eb, orow0);
      else
        hipLaunchKernelGGL(kv_pool_kernel<false>, dim3(grid_for(work, 256)), dim3(256), 0, st,
                           (int64_t)g.B, (int64_t)g.H, G, l, cpr, (const char*)in.ptr,
                           in.sb * eb, in.sn * eb, in.sh * eb, (char*)out.ptr, out.sb * eb,
                           out.sn * eb, out.sh * eb, orow0);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace bsa
