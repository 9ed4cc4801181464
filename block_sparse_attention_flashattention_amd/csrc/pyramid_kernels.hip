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

// Levels 1 and 2 of one tensor in one pass: one thread per (b, pair g of
// level-1 rows, h, 16-byte chunk) reads tokens 4g .. 4g+3 once and writes
// level-1 rows 2g and 2g+1 and, with two pooled levels, level-2 row g. Each
// sum is formed exactly as a separate pass per level would (from zero, one
// token at a time in ascending order: the level-2 sum continues the first
// level-1 sum), so the rows are the same bits. The last pair may hold one
// level-1 row (an odd count of them, only with one pooled level).
template <bool BF16>
__global__ void kv_pool_kernel(int64_t B, int64_t H, int64_t G1, int32_t two_levels,
                               int64_t cpr, const char* __restrict__ in, int64_t isb,
                               int64_t isn, int64_t ish, char* __restrict__ out, int64_t osb,
                               int64_t osn, int64_t osh, int64_t orow2) {
  const int64_t NG = (G1 + 1) / 2;
  const int64_t total = B * NG * H * cpr;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % cpr;
    const int64_t r = t / cpr;
    const int64_t h = r % H;
    const int64_t bg = r / H;
    const int64_t g = bg % NG, b = bg / NG;
    const bool pair = 2 * g + 1 < G1;
    const char* src = in + b * isb + (4 * g) * isn + h * ish + c * 16;
    char* dst = out + b * osb + h * osh + c * 16;
    if constexpr (BF16) {
      auto ld = [&](int i) {
        return __builtin_convertvector(__builtin_bit_cast(bf16x8, *(const u32x4*)(src + i * isn)),
                                       f32x8);
      };
      auto st = [&](int64_t row, f32x8 v) {
        *(u32x4*)(dst + row * osn) = __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));
      };
      const f32x8 x0 = ld(0), x1 = ld(1);
      f32x8 a = {};
      a = a + x0;
      a = a + x1;
      st(2 * g, a * 0.5f);
      if (pair) {
        const f32x8 x2 = ld(2), x3 = ld(3);
        f32x8 e = {};
        e = e + x2;
        e = e + x3;
        st(2 * g + 1, e * 0.5f);
        if (two_levels) st(orow2 + g, ((a + x2) + x3) * 0.25f);
      }
    } else {
      auto ld = [&](int i) { return *(const f32x4*)(src + i * isn); };
      auto st = [&](int64_t row, f32x4 v) { *(f32x4*)(dst + row * osn) = v; };
      const f32x4 x0 = ld(0), x1 = ld(1);
      f32x4 a = {};
      a = a + x0;
      a = a + x1;
      st(2 * g, a * 0.5f);
      if (pair) {
        const f32x4 x2 = ld(2), x3 = ld(3);
        f32x4 e = {};
        e = e + x2;
        e = e + x3;
        st(2 * g + 1, e * 0.5f);
        if (two_levels) st(orow2 + g, ((a + x2) + x3) * 0.25f);
      }
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
  if (n_levels < 2) return hipSuccess;
  if (n_levels > 3) return hipErrorInvalidValue;  // levels 1 and 2 at most
  const int64_t G1 = g.N >> 1;
  const int64_t work = (int64_t)g.B * ((G1 + 1) / 2) * g.H * cpr;
  if (work == 0) return hipSuccess;
  const int32_t two = n_levels == 3 ? 1 : 0;
  const int64_t orow2 = (rb[2] - rb[1]) * 64;
  for (int kvsel = 0; kvsel < 2; ++kvsel) {
    const TensorArg& in = kvsel ? v : k;
    const TensorArg& out = kvsel ? vp : kp;
    if (elem_bytes == 2)
      hipLaunchKernelGGL(kv_pool_kernel<true>, dim3(grid_for(work, 256)), dim3(256), 0, st,
                         (int64_t)g.B, (int64_t)g.H, G1, two, cpr, (const char*)in.ptr,
                         in.sb * eb, in.sn * eb, in.sh * eb, (char*)out.ptr, out.sb * eb,
                         out.sn * eb, out.sh * eb, orow2);
    else
      hipLaunchKernelGGL(kv_pool_kernel<false>, dim3(grid_for(work, 256)), dim3(256), 0, st,
                         (int64_t)g.B, (int64_t)g.H, G1, two, cpr, (const char*)in.ptr,
                         in.sb * eb, in.sn * eb, in.sh * eb, (char*)out.ptr, out.sb * eb,
                         out.sn * eb, out.sh * eb, orow2);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace bsa
