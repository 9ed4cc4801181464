// permute_kernels.hip -- token orders before blocking, and the gather and
// scatter that move Q, K, V into such an order and O back (gfx950).
//
// Pages: [PARO] PAROAttention summary page (arXiv:2506.16054), section 二:
// flattening a video to one sequence separates tokens that attend to each
// other; reordering them by one of the six orders of the frame, row and
// column axes (one per head) turns scattered patterns into block-shaped
// ones. [VMoBA] VMoBA summary page (arXiv:2506.23858), section 三: blocks
// made of temporal chunks, spatial patches or spatio-temporal cubes.
//
// Both kernels are pure data movement (integer index math; bytes copied as
// they are), bound by HBM bandwidth. The per-head choice among the six axis
// orders counts the tiles a pooled mask keeps under each order (exact
// integer sums; the orchestration is in api.cpp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One thread per original token i = (t*Hs + y)*Ws + x: its new position
// i', and perm[i'] = i.
//   kind 0: axes (A, B, C) = slowest, middle, fastest of (t, y, x):
//           i' = (co[A]*ext[B] + co[B])*ext[C] + co[C].
//   kind 1: boxes of (ct, cy, cx) tokens, smaller at the far edges, in
//           (t, y, x) order, tokens inside a box in (t, y, x) order:
//           i' = tokens of all earlier boxes + offset inside the box.
__global__ void make_perm_kernel(int64_t T, int64_t Hs, int64_t Ws, int32_t kind, int32_t a0,
                                 int32_t a1, int32_t a2, int32_t* __restrict__ perm) {
  const int64_t N = T * Hs * Ws;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < N;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / (Hs * Ws), y = (i / Ws) % Hs, x = i % Ws;
    int64_t ip;
    if (kind == 0) {
      const int64_t co[3] = {t, y, x}, ext[3] = {T, Hs, Ws};
      ip = (co[a0] * ext[a1] + co[a1]) * ext[a2] + co[a2];
    } else {
      const int64_t bt = t / a0, by = y / a1, bx = x / a2;
      const int64_t st = min((int64_t)a0, T - bt * a0);
      const int64_t sy = min((int64_t)a1, Hs - by * a1);
      const int64_t sx = min((int64_t)a2, Ws - bx * a2);
      const int64_t before = bt * a0 * Hs * Ws + st * (by * a1) * Ws + st * sy * (bx * a2);
      ip = before + ((t - bt * a0) * sy + (y - by * a1)) * sx + (x - bx * a2);
    }
    perm[ip] = (int32_t)i;
  }
}

// One thread per 16 bytes of a row: gather out[b][i'][h] = in[b][perm_h[i']][h]
// or scatter out[b][perm_h[i']][h] = in[b][i'][h]; perm_h = perm + h*phs.
// Consecutive threads walk the head_dim bytes, then heads, then positions i'.
__global__ void permute_rows_kernel(int64_t B, int64_t N, int64_t H, int64_t cpr,
                                    const int32_t* __restrict__ perm, int64_t phs,
                                    int32_t scatter, const char* __restrict__ in, int64_t isb,
                                    int64_t isn, int64_t ish, char* __restrict__ out,
                                    int64_t osb, int64_t osn, int64_t osh) {
  const int64_t total = B * N * H * cpr;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % cpr;
    const int64_t r = t / cpr;
    const int64_t h = r % H;
    const int64_t bi = r / H;
    const int64_t i = bi % N, b = bi / N;
    const int64_t j = perm[h * phs + i];
    if ((uint64_t)j >= (uint64_t)N) continue;  // not a token index: nothing moves
    const int64_t src = scatter ? i : j, dst = scatter ? j : i;
    const u32x4 v = *(const u32x4*)(in + b * isb + src * isn + h * ish + c * 16);
    *(u32x4*)(out + b * osb + dst * osn + h * osh + c * 16) = v;
  }
}

// counts[i] = 0 for i < n (a kernel rather than a memset, so that the call
// can sit in a captured graph).
__global__ void zero_counts_kernel(unsigned long long* counts, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    counts[i] = 0;
}

// Kept tiles of each (b, h) mask slice of `per` bytes, added to
// counts[h * kOrders + order]: 16 mask bytes per thread and step, a wave
// reduction, one 64-bit atomic per wave (integer sums: any order gives the
// same total). grid.y = B * H.
constexpr int kOrders = 6;
__global__ void count_kept_kernel(int64_t per, int32_t H, int32_t order,
                                  const uint8_t* __restrict__ mask,
                                  unsigned long long* __restrict__ counts) {
  const int64_t bh = blockIdx.y;
  const uint8_t* m = mask + bh * per;
  unsigned long long n = 0;
  for (int64_t i = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * 16; i < per;
       i += (int64_t)gridDim.x * blockDim.x * 16) {
    if (i + 16 <= per && ((uintptr_t)(m + i) & 15) == 0) {
      const u32x4 v = *(const u32x4*)(m + i);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) n += ((v[w] >> (8 * b)) & 0xff) != 0;
    } else {
      for (int64_t j = i; j < per && j < i + 16; ++j) n += m[j] != 0;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off);
  if ((threadIdx.x & 63) == 0 && n) atomicAdd(&counts[(bh % H) * kOrders + order], n);
}

// Per head: the order with the fewest kept tiles, ties to the lower index.
__global__ void choose_order_kernel(int32_t H, const unsigned long long* __restrict__ counts,
                                    int32_t* __restrict__ order_out) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  int best = 0;
  for (int o = 1; o < kOrders; ++o)
    if (counts[h * kOrders + o] < counts[h * kOrders + best]) best = o;
  order_out[h] = best;
}

inline unsigned grid_for(int64_t work, int threads, int64_t cap = 1 << 20) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_make_permutation(const Geom& g, int32_t kind, const int32_t* axes,
                                   int32_t* perm, hipStream_t st) {
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(make_perm_kernel, dim3(grid_for(g.N, 256)), dim3(256), 0, st, (int64_t)g.T,
                     (int64_t)g.Hs, (int64_t)g.Ws, kind, axes[0], axes[1], axes[2], perm);
  return hipGetLastError();
}

hipError_t launch_permute_tokens(const Geom& g, int elem_bytes, const int32_t* perm,
                                 int64_t perm_head_stride, int32_t scatter, TensorArg in,
                                 TensorArg out, hipStream_t st) {
  const int64_t cpr = (int64_t)g.D * elem_bytes / 16;
  const int64_t total = (int64_t)g.B * g.N * g.H * cpr;
  if (total == 0) return hipSuccess;
  const int64_t eb = elem_bytes;
  hipLaunchKernelGGL(permute_rows_kernel, dim3(grid_for(total, 256)), dim3(256), 0, st,
                     (int64_t)g.B, g.N, (int64_t)g.H, cpr, perm, perm_head_stride, scatter,
                     (const char*)in.ptr, in.sb * eb, in.sn * eb, in.sh * eb, (char*)out.ptr,
                     out.sb * eb, out.sn * eb, out.sh * eb);
  return hipGetLastError();
}

hipError_t launch_zero_counts(unsigned long long* counts, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_counts_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, counts, n);
  return hipGetLastError();
}

hipError_t launch_count_kept(const Geom& g, int32_t order, const uint8_t* mask,
                             unsigned long long* counts, hipStream_t st) {
  const int64_t per = g.nQ * g.nK, BH = (int64_t)g.B * g.H;
  if (per == 0 || BH == 0) return hipSuccess;
  const unsigned gx = grid_for((per + 16 * 256 - 1) / (16 * 256), 1, 1024);
  hipLaunchKernelGGL(count_kept_kernel, dim3(gx, (unsigned)BH), dim3(256), 0, st, per, g.H,
                     order, mask, counts);
  return hipGetLastError();
}

hipError_t launch_choose_order(int32_t H, const unsigned long long* counts, int32_t* order_out,
                               hipStream_t st) {
  if (H == 0) return hipSuccess;
  hipLaunchKernelGGL(choose_order_kernel, dim3((H + 63) / 64), dim3(64), 0, st, H, counts,
                     order_out);
  return hipGetLastError();
}

}  // namespace bsa
