// attn_f32.hip -- fp32 path of the block-sparse attention forward (gfx950).
//
// A plain VALU kernel for fp32 inputs (the small fp32 workload): one
// workgroup per (b, h, row block), one thread per query row, K and V tiles of
// the listed key blocks staged in LDS. Online softmax in log2 units
// ([Lite] LiteAttention summary page, sections 五 and 六), whole tiles kept
// or dropped by the list ([PSA] "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍").
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kBk = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  int64_t qsb, qsn, qsh, ksb, ksn, ksh, vsb, vsn, vsh, osb, osn, osh;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* kv_idx;
  float* tile_gap;
  int32_t lists_shared;
  float sl2;  // scale * log2(e)
  int64_t N, nQ, nK;
  int32_t H;
};

template <int D, int BQ>
__global__ __launch_bounds__(BQ) void attn_f32_kernel(const F32Params p) {
  __shared__ float Ks[kBk][D + 1];
  __shared__ float Vs[kBk][D];
  __shared__ float Ss[kBk][BQ];
  __shared__ float gp[BQ];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;  // (b*H + h)*nQ + a
  const int64_t bh = row / p.nQ, a = row - bh * p.nQ;
  const int64_t b = bh / p.H, h = bh - b * p.H;
  const int64_t i = a * BQ + tid;
  const bool valid = i < p.N;

  float qv[D], ov[D];
  const float* qp = p.q + b * p.qsb + i * p.qsn + h * p.qsh;
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = valid ? qp[x] : 0.f;
    ov[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int64_t e0 = 0, e1 = p.nK, gbase = 0;
  if (p.row_ptr) {
    const int64_t lr = p.lists_shared ? a : row;
    e0 = p.row_ptr[lr];
    e1 = p.row_ptr[lr + 1];
    if (p.lists_shared) gbase = bh * (int64_t)p.row_ptr[p.nQ];
  }
  const float* kb = p.k + b * p.ksb + h * p.ksh;
  const float* vb = p.v + b * p.vsb + h * p.vsh;
  for (int64_t e = e0; e < e1; ++e) {
    const int64_t c = p.row_ptr ? p.kv_idx[e] : e;
    const int64_t j0 = c * kBk;
    const int nj = (int)min((int64_t)kBk, p.N - j0);
    __syncthreads();
    for (int t = tid; t < kBk * D; t += BQ) {
      const int r = t / D, x = t - r * D;
      Ks[r][x] = r < nj ? kb[(j0 + r) * p.ksn + x] : 0.f;
      Vs[r][x] = r < nj ? vb[(j0 + r) * p.vsn + x] : 0.f;
    }
    __syncthreads();
    float mloc = -INFINITY;
    for (int r = 0; r < nj; ++r) {
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) s = fmaf(qv[x], Ks[r][x], s);
      s *= p.sl2;
      Ss[r][tid] = s;
      mloc = fmaxf(mloc, s);
    }
    if (p.tile_gap) gp[tid] = valid ? mloc - m : -INFINITY;
    const float mnew = fmaxf(m, mloc);
    const float alpha = exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int x = 0; x < D; ++x) ov[x] *= alpha;
    for (int r = 0; r < nj; ++r) {
      const float pr = exp2f(Ss[r][tid] - mnew);
      l += pr;
#pragma unroll
      for (int x = 0; x < D; ++x) ov[x] = fmaf(pr, Vs[r][x], ov[x]);
    }
    m = mnew;
    if (p.tile_gap) {
      __syncthreads();
      if (tid == 0) {
        float g = -INFINITY;
        for (int t = 0; t < BQ; ++t) g = fmaxf(g, gp[t]);
        p.tile_gap[gbase + e] = g;
      }
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = p.o + b * p.osb + i * p.osn + h * p.osh;
#pragma unroll
  for (int x = 0; x < D; ++x) op[x] = ov[x] * inv;
  if (p.lse) p.lse[bh * p.N + i] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int D, int BQ>
hipError_t launch(const Geom& g, const F32Params& p, hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.H * g.nQ;
  hipLaunchKernelGGL((attn_f32_kernel<D, BQ>), dim3((unsigned)rows), dim3(BQ), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const Geom& g, const AttnArgs& a, hipStream_t st) {
  if ((int64_t)g.B * g.H * g.nQ == 0) return hipSuccess;
  F32Params p;
  p.q = (const float*)a.q.ptr;
  p.k = (const float*)a.k.ptr;
  p.v = (const float*)a.v.ptr;
  p.o = (float*)a.o;
  p.qsb = a.q.sb; p.qsn = a.q.sn; p.qsh = a.q.sh;
  p.ksb = a.k.sb; p.ksn = a.k.sn; p.ksh = a.k.sh;
  p.vsb = a.v.sb; p.vsn = a.v.sn; p.vsh = a.v.sh;
  p.osb = a.osb; p.osn = a.osn; p.osh = a.osh;
  p.lse = a.lse;
  p.row_ptr = a.row_ptr;
  p.kv_idx = a.kv_idx;
  p.tile_gap = a.tile_gap;
  p.lists_shared = a.lists_shared;
  p.sl2 = a.scale * kLog2e;
  p.N = g.N; p.nQ = g.nQ; p.nK = g.nK; p.H = g.H;
  if (g.D == 64) return g.Bq == 64 ? launch<64, 64>(g, p, st) : launch<64, 128>(g, p, st);
  return g.Bq == 64 ? launch<128, 64>(g, p, st) : launch<128, 128>(g, p, st);
}

}  // namespace bsa
