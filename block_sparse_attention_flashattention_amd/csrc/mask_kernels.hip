// mask_kernels.hip -- block-mask builders, list compaction and ordering and
// the skip-mask update of libbsa (gfx950). These are small, latency- or HBM-bound kernels
// around the attention forward; none of them is a dense contraction.
//
// Pages: [Radial] "MIT实验室推出Radial Attention：让视频AI生成快如闪电的神奇技术";
// [PSA] "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍";
// [VMoBA] VMoBA summary page (arXiv:2506.23858); [Lite] LiteAttention
// summary page (arXiv:2511.11062).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kWave = 64;

// ------------------------------------------------------------------ radial
// Window of frame distance `dist` under the radial rule ([Radial]: weight
// falls off with frame distance; a fixed map; n log n cost). The band of a
// distance is its number of base-beta digits; the half-width is h0 divided
// by beta once per band down to half a key block (bands 0..rstar); farther
// bands keep that width and thin out the distances instead.
__device__ inline bool radial_distance_kept(int64_t dist, int32_t h0, int32_t beta,
                                            int32_t rstar, int32_t half_blk, int64_t* h) {
  int band = 0;
  for (int64_t x = dist; x > 0; x /= beta) ++band;
  if (band <= rstar) {
    int64_t w = h0;
    for (int i = 0; i < band; ++i) w /= beta;
    *h = w;
    return true;
  }
  int64_t period = 1;
  for (int i = rstar; i < band; ++i) period *= beta;
  *h = half_blk;
  return dist % period == 0;
}

// One thread per tile. For each pair of frames the two blocks touch, the
// tile holds a kept token pair iff the distance is kept and the gap between
// the blocks' in-frame position intervals is below the window.
__global__ void radial_mask_kernel(int64_t N, int64_t F, int32_t Bq, int32_t Bk, int64_t nK,
                                   int64_t tiles, int32_t h0, int32_t beta, int32_t rstar,
                                   uint8_t* __restrict__ mask) {
  const int64_t half_blk = Bk / 2;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < tiles;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t a = t / nK, c = t - a * nK;
    const int64_t i0 = a * Bq, i1 = min(N, i0 + Bq);
    const int64_t j0 = c * Bk, j1 = min(N, j0 + Bk);
    bool keep = false;
    for (int64_t tq = i0 / F; tq <= (i1 - 1) / F && !keep; ++tq) {
      const int64_t qlo = max(i0, tq * F) - tq * F;
      const int64_t qhi = min(i1, tq * F + F) - 1 - tq * F;
      for (int64_t tk = j0 / F; tk <= (j1 - 1) / F && !keep; ++tk) {
        const int64_t klo = max(j0, tk * F) - tk * F;
        const int64_t khi = min(j1, tk * F + F) - 1 - tk * F;
        const int64_t gap = max((int64_t)0, max(klo - qhi, qlo - khi));
        int64_t h;
        if (radial_distance_kept(tq > tk ? tq - tk : tk - tq, h0, beta, rstar,
                                 (int32_t)half_blk, &h) &&
            gap < h)
          keep = true;
      }
    }
    mask[t] = keep ? 1 : 0;
  }
}

// ------------------------------------------------------------------ pooled
// Four consecutive input elements (channels x .. x+3, 16-byte aligned rows)
// as loaded: 8 bytes of bf16 (DT 0) or 16 of fp32 (DT 1).
template <int DT>
struct Raw4;
template <>
struct Raw4<0> {
  uint2 u;
};
template <>
struct Raw4<1> {
  float4 f;
};
template <int DT>
__device__ inline Raw4<DT> load4(const void* p, int64_t off) {
  if constexpr (DT == 0) return {*(const uint2*)((const uint16_t*)p + off)};
  else return {*(const float4*)((const float*)p + off)};
}
// acc[c] += element c, widened to fp64 (exact), one rounded add per channel.
template <int DT>
__device__ inline void add4(double (&acc)[4], const Raw4<DT>& r) {
  if constexpr (DT == 0) {
    acc[0] = acc[0] + (double)__uint_as_float(r.u.x << 16);
    acc[1] = acc[1] + (double)__uint_as_float(r.u.x & 0xffff0000u);
    acc[2] = acc[2] + (double)__uint_as_float(r.u.y << 16);
    acc[3] = acc[3] + (double)__uint_as_float(r.u.y & 0xffff0000u);
  } else {
    acc[0] = acc[0] + (double)r.f.x;
    acc[1] = acc[1] + (double)r.f.y;
    acc[2] = acc[2] + (double)r.f.z;
    acc[3] = acc[3] + (double)r.f.w;
  }
}

// Block means of Q (row blocks) and K (column blocks): one thread per
// (b*H + h, block, four channels); each channel's tokens summed in ascending
// order, one division. The sum is a chain of dependent adds, so the loads of
// U tokens are issued together, as raw words, before they are added in order:
// the kernel is bound by memory latency unless many loads are in flight.
template <int DT, int U>
__global__ void pool_mean_kernel(int64_t N, int32_t H, int32_t D, int32_t Bq, int32_t Bk,
                                 int64_t nQ, int64_t nK, int64_t BH, TensorArg q, TensorArg k,
                                 double* __restrict__ qbar, double* __restrict__ kbar) {
  const int32_t D4 = D / 4;
  const int64_t per = (nQ + nK) * D4;
  const int64_t total = BH * per;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = t / per;
    const int64_t rem = t - bh * per;
    const int64_t blk = rem / D4;
    const int32_t x = 4 * (int32_t)(rem - blk * D4);
    const int64_t b = bh / H, h = bh - b * H;
    const bool isq = blk < nQ;
    const int64_t bi = isq ? blk : blk - nQ;
    const int32_t bs = isq ? Bq : Bk;
    const TensorArg& in = isq ? q : k;
    const int64_t i0 = bi * bs, i1 = min(N, i0 + bs);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const int64_t base = b * in.sb + h * in.sh + x;
    int64_t i = i0;
    for (; i + U <= i1; i += U) {
      Raw4<DT> r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) r[u] = load4<DT>(in.ptr, base + (i + u) * in.sn);
#pragma unroll
      for (int u = 0; u < U; ++u) add4<DT>(acc, r[u]);
    }
    for (; i < i1; ++i) add4<DT>(acc, load4<DT>(in.ptr, base + i * in.sn));
    const double n = (double)(i1 - i0);
    double* out = isq ? qbar + (bh * nQ + bi) * D : kbar + (bh * nK + bi) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) out[x + c] = acc[c] / n;
  }
}

// Pooled scores S[bh][a][c] = scale * (sum over x ascending of qbar*kbar),
// every product and sum rounded on its own (no fused multiply-add). A
// workgroup of 8 x 32 threads computes a 64 x 64 tile: thread (ty, tx) owns
// rows 8ty .. 8ty+7 and columns 2tx, 2tx+1, and every output keeps its own
// sum in ascending channel order (16 independent chains per thread). The
// channels are staged through LDS 16 at a time, channel-major, so a thread's
// eight rows (two columns) are contiguous and come in a few wide reads; the
// next stage's operands are loaded into registers while the current one is
// computed. The kernel is bound by the fp64 multiply and add issue.
constexpr int kScoreTy = 8, kScoreTx = 32;             // threads per column / row of the tile
constexpr int kScoreRows = 8, kScoreCols = 2;          // outputs per thread
constexpr int kScoreTile = kScoreTy * kScoreRows;      // 64 rows and 64 columns per tile
static_assert(kScoreTx * kScoreCols == kScoreTile, "square tile");
constexpr int kScoreThreads = kScoreTy * kScoreTx;
constexpr int kScoreX = 16;                            // channels per LDS stage
__global__ __launch_bounds__(kScoreThreads) void pooled_scores_kernel(
    int32_t D, int64_t nQ, int64_t nK, double scale, const double* __restrict__ qbar,
    const double* __restrict__ kbar, double* __restrict__ S) {
#pragma clang fp contract(off)
  // [channel][row]; two doubles of padding keep the staging stores spread
  __shared__ __attribute__((aligned(16))) double qs[kScoreX][kScoreTile + 2];
  __shared__ __attribute__((aligned(16))) double ks[kScoreX][kScoreTile + 2];
  const int64_t bh = blockIdx.z;
  const int64_t a0 = (int64_t)blockIdx.y * kScoreTile, c0 = (int64_t)blockIdx.x * kScoreTile;
  const int tid = threadIdx.x, tx = tid % kScoreTx, ty = tid / kScoreTx;
  double acc[kScoreRows][kScoreCols];
#pragma unroll
  for (int i = 0; i < kScoreRows; ++i)
#pragma unroll
    for (int j = 0; j < kScoreCols; ++j) acc[i][j] = 0.0;
  constexpr int kPer = kScoreTile * kScoreX / kScoreThreads;  // staged values per thread
  double pq[kPer], pk[kPer];
  auto fetch = [&](int x0) {
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int e = tid + s * kScoreThreads;  // e = row * kScoreX + channel
      const int r = e / kScoreX, x = x0 + e % kScoreX;
      pq[s] = (a0 + r < nQ && x < D) ? qbar[(bh * nQ + a0 + r) * D + x] : 0.0;
      pk[s] = (c0 + r < nK && x < D) ? kbar[(bh * nK + c0 + r) * D + x] : 0.0;
    }
  };
  fetch(0);
  for (int x0 = 0; x0 < D; x0 += kScoreX) {
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int e = tid + s * kScoreThreads;
      qs[e % kScoreX][e / kScoreX] = pq[s];
      ks[e % kScoreX][e / kScoreX] = pk[s];
    }
    __syncthreads();
    if (x0 + kScoreX < D) fetch(x0 + kScoreX);
    const int xn = min(kScoreX, D - x0);
    for (int xx = 0; xx < xn; ++xx) {
      double qv[kScoreRows], kv[kScoreCols];
#pragma unroll
      for (int i = 0; i < kScoreRows; ++i) qv[i] = qs[xx][ty * kScoreRows + i];
#pragma unroll
      for (int j = 0; j < kScoreCols; ++j) kv[j] = ks[xx][tx * kScoreCols + j];
#pragma unroll
      for (int i = 0; i < kScoreRows; ++i)
#pragma unroll
        for (int j = 0; j < kScoreCols; ++j)
          acc[i][j] = __dadd_rn(acc[i][j], __dmul_rn(qv[i], kv[j]));
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kScoreRows; ++i)
#pragma unroll
    for (int j = 0; j < kScoreCols; ++j) {
      const int64_t a = a0 + ty * kScoreRows + i, c = c0 + tx * kScoreCols + j;
      if (a < nQ && c < nK) S[(bh * nQ + a) * nK + c] = __dmul_rn(scale, acc[i][j]);
    }
}

// acc + a[0] + a[1] + ... + a[n-1], added one at a time in that order (the
// rounding of a loop on one thread). Every lane of the calling wave reads the
// same LDS words (a broadcast), 16 ahead of the additions that use them.
__device__ inline double ordered_sum(const double* a, int64_t n, double acc) {
  int64_t c = 0;
  for (; c + 16 <= n; c += 16) {
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = a[c + u];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc = acc + v[u];
  }
  for (; c < n; ++c) acc = acc + a[c];
  return acc;
}

// The same sum as ordered_sum (acc + a[0] + ... + a[n-1] in that order), with
// the LDS reads two values at a time and one 16-value chunk ahead of the
// additions, so the chain of adds does not wait for the reads. `a` is
// 16-byte aligned.
__device__ inline double ordered_sum_ahead(const double* a, int64_t n, double acc) {
  typedef double d2 __attribute__((ext_vector_type(2)));
  const d2* a2 = (const d2*)a;
  int64_t c = 0;
  if (n >= 16) {
    d2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = a2[u];
    for (; c + 32 <= n; c += 16) {
      d2 y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = a2[(c + 16) / 2 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc = acc + x[u].x;
        acc = acc + x[u].y;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = y[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc = acc + x[u].x;
      acc = acc + x[u].y;
    }
    c += 16;
  }
  for (; c < n; ++c) acc = acc + a[c];
  return acc;
}

// Order-preserving map of a double to 64 bits (larger value -> larger key;
// -0 and +0 map alike).
__device__ inline uint64_t order_key(double v) {
  if (v == 0.0) v = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}


constexpr int kSelectThreads = 256;
constexpr int kPooledMaxBlocks = 2048;  // rows held in LDS by the select kernels
// Longer rows (up to kLongMaxBlocks key blocks) take the long-row kernels:
// one lane per row for the row statistics, one workgroup per row, keys in
// registers, for the selection.
constexpr int kLongMaxBlocks = 8192;
constexpr int kLongThreads = 512;
constexpr int kLongKeys = kLongMaxBlocks / kLongThreads;  // keys per thread
constexpr int kLongBatch = 512;   // pairs sorted per step of the cumulative walk
constexpr int kLongCap = 1024;    // LDS entries of a step
// First mask byte of a row left to the full sort (mask values are 0..3).
constexpr uint8_t kSelectMarker = 0xFF;
// Rows per workgroup of the one-wave-per-row select (at most; fewer when their
// LDS would pass 64 KiB), and of the pass that finishes the rows it marked
// (their markers read by one wave at once).
constexpr int kSelectRowsPerGroup = 4;
constexpr int kMarkedRowsPerGroup = 64;
static_assert(kMarkedRowsPerGroup <= kWave, "one marker per lane");

// Bitonic sort of the pairs (ks[t], ki[t]), t < P, P a power of two, into
// descending order_key of the score, ascending block index on equal keys
// (for scores: higher score first, lower block on ties; -0 and +0 alike).
// Padding to a power of two is key 0 with index -1, below every score's key.
// Keys and indices in separate arrays (12 bytes of LDS traffic per access
// instead of a padded 16-byte record); each compare-exchange is branch-free
// (both elements written back). The used waves each own a contiguous segment
// of P / nwu keys; a stage whose pairs stay in the segment runs without a
// workgroup barrier (a wave's LDS accesses are ordered), only the stages with
// partner distance >= P / nwu synchronise the workgroup.
__device__ inline void sort_keys(uint64_t* ks, int32_t* ki, int P) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int pairs = P / 2;
  // waves with pairs to order, pairs per used wave, keys per used wave
  const int nwu = __builtin_amdgcn_readfirstlane(min(nw, max(1, pairs / 64)));
  const int pw = __builtin_amdgcn_readfirstlane(pairs / nwu);
  const int seg = __builtin_amdgcn_readfirstlane(P / nwu);
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const bool cross = j >= seg;
      if (cross) __syncthreads();
      if (w < nwu) {
        const int lj = __builtin_ctz(j);
        for (int p = w * pw + lane; p < (w + 1) * pw; p += 64) {
          const int i = ((p >> lj) << (lj + 1)) | (p & (j - 1));
          const int l = i | j;
          const uint64_t xs = ks[i], ys = ks[l];
          const int xi = ki[i], yi = ki[l];
          const bool up = (i & kk) == 0;
          // y belongs before x (indices are distinct except among padding)
          const bool yfirst = ys > xs || (ys == xs && yi < xi);
          const bool swap = up == yfirst;
          ks[i] = swap ? ys : xs;
          ki[i] = swap ? yi : xi;
          ks[l] = swap ? xs : ys;
          ki[l] = swap ? xi : yi;
        }
      }
      if (cross)
        __syncthreads();
      else
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  }
  __syncthreads();
}

constexpr int kTopM = 128;  // cumulative mass: pairs sorted before a full sort is needed

// The same bitonic network as sort_keys for kTopM = 128 pairs, run by one
// wave in registers: element e sits in lane e % 64, register e / 64;
// partners at distance 64 are the lane's two registers, closer ones come
// from lane ^ j by a cross-lane shuffle, so no stage waits on LDS. Reads the
// pairs from (ks, ki) and writes them back sorted; called by the first wave.
__device__ inline void sort128_wave(uint64_t* ks, int32_t* ki) {
  const int lane = threadIdx.x & 63;
  uint64_t k[2] = {ks[lane], ks[lane + 64]};
  int32_t x[2] = {ki[lane], ki[lane + 64]};
  for (int kk = 2; kk <= 128; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j == 64) {
        // elements lane (lower) and lane + 64 of this lane; kk = 128, so the
        // lower position takes the element that comes first
        const bool first0 = k[0] > k[1] || (k[0] == k[1] && x[0] < x[1]);
        if (!first0) {
          const uint64_t kt = k[0];
          const int32_t xt = x[0];
          k[0] = k[1];
          x[0] = x[1];
          k[1] = kt;
          x[1] = xt;
        }
        continue;
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = r * 64 + lane;
        const uint32_t lo = __shfl_xor((uint32_t)k[r], j);
        const uint32_t hi = __shfl_xor((uint32_t)(k[r] >> 32), j);
        const uint64_t ko = ((uint64_t)hi << 32) | lo;
        const int32_t xo = __shfl_xor(x[r], j);
        const bool lower = (e & j) == 0, up = (e & kk) == 0;
        const bool mine_first = k[r] > ko || (k[r] == ko && x[r] < xo);
        // the lower position of an ascending pair holds the first element
        const bool keep = (lower == up) == mine_first;
        k[r] = keep ? k[r] : ko;
        x[r] = keep ? x[r] : xo;
      }
    }
  }
  ks[lane] = k[0];
  ki[lane] = x[0];
  ks[lane + 64] = k[1];
  ki[lane + 64] = x[1];
}

// Slot for this lane's item among those of the workgroup with `pred` set, in
// no particular order: one LDS atomic per wave (on *count) instead of one per
// item. Called by every lane of the wave.
__device__ inline int wave_append(bool pred, int32_t* count) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = __builtin_amdgcn_ballot_w64(pred);
  int base = 0;
  if (lane == 0 && m) base = atomicAdd(count, __popcll(m));
  base = __shfl(base, 0);
  return base + __popcll(m & ((1ull << lane) - 1));
}

// Key of the T-th pair of the row in (score desc, index asc) order, fixed 4
// bits at a time from the top (radix select over order_key of the scores),
// and how many pairs with exactly that key are among the first T (taken in
// ascending block index) and exist in all. Once at most 64 pairs match the
// fixed prefix, one wave ranks those pairs' keys directly instead of running
// the remaining passes. Called by the whole workgroup.
struct RowCut {
  uint64_t key;
  int32_t take_eq;
  int32_t n_eq;
};
__device__ inline RowCut select_kth(const double* s, int64_t nK, int T) {
  __shared__ int32_t hist[16];
  __shared__ uint64_t rs_prefix;
  __shared__ int32_t rs_want, rs_eq;
  __shared__ uint64_t cand[64];
  __shared__ int32_t ncand;
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) {
    rs_prefix = 0;
    rs_want = T;
    rs_eq = INT32_MAX;
  }
  if (tid < 16) hist[tid] = 0;
  __syncthreads();
  for (int shift = 60; shift >= 0; shift -= 4) {
    const uint64_t prefix = rs_prefix;
    const uint64_t pmask = shift >= 60 ? 0 : (~0ull << (shift + 4));
    // per-wave digit counts by ballot (lane d counts digit d), one LDS atomic
    // per wave and digit: the keys crowd into few digits, where one atomic
    // per key would serialise
    int mycnt = 0;
    for (int64_t c0 = 0; c0 < nK; c0 += blockDim.x) {
      const int64_t c = c0 + tid;
      const uint64_t u = c < nK ? order_key(s[c]) : 0;
      const bool match = c < nK && (u & pmask) == prefix;
      const int dig = (int)((u >> shift) & 15);
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const int n = __popcll(__builtin_amdgcn_ballot_w64(match && dig == d));
        mycnt += lane == d ? n : 0;
      }
    }
    if (lane < 16 && mycnt) atomicAdd(&hist[lane], mycnt);
    __syncthreads();
    if (tid < 64) {
      // the highest bucket b whose count from the top (buckets b .. 15)
      // reaches the pairs still wanted
      const int want = rs_want;
      int sfx = 0;
      if (lane < 16)
        for (int j = lane; j < 16; ++j) sfx += hist[j];
      const uint64_t m = __builtin_amdgcn_ballot_w64(lane < 16 && sfx >= want);
      const int b = m ? 63 - __builtin_clzll(m) : 0;
      if (lane == b) {
        rs_prefix = prefix | ((uint64_t)b << shift);
        rs_want = want - (sfx - hist[b]);
        rs_eq = hist[b];
      }
      // cleared for the next pass once this wave has read it (a wave's LDS
      // accesses are ordered); the barrier below publishes it
      if (lane < 16) hist[lane] = 0;
    }
    __syncthreads();
    if (shift > 0 && rs_eq <= 64) {
      // the pairs left: key bits above shift equal to the prefix
      const uint64_t pm = ~0ull << shift, pre = rs_prefix;
      if (tid == 0) ncand = 0;
      __syncthreads();
      for (int64_t c0 = 0; c0 < nK; c0 += blockDim.x) {
        const int64_t c = c0 + tid;
        const uint64_t u = c < nK ? order_key(s[c]) : 0;
        const bool hit = c < nK && (u & pm) == pre;
        const int pos = wave_append(hit, &ncand);
        if (hit) cand[pos] = u;
      }
      __syncthreads();
      if (tid < 64) {
        // the want-th largest key among them, its multiplicity and how many
        // of its pairs are wanted
        const int m = ncand, want = rs_want;
        const uint64_t mine = lane < m ? cand[lane] : 0;
        int above = 0, same = 0;
        for (int j = 0; j < m; ++j) {
          const uint64_t o = cand[j];
          above += o > mine;
          same += o == mine;
        }
        const bool hit = lane < m && above < want && want <= above + same;
        const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
        if (lane == __builtin_ctzll(hm)) {
          rs_prefix = mine;
          rs_want = want - above;
          rs_eq = same;
        }
      }
      __syncthreads();
      break;
    }
  }
  return RowCut{rs_prefix, rs_want, rs_eq};
}

// Called by the first wave. Walks the probabilities pv[0..n) of a row in
// sorted order, adding them to a running sum one at a time in that order (the
// rounding of a loop on one thread); entry t (block idx[t]) gets level
// #{l < nl : sum before t >= tau_l} (entry 0 level 0) and is flagged 1 +
// level when that is below nl. The sums form one chain of adds without a
// branch; lane u keeps the sum before entry c0 + u of each 16-entry chunk, and
// the levels are set in parallel. Stops after the chunk in which the sum
// reaches tau_{nl-1} (every later entry is dropped); returns whether it did.
// The thresholds are non-decreasing; nl is 1..4.
// CH entries per chunk (16, or 8 where registers are scarce; the sums are
// the same either way).
// With run_io the walk continues a row's earlier walk: the sum starts from
// *run_io and is left there, and the entries are the row's pos0, pos0 + 1, ...
template <int CH = 16>
__device__ inline bool walk_mass(const double* pv, const int32_t* idx, int64_t n, double tau0,
                                 double tau1, double tau2, double tau3, int nl, uint8_t* flag,
                                 double* run_io = nullptr, int64_t pos0 = 0) {
  const int lane = threadIdx.x & 63;
  const double last = nl == 1 ? tau0 : (nl == 2 ? tau1 : (nl == 3 ? tau2 : tau3));
  double run = run_io ? *run_io : 0.0;
  for (int c0 = 0; c0 < (int)n; c0 += CH) {
    const int m = min(CH, (int)n - c0);
    double v[CH];
    if (m == CH) {  // a whole chunk: contiguous reads
#pragma unroll
      for (int u = 0; u < CH; ++u) v[u] = pv[c0 + u];
    } else {
#pragma unroll
      for (int u = 0; u < CH; ++u) v[u] = u < m ? pv[c0 + min(u, m - 1)] : 0.0;
    }
    // (entries past n add 0: run + 0 = run, the sum being >= +0)
    // the chain first (each intermediate sum in its own register), the
    // lane's pick afterwards, so that no select waits inside the chain
    double pre[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      pre[u] = run;
      run = run + v[u];
    }
    double ex = pre[0];
#pragma unroll
    for (int u = 1; u < CH; ++u) ex = lane == u ? pre[u] : ex;
    if (lane < m) {
      int lvl = 0;
      if (pos0 + c0 + lane > 0)
        lvl = (ex >= tau0 ? 1 : 0) + (nl > 1 && ex >= tau1 ? 1 : 0) +
              (nl > 2 && ex >= tau2 ? 1 : 0) + (nl > 3 && ex >= tau3 ? 1 : 0);
      if (lvl < nl) flag[idx[c0 + lane]] = (uint8_t)(1 + lvl);
    }
    if (run >= last) {
      if (run_io) *run_io = run;
      return true;
    }
  }
  if (run_io) *run_io = run;
  return false;
}

// One workgroup per (b, h, a): sort of the row's blocks by (score desc, index
// asc), then top-k, the shortest prefix reaching the cumulative softmax mass
// tau_p, or the pyramid levels. Z = sum of exp(S - max) in ascending block
// order and the running sum of p = e / Z in sorted order are sequential, as
// one thread would add them (the first wave reads 64 terms per LDS access);
// the quotients are formed in parallel beforehand.
__global__ void pooled_select_kernel(int64_t nK, int32_t P, int32_t mode, double param,
                                     double tau1, double tau2, double tau3, int32_t n_levels,
                                     const double* __restrict__ S, uint8_t* __restrict__ mask,
                                     int32_t only_marked, int64_t R) {
  extern __shared__ double smd[];
  double* s = smd;                    // [nK] scores, block order
  double* ks = smd + nK;              // [P] sort keys: scores, then p in sorted order
  int32_t* ki = (int32_t*)(ks + P);   // [P] their block indices (-1: padding)
  uint8_t* flag = (uint8_t*)(ki + P);  // [nK]
  __shared__ int32_t keep_sh;
  __shared__ double z_sh;
  // after pooled_select_wave_kernel: only the rows it left marked, out of
  // kMarkedRowsPerGroup rows per workgroup whose markers one wave reads at
  // once (few workgroups, and no row loop, in the usual case of no marked
  // row); else row blockIdx.x. Bit t of `todo` stands for row row0 + t.
  const int64_t row0 = (int64_t)blockIdx.x * (only_marked ? kMarkedRowsPerGroup : 1);
  uint64_t todo = 1;
  if (only_marked) {
    __shared__ uint64_t marked_sh;
    if (threadIdx.x < kWave) {
      const int64_t r = row0 + threadIdx.x;
      const uint64_t bits = __ballot(r < R && mask[r * nK] == kSelectMarker);
      if (threadIdx.x == 0) marked_sh = bits;
    }
    __syncthreads();
    todo = marked_sh;
  }
  for (; todo != 0; todo &= todo - 1) {
    const int64_t row = row0 + __builtin_ctzll(todo);
    uint8_t* mrow = mask + row * nK;
    const double* srow = S + row * nK;
    for (int c = threadIdx.x; c < nK; c += blockDim.x) {
      s[c] = srow[c];
      flag[c] = 0;
    }
    __syncthreads();
    // Fast paths for long rows, no full sort: top-k marks the pairs before the
    // k-th key; cumulative mass sorts only the first kTopM pairs (the head of
    // the full order) and stops there if the mass is reached. A cut inside a
    // run of equal keys, or mass not reached, takes the full sort below.
    if (!only_marked && (mode == 0 || mode == 1) && nK > kTopM &&
        !(mode == 0 && param >= (double)nK)) {
      const int T = mode == 0 ? (int)max(1.0, param) : kTopM;
      const RowCut cut = select_kth(s, nK, T);
      if (cut.take_eq == cut.n_eq) {  // every pair with the cut key is taken
        if (mode == 0) {
          for (int c = threadIdx.x; c < nK; c += blockDim.x)
            mrow[c] = order_key(s[c]) >= cut.key ? 1 : 0;
          return;
        }
        __shared__ uint64_t ck[kTopM];  // sort keys, then the probabilities
        __shared__ int32_t ci[kTopM];
        __shared__ int32_t ncand;
        double* cs = (double*)ck;
        if (threadIdx.x == 0) ncand = 0;
        __syncthreads();
        for (int64_t c0 = 0; c0 < nK; c0 += blockDim.x) {
          const int c = (int)(c0 + threadIdx.x);
          const uint64_t u = c < nK ? order_key(s[c]) : 0;
          const bool hit = c < nK && u >= cut.key;
          const int pos = wave_append(hit, &ncand);
          if (hit) {
            ck[pos] = u;
            ci[pos] = c;
          }
        }
        __syncthreads();
        if (threadIdx.x < 64) sort128_wave(ck, ci);
        __syncthreads();
        const double smax0 = s[ci[0]];
        for (int c = threadIdx.x; c < nK; c += blockDim.x) ks[c] = exp(s[c] - smax0);
        __syncthreads();
        if (threadIdx.x < 64) {
          const double Z = ordered_sum(ks, nK, 0.0);
          if (threadIdx.x == 0) z_sh = Z;
        }
        __syncthreads();
        const double Z0 = z_sh;
        for (int t = threadIdx.x; t < kTopM; t += blockDim.x) cs[t] = ks[ci[t]] / Z0;
        __syncthreads();
        // flags of the first kTopM pairs; if the mass is not reached there,
        // they are a subset of what the full sort below keeps
        if (threadIdx.x < 64) {
          const bool reached = walk_mass(cs, ci, kTopM, param, param, param, param, 1, flag);
          if (threadIdx.x == 0) keep_sh = reached ? 1 : 0;
        }
        __syncthreads();
        if (keep_sh) {
          for (int c = threadIdx.x; c < nK; c += blockDim.x) mrow[c] = flag[c];
          return;
        }
      }
    }
    uint64_t* kk = (uint64_t*)ks;  // sort keys, then the probabilities in ks
    for (int c = threadIdx.x; c < P; c += blockDim.x) {
      kk[c] = c < nK ? order_key(s[c]) : 0;
      ki[c] = c < nK ? c : -1;
    }
    __syncthreads();
    sort_keys(kk, ki, P);
    const double smax = s[ki[0]];
    int32_t keep;
    if (mode == 0) {
      keep = (int32_t)min((double)nK, param);
    } else {
      // e = exp(S - max) in block order, over the scores (once every thread
      // has read the maximum from them)
      __syncthreads();
      for (int c = threadIdx.x; c < nK; c += blockDim.x) s[c] = exp(s[c] - smax);
      __syncthreads();
      if (threadIdx.x < 64) {
        const double Z = ordered_sum(s, nK, 0.0);
        if (threadIdx.x == 0) z_sh = Z;
      }
      __syncthreads();
      const double Z = z_sh;
      // p_t = e[idx_t] / Z in sorted order, each quotient on its own; the
      // sorted scores are not needed any more
      for (int t = threadIdx.x; t < nK; t += blockDim.x) ks[t] = s[ki[t]] / Z;
      __syncthreads();
      // mode 1: the shortest prefix whose running mass reaches tau_p (entry t
      // kept while the mass before it is below tau_p); mode 4, pyramid levels
      // ([PSA]: a resolution level per block pair by importance thresholds):
      // a block joins the current level, and the level advances past every
      // threshold that the running mass including that block has reached
      keep = 0;
      if (threadIdx.x < 64)
        walk_mass(ks, ki, nK, param, tau1, tau2, tau3, mode == 4 ? n_levels : 1, flag);
      __syncthreads();
    }
    for (int t = threadIdx.x; t < keep; t += blockDim.x) flag[ki[t]] = 1;
    __syncthreads();
    for (int c = threadIdx.x; c < nK; c += blockDim.x) mrow[c] = flag[c];
    __syncthreads();  // the next row refills the shared arrays
  }
}

// The common per-row case (top-k, and cumulative mass whose prefix lies in
// the first kTopM pairs) with one wave per row and four rows per workgroup:
// the work of a row is mostly sequential (the ordered sums), so a row holds
// one wave instead of a workgroup, no step waits on a workgroup barrier, and
// four times as many rows run at once. Same arithmetic as the fast path of
// pooled_select_kernel: the cut key by a radix select (one bit per pass, the
// last few candidates ranked directly), the first kTopM pairs sorted, Z in
// ascending block order, the running mass in sorted order. A row whose cut
// falls inside a run of equal keys (cumulative mass), or whose mass is not
// reached within kTopM pairs, gets kSelectMarker in its first mask byte and
// is finished by pooled_select_kernel (only_marked).

__host__ __device__ inline size_t select_wave_lds(int64_t nK) {
  // scores, then exponentials, then flags [nK] doubles; candidate keys /
  // probabilities [kTopM] and their indices [kTopM]
  return (sizeof(double) * (size_t)nK + 12 * kTopM + 15) / 16 * 16;  // 16-byte aligned slices
}

template <int NC>  // 64-key chunks per row held in registers (nK <= 64 * NC)
__global__ __launch_bounds__(kWave * kSelectRowsPerGroup) void pooled_select_wave_kernel(
    int64_t R, int64_t nK, int32_t mode, double param, const double* __restrict__ S,
    uint8_t* __restrict__ mask) {
  extern __shared__ double smw[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + w;
  if (row >= R) return;  // the whole wave (no workgroup barrier below)
  char* base = (char*)smw + (size_t)w * select_wave_lds(nK);
  double* s = (double*)base;
  uint64_t* ck = (uint64_t*)(s + nK);
  int32_t* ci = (int32_t*)(ck + kTopM);
  const double* srow = S + row * nK;
  uint8_t* mrow = mask + row * nK;
  // the row's scores (all loads in flight together) into LDS, and their
  // sort keys into registers: key[i] is block 64 i + lane (0 past the row,
  // below every score's key, and never counted)
  uint64_t key[NC];
  {
    double v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = i * kWave + lane;
      v[i] = c < nK ? srow[c] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = i * kWave + lane;
      key[i] = c < nK ? order_key(v[i]) : 0;
      if (c < nK) s[c] = v[i];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // ---- key of the T-th pair in (score desc, index asc) order, one bit per
  // pass from the highest bit in which the row's keys differ; `want` counts
  // the pairs still wanted among those matching the bits fixed so far. The
  // passes over the upper half of the key compare 32-bit words only.
  const int T = mode == 0 ? (int)max(1.0, param) : kTopM;
  uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (i * kWave + lane < nK) {
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t xa = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(kmax >> 32), off) << 32) |
                        (uint32_t)__shfl_xor((int)(uint32_t)kmax, off);
    const uint64_t xi = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(kmin >> 32), off) << 32) |
                        (uint32_t)__shfl_xor((int)(uint32_t)kmin, off);
    kmax = xa > kmax ? xa : kmax;
    kmin = xi < kmin ? xi : kmin;
  }
  const int top = kmax == kmin ? -1 : 63 - __builtin_clzll(kmax ^ kmin);
  // bits above `top` are common to every key of the row
  uint64_t prefix = top >= 63 ? 0 : kmax & (~0ull << (top + 1));
  int want = T;
  uint64_t cut = kmax;
  int take_eq = want, n_eq = (int)nK;  // every key equal (top < 0)
  for (int bit = top; bit >= 0; --bit) {
    int ones = 0, match = 0;
    if (bit >= 32) {
      const int b32 = bit - 32;
      const uint32_t hi = b32 == 31 ? 0u : (~0u << (b32 + 1));
      const uint32_t ph = (uint32_t)(prefix >> 32);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const uint32_t kh = (uint32_t)(key[i] >> 32);
        const bool m = i * kWave + lane < nK && (kh & hi) == ph;
        ones += __popcll(__builtin_amdgcn_ballot_w64(m && ((kh >> b32) & 1u)));
        match += __popcll(__builtin_amdgcn_ballot_w64(m));
      }
    } else {
      const uint32_t lo = bit == 31 ? 0u : (~0u << (bit + 1));
      const uint32_t ph = (uint32_t)(prefix >> 32), pl = (uint32_t)prefix;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const uint32_t kh = (uint32_t)(key[i] >> 32), kl = (uint32_t)key[i];
        const bool m = i * kWave + lane < nK && kh == ph && (kl & lo) == pl;
        ones += __popcll(__builtin_amdgcn_ballot_w64(m && ((kl >> bit) & 1u)));
        match += __popcll(__builtin_amdgcn_ballot_w64(m));
      }
    }
    int left;
    if (ones >= want) {
      prefix |= 1ull << bit;
      left = ones;
    } else {
      want -= ones;
      left = match - ones;
    }
    if (left == match && left > kWave && bit > 0) {
      // no pair dropped out: skip the bits below in which the pairs left all
      // agree (their largest and smallest key share them)
      const uint64_t pm = ~0ull << bit;
      uint64_t gmax = 0, gmin = ~0ull;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        if (i * kWave + lane < nK && (key[i] & pm) == prefix) {
          gmax = key[i] > gmax ? key[i] : gmax;
          gmin = key[i] < gmin ? key[i] : gmin;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t xa =
            ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(gmax >> 32), off) << 32) |
            (uint32_t)__shfl_xor((int)(uint32_t)gmax, off);
        const uint64_t xi =
            ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(gmin >> 32), off) << 32) |
            (uint32_t)__shfl_xor((int)(uint32_t)gmin, off);
        gmax = xa > gmax ? xa : gmax;
        gmin = xi < gmin ? xi : gmin;
      }
      if (gmax == gmin) {  // every pair left has the same key
        cut = gmax;
        take_eq = want;
        n_eq = left;
        break;
      }
      const int nb = 63 - __builtin_clzll(gmax ^ gmin);  // below `bit`
      prefix = gmax & (~0ull << (nb + 1));
      bit = nb + 1;  // the next pass decides bit nb
      continue;
    }
    if (left <= kWave) {
      // the pairs left (bits from `bit` up equal the prefix), one per lane;
      // the want-th largest key among them and its multiplicity
      const uint64_t pm = ~0ull << bit;
      int got = 0;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const bool hit = i * kWave + lane < nK && (key[i] & pm) == prefix;
        const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
        if (hit) ck[got + __popcll(hm & ((1ull << lane) - 1))] = key[i];
        got += __popcll(hm);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const uint64_t mine = lane < got ? ck[lane] : 0;
      int above = 0, same = 0;
      for (int j = 0; j < got; ++j) {
        const uint64_t o = ck[j];
        above += o > mine;
        same += o == mine;
      }
      const bool pick = lane < got && above < want && want <= above + same;
      const int src = __builtin_ctzll(__builtin_amdgcn_ballot_w64(pick));
      cut = ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(mine >> 32), src) << 32) |
            (uint32_t)__shfl((int)(uint32_t)mine, src);
      take_eq = __shfl(want - above, src);
      n_eq = __shfl(same, src);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      break;
    }
    if (bit == 0) {  // more than a wave of pairs share the cut key
      cut = prefix;
      take_eq = want;
      n_eq = left;
    }
  }
  if (mode == 0) {
    // keys above the cut, and of those equal to it the first take_eq in
    // ascending block order
    int seen = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = i * kWave + lane;
      const bool eq = c < nK && key[i] == cut;
      const uint64_t em = __builtin_amdgcn_ballot_w64(eq);
      const int rank = seen + __popcll(em & ((1ull << lane) - 1));
      if (c < nK) mrow[c] = (key[i] > cut || (eq && rank < take_eq)) ? 1 : 0;
      seen += __popcll(em);
    }
    return;
  }
  if (take_eq != n_eq) {  // cut inside a run of equal keys: the full sort decides
    if (lane == 0) mrow[0] = kSelectMarker;
    return;
  }
  // ---- the kTopM pairs at or above the cut, sorted
  {
    int got = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = i * kWave + lane;
      const bool hit = c < nK && key[i] >= cut;
      const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
      const int pos = got + __popcll(hm & ((1ull << lane) - 1));
      if (hit) {
        ck[pos] = key[i];
        ci[pos] = (int32_t)c;
      }
      got += __popcll(hm);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  sort128_wave(ck, ci);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // ---- e = exp(S - max) in place, Z in ascending block order, p of the
  // sorted pairs, running mass
  const double smax0 = s[ci[0]];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int64_t c = lane; c < nK; c += kWave) s[c] = exp(s[c] - smax0);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const double Z = ordered_sum_ahead(s, nK, 0.0);
  double* cs = (double*)ck;
  for (int t = lane; t < kTopM; t += kWave) cs[t] = s[ci[t]] / Z;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint8_t* flag = (uint8_t*)s;  // the exponentials are used up
  for (int64_t c = lane; c < nK; c += kWave) flag[c] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const bool reached = walk_mass<8>(cs, ci, kTopM, param, param, param, param, 1, flag);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (!reached) {
    if (lane == 0) mrow[0] = kSelectMarker;
    return;
  }
  for (int64_t c = lane; c < nK; c += kWave) mrow[c] = flag[c];
}

// Pyramid levels (mode 4) for rows of 129 to 1,024 blocks, one wave per row
// and up to four rows per workgroup: the walk of the levels runs over most
// of a row's blocks, so the row is sorted whole, in registers (the bitonic
// network of sort_keys: element e = 64 i + lane sits in register i of lane
// e % 64; partners 64 or more apart are two registers of one lane, closer
// ones come from lane ^ j by a cross-lane shuffle). Same arithmetic as
// pooled_select_kernel: e = exp(S - max) in block order, Z their sum in
// ascending block order, p = e / Z of the sorted pairs, and the levels from
// the running mass (walk_mass).
template <int NC>
__device__ inline void sort_wave(uint64_t (&k)[NC], int32_t (&x)[NC]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 2; kk <= 64 * NC; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int rj = j / 64;
#pragma unroll
        for (int r = 0; r < NC; ++r) {
          if (r & rj) continue;  // r is the lower register of the pair (r, r + rj)
          const int e = r * 64 + lane;
          const bool up = (e & kk) == 0;
          const bool first = k[r] > k[r + rj] || (k[r] == k[r + rj] && x[r] < x[r + rj]);
          if (first != up) {
            const uint64_t kt = k[r];
            const int32_t xt = x[r];
            k[r] = k[r + rj];
            x[r] = x[r + rj];
            k[r + rj] = kt;
            x[r + rj] = xt;
          }
        }
        continue;
      }
#pragma unroll
      for (int r = 0; r < NC; ++r) {
        const int e = r * 64 + lane;
        const uint32_t lo = __shfl_xor((uint32_t)k[r], j);
        const uint32_t hi = __shfl_xor((uint32_t)(k[r] >> 32), j);
        const uint64_t ko = ((uint64_t)hi << 32) | lo;
        const int32_t xo = __shfl_xor(x[r], j);
        const bool lower = (e & j) == 0, up = (e & kk) == 0;
        const bool mine_first = k[r] > ko || (k[r] == ko && x[r] < xo);
        // the lower position of an ascending pair holds the first element
        const bool keep = (lower == up) == mine_first;
        k[r] = keep ? k[r] : ko;
        x[r] = keep ? x[r] : xo;
      }
    }
  }
}

// LDS of one row of pooled_levels_wave_kernel: exponentials [nK] doubles
// (then the flags), sorted probabilities [nK] doubles, sorted blocks [nK]
// int32, each slice 16-byte aligned.
__host__ __device__ inline size_t levels_slice(int64_t nK, int bytes) {
  return ((size_t)nK * bytes + 15) / 16 * 16;
}
__host__ __device__ inline size_t levels_wave_lds(int64_t nK) {
  return 2 * levels_slice(nK, 8) + levels_slice(nK, 4);
}

template <int NC>  // 64-key chunks per row held in registers (nK <= 64 * NC)
__global__ __launch_bounds__(kWave * kSelectRowsPerGroup) void pooled_levels_wave_kernel(
    int64_t R, int64_t nK, double tau0, double tau1, double tau2, double tau3,
    int32_t n_levels, const double* __restrict__ S, uint8_t* __restrict__ mask) {
  extern __shared__ double sml[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + w;
  if (row >= R) return;  // the whole wave (no workgroup barrier below)
  char* base = (char*)sml + (size_t)w * levels_wave_lds(nK);
  double* e = (double*)base;
  double* cs = (double*)(base + levels_slice(nK, 8));
  int32_t* ci = (int32_t*)(base + 2 * levels_slice(nK, 8));
  const double* srow = S + row * nK;
  uint8_t* mrow = mask + row * nK;
  // scores (all loads in flight together), their sort keys and blocks; keys
  // past the row are 0, below every score's key, and sort last
  double v[NC];
  uint64_t key[NC];
  int32_t blk[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = i * kWave + lane;
    v[i] = c < nK ? srow[c] : 0.0;
  }
  double smax = -INFINITY;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = i * kWave + lane;
    key[i] = c < nK ? order_key(v[i]) : 0;
    blk[i] = (int32_t)c;
    if (c < nK) smax = fmax(smax, v[i]);
  }
  for (int off = 32; off >= 1; off >>= 1) smax = fmax(smax, __shfl_xor(smax, off));
  // e = exp(S - max) in block order, and Z their sum in ascending block order
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = i * kWave + lane;
    if (c < nK) e[c] = exp(v[i] - smax);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const double Z = ordered_sum_ahead(e, nK, 0.0);
  sort_wave<NC>(key, blk);
  // p of the sorted pairs, each quotient on its own
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t t = i * kWave + lane;
    if (t < nK) {
      cs[t] = e[blk[i]] / Z;
      ci[t] = blk[i];
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint8_t* flag = (uint8_t*)e;  // the exponentials are used up
  for (int64_t c = lane; c < nK; c += kWave) flag[c] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  walk_mass<8>(cs, ci, nK, tau0, tau1, tau2, tau3, n_levels, flag);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int64_t c = lane; c < nK; c += kWave) mrow[c] = flag[c];
}

// ------------------------------------------------------- global selection
// Head-wide selection over every (row block, key block) pair ([VMoBA]
// section 三: rank all query/block relevances together and serve the
// strongest first; the number of blocks a head keeps follows how
// concentrated its attention is). Mode 2 ranks pairs by S, mode 3 by the row
// softmax p = exp(S - max_row S) / Z_row (Z summed in ascending block order,
// as in mode 1), ties to the lower pair index a*nK + c. Mode 2 keeps the
// first k pairs, mode 3 the shortest prefix whose mass reaches tau_p * nQ
// (all pairs when tau_p = 1 or the total falls short). Every row also keeps
// its best block (S desc, c asc).

// One wave per row: best block, and for mode 3 the row's probabilities
// (exponentials in parallel, Z summed sequentially in ascending block order
// as in mode 1, then one division each).
__global__ __launch_bounds__(kWave) void pooled_rowstats_kernel(int64_t nK, int32_t mode,
                                                               const double* __restrict__ S,
                                                               double* __restrict__ P,
                                                               int32_t* __restrict__ best) {
  __shared__ double ex[kPooledMaxBlocks];
  __shared__ double zsh;
  const int lane = threadIdx.x;
  const int64_t r = blockIdx.x;
  const double* s = S + r * nK;
  double m = -INFINITY;
  int32_t arg = INT32_MAX;
  for (int64_t c = lane; c < nK; c += kWave) {
    if (s[c] > m || (s[c] == m && c < arg)) {
      m = s[c];
      arg = (int32_t)c;
    }
  }
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const double m2 = __shfl_xor(m, off);
    const int32_t a2 = __shfl_xor(arg, off);
    if (m2 > m || (m2 == m && a2 < arg)) {
      m = m2;
      arg = a2;
    }
  }
  if (lane == 0) best[r] = arg;
  if (mode != 3) return;
  for (int64_t c = lane; c < nK; c += kWave) ex[c] = exp(s[c] - m);
  __syncthreads();
  if (lane == 0) {
    double Z = 0.0;
    for (int64_t c = 0; c < nK; ++c) Z = Z + ex[c];
    zsh = Z;
  }
  __syncthreads();
  const double Z = zsh;
  double* pr = P + r * nK;
  for (int64_t c = lane; c < nK; c += kWave) pr[c] = ex[c] / Z;
}


// The cut of one head, found 4 bits at a time from the top (radix select in
// (key desc, index asc) order). `need_c` / `need_m` are the pairs / mass
// still to take below the keys already fixed as larger.
struct HeadCut {
  uint64_t prefix;  // key bits fixed so far
  double need_m;
  int64_t need_c;
  int64_t ties;     // pairs whose key equals the final prefix
  int64_t last;     // tied pairs with index <= last are kept
  int32_t all;      // every pair is kept
  int32_t done;     // groups of the current histogram pass that have finished
};

constexpr int kGselThreads = 256;
constexpr int kGselGroups = 32;  // workgroups per head in a histogram pass
constexpr int kGselFullPasses = 4;  // passes over every pair; the fifth keeps the candidates
constexpr int kGselBatch = 8;       // pairs per thread whose loads are issued together

// Per-thread capacity of the candidate store: thread t of a group visits at
// most ceil(per / kGselThreads) pairs.
__host__ __device__ inline int64_t gsel_cand_cap(int64_t n) {
  const int64_t per = (n + kGselGroups - 1) / kGselGroups;
  return (per + kGselThreads - 1) / kGselThreads;
}

__global__ void gsel_init_kernel(int64_t BH, int64_t nQ, int64_t nK, int32_t mode, double param,
                                 HeadCut* __restrict__ cut) {
  const int64_t bh = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  const int64_t n = nQ * nK;
  HeadCut c;
  c.prefix = 0;
  c.need_m = param * (double)nQ;
  c.need_c = mode == 2 ? (int64_t)param : 0;
  c.ties = 0;
  c.last = n;
  c.all = (mode == 2 ? param >= (double)n : param >= 1.0) ? 1 : 0;
  c.done = 0;
  cut[bh] = c;
}

// One histogram pass: per (head, group of pairs) the count and mass of the
// pairs matching the prefix, by the 4-bit digit at `shift`. Each thread
// walks its pairs in a fixed order into its own LDS slots; slots are then
// summed in a fixed tree, so the masses are deterministic. The last group of
// a head to finish then adds the groups' histograms in group order and fixes
// the next digit: the highest bucket in which the remaining count (mode 2)
// or mass (mode 3) is reached. When the mass is never reached the walk ends
// in the lowest bucket with the rest counted above it, which keeps every
// pair.
// After the first passes few pairs still match the prefix: the pass with
// phase 1 also stores each thread's matching keys (and masses) in its own
// slice of the candidate store, in its visiting order, and gsel_finish_kernel
// runs the remaining passes over those alone.
__global__ __launch_bounds__(kGselThreads) void gsel_hist_kernel(
    int64_t nQ, int64_t nK, int32_t mode, int32_t shift, const double* __restrict__ S,
    const double* __restrict__ P, HeadCut* cut, int64_t* pc, double* pm, int32_t phase,
    uint64_t* ck, double* cm, int32_t* ccnt) {
  __shared__ double hm[16][kGselThreads];
  __shared__ int32_t hc[16][kGselThreads];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.y, g = blockIdx.x, n = nQ * nK;
  const HeadCut c = cut[bh];
  if (c.all) return;
  for (int b = 0; b < 16; ++b) {
    hm[b][tid] = 0.0;
    hc[b][tid] = 0;
  }
  const uint64_t pmask = shift >= 60 ? 0 : (~0ull << (shift + 4));
  const int64_t per = (n + kGselGroups - 1) / kGselGroups;
  const int64_t e0 = g * per, e1 = min(n, e0 + per);
  const double* keys = (mode == 2 ? S : P) + bh * n;
  const double* mass = P + bh * n;
  // candidate slice of this thread: entries cbase + j * kGselThreads
  const int64_t cbase = (bh * kGselGroups + g) * gsel_cand_cap(n) * kGselThreads + tid;
  int32_t* my_cnt = ccnt + (bh * kGselGroups + g) * kGselThreads + tid;
  // Each thread's pairs are handled in its fixed visiting order; their keys
  // (and masses) are loaded kGselBatch at a time before they are counted, so
  // that the loads are in flight together instead of one memory latency per
  // pair.
  {
    int32_t j = 0;
    for (int64_t eb = e0 + tid; eb < e1; eb += (int64_t)kGselBatch * kGselThreads) {
      uint64_t ub[kGselBatch];
      double mb[kGselBatch];
#pragma unroll
      for (int i = 0; i < kGselBatch; ++i) {
        const int64_t e = eb + (int64_t)i * kGselThreads;
        ub[i] = e < e1 ? order_key(keys[e]) : 0;
        mb[i] = (mode == 3 && e < e1) ? mass[e] : 0.0;
      }
#pragma unroll
      for (int i = 0; i < kGselBatch; ++i) {
        const int64_t e = eb + (int64_t)i * kGselThreads;
        const uint64_t u = ub[i];
        if (e >= e1 || (u & pmask) != c.prefix) continue;
        const int b = (int)((u >> shift) & 15);
        hc[b][tid] += 1;
        if (mode == 3) hm[b][tid] = hm[b][tid] + mb[i];
        if (phase == 1) {
          ck[cbase + (int64_t)j * kGselThreads] = u;
          if (mode == 3) cm[cbase + (int64_t)j * kGselThreads] = mb[i];
          ++j;
        }
      }
    }
    if (phase == 1) *my_cnt = j;
  }
  __syncthreads();
  // slot i += slot i + off for every bucket, off halving: the fixed tree of
  // sums, its 16 * off additions of a level spread over all threads
  for (int off = kGselThreads / 2; off >= 1; off >>= 1) {
    for (int idx = tid; idx < 16 * off; idx += kGselThreads) {
      const int b = idx / off, i = idx - b * off;
      hc[b][i] += hc[b][i + off];
      hm[b][i] = hm[b][i] + hm[b][i + off];
    }
    __syncthreads();
  }
  __shared__ int is_last;
  if (tid < 64) {  // the first wave publishes this group's histogram, then counts it in
    if (tid < 16) {
      pc[(bh * kGselGroups + g) * 16 + tid] = hc[tid][0];
      pm[(bh * kGselGroups + g) * 16 + tid] = hm[tid][0];
    }
    __threadfence();
    if (tid == 0) is_last = atomicAdd(&cut[bh].done, 1) == kGselGroups - 1;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();  // the other groups' histograms are visible from here
  __shared__ int64_t bc[16];
  __shared__ double bm[16];
  if (tid < 16) {
    int64_t cb = 0;
    double mb = 0.0;
    for (int gg = 0; gg < kGselGroups; ++gg) {
      cb += pc[(bh * kGselGroups + gg) * 16 + tid];
      mb = mb + pm[(bh * kGselGroups + gg) * 16 + tid];
    }
    bc[tid] = cb;
    bm[tid] = mb;
  }
  __syncthreads();
  if (tid == 0) {
    HeadCut h = c;
    int chosen = 0;
    for (int b = 15; b >= 0; --b) {
      const bool here = mode == 2 ? bc[b] >= h.need_c : (bc[b] > 0 && bm[b] >= h.need_m);
      if (here || b == 0) {
        chosen = b;
        h.ties = bc[b];
        break;
      }
      h.need_c -= bc[b];
      h.need_m = h.need_m - bm[b];
    }
    h.prefix |= (uint64_t)chosen << shift;
    h.done = 0;  // the next pass counts its groups again
    cut[bh] = h;
  }
}

// The digits after the candidate store is filled, in one workgroup per head.
// While more candidates match the prefix than fit in LDS, a pass fixes the
// next 4-bit digit as gsel_hist_kernel does (thread t walks its slices (g, t)
// in a fixed order; its per-bucket counts and masses are summed in the same
// fixed tree). Then the matching candidates are compacted into LDS in that
// same visiting order (a
// count pass, an exclusive scan over the threads, a write pass), sorted by
// key (descending, then by position) and walked run by run of equal keys: a
// run whose count (mode 2) or mass (mode 3, its masses added in sorted order)
// reaches what is still needed holds the cut; otherwise its pairs are taken
// and the walk goes on, ending in the last run when nothing reaches.
// Deterministic.
constexpr int kFinishCap = 2048;  // candidates sorted in LDS

__global__ __launch_bounds__(kGselThreads) void gsel_finish_kernel(
    int64_t nQ, int64_t nK, int32_t mode, int32_t first_shift, HeadCut* cut,
    const uint64_t* __restrict__ ck, const double* __restrict__ cm,
    const int32_t* __restrict__ ccnt) {
  // sort arrays (40 KiB) or digit slots (48 KiB), one at a time
  __shared__ __attribute__((aligned(16))) char pool[16 * kGselThreads * 12];
  uint64_t* lk = (uint64_t*)pool;                                // [kFinishCap] keys, 0 = pad
  int32_t* li = (int32_t*)(pool + 8 * kFinishCap);               // positions in lm, -1 = pad
  double* lm = (double*)(pool + 12 * kFinishCap);                // masses, compacted order
  double(*hm)[kGselThreads] = (double(*)[kGselThreads])pool;     // [16][threads]
  int32_t(*hc)[kGselThreads] = (int32_t(*)[kGselThreads])(pool + 8 * 16 * kGselThreads);
  __shared__ int32_t toff[kGselThreads + 1];
  __shared__ HeadCut hs;
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x, n = nQ * nK;
  if (tid == 0) hs = cut[bh];
  __syncthreads();
  if (hs.all) return;
  const int64_t cap = gsel_cand_cap(n);
  // this thread's candidates matching (pm, pre), in a fixed order: groups in
  // chunks of kVisit, and within a chunk entry j of every group before entry
  // j + 1, so that a chunk's loads (keys, and masses when asked) are in
  // flight together (a slice holds about one candidate per group)
  constexpr int kVisit = 16;
  int32_t mg[kGselGroups];
#pragma unroll
  for (int g = 0; g < kGselGroups; ++g) mg[g] = ccnt[(bh * kGselGroups + g) * kGselThreads + tid];
  auto visit = [&](uint64_t pm, uint64_t pre, bool with_mass, auto&& fn) {
#pragma unroll
    for (int g0 = 0; g0 < kGselGroups; g0 += kVisit) {
      int32_t jmax = 0;
#pragma unroll
      for (int i = 0; i < kVisit; ++i) jmax = max(jmax, mg[g0 + i]);
      for (int32_t j = 0; j < jmax; ++j) {
        uint64_t ub[kVisit];
        double mb[kVisit];
#pragma unroll
        for (int i = 0; i < kVisit; ++i) {
          const int64_t slot = ((bh * kGselGroups + g0 + i) * cap + j) * kGselThreads + tid;
          const bool in = j < mg[g0 + i];
          ub[i] = in ? ck[slot] : 0;
          mb[i] = in && with_mass ? cm[slot] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < kVisit; ++i)
          if (j < mg[g0 + i] && (ub[i] & pm) == pre) fn(ub[i], mb[i]);
      }
    }
  };
  // exclusive prefix over the threads of per-thread counts (toff[t] is
  // thread t's offset, toff[kGselThreads] the total): within each wave by
  // shuffles, then across the four waves
  __shared__ int32_t wsum[kGselThreads / 64];
  auto scan_counts = [&](int32_t mine) {
    const int lane = tid & 63, wv = tid >> 6;
    int32_t x = mine;
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int32_t base = 0;
    for (int v = 0; v < wv; ++v) base += wsum[v];
    toff[tid] = base + x - mine;
    if (tid == kGselThreads - 1) toff[kGselThreads] = base + x;
    __syncthreads();
  };
  const bool m3 = mode == 3;
  int shift = first_shift;  // bits above shift + 3 are fixed
  int32_t total = 0;
  for (;;) {
    const uint64_t pm = shift >= 0 ? ~0ull << (shift + 4) : ~0ull, pre = hs.prefix;
    int32_t mine = 0;
    visit(pm, pre, false, [&](uint64_t, double) { ++mine; });
    scan_counts(mine);
    total = toff[kGselThreads];
    if (total <= kFinishCap) break;
    if (shift < 0) {  // every key bit fixed: one run of equal keys holds the cut
      if (tid == 0) {
        HeadCut h = hs;
        h.ties = total;
        h.done = 0;
        cut[bh] = h;
      }
      return;
    }
    // one more digit over the candidates
    int32_t cnt[16];
    double mas[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      cnt[d] = 0;
      mas[d] = 0.0;
    }
    visit(pm, pre, m3, [&](uint64_t u, double mv) {
      const int b = (int)((u >> shift) & 15);
#pragma unroll
      for (int d = 0; d < 16; ++d) {  // registers indexed by constants only
        cnt[d] += d == b ? 1 : 0;
        if (m3 && d == b) mas[d] = mas[d] + mv;
      }
    });
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      hc[d][tid] = cnt[d];
      hm[d][tid] = mas[d];
    }
    __syncthreads();
    for (int off = kGselThreads / 2; off >= 1; off >>= 1) {
      for (int idx = tid; idx < 16 * off; idx += kGselThreads) {
        const int d = idx / off, i = idx - d * off;
        hc[d][i] += hc[d][i + off];
        hm[d][i] = hm[d][i] + hm[d][i + off];
      }
      __syncthreads();
    }
    if (tid == 0) {
      HeadCut h = hs;
      int chosen = 0;
      for (int d = 15; d >= 0; --d) {
        const bool here =
            mode == 2 ? hc[d][0] >= h.need_c : (hc[d][0] > 0 && hm[d][0] >= h.need_m);
        if (here || d == 0) {
          chosen = d;
          h.ties = hc[d][0];
          break;
        }
        h.need_c -= hc[d][0];
        h.need_m = h.need_m - hm[d][0];
      }
      h.prefix |= (uint64_t)chosen << shift;
      hs = h;
    }
    __syncthreads();
    shift -= 4;
  }
  // compact, sort
  const uint64_t pm = shift >= 0 ? ~0ull << (shift + 4) : ~0ull, pre = hs.prefix;
  int32_t pos = toff[tid];
  visit(pm, pre, m3, [&](uint64_t u, double mv) {
    lk[pos] = u;
    li[pos] = pos;
    lm[pos] = mv;
    ++pos;
  });
  int P = 2;
  while (P < total) P <<= 1;
  for (int i = total + tid; i < P; i += kGselThreads) {
    lk[i] = 0;
    li[i] = -1;
  }
  __syncthreads();
  sort_keys(lk, li, P);
  // Walk, by the first wave, 64 sorted entries at a time: the running count
  // and mass (mass added by a fixed shuffle tree within each chunk, chunks in
  // order). The cut run is the first run of equal keys whose end reaches what
  // is needed (count: need_c, mass: need_m), else the last run; what the ties
  // kernel still needs is need less all runs before the cut run.
  if (tid < 64) {
    const int lane = tid;
    HeadCut h = hs;
    uint64_t key = pre;  // no candidate left: the prefix stands
    int64_t ties = 0, start_c = 0;
    double start_m = 0.0;
    int64_t last_end = 0;      // entries before the current run
    double last_end_m = 0.0;   // their mass
    double carry = 0.0;        // mass of the chunks before this one
    for (int t0 = 0; t0 < total; t0 += 64) {
      const int t = t0 + lane;
      const bool in = t < total;
      const uint64_t kt = in ? lk[t] : 0;
      double cum = in && m3 ? lm[li[t]] : 0.0;
      for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(cum, d);
        if (lane >= d) cum = cum + y;
      }
      cum = carry + cum;
      const bool run_end = in && (t == total - 1 || lk[t + 1] != kt);
      const bool reach =
          run_end && (mode == 2 ? (int64_t)(t + 1) >= h.need_c : cum >= h.need_m);
      const uint64_t ends = __builtin_amdgcn_ballot_w64(run_end);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(reach);
      const uint64_t last = __builtin_amdgcn_ballot_w64(in && t == total - 1);
      if (hit || last) {  // the cut run ends at entry t0 + src
        const int src = __builtin_ctzll(hit ? hit : last);
        const uint64_t below = ends & ((1ull << src) - 1);
        if (below) {
          const int e = 63 - __builtin_clzll(below);
          start_c = t0 + e + 1;
          start_m = __shfl(cum, e);
        } else {
          start_c = last_end;
          start_m = last_end_m;
        }
        const uint32_t khi = (uint32_t)__shfl((int)(uint32_t)(kt >> 32), src);
        const uint32_t klo = (uint32_t)__shfl((int)(uint32_t)kt, src);
        key = ((uint64_t)khi << 32) | klo;
        ties = t0 + src + 1 - start_c;
        break;
      }
      if (ends) {
        const int e = 63 - __builtin_clzll(ends);
        last_end = t0 + e + 1;
        last_end_m = __shfl(cum, e);
      }
      carry = __shfl(cum, 63);
    }
    if (lane == 0) {
      h.need_c -= start_c;
      h.need_m = h.need_m - start_m;
      h.prefix = key;
      h.ties = ties;
      h.done = 0;
      cut[bh] = h;
    }
  }
}

// One thread per head: among several pairs with the cut key, the ones taken
// come first in index order (rare: equal keys).
__global__ void gsel_ties_kernel(int64_t BH, int64_t n, int32_t mode, const double* __restrict__ S,
                                 const double* __restrict__ P, HeadCut* __restrict__ cut) {
  const int64_t bh = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  HeadCut c = cut[bh];
  if (c.all || c.ties <= 1) return;
  const double* keys = (mode == 2 ? S : P) + bh * n;
  const double* mass = P + bh * n;
  int64_t need = c.need_c;
  double acc = 0.0;
  for (int64_t e = 0; e < n; ++e) {
    if (order_key(keys[e]) != c.prefix) continue;
    if (mode == 2) {
      if (--need == 0) {
        c.last = e;
        break;
      }
    } else {
      acc = acc + mass[e];
      if (acc >= c.need_m) {
        c.last = e;
        break;
      }
    }
  }
  cut[bh] = c;
}

// One thread per pair: keep the pairs before the cut and every row's best block.
__global__ void gsel_mark_kernel(int64_t BH, int64_t nQ, int64_t nK, int32_t mode,
                                 const double* __restrict__ S, const double* __restrict__ P,
                                 const int32_t* __restrict__ best,
                                 const HeadCut* __restrict__ cut, uint8_t* __restrict__ mask) {
  const int64_t n = nQ * nK, total = BH * n;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bh = t / n, e = t - bh * n, a = e / nK, c = e - a * nK;
    const HeadCut h = cut[bh];
    const uint64_t u = order_key((mode == 2 ? S : P)[t]);
    const bool keep = h.all || u > h.prefix || (u == h.prefix && e <= h.last) ||
                      best[bh * nQ + a] == (int32_t)c;
    mask[t] = keep ? 1 : 0;
  }
}

// ------------------------------------------------------- long rows
// Row statistics with one lane per row (64 rows per workgroup): the row's
// maximum score and its first block (S desc, c asc), then Z = sum of
// exp(S - max) in ascending block order, one add at a time as in the short
// kernels. Scores pass through LDS in 64 x 64 tiles, read row segment by
// row segment (coalesced) and walked by the lane of their row.
__global__ __launch_bounds__(kWave) void pooled_rowz_kernel(int64_t R, int64_t nK,
                                                           const double* __restrict__ S,
                                                           double* __restrict__ zrow,
                                                           double* __restrict__ mrow,
                                                           int32_t* __restrict__ best) {
  __shared__ double tile[kWave][kWave + 1];
  const int lane = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kWave, r = r0 + lane;
  auto load_tile = [&](int64_t c0) {
#pragma unroll 16
    for (int i = 0; i < kWave; ++i) {
      const int64_t rr = r0 + i, cc = c0 + lane;
      tile[i][lane] = (rr < R && cc < nK) ? S[rr * nK + cc] : 0.0;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };
  double m = -INFINITY;
  int32_t arg = INT32_MAX;
  for (int64_t c0 = 0; c0 < nK; c0 += kWave) {
    load_tile(c0);
    const int w = (int)min((int64_t)kWave, nK - c0);
    for (int j = 0; j < w; ++j) {
      const double v = tile[lane][j];
      if (v > m || (v == m && c0 + j < arg)) {
        m = v;
        arg = (int32_t)(c0 + j);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  double Z = 0.0;
  for (int64_t c0 = 0; c0 < nK; c0 += kWave) {
    load_tile(c0);
    const int w = (int)min((int64_t)kWave, nK - c0);
    for (int j = 0; j < w; ++j) Z = Z + exp(tile[lane][j] - m);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  if (r < R) {
    zrow[r] = Z;
    mrow[r] = m;
    if (best) best[r] = arg;
  }
}

// Head-wide mass for long rows: p = exp(S - max) / Z of the row, elementwise.
__global__ void pooled_prob_kernel(int64_t total, int64_t nK, const double* __restrict__ S,
                                   const double* __restrict__ zrow,
                                   const double* __restrict__ mrow, double* __restrict__ P) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / nK;
    P[t] = exp(S[t] - mrow[r]) / zrow[r];
  }
}

// Inverse of order_key (the score of a key; -0 comes back as +0).
__device__ inline double key_score(uint64_t u) {
  const uint64_t b = (u >> 63) ? (u & ~(1ull << 63)) : ~u;
  return __longlong_as_double((long long)b);
}

// Per-row selection for long rows, one workgroup per row; block c is key
// kk of thread c % 256 with kk = c / 256 (coalesced loads; ascending block
// order is (kk, thread)). Sums over the workgroup go through per-wave ballots
// and a small LDS array. Top-k: the key of the k-th pair by a radix select
// (one bit per pass, from the highest bit in which the keys in play differ,
// skipping bits they all share), then the pairs above it and the first of
// those equal to it in block order. Cumulative mass and pyramid levels: the
// pairs in (score desc, block asc) order in steps: the pairs above the
// kLongBatch-th largest key still in play, sorted in LDS, then the run of
// pairs equal to that key in block order, each walked with the running mass
// of walk_mass (p = exp(S - max) / Z with the row's max and Z from
// pooled_rowz_kernel), until the last threshold is reached or every pair has
// been walked. The same arithmetic as the short kernels and the oracle.
struct LongCut {
  uint64_t key;
  int32_t take_eq;  // pairs equal to key among the T wanted
  int32_t n_eq;     // pairs equal to key in play
};

__global__ __launch_bounds__(kLongThreads) void pooled_select_long_kernel(
    int64_t nK, int32_t mode, double param, double tau1, double tau2, double tau3, int32_t n_levels,
    const double* __restrict__ S, const double* __restrict__ zrow,
    const double* __restrict__ mrow, uint8_t* __restrict__ mask) {
  __shared__ uint64_t ck[kLongCap];  // step keys, then their probabilities
  __shared__ int32_t ci[kLongCap];   // their blocks
  __shared__ uint8_t flag[kLongMaxBlocks];
  __shared__ int64_t red_i[kLongThreads / 64][2];
  __shared__ uint64_t red_u[kLongThreads / 64][2];
  __shared__ double run_sh;
  __shared__ int32_t done_sh;
  __shared__ int32_t na_sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int NW = kLongThreads / 64;
  const int64_t row = blockIdx.x;
  const double* srow = S + row * nK;
  uint8_t* out = mask + row * nK;
  uint64_t key[kLongKeys];
  {
    double v[kLongKeys];
#pragma unroll
    for (int kk = 0; kk < kLongKeys; ++kk) {
      const int64_t c = (int64_t)kk * kLongThreads + tid;
      v[kk] = c < nK ? srow[c] : 0.0;
    }
#pragma unroll
    for (int kk = 0; kk < kLongKeys; ++kk) {
      const int64_t c = (int64_t)kk * kLongThreads + tid;
      key[kk] = c < nK ? order_key(v[kk]) : 0;
      if (c < nK) flag[c] = 0;
    }
  }
  // workgroup sums of two per-thread counts / min-max of keys
  auto sum2 = [&](int64_t a, int64_t b, int64_t& sa, int64_t& sb) {
    for (int off = 32; off >= 1; off >>= 1) {
      a += __shfl_xor(a, off);
      b += __shfl_xor(b, off);
    }
    if (lane == 0) {
      red_i[wv][0] = a;
      red_i[wv][1] = b;
    }
    __syncthreads();
    sa = sb = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      sa += red_i[v][0];
      sb += red_i[v][1];
    }
    __syncthreads();
  };
  auto minmax = [&](uint64_t mx, uint64_t mn, uint64_t& gmx, uint64_t& gmn) {
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t xa =
          ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(mx >> 32), off) << 32) |
          (uint32_t)__shfl_xor((int)(uint32_t)mx, off);
      const uint64_t xi =
          ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(mn >> 32), off) << 32) |
          (uint32_t)__shfl_xor((int)(uint32_t)mn, off);
      mx = xa > mx ? xa : mx;
      mn = xi < mn ? xi : mn;
    }
    if (lane == 0) {
      red_u[wv][0] = mx;
      red_u[wv][1] = mn;
    }
    __syncthreads();
    gmx = 0;
    gmn = ~0ull;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      gmx = red_u[v][0] > gmx ? red_u[v][0] : gmx;
      gmn = red_u[v][1] < gmn ? red_u[v][1] : gmn;
    }
    __syncthreads();
  };
  // the T-th largest key among those below `hi` (every key when !bounded);
  // bits from `from` down are undecided, the ones above equal `prefix` for
  // every key in play
  auto select = [&](int64_t T, bool bounded, uint64_t hi, int64_t n_play) -> LongCut {
    auto in_play = [&](int kk) {
      return (int64_t)kk * kLongThreads + tid < nK && (!bounded || key[kk] < hi);
    };
    uint64_t mx = 0, mn = ~0ull;
#pragma unroll
    for (int kk = 0; kk < kLongKeys; ++kk)
      if (in_play(kk)) {
        mx = key[kk] > mx ? key[kk] : mx;
        mn = key[kk] < mn ? key[kk] : mn;
      }
    uint64_t gmx, gmn;
    minmax(mx, mn, gmx, gmn);
    int64_t want = T;
    if (gmx == gmn) return LongCut{gmx, (int32_t)want, (int32_t)n_play};  // one key in play
    int bit = 63 - __builtin_clzll(gmx ^ gmn);
    uint64_t prefix = bit >= 63 ? 0 : gmx & (~0ull << (bit + 1));
    for (;;) {
      const uint64_t hm = bit >= 63 ? 0 : ~0ull << (bit + 1);
      int64_t ones = 0, match = 0;
#pragma unroll
      for (int kk = 0; kk < kLongKeys; ++kk) {
        const bool m = in_play(kk) && (key[kk] & hm) == prefix;
        ones += m && ((key[kk] >> bit) & 1);
        match += m;
      }
      int64_t so, sm;
      sum2(ones, match, so, sm);
      int64_t left;
      if (so >= want) {
        prefix |= 1ull << bit;
        left = so;
      } else {
        want -= so;
        left = sm - so;
      }
      if (bit == 0) return LongCut{prefix, (int32_t)want, (int32_t)left};
      // the bits below on which the keys left all agree
      const uint64_t pm = ~0ull << bit;
      mx = 0;
      mn = ~0ull;
#pragma unroll
      for (int kk = 0; kk < kLongKeys; ++kk)
        if (in_play(kk) && (key[kk] & pm) == prefix) {
          mx = key[kk] > mx ? key[kk] : mx;
          mn = key[kk] < mn ? key[kk] : mn;
        }
      minmax(mx, mn, gmx, gmn);
      if (gmx == gmn) return LongCut{gmx, (int32_t)want, (int32_t)left};
      bit = 63 - __builtin_clzll(gmx ^ gmn);
      prefix = gmx & (~0ull << (bit + 1));
    }
  };
  // rank of this thread's key kk among those with eq set, in block order:
  // calls fn(kk, rank) for each; returns the number of them
  auto in_block_order = [&](auto&& pred, auto&& fn) -> int64_t {
    int64_t seen = 0;
#pragma unroll
    for (int kk = 0; kk < kLongKeys; ++kk) {  // unrolled: keys stay in registers
      if ((int64_t)kk * kLongThreads < nK) {  // uniform
        const bool e = (int64_t)kk * kLongThreads + tid < nK && pred(kk);
        const uint64_t bm = __builtin_amdgcn_ballot_w64(e);
        if (lane == 0) red_i[wv][0] = __popcll(bm);
        __syncthreads();
        int64_t base = seen;
        for (int v = 0; v < wv; ++v) base += red_i[v][0];
        for (int v = 0; v < NW; ++v) seen += red_i[v][0];
        __syncthreads();
        if (e) fn(kk, base + __popcll(bm & ((1ull << lane) - 1)));
      }
    }
    return seen;
  };
  const double smax = mrow[row], Z = zrow[row];
  if (mode == 0) {
    const int64_t T = (int64_t)min((double)nK, param);
    const LongCut cut = select(T, false, 0, nK);
#pragma unroll
    for (int kk = 0; kk < kLongKeys; ++kk) {
      const int64_t c = (int64_t)kk * kLongThreads + tid;
      if (c < nK && key[kk] > cut.key) flag[c] = 1;
    }
    in_block_order([&](int kk) { return key[kk] == cut.key; },
                   [&](int kk, int64_t rank) {
                     if (rank < cut.take_eq) flag[(int64_t)kk * kLongThreads + tid] = 1;
                   });
  } else {
    const int nl = mode == 4 ? n_levels : 1;
    if (tid == 0) {
      run_sh = 0.0;
      done_sh = 0;
    }
    __syncthreads();
    int64_t walked = 0;
    bool bounded = false;
    uint64_t hi = 0;
    for (;;) {
      int64_t cnt = 0, dummy = 0;
#pragma unroll
      for (int kk = 0; kk < kLongKeys; ++kk)
        cnt += (int64_t)kk * kLongThreads + tid < nK && (!bounded || key[kk] < hi);
      int64_t left;
      sum2(cnt, dummy, left, dummy);
      if (left == 0) break;
      const LongCut cut = select(min(left, (int64_t)kLongBatch), bounded, hi, left);
      // the pairs above the cut key still in play, sorted
      if (tid == 0) na_sh = 0;
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kLongKeys; ++kk) {
        const int64_t c = (int64_t)kk * kLongThreads + tid;
        const bool a = c < nK && key[kk] > cut.key && (!bounded || key[kk] < hi);
        const int pos = wave_append(a, &na_sh);
        if (a) {
          ck[pos] = key[kk];
          ci[pos] = (int32_t)c;
        }
      }
      __syncthreads();
      const int na = na_sh;
      __syncthreads();
      if (na > 0) {
        int P = 2;
        while (P < na) P <<= 1;
        for (int i = na + tid; i < P; i += kLongThreads) {
          ck[i] = 0;
          ci[i] = -1;
        }
        __syncthreads();
        sort_keys(ck, ci, P);
        double* cs = (double*)ck;
        for (int t = tid; t < na; t += kLongThreads) cs[t] = exp(key_score(ck[t]) - smax) / Z;
        __syncthreads();
        if (tid < 64) {
          double run = run_sh;
          const bool reached = walk_mass<8>(cs, ci, na, param, tau1, tau2, tau3, nl, flag, &run,
                                            walked);
          if (lane == 0) {
            run_sh = run;
            done_sh = reached;
          }
        }
        __syncthreads();
        walked += na;
        if (done_sh) break;
      }
      // the run of pairs equal to the cut key, in block order, kLongCap at a time
      const double pe = exp(key_score(cut.key) - smax) / Z;
      for (int64_t r0 = 0;; r0 += kLongCap) {
        const int64_t got = in_block_order(
            [&](int kk) { return key[kk] == cut.key; },
            [&](int kk, int64_t rank) {
              if (rank >= r0 && rank < r0 + kLongCap) {
                ci[rank - r0] = (int32_t)((int64_t)kk * kLongThreads + tid);
                ((double*)ck)[rank - r0] = pe;
              }
            });
        const int64_t m = min((int64_t)kLongCap, got - r0);
        __syncthreads();
        if (m > 0 && tid < 64) {
          double run = run_sh;
          const bool reached = walk_mass<8>((const double*)ck, ci, m, param, tau1, tau2, tau3, nl,
                                            flag, &run, walked);
          if (lane == 0) {
            run_sh = run;
            done_sh = reached;
          }
        }
        __syncthreads();
        walked += max((int64_t)0, m);
        if (done_sh || r0 + kLongCap >= got) break;
      }
      if (done_sh) break;
      bounded = true;
      hi = cut.key;
    }
  }
  __syncthreads();
  for (int64_t c = tid; c < nK; c += kLongThreads) out[c] = flag[c];
}

// ------------------------------------------------------- pyramid lists
// Eighth mask (8-row eighths of a 64-row augmented block) that row r
// selects in augmented block ab ([PSA]: logical block size decoupled from the
// hardware tile): ab in level region l covers logical blocks
// c = (ab - rb_l) * 2^l + i, i < 2^l, each owning 8 / 2^l eighths; block c
// contributes its eighths when its mask value is 1 + l (other values select
// nothing there).
struct PyrRegions {
  int64_t rb[5];  // first augmented block of levels 0..3, then the end
  int32_t n_levels;
};

__device__ inline uint32_t pyr_eighths(const uint8_t* mrow, int64_t nK, const PyrRegions& R,
                                       int64_t ab) {
  int l = 0;
  while (l + 1 < R.n_levels && ab >= R.rb[l + 1]) ++l;
  const int per = 1 << l;            // logical blocks per augmented block
  const int epb = 8 >> l;            // eighths per logical block
  uint32_t q = 0;
  for (int i = 0; i < per; ++i) {
    const int64_t c = (ab - R.rb[l]) * per + i;
    if (c < nK && mrow[c] == 1 + l) q |= ((1u << epb) - 1) << (i * epb);
  }
  return q;
}

// One wave per list row: row_ptr[r + 1] = augmented blocks with an eighth.
__global__ void pyr_count_kernel(int64_t R, int64_t nQ, int64_t nK, PyrRegions reg,
                                 const uint8_t* __restrict__ mask, int64_t mhs,
                                 int32_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (r >= R) return;
  const int64_t bh = r / nQ, a = r - bh * nQ;
  const uint8_t* mrow = mask + bh * mhs + a * nK;
  const int64_t nA = reg.rb[reg.n_levels];
  int32_t cnt = 0;
  for (int64_t a0 = 0; a0 < nA; a0 += kWave) {
    const int64_t ab = a0 + lane;
    const bool on = ab < nA && pyr_eighths(mrow, nK, reg, ab) != 0;
    cnt += __popcll(__ballot(on));
  }
  if (lane == 0) row_ptr[r + 1] = cnt;
}

__global__ void pyr_scatter_kernel(int64_t R, int64_t nQ, int64_t nK, PyrRegions reg,
                                   const uint8_t* __restrict__ mask, int64_t mhs,
                                   const int32_t* __restrict__ row_ptr,
                                   int32_t* __restrict__ kv_idx,
                                   int32_t* __restrict__ kv_eighths) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= R) return;
  const int64_t bh = r / nQ, a = r - bh * nQ;
  const uint8_t* mrow = mask + bh * mhs + a * nK;
  const int64_t nA = reg.rb[reg.n_levels];
  int64_t out = row_ptr[r];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t a0 = 0; a0 < nA; a0 += kWave) {
    const int64_t ab = a0 + lane;
    const uint32_t q = ab < nA ? pyr_eighths(mrow, nK, reg, ab) : 0u;
    const uint64_t bal = __ballot(q != 0);
    if (q) {
      const int64_t o = out + __popcll(bal & below);
      kv_idx[o] = (int32_t)ab;
      kv_eighths[o] = (int32_t)q;
    }
    out += __popcll(bal);
  }
}

// -------------------------------------------------------------- compaction
__device__ inline bool tile_listed(const uint8_t* mask, int64_t mhs, const uint8_t* skip,
                                   int64_t r, int64_t nQ, int64_t nK, int64_t c) {
  const int64_t bh = r / nQ, a = r - bh * nQ;
  bool on = mask[bh * mhs + a * nK + c] != 0;
  if (skip && skip[r * nK + c]) on = false;
  return on;
}

// One wave per list row: row_ptr[r + 1] = number of listed tiles.
__global__ void compact_count_kernel(int64_t R, int64_t nQ, int64_t nK,
                                     const uint8_t* __restrict__ mask, int64_t mhs,
                                     const uint8_t* __restrict__ skip,
                                     int32_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (r >= R) return;
  int32_t cnt = 0;
  for (int64_t c0 = 0; c0 < nK; c0 += kWave) {
    const int64_t c = c0 + lane;
    const bool on = c < nK && tile_listed(mask, mhs, skip, r, nQ, nK, c);
    cnt += __popcll(__ballot(on));
  }
  if (lane == 0) row_ptr[r + 1] = cnt;
}

// Single workgroup: in-place inclusive scan of row_ptr[1..R].
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void compact_scan_kernel(int64_t R,
                                                                    int32_t* __restrict__ row_ptr) {
  __shared__ int32_t part[kScanThreads];
  const int64_t chunk = (R + kScanThreads - 1) / kScanThreads;
  const int64_t lo = 1 + threadIdx.x * chunk, hi = min(R + 1, lo + chunk);
  int32_t sum = 0;
  for (int64_t i = lo; i < hi; ++i) sum += row_ptr[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int64_t i = lo; i < hi; ++i) {
    run += row_ptr[i];
    row_ptr[i] = run;
  }
}

// One wave per list row: write the listed key blocks in ascending order.
__global__ void compact_scatter_kernel(int64_t R, int64_t nQ, int64_t nK,
                                       const uint8_t* __restrict__ mask, int64_t mhs,
                                       const uint8_t* __restrict__ skip,
                                       const int32_t* __restrict__ row_ptr,
                                       int32_t* __restrict__ kv_idx) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= R) return;
  int64_t out = row_ptr[r];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t c0 = 0; c0 < nK; c0 += kWave) {
    const int64_t c = c0 + lane;
    const bool on = c < nK && tile_listed(mask, mhs, skip, r, nQ, nK, c);
    const uint64_t bal = __ballot(on);
    if (on) kv_idx[out + __popcll(bal & below)] = (int32_t)c;
    out += __popcll(bal);
  }
}

__global__ void zero_row_ptr_kernel(int32_t* row_ptr) { row_ptr[0] = 0; }

// ------------------------------------------------------------- skip update
// One wave per list row: tiles whose gap lies at or below -tau2 join the
// carried skip set ([Lite] sections 三 and 六).
__global__ void skip_update_kernel(int64_t R, int64_t nK, const int32_t* __restrict__ row_ptr,
                                   const int32_t* __restrict__ kv_idx,
                                   const float* __restrict__ gap, float neg_tau2,
                                   uint8_t* __restrict__ skip) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= R) return;
  const int32_t e1 = row_ptr[r + 1];
  for (int32_t e = row_ptr[r] + lane; e < e1; e += kWave)
    if (gap[e] <= neg_tau2) skip[r * nK + kv_idx[e]] = 1;
}

// ------------------------------------------------------------ list order
// Radial-centric visiting order of each list row ([Lite] section 五: visiting
// key blocks outward from the row's own position reaches the row maximum
// sooner, so the running-maximum test can skip more). Key blocks are ordered
// by the distance between token midpoints of key block and row block (twice
// the midpoints, in integers), ties to the lower block index.
// The ascending input splits at the row's midpoint into a left run whose
// distances fall and a right run whose distances rise; the output position
// of an entry is its rank in its own run plus the number of entries of the
// other run that precede it, found by binary search. One wave per list row,
// lanes over its entries. order 0 copies. Every write lands inside the row.
__device__ inline int64_t mid2(int64_t c, int64_t blk, int64_t N) {
  return c * blk + min(N, (c + 1) * blk) - 1;
}

__global__ void order_lists_kernel(int64_t R, int64_t nQ, int64_t N, int32_t Bq, int32_t Bk,
                                   int32_t order, const int32_t* __restrict__ row_ptr,
                                   const int32_t* __restrict__ kv_in,
                                   int32_t* __restrict__ kv_out) {
  const int lane = threadIdx.x % kWave;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= R) return;
  const int32_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
  const int32_t n = e1 - e0;
  if (order == 0) {
    for (int32_t e = lane; e < n; e += kWave) kv_out[e0 + e] = kv_in[e0 + e];
    return;
  }
  const int32_t* in = kv_in + e0;
  const int64_t cq2 = mid2(r % nQ, Bq, N);
  // p = number of entries left of the row midpoint (mid2 < cq2)
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    const int32_t m = (lo + hi) / 2;
    if (mid2(in[m], Bk, N) < cq2) lo = m + 1;
    else hi = m;
  }
  const int32_t p = lo;
  for (int32_t e = lane; e < n; e += kWave) {
    const int64_t d = mid2(in[e], Bk, N) - cq2;
    int32_t rank;
    if (e < p) {
      // left run, distance -d falls with e; right entries strictly nearer come first
      int32_t l2 = p, h2 = n;
      while (l2 < h2) {
        const int32_t m = (l2 + h2) / 2;
        if (mid2(in[m], Bk, N) - cq2 < -d) l2 = m + 1;
        else h2 = m;
      }
      rank = (p - 1 - e) + (l2 - p);
    } else {
      // right run, distance d rises with e; left entries as near or nearer come first
      int32_t l2 = 0, h2 = p;
      while (l2 < h2) {
        const int32_t m = (l2 + h2) / 2;
        if (cq2 - mid2(in[m], Bk, N) > d) l2 = m + 1;
        else h2 = m;
      }
      rank = (e - p) + (p - l2);
    }
    kv_out[e0 + rank] = in[e];
  }
}

inline unsigned grid_for(int64_t work, int threads, int64_t cap = 1 << 20) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_radial_mask(const Geom& g, int32_t h0, int32_t beta, uint8_t* mask,
                              hipStream_t st) {
  const int64_t tiles = g.nQ * g.nK;
  if (tiles == 0) return hipSuccess;
  int32_t rstar = 0;
  for (int64_t w = h0 / beta; w >= g.Bk / 2; w /= beta) ++rstar;
  hipLaunchKernelGGL(radial_mask_kernel, dim3(grid_for(tiles, 256)), dim3(256), 0, st, g.N,
                     g.F, g.Bq, g.Bk, g.nK, tiles, h0, beta, rstar, mask);
  return hipGetLastError();
}

size_t pooled_workspace_bytes(const Geom& g) {
  // qbar, kbar, scores; then for the head-wide modes: probabilities, per-group
  // histogram partials (counts and masses), one cut per head, best blocks,
  // and (from a 256-byte boundary) the candidate store: keys, masses and
  // per-thread counts
  const int64_t BH = (int64_t)g.B * g.H;
  const int64_t n = BH * (g.nQ + g.nK) * g.D + 2 * BH * g.nQ * g.nK;
  size_t bytes = (size_t)n * sizeof(double);
  bytes += (size_t)BH * kGselGroups * 16 * (sizeof(int64_t) + sizeof(double));
  bytes += (size_t)BH * sizeof(HeadCut);
  bytes += (size_t)BH * g.nQ * sizeof(int32_t);
  bytes = (bytes + 255) / 256 * 256;
  const int64_t cand = BH * kGselGroups * gsel_cand_cap(g.nQ * g.nK) * kGselThreads;
  bytes += (size_t)cand * (sizeof(uint64_t) + sizeof(double));
  bytes += (size_t)BH * kGselGroups * kGselThreads * sizeof(int32_t);
  return (bytes + 255) / 256 * 256;
}

int pooled_max_blocks() { return kLongMaxBlocks; }

size_t pooled_scratch_need(const Geom& g, int32_t mode) {
  if (mode == 2 || mode == 3) return pooled_workspace_bytes(g);
  // per-row modes: pooled means of Q and K and the score matrix only (and,
  // for long rows, each row's maximum and Z)
  const int64_t BH = (int64_t)g.B * g.H;
  size_t n = (size_t)(BH * (g.nQ + g.nK) * g.D + BH * g.nQ * g.nK);
  if (g.nK > kPooledMaxBlocks) n += (size_t)(2 * BH * g.nQ);
  return (n * sizeof(double) + 255) / 256 * 256;
}

// Scratch of the pooled builder for callers that cannot allocate: one
// file-scope device array, held by every GPU the library runs on until the
// process ends. In host code the array's name is only a host-side stand-in;
// its device address comes from hipGetSymbolAddress, looked up once per
// device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_pooled_mask(const Geom& g, int dtype, TensorArg q, TensorArg k, double scale,
                              int32_t mode, double param, uint8_t* mask, void* ws,
                              hipStream_t st, const double* levels, int32_t n_levels) {
  const int64_t BH = (int64_t)g.B * g.H;
  if (BH == 0 || g.N == 0) return hipSuccess;
  double* qbar = (double*)ws;
  double* kbar = qbar + BH * g.nQ * g.D;
  double* S = kbar + BH * g.nK * g.D;
  const int64_t work = BH * (g.nQ + g.nK) * (g.D / 4);
  if (dtype == 0)
    hipLaunchKernelGGL((pool_mean_kernel<0, 16>), dim3(grid_for(work, 256)), dim3(256), 0, st,
                       g.N, g.H, g.D, g.Bq, g.Bk, g.nQ, g.nK, BH, q, k, qbar, kbar);
  else
    hipLaunchKernelGGL((pool_mean_kernel<1, 8>), dim3(grid_for(work, 256)), dim3(256), 0, st,
                       g.N, g.H, g.D, g.Bq, g.Bk, g.nQ, g.nK, BH, q, k, qbar, kbar);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 grid((unsigned)((g.nK + kScoreTile - 1) / kScoreTile),
            (unsigned)((g.nQ + kScoreTile - 1) / kScoreTile), (unsigned)BH);
  hipLaunchKernelGGL(pooled_scores_kernel, grid, dim3(kScoreThreads), 0, st,
                     g.D, g.nQ, g.nK, scale, qbar, kbar, S);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mode == 2 || mode == 3) return launch_pooled_global(g, mode, param, mask, ws, st);
  const int64_t R = BH * g.nQ;
  if (g.nK > kPooledMaxBlocks) {
    // long rows: row maxima and Z after the scores, then one workgroup per row
    double* zrow = S + R * g.nK;
    double* mrow = zrow + R;
    hipLaunchKernelGGL(pooled_rowz_kernel, dim3((unsigned)((R + kWave - 1) / kWave)),
                       dim3(kWave), 0, st, R, g.nK, S, zrow, mrow, (int32_t*)nullptr);
    hipLaunchKernelGGL(pooled_select_long_kernel, dim3((unsigned)R), dim3(kLongThreads), 0, st,
                       g.nK, mode, param, levels ? levels[1] : 0.0, levels ? levels[2] : 0.0, levels ? levels[3] : 0.0,
                       n_levels, S, zrow, mrow, mask);
    return hipGetLastError();
  }
  if (mode == 4 && g.nK > 2 * kWave && g.nK <= 16 * kWave) {
    // pyramid levels: one wave per row, the row sorted in registers
    const size_t per = levels_wave_lds(g.nK);
    const int64_t rpg = std::max<int64_t>(
        1, std::min<int64_t>(kSelectRowsPerGroup, (int64_t)(65536 / per)));
    const dim3 grid((unsigned)((R + rpg - 1) / rpg)), block((unsigned)(kWave * rpg));
    const double t0 = levels[0], t1 = levels[1], t2 = levels[2], t3 = levels[3];
    if (g.nK <= 4 * kWave)
      hipLaunchKernelGGL(pooled_levels_wave_kernel<4>, grid, block, per * rpg, st, R, g.nK, t0,
                         t1, t2, t3, n_levels, S, mask);
    else if (g.nK <= 8 * kWave)
      hipLaunchKernelGGL(pooled_levels_wave_kernel<8>, grid, block, per * rpg, st, R, g.nK, t0,
                         t1, t2, t3, n_levels, S, mask);
    else
      hipLaunchKernelGGL(pooled_levels_wave_kernel<16>, grid, block, per * rpg, st, R, g.nK, t0,
                         t1, t2, t3, n_levels, S, mask);
    return hipGetLastError();
  }
  int32_t P = 1;
  while (P < g.nK) P <<= 1;
  int32_t only_marked = 0;
  if ((mode == 0 || mode == 1) && g.nK > kTopM && !(mode == 0 && param >= (double)g.nK)) {
    const size_t per = select_wave_lds(g.nK);
    const int64_t rpg = std::min<int64_t>(kSelectRowsPerGroup, (int64_t)(65536 / per));
    const dim3 grid((unsigned)((R + rpg - 1) / rpg)), block((unsigned)(kWave * rpg));
    if (g.nK <= 8 * kWave)
      hipLaunchKernelGGL(pooled_select_wave_kernel<8>, grid, block, per * rpg, st, R, g.nK, mode,
                         param, S, mask);
    else if (g.nK <= 16 * kWave)
      hipLaunchKernelGGL(pooled_select_wave_kernel<16>, grid, block, per * rpg, st, R, g.nK, mode,
                         param, S, mask);
    else
      hipLaunchKernelGGL(pooled_select_wave_kernel<32>, grid, block, per * rpg, st, R, g.nK, mode,
                         param, S, mask);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (mode == 0) return hipSuccess;  // top-k never needs the full sort
    only_marked = 1;
  }
  const size_t sh2 = sizeof(double) * (g.nK + P) + sizeof(int32_t) * P + g.nK;
  const int64_t groups = only_marked ? (R + kMarkedRowsPerGroup - 1) / kMarkedRowsPerGroup : R;
  hipLaunchKernelGGL(pooled_select_kernel, dim3((unsigned)groups), dim3(kSelectThreads), sh2, st,
                     g.nK, P, mode, param, levels ? levels[1] : 0.0, levels ? levels[2] : 0.0, levels ? levels[3] : 0.0,
                     n_levels, S, mask, only_marked, R);
  return hipGetLastError();
}

hipError_t launch_pooled_global(const Geom& g, int32_t mode, double param, uint8_t* mask,
                                void* ws, hipStream_t st) {
  const int64_t BH = (int64_t)g.B * g.H;
  if (BH == 0 || g.N == 0) return hipSuccess;
  const int64_t n = g.nQ * g.nK;
  double* S = (double*)ws + BH * (g.nQ + g.nK) * g.D;
  double* P = S + BH * n;
  int64_t* pc = (int64_t*)(P + BH * n);
  double* pm = (double*)(pc + BH * kGselGroups * 16);
  HeadCut* cut = (HeadCut*)(pm + BH * kGselGroups * 16);
  int32_t* best = (int32_t*)(cut + BH);
  const int64_t cand = BH * kGselGroups * gsel_cand_cap(n) * kGselThreads;
  const size_t head = ((size_t)((char*)(best + BH * g.nQ) - (char*)ws) + 255) / 256 * 256;
  uint64_t* ck = (uint64_t*)((char*)ws + head);  // same offset as pooled_workspace_bytes
  double* cm = (double*)(ck + cand);
  int32_t* ccnt = (int32_t*)(cm + cand);
  if (g.nK > kPooledMaxBlocks) {
    // long rows: maxima, Z and best blocks one lane per row (kept in the
    // candidate store until the probabilities are formed), then p elementwise
    double* zrow = (double*)ck;
    double* mrow = zrow + BH * g.nQ;
    hipLaunchKernelGGL(pooled_rowz_kernel, dim3((unsigned)((BH * g.nQ + kWave - 1) / kWave)),
                       dim3(kWave), 0, st, BH * g.nQ, g.nK, S, zrow, mrow, best);
    if (mode == 3)
      hipLaunchKernelGGL(pooled_prob_kernel, dim3(grid_for(BH * n, 256)), dim3(256), 0, st,
                         BH * n, g.nK, S, zrow, mrow, P);
  } else {
    hipLaunchKernelGGL(pooled_rowstats_kernel, dim3((unsigned)(BH * g.nQ)), dim3(kWave), 0, st,
                       g.nK, mode, S, P, best);
  }
  hipLaunchKernelGGL(gsel_init_kernel, dim3(grid_for(BH, 64)), dim3(64), 0, st, BH, g.nQ, g.nK,
                     mode, param, cut);
  // passes over every pair, the last of them filling the candidate store;
  // then the remaining digits over the candidates in one launch
  int shift = 60;
  for (int pass = 0; pass <= kGselFullPasses; ++pass, shift -= 4) {
    const int32_t phase = pass < kGselFullPasses ? 0 : 1;
    hipLaunchKernelGGL(gsel_hist_kernel, dim3(kGselGroups, (unsigned)BH), dim3(kGselThreads), 0,
                       st, g.nQ, g.nK, mode, shift, S, P, cut, pc, pm, phase, ck, cm, ccnt);
  }
  hipLaunchKernelGGL(gsel_finish_kernel, dim3((unsigned)BH), dim3(kGselThreads), 0, st, g.nQ,
                     g.nK, mode, shift, cut, ck, cm, ccnt);
  hipLaunchKernelGGL(gsel_ties_kernel, dim3(grid_for(BH, 64)), dim3(64), 0, st, BH, n, mode, S, P,
                     cut);
  hipLaunchKernelGGL(gsel_mark_kernel, dim3(grid_for(BH * n, 256)), dim3(256), 0, st, BH, g.nQ,
                     g.nK, mode, S, P, best, cut, mask);
  return hipGetLastError();
}

hipError_t launch_compact_count_scan(const Geom& g, int64_t R, const uint8_t* mask,
                                     int64_t mhs, const uint8_t* skip, int32_t* row_ptr,
                                     hipStream_t st) {
  const int waves = 4;
  hipLaunchKernelGGL(compact_count_kernel, dim3(grid_for(R, waves, INT32_MAX)),
                     dim3(waves * kWave), 0, st, R, g.nQ, g.nK, mask, mhs, skip, row_ptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, R, row_ptr);
  return hipGetLastError();
}

hipError_t launch_compact_scatter(const Geom& g, int64_t R, const uint8_t* mask, int64_t mhs,
                                  const uint8_t* skip, const int32_t* row_ptr, int32_t* kv_idx,
                                  hipStream_t st) {
  const int waves = 4;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3(grid_for(R, waves, INT32_MAX)),
                     dim3(waves * kWave), 0, st, R, g.nQ, g.nK, mask, mhs, skip, row_ptr,
                     kv_idx);
  return hipGetLastError();
}

hipError_t launch_pyramid_lists(const Geom& g, int32_t n_levels, const int64_t* rb,
                                const uint8_t* mask, int64_t mhs, int32_t* row_ptr,
                                int32_t* kv_idx, int32_t* kv_eighths, bool count_only,
                                hipStream_t st) {
  const int64_t R = (int64_t)g.B * g.H * g.nQ;
  PyrRegions reg;
  for (int i = 0; i < 5; ++i) reg.rb[i] = i <= n_levels ? rb[i] : rb[n_levels];
  reg.n_levels = n_levels;
  const int waves = 4;
  if (count_only) {
    hipLaunchKernelGGL(pyr_count_kernel, dim3(grid_for(R, waves, INT32_MAX)), dim3(waves * kWave),
                       0, st, R, g.nQ, g.nK, reg, mask, mhs, row_ptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, R, row_ptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(pyr_scatter_kernel, dim3(grid_for(R, waves, INT32_MAX)), dim3(waves * kWave),
                     0, st, R, g.nQ, g.nK, reg, mask, mhs, row_ptr, kv_idx, kv_eighths);
  return hipGetLastError();
}

hipError_t launch_zero_row_ptr(int32_t* row_ptr, hipStream_t st) {
  hipLaunchKernelGGL(zero_row_ptr_kernel, dim3(1), dim3(1), 0, st, row_ptr);
  return hipGetLastError();
}

hipError_t launch_order_lists(const Geom& g, int64_t R, int32_t order, const int32_t* row_ptr,
                              const int32_t* kv_in, int32_t* kv_out, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int waves = 4;
  hipLaunchKernelGGL(order_lists_kernel, dim3(grid_for(R, waves, INT32_MAX)), dim3(waves * kWave),
                     0, st, R, g.nQ, g.N, g.Bq, g.Bk, order, row_ptr, kv_in, kv_out);
  return hipGetLastError();
}

hipError_t launch_skip_update(const Geom& g, const int32_t* row_ptr, const int32_t* kv_idx,
                              const float* tile_gap, float tau2, uint8_t* skip,
                              hipStream_t st) {
  const int64_t R = (int64_t)g.B * g.H * g.nQ;
  if (R == 0) return hipSuccess;
  const int waves = 4;
  hipLaunchKernelGGL(skip_update_kernel, dim3(grid_for(R, waves, INT32_MAX)),
                     dim3(waves * kWave), 0, st, R, g.nK, row_ptr, kv_idx, tile_gap, -tau2,
                     skip);
  return hipGetLastError();
}

}  // namespace bsa
