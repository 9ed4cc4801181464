// attn_bf16.hip -- bf16 MFMA block-sparse attention forward for gfx950.
//
// Method: whole (row block, key block) tiles are kept or dropped
// ([PSA] "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍", binary block
// sparsity); each workgroup walks only the listed key blocks of its row
// block, so a dropped tile costs no load, no softmax and no MFMA
// ([Lite] LiteAttention summary page, sections 三 and 六). Softmax is the
// online form in log2 units; the per-tile gap (local max minus running max)
// feeds the carried skip mask ([Lite] section 五), reduced across waves once
// per tile on the barrier the pipeline already has ([Lite] section 六 defers
// the cross-warp reduction for the same reason).
//
// gfx950 mapping (one workgroup per (b, h, row block); BQ/32 waves, each wave
// owns 32 query rows):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K tile rows from LDS,
//    B = the wave's Q rows held in registers for the whole kernel. In the
//    32x32 accumulator a lane holds one query row (lane % 32) and 16 of the
//    32 keys of a block, so a row max is 31 in-lane maxima plus one
//    cross-half swap (v_permlane32_swap), and row sums stay per lane half
//    until the epilogue.
//  * O^T = V^T P^T: the score accumulator registers, rounded to bf16, are
//    directly the B operand (same lane -> query row); the key order inside a
//    16-key step is permuted identically in A and B, so no data moves across
//    lanes. V is stored transposed in LDS (Vt[d][key]) so each A operand is
//    two 8-byte reads; the transpose happens on the way in: each thread
//    loads 8 key rows of one dword column and repacks them with v_perm.
//  * K/V tiles are double-buffered in LDS with register staging: the global
//    loads of tile i+1 are issued before the MFMAs of tile i; one barrier
//    per tile.
//  * Workgroup ids are remapped so consecutive row blocks of a head land on
//    the same XCD (hardware dispatch is round-robin over the 8 XCDs), which
//    keeps the K/V tiles neighbouring row blocks share in that XCD's L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBk = 64;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Bf16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
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

__device__ inline float other_half(float x) {
  // v_permlane32_swap: lanes 0-31 receive lanes 32-63 and vice versa.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(threadIdx.x % 64 < 32 ? r[1] : r[0]);
}

template <int D, int BQ>
struct Cfg {
  static constexpr int NW = BQ / 32;        // waves
  static constexpr int NT = NW * 64;        // threads
  static constexpr int KS = D / 16;         // k-steps of Q K^T
  static constexpr int DB = D / 32;         // 32-wide d blocks of O
  static constexpr int KLD = D + 8;         // K tile row stride (elements)
  static constexpr int VLD = kBk + 4;       // V^T tile row stride (elements)
  static constexpr int KTILE = kBk * KLD;
  static constexpr int VTILE = D * VLD;
  static constexpr int KCH = kBk * (D / 8) / NT;  // 16-byte K chunks per thread
  static constexpr int VIT = 8 * (D / 2) / NT;    // 8-row V column groups per thread
  static_assert(KCH >= 1 && VIT >= 1, "tile loader split");
  static_assert(BQ * (D + 8) <= 2 * KTILE, "O staging must fit in the K buffers");
};

template <int D, int BQ>
struct Stage {
  u32x4 k[Cfg<D, BQ>::KCH];
  uint32_t v[Cfg<D, BQ>::VIT][8];
};

template <int D, int BQ>
__device__ inline void load_tile(const Bf16Params& p, const uint16_t* kbase,
                                 const uint16_t* vbase, int64_t c, int tid,
                                 Stage<D, BQ>& st) {
  using C = Cfg<D, BQ>;
  const int64_t j0 = c * kBk;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int id = tid + i * C::NT;
    const int r = id / (D / 8), c8 = id % (D / 8);
    const int64_t kv = j0 + r;
    st.k[i] = kv < p.N ? *(const u32x4*)(kbase + kv * p.ksn + c8 * 8) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < C::VIT; ++it) {
    const int id = tid + it * C::NT;
    const int g8 = id / (D / 2), pc = id % (D / 2);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t kv = j0 + g8 * 8 + r;
      st.v[it][r] = kv < p.N ? *(const uint32_t*)(vbase + kv * p.vsn + 2 * pc) : 0u;
    }
  }
}

template <int D, int BQ>
__device__ inline void store_tile(uint16_t* Ks, uint16_t* Vt, int tid, const Stage<D, BQ>& st) {
  using C = Cfg<D, BQ>;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int id = tid + i * C::NT;
    const int r = id / (D / 8), c8 = id % (D / 8);
    *(u32x4*)(Ks + r * C::KLD + c8 * 8) = st.k[i];
  }
#pragma unroll
  for (int it = 0; it < C::VIT; ++it) {
    const int id = tid + it * C::NT;
    const int g8 = id / (D / 2), pc = id % (D / 2);
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = st.v[it][2 * w], y = st.v[it][2 * w + 1];
      lo[w] = __builtin_amdgcn_perm(y, x, 0x05040100u);  // low halves: column 2*pc
      hi[w] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // high halves: column 2*pc+1
    }
    uint16_t* r0 = Vt + (2 * pc) * C::VLD + g8 * 8;
    uint16_t* r1 = r0 + C::VLD;
    *(u32x2*)(r0) = u32x2{lo[0], lo[1]};
    *(u32x2*)(r0 + 4) = u32x2{lo[2], lo[3]};
    *(u32x2*)(r1) = u32x2{hi[0], hi[1]};
    *(u32x2*)(r1 + 4) = u32x2{hi[2], hi[3]};
  }
}

template <int D, int BQ, bool GAP>
__global__ __launch_bounds__(BQ * 2, 2) void attn_bf16_kernel(const Bf16Params p) {
  using C = Cfg<D, BQ>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][C::VTILE];
  __shared__ float gp[2][C::NW];

  const int tid = threadIdx.x;
  const int lane = tid % 64, w = tid / 64;
  const int n = lane % 32, hh = lane / 32;

  // XCD-aware remap: hardware sends workgroup x to XCD x % 8; give each XCD a
  // contiguous range of (head, row block) ids.
  const int64_t G = gridDim.x, wg = blockIdx.x;
  const int64_t xcd = wg % kXcds, kk = wg / kXcds, q8 = G / kXcds, r8 = G % kXcds;
  const int64_t row = xcd * q8 + min(xcd, r8) + kk;  // (b*H + h)*nQ + a
  const int64_t bh = row / p.nQ, a = row - bh * p.nQ;
  const int64_t b = bh / p.H, h = bh - b * p.H;

  // Q rows of this wave as MFMA B operands (k-slice hh*8..+7 of each 16-step).
  const int64_t qrow = a * BQ + w * 32 + n;
  const bool qvalid = qrow < p.N;
  bf16x8 qf[C::KS];
  {
    const uint16_t* qp = p.q + b * p.qsb + qrow * p.qsn + h * p.qsh + hh * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 raw = qvalid ? *(const u32x4*)(qp + ks * 16) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  int64_t e0 = 0, e1 = p.nK, gbase = 0;
  if (p.row_ptr) {
    const int64_t lr = p.lists_shared ? a : row;
    e0 = p.row_ptr[lr];
    e1 = p.row_ptr[lr + 1];
    if (GAP && p.lists_shared) gbase = bh * (int64_t)p.row_ptr[p.nQ];
  }
  const int64_t L = e1 - e0;
  const uint16_t* kbase = p.k + b * p.ksb + h * p.ksh;
  const uint16_t* vbase = p.v + b * p.vsb + h * p.vsh;

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // log2 units
  float l_lane = 0.f;       // this lane half's share of the row sum

  Stage<D, BQ> stg;
  if (L > 0) {
    load_tile<D, BQ>(p, kbase, vbase, p.row_ptr ? p.kv_idx[e0] : e0, tid, stg);
    store_tile<D, BQ>(Ks[0], Vt[0], tid, stg);
  }
  __syncthreads();

  for (int64_t it = 0; it < L; ++it) {
    const int buf = (int)(it & 1);
    const int64_t c = p.row_ptr ? p.kv_idx[e0 + it] : e0 + it;
    const bool has_next = it + 1 < L;
    if (has_next)
      load_tile<D, BQ>(p, kbase, vbase, p.row_ptr ? p.kv_idx[e0 + it + 1] : e0 + it + 1, tid,
                       stg);

    // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks).
    const uint16_t* ks_ = Ks[buf];
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 av = *(const bf16x8*)(ks_ + (kb * 32 + n) * C::KLD + ks * 16 + hh * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax. Lane value j of block kb is key
    // kb*32 + 8*(j/4) + 4*hh + j%4 of the tile.
    const bool ragged = (c + 1) * kBk > p.N;
    const int64_t jv = p.N - c * kBk;  // valid keys in this tile
    float mloc = -INFINITY;
    if (!ragged) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mloc = fmaxf(mloc, sacc[kb][j]);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * 32 + 8 * (j / 4) + 4 * hh + (j % 4);
          if (key < jv) mloc = fmaxf(mloc, sacc[kb][j]);
        }
    }
    mloc = fmaxf(mloc, other_half(mloc));
    const float m_loc2 = mloc * p.sl2;
    if (GAP) {
      float g = qvalid ? m_loc2 - m_run : -INFINITY;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) g = fmaxf(g, __shfl_xor(g, off, 32));
      if (lane == 0) gp[buf][w] = g;
    }
    const float m_new = fmaxf(m_run, m_loc2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x8 pv;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = half * 8 + t;
          float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j], p.sl2, -m_new));
          if (ragged) {
            const int key = kb * 32 + 8 * (j / 4) + 4 * hh + (j % 4);
            pr = key < jv ? pr : 0.f;
          }
          rs += pr;
          pv[t] = pr;
        }
        pb[kb][half] = __builtin_convertvector(pv, bf16x8);
      }
    }
    l_lane = l_lane * alpha + rs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T. For the 16-key step (kb, half) the B operand is
    // pb[kb][half]; element t of lane half hh is key
    // kb*32 + 16*half + 8*(t/4) + 4*hh + t%4, so the A operand reads those
    // keys of Vt row d: two runs of four.
    const uint16_t* vt = Vt[buf];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kbase_ = kb * 32 + 16 * half + 4 * hh;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const uint16_t* rp = vt + (db * 32 + n) * C::VLD + kbase_;
          const u32x2 lo = *(const u32x2*)(rp);
          const u32x2 hi = *(const u32x2*)(rp + 8);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kb][half], oacc[db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile<D, BQ>(Ks[buf ^ 1], Vt[buf ^ 1], tid, stg);
    __syncthreads();
    if (GAP && tid == 0) {
      float g = gp[buf][0];
#pragma unroll
      for (int x = 1; x < C::NW; ++x) g = fmaxf(g, gp[buf][x]);
      p.tile_gap[gbase + e0 + it] = g;
    }
  }

  // ---- epilogue: O = O^T / l through LDS for coalesced 16-byte stores.
  const float l_tot = l_lane + other_half(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __syncthreads();
  uint16_t* Os = &Ks[0][0];
  constexpr int OLD = D + 8;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 tmp;
#pragma unroll
      for (int t = 0; t < 4; ++t) tmp[t] = oacc[db][4 * j4 + t] * inv;
      const bf16x4 ov = __builtin_convertvector(tmp, bf16x4);
      *(bf16x4*)(Os + (w * 32 + n) * OLD + db * 32 + 8 * j4 + 4 * hh) = ov;
    }
  }
  __syncthreads();
  uint16_t* obase = p.o + b * p.osb + h * p.osh;
#pragma unroll
  for (int i = 0; i < BQ * (D / 8) / C::NT; ++i) {
    const int id = tid + i * C::NT;
    const int r = id / (D / 8), c8 = id % (D / 8);
    const int64_t orow = a * BQ + r;
    if (orow < p.N) *(u32x4*)(obase + orow * p.osn + c8 * 8) = *(const u32x4*)(Os + r * OLD + c8 * 8);
  }
  if (p.lse && hh == 0 && qvalid)
    p.lse[bh * p.N + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int BQ>
hipError_t launch(const Geom& g, const Bf16Params& p, hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.H * g.nQ;
  if (p.tile_gap)
    hipLaunchKernelGGL((attn_bf16_kernel<D, BQ, true>), dim3((unsigned)rows),
                       dim3(Cfg<D, BQ>::NT), 0, st, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, BQ, false>), dim3((unsigned)rows),
                       dim3(Cfg<D, BQ>::NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Geom& g, const AttnArgs& a, hipStream_t st) {
  if ((int64_t)g.B * g.H * g.nQ == 0) return hipSuccess;
  Bf16Params p;
  p.q = (const uint16_t*)a.q.ptr;
  p.k = (const uint16_t*)a.k.ptr;
  p.v = (const uint16_t*)a.v.ptr;
  p.o = (uint16_t*)a.o;
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
