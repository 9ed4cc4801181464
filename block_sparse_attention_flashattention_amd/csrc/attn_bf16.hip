// attn_bf16.hip -- bf16 MFMA block-sparse attention forward for gfx950.
//
// Method: whole (row block, key block) tiles are kept or dropped
// ([PSA] "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍", binary block
// sparsity); each workgroup walks only the listed key blocks of its row
// block, so a dropped tile costs no load, no softmax and no MFMA
// ([Lite] LiteAttention summary page, sections 三 and 六). Softmax is the
// online form in log2 units; the per-tile gap (local max minus running max)
// feeds the carried skip mask ([Lite] section 五); the cross-wave part of
// that reduction is an order-independent atomic max per tile, so no wave
// waits on another for it ([Lite] section 六 defers the cross-warp
// reduction for the same reason).
//
// gfx950 mapping (one workgroup per (b, h, row block); BQ/32 waves, each wave
// owns 32 query rows):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K tile rows read from
//    LDS, B = the wave's Q rows held in registers for the whole kernel. In the
//    32x32 accumulator a lane holds one query row (lane % 32) and 16 of the
//    32 keys of a block, so a row max is in-lane maxima plus one cross-half
//    swap (v_permlane32_swap) and row sums stay per lane half until the end.
//  * O^T = V^T P^T: the score registers, rounded to bf16, are the B operand
//    as they stand (same lane -> query row); the A operand V^T is gathered
//    from the row-major V tile with ds_read_b64_tr_b16 (two per MFMA), whose
//    16-lane transpose delivers exactly the keys the score layout holds.
//  * K and V tiles go global -> LDS with 16-byte buffer loads that write LDS
//    directly (no register staging). A per-tile buffer resource bounds the
//    valid rows, so the ragged last key block reads zeros in hardware. The
//    global side is XOR-swizzled per row so both LDS read patterns (b128 for
//    K, b64 transpose for V) are free of bank conflicts without padding.
//  * Software pipeline, one barrier per tile. While the exponentials of tile
//    i run on the VALU, the matrix core computes the scores of tile i+1;
//    while it accumulates P_i V_i, the VALU reduces the row maxima of tile
//    i+1. Each of the two phases is laid out slot by slot: one MFMA per slot,
//    its share of the VALU work, and the LDS fragment reads for the MFMA
//    three slots ahead, with a scheduling fence between slots so that the
//    compiler keeps this interleave. K and V have two LDS stages each (tiles
//    i+2 and i+1 are requested right after the barrier of step i): 64 KiB,
//    two workgroups per CU. The loop is unrolled by two so that every stage
//    address is a constant offset of the LDS read instructions.
//  * Rescaling of O is lazy: the exponent base moves only when the row max
//    grows by more than 2^8, which keeps p <= 256 and leaves the result exact
//    up to rounding (numerator and denominator share the base).
//  * Workgroup ids are remapped so the row blocks an XCD runs together share
//    K/V tiles in its L2 (see the mapping in the kernel).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBk = 64;
constexpr int kXcds = 8;
constexpr int kBand = 2;  // row-block slots per position band
constexpr int kKStages = 2;
constexpr int kVStages = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2 units
// Pyramid step lists: capacity, in 32-bit group descriptors, of the
// per-workgroup list of selected 16-row groups (two per step with row blocks
// of 64, four with row blocks of 128); with its count the LDS still holds
// four (two) workgroups per CU.
constexpr int kStepCap = 2046;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family
constexpr int kPfK = 3;  // K fragment reads issued ahead of their score MFMA (slots)
constexpr int kPfV = 3;  // V fragment reads issued ahead of their P V MFMA (slots)

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
  int32_t T, U;  // frames; row-block slots per frame (ceil(F / BQ)), 0 = plain order
  int64_t F;     // tokens per frame
  // pyramid attention: key blocks >= rb1 are pooled levels held in kp / vp
  // (same row strides as k / v); level l region = blocks [rb_l, rb_{l+1}),
  // N >> l valid rows; kv_eighths = selected 8-row eighths per entry
  const uint16_t* kp;
  const uint16_t* vp;
  int64_t kpsb, kpsh, vpsb, vpsh;
  const int32_t* kv_eighths;
  int32_t rb1, rb2, rb3, rb4;
};

__device__ inline float other_half(float x) {
  // v_permlane32_swap: lanes 0-31 receive lanes 32-63 and vice versa.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float((threadIdx.x & 63) < 32 ? r[1] : r[0]);
}

// Read of list data at a wave-uniform index through the constant address
// space, so it becomes a scalar load (counted by lgkmcnt, not vmcnt).
__device__ inline int32_t load_uniform(const int32_t* base, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)base)[i];
}

// Maximum that propagates NaN (IEEE maximum, v_maximum3_f32 when chained),
// for row maxima of scores and for tile gaps. fmaxf must first quiet every
// input not known to be canonical (matrix-core results, DPP moves), which
// costs one more instruction per input; the values here are finite or
// +-inf, where the two agree.
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over lanes 0..31 (every lane receives it): DPP within each 16-lane
// row (swap neighbours, swap pairs, mirror 8, mirror 16), then the two rows
// through scalar registers. No LDS traffic, unlike a bpermute shuffle. A
// NaN input (impossible for valid rows) would propagate, and a NaN gap never
// marks a tile.
template <int CTRL>
__device__ inline float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ inline float max_lanes32(float v) {
  v = vmax(v, dpp_move<0xB1>(v));   // quad_perm(1, 0, 3, 2)
  v = vmax(v, dpp_move<0x4E>(v));   // quad_perm(2, 3, 0, 1)
  v = vmax(v, dpp_move<0x141>(v));  // row_half_mirror
  v = vmax(v, dpp_move<0x140>(v));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  return vmax(r0, r1);
}

// Value of lane 0 (an SGPR) for quantities that are uniform across the wave.
__device__ inline int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline uint64_t wave_uniform64(uint64_t x) {
  return (uint64_t)(uint32_t)wave_uniform((int)(uint32_t)x) |
         ((uint64_t)(uint32_t)wave_uniform((int)(uint32_t)(x >> 32)) << 32);
}

// Wait until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }
// Wait for every LDS and scalar-memory access of this wave. Issued through
// the builtin (not inline assembly) so that the compiler's own wait-count
// pass sees it and knows that no scalar load is outstanding afterwards.
// Encoding: vmcnt 63 (bits 3:0 and 15:14), expcnt 7 (bits 6:4), lgkmcnt 0.
__device__ inline void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Float max into global memory, independent of arrival order: non-negative
// values order like signed ints, negative ones inversely like unsigned ints.
__device__ inline void atomic_max_float(float* addr, float v) {
  if (__float_as_int(v) >= 0)
    atomicMax((int*)addr, __float_as_int(v));
  else
    atomicMin((unsigned int*)addr, __float_as_uint(v));
}

// LDS layout of a 64-row tile of D bf16 per row: rows of D*2 bytes, 16-byte
// chunk c of row r stored at chunk c ^ f(r). K uses fK (conflict-free b128
// reads of 16 consecutive rows), V uses fV (conflict-free transpose reads of
// 4-row x 32-byte blocks).
template <int D, int ROWS = kBk>
struct Tile {
  static constexpr int CPR = D / 8;        // chunks per row
  static constexpr int RB = D * 2;         // bytes per row
  static constexpr int BYTES = ROWS * RB;  // bytes per stage
  static constexpr int RPI = 1024 / RB;    // rows per 64-lane 16-byte load
  static constexpr int IPT = ROWS / RPI;   // loads per stage
  __device__ static int fK(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int fV(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// BQ rows per workgroup (32 per wave); SUB keys per pipeline step (a whole
// 64-key block, or half of one so that two-wave workgroups fit four per CU).
template <int D, int BQ, int SUB>
struct Cfg {
  using T = Tile<D, SUB>;
  static constexpr int NW = BQ / 32;                // waves
  static constexpr int NT = NW * 64;                // threads
  static constexpr int KS = D / 16;                 // k-steps of Q K^T
  static constexpr int DB = D / 32;                 // 32-wide d blocks of O
  static constexpr int KB = SUB / 32;               // 32-key blocks per step
  static constexpr int NSUB = kBk / SUB;            // steps per key block
  static constexpr int LPW = T::IPT / NW;           // loads per stage per wave (K or V)
  static constexpr int VOFF = kKStages * T::BYTES;  // V stages follow the K stages
  static constexpr int SMEM = (kKStages + kVStages) * T::BYTES;
  static constexpr int OLD = D + 8;                 // O staging row stride (elements)
  static constexpr int NA = KS * KB;                // score MFMAs per step
  static constexpr int NB = KB * 2 * DB;            // P V MFMAs per step
  static constexpr int EPS = 16 * KB / NA;          // probabilities per score MFMA (per lane)
  static constexpr int MPS = 16 * KB / NB;          // max inputs per P V MFMA (per lane)
  static_assert(LPW >= 1, "tile loader split");
  static_assert(EPS % 2 == 0 && MPS % 2 == 0 && EPS * NA == 16 * KB && MPS * NB == 16 * KB,
                "softmax work splits evenly over the MFMA slots");
  static_assert(kPfK < NA && kPfV < NB, "fragment prefetch depth");
  static_assert(BQ * OLD * 2 <= SMEM, "O staging must fit in the stages");
};

// Per-lane voffsets of this wave's LPW direct loads of one K stage and one V
// stage (swizzles fK and fV applied on the global side).
template <int LPW>
struct LoadPlan {
  uint32_t k[LPW];
  uint32_t v[LPW];
};

// SPLIT: every load fills rows of one 16-row group of the tile (4 or 8
// rows each) and takes them from that group's own descriptor, which starts
// at the row landing in the group's first tile row, so that the groups of a
// stage may come from different places (issue_rows_grouped).
template <int D, int NW, int LPW, bool SPLIT = false>
__device__ inline void make_plan(LoadPlan<LPW>& lp, int w, int lane, int64_t ksn, int64_t vsn) {
  using T = Tile<D>;
  static_assert(!SPLIT || 16 % T::RPI == 0, "a load's rows lie in one 16-row group");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int idx = w + NW * i;
    const int r = T::RPI * idx + lane / T::CPR;
    const int rg = SPLIT ? (r & 15) : r;  // row within its descriptor
    const int phys = lane % T::CPR;
    lp.k[i] = (uint32_t)(rg * ksn * 2 + (phys ^ T::fK(r)) * 16);
    lp.v[i] = (uint32_t)(rg * vsn * 2 + (phys ^ T::fV(r)) * 16);
  }
}

// 16 bytes per lane from global memory straight into LDS; lane l's bytes
// land at M0 + 16*l. Written as inline assembly on purpose: the compiler's
// wait-count pass cannot tell LDS stages apart and would otherwise drain every
// outstanding load before each LDS read, which defeats prefetching. The
// kernel orders these loads itself (explicit vmcnt waits and barriers). The
// s_nop is the one wait state required between an M0 write and an LDS DMA
// load that reads it. Rows at or beyond the descriptor's num_records read as
// zero.
template <uint32_t OFS>
__device__ inline void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc), "n"(OFS) : "memory", "m0", "scc");
}

// This wave's share of the direct global -> LDS loads of `rows` (0..SUB)
// key rows starting at j0 into the stage at byte offset SO; `wave_lds` is the
// LDS address of this wave's first 1 KiB slot (LDS base + 1024 * wave).
template <int NW, int LPW, uint32_t SO, int I = 0>
__device__ inline void issue_rows(const uint32_t* off, const i32x4& rs, uint32_t wave_lds) {
  if constexpr (I < LPW) {
    dma16<SO + NW * I * 1024>(rs, wave_lds, off[I]);
    issue_rows<NW, LPW, SO, I + 1>(off, rs, wave_lds);
  }
}

// Descriptors of the (2 or 4) 16-row groups of a stage, as named members
// rather than an array, so that picking one never goes through memory.
struct GroupRsrc {
  i32x4 r0, r1, r2, r3;
  __device__ void set(int g, const i32x4& v) {
    if (g == 0) r0 = v;
    else if (g == 1) r1 = v;
    else if (g == 2) r2 = v;
    else r3 = v;
  }
  __device__ i32x4 get(int g) const { return g == 0 ? r0 : (g == 1 ? r1 : (g == 2 ? r2 : r3)); }
};

// issue_rows for a split plan: load I of wave w fills tile rows from
// RPI * (w + NW * I), in group RPI * (w + NW * I) / 16, from that group's
// descriptor. When one round of the workgroup's loads (RPI * NW rows)
// divides 16 rows, the group does not depend on the wave and is a constant;
// otherwise it is picked at run time (one wave-uniform index).
template <int NW, int LPW, int RPI, uint32_t SO, int I = 0>
__device__ __attribute__((always_inline)) inline void issue_rows_grouped(
    const uint32_t* off, const GroupRsrc& rs, int w, uint32_t wave_lds) {
  static_assert((RPI * NW <= 16 && 16 % (RPI * NW) == 0) || (RPI * NW) % 16 == 0,
                "loads of one round align with the 16-row groups");
  if constexpr (I < LPW) {
    i32x4 r;
    if constexpr (RPI * NW <= 16) {
      r = rs.get(RPI * NW * I / 16);
    } else {
      r = rs.get(wave_uniform(RPI * (w + NW * I) / 16));
      r = i32x4{wave_uniform(r[0]), wave_uniform(r[1]), wave_uniform(r[2]), wave_uniform(r[3])};
    }
    dma16<SO + NW * I * 1024>(r, wave_lds, off[I]);
    issue_rows_grouped<NW, LPW, RPI, SO, I + 1>(off, rs, w, wave_lds);
  }
}

// Buffer descriptor for `rows` key rows from row j0 of a (b, h) slice with
// row stride sn elements; reads at or beyond the last row return zero.
__device__ inline i32x4 rows_rsrc(const uint16_t* base, int64_t sn, int j0, int rows) {
  const uint64_t a = (uint64_t)(base + (int64_t)j0 * sn);
  // wave-uniform by construction; readfirstlane keeps the descriptor in SGPRs
  // (the row count first, so that its product is a scalar multiply)
  const int32_t r = wave_uniform(rows);
  return i32x4{wave_uniform((int32_t)(uint32_t)a), wave_uniform((int32_t)((a >> 32) & 0xffff)),
               r * (int32_t)sn * 2, kRsrcWord3};
}

__device__ inline bf16x8 join(i16x4 lo, i16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// Key of lane value j (0..15) of 32-key block kb: kb*32 + 8*(j/4) + 4*hh + j%4.
__device__ inline int key_of(int kb, int j, int hh) { return kb * 32 + 8 * (j / 4) + 4 * hh + (j % 4); }

// A step of the pyramid step list: the 32-bit descriptors of its NG 16-row
// groups (see attn_bf16_kernel); where the step list is not in use, a list
// entry's key block, in g[0].
template <int NG>
struct GroupCode {
  uint32_t g[NG];
  __device__ GroupCode() : g{} {}
  __device__ GroupCode(int v) : g{} { g[0] = (uint32_t)v; }
  __device__ operator int() const { return (int)g[0]; }
};
template <int NG>
__device__ inline uint32_t code_word(const GroupCode<NG>& c, int i) { return c.g[i]; }
__device__ inline uint32_t code_word(int, int) { return 0; }  // plain list entry: no groups

template <int D, int BQ, int SUB, bool GAP, bool PYR>
__global__ __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(const Bf16Params p) {
  static_assert(!(GAP && PYR), "tile gaps are defined on single-level lists");
  using C = Cfg<D, BQ, SUB>;
  using T = typename C::T;
  constexpr int KB = C::KB, NSUB = C::NSUB;
  // pyramid lists stepped as 16-row groups (SL): groups with no selected
  // eighth are left out (they would only compute masked keys), and the
  // selected ones are packed GS per step (two per 32-key step, four per
  // 64-key step), from any tiles and levels; each group has its own level,
  // valid rows and load descriptor. Keys 16 g .. 16 g + 15 of a step are
  // group g: a lane's scores j < 8 of 32-key block kb are group 2 kb, the
  // others group 2 kb + 1.
  constexpr bool SL = PYR;
  constexpr int GS = 2 * KB;
  // eighth mask of a step with every key selected (4 bits per 32 keys)
  constexpr int QF = (1 << (4 * KB)) - 1;
  // step codes: list entries (key blocks), or with the pyramid step list the
  // group descriptors of the step
  using CodeT = std::conditional_t<SL, GroupCode<GS>, int>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  // group descriptors (see the pyramid step list below)
  __shared__ __attribute__((aligned(16))) int32_t steplist[SL ? kStepCap : 2];
  __shared__ int32_t steps_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_uniform(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;

  // Workgroup -> (head, row block). Hardware dispatch sends workgroup x to
  // XCD x % 8; each XCD gets a contiguous range of the order below, so the
  // row blocks it runs together share their K/V tiles in its L2. Within a
  // head the order is position-major when U > 0 (shared lists): bands of
  // kBand row-block slots per frame, all frames of a band before the next
  // band. Row blocks at the same in-frame position in different frames visit
  // the same key frames in the same ascending order, so concurrently running
  // ones reuse each other's tiles while they are still cached. With U = 0
  // (per-head lists, tiny frames) row blocks run in plain order.
  const int64_t G = gridDim.x, wg = blockIdx.x;
  const int64_t xcd = wg % kXcds, kk = wg / kXcds, q8 = G / kXcds, r8 = G % kXcds;
  const int64_t lid = xcd * q8 + min(xcd, r8) + kk;
  const int64_t per_head = p.U ? (int64_t)p.T * p.U : p.nQ;
  const int64_t bh = lid / per_head;
  int64_t a = lid - bh * per_head;  // plain order when frames are tiny (U == 0)
  if (p.U) {
    const int64_t r = lid - bh * per_head;
    const int64_t nb = (p.U + kBand - 1) / kBand;
    const int64_t band = min(r / ((int64_t)p.T * kBand), nb - 1);
    const int64_t r2 = r - band * p.T * kBand;
    const int64_t bw = band == nb - 1 ? p.U - band * kBand : kBand;
    const int64_t t = r2 / bw, u = band * kBand + (r2 - t * bw);
    const int64_t f0 = (t * p.F + BQ - 1) / BQ, f1 = ((t + 1) * p.F + BQ - 1) / BQ;
    if (u >= f1 - f0) return;  // this frame has fewer row blocks than slots
    a = f0 + u;
  }
  const int64_t row = bh * p.nQ + a;  // list row when lists are per head
  const int64_t b = bh / p.H, h = bh - b * p.H;

  // List entries, steps and key rows fit in 32 bits (row_ptr is int32 and
  // N < 2^31); 32-bit scalar arithmetic keeps the loop's index math on the
  // scalar unit.
  int e0 = 0, e1 = (int)p.nK;
  int64_t gbase = 0;
  if (p.row_ptr) {
    const int64_t lr = p.lists_shared ? a : row;
    e0 = load_uniform(p.row_ptr, lr);
    e1 = load_uniform(p.row_ptr, lr + 1);
    if (GAP && p.lists_shared) gbase = bh * (int64_t)load_uniform(p.row_ptr, p.nQ);
  }
  const int L = e1 - e0;      // listed key blocks
  int LS = L * NSUB;          // pipeline steps (SUB keys each)
  const int N32 = (int)p.N;
  const uint16_t* kbase = p.k + b * p.ksb + h * p.ksh;
  const uint16_t* vbase = p.v + b * p.vsb + h * p.vsh;
  const uint16_t* kpbase = PYR ? p.kp + b * p.kpsb + h * p.kpsh : nullptr;
  const uint16_t* vpbase = PYR ? p.vp + b * p.vpsb + h * p.vpsh : nullptr;
  // Step u covers keys [j0, j0 + SUB) with j0 = 64 * (key block of list
  // entry i) + SUB * part: i = u / NSUB and part = u % NSUB (static in the
  // unrolled loop below), or both from the step list.
  auto entry_of = [&](int u) -> int { return u / NSUB; };
  auto part_of = [&](int u) -> int { return u % NSUB; };
  auto block_of = [&](int u) -> int {
    const int i = entry_of(u);
    return p.row_ptr ? load_uniform(p.kv_idx, e0 + i) : e0 + i;
  };
  // Pyramid level of a key block (0 outside pyramid lists), the first row of
  // the step in its source tensor (k or kp), and the valid rows of the step
  // (level l region holds N >> l rows).
  auto level_of = [&](int c) -> int {
    if constexpr (!PYR) return 0;
    return c < p.rb1 ? 0 : (c < p.rb2 ? 1 : (c < p.rb3 ? 2 : 3));
  };
  auto first_key = [&](int c, int part) -> int {
    if constexpr (PYR)
      if (c >= p.rb1) return (c - p.rb1) * kBk + part * SUB;
    return c * kBk + part * SUB;
  };
  auto valid_keys = [&](int c, int part) -> int {
    if constexpr (PYR) {
      if (c < 0 || c >= p.rb4) return 0;  // not an augmented block: nothing read
      const int l = level_of(c);
      const int rb_l = l == 0 ? 0 : (l == 1 ? p.rb1 : (l == 2 ? p.rb2 : p.rb3));
      return max(0, min(SUB, (N32 >> l) - ((c - rb_l) * kBk + part * SUB)));
    }
    return max(0, min(SUB, N32 - first_key(c, part)));
  };
  // Selected eighths of step u's keys, as a mask over the step's 8-key
  // eighths, bit i = keys 8i .. 8i+7 of the step (all set outside pyramid
  // lists).
  auto eighths_of = [&](int u) -> int {
    if constexpr (!PYR) return QF;
    const int q = load_uniform(p.kv_eighths, e0 + entry_of(u));
    return NSUB == 2 ? (q >> (4 * part_of(u))) & 0xF : q;
  };

  // Pyramid step list: wave 0 lists the row's 16-row groups (pairs of
  // eighths) that hold a selected eighth, in list order, as 32-bit
  // descriptors: first key row in k or kp / 16 << 11 | valid rows << 4 |
  // level << 2 | the group's two eighth bits. Step u is groups GS u ..
  // GS u + GS - 1 (zero, empty, descriptors pad the last step), read as one
  // 64- or 128-bit LDS word with no address arithmetic on levels.
  bool use_sl = false;
  auto g_row0 = [](uint32_t d) -> int { return (int)(d >> 11) << 4; };
  auto g_valid = [](uint32_t d) -> int { return (int)(d >> 4) & 31; };
  auto g_level = [](uint32_t d) -> int { return (int)(d >> 2) & 3; };
  auto g_eighths = [](uint32_t d) -> int { return (int)d & 3; };
  if constexpr (SL) {
    // else every listed tile is stepped through, its groups taken from the
    // list entry (row offsets fit 20 bits below 2^24; a list longer than the
    // capacity is not used)
    if (N32 < (1 << 24)) {
      if (w == 0) {
        int base = 0;
        const uint64_t below = (1ull << lane) - 1;
        for (int j0 = 0; j0 < L; j0 += 64) {
          const int j = j0 + lane;
          const int q = j < L ? p.kv_eighths[e0 + j] : 0;
          const int c = j < L ? p.kv_idx[e0 + j] : 0;
          int pos = base, cnt = 0;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(((q >> (2 * g)) & 3) != 0);
            pos += __popcll(m & below);
            cnt += __popcll(m);
          }
          if (q) {
            const int l = level_of(c);
            const int rb_l = l == 0 ? 0 : (l == 1 ? p.rb1 : (l == 2 ? p.rb2 : p.rb3));
            const int row0 = first_key(c, 0), lrow0 = (c - rb_l) * kBk;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int e = (q >> (2 * g)) & 3;
              if (e) {
                const int valid = max(0, min(16, (N32 >> l) - (lrow0 + 16 * g)));
                if (pos < kStepCap)
                  steplist[pos] = (int32_t)((((uint32_t)(row0 + 16 * g) >> 4) << 11) |
                                            (uint32_t)(valid << 4) | (uint32_t)(l << 2) |
                                            (uint32_t)e);
                ++pos;
              }
            }
          }
          base += cnt;
        }
        if (lane == 0) {
          for (int pz = base; pz < kStepCap && pz % GS; ++pz) steplist[pz] = 0;
          steps_sh = base;
        }
      }
      __syncthreads();
      const int G = (steps_sh + GS - 1) / GS * GS;  // groups, padded to whole steps
      if (G <= kStepCap) {
        use_sl = true;
        LS = G / GS;
      }
    }
  }
  // descriptors of step u as read from LDS, and the same made wave-uniform
  auto step_words = [&](int u) -> CodeT {
    CodeT d{};
    if constexpr (SL) {
#pragma unroll
      for (int i = 0; i < GS; ++i) d.g[i] = (uint32_t)steplist[u * GS + i];
    }
    return d;
  };
  auto uniform_code = [&](CodeT d) -> CodeT {
    if constexpr (SL) {
#pragma unroll
      for (int i = 0; i < GS; ++i) d.g[i] = (uint32_t)wave_uniform((int)d.g[i]);
    }
    return d;
  };
  auto step_code = [&](int u) -> CodeT { return uniform_code(step_words(u)); };

  LoadPlan<C::LPW> lp;
  make_plan<D, C::NW, C::LPW, SL>(lp, w, lane, p.ksn, p.vsn);
  // Stage byte offsets: step u uses K stage u % 2 and V stage u % 2.
  const uint32_t wave_lds =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem + (uint32_t)w * 1024;
  constexpr int kso[2] = {0, T::BYTES};
  constexpr int vso[2] = {C::VOFF, C::VOFF + T::BYTES};
  // (with the split plan of SL, a step's GS 16-row groups of its block)
  auto issue_k = [&](auto so_c, int c, int part) {
    const int j0 = first_key(c, part), vk = valid_keys(c, part);
    const uint16_t* base = (PYR && c >= p.rb1) ? kpbase : kbase;
    if constexpr (SL) {
      GroupRsrc rs;
#pragma unroll
      for (int g = 0; g < GS; ++g)
        rs.set(g, rows_rsrc(base, p.ksn, j0 + 16 * g, max(0, min(16, vk - 16 * g))));
      issue_rows_grouped<C::NW, C::LPW, T::RPI, decltype(so_c)::value>(lp.k, rs, w, wave_lds);
    } else {
      issue_rows<C::NW, C::LPW, decltype(so_c)::value>(lp.k, rows_rsrc(base, p.ksn, j0, vk),
                                                       wave_lds);
    }
  };
  auto issue_v = [&](auto so_c, int c, int part) {
    const int j0 = first_key(c, part), vk = valid_keys(c, part);
    const uint16_t* base = (PYR && c >= p.rb1) ? vpbase : vbase;
    if constexpr (SL) {
      GroupRsrc rs;
#pragma unroll
      for (int g = 0; g < GS; ++g)
        rs.set(g, rows_rsrc(base, p.vsn, j0 + 16 * g, max(0, min(16, vk - 16 * g))));
      issue_rows_grouped<C::NW, C::LPW, T::RPI, decltype(so_c)::value>(lp.v, rs, w, wave_lds);
    } else {
      issue_rows<C::NW, C::LPW, decltype(so_c)::value>(lp.v, rows_rsrc(base, p.vsn, j0, vk),
                                                       wave_lds);
    }
  };
  // a step of the pyramid step list: each group from its own level's tensor
  auto issue_kd = [&](auto so_c, const CodeT& d) {
    if constexpr (SL) {
      GroupRsrc rs;
#pragma unroll
      for (int g = 0; g < GS; ++g)
        rs.set(g, rows_rsrc(g_level(d.g[g]) ? kpbase : kbase, p.ksn, g_row0(d.g[g]),
                            g_valid(d.g[g])));
      issue_rows_grouped<C::NW, C::LPW, T::RPI, decltype(so_c)::value>(lp.k, rs, w, wave_lds);
    }
  };
  auto issue_vd = [&](auto so_c, const CodeT& d) {
    if constexpr (SL) {
      GroupRsrc rs;
#pragma unroll
      for (int g = 0; g < GS; ++g)
        rs.set(g, rows_rsrc(g_level(d.g[g]) ? vpbase : vbase, p.vsn, g_row0(d.g[g]),
                            g_valid(d.g[g])));
      issue_rows_grouped<C::NW, C::LPW, T::RPI, decltype(so_c)::value>(lp.v, rs, w, wave_lds);
    }
  };
  using K0 = std::integral_constant<uint32_t, kso[0]>;
  using K1 = std::integral_constant<uint32_t, kso[1]>;
  using V0 = std::integral_constant<uint32_t, vso[0]>;
  using V1 = std::integral_constant<uint32_t, vso[1]>;
  constexpr int PART1 = NSUB == 2 ? 1 : 0;  // part of step 1 (and of every odd step)

  // Key blocks of steps it, it+1, it+2 (rolling), their eighth masks and,
  // for step lists, their parts; with the pyramid step list in use, c0..c2
  // hold the steps' descriptors instead.
  CodeT c0 = 0, c1 = 0, c2 = 0;
  int q0 = QF, q1 = QF, q2 = QF;
  int r0 = 0, r1 = PART1, r2 = 0;
  if (SL && use_sl) {
    if (LS > 0) {
      c0 = step_code(0);
      issue_kd(K0{}, c0);
      issue_vd(V0{}, c0);
    }
    if (LS > 1) {
      c1 = step_code(1);
      issue_kd(K1{}, c1);
    }
    if (LS > 2) c2 = step_code(2);
  } else {
    if (LS > 0) {
      c0 = block_of(0);
      q0 = eighths_of(0);
      issue_k(K0{}, c0, r0);
      issue_v(V0{}, c0, r0);
    }
    if (LS > 1) {
      c1 = block_of(1);
      q1 = eighths_of(1);
      issue_k(K1{}, c1, r1);
    }
    if (LS > 2) {
      c2 = block_of(2);
      q2 = eighths_of(2);
    }
  }

  // Q rows of this wave as MFMA B operands (k-slice hh*8..+7 of each 16-step).
  const int64_t qrow = a * BQ + w * 32 + n;
  const bool qvalid = qrow < p.N;
  bf16x8 qf[C::KS];
  {
    const uint16_t* qp = p.q + b * p.qsb + (qvalid ? qrow : 0) * p.qsn + h * p.qsh + hh * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 raw = *(const u32x4*)(qp + ks * 16);
      if (!qvalid) raw = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // LDS read offsets (bytes within a tile). K operand of key block kb at
  // k-step ks: row kb*32 + n, logical chunk 2*ks + hh. V^T operand of d block
  // db: lane group g = lane/16 reads rows 4*(g/2) + (lane%16)/4 (+ key base)
  // and element column 32*db + 16*(g%2) + 4*(lane%4).
  uint32_t koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = n * T::RB + (((2 * ks + hh) ^ T::fK(n)) * 16);
  uint32_t voff[C::DB];
  {
    const int g = lane >> 4, s = lane & 15, kr = s >> 2, j = s & 3;
    const int r = 4 * (g >> 1) + kr;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int colb = 2 * (32 * db + 16 * (g & 1) + 4 * j);
      voff[db] = r * T::RB + (((colb >> 4) ^ T::fV(r)) * 16) + (colb & 15);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_use = -INFINITY;   // exponent base of p and l (log2 units)
  float m_true = -INFINITY;  // running row max (log2 units), for the tile gaps
  float m_blk = -INFINITY;   // row max of the current key block's steps so far
  // Gaps of up to 64 consecutive list entries, lane j holding entry gbatch + j,
  // folded into tile_gap with one 64-lane atomic per batch.
  float gbuf = -INFINITY;
  int gbatch = 0;
  auto flush_gaps = [&](int count) {
    if (lane < count) atomic_max_float(p.tile_gap + gbase + e0 + gbatch + lane, gbuf);
    gbuf = -INFINITY;
  };
  float l_lane = 0.f;        // this lane half's share of the row sum

  // ---- pipeline pieces
  // Scores of one K stage: KB 32-key blocks.
  auto scores = [&](const char* kt, f32x16(&sacc)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 av = *(const bf16x8*)(kt + koff[ks] + kb * 32 * T::RB);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
  };
  // Row max of a step's scores in log2 units. When `masked`, keys at or
  // beyond jv (only the last key block can be ragged) are set to -inf first,
  // which also makes their probabilities 0. A step with no valid key (second
  // half of a short last block) has max -inf.
  // Keys at or beyond jv, and keys in eighths outside qm (pyramid lists),
  // are set to -inf: they take no part in the max and get probability 0.
  auto mask_keys = [&](f32x16(&sacc)[KB], int jv, int qm) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (key_of(kb, j, hh) >= jv || !((qm >> (4 * kb + j / 4)) & 1))
          sacc[kb][j] = -INFINITY;
  };
  // The same for the GS 16-row groups of a pyramid step: valid rows jv[g]
  // of group g, eighth bits qm.
  auto mask_keys_grouped = [&](f32x16(&sacc)[KB], const int (&jv)[GS], int qm) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = key_of(kb, j, hh), g = 2 * kb + (j >= 8 ? 1 : 0);
        if (key - 16 * g >= jv[g] || !((qm >> (4 * kb + j / 4)) & 1)) sacc[kb][j] = -INFINITY;
      }
  };
  auto tile_max = [&](f32x16(&sacc)[KB], bool masked, int jv, int qm) -> float {
    if (masked) mask_keys(sacc, jv, qm);
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) mloc = vmax(vmax(mloc, sacc[kb][j]), sacc[kb][j + 1]);
    mloc = vmax(mloc, other_half(mloc));
    return mloc * p.sl2;
  };
  // Row max (log2 units) of a pyramid step whose group g has level lv[g]: a
  // key of level l scores + l.
  auto tile_max_grouped = [&](f32x16(&sacc)[KB], bool masked, const int (&jv)[GS], int qm,
                              const float (&lv)[GS]) -> float {
    if (masked) mask_keys_grouped(sacc, jv, qm);
    float mg[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) mg[g] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const int g = 2 * kb + (j >= 8 ? 1 : 0);
        mg[g] = vmax(vmax(mg[g], sacc[kb][j]), sacc[kb][j + 1]);
      }
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < GS; ++g) m = vmax(m, fmaf(mg[g], p.sl2, lv[g]));
    return vmax(m, other_half(m));
  };
  // Tile gap (once the key block's last step is in) and exponent-base update
  // for a step whose row max is m_loc2. O must already hold every earlier
  // step when this runs (it may be rescaled).
  auto apply_max = [&](float m_loc2, int u, int part) {
    if (GAP) {
      m_blk = part == 0 ? m_loc2 : fmaxf(m_blk, m_loc2);
      if (part == NSUB - 1) {
        // lanes n and n + 32 hold the same row, so lanes 0..31 cover the wave
        const float g = max_lanes32(qvalid ? m_blk - m_true : -INFINITY);
        const int ie = u / NSUB;
        if (lane == (ie & 63)) gbuf = g;
        if ((ie & 63) == 63) {
          flush_gaps(64);
          gbatch += 64;
        }
        m_true = fmaxf(m_true, m_blk);
      }
    }
    if (__builtin_amdgcn_ballot_w64(m_loc2 > m_use + kRescaleSlack)) {
      const float m_new = fmaxf(m_use, m_loc2);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    }
  };
  // p = 2^(s*scale*log2e + bias - m) rounded to bf16, and its row sum, with
  // bias[2 kb + half] on values 8 half .. 8 half + 7 of key block kb (the
  // groups of a pyramid step; all equal elsewhere). Masked keys hold -inf
  // and give 0 (sl2 > 0 always, see launch_attn_bf16).
  auto probs = [&](const f32x16(&sacc)[KB], bf16x8(&pb)[KB][2], const float (&bias)[GS]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x8 pv;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          pv[t] = __builtin_amdgcn_exp2f(
              fmaf(sacc[kb][half * 8 + t], p.sl2, bias[2 * kb + half] - m_use));
        pb[kb][half] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
        for (int t = 0; t < 8; t += 2)
          l_lane = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[kb][half][t], pb[kb][half][t + 1]},
                                                   bf16x2{(__bf16)1.0f, (__bf16)1.0f}, l_lane,
                                                   false);
      }
    }
  };
  // O^T += V^T P^T over one V stage. For the 16-key step (kb, half) the B
  // operand is pb[kb][half]; element t of lane half hh is key
  // kb*32 + 16*half + 8*(t/4) + 4*hh + t%4, which two transpose reads of the
  // V tile deliver in that order.
  auto accumulate = [&](const char* vt, const bf16x8(&pb)[KB][2]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kofs = (kb * 32 + 16 * half) * T::RB;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const i16x4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db] + kofs));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vt + voff[db] + kofs + 8 * T::RB));
          oacc[db] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(lo, hi), pb[kb][half], oacc[db], 0, 0, 0);
        }
      }
    }
  };

  // V(j+1) and K(j+2) are issued right after the barrier of step j, into
  // stages last read before that barrier, and waited for at the start of
  // step j+1.
  f32x16 sA[KB], sB[KB];
  // Per-step quantities from a block (and part), or with LSL from a step
  // code; glev / gvalid per 16-row group g of a pyramid step (SL kernels).
  auto lev = [&](auto, CodeT c) -> int { return level_of((int)c); };
  auto vkeys = [&](auto, CodeT c, int part) -> int { return valid_keys((int)c, part); };
  auto glev = [&](auto lsl_c, const CodeT& c, int g) -> int {
    if constexpr (decltype(lsl_c)::value) return g_level(code_word(c, g));
    else return level_of((int)c);
  };
  auto gvalid = [&](auto lsl_c, const CodeT& c, int part, int g) -> int {
    if constexpr (decltype(lsl_c)::value) {
      return g_valid(code_word(c, g));
    } else {
      const int vk = valid_keys((int)c, part);
      return max(0, min(16, vk - 16 * g));
    }
  };
  auto qmask = [&](auto lsl_c, const CodeT& c, int q) -> int {
    if constexpr (decltype(lsl_c)::value) {
      int m = 0;
#pragma unroll
      for (int g = 0; g < GS; ++g) m |= g_eighths(code_word(c, g)) << (2 * g);
      return m;
    } else {
      return q;
    }
  };
  // valid rows and levels of the groups of a pyramid step, and whether any
  // of its keys must be masked
  auto group_info = [&](auto lsl_c, const CodeT& c, int part, int qm, int (&jv)[GS],
                        float (&lv)[GS]) -> bool {
    bool masked = qm != QF;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      jv[g] = gvalid(lsl_c, c, part, g);
      lv[g] = (float)glev(lsl_c, c, g);
      masked = masked || jv[g] < 16;
    }
    return masked;
  };
  auto first_scores = [&](auto lsl_c) __attribute__((always_inline)) {
    if (LS > 0) {
      // prologue: scores and max of step 0
      if (LS > 1) wait_vmcnt<2 * C::LPW>();  // K0 done; V0, K1 may fly
      else wait_vmcnt<C::LPW>();
      barrier();
      scores(smem + kso[0], sA);
      if constexpr (SL) {
        int jv[GS];
        float lv[GS];
        const int qm0 = qmask(lsl_c, c0, q0);
        const bool masked = group_info(lsl_c, c0, r0, qm0, jv, lv);
        apply_max(tile_max_grouped(sA, masked, jv, qm0, lv), 0, 0);
      } else {
        const int jv = vkeys(lsl_c, c0, r0), qm0 = qmask(lsl_c, c0, q0);
        apply_max(tile_max(sA, jv < SUB || qm0 != QF, jv, qm0) + (float)lev(lsl_c, c0), 0, 0);
      }
    }
  };
  if constexpr (!SL) first_scores(std::false_type{});
  // One pipeline step: step `it` has scores in `cur`; when `has_next`, the
  // scores of step it+1 are computed into `nxt` meanwhile. Every LDS read of
  // the previous step has completed before the barrier (lgkmcnt(0)), so the
  // stages it read may be refilled right after it. `par` = it % 2.
  // With LSL (pyramid step list in use) the descriptor of step it+3 is read
  // from LDS at the top of step it, at a clamped index so that the read is
  // unconditional, and decoded at the end of the step, when the step's own
  // LDS waits have covered it. The list path instead reads list entries with
  // scalar loads, which lgkmcnt counts together with LDS reads.
  auto step = [&](int it, f32x16(&cur)[KB], f32x16(&nxt)[KB], bool has_next, auto par_c,
                  auto lsl_c) __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;
    constexpr bool LSL = decltype(lsl_c)::value;
    constexpr int part0 = NSUB == 2 ? par : 0, part1 = NSUB == 2 ? 1 - par : 0;
    const int pk = SL ? r2 : part0, pv = SL ? r1 : part1;  // parts of steps it+2, it+1
    using KS_ = std::integral_constant<uint32_t, kso[par]>;
    using VS_ = std::integral_constant<uint32_t, vso[1 - par]>;
    wait_vmcnt<0>();  // V(it) and K(it+1) done
    wait_lds();
    barrier();
    if constexpr (LSL) {
      if (it + 1 < LS) issue_vd(VS_{}, c1);
      if (it + 2 < LS) issue_kd(KS_{}, c2);
    } else {
      if (it + 1 < LS) issue_v(VS_{}, c1, pv);
      if (it + 2 < LS) issue_k(KS_{}, c2, pk);
    }
    CodeT code3{};
    if constexpr (LSL) code3 = step_words(min(it + 3, kStepCap / GS - 1));
    bf16x8 pb[KB][2];
    if (has_next) {
      const char* kt = smem + kso[1 - par];
      const char* vt = smem + vso[par];
      // K fragment of score MFMA i (k-step i / KB, key block i % KB) and V^T
      // fragment of P V MFMA i (key block, 16-key half, d block).
      auto kread = [&](int i) -> bf16x8 {
        return *(const bf16x8*)(kt + koff[i / KB] + (i % KB) * 32 * T::RB);
      };
      auto vread = [&](int i) -> bf16x8 {
        const int kb = i / (2 * C::DB), half = (i / C::DB) % 2, db = i % C::DB;
        const int kofs = (kb * 32 + 16 * half) * T::RB;
        const i16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db] + kofs));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + voff[db] + kofs + 8 * T::RB));
        return join(lo, hi);
      };
      bf16x8 kbuf[kPfK + 1];
      bf16x8 vbuf[kPfV + 1];
      uint32_t pw[KB][2][4];  // probabilities as packed bf16 pairs
      // Phase A: slot i issues score MFMA i of step it+1 and forms EPS
      // probabilities of step it (exp2, bf16 pair, row-sum dot).
      // a pooled key stands for 2^level tokens: its weight 2^level p, i.e.
      // + level in the log2 exponent
      float nm[GS];  // bias - m_use of each group of step it
#pragma unroll
      for (int g = 0; g < GS; ++g)
        nm[g] = (float)(SL ? glev(lsl_c, c0, g) : lev(lsl_c, c0)) - m_use;
#pragma unroll
      for (int i = 0; i < kPfK; ++i) kbuf[i] = kread(i);
      // the first fragment reads go out together, ahead of the first MFMA
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C::NA; ++i) {
        if (i + kPfK < C::NA) kbuf[(i + kPfK) % (kPfK + 1)] = kread(i + kPfK);
        if (i >= C::NA - kPfV) vbuf[i - (C::NA - kPfV)] = vread(i - (C::NA - kPfV));
        const int ks = i / KB, kb = i % KB;
        nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbuf[i % (kPfK + 1)], qf[ks],
                                                          ks == 0 ? f32x16{} : nxt[kb], 0, 0, 0);
#pragma unroll
        for (int e2 = 0; e2 < C::EPS; e2 += 2) {
          const int e = i * C::EPS + e2, kb2 = e / 16, j = e % 16;
          const float neg_m = nm[2 * kb2 + (j >= 8 ? 1 : 0)];  // j, j + 1 in one group
          const float x0 = __builtin_amdgcn_exp2f(fmaf(cur[kb2][j], p.sl2, neg_m));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(cur[kb2][j + 1], p.sl2, neg_m));
          const bf16x2 pr = __builtin_convertvector((f32x2{x0, x1}), bf16x2);
          pw[kb2][j / 8][(j % 8) / 2] = __builtin_bit_cast(uint32_t, pr);
          l_lane = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, l_lane,
                                                   false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          pb[kb][half] = __builtin_bit_cast(
              bf16x8, (u32x4{pw[kb][half][0], pw[kb][half][1], pw[kb][half][2], pw[kb][half][3]}));
          // the probabilities stay in phase A (not sunk past the branch below)
          asm volatile("" ::"v"(pb[kb][half]));
        }
      asm volatile("" ::"v"(l_lane));
      float lv1[GS];  // levels of the groups of step it+1 (SL)
      if constexpr (SL) {
        int jv[GS];
        const int qm1 = qmask(lsl_c, c1, q1);
        if (group_info(lsl_c, c1, pv, qm1, jv, lv1)) mask_keys_grouped(nxt, jv, qm1);
      } else {
        const int jv = vkeys(lsl_c, c1, pv), qm1 = qmask(lsl_c, c1, q1);
        if (jv < SUB || qm1 != QF) mask_keys(nxt, jv, qm1);
      }
      // Phase B: slot i issues P V MFMA i of step it and folds MPS scores of
      // step it+1 into the row max.
      float mloc = -INFINITY;
      float mg[GS];  // per group (SL)
#pragma unroll
      for (int g = 0; g < GS; ++g) mg[g] = -INFINITY;
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
        if (i + kPfV < C::NB) vbuf[(i + kPfV) % (kPfV + 1)] = vread(i + kPfV);
        const int kb = i / (2 * C::DB), half = (i / C::DB) % 2, db = i % C::DB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vbuf[i % (kPfV + 1)], pb[kb][half],
                                                           oacc[db], 0, 0, 0);
#pragma unroll
        for (int e2 = 0; e2 < C::MPS; e2 += 2) {
          const int e = i * C::MPS + e2, kb2 = e / 16, j = e % 16;
          if constexpr (SL) {
            const int g = 2 * kb2 + (j >= 8 ? 1 : 0);
            mg[g] = vmax(vmax(mg[g], nxt[kb2][j]), nxt[kb2][j + 1]);
          } else {
            mloc = vmax(vmax(mloc, nxt[kb2][j]), nxt[kb2][j + 1]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (SL) {
        float m = -INFINITY;
#pragma unroll
        for (int g = 0; g < GS; ++g) m = vmax(m, fmaf(mg[g], p.sl2, lv1[g]));
        m = vmax(m, other_half(m));
        apply_max(m, it + 1, part1);
      } else {
        mloc = vmax(mloc, other_half(mloc));
        apply_max(mloc * p.sl2 + (float)lev(lsl_c, c1), it + 1, part1);
      }
    } else {
      float bias[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) bias[g] = (float)(SL ? glev(lsl_c, c0, g) : lev(lsl_c, c0));
      probs(cur, pb, bias);
      accumulate(smem + vso[par], pb);
    }
    // The list entries of step it+3 are read here, after the last LDS wait
    // of the step: scalar loads count in lgkmcnt and may complete out of
    // order, so one in flight would turn every LDS wait above into a wait for
    // everything.
    CodeT c3 = 0;
    int q3 = QF, r3 = 0;
    if constexpr (LSL) {
      const CodeT code = uniform_code(code3);
      if (it + 3 < LS) c3 = code;
    } else {
      c3 = it + 3 < LS ? block_of(it + 3) : 0;
      q3 = (PYR && it + 3 < LS) ? eighths_of(it + 3) : QF;
      r3 = (SL && it + 3 < LS) ? part_of(it + 3) : 0;
    }
    c0 = c1;
    c1 = c2;
    c2 = c3;
    q0 = q1;
    q1 = q2;
    q2 = q3;
    r0 = r1;
    r1 = r2;
    r2 = r3;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // the whole pipeline, as its own loop for each way of reading the list
  auto run = [&](auto lsl_c) __attribute__((always_inline)) {
    first_scores(lsl_c);
    int it = 0;
    for (; it + 2 < LS; it += 2) {
      step(it, sA, sB, true, P0{}, lsl_c);
      step(it + 1, sB, sA, true, P1{}, lsl_c);
    }
    if (it + 1 < LS) {
      step(it, sA, sB, true, P0{}, lsl_c);
      step(it + 1, sB, sA, false, P1{}, lsl_c);
    } else if (it < LS) {
      step(it, sA, sB, false, P0{}, lsl_c);
    }
  };
  if constexpr (SL) {
    if (use_sl)
      run(std::true_type{});
    else
      run(std::false_type{});
  } else {
    using F = std::false_type;
    int it = 0;
    for (; it + 2 < LS; it += 2) {
      step(it, sA, sB, true, P0{}, F{});
      step(it + 1, sB, sA, true, P1{}, F{});
    }
    if (it + 1 < LS) {
      step(it, sA, sB, true, P0{}, F{});
      step(it + 1, sB, sA, false, P1{}, F{});
    } else if (it < LS) {
      step(it, sA, sB, false, P0{}, F{});
    }
  }

  if (GAP && L > gbatch) flush_gaps(L - gbatch);
  // ---- epilogue: O = O^T / l through LDS for coalesced 16-byte stores.
  const float l_tot = l_lane + other_half(l_lane);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  wait_vmcnt<0>();
  wait_lds();
  barrier();  // every wave is done reading the stages
  uint16_t* Os = (uint16_t*)smem;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 tmp;
#pragma unroll
      for (int t = 0; t < 4; ++t) tmp[t] = oacc[db][4 * j4 + t] * inv;
      const bf16x4 ov = __builtin_convertvector(tmp, bf16x4);
      *(bf16x4*)(Os + (w * 32 + n) * C::OLD + db * 32 + 8 * j4 + 4 * hh) = ov;
    }
  }
  wait_lds();
  barrier();
  uint16_t* obase = p.o + b * p.osb + h * p.osh;
#pragma unroll
  for (int i = 0; i < BQ * (D / 8) / C::NT; ++i) {
    const int id = tid + i * C::NT;
    const int r = id / (D / 8), c8 = id % (D / 8);
    const int64_t orow = a * BQ + r;
    if (orow < p.N)
      *(u32x4*)(obase + orow * p.osn + c8 * 8) = *(const u32x4*)(Os + r * C::OLD + c8 * 8);
  }
  if (p.lse && hh == 0 && qvalid)
    p.lse[bh * p.N + qrow] = l_tot > 0.f ? (m_use + log2f(l_tot)) * kLn2 : -INFINITY;
}

// tile_gap[0 .. count) = -inf, count = row_ptr[R] * mult (read on the device).
__global__ void gap_init_kernel(float* gap, const int32_t* row_ptr, int64_t R, int64_t mult) {
  const int64_t count = (int64_t)row_ptr[R] * mult;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    gap[i] = -INFINITY;
}

template <int D, int BQ>
hipError_t launch(const Geom& g, const Bf16Params& p, hipStream_t st) {
  // Two-wave workgroups step through half key blocks (32 KiB of LDS, four
  // workgroups per CU); four-wave ones through whole blocks.
  constexpr int SUB = BQ == 64 ? 32 : 64;
  using C = Cfg<D, BQ, SUB>;
  const int64_t rows = (int64_t)g.B * g.H * (p.U ? (int64_t)g.T * p.U : g.nQ);
  if (p.tile_gap) {
    // per-wave gaps are folded in with an atomic max starting from -inf
    const int64_t R = p.lists_shared ? g.nQ : (int64_t)g.B * g.H * g.nQ;
    const int64_t mult = p.lists_shared ? (int64_t)g.B * g.H : 1;
    hipLaunchKernelGGL(gap_init_kernel, dim3(1024), dim3(256), 0, st, p.tile_gap, p.row_ptr, R,
                       mult);
    hipLaunchKernelGGL((attn_bf16_kernel<D, BQ, SUB, true, false>), dim3((unsigned)rows),
                       dim3(C::NT), 0, st, p);
  } else if (p.kv_eighths) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, BQ, SUB, false, true>), dim3((unsigned)rows),
                       dim3(C::NT), 0, st, p);
  } else {
    hipLaunchKernelGGL((attn_bf16_kernel<D, BQ, SUB, false, false>), dim3((unsigned)rows),
                       dim3(C::NT), 0, st, p);
  }
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
  p.kp = (const uint16_t*)a.kp.ptr;
  p.vp = (const uint16_t*)a.vp.ptr;
  p.kpsb = a.kp.sb; p.kpsh = a.kp.sh;
  p.vpsb = a.vp.sb; p.vpsh = a.vp.sh;
  p.kv_eighths = a.kv_eighths;
  p.rb1 = (int32_t)a.pyr_rb[1];
  p.rb2 = (int32_t)a.pyr_rb[2];
  p.rb3 = (int32_t)a.pyr_rb[3];
  p.rb4 = (int32_t)a.pyr_rb[4];
  // Scores enter every exponent as s * sl2. A zero scale is taken as the
  // smallest normal float instead: finite scores then still contribute
  // 2^(~0) (off by far less than bf16 rounding) while masked keys (-inf)
  // keep probability 0 instead of turning into NaN.
  p.sl2 = fmaxf(a.scale * kLog2e, 1.17549435e-38f);
  p.N = g.N; p.nQ = g.nQ; p.nK = g.nK; p.H = g.H;
  p.T = g.T; p.F = g.F; p.U = (int32_t)((g.F + g.Bq - 1) / g.Bq);
  if ((int64_t)g.T * p.U > g.nQ + g.nQ / 4) p.U = 0;  // tiny frames: plain row order
  // Per-head lists come from content-based masks (pooled, pyramid, skip
  // carry), where neighbouring row blocks of a head pick similar key blocks:
  // plain row order shares their tiles in L2. Shared lists (the radial mask)
  // band by frame distance, so row blocks at the same in-frame position of
  // different frames are the ones that visit the same key frames.
  if (a.row_ptr && !a.lists_shared) p.U = 0;
  if (g.D == 64) return g.Bq == 64 ? launch<64, 64>(g, p, st) : launch<64, 128>(g, p, st);
  return g.Bq == 64 ? launch<128, 64>(g, p, st) : launch<128, 128>(g, p, st);
}

}  // namespace bsa
