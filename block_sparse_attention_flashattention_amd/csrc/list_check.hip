// list_check.hip -- debug validation of block lists (CSR row pointers and
// key-block indices), on the host or on the device.
//
// A list row must hold each kept key block once, inside [0, n_blocks)
// ([Lite] LiteAttention summary page, sections 三 and 六: the forward walks
// only the listed tiles, so a malformed list would load tiles outside the key
// range or count a tile twice). The rules, in the order they are reported:
//   1  row_ptr[0] != 0
//   2  row_ptr[r+1] < row_ptr[r]
//   3  row_ptr[r+1] > kv_len
//   4  an entry outside [0, n_blocks)
//   5  an entry repeated within its row
//   6  a row not strictly ascending (checked only when ascending order is
//      required)
// The first failing row (lowest index, then lowest rule) is reported. The
// device check never reads outside row_ptr[0..R] and kv_idx[0..kv_len).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kBitmapKeys = 65536;  // LDS bitmap of 8 KiB for the repeat test

// (row << 3) | rule of the first failure; all ones = none. Written by the
// kernels below only, read back by the host through its symbol.
__device__ unsigned long long g_first_bad;

__device__ inline void report(int64_t row, int rule) {
  atomicMin(&g_first_bad, ((unsigned long long)row << 3) | (unsigned long long)rule);
}

__global__ void reset_kernel() { g_first_bad = ~0ull; }

// Row pointers: one thread per row. kv_len < 0: no bound on row_ptr[R].
__global__ void row_ptr_kernel(const int32_t* row_ptr, int64_t R, int64_t kv_len) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && row_ptr[0] != 0) report(0, 1);
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < R;
       r += (int64_t)gridDim.x * blockDim.x) {
    if (row_ptr[r + 1] < row_ptr[r]) report(r, 2);
    if (kv_len >= 0 && (int64_t)row_ptr[r + 1] > kv_len) report(r, 3);
  }
}

// Entries: one workgroup per row. kv_len < 0 takes row_ptr[R] as the length.
__global__ void entries_kernel(const int32_t* row_ptr, const int32_t* kv, int64_t R,
                               int64_t kv_len, int64_t n_blocks, int ascending) {
  __shared__ uint32_t seen[kBitmapKeys / 32];
  const int64_t len = kv_len < 0 ? (int64_t)row_ptr[R] : kv_len;
  const bool bitmap = !ascending && n_blocks <= kBitmapKeys;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    // clamp to the readable range; rows whose pointers are out of order are
    // reported by row_ptr_kernel
    const int64_t e0 = min(max((int64_t)row_ptr[r], (int64_t)0), len);
    const int64_t e1 = min(max((int64_t)row_ptr[r + 1], e0), len);
    if (bitmap) {
      for (int64_t i = threadIdx.x; i < (n_blocks + 31) / 32; i += blockDim.x) seen[i] = 0;
      __syncthreads();
    }
    for (int64_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
      const int32_t c = kv[e];
      if (c < 0 || c >= n_blocks) {
        report(r, 4);
        continue;
      }
      if (ascending) {
        if (e + 1 < e1 && kv[e + 1] <= c) report(r, kv[e + 1] == c ? 5 : 6);
      } else if (bitmap) {
        const uint32_t bit = 1u << (c & 31);
        if (atomicOr(&seen[c >> 5], bit) & bit) report(r, 5);
      } else {
        for (int64_t f = e + 1; f < e1; ++f)
          if (kv[f] == c) report(r, 5);
      }
    }
    if (bitmap) __syncthreads();  // the bitmap is cleared again for the next row
  }
}

}  // namespace

int64_t check_lists_host(const int32_t* row_ptr, const int32_t* kv, int64_t R, int64_t kv_len,
                         int64_t n_blocks, bool ascending, int* rule) {
  if (row_ptr[0] != 0) {
    *rule = 1;
    return 0;
  }
  std::vector<uint8_t> seen(ascending ? 0 : (size_t)n_blocks, 0);
  for (int64_t r = 0; r < R; ++r) {
    if (row_ptr[r + 1] < row_ptr[r]) {
      *rule = 2;
      return r;
    }
    if ((int64_t)row_ptr[r + 1] > kv_len) {
      *rule = 3;
      return r;
    }
    // the readable range only, as on the device
    const int64_t e0 = std::min(std::max((int64_t)row_ptr[r], (int64_t)0), kv_len);
    const int64_t e1 = std::min(std::max((int64_t)row_ptr[r + 1], e0), kv_len);
    int bad = 0;
    for (int64_t e = e0; e < e1; ++e) {
      const int32_t c = kv[e];
      int rl = 0;
      if (c < 0 || c >= n_blocks) rl = 4;
      else if (ascending && e + 1 < e1 && kv[e + 1] <= c) rl = kv[e + 1] == c ? 5 : 6;
      else if (!ascending && seen[c]) rl = 5;
      if (!ascending && c >= 0 && c < n_blocks) seen[c] = 1;
      if (rl && (!bad || rl < bad)) bad = rl;
    }
    if (!ascending)
      for (int64_t e = e0; e < e1; ++e)
        if (kv[e] >= 0 && kv[e] < n_blocks) seen[kv[e]] = 0;
    if (bad) {
      *rule = bad;
      return r;
    }
  }
  *rule = 0;
  return -1;
}

hipError_t check_lists_device(const int32_t* row_ptr, const int32_t* kv, int64_t R,
                              int64_t kv_len, int64_t n_blocks, bool ascending, int* rule,
                              int64_t* row, hipStream_t st) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, st);
  const int64_t nb1 = std::min<int64_t>((R + kThreads - 1) / kThreads, 4096);
  const unsigned g1 = (unsigned)std::max<int64_t>(1, nb1);
  const unsigned g2 = (unsigned)std::max<int64_t>(1, std::min<int64_t>(R, 8192));
  hipLaunchKernelGGL(row_ptr_kernel, dim3(g1), dim3(kThreads), 0, st, row_ptr, R, kv_len);
  hipLaunchKernelGGL(entries_kernel, dim3(g2), dim3(kThreads), 0, st, row_ptr, kv, R, kv_len,
                     n_blocks, ascending ? 1 : 0);
  hipError_t e = hipGetLastError();
  unsigned long long first = ~0ull;
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(&first, HIP_SYMBOL(g_first_bad), sizeof first, 0,
                                 hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *rule = first == ~0ull ? 0 : (int)(first & 7);
  *row = first == ~0ull ? -1 : (int64_t)(first >> 3);
  return hipSuccess;
}

}  // namespace bsa
