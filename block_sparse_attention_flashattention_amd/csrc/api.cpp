// api.cpp -- the C ABI of libbsa (declared in include/bsa.h): host-side
// argument validation, then kernel launches on the caller's stream.
// Validation touches no GPU state, so every error path is testable on a host
// without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsa.h"
#include "bsa_internal.h"

namespace bsa {
int pooled_max_blocks();
}

namespace {

thread_local char g_err[512];

bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bsa_status ok() {
  g_err[0] = 0;
  return BSA_OK;
}

bsa_status device(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kI32Max = 2147483647;

bsa_status make_geom(const bsa_shape* s, bsa::Geom* g) {
  if (!s) return fail(BSA_ERR_INVALID, "shape is NULL");
  if (s->batch < 0 || s->heads < 0 || s->frames < 0 || s->height < 0 || s->width < 0)
    return fail(BSA_ERR_INVALID, "negative batch/heads/frames/height/width");
  if (s->head_dim <= 0 || s->block_q <= 0 || s->block_k <= 0)
    return fail(BSA_ERR_INVALID, "head_dim and block sizes must be positive");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", s->head_dim);
  if (s->block_q != 64 && s->block_q != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block_q %d not in {64, 128}", s->block_q);
  if (s->block_k != 64) return fail(BSA_ERR_UNSUPPORTED, "block_k %d is not 64", s->block_k);
  const int64_t F = (int64_t)s->height * s->width;
  const int64_t N = F * s->frames;
  if (N > kI32Max) return fail(BSA_ERR_INVALID, "N = %lld tokens does not fit in int32", (long long)N);
  g->B = s->batch; g->H = s->heads; g->D = s->head_dim;
  g->T = s->frames; g->Hs = s->height; g->Ws = s->width;
  g->Bq = s->block_q; g->Bk = s->block_k;
  g->N = N; g->F = F;
  g->nQ = (N + g->Bq - 1) / g->Bq;
  g->nK = (N + g->Bk - 1) / g->Bk;
  if ((int64_t)g->B * g->H * g->nQ > kI32Max)
    return fail(BSA_ERR_INVALID, "batch*heads*row blocks does not fit in int32");
  return BSA_OK;
}

bool empty(const bsa::Geom& g) { return g.N == 0 || g.B == 0 || g.H == 0; }

bsa_status check_tensor(const char* name, const bsa_tensor& t, int elem_bytes) {
  if (!t.ptr) return fail(BSA_ERR_INVALID, "%s.ptr is NULL", name);
  if ((uintptr_t)t.ptr % 16) return fail(BSA_ERR_INVALID, "%s.ptr is not 16-byte aligned", name);
  const int64_t q = 16 / elem_bytes;
  if (t.stride_b < 0 || t.stride_n < 0 || t.stride_h < 0)
    return fail(BSA_ERR_INVALID, "%s has a negative stride", name);
  if (t.stride_b % q || t.stride_n % q || t.stride_h % q)
    return fail(BSA_ERR_INVALID, "%s strides must be multiples of %lld elements", name,
                (long long)q);
  return BSA_OK;
}

bsa::TensorArg arg(const bsa_tensor& t) { return {t.ptr, t.stride_b, t.stride_n, t.stride_h}; }

int elem_bytes(bsa_dtype dt) { return dt == BSA_BF16 ? 2 : 4; }

const char* rule_text(int rule) {
  switch (rule) {
    case 1: return "row_ptr[0] is not 0";
    case 2: return "row_ptr decreases";
    case 3: return "row_ptr beyond kv_len";
    case 4: return "entry outside the key blocks";
    case 5: return "entry repeated in the row";
    case 6: return "row not in ascending order";
  }
  return "?";
}

bsa_status list_result(int64_t row, int rule) {
  if (rule == 0) return ok();
  return fail(BSA_ERR_INVALID, "block lists, row %lld: rule %d (%s)", (long long)row, rule,
              rule_text(rule));
}

// Lists of a consuming call, checked on the device when BSA_CHECK=1.
bsa_status debug_check(const bsa::Geom& g, bool shared, const int32_t* row_ptr,
                       const int32_t* kv_idx, int64_t n_blocks, bool ascending,
                       hipStream_t st) {
  const char* env = getenv("BSA_CHECK");
  if (!env || strcmp(env, "1") != 0 || !row_ptr) return BSA_OK;
  const int64_t R = shared ? g.nQ : (int64_t)g.B * g.H * g.nQ;
  if (R == 0) return BSA_OK;
  int rule = 0;
  int64_t row = -1;
  hipError_t e = bsa::check_lists_device(row_ptr, kv_idx, R, -1, n_blocks, ascending, &rule, &row,
                                         st);
  if (e != hipSuccess) return device(e, "block list check");
  return list_result(row, rule);
}

}  // namespace

extern "C" {

const char* bsa_status_string(bsa_status st) {
  switch (st) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_CAPACITY: return "kv_idx capacity too small";
    case BSA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* bsa_last_error(void) { return g_err; }

bsa_status bsa_build_mask_radial(const bsa_shape* s, int32_t h0, int32_t decay_base,
                                 uint8_t* mask, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (decay_base < 2) return fail(BSA_ERR_INVALID, "decay_base %d < 2", decay_base);
  if (h0 < g.Bk / 2 || h0 >= (1 << 30))
    return fail(BSA_ERR_INVALID, "h0 %d outside [block_k/2, 2^30)", h0);
  if (g.N == 0) return ok();
  if (!mask) return fail(BSA_ERR_INVALID, "mask is NULL");
  return device(bsa::launch_radial_mask(g, h0, decay_base, mask, (hipStream_t)stream),
                "radial mask launch");
}

size_t bsa_pooled_workspace_bytes(const bsa_shape* s) {
  bsa::Geom g;
  if (make_geom(s, &g) != BSA_OK) return 0;
  return bsa::pooled_workspace_bytes(g);
}

}  // extern "C"

namespace {

// Checks shared by the pooled builders: everything but the scratch.
bsa_status check_pooled(const bsa::Geom& g, bsa_dtype dt, const bsa_tensor& q,
                        const bsa_tensor& k, double scale, int32_t mode, double param,
                        const uint8_t* mask) {
  bsa_status st;
  if (dt != BSA_BF16 && dt != BSA_F32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (!isfinite(scale)) return fail(BSA_ERR_INVALID, "scale is not finite");
  if (mode == 0 || mode == 2) {
    if (!(param >= 1.0) || param != floor(param) || param > 2147483647.0)
      return fail(BSA_ERR_INVALID, "top-k needs an integer k >= 1, got %g", param);
  } else if (mode == 1 || mode == 3) {
    if (!(param > 0.0 && param <= 1.0))
      return fail(BSA_ERR_INVALID, "cumulative mass tau_p must be in (0, 1], got %g", param);
  } else {
    return fail(BSA_ERR_INVALID, "mode %d not in {0, 1, 2, 3}", mode);
  }
  if (g.nK > bsa::pooled_max_blocks())
    return fail(BSA_ERR_UNSUPPORTED, "pooled selection supports at most %d key blocks",
                bsa::pooled_max_blocks());
  if (empty(g)) return BSA_OK;
  if ((st = check_tensor("q", q, elem_bytes(dt))) != BSA_OK) return st;
  if ((st = check_tensor("k", k, elem_bytes(dt))) != BSA_OK) return st;
  if (!mask) return fail(BSA_ERR_INVALID, "mask is NULL");
  return BSA_OK;
}

}  // namespace

extern "C" {

bsa_status bsa_build_mask_pooled_noalloc(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                         bsa_tensor k, double scale, int32_t mode, double param,
                                         uint8_t* mask, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if ((st = check_pooled(g, dt, q, k, scale, mode, param, mask)) != BSA_OK) return st;
  if (empty(g)) return ok();
  const size_t need = bsa::pooled_scratch_need(g, mode);
  if (need > bsa::kStaticScratchBytes)
    return fail(BSA_ERR_CAPACITY,
                "mode %d at this shape needs %zu bytes of scratch; the library's static scratch "
                "holds %zu (use bsa_build_mask_pooled with a workspace)",
                mode, need, bsa::kStaticScratchBytes);
  void* ws = nullptr;
  hipError_t e = bsa::static_scratch(&ws);
  if (e != hipSuccess) return device(e, "static scratch lookup");
  return device(bsa::launch_pooled_mask(g, dt == BSA_BF16 ? 0 : 1, arg(q), arg(k), scale, mode,
                                        param, mask, ws, (hipStream_t)stream),
                "pooled mask launch");
}

bsa_status bsa_build_mask_pooled(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                 bsa_tensor k, double scale, int32_t mode, double param,
                                 uint8_t* mask, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if ((st = check_pooled(g, dt, q, k, scale, mode, param, mask)) != BSA_OK) return st;
  if (empty(g)) return ok();
  const size_t need = bsa::pooled_workspace_bytes(g);
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_INVALID, "workspace needs %zu bytes", need);
  if ((uintptr_t)workspace % 256) return fail(BSA_ERR_INVALID, "workspace not 256-byte aligned");
  return device(bsa::launch_pooled_mask(g, dt == BSA_BF16 ? 0 : 1, arg(q), arg(k), scale, mode,
                                        param, mask, workspace, (hipStream_t)stream),
                "pooled mask launch");
}

bsa_status bsa_compact_block_lists(const bsa_shape* s, const uint8_t* mask,
                                   int64_t mask_head_stride, const uint8_t* skip,
                                   int32_t* row_ptr, int32_t* kv_idx, int64_t kv_capacity,
                                   int64_t* nnz_host, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  const bool shared = mask_head_stride == 0 && skip == nullptr;
  if (mask_head_stride != 0 && mask_head_stride < g.nQ * g.nK)
    return fail(BSA_ERR_INVALID, "mask_head_stride must be 0 or >= nQ*nK");
  if (kv_capacity < 0) return fail(BSA_ERR_INVALID, "kv_capacity < 0");
  if (!row_ptr) return fail(BSA_ERR_INVALID, "row_ptr is NULL");
  const int64_t R = shared ? g.nQ : (int64_t)g.B * g.H * g.nQ;
  if (R * g.nK > kI32Max)
    return fail(BSA_ERR_UNSUPPORTED, "list rows x key blocks exceeds int32 list offsets");
  hipStream_t str = (hipStream_t)stream;
  if (R == 0 || g.nK == 0) {
    if (nnz_host) *nnz_host = 0;
    return device(bsa::launch_zero_row_ptr(row_ptr, str), "compaction launch");
  }
  if (!mask) return fail(BSA_ERR_INVALID, "mask is NULL");
  if (!kv_idx && kv_capacity > 0) return fail(BSA_ERR_INVALID, "kv_idx is NULL");
  if (!nnz_host && kv_capacity < R * g.nK)
    return fail(BSA_ERR_CAPACITY,
                "without nnz_host, kv_capacity must cover every tile (%lld)",
                (long long)(R * g.nK));
  const int64_t mhs = mask_head_stride;
  hipError_t e = bsa::launch_compact_count_scan(g, R, mask, mhs, skip, row_ptr, str);
  if (e != hipSuccess) return device(e, "compaction count");
  if (nnz_host) {
    int32_t nnz = 0;
    e = hipMemcpyAsync(&nnz, row_ptr + R, sizeof nnz, hipMemcpyDeviceToHost, str);
    if (e == hipSuccess) e = hipStreamSynchronize(str);
    if (e != hipSuccess) return device(e, "compaction count readback");
    *nnz_host = nnz;
    if (nnz > kv_capacity)
      return fail(BSA_ERR_CAPACITY, "%d kept tiles exceed kv_capacity %lld", nnz,
                  (long long)kv_capacity);
    if (nnz > 0 && !kv_idx) return fail(BSA_ERR_INVALID, "kv_idx is NULL");
  }
  return device(bsa::launch_compact_scatter(g, R, mask, mhs, skip, row_ptr, kv_idx, str),
                "compaction scatter");
}

bsa_status bsa_order_block_lists(const bsa_shape* s, int32_t order, const int32_t* row_ptr,
                                 int32_t lists_shared, const int32_t* kv_in, int32_t* kv_out,
                                 void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (order != 0 && order != 1) return fail(BSA_ERR_INVALID, "order %d not in {0, 1}", order);
  if (lists_shared != 0 && lists_shared != 1)
    return fail(BSA_ERR_INVALID, "lists_shared must be 0 or 1");
  const int64_t R = lists_shared ? g.nQ : (int64_t)g.B * g.H * g.nQ;
  if (R * g.nK > kI32Max)
    return fail(BSA_ERR_UNSUPPORTED, "list rows x key blocks exceeds int32 list offsets");
  if (R == 0 || g.nK == 0) return ok();
  if (!row_ptr || !kv_in || !kv_out)
    return fail(BSA_ERR_INVALID, "row_ptr, kv_in and kv_out are required");
  if (kv_in == kv_out) return fail(BSA_ERR_INVALID, "kv_out must not alias kv_in");
  if ((st = debug_check(g, lists_shared, row_ptr, kv_in, g.nK, true, (hipStream_t)stream)) !=
      BSA_OK)
    return st;
  return device(bsa::launch_order_lists(g, R, order, row_ptr, kv_in, kv_out, (hipStream_t)stream),
                "list order launch");
}

bsa_status bsa_make_token_permutation(const bsa_shape* s, int32_t kind, const int32_t* axes,
                                      int32_t* perm, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (!axes) return fail(BSA_ERR_INVALID, "axes is NULL");
  if (kind == 0) {
    const int32_t a = axes[0], b = axes[1], c = axes[2];
    if (a < 0 || b < 0 || c < 0 || a > 2 || b > 2 || c > 2 || a == b || b == c || a == c)
      return fail(BSA_ERR_INVALID, "axis order (%d, %d, %d) is not a permutation of (0, 1, 2)",
                  a, b, c);
  } else if (kind == 1) {
    if (axes[0] < 1 || axes[1] < 1 || axes[2] < 1)
      return fail(BSA_ERR_INVALID, "box extents (%d, %d, %d) must be >= 1", axes[0], axes[1],
                  axes[2]);
  } else {
    return fail(BSA_ERR_INVALID, "kind %d not in {0, 1}", kind);
  }
  if (g.N == 0) return ok();
  if (!perm) return fail(BSA_ERR_INVALID, "perm is NULL");
  return device(bsa::launch_make_permutation(g, kind, axes, perm, (hipStream_t)stream),
                "permutation launch");
}

bsa_status bsa_permute_tokens(const bsa_shape* s, bsa_dtype dt, const int32_t* perm,
                              int64_t perm_head_stride, int32_t scatter, bsa_tensor in,
                              bsa_tensor out, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (dt != BSA_BF16 && dt != BSA_F32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (scatter != 0 && scatter != 1) return fail(BSA_ERR_INVALID, "scatter must be 0 or 1");
  if (perm_head_stride != 0 && perm_head_stride < g.N)
    return fail(BSA_ERR_INVALID, "perm_head_stride must be 0 or >= N");
  if (empty(g)) return ok();
  if (!perm) return fail(BSA_ERR_INVALID, "perm is NULL");
  const int eb = elem_bytes(dt);
  if ((st = check_tensor("in", in, eb)) != BSA_OK) return st;
  if ((st = check_tensor("out", out, eb)) != BSA_OK) return st;
  if (in.ptr == out.ptr) return fail(BSA_ERR_INVALID, "out must not alias in");
  return device(bsa::launch_permute_tokens(g, eb, perm, perm_head_stride, scatter, arg(in),
                                           arg(out), (hipStream_t)stream),
                "permute launch");
}

// Workspace of bsa_choose_token_orders, each part from a 256-byte boundary:
// the order's permutation, Q and K gathered into it (contiguous [B][N][H][d]),
// the pooled mask, the per-head counts and the pooled builder's scratch.
struct OrderWs {
  size_t perm, qp, kp, mask, counts, pooled, total;
};
static OrderWs order_ws_layout(const bsa::Geom& g, int eb) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  OrderWs w;
  const size_t tok = (size_t)g.B * g.N * g.H * g.D * eb;
  w.perm = 0;
  w.qp = w.perm + up((size_t)g.N * sizeof(int32_t));
  w.kp = w.qp + up(tok);
  w.mask = w.kp + up(tok);
  w.counts = w.mask + up((size_t)g.B * g.H * g.nQ * g.nK);
  w.pooled = w.counts + up((size_t)g.H * 6 * sizeof(unsigned long long));
  w.total = w.pooled + up(bsa::pooled_scratch_need(g, 1));
  return w;
}

size_t bsa_token_orders_workspace_bytes(const bsa_shape* s, bsa_dtype dt) {
  bsa::Geom g;
  if (make_geom(s, &g) != BSA_OK || (dt != BSA_BF16 && dt != BSA_F32)) return 0;
  return order_ws_layout(g, elem_bytes(dt)).total;
}

bsa_status bsa_choose_token_orders(const bsa_shape* s, bsa_dtype dt, bsa_tensor q, bsa_tensor k,
                                   double scale, int32_t mode, double param, int32_t* order_out,
                                   uint64_t* counts_out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (mode != 0 && mode != 1)
    return fail(BSA_ERR_INVALID, "order choice scores per-row selection (mode 0 or 1), got %d",
                mode);
  if (!order_out && !empty(g)) return fail(BSA_ERR_INVALID, "order_out is NULL");
  if ((st = check_pooled(g, dt, q, k, scale, mode, param, (const uint8_t*)order_out)) != BSA_OK)
    return st;
  if (empty(g)) return ok();
  const int eb = elem_bytes(dt);
  const OrderWs L = order_ws_layout(g, eb);
  if (!workspace || workspace_bytes < L.total)
    return fail(BSA_ERR_INVALID, "workspace needs %zu bytes", L.total);
  if ((uintptr_t)workspace % 256) return fail(BSA_ERR_INVALID, "workspace not 256-byte aligned");
  char* base = (char*)workspace;
  int32_t* perm = (int32_t*)(base + L.perm);
  uint8_t* mask = (uint8_t*)(base + L.mask);
  unsigned long long* counts =
      counts_out ? (unsigned long long*)counts_out : (unsigned long long*)(base + L.counts);
  const int64_t sn = (int64_t)g.H * g.D, sb = (int64_t)g.N * sn;
  const bsa::TensorArg qp{base + L.qp, sb, sn, g.D}, kp{base + L.kp, sb, sn, g.D};
  const hipStream_t hs = (hipStream_t)stream;
  static const int32_t kAxes[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2},
                                      {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
  hipError_t e = bsa::launch_zero_counts(counts, (int64_t)g.H * 6, hs);
  for (int o = 0; o < 6 && e == hipSuccess; ++o) {
    e = bsa::launch_make_permutation(g, 0, kAxes[o], perm, hs);
    if (e == hipSuccess) e = bsa::launch_permute_tokens(g, eb, perm, 0, 0, arg(q), qp, hs);
    if (e == hipSuccess) e = bsa::launch_permute_tokens(g, eb, perm, 0, 0, arg(k), kp, hs);
    if (e == hipSuccess)
      e = bsa::launch_pooled_mask(g, dt == BSA_BF16 ? 0 : 1, qp, kp, scale, mode, param, mask,
                                  base + L.pooled, hs);
    if (e == hipSuccess) e = bsa::launch_count_kept(g, o, mask, counts, hs);
  }
  if (e == hipSuccess) e = bsa::launch_choose_order(g.H, counts, order_out, hs);
  return device(e, "token order choice launch");
}

// Level regions of pyramid lists: rb[l] = first augmented key block of level
// l (each level's N >> l pooled rows padded to whole 64-row blocks).
static void pyramid_regions(const bsa::Geom& g, int32_t n_levels, int64_t rb[5]) {
  rb[0] = 0;
  for (int l = 1; l <= 4; ++l)
    rb[l] = l <= n_levels ? rb[l - 1] + (((g.N >> (l - 1)) + g.Bk - 1) / g.Bk) : rb[l - 1];
}

static bsa_status check_levels(const bsa::Geom& g, int32_t n_levels) {
  if (n_levels < 1 || n_levels > 4) return fail(BSA_ERR_INVALID, "n_levels %d not in 1..4", n_levels);
  if (g.N % (int64_t(1) << (n_levels - 1)))
    return fail(BSA_ERR_UNSUPPORTED, "N = %lld is not a multiple of %d (pooling groups)",
                (long long)g.N, 1 << (n_levels - 1));
  return BSA_OK;
}

int64_t bsa_pyramid_rows(const bsa_shape* s, int32_t n_levels) {
  bsa::Geom g;
  if (make_geom(s, &g) != BSA_OK || n_levels < 1 || n_levels > 4) return -1;
  int64_t rb[5];
  pyramid_regions(g, n_levels, rb);
  return (rb[n_levels] - rb[1 < n_levels ? 1 : n_levels]) * g.Bk;
}

bsa_status bsa_build_kv_pyramid(const bsa_shape* s, bsa_dtype dt, int32_t n_levels, bsa_tensor k,
                                bsa_tensor v, bsa_tensor k_pyr, bsa_tensor v_pyr, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (dt != BSA_BF16 && dt != BSA_F32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if ((st = check_levels(g, n_levels)) != BSA_OK) return st;
  if (empty(g) || n_levels == 1) return ok();
  const int eb = elem_bytes(dt);
  if ((st = check_tensor("k", k, eb)) != BSA_OK) return st;
  if ((st = check_tensor("v", v, eb)) != BSA_OK) return st;
  if ((st = check_tensor("k_pyr", k_pyr, eb)) != BSA_OK) return st;
  if ((st = check_tensor("v_pyr", v_pyr, eb)) != BSA_OK) return st;
  int64_t rb[5];
  pyramid_regions(g, n_levels, rb);
  return device(bsa::launch_kv_pyramid(g, eb, n_levels, rb, arg(k), arg(v), arg(k_pyr),
                                       arg(v_pyr), (hipStream_t)stream),
                "key/value pyramid launch");
}

bsa_status bsa_build_mask_pyramid(const bsa_shape* s, bsa_dtype dt, bsa_tensor q, bsa_tensor k,
                                  double scale, int32_t n_levels, const double* levels_tau,
                                  uint8_t* mask, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (dt != BSA_BF16 && dt != BSA_F32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (!isfinite(scale)) return fail(BSA_ERR_INVALID, "scale is not finite");
  if (n_levels < 1 || n_levels > 4) return fail(BSA_ERR_INVALID, "n_levels %d not in 1..4", n_levels);
  if (!levels_tau) return fail(BSA_ERR_INVALID, "levels_tau is NULL");
  double taus[4] = {0, 0, 0, 0};
  for (int l = 0; l < n_levels; ++l) {
    taus[l] = levels_tau[l];
    if (!(taus[l] > 0.0 && taus[l] <= 1.0) || (l > 0 && taus[l] < taus[l - 1]))
      return fail(BSA_ERR_INVALID, "level thresholds must be non-decreasing in (0, 1]");
  }
  if (g.nK > bsa::pooled_max_blocks())
    return fail(BSA_ERR_UNSUPPORTED, "pooled selection supports at most %d key blocks",
                bsa::pooled_max_blocks());
  if (empty(g)) return ok();
  if ((st = check_tensor("q", q, elem_bytes(dt))) != BSA_OK) return st;
  if ((st = check_tensor("k", k, elem_bytes(dt))) != BSA_OK) return st;
  if (!mask) return fail(BSA_ERR_INVALID, "mask is NULL");
  const size_t need = bsa::pooled_workspace_bytes(g);
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_INVALID, "workspace needs %zu bytes", need);
  if ((uintptr_t)workspace % 256) return fail(BSA_ERR_INVALID, "workspace not 256-byte aligned");
  return device(bsa::launch_pooled_mask(g, dt == BSA_BF16 ? 0 : 1, arg(q), arg(k), scale, 4,
                                        taus[0], mask, workspace, (hipStream_t)stream, taus,
                                        n_levels),
                "pyramid mask launch");
}

bsa_status bsa_compact_pyramid_lists(const bsa_shape* s, int32_t n_levels, const uint8_t* mask,
                                     int64_t mask_head_stride, int32_t* row_ptr, int32_t* kv_idx,
                                     int32_t* kv_eighths, int64_t kv_capacity,
                                     int64_t* nnz_host, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (n_levels < 1 || n_levels > 4) return fail(BSA_ERR_INVALID, "n_levels %d not in 1..4", n_levels);
  if (mask_head_stride != 0 && mask_head_stride < g.nQ * g.nK)
    return fail(BSA_ERR_INVALID, "mask_head_stride must be 0 or >= nQ*nK");
  if (kv_capacity < 0) return fail(BSA_ERR_INVALID, "kv_capacity < 0");
  if (!row_ptr) return fail(BSA_ERR_INVALID, "row_ptr is NULL");
  int64_t rb[5];
  pyramid_regions(g, n_levels, rb);
  const int64_t R = (int64_t)g.B * g.H * g.nQ, nA = rb[n_levels];
  if (R * nA > kI32Max)
    return fail(BSA_ERR_UNSUPPORTED, "list rows x augmented blocks exceeds int32 list offsets");
  hipStream_t str = (hipStream_t)stream;
  if (R == 0 || g.nK == 0) {
    if (nnz_host) *nnz_host = 0;
    return device(bsa::launch_zero_row_ptr(row_ptr, str), "pyramid lists launch");
  }
  if (!mask) return fail(BSA_ERR_INVALID, "mask is NULL");
  if ((!kv_idx || !kv_eighths) && kv_capacity > 0)
    return fail(BSA_ERR_INVALID, "kv_idx and kv_eighths are required");
  if (!nnz_host && kv_capacity < R * nA)
    return fail(BSA_ERR_CAPACITY, "without nnz_host, kv_capacity must cover every tile (%lld)",
                (long long)(R * nA));
  hipError_t e = bsa::launch_pyramid_lists(g, n_levels, rb, mask, mask_head_stride, row_ptr,
                                           nullptr, nullptr, true, str);
  if (e != hipSuccess) return device(e, "pyramid list count");
  if (nnz_host) {
    int32_t nnz = 0;
    e = hipMemcpyAsync(&nnz, row_ptr + R, sizeof nnz, hipMemcpyDeviceToHost, str);
    if (e == hipSuccess) e = hipStreamSynchronize(str);
    if (e != hipSuccess) return device(e, "pyramid list count readback");
    *nnz_host = nnz;
    if (nnz > kv_capacity)
      return fail(BSA_ERR_CAPACITY, "%d tiles exceed kv_capacity %lld", nnz,
                  (long long)kv_capacity);
    if (nnz > 0 && (!kv_idx || !kv_eighths))
      return fail(BSA_ERR_INVALID, "kv_idx and kv_eighths are required");
  }
  return device(bsa::launch_pyramid_lists(g, n_levels, rb, mask, mask_head_stride, row_ptr,
                                          kv_idx, kv_eighths, false, str),
                "pyramid list scatter");
}

bsa_status bsa_pyramid_attn_fwd(const bsa_shape* s, bsa_dtype dt, bsa_tensor q, bsa_tensor k,
                                bsa_tensor v, bsa_tensor k_pyr, bsa_tensor v_pyr,
                                int32_t n_levels, bsa_tensor o, float* lse,
                                const int32_t* row_ptr, const int32_t* kv_idx,
                                const int32_t* kv_eighths, float scale, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (dt != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "pyramid attention runs on bf16 inputs");
  if ((st = check_levels(g, n_levels)) != BSA_OK) return st;
  if (!isfinite(scale) || scale < 0.f)
    return fail(BSA_ERR_INVALID, "scale must be finite and >= 0");
  if (!row_ptr || !kv_idx || !kv_eighths)
    return fail(BSA_ERR_INVALID, "row_ptr, kv_idx and kv_eighths are required");
  if (empty(g)) return ok();
  const int eb = 2;
  if ((st = check_tensor("q", q, eb)) != BSA_OK) return st;
  if ((st = check_tensor("k", k, eb)) != BSA_OK) return st;
  if ((st = check_tensor("v", v, eb)) != BSA_OK) return st;
  if ((st = check_tensor("o", o, eb)) != BSA_OK) return st;
  if (o.ptr == q.ptr || o.ptr == k.ptr || o.ptr == v.ptr)
    return fail(BSA_ERR_INVALID, "o must not alias q, k or v");
  if (g.N > 1 && (k.stride_n < g.D || v.stride_n < g.D))
    return fail(BSA_ERR_INVALID, "k and v need stride_n >= head_dim");
  if (k.stride_n > (int64_t)(1 << 23) || v.stride_n > (int64_t)(1 << 23))
    return fail(BSA_ERR_UNSUPPORTED, "k/v stride_n above 2^23 elements");
  if (n_levels > 1) {
    if ((st = check_tensor("k_pyr", k_pyr, eb)) != BSA_OK) return st;
    if ((st = check_tensor("v_pyr", v_pyr, eb)) != BSA_OK) return st;
    if (k_pyr.stride_n != k.stride_n || v_pyr.stride_n != v.stride_n)
      return fail(BSA_ERR_INVALID, "k_pyr / v_pyr need the row stride of k / v");
  }
  bsa::AttnArgs a;
  a.q = arg(q); a.k = arg(k); a.v = arg(v);
  a.o = o.ptr; a.osb = o.stride_b; a.osn = o.stride_n; a.osh = o.stride_h;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.kv_idx = kv_idx;
  a.lists_shared = 0;
  a.scale = scale;
  a.tile_gap = nullptr;
  a.kp = n_levels > 1 ? arg(k_pyr) : arg(k);
  a.vp = n_levels > 1 ? arg(v_pyr) : arg(v);
  a.kv_eighths = kv_eighths;
  pyramid_regions(g, n_levels, a.pyr_rb);
  if ((st = debug_check(g, false, row_ptr, kv_idx, a.pyr_rb[n_levels], false,
                        (hipStream_t)stream)) != BSA_OK)
    return st;
  return device(bsa::launch_attn_bf16(g, a, (hipStream_t)stream), "pyramid attention launch");
}

bsa_status bsa_sparse_attn_fwd(const bsa_shape* s, bsa_dtype dt, bsa_tensor q, bsa_tensor k,
                               bsa_tensor v, bsa_tensor o, float* lse, const int32_t* row_ptr,
                               const int32_t* kv_idx, int32_t lists_shared, float scale,
                               float* tile_gap, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (dt != BSA_BF16 && dt != BSA_F32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  if (!isfinite(scale) || scale < 0.f)
    return fail(BSA_ERR_INVALID, "scale must be finite and >= 0");
  if (lists_shared != 0 && lists_shared != 1)
    return fail(BSA_ERR_INVALID, "lists_shared must be 0 or 1");
  if ((row_ptr == nullptr) != (kv_idx == nullptr))
    return fail(BSA_ERR_INVALID, "row_ptr and kv_idx must both be set or both be NULL");
  if (tile_gap && !row_ptr) return fail(BSA_ERR_INVALID, "tile_gap needs block lists");
  // Gaps feed bsa_update_skip_mask, which reads per-head lists only.
  if (tile_gap && lists_shared)
    return fail(BSA_ERR_UNSUPPORTED, "tile_gap needs per-head lists (lists_shared = 0)");
  if (empty(g)) return ok();
  const int eb = elem_bytes(dt);
  if ((st = check_tensor("q", q, eb)) != BSA_OK) return st;
  if ((st = check_tensor("k", k, eb)) != BSA_OK) return st;
  if ((st = check_tensor("v", v, eb)) != BSA_OK) return st;
  if ((st = check_tensor("o", o, eb)) != BSA_OK) return st;
  if (o.ptr == q.ptr || o.ptr == k.ptr || o.ptr == v.ptr)
    return fail(BSA_ERR_INVALID, "o must not alias q, k or v");
  // Key/value rows of a tile are addressed with 32-bit offsets from the tile's
  // first row and bounds-checked by byte range, which needs rows that do not
  // overlap and a 64-row tile span below 2^31 bytes.
  if (g.N > 1 && (k.stride_n < g.D || v.stride_n < g.D))
    return fail(BSA_ERR_INVALID, "k and v need stride_n >= head_dim");
  if (k.stride_n > (int64_t)(1 << 23) || v.stride_n > (int64_t)(1 << 23))
    return fail(BSA_ERR_UNSUPPORTED, "k/v stride_n above 2^23 elements");
  bsa::AttnArgs a;
  a.q = arg(q); a.k = arg(k); a.v = arg(v);
  a.o = o.ptr; a.osb = o.stride_b; a.osn = o.stride_n; a.osh = o.stride_h;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.kv_idx = kv_idx;
  a.lists_shared = lists_shared;
  a.scale = scale;
  a.tile_gap = tile_gap;
  hipStream_t str = (hipStream_t)stream;
  if ((st = debug_check(g, lists_shared, row_ptr, kv_idx, g.nK, false, str)) != BSA_OK) return st;
  return device(dt == BSA_BF16 ? bsa::launch_attn_bf16(g, a, str) : bsa::launch_attn_f32(g, a, str),
                "attention launch");
}

bsa_status bsa_update_skip_mask(const bsa_shape* s, const int32_t* row_ptr,
                                const int32_t* kv_idx, const float* tile_gap, float tau,
                                uint8_t* skip, void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (!(tau > 0.f)) return fail(BSA_ERR_INVALID, "tau must be > 0");
  if ((int64_t)g.B * g.H * g.nQ * g.nK > kI32Max)
    return fail(BSA_ERR_UNSUPPORTED, "list rows x key blocks exceeds int32 list offsets");
  if (empty(g)) return ok();
  if (!row_ptr || !kv_idx || !tile_gap || !skip)
    return fail(BSA_ERR_INVALID, "row_ptr, kv_idx, tile_gap and skip are required");
  const float tau2 = (float)((double)tau * 1.4426950408889634);
  if ((st = debug_check(g, false, row_ptr, kv_idx, g.nK, false, (hipStream_t)stream)) != BSA_OK)
    return st;
  return device(bsa::launch_skip_update(g, row_ptr, kv_idx, tile_gap, tau2, skip,
                                        (hipStream_t)stream),
                "skip update launch");
}

bsa_status bsa_check_block_lists(const bsa_shape* s, int32_t lists_shared,
                                 const int32_t* row_ptr, const int32_t* kv_idx, int64_t kv_len,
                                 int64_t n_blocks, int32_t ascending, int32_t on_device,
                                 void* stream) {
  bsa::Geom g;
  bsa_status st = make_geom(s, &g);
  if (st != BSA_OK) return st;
  if (lists_shared != 0 && lists_shared != 1)
    return fail(BSA_ERR_INVALID, "lists_shared must be 0 or 1");
  if (on_device != 0 && on_device != 1) return fail(BSA_ERR_INVALID, "on_device must be 0 or 1");
  if (kv_len < 0 || n_blocks < 0) return fail(BSA_ERR_INVALID, "kv_len and n_blocks must be >= 0");
  if (!row_ptr) return fail(BSA_ERR_INVALID, "row_ptr is NULL");
  if (!kv_idx && kv_len > 0) return fail(BSA_ERR_INVALID, "kv_idx is NULL");
  const int64_t R = lists_shared ? g.nQ : (int64_t)g.B * g.H * g.nQ;
  const int64_t nb = n_blocks ? n_blocks : g.nK;
  int rule = 0;
  int64_t row = -1;
  if (!on_device) {
    row = bsa::check_lists_host(row_ptr, kv_idx, R, kv_len, nb, ascending != 0, &rule);
    return list_result(row, rule);
  }
  hipError_t e = bsa::check_lists_device(row_ptr, kv_idx, R, kv_len, nb, ascending != 0, &rule,
                                         &row, (hipStream_t)stream);
  if (e != hipSuccess) return device(e, "block list check");
  return list_result(row, rule);
}

}  // extern "C"
