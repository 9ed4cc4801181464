/*
 * bsa.h -- C ABI of libbsa: block-sparse, bidirectional softmax attention over
 * a flattened frames x height x width video token sequence, for MI355X (gfx950).
 *
 * Pages this interface follows (web pages that describe the method):
 *   [Lite]   LiteAttention summary page (arXiv:2511.11062), numbered sections.
 *   [VMoBA]  VMoBA summary page (arXiv:2506.23858), numbered sections.
 *   [Radial] "MIT实验室推出Radial Attention：让视频AI生成快如闪电的神奇技术"
 *            (arXiv:2506.19852).
 *   [PARO]   PAROAttention summary page (arXiv:2506.16054), numbered sections.
 *   [PSA]    "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍"
 *            (arXiv:2512.04025).
 * Every page presents its method as a drop-in replacement for dense attention
 * ([Lite] section 六 extends an existing attention API with a persistent skip
 * mask; [VMoBA] section 六 a standard replacement interface; [PSA] plug and
 * play), so the calls below take the tensors a dense attention call takes,
 * plus the block mask or block lists.
 *
 * Conventions shared by all calls
 * -------------------------------
 * Tokens: i = (t*height + y)*width + x, N = frames*height*width,
 *   F = height*width tokens per frame. Row (query) block a covers tokens
 *   [a*block_q, min(N, (a+1)*block_q)), column (key) block c covers
 *   [c*block_k, min(N, (c+1)*block_k)); nQ = ceil(N/block_q),
 *   nK = ceil(N/block_k). Ragged last blocks keep their true sizes: padding
 *   tokens never enter a maximum, sum or mean.
 * Tensors (bsa_tensor): element (b, i, h, x) of Q, K, V or O lives at
 *   ptr + b*stride_b + i*stride_n + h*stride_h + x (strides in elements,
 *   head_dim contiguous). The usual layout is [B][N][H][d].
 * Masks: uint8, 0 = drop the tile, nonzero = keep. A per-head mask is
 *   [B][H][nQ][nK]; a shared mask is [nQ][nK] (head stride 0).
 * Block lists (CSR): list row r = (b*H + h)*nQ + a (or just a when one list
 *   serves every (b, h)); kv_idx[row_ptr[r] .. row_ptr[r+1]) holds the kept
 *   key blocks of that row, in ascending order as compaction writes them or
 *   in the visiting order bsa_order_block_lists gives them.
 * Memory: every tensor, mask and list pointer is a DEVICE pointer owned by
 *   the caller; the library allocates no device memory and keeps no state
 *   besides its loaded kernels and a thread-local error string.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = legacy default
 *   stream). Calls validate their arguments on the host before touching the
 *   GPU, enqueue their kernels on `stream` and return without synchronising
 *   unless documented otherwise.
 * Errors: no call throws; each returns a bsa_status. BSA_ERR_INVALID and
 *   BSA_ERR_UNSUPPORTED are returned before anything is enqueued.
 *   bsa_last_error() gives a thread-local text for the last failing call.
 * Sizes: zero-sized shapes (B, H or N = 0) are valid and enqueue nothing
 *   except the single row_ptr[0] = 0 of compaction.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define BSA_API __attribute__((visibility("default")))
#else
#define BSA_API
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID = 1,     /* null required pointer, bad size, misalignment, bad knob */
  BSA_ERR_UNSUPPORTED = 2, /* head_dim, block size or dtype outside the compiled set */
  BSA_ERR_CAPACITY = 3,    /* kv_capacity smaller than the number of kept tiles */
  BSA_ERR_DEVICE = 4       /* a HIP call failed; see bsa_last_error() */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype;

typedef struct {
  int32_t batch, heads, head_dim; /* B, H, d (d in {64, 128}) */
  int32_t frames, height, width;  /* T, Hs, Ws; N = T*Hs*Ws < 2^31 */
  int32_t block_q, block_k;       /* block_q in {64, 128}; block_k = 64 */
} bsa_shape;

typedef struct {
  void* ptr;                          /* device pointer, 16-byte aligned */
  int64_t stride_b, stride_n, stride_h; /* in elements; multiples of 8 (bf16) or 4 (f32) */
} bsa_tensor;

/*
 * Static radial mask ([Radial]: attention weakens with temporal and spatial
 * distance, each frame attends mostly to its nearest frames with a weight that
 * falls with frame distance, and the map is fixed ahead of time; cost grows as
 * n log n).
 * Frame distance dt = |t(i) - t(j)| falls in band r = number of base-
 * `decay_base` digits of dt (r = 0 for dt = 0). The in-frame half-width is
 * h_r = floor(h0 / decay_base^r) while h_r >= block_k/2 (bands 0..r*); beyond
 * r*, the half-width stays block_k/2 and only every decay_base^(r - r*)-th
 * distance of band r is kept. Token pair (i, j) is kept iff its distance is
 * kept and |s(i) - s(j)| < h_eff, s = in-frame position. Tile (a, c) is kept
 * iff any token pair of row block a and column block c is kept.
 *   h0          window half-width at distance 0, tokens; block_k/2 <= h0 < 2^30
 *   decay_base  >= 2
 *   mask        out, [nQ][nK] (shared by all batches and heads)
 * Integer only; the result is deterministic and exact.
 */
BSA_API bsa_status bsa_build_mask_radial(const bsa_shape* s, int32_t h0, int32_t decay_base,
                                 uint8_t* mask, void* stream);

/*
 * Bytes of device workspace bsa_build_mask_pooled needs for shape s, any
 * mode (pooled means of Q and K and the scores in fp64; for the head-wide
 * modes also the row probabilities and the selection's per-head state);
 * a multiple of 256.
 */
BSA_API size_t bsa_pooled_workspace_bytes(const bsa_shape* s);

/*
 * Dynamic mask from mean-pooled block scores ([PSA]: average pooling of keys
 * block by block; [VMoBA] sections 三 and 六: block relevance from pooled
 * scores by matrix operations, and a threshold that sets how many blocks a
 * query keeps according to how concentrated its attention is).
 * Per (b, h), in fp64 with a fixed operation order:
 *   qbar_a = (sum_{i in row block a} q_i) / |R_a|, sum in ascending i;
 *   kbar_c likewise;
 *   S_ac = scale * sum_x qbar_ax * kbar_cx, x ascending, no fused multiply-add;
 *   row a orders c by (S desc, c asc) and keeps
 *     mode 0: the first min(param, nK) blocks (param = k >= 1), or
 *     mode 1: the shortest prefix whose running sum of p_c reaches param,
 *             p_c = exp(S_ac - max S_a) / Z, Z summed in ascending c,
 *             param = tau_p in (0, 1] (all blocks if the sum never reaches it).
 *   Head-wide modes ([VMoBA] section 三: rank every query block against every
 *   key block together and serve the strongest pairs first; a head keeps as
 *   many blocks as its attention concentration calls for): all nQ*nK pairs
 *   of (b, h) are ordered by (key desc, a*nK + c asc) and
 *     mode 2: the first min(param, nQ*nK) pairs are kept, key S_ac
 *             (param = k >= 1), or
 *     mode 3: key p_ac (the row softmax of mode 1); the shortest prefix whose
 *             running mass reaches param * nQ is kept (param = tau_p in
 *             (0, 1]; all pairs for tau_p = 1 or if the mass falls short).
 *             The mass is summed in a fixed parallel order, so a pair whose
 *             prefix sum lies within rounding (~1e-12 relative) of the target
 *             can differ from a sequential sum.
 *   In modes 2 and 3 every row also keeps its best block (S desc, c asc), so
 *   no row is empty.
 *   q, k        inputs of dtype dt ([B][N][H][d] by strides)
 *   mask        out, [B][H][nQ][nK]
 *   workspace   device buffer of at least bsa_pooled_workspace_bytes(s)
 *               bytes, 256-byte aligned; contents on return are unspecified.
 * Supports nK <= 8192 key blocks (BSA_ERR_UNSUPPORTED beyond); rows of more
 * than 2048 blocks (the 4x-length video grid has 7,425) take a path with one
 * workgroup per row and the same results.
 */
BSA_API bsa_status bsa_build_mask_pooled(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                 bsa_tensor k, double scale, int32_t mode, double param,
                                 uint8_t* mask, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * bsa_build_mask_pooled without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same modes, parameters, result and
 * errors as bsa_build_mask_pooled; the scratch it needs comes from a static
 * device array inside the library of 64 MiB (64 << 20 bytes) per GPU, held
 * from library load until the process ends. Modes 0 and 1 need
 * 8*(B*H*(nQ + nK)*d + B*H*nQ*nK) bytes rounded up to 256 (the 480p layer
 * with 12 heads: 37.7 MB; 16*B*H*nQ bytes more when nK > 2048), modes 2
 * and 3 bsa_pooled_workspace_bytes(s);
 * a shape and mode that need more return BSA_ERR_CAPACITY before anything is
 * enqueued. The call allocates nothing. Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on the same GPU (other streams,
 * other host threads) race and must be serialised by the caller.
 */
BSA_API bsa_status bsa_build_mask_pooled_noalloc(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                                 bsa_tensor k, double scale, int32_t mode,
                                                 double param, uint8_t* mask, void* stream);

/*
 * Per-row lists of kept key blocks ([Lite] sections 三 and 六: a skipped tile
 * must cost no softmax and no memory transfer, so the loader walks only the
 * listed tiles).
 * Tile (b, h, a, c) is listed iff mask[(b*H + h)*mask_head_stride + a*nK + c]
 * != 0 and (skip == NULL or skip[((b*H + h)*nQ + a)*nK + c] == 0).
 *   mask_head_stride  0 (one mask for every head) or >= nQ*nK
 *   skip              nullable, [B][H][nQ][nK]
 *   row_ptr           out, int32 [R+1], R = nQ if mask_head_stride == 0 and
 *                     skip == NULL (one list for all (b, h)), else B*H*nQ
 *   kv_idx            out, int32 [kv_capacity]
 *   nnz_host          nullable host pointer. When given, the call counts the
 *                     kept tiles, synchronises the stream, stores the count and
 *                     returns BSA_ERR_CAPACITY without writing kv_idx if it
 *                     exceeds kv_capacity. When NULL, kv_capacity must be at
 *                     least R*nK (the worst case) or BSA_ERR_CAPACITY is
 *                     returned before anything is enqueued.
 * Exact integer work; lists are in ascending key-block order.
 */
BSA_API bsa_status bsa_compact_block_lists(const bsa_shape* s, const uint8_t* mask,
                                   int64_t mask_head_stride, const uint8_t* skip,
                                   int32_t* row_ptr, int32_t* kv_idx, int64_t kv_capacity,
                                   int64_t* nnz_host, void* stream);

/*
 * Visiting order of the listed key blocks ([Lite] section 五: a radial-centric
 * order of the tiles reaches a row's maximum sooner, which lets the
 * running-maximum skip test mark more tiles; section 十 expects 10-20% more
 * sparsity from a better order). The forward pass visits each row's list in
 * the order it is stored, so reordering a list changes the tile gaps (and
 * with them the skip decisions), never the attention result beyond rounding.
 *   order       0: ascending key-block order (a copy); 1: radial-centric:
 *               key blocks by increasing |ck2 - cq2| with ck2 = c*block_k +
 *               min(N, (c+1)*block_k) - 1 and cq2 = a*block_q + min(N,
 *               (a+1)*block_q) - 1 (twice the token midpoints of key block c
 *               and of the row's block a), ties to the lower c.
 *   row_ptr     the lists' row pointers ([R+1], R = nQ when lists_shared,
 *               else B*H*nQ); row r belongs to row block a = r % nQ
 *   kv_in       lists in ascending order, as bsa_compact_block_lists writes
 *               them (other inputs give an unspecified arrangement of each
 *               row's entries, still written inside that row)
 *   kv_out      out, same row_ptr; must not alias kv_in
 * Exact integer work; deterministic.
 */
BSA_API bsa_status bsa_order_block_lists(const bsa_shape* s, int32_t order, const int32_t* row_ptr,
                                 int32_t lists_shared, const int32_t* kv_in, int32_t* kv_out,
                                 void* stream);

/*
 * Token order before blocking ([PARO] section 二: flattening the video to one
 * sequence separates tokens that attend to each other; reordering by one of
 * the six orders of the frame, row and column axes, chosen per head, makes
 * the attention block-shaped. [VMoBA] section 三: blocks made of temporal
 * chunks, spatial patches or spatio-temporal cubes).
 * Writes perm[i'] = the original token (i = (t*height + y)*width + x) that
 * new position i' holds:
 *   kind 0: axes = (slowest, middle, fastest) axis, a permutation of
 *           (0 = frame, 1 = row, 2 = column); (0, 1, 2) is the identity.
 *   kind 1: axes = box extent (frames, rows, columns), each >= 1: boxes in
 *           (frame, row, column) order, tokens inside a box in (frame, row,
 *           column) order, boxes at the far edges smaller. Boxes covering
 *           whole frames are temporal chunks (the identity order); boxes of
 *           one frame are spatial patches; deeper boxes are cubes.
 *   perm        out, int32 [N] (device)
 * Exact integer work. One call per order; per-head orders are built into
 * consecutive [N] slices of one [H][N] array.
 */
BSA_API bsa_status bsa_make_token_permutation(const bsa_shape* s, int32_t kind,
                                      const int32_t* axes /* host, [3] */, int32_t* perm,
                                      void* stream);

/*
 * Per-head choice of the token order ([PARO] section 二: each head takes the
 * one of the six frame/row/column axis orders under which its attention is
 * most sparsity-friendly; the quantization side of that choice is not built).
 * Reading taken: order o (the axis orders of bsa_make_token_permutation kind
 * 0 in lexicographic order: 0 = (0,1,2) the identity, 1 = (0,2,1),
 * 2 = (1,0,2), 3 = (1,2,0), 4 = (2,0,1), 5 = (2,1,0)) scores, for head h, the
 * number of tiles that bsa_build_mask_pooled (mode 0 or 1 with param) keeps
 * for that head, summed over the batch, when Q and K are gathered into order
 * o; the head takes the order with the fewest, ties to the lower index.
 * Exact integer counts over bit-exact masks.
 *   order_out   out, int32 [H] (device): the chosen order per head
 *   counts_out  out, uint64 [H][6] (device) kept tiles per head and order,
 *               or NULL
 *   workspace   device buffer of at least bsa_token_orders_workspace_bytes
 *               (s, dt) bytes, 256-byte aligned (Q and K in one order, one
 *               pooled mask and the pooled builder's scratch)
 * Same limits and errors as bsa_build_mask_pooled; modes other than 0 and 1
 * return BSA_ERR_INVALID.
 */
BSA_API size_t bsa_token_orders_workspace_bytes(const bsa_shape* s, bsa_dtype dt);
BSA_API bsa_status bsa_choose_token_orders(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                           bsa_tensor k, double scale, int32_t mode,
                                           double param, int32_t* order_out,
                                           uint64_t* counts_out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * Moves the tokens of a [B][N][H][d] tensor into or out of a token order
 * (pure data movement; bytes are copied as they are):
 *   scatter 0 (gather):  out[b][i'][h] = in[b][perm_h[i']][h]
 *   scatter 1 (scatter): out[b][perm_h[i']][h] = in[b][i'][h]
 * with perm_h = perm + h*perm_head_stride (0: one order for every head, else
 * >= N). Q, K and V are gathered before masks, lists and the forward call,
 * and the forward's O is scattered back; attention over the new order
 * differs from the original only through which tiles the mask keeps.
 * perm should hold each of 0..N-1 once; an entry outside [0, N) moves
 * nothing. out must not alias in.
 */
BSA_API bsa_status bsa_permute_tokens(const bsa_shape* s, bsa_dtype dt, const int32_t* perm,
                              int64_t perm_head_stride, int32_t scatter, bsa_tensor in,
                              bsa_tensor out, void* stream);

/*
 * Block-sparse attention forward ([PSA]: whole blocks are kept or dropped;
 * [Lite] section 六: online softmax over the tiles of a persistent skip list;
 * bidirectional, no causal mask). For query i of row block a of head (b, h),
 * with J_i the union of the listed key blocks of that row:
 *   s_ij = scale * q_i . k_j,  o_i = sum_{j in J_i} softmax_j(s_ij) v_j,
 *   lse_i = log sum_{j in J_i} exp(s_ij)   (natural log).
 * An empty list gives o_i = 0 and lse_i = -inf.
 *   dt          BSA_BF16 (MFMA path, fp32 accumulation and softmax, O rounded
 *               to bf16 nearest-even) or BSA_F32 (fp32 path)
 *   q, k, v     inputs; o output, same dtype
 *   lse         nullable, out fp32 [B][H][N]
 *   row_ptr, kv_idx  lists as produced by bsa_compact_block_lists; both NULL
 *               means every tile (dense attention)
 *   lists_shared 1: one list row per a for every (b, h) (row_ptr [nQ+1]);
 *               0: row_ptr [B*H*nQ+1]
 *   tile_gap    nullable, out fp32, one value per list entry; needs
 *               per-head lists (lists_shared = 0, else BSA_ERR_UNSUPPORTED),
 *               the lists bsa_update_skip_mask reads:
 *               with the listed tiles of a row visited in list order and
 *               m_run(r) the running maximum of row r's scaled scores over
 *               the tiles visited before, the maximum over valid rows r of
 *               (max_{j in tile} s_rj - m_run(r)) in log2 units
 *               (scores times log2(e)); +inf for the first tile of a row
 *               ([Lite] section 五: a tile far below the accumulated maximum
 *               contributes exponentially little).
 * Q, K, V must not alias O. K and V need head_dim <= stride_n <= 2^23.
 */
BSA_API bsa_status bsa_sparse_attn_fwd(const bsa_shape* s, bsa_dtype dt, bsa_tensor q, bsa_tensor k,
                               bsa_tensor v, bsa_tensor o, float* lse, const int32_t* row_ptr,
                               const int32_t* kv_idx, int32_t lists_shared, float scale,
                               float* tile_gap, void* stream);

/*
 * Carry the skip decisions forward ([Lite] sections 二, 三 and 六: decide
 * early, then reuse the decisions for every later denoising step; the skip
 * set only grows). For every entry e of list row r = (b*H + h)*nQ + a:
 *   skip[r*nK + kv_idx[e]] |= (tile_gap[e] <= -tau2),  tau2 = fp32(tau * log2(e)),
 * with tau > 0 in natural-log units of the scaled scores.
 *   row_ptr, kv_idx  per-head lists (B*H*nQ rows), as used by the forward call
 *                    that produced tile_gap
 *   skip             in/out, [B][H][nQ][nK]
 */
BSA_API bsa_status bsa_update_skip_mask(const bsa_shape* s, const int32_t* row_ptr,
                                const int32_t* kv_idx, const float* tile_gap, float tau,
                                uint8_t* skip, void* stream);

/*
 * Pyramid attention ([PSA]: key/value blocks kept at several resolutions,
 * each level the average pooling of the finer one; each (query block, key
 * block) pair attends at the level its importance earns, set by thresholds;
 * the probabilities stay consistent across levels; the logical block size is
 * decoupled from the hardware tile).
 * Levels l = 0 .. n_levels-1 (n_levels in 1..4; N must be a multiple of
 * 2^(n_levels-1), else BSA_ERR_UNSUPPORTED): level l of key block c holds
 * block_k / 2^l pooled keys, each the mean of 2^l consecutive tokens of K and
 * of V; a pooled key stands for its 2^l tokens, so its score gets + l ln 2.
 * Level masks are uint8: 0 = dropped, 1 + l = level l.
 * Augmented key blocks: level l occupies blocks [rb_l, rb_{l+1}) with
 * rb_0 = 0 and rb_{l+1} = rb_l + ceil((N >> l) / block_k); blocks below rb_1
 * are the original K / V, the others rows of k_pyr / v_pyr (level 1 first).
 */

/* Rows of k_pyr / v_pyr for n_levels (0 for one level); -1 if invalid. */
BSA_API int64_t bsa_pyramid_rows(const bsa_shape* s, int32_t n_levels);

/*
 * Pooled levels 1 .. n_levels-1 of K and V: row (rb_l - rb_1)*block_k + g of
 * k_pyr is the mean of K rows [g*2^l, (g+1)*2^l), summed in fp32 in ascending
 * order, divided by 2^l and rounded to dt (nearest even); likewise v_pyr from
 * V. k_pyr, v_pyr: [B][bsa_pyramid_rows][H][d] by strides; padding rows at
 * the end of each level are left unwritten.
 */
BSA_API bsa_status bsa_build_kv_pyramid(const bsa_shape* s, bsa_dtype dt, int32_t n_levels,
                                bsa_tensor k, bsa_tensor v, bsa_tensor k_pyr,
                                bsa_tensor v_pyr, void* stream);

/*
 * Level mask from the pooled block scores of bsa_build_mask_pooled (same
 * workspace): row a walks its key blocks in (S desc, c asc) order summing the
 * row softmax mass p_c of mode 1; a block joins the current level, then the
 * level advances past every threshold the running sum (including that block)
 * has reached; blocks after the last level are dropped. levels_tau (host,
 * [n_levels]) non-decreasing in (0, 1]. The row's best block is at level 0.
 * Same key-block limit as bsa_build_mask_pooled (nK <= 8192).
 *   mask  out, [B][H][nQ][nK], values 0 .. n_levels
 */
BSA_API bsa_status bsa_build_mask_pyramid(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                  bsa_tensor k, double scale, int32_t n_levels,
                                  const double* levels_tau, uint8_t* mask, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Lists of augmented tiles for a level mask: per row r = (b*H + h)*nQ + a (one
 * list per (b, h) always), the augmented blocks holding at least one
 * selected 8-row eighth, ascending, and kv_eighths[e] = bit mask of the
 * selected eighths (bit i = rows [8i, 8i+8) of the tile). Key block c at
 * level l covers pooled rows [c*block_k/2^l, (c+1)*block_k/2^l) of level l,
 * i.e. 8/2^l eighths of augmented block rb_l + c/2^l. Mask values above
 * n_levels select nothing.
 *   mask_head_stride  0 (one mask for all heads) or >= nQ*nK
 *   kv_capacity, nnz_host  as in bsa_compact_block_lists (worst case
 *                  B*H*nQ*rb_{n_levels})
 */
BSA_API bsa_status bsa_compact_pyramid_lists(const bsa_shape* s, int32_t n_levels,
                                     const uint8_t* mask, int64_t mask_head_stride,
                                     int32_t* row_ptr, int32_t* kv_idx, int32_t* kv_eighths,
                                     int64_t kv_capacity, int64_t* nnz_host, void* stream);

/*
 * Pyramid attention forward (bf16 inputs; fp32 accumulation and softmax, O
 * rounded to bf16). For query i of row block a, the keys are the rows of the
 * selected eighths of the row's augmented tiles (padding rows past a level's
 * N >> l never count); a key of level l scores scale * q_i . k + l ln 2; o_i
 * is the softmax-weighted mean of the matching value rows, lse_i the natural
 * log of the weight sum (-inf and o_i = 0 for an empty list).
 *   k_pyr, v_pyr  as written by bsa_build_kv_pyramid, with the row stride
 *                 (stride_n) of k and v; ignored for one level
 *   row_ptr, kv_idx, kv_eighths  as written by bsa_compact_pyramid_lists
 */
BSA_API bsa_status bsa_pyramid_attn_fwd(const bsa_shape* s, bsa_dtype dt, bsa_tensor q,
                                bsa_tensor k, bsa_tensor v, bsa_tensor k_pyr,
                                bsa_tensor v_pyr, int32_t n_levels, bsa_tensor o, float* lse,
                                const int32_t* row_ptr, const int32_t* kv_idx,
                                const int32_t* kv_eighths, float scale, void* stream);

/*
 * Debug check of block lists ([Lite] sections 三 and 六: the forward walks only
 * the listed tiles, so a row must name each of its kept key blocks once, and
 * only blocks that exist). Rules, reported for the first failing row r
 * (lowest r, then lowest rule):
 *   1 row_ptr[0] != 0;  2 row_ptr[r+1] < row_ptr[r];  3 row_ptr[r+1] > kv_len;
 *   4 an entry outside [0, n_blocks);  5 an entry twice in one row;
 *   6 (ascending = 1 only) a row not in strictly ascending order.
 *   lists_shared  1: R = nQ list rows; 0: R = B*H*nQ
 *   n_blocks      key blocks an entry may name (0 = nK; for pyramid lists
 *                 the number of augmented blocks)
 *   kv_len        entries of kv_idx that may be read (>= 0)
 *   on_device     0: row_ptr and kv_idx are HOST pointers, checked on the
 *                 calling thread (stream unused); 1: DEVICE pointers, checked
 *                 by kernels on `stream`; the call then synchronises stream
 * Reads only row_ptr[0..R] and kv_idx[0..kv_len). Returns BSA_OK, or
 * BSA_ERR_INVALID with "row r: rule k ..." in bsa_last_error().
 * With the environment variable BSA_CHECK=1, bsa_sparse_attn_fwd,
 * bsa_update_skip_mask, bsa_order_block_lists and bsa_pyramid_attn_fwd run
 * this check on their device lists first (kv_len = row_ptr[R]; ascending
 * order required for the input of bsa_order_block_lists), synchronising the
 * stream, and return BSA_ERR_INVALID without launching anything when it fails.
 */
BSA_API bsa_status bsa_check_block_lists(const bsa_shape* s, int32_t lists_shared,
                                         const int32_t* row_ptr, const int32_t* kv_idx,
                                         int64_t kv_len, int64_t n_blocks, int32_t ascending,
                                         int32_t on_device, void* stream);

/* Static text for a status code. */
BSA_API const char* bsa_status_string(bsa_status st);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
BSA_API const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
