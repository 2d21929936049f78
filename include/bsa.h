/*
 * bsa.h -- C ABI of libbsa.so: block-sparse attention forward and the top-k
 * gathered sparse attention forward, for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers marked "device" point to GPU memory owned by the caller (the
 *   library allocates no device memory and keeps no pointer after a call
 *   returns, except inside a caller-owned plan buffer).
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   All compute calls are asynchronous and ordered on that stream.  Only
 *   bsa_plan_nnz (one integer to the host), bsa_plan_check and calls made
 *   in debug mode (below) synchronise it.
 * - Return value: BSA_OK (0) or a negative bsa_status_t.  Host-side argument
 *   validation runs before any HIP call, so an invalid call touches neither
 *   the GPU nor the output buffers.  Launch failures are reported as
 *   BSA_ERR_HIP; faults inside a kernel surface at the caller's next sync.
 *   bsa_last_error() returns a thread-local message for the last failure.
 * - Debug mode (environment variable BSA_DEBUG set and not "0" when the
 *   library is first used, or bsa_set_debug(1)): every call that reads a
 *   plan first copies the plan to the host, checks it as bsa_plan_check
 *   does and synchronises the stream; an inconsistent plan returns
 *   BSA_ERR_BAD_PLAN and nothing is launched.
 * - Tensors are dense and row-major (last index fastest), with the shapes
 *   given below.  q/k/v/kv/out must be 16-byte aligned.
 * - Nothing throws across this boundary.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = -1,     /* null pointer, non-positive size, bad scale */
  BSA_ERR_UNSUPPORTED = -2,     /* shape or dtype with no compiled kernel */
  BSA_ERR_MISALIGNED = -3,      /* pointer not 16-byte aligned */
  BSA_ERR_PLAN_MISMATCH = -4,   /* plan dims do not match the call */
  BSA_ERR_BUFFER_TOO_SMALL = -5,/* plan buffer smaller than bsa_plan_buffer_bytes */
  BSA_ERR_HIP = -6,             /* a HIP runtime call or launch failed */
  BSA_ERR_BAD_PLAN = -7         /* plan contents inconsistent (plan checks) */
} bsa_status_t;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype_t;

/*
 * A plan: a host-side value that describes a caller-owned device buffer
 * holding the per-row CSR of a block layout.  Filled by bsa_plan; immutable
 * afterwards; valid for any batch size (the layout has no batch axis) and
 * reusable across calls until the caller frees the buffer.
 *
 * Rows are r = h * Mb + m.  Buffer sections (each starting on a 256-byte
 * boundary, offsets returned by bsa_plan_sections):
 *   row_ptr   int32 [H*Mb + 1]  exclusive prefix sum of per-row live counts
 *   row_order int32 [H*Mb]      rows head by head; inside a head by live
 *                               count descending, ties by m ascending
 *   nnz_total int32 [1]         number of live tiles (= row_ptr[H*Mb])
 *   col_idx   int32 [H*Mb*Nb]   live block columns of each row, ascending;
 *                               only the first nnz_total entries are written
 * and the pairs of neighbouring block rows (offsets returned by
 * bsa_plan_pair_sections), pair q = h * Mp + p, Mp = ceil(Mb / 2), joining
 * rows 2p and 2p + 1 of head h (the second absent when Mb is odd):
 *   pair_ptr   int32 [H*Mp + 1] exclusive prefix sum of the union counts
 *   pair_order int32 [H*Mp]     pairs head by head, by union count
 *                               descending, ties by p ascending
 *   pair_info  int32 [2]        pair_total (= pair_ptr[H*Mp]); use_pairs:
 *                               1 when 4 * pair_total <= 3 * nnz_total
 *   pair_cols  int32 [H*Mp*Nb]  the union of the two rows' live columns,
 *                               ascending, each entry n + 2^24 * mask
 *                               (mask bit 0: row 2p lists n; bit 1: row
 *                               2p + 1 does); pair_total entries written
 * Layouts made of local windows, global columns and strides list nearly the
 * same columns in neighbouring block rows; when use_pairs is set, bsa_forward
 * (bf16, bs = 64, no score-changing option) runs one work item per pair and
 * loads each tile the two rows share once.
 */
typedef struct {
  int32_t H, Mb, Nb;
  int32_t reserved;
  void *dev_buf;
  size_t dev_bytes;
} bsa_plan_t;

/* Bytes a plan buffer needs for an [H, Mb, Nb] layout (worst case: every
 * tile live).  Returns 0 if a dimension is non-positive or H*Mb*Nb >= 2^31. */
size_t bsa_plan_buffer_bytes(int32_t H, int32_t Mb, int32_t Nb);

/* Byte offsets of the four plan sections inside the plan buffer
 * (row_ptr, row_order, nnz_total, col_idx).  Host-only; returns
 * BSA_ERR_INVALID_ARG for bad dimensions or a null output pointer. */
int bsa_plan_sections(int32_t H, int32_t Mb, int32_t Nb, size_t offsets_out[4]);

/* Byte offsets of the four pair sections (pair_ptr, pair_order, pair_info,
 * pair_cols) inside the plan buffer.  Host-only; errors as
 * bsa_plan_sections. */
int bsa_plan_pair_sections(int32_t H, int32_t Mb, int32_t Nb, size_t offsets_out[4]);

/*
 * Build the plan of a block layout.
 *
 * Operation: the layout (DeepSpeed sparse-attention utils page, "I/O
 * Contract") is an int32 tensor [H, Mb, Nb] in which a non-zero entry marks a
 * live b x b tile of Q K^T.  Storing only the live tiles with their column
 * indices is the CSR form of the next.gr "Block Sparse Attention Techniques"
 * tutorial, section 3.2.  Per-row counts, their prefix scan and the per-row
 * column lists follow from it; row_order adds the load-balance order, and the
 * pair sections the same lists for pairs of neighbouring block rows.
 *
 *   layout    device, int32 [H, Mb, Nb], read only
 *   dev_buf   device, caller-owned, >= bsa_plan_buffer_bytes(H, Mb, Nb) bytes,
 *             256-byte aligned; overwritten
 *   plan_out  host, filled on success
 * Errors: BSA_ERR_INVALID_ARG (null pointers, dims <= 0 or H*Mb*Nb >= 2^31),
 * BSA_ERR_MISALIGNED (dev_buf not 256-byte aligned), BSA_ERR_BUFFER_TOO_SMALL,
 * BSA_ERR_HIP.
 */
int bsa_plan(const int32_t *layout, int32_t H, int32_t Mb, int32_t Nb,
             void *dev_buf, size_t dev_bytes, bsa_plan_t *plan_out, void *stream);

/* Copy nnz_total of a built plan to the host; synchronises `stream`. */
int bsa_plan_nnz(const bsa_plan_t *plan, int64_t *nnz_host, void *stream);

/*
 * Block-sparse attention forward.
 *
 * Operation: for batch b, head h and query token i (query block m = i / bs),
 *   s_ij = scale * sum_d q[b,h,i,d] k[b,h,j,d]  over key tokens j of the live
 *          tiles (h, m, n) of the plan, -inf elsewhere;
 *   out[b,h,i,:] = sum_j softmax_j(s_i.) v[b,h,j,:];
 *   lse[b,h,i]   = log(sum_j exp(s_ij))  (natural log).
 * This is the scaled dot-product attention of the next.gr tutorial
 * (section 1) with the -inf masking of its Longformer formula, restricted to
 * the live tiles, each tile being a dense b x b piece of work (Language AI
 * Handbook, "Block Structure").  A row whose block row has no live tile gets
 * out = 0 and lse = -inf.  Tiles are computed with bf16 products and fp32
 * accumulation; fp32 inputs (BSA_F32) are rounded to bf16 (nearest-even) on
 * load and written back as fp32.
 *
 *   q     device [B, H, Sq, d] of dtype
 *   k, v  device [B, H, Sk, d] of dtype
 *   plan  host pointer to a plan built for this layout; H must equal plan->H,
 *         ceil(Sq / bs) must equal plan->Mb and ceil(Sk / bs) plan->Nb,
 *         otherwise the call returns BSA_ERR_PLAN_MISMATCH.  Lengths that are
 *         not multiples of bs cut the last block row / column at the sequence
 *         end (Language AI Handbook, create_block_sparse_mask): keys past Sk
 *         take no weight and rows past Sq are neither read nor written
 *   bs    block size: 16, 32, 64 or 128;   d: 32, 64 or 128
 *   scale finite and > 0 (the Python binding defaults it to 1/sqrt(d))
 *   out   device [B, H, Sq, d] of dtype, written
 *   lse   device fp32 [B, H, Sq], written; may be NULL
 * Errors: BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_MISALIGNED,
 * BSA_ERR_PLAN_MISMATCH, BSA_ERR_HIP.
 */
int bsa_forward(const void *q, const void *k, const void *v, const bsa_plan_t *plan,
                int32_t B, int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d,
                bsa_dtype_t dtype, float scale, void *out, float *lse, void *stream);

/* Options of bsa_forward_ex.  A zeroed struct (or a NULL pointer) gives the
 * plain bsa_forward. */
typedef struct {
  const float *attn_sink; /* device fp32 [H], 4-byte aligned, or NULL */
  float soft_cap;         /* > 0: tanh logit cap; 0: none */
  int32_t causal;         /* nonzero: also mask key token j > query token i */
  int32_t kv_heads;       /* K/V heads Hkv (H % Hkv == 0); 0 means H */
  const int32_t *q_segment_ids;  /* device int32 [B, Sq] or NULL (packed sequences) */
  const int32_t *kv_segment_ids; /* device int32 [B, Sk]; given iff q_segment_ids is */
} bsa_forward_opts_t;

/*
 * Block-sparse attention forward with the optional terms of the ejkernel
 * BlockSparseAttention operation ("ejkernel: BlockSparseAttention" page,
 * arguments softmax_aux, logits_soft_cap, causal and the key/value head
 * count).  With opts zeroed it computes exactly what bsa_forward computes.
 * Otherwise, in the notation of bsa_forward:
 *   soft_cap > 0:  s_ij <- soft_cap * tanh(s_ij / soft_cap), applied to the
 *                  scaled score before any masking (Gemma-2 style capping);
 *   causal:        s_ij = -inf also where j > i (token positions counted from
 *                  0 in both q and k), on top of the layout's mask;
 *   attn_sink:     the softmax denominator of head h also holds
 *                  exp(attn_sink[h]) (the sink logit is neither scaled nor
 *                  capped), so lse includes it and a row with no live key gets
 *                  out = 0 and lse = attn_sink[h];
 *   kv_heads:      k and v are [B, Hkv, Sk, d]; query head h reads K/V head
 *                  h / (H / Hkv) (grouped-query attention);
 *   segment ids:   (the operation's q_segment_ids / kv_segment_ids, for
 *                  several sequences packed into one) s_ij = -inf also where
 *                  q_segment_ids[b, i] != kv_segment_ids[b, j] (int32
 *                  arrays [B, Sq] and [B, Sk] in device memory).
 * Arguments, layouts and ownership as for bsa_forward; opts is a host pointer
 * read during the call.  Errors as for bsa_forward, plus BSA_ERR_INVALID_ARG
 * for kv_heads < 0 or not dividing H, a soft_cap that is negative or not
 * finite, or only one of the two segment-id arrays, and BSA_ERR_MISALIGNED
 * for an attn_sink or segment-id array not 4-byte aligned.
 */
int bsa_forward_ex(const void *q, const void *k, const void *v, const bsa_plan_t *plan,
                   int32_t B, int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d,
                   bsa_dtype_t dtype, float scale, const bsa_forward_opts_t *opts, void *out,
                   float *lse, void *stream);

/* Column plan of a layout, for the backward: per key block n of query head
 * h the live query blocks m, and the order of the key-block work items. */
typedef struct {
  int32_t H, Hkv, Mb, Nb;
  void *dev_buf;
  size_t dev_bytes;
} bsa_plan_cols_t;

/* Bytes a column-plan buffer needs (worst case: every tile live); 0 for bad
 * dimensions (non-positive, Hkv not dividing H, or H*Mb*Nb >= 2^31). */
size_t bsa_plan_cols_buffer_bytes(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb);

/* Byte offsets of the four column-plan sections (col_ptr, col_order,
 * nnz_total, row_idx).  Host-only. */
int bsa_plan_cols_sections(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, size_t offsets_out[4]);

/*
 * Build the column plan of a block layout: the transposed CSR the backward
 * walks to accumulate dK and dV of one key block (next.gr tutorial, section
 * 3.2 for the CSR form; "Gradient Propagation in Block Sparse Attention" for
 * gradients flowing through the live blocks only).
 *
 *   col_ptr   [H*Nb+1]: column c = h*Nb + n holds row_idx[col_ptr[c] ..
 *             col_ptr[c+1]), the live query blocks m in ascending order
 *   col_order [Hkv*Nb]: key-block work items kvh*Nb + n, K/V head by K/V
 *             head, each by its live tile count summed over the H/Hkv query
 *             heads of the group, descending, ties by n ascending
 *   layout    device, int32 [H, Mb, Nb], read only
 *   Hkv       K/V heads (0 means H); H % Hkv == 0 and (H/Hkv)*Mb <= 16384
 *   dev_buf   device, caller-owned, >= bsa_plan_cols_buffer_bytes bytes,
 *             256-byte aligned; overwritten
 * Errors: BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_MISALIGNED,
 * BSA_ERR_BUFFER_TOO_SMALL, BSA_ERR_HIP.
 */
int bsa_plan_cols(const int32_t *layout, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                  void *dev_buf, size_t dev_bytes, bsa_plan_cols_t *plan_out, void *stream);

/*
 * Consistency checks of plan contents.  The kernels take the plan's arrays
 * as the CSR lists of the live tiles (next.gr tutorial, section 3.2) and
 * index memory with them; a plan damaged after bsa_plan / bsa_plan_cols (or
 * written by other code) could send them outside their buffers.  Checked:
 *   plan:        row_ptr starts at 0, every row count in [0, Nb], row_ptr's
 *                last entry equals nnz_total; each row's col_idx strictly
 *                ascending in [0, Nb); row_order a permutation of [0, H*Mb);
 *                pair_info[1] in {0, 1}; pair_ptr as row_ptr with total
 *                pair_info[0]; every pair's entries equal the merged lists of
 *                its two rows with their row tags; pair_order a permutation
 *   column plan: the same for col_ptr / row_idx (values in [0, Mb)) and
 *                col_order a permutation of [0, Hkv*Nb)
 *   both:        equal nnz_total and every tile of the plan present in the
 *                column plan (one is the other's transpose)
 * Returns BSA_OK, BSA_ERR_BAD_PLAN with the first violation in
 * bsa_last_error(), or the argument errors of the calls that take plans.
 *
 * bsa_plan_check: the device plans (either may be NULL, not both), copied to
 *   the host after the work queued on `stream`; synchronises the stream.
 * bsa_plan_check_host: host copies of the plan buffers (plan_bytes /
 *   cols_bytes bytes, laid out as bsa_plan_sections /
 *   bsa_plan_cols_sections give; either may be NULL, not both) for the
 *   layout dimensions H, Hkv (0 means H), Mb, Nb.  Makes no HIP call.
 * bsa_set_debug: turns debug mode on (nonzero) or off for the process;
 *   returns the previous setting.
 */
int bsa_plan_check(const bsa_plan_t *plan, const bsa_plan_cols_t *plan_cols, void *stream);
int bsa_plan_check_host(const void *plan_host, size_t plan_bytes, const void *cols_host,
                        size_t cols_bytes, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb);
int bsa_set_debug(int on);

/* Bytes of the backward's workspace: two fp32 values per query row. */
size_t bsa_backward_workspace_bytes(int32_t B, int32_t H, int32_t Sq);

/*
 * Block-sparse attention backward: gradients of bsa_forward_ex's out.
 *
 * Operation: the chain rule of the forward, through the live tiles only
 * (next.gr tutorial, "Gradient Propagation in Block Sparse Attention", and
 * its block-structured Jacobian).  With c_ij the (capped) scaled score,
 * P_ij = exp(c_ij - lse_i) and D_i = dout_i . out_i:
 *   dv_j    = sum_i P_ij dout_i
 *   ds_ij   = P_ij (dout_i . v_j - D_i) * (1 - tanh^2(s_ij / cap)) (no factor
 *             without a cap)
 *   dq_i    = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i
 *   dsink_h = -sum over b, i of exp(sink_h - lse_i) D_i
 * Under grouped heads dk and dv of a K/V head sum over its query heads.
 * Masked entries (outside the layout, or above the diagonal with causal)
 * contribute nothing.
 *
 *   q, k, v, plan, B, H, Sq, Sk, bs, d, scale, opts: exactly as passed to
 *         the forward that produced out and lse (same options)
 *   out   device [B, H, Sq, d] of dtype, the forward's output
 *   dout  device [B, H, Sq, d] of dtype, upstream gradient
 *   lse   device fp32 [B, H, Sq], the forward's lse (required)
 *   plan_cols  host pointer to a column plan of the same layout with
 *         Hkv = the K/V head count (BSA_ERR_PLAN_MISMATCH otherwise)
 *   workspace  device, caller-owned, >= bsa_backward_workspace_bytes,
 *         16-byte aligned; overwritten (holds D and lse * log2 e)
 *   dq    device [B, H, Sq, d] of dtype, written
 *   dk, dv  device [B, Hkv, Sk, d] of dtype, written (every row)
 *   dsink device fp32 [H], written when opts->attn_sink is set; may be NULL
 * Supported: dtype BSA_BF16 or BSA_F32 (fp32 tiles are rounded to bf16 on
 * load, as in the forward; products accumulate in fp32), bs in {16, 32, 64, 128},
 * d in {32, 64, 128}.
 * Deterministic: no atomics, so repeated calls give identical bits.
 * Errors: as bsa_forward_ex, plus BSA_ERR_BUFFER_TOO_SMALL for a short
 * workspace.
 */
int bsa_backward(const void *q, const void *k, const void *v, const void *out, const void *dout,
                 const float *lse, const bsa_plan_t *plan, const bsa_plan_cols_t *plan_cols,
                 int32_t B, int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d,
                 bsa_dtype_t dtype, float scale, const bsa_forward_opts_t *opts, void *workspace,
                 size_t workspace_bytes, void *dq, void *dk, void *dv, float *dsink,
                 void *stream);

/* Query rows (B * H * Sq) bsa_backward_noalloc can serve: 2^21. */
size_t bsa_backward_noalloc_max_rows(void);

/*
 * bsa_backward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid hipMalloc.  It
 * computes exactly what bsa_backward computes, with the same kernels; the
 * per-row D and lse values go to a static device array of 16 MiB that the
 * library holds on each GPU it runs on until the process ends (looked up on
 * the first call made with that device current).  The caller still passes
 * every input and output, as for bsa_backward.
 *
 *   arguments  as bsa_backward, minus workspace and workspace_bytes
 *   limit      B * H * Sq <= bsa_backward_noalloc_max_rows() (2^21 rows);
 *              larger calls return BSA_ERR_UNSUPPORTED before any HIP call
 * Nothing in the array needs to start at zero: every value is written by the
 * call before it is read.  All calls on one GPU share its array, so calls that
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and give wrong gradients; calls ordered on one stream do not.
 * Errors: as bsa_backward, plus BSA_ERR_HIP when the array's address cannot be
 * obtained.
 */
int bsa_backward_noalloc(const void *q, const void *k, const void *v, const void *out,
                         const void *dout, const float *lse, const bsa_plan_t *plan,
                         const bsa_plan_cols_t *plan_cols, int32_t B, int32_t H, int32_t Sq,
                         int32_t Sk, int32_t bs, int32_t d, bsa_dtype_t dtype, float scale,
                         const bsa_forward_opts_t *opts, void *dq, void *dk, void *dv,
                         float *dsink, void *stream);

/* Bytes of the adaptive-layout workspace: (H*Mb + Hkv*Nb) * d floats. */
size_t bsa_layout_adaptive_workspace_bytes(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                                           int32_t d);

/*
 * Content-adaptive block layout of one batch item.
 *
 * Operation (next.gr tutorial, "Fixed vs. Adaptive Block Sparsity": a pair
 * is live when the similarity of its queries and keys reaches a threshold,
 * cosine similarity named as the metric; Language AI Handbook: blocks chosen
 * from similarity scores at a coarser granularity than tokens).  Each block
 * is represented by the mean of its rows:
 *   score(h, m, n)  = cos(mean q[h, m*bs .. m*bs+bs-1, :],
 *                         mean k[h / (H/Hkv), n*bs .. n*bs+bs-1, :])
 *                     (0 when either mean is the zero vector)
 *   layout[h][m][n] = score >= tau, then 0 where causal and n > m, then 1
 *                     where keep_diagonal and n == m
 * The layout feeds bsa_plan / bsa_plan_cols directly.
 *
 *   q     device [H, Sq, d], k device [Hkv, Sk, d] of dtype (one batch item)
 *   Hkv   0 means H; must divide H.  Sq, Sk multiples of bs; bs a multiple of
 *         16; d in {32, 64, 128}
 *   tau   finite threshold (cosine scale, [-1, 1] meaningful)
 *   workspace  device, caller-owned, >= bsa_layout_adaptive_workspace_bytes,
 *         16-byte aligned; overwritten (the unit block means)
 *   layout_out device int32 [H, Sq/bs, Sk/bs], written
 *   scores_out device fp32 [H, Sq/bs, Sk/bs] or NULL, written when given
 * Scores are fp32 sums in a fixed order, so repeated calls agree bit for
 * bit.  Errors: BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_MISALIGNED,
 * BSA_ERR_BUFFER_TOO_SMALL, BSA_ERR_HIP.
 */
int bsa_layout_adaptive(const void *q, const void *k, int32_t H, int32_t Hkv, int32_t Sq,
                        int32_t Sk, int32_t bs, int32_t d, bsa_dtype_t dtype, float tau,
                        int32_t causal, int32_t keep_diagonal, void *workspace,
                        size_t workspace_bytes, int32_t *layout_out, float *scores_out,
                        void *stream);

/*
 * Top-k gathered sparse attention forward with a per-head attention sink.
 *
 * Operation (DeepSeek-V4.1 "Sparse attention / Weighted row sum" page,
 * sparse_attn_kernel and sparse_attn): for batch b and query position m, the
 * valid slots t (idx[b,m,t] != -1) name rows of kv, the same rows for every
 * head; for head h
 *   s_t   = scale * q[b,m,h,:] . kv[b, idx[b,m,t], :]
 *   out   = sum_t exp(s_t) kv[b, idx_t, :] / (sum_t exp(s_t) + exp(sink_h))
 * The sink is an unscaled fp32 logit (NULL: no sink term).  A position with
 * no valid slot gets out = 0.  Indices outside [0, N) are treated like -1.
 *
 *   q     device bf16 [B, M, H, d];  kv device bf16 [B, N, d]
 *   idx   device int32 [B, M, topk]; attn_sink device fp32 [H] or NULL
 *   any H >= 1 (up to 64 * 65535; heads are served in groups of 64, each
 *   group gathering the position's rows once); d in {128, 256, 512};
 *   topk >= 1 (no alignment needed); one batch's kv (N * d * 2 bytes) at
 *   most 4 GiB - 1 KiB
 *   out   device bf16 [B, M, H, d], written
 * The sums run over the valid slots in a fixed order (with topk <= 2048,
 * grouped by range of kv rows, slot order within a range), so repeated
 * calls agree bit for bit; a reordered index list changes only rounding.
 * Errors: BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_MISALIGNED,
 * BSA_ERR_HIP.
 */
int topk_sparse_attn(const void *q, const void *kv, const int32_t *idx,
                     const float *attn_sink, int32_t B, int32_t M, int32_t N,
                     int32_t H, int32_t d, int32_t topk, float scale, void *out,
                     void *stream);

/* Static text for a status code. */
const char *bsa_status_string(int status);

/* Thread-local text describing the last failed call on this thread. */
const char *bsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H_ */
