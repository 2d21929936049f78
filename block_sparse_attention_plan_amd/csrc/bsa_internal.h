// Host-side interfaces between the C ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsa {

// Plan buffer geometry: byte offsets of row_ptr, row_order, nnz_total,
// col_idx, then of the pair sections pair_ptr, pair_order, pair_info
// (pair_total, use_pairs) and pair_cols, and the total size.  All sections
// start on 256-byte boundaries.
struct PlanGeometry {
  size_t off_row_ptr, off_row_order, off_nnz, off_col_idx;
  size_t off_pair_ptr, off_pair_order, off_pair_info, off_pair_cols;
  size_t total;
};
bool plan_geometry(int32_t H, int32_t Mb, int32_t Nb, PlanGeometry *g);

// Largest Nb the planner handles (its per-head count histogram lives in LDS).
constexpr int32_t kPlanMaxNb = 16384;

hipError_t launch_plan(const int32_t *layout, int32_t H, int32_t Mb, int32_t Nb,
                       int32_t *row_ptr, int32_t *row_order, int32_t *nnz_total,
                       int32_t *col_idx, int32_t *pair_ptr, int32_t *pair_order,
                       int32_t *pair_info, int32_t *pair_cols, hipStream_t stream);

// Per-call options of the forward kernels (already validated).
struct FwdOptions {
  const float *sink;  // [H] per-head sink logits, or nullptr
  float cap_k;        // 2*scale*log2(e)/cap for the tanh logit cap, 0 without one
  float cap_b;        // cap/scale
  int32_t causal;     // nonzero: key token j > query token i is masked too
  int32_t kv_group;   // query heads per K/V head (1 without grouping)
  int32_t sq, sk;     // sequence lengths; the last block is cut where they are
                      // not multiples of the block size
  const int32_t *qseg;  // [B, sq] segment ids of the queries, or nullptr
  const int32_t *kseg;  // [B, sk] segment ids of the keys (set with qseg)
};

// The plan's device arrays as the forward reads them: the rows, and the pairs
// of neighbouring rows with their use flag (pair_info[1]).
struct PlanArrays {
  const int32_t *row_ptr, *col_idx, *row_order;
  const int32_t *pair_ptr, *pair_cols, *pair_order, *pair_info;
};

// Returns hipErrorInvalidValue when no kernel instance matches (bs, d, f32).
hipError_t launch_forward(const void *q, const void *k, const void *v, const PlanArrays &plan,
                          int32_t B, int32_t H, int32_t Mb, int32_t Nb, int32_t bs, int32_t d,
                          bool f32, float scale, const FwdOptions &opt, void *out, float *lse,
                          hipStream_t stream);
bool forward_supported(int32_t bs, int32_t d);

// Column plan (backward): byte offsets of col_ptr, col_order, nnz_total,
// row_idx and the total size, all sections 256-byte aligned.
struct PlanColsGeometry {
  size_t off_col_ptr, off_col_order, off_nnz, off_row_idx, total;
};
bool plan_cols_geometry(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, PlanColsGeometry *g);
hipError_t launch_plan_cols(const int32_t *layout, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                            int32_t *col_ptr, int32_t *col_order, int32_t *nnz_total,
                            int32_t *row_idx, hipStream_t stream);

// Host-side consistency checks of plans copied to host memory (buf holds
// `bytes` bytes laid out as the plan buffer).  Each returns false with the
// first violation described in msg; the transpose check assumes both plans
// passed their own check.
bool check_plan_host(const void *buf, size_t bytes, int32_t H, int32_t Mb, int32_t Nb, char *msg,
                     size_t mlen);
bool check_plan_cols_host(const void *buf, size_t bytes, int32_t H, int32_t Hkv, int32_t Mb,
                          int32_t Nb, char *msg, size_t mlen);
bool check_transpose_host(const void *rows, const void *cols, int32_t H, int32_t Hkv, int32_t Mb,
                          int32_t Nb, char *msg, size_t mlen);

// Everything the backward launchers need (already validated).
struct BwdArgs {
  const void *q, *k, *v, *out, *dout;
  const float *lse;                                    // forward lse (natural log)
  const int32_t *row_ptr, *col_idx, *row_order;        // row plan
  const int32_t *col_ptr, *row_idx, *col_order;        // column plan
  int32_t B, H, Mb, Nb, bs, d;
  bool f32;                                            // fp32 I/O (bf16 products)
  float scale;
  FwdOptions opt;
  float *Dv, *lse2;                                    // workspace, B*H*Mb*bs floats each
  void *dq, *dk, *dv;
  float *dsink;                                        // [H] or nullptr
};
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
bool backward_supported(int32_t bs, int32_t d);

// Content-adaptive layout of one batch item; unit = workspace of
// (H*Mb + Hkv*Nb)*d floats; scores may be nullptr.
hipError_t launch_adaptive(const void *q, const void *k, int32_t H, int32_t Hkv, int32_t Mb,
                           int32_t Nb, int32_t bs, int32_t d, bool f32, float tau, int32_t causal,
                           int32_t keep_diagonal, float *unit, int32_t *layout, float *scores,
                           hipStream_t stream);
bool adaptive_supported(int32_t bs, int32_t d);

hipError_t launch_topk(const void *q, const void *kv, const int32_t *idx,
                       const float *sink, int32_t B, int32_t M, int32_t N, int32_t H,
                       int32_t d, int32_t topk, float scale, void *out,
                       hipStream_t stream);
bool topk_supported(int32_t H, int32_t d);

}  // namespace bsa
