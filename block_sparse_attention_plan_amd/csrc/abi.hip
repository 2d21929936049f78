// C ABI of libbsa: argument validation, error reporting and dispatch to the
// kernel launchers.  Every check here runs on the host before any HIP call.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "bsa.h"
#include "bsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char *where) {
  return fail(BSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The integer a caller passed as a bsa_dtype_t.  A C caller may pass any int;
// reading it through the enum type would be undefined for values outside the
// enumerators, so the bits are copied out instead.
int dtype_code(const bsa_dtype_t &d) {
  int v;
  static_assert(sizeof(v) == sizeof(d), "bsa_dtype_t is int-sized");
  std::memcpy(&v, &d, sizeof(v));
  return v;
}

// Blocks covering S tokens: the last one is cut where S is not a multiple.
int64_t blocks(int32_t S, int32_t bs) { return ((int64_t)S + bs - 1) / bs; }

int check_plan(const bsa_plan_t *plan, bsa::PlanGeometry *g) {
  if (plan == nullptr) return fail(BSA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->dev_buf == nullptr) return fail(BSA_ERR_INVALID_ARG, "plan has no buffer");
  if (!bsa::plan_geometry(plan->H, plan->Mb, plan->Nb, g))
    return fail(BSA_ERR_INVALID_ARG, "plan has invalid dimensions");
  if (plan->dev_bytes < g->total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "plan buffer is %zu bytes, needs %zu", plan->dev_bytes,
                g->total);
  return BSA_OK;
}

template <typename P>
P *at(void *base, size_t off) {
  return reinterpret_cast<P *>(static_cast<char *>(base) + off);
}

int check_plan_cols(const bsa_plan_cols_t *pc, bsa::PlanColsGeometry *g) {
  if (pc == nullptr) return fail(BSA_ERR_INVALID_ARG, "column plan is NULL");
  if (pc->dev_buf == nullptr) return fail(BSA_ERR_INVALID_ARG, "column plan has no buffer");
  if (!bsa::plan_cols_geometry(pc->H, pc->Hkv, pc->Mb, pc->Nb, g))
    return fail(BSA_ERR_INVALID_ARG, "column plan has invalid dimensions");
  if (pc->dev_bytes < g->total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "column plan buffer is %zu bytes, needs %zu",
                pc->dev_bytes, g->total);
  return BSA_OK;
}

// Debug mode (environment variable BSA_DEBUG set to anything but "" or "0",
// or bsa_set_debug): every call that reads a plan first copies it to the
// host and checks it, and refuses to launch on an inconsistent one.
std::atomic<int> g_debug{-1};   // -1: environment not read yet

bool debug_on() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char *e = std::getenv("BSA_DEBUG");
    int want = (e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0) ? 1 : 0;
    g_debug.compare_exchange_strong(v, want);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v != 0;
}

// `bytes` bytes of device memory into a host vector, after the work already
// queued on the stream.
int fetch(const void *dev, size_t bytes, std::vector<char> *host, hipStream_t stream,
          const char *who) {
  host->resize(bytes);
  hipError_t e = hipMemcpyAsync(host->data(), dev, bytes, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return BSA_OK;
}

// Checks host copies of a plan and/or a column plan (either may be NULL) and,
// given both, that one is the other's transpose.
int check_host_copies(const void *rows, size_t rows_bytes, const void *cols, size_t cols_bytes,
                      int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, const char *who) {
  char msg[320];
  if (rows != nullptr && !bsa::check_plan_host(rows, rows_bytes, H, Mb, Nb, msg, sizeof(msg)))
    return fail(BSA_ERR_BAD_PLAN, "%s: plan: %s", who, msg);
  if (cols != nullptr &&
      !bsa::check_plan_cols_host(cols, cols_bytes, H, Hkv, Mb, Nb, msg, sizeof(msg)))
    return fail(BSA_ERR_BAD_PLAN, "%s: column plan: %s", who, msg);
  if (rows != nullptr && cols != nullptr &&
      !bsa::check_transpose_host(rows, cols, H, Hkv, Mb, Nb, msg, sizeof(msg)))
    return fail(BSA_ERR_BAD_PLAN, "%s: plans disagree: %s", who, msg);
  return BSA_OK;
}

// The device-side plans (already validated as arguments) checked through
// host copies.
int check_device_plans(const bsa_plan_t *plan, const bsa_plan_cols_t *pc, void *stream,
                       const char *who) {
  std::vector<char> rows, cols;
  size_t rows_bytes = 0, cols_bytes = 0;
  int32_t H = 0, Hkv = 0, Mb = 0, Nb = 0;
  if (plan != nullptr) {
    bsa::PlanGeometry g;
    int st = check_plan(plan, &g);
    if (st != BSA_OK) return st;
    st = fetch(plan->dev_buf, g.total, &rows, (hipStream_t)stream, who);
    if (st != BSA_OK) return st;
    rows_bytes = g.total;
    H = plan->H; Mb = plan->Mb; Nb = plan->Nb; Hkv = H;
  }
  if (pc != nullptr) {
    bsa::PlanColsGeometry g;
    int st = check_plan_cols(pc, &g);
    if (st != BSA_OK) return st;
    if (plan != nullptr && (pc->H != H || pc->Mb != Mb || pc->Nb != Nb))
      return fail(BSA_ERR_PLAN_MISMATCH, "%s: the plans have different dimensions", who);
    st = fetch(pc->dev_buf, g.total, &cols, (hipStream_t)stream, who);
    if (st != BSA_OK) return st;
    cols_bytes = g.total;
    H = pc->H; Hkv = pc->Hkv; Mb = pc->Mb; Nb = pc->Nb;
  }
  return check_host_copies(plan != nullptr ? rows.data() : nullptr, rows_bytes,
                           pc != nullptr ? cols.data() : nullptr, cols_bytes, H, Hkv, Mb, Nb, who);
}

// Options of the forward (and of the backward, which must repeat them),
// validated and turned into kernel form.  `who` prefixes error messages.
int make_options(const bsa_forward_opts_t *opts, int32_t H, float scale, bsa::FwdOptions *fo,
                 const char *who) {
  *fo = bsa::FwdOptions{nullptr, 0.f, 0.f, 0, 1, 0, 0, nullptr, nullptr};
  if (opts == nullptr) return BSA_OK;
  const int32_t hkv = opts->kv_heads == 0 ? H : opts->kv_heads;
  if (hkv < 1 || H % hkv != 0)
    return fail(BSA_ERR_INVALID_ARG, "%s: kv_heads=%d must divide H=%d", who,
                (int)opts->kv_heads, (int)H);
  if (!(std::isfinite(opts->soft_cap) && opts->soft_cap >= 0.f))
    return fail(BSA_ERR_INVALID_ARG, "%s: soft_cap must be finite and >= 0", who);
  if (opts->attn_sink != nullptr && !aligned(opts->attn_sink, 4))
    return fail(BSA_ERR_MISALIGNED, "%s: attn_sink must be 4-byte aligned", who);
  fo->sink = opts->attn_sink;
  if (opts->soft_cap > 0.f) {
    // tanh(x) = 1 - 2 / (exp(2x) + 1) with x = scale * s / cap, evaluated
    // as exp2(s * cap_k); the kernel multiplies the result by cap_b and
    // later by scale, so that the capped score is cap * tanh(x).
    fo->cap_k = (float)(2.0 * (double)scale * 1.4426950408889634 / (double)opts->soft_cap);
    fo->cap_b = (float)((double)opts->soft_cap / (double)scale);
    if (!(std::isfinite(fo->cap_k) && std::isfinite(fo->cap_b) && fo->cap_b > 0.f))
      return fail(BSA_ERR_INVALID_ARG, "%s: soft_cap %g out of range for scale %g", who,
                  (double)opts->soft_cap, (double)scale);
  }
  fo->causal = opts->causal != 0;
  fo->kv_group = H / hkv;
  if ((opts->q_segment_ids == nullptr) != (opts->kv_segment_ids == nullptr))
    return fail(BSA_ERR_INVALID_ARG, "%s: segment ids come in pairs (queries and keys)", who);
  if ((opts->q_segment_ids != nullptr && !aligned(opts->q_segment_ids, 4)) ||
      (opts->kv_segment_ids != nullptr && !aligned(opts->kv_segment_ids, 4)))
    return fail(BSA_ERR_MISALIGNED, "%s: segment ids must be 4-byte aligned", who);
  fo->qseg = opts->q_segment_ids;
  fo->kseg = opts->kv_segment_ids;
  return BSA_OK;
}

}  // namespace

// Scratch of bsa_backward_noalloc: the D and lse*log2(e) values the backward
// keeps per query row, in a file-scope device array instead of a caller's
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
static constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // 2^21 query rows
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for later calls.
int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "bsa_backward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_backward_noalloc: device %d beyond %d", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "bsa_backward_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

// The backward behind both entry points.  With use_scratch the D / lse
// values go to the static scratch (workspace and workspace_bytes unused);
// otherwise to the caller's workspace.  Every check runs before any HIP call.
int backward_impl(const char *who, const void *q, const void *k, const void *v, const void *out,
                  const void *dout, const float *lse, const bsa_plan_t *plan,
                  const bsa_plan_cols_t *plan_cols, int32_t B, int32_t H, int32_t Sq, int32_t Sk,
                  int32_t bs, int32_t d, int dtype, float scale,
                  const bsa_forward_opts_t *opts, bool use_scratch, void *workspace,
                  size_t workspace_bytes, void *dq, void *dk, void *dv, float *dsink,
                  void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
      (!use_scratch && workspace == nullptr))
    return fail(BSA_ERR_INVALID_ARG, "%s: NULL tensor pointer", who);
  bsa::PlanGeometry g;
  int st = check_plan(plan, &g);
  if (st != BSA_OK) return st;
  bsa::PlanColsGeometry gc;
  st = check_plan_cols(plan_cols, &gc);
  if (st != BSA_OK) return st;
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0 || bs <= 0 || d <= 0)
    return fail(BSA_ERR_INVALID_ARG, "%s: sizes must be positive", who);
  if (H != plan->H || blocks(Sq, bs) != plan->Mb || blocks(Sk, bs) != plan->Nb)
    return fail(BSA_ERR_PLAN_MISMATCH,
                "%s: H=%d Sq=%d Sk=%d bs=%d do not match plan H=%d Mb=%d Nb=%d", who, H, Sq,
                Sk, bs, plan->H, plan->Mb, plan->Nb);
  if (dtype != BSA_BF16 && dtype != BSA_F32)
    return fail(BSA_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(BSA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", who);
  bsa::FwdOptions fo;
  st = make_options(opts, H, scale, &fo, who);
  if (st != BSA_OK) return st;
  fo.sq = Sq;
  fo.sk = Sk;
  if (plan_cols->H != H || plan_cols->Mb != plan->Mb || plan_cols->Nb != plan->Nb ||
      plan_cols->Hkv != H / fo.kv_group)
    return fail(BSA_ERR_PLAN_MISMATCH,
                "%s: column plan H=%d Hkv=%d Mb=%d Nb=%d does not match H=%d Hkv=%d "
                "Mb=%d Nb=%d", who, plan_cols->H, plan_cols->Hkv, plan_cols->Mb, plan_cols->Nb, H,
                H / fo.kv_group, plan->Mb, plan->Nb);
  if (!bsa::backward_supported(bs, d))
    return fail(BSA_ERR_UNSUPPORTED, "%s: no kernel for bs=%d d=%d", who, bs, d);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || (!use_scratch && !aligned(workspace, 16)) ||
      (dsink != nullptr && !aligned(dsink, 4)))
    return fail(BSA_ERR_MISALIGNED, "%s: tensors must be 16-byte aligned", who);
  const size_t ws = bsa_backward_workspace_bytes(B, H, Sq);
  if (use_scratch) {
    if (ws > kNoAllocScratchBytes)
      return fail(BSA_ERR_UNSUPPORTED,
                  "%s: B*H*Sq = %lld query rows need %zu bytes of scratch; the static scratch "
                  "holds %zu bytes (%zu rows)", who, (long long)B * H * Sq, ws,
                  kNoAllocScratchBytes, kNoAllocScratchBytes / (2 * sizeof(float)));
  } else if (workspace_bytes < ws) {
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "%s: workspace is %zu bytes, needs %zu", who,
                workspace_bytes, ws);
  }
  const int64_t work = (int64_t)B * H * plan->Mb;
  const int64_t rows = (int64_t)B * H * Sq;
  if (work > 0x7ffffff0LL || (int64_t)B * H * plan->Nb > 0x7ffffff0LL)
    return fail(BSA_ERR_UNSUPPORTED, "%s: problem too large", who);
  if (use_scratch) {
    st = scratch_address(&workspace);
    if (st != BSA_OK) return st;
  }
  if (debug_on()) {
    st = check_device_plans(plan, plan_cols, stream, who);
    if (st != BSA_OK) return st;
  }
  bsa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
  a.row_ptr = at<int32_t>(plan->dev_buf, g.off_row_ptr);
  a.col_idx = at<int32_t>(plan->dev_buf, g.off_col_idx);
  a.row_order = at<int32_t>(plan->dev_buf, g.off_row_order);
  a.col_ptr = at<int32_t>(plan_cols->dev_buf, gc.off_col_ptr);
  a.row_idx = at<int32_t>(plan_cols->dev_buf, gc.off_row_idx);
  a.col_order = at<int32_t>(plan_cols->dev_buf, gc.off_col_order);
  a.B = B; a.H = H; a.Mb = plan->Mb; a.Nb = plan->Nb; a.bs = bs; a.d = d;
  a.f32 = dtype == BSA_F32;
  a.scale = scale;
  a.opt = fo;
  a.Dv = static_cast<float *>(workspace);
  a.lse2 = static_cast<float *>(workspace) + rows;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsink = fo.sink != nullptr ? dsink : nullptr;
  hipError_t e = bsa::launch_backward(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return BSA_OK;
}

}  // namespace

extern "C" {

size_t bsa_plan_buffer_bytes(int32_t H, int32_t Mb, int32_t Nb) {
  bsa::PlanGeometry g;
  if (!bsa::plan_geometry(H, Mb, Nb, &g)) return 0;
  return g.total;
}

int bsa_plan_sections(int32_t H, int32_t Mb, int32_t Nb, size_t offsets_out[4]) {
  bsa::PlanGeometry g;
  if (offsets_out == nullptr) return fail(BSA_ERR_INVALID_ARG, "offsets_out is NULL");
  if (!bsa::plan_geometry(H, Mb, Nb, &g))
    return fail(BSA_ERR_INVALID_ARG, "invalid layout dimensions H=%d Mb=%d Nb=%d", H, Mb, Nb);
  offsets_out[0] = g.off_row_ptr;
  offsets_out[1] = g.off_row_order;
  offsets_out[2] = g.off_nnz;
  offsets_out[3] = g.off_col_idx;
  return BSA_OK;
}

int bsa_plan_pair_sections(int32_t H, int32_t Mb, int32_t Nb, size_t offsets_out[4]) {
  bsa::PlanGeometry g;
  if (offsets_out == nullptr) return fail(BSA_ERR_INVALID_ARG, "offsets_out is NULL");
  if (!bsa::plan_geometry(H, Mb, Nb, &g))
    return fail(BSA_ERR_INVALID_ARG, "invalid layout dimensions H=%d Mb=%d Nb=%d", H, Mb, Nb);
  offsets_out[0] = g.off_pair_ptr;
  offsets_out[1] = g.off_pair_order;
  offsets_out[2] = g.off_pair_info;
  offsets_out[3] = g.off_pair_cols;
  return BSA_OK;
}

int bsa_plan(const int32_t *layout, int32_t H, int32_t Mb, int32_t Nb, void *dev_buf,
             size_t dev_bytes, bsa_plan_t *plan_out, void *stream) {
  if (layout == nullptr || dev_buf == nullptr || plan_out == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan: NULL pointer argument");
  bsa::PlanGeometry g;
  if (!bsa::plan_geometry(H, Mb, Nb, &g))
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan: invalid dimensions H=%d Mb=%d Nb=%d", H, Mb, Nb);
  if (Nb > bsa::kPlanMaxNb)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_plan: Nb=%d exceeds %d", Nb, bsa::kPlanMaxNb);
  if (!aligned(dev_buf, 256)) return fail(BSA_ERR_MISALIGNED, "bsa_plan: buffer not 256-byte aligned");
  if (dev_bytes < g.total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "bsa_plan: buffer is %zu bytes, needs %zu", dev_bytes,
                g.total);
  hipError_t e = bsa::launch_plan(layout, H, Mb, Nb, at<int32_t>(dev_buf, g.off_row_ptr),
                                  at<int32_t>(dev_buf, g.off_row_order),
                                  at<int32_t>(dev_buf, g.off_nnz),
                                  at<int32_t>(dev_buf, g.off_col_idx),
                                  at<int32_t>(dev_buf, g.off_pair_ptr),
                                  at<int32_t>(dev_buf, g.off_pair_order),
                                  at<int32_t>(dev_buf, g.off_pair_info),
                                  at<int32_t>(dev_buf, g.off_pair_cols), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_plan launch");
  plan_out->H = H;
  plan_out->Mb = Mb;
  plan_out->Nb = Nb;
  plan_out->reserved = 0;
  plan_out->dev_buf = dev_buf;
  plan_out->dev_bytes = dev_bytes;
  return BSA_OK;
}

int bsa_plan_nnz(const bsa_plan_t *plan, int64_t *nnz_host, void *stream) {
  bsa::PlanGeometry g;
  int st = check_plan(plan, &g);
  if (st != BSA_OK) return st;
  if (nnz_host == nullptr) return fail(BSA_ERR_INVALID_ARG, "bsa_plan_nnz: nnz_host is NULL");
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, at<int32_t>(plan->dev_buf, g.off_nnz), sizeof(v),
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_plan_nnz copy");
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_plan_nnz sync");
  *nnz_host = v;
  return BSA_OK;
}

}  // extern "C"

namespace {

// The forward behind bsa_forward and bsa_forward_ex (dtype as the caller's int).
int forward_impl(const void *q, const void *k, const void *v, const bsa_plan_t *plan, int32_t B,
                 int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d, int dtype, float scale,
                 const bsa_forward_opts_t *opts, void *out, float *lse, void *stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_forward: NULL tensor pointer");
  bsa::PlanGeometry g;
  int st = check_plan(plan, &g);
  if (st != BSA_OK) return st;
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk <= 0 || bs <= 0 || d <= 0)
    return fail(BSA_ERR_INVALID_ARG, "bsa_forward: sizes must be positive");
  if (H != plan->H || blocks(Sq, bs) != plan->Mb || blocks(Sk, bs) != plan->Nb)
    return fail(BSA_ERR_PLAN_MISMATCH,
                "bsa_forward: H=%d Sq=%d Sk=%d bs=%d do not match plan H=%d Mb=%d Nb=%d", H, Sq,
                Sk, bs, plan->H, plan->Mb, plan->Nb);
  if (dtype != BSA_BF16 && dtype != BSA_F32)
    return fail(BSA_ERR_INVALID_ARG, "bsa_forward: unknown dtype %d", dtype);
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(BSA_ERR_INVALID_ARG, "bsa_forward: scale must be finite and > 0");
  if (!bsa::forward_supported(bs, d))
    return fail(BSA_ERR_UNSUPPORTED, "bsa_forward: no kernel for bs=%d d=%d", bs, d);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse != nullptr && !aligned(lse, 4)))
    return fail(BSA_ERR_MISALIGNED, "bsa_forward: tensors must be 16-byte aligned");
  const int64_t work = (int64_t)B * plan->H * plan->Mb;
  if (work > 0x7ffffff0LL) return fail(BSA_ERR_UNSUPPORTED, "bsa_forward: problem too large");
  bsa::FwdOptions fo;
  st = make_options(opts, H, scale, &fo, "bsa_forward");
  if (st != BSA_OK) return st;
  fo.sq = Sq;
  fo.sk = Sk;
  if (debug_on()) {
    st = check_device_plans(plan, nullptr, stream, "bsa_forward");
    if (st != BSA_OK) return st;
  }
  const bsa::PlanArrays pa{at<int32_t>(plan->dev_buf, g.off_row_ptr),
                           at<int32_t>(plan->dev_buf, g.off_col_idx),
                           at<int32_t>(plan->dev_buf, g.off_row_order),
                           at<int32_t>(plan->dev_buf, g.off_pair_ptr),
                           at<int32_t>(plan->dev_buf, g.off_pair_cols),
                           at<int32_t>(plan->dev_buf, g.off_pair_order),
                           at<int32_t>(plan->dev_buf, g.off_pair_info)};
  hipError_t e = bsa::launch_forward(q, k, v, pa, B, plan->H, plan->Mb, plan->Nb, bs, d,
                                     dtype == BSA_F32, scale, fo, out, lse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_forward launch");
  return BSA_OK;
}

}  // namespace

extern "C" {

int bsa_forward_ex(const void *q, const void *k, const void *v, const bsa_plan_t *plan,
                   int32_t B, int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d,
                   bsa_dtype_t dtype, float scale, const bsa_forward_opts_t *opts, void *out,
                   float *lse, void *stream) {
  return forward_impl(q, k, v, plan, B, H, Sq, Sk, bs, d, dtype_code(dtype), scale, opts, out,
                      lse, stream);
}

int bsa_forward(const void *q, const void *k, const void *v, const bsa_plan_t *plan, int32_t B,
                int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d, bsa_dtype_t dtype,
                float scale, void *out, float *lse, void *stream) {
  return forward_impl(q, k, v, plan, B, H, Sq, Sk, bs, d, dtype_code(dtype), scale, nullptr, out,
                      lse, stream);
}

size_t bsa_plan_cols_buffer_bytes(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb) {
  bsa::PlanColsGeometry g;
  if (!bsa::plan_cols_geometry(H, Hkv, Mb, Nb, &g)) return 0;
  return g.total;
}

int bsa_plan_cols_sections(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, size_t offsets_out[4]) {
  bsa::PlanColsGeometry g;
  if (offsets_out == nullptr) return fail(BSA_ERR_INVALID_ARG, "offsets_out is NULL");
  if (!bsa::plan_cols_geometry(H, Hkv, Mb, Nb, &g))
    return fail(BSA_ERR_INVALID_ARG, "invalid dimensions H=%d Hkv=%d Mb=%d Nb=%d", H, Hkv, Mb,
                Nb);
  offsets_out[0] = g.off_col_ptr;
  offsets_out[1] = g.off_col_order;
  offsets_out[2] = g.off_nnz;
  offsets_out[3] = g.off_row_idx;
  return BSA_OK;
}

int bsa_plan_cols(const int32_t *layout, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                  void *dev_buf, size_t dev_bytes, bsa_plan_cols_t *plan_out, void *stream) {
  if (layout == nullptr || dev_buf == nullptr || plan_out == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_cols: NULL pointer argument");
  if (Hkv == 0) Hkv = H;
  bsa::PlanColsGeometry g;
  if (!bsa::plan_cols_geometry(H, Hkv, Mb, Nb, &g))
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_cols: invalid dimensions H=%d Hkv=%d Mb=%d Nb=%d",
                H, Hkv, Mb, Nb);
  if ((int64_t)(H / Hkv) * Mb > bsa::kPlanMaxNb)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_plan_cols: (H/Hkv)*Mb=%lld exceeds %d",
                (long long)(H / Hkv) * Mb, bsa::kPlanMaxNb);
  if (!aligned(dev_buf, 256))
    return fail(BSA_ERR_MISALIGNED, "bsa_plan_cols: buffer not 256-byte aligned");
  if (dev_bytes < g.total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "bsa_plan_cols: buffer is %zu bytes, needs %zu",
                dev_bytes, g.total);
  hipError_t e = bsa::launch_plan_cols(layout, H, Hkv, Mb, Nb, at<int32_t>(dev_buf, g.off_col_ptr),
                                       at<int32_t>(dev_buf, g.off_col_order),
                                       at<int32_t>(dev_buf, g.off_nnz),
                                       at<int32_t>(dev_buf, g.off_row_idx), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_plan_cols launch");
  plan_out->H = H;
  plan_out->Hkv = Hkv;
  plan_out->Mb = Mb;
  plan_out->Nb = Nb;
  plan_out->dev_buf = dev_buf;
  plan_out->dev_bytes = dev_bytes;
  return BSA_OK;
}

size_t bsa_backward_workspace_bytes(int32_t B, int32_t H, int32_t Sq) {
  if (B <= 0 || H <= 0 || Sq <= 0) return 0;
  return (size_t)2 * B * H * Sq * sizeof(float);
}

int bsa_backward(const void *q, const void *k, const void *v, const void *out, const void *dout,
                 const float *lse, const bsa_plan_t *plan, const bsa_plan_cols_t *plan_cols,
                 int32_t B, int32_t H, int32_t Sq, int32_t Sk, int32_t bs, int32_t d,
                 bsa_dtype_t dtype, float scale, const bsa_forward_opts_t *opts, void *workspace,
                 size_t workspace_bytes, void *dq, void *dk, void *dv, float *dsink,
                 void *stream) {
  return backward_impl("bsa_backward", q, k, v, out, dout, lse, plan, plan_cols, B, H, Sq, Sk,
                       bs, d, dtype_code(dtype), scale, opts, false, workspace, workspace_bytes,
                       dq, dk, dv, dsink, stream);
}

size_t bsa_backward_noalloc_max_rows(void) { return kNoAllocScratchBytes / (2 * sizeof(float)); }

int bsa_backward_noalloc(const void *q, const void *k, const void *v, const void *out,
                         const void *dout, const float *lse, const bsa_plan_t *plan,
                         const bsa_plan_cols_t *plan_cols, int32_t B, int32_t H, int32_t Sq,
                         int32_t Sk, int32_t bs, int32_t d, bsa_dtype_t dtype, float scale,
                         const bsa_forward_opts_t *opts, void *dq, void *dk, void *dv,
                         float *dsink, void *stream) {
  return backward_impl("bsa_backward_noalloc", q, k, v, out, dout, lse, plan, plan_cols, B, H,
                       Sq, Sk, bs, d, dtype_code(dtype), scale, opts, true, nullptr, 0, dq, dk,
                       dv, dsink, stream);
}

size_t bsa_layout_adaptive_workspace_bytes(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                                           int32_t d) {
  if (H <= 0 || Hkv <= 0 || Mb <= 0 || Nb <= 0 || d <= 0) return 0;
  return ((size_t)H * Mb + (size_t)Hkv * Nb) * (size_t)d * sizeof(float);
}

int bsa_layout_adaptive(const void *q, const void *k, int32_t H, int32_t Hkv, int32_t Sq,
                        int32_t Sk, int32_t bs, int32_t d, bsa_dtype_t dtype, float tau,
                        int32_t causal, int32_t keep_diagonal, void *workspace,
                        size_t workspace_bytes, int32_t *layout_out, float *scores_out,
                        void *stream) {
  if (q == nullptr || k == nullptr || workspace == nullptr || layout_out == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: NULL pointer argument");
  if (H <= 0 || Sq <= 0 || Sk <= 0 || bs <= 0 || d <= 0)
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: sizes must be positive");
  if (Hkv == 0) Hkv = H;
  if (Hkv < 1 || H % Hkv != 0)
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: Hkv=%d must divide H=%d", Hkv, H);
  if (Sq % bs != 0 || Sk % bs != 0)
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: Sq=%d and Sk=%d must be multiples of "
                "bs=%d", Sq, Sk, bs);
  const int dt = dtype_code(dtype);
  if (dt != BSA_BF16 && dt != BSA_F32)
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: unknown dtype %d", dt);
  if (!std::isfinite(tau))
    return fail(BSA_ERR_INVALID_ARG, "bsa_layout_adaptive: tau must be finite");
  if (!bsa::adaptive_supported(bs, d))
    return fail(BSA_ERR_UNSUPPORTED, "bsa_layout_adaptive: no kernel for bs=%d d=%d", bs, d);
  const int32_t Mb = Sq / bs, Nb = Sk / bs;
  if ((int64_t)H * Mb * Nb >= (int64_t(1) << 31) || (int64_t)H * Mb + (int64_t)Hkv * Nb >= (1 << 30))
    return fail(BSA_ERR_UNSUPPORTED, "bsa_layout_adaptive: problem too large");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(workspace, 16) || !aligned(layout_out, 4) ||
      (scores_out != nullptr && !aligned(scores_out, 4)))
    return fail(BSA_ERR_MISALIGNED, "bsa_layout_adaptive: misaligned pointer");
  const size_t ws = bsa_layout_adaptive_workspace_bytes(H, Hkv, Mb, Nb, d);
  if (workspace_bytes < ws)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "bsa_layout_adaptive: workspace is %zu bytes, needs %zu",
                workspace_bytes, ws);
  hipError_t e = bsa::launch_adaptive(q, k, H, Hkv, Mb, Nb, bs, d, dt == BSA_F32, tau,
                                      causal != 0, keep_diagonal != 0,
                                      static_cast<float *>(workspace), layout_out, scores_out,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_layout_adaptive launch");
  return BSA_OK;
}

int topk_sparse_attn(const void *q, const void *kv, const int32_t *idx, const float *attn_sink,
                     int32_t B, int32_t M, int32_t N, int32_t H, int32_t d, int32_t topk,
                     float scale, void *out, void *stream) {
  if (q == nullptr || kv == nullptr || idx == nullptr || out == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "topk_sparse_attn: NULL tensor pointer");
  if (B <= 0 || M <= 0 || N <= 0 || H <= 0 || d <= 0 || topk <= 0)
    return fail(BSA_ERR_INVALID_ARG, "topk_sparse_attn: sizes must be positive");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(BSA_ERR_INVALID_ARG, "topk_sparse_attn: scale must be finite and > 0");
  if (!bsa::topk_supported(H, d))
    return fail(BSA_ERR_UNSUPPORTED, "topk_sparse_attn: no kernel for H=%d d=%d", H, d);
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      (attn_sink != nullptr && !aligned(attn_sink, 4)))
    return fail(BSA_ERR_MISALIGNED, "topk_sparse_attn: tensors must be 16-byte aligned");
  if ((int64_t)B * M > 0x7fffffffLL || ((int64_t)H + 63) / 64 > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "topk_sparse_attn: problem too large");
  if ((int64_t)N * d * 2 > 0xfffffc00LL)  // the kernel's row offsets wrap past this for -1
    return fail(BSA_ERR_UNSUPPORTED, "topk_sparse_attn: one batch of kv exceeds 4 GiB - 1 KiB");
  hipError_t e = bsa::launch_topk(q, kv, idx, attn_sink, B, M, N, H, d, topk, scale, out,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "topk_sparse_attn launch");
  return BSA_OK;
}

int bsa_set_debug(int on) {
  const int prev = debug_on() ? 1 : 0;
  g_debug.store(on != 0 ? 1 : 0);
  return prev;
}

int bsa_plan_check(const bsa_plan_t *plan, const bsa_plan_cols_t *plan_cols, void *stream) {
  if (plan == nullptr && plan_cols == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_check: no plan given");
  return check_device_plans(plan, plan_cols, stream, "bsa_plan_check");
}

int bsa_plan_check_host(const void *plan_host, size_t plan_bytes, const void *cols_host,
                        size_t cols_bytes, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb) {
  if (plan_host == nullptr && cols_host == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_check_host: no plan given");
  if (Hkv == 0) Hkv = H;
  if (H <= 0 || Hkv <= 0 || Mb <= 0 || Nb <= 0 || H % Hkv != 0)
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_check_host: invalid dimensions H=%d Hkv=%d Mb=%d Nb=%d",
                H, Hkv, Mb, Nb);
  bsa::PlanGeometry g;
  bsa::PlanColsGeometry gc;
  if (!bsa::plan_geometry(H, Mb, Nb, &g) || !bsa::plan_cols_geometry(H, Hkv, Mb, Nb, &gc))
    return fail(BSA_ERR_INVALID_ARG, "bsa_plan_check_host: invalid dimensions");
  if (plan_host != nullptr && plan_bytes < g.total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL, "bsa_plan_check_host: plan copy is %zu bytes, needs %zu",
                plan_bytes, g.total);
  if (cols_host != nullptr && cols_bytes < gc.total)
    return fail(BSA_ERR_BUFFER_TOO_SMALL,
                "bsa_plan_check_host: column plan copy is %zu bytes, needs %zu", cols_bytes,
                gc.total);
  return check_host_copies(plan_host, plan_bytes, cols_host, cols_bytes, H, Hkv, Mb, Nb,
                           "bsa_plan_check_host");
}

const char *bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BSA_ERR_MISALIGNED: return "misaligned pointer";
    case BSA_ERR_PLAN_MISMATCH: return "plan does not match the call";
    case BSA_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case BSA_ERR_HIP: return "HIP runtime error";
    case BSA_ERR_BAD_PLAN: return "inconsistent plan contents";
    default: return "unknown status";
  }
}

const char *bsa_last_error(void) { return g_last_error; }

}  // extern "C"
