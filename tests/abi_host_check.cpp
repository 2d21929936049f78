// Host-side checks of the C ABI for a sanitizer build: every call below
// returns from argument validation before any HIP call, so the program needs
// no GPU.  Built with AddressSanitizer and UndefinedBehaviorSanitizer against
// the host-sanitized libbsa.so (tests/test_sanitized_host.py); a memory error
// or undefined behaviour in the validation, geometry or error-reporting code
// aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>
#include <limits>

#include "bsa.h"

static int g_failed = 0;

#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failed;                                                         \
    }                                                                     \
  } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

static bsa_plan_t plan_of(int32_t H, int32_t Mb, int32_t Nb, uintptr_t buf, size_t bytes) {
  bsa_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.H = H;
  p.Mb = Mb;
  p.Nb = Nb;
  p.dev_buf = fake(buf);
  p.dev_bytes = bytes;
  return p;
}

static void plan_checks() {
  CHECK(bsa_plan_buffer_bytes(0, 4, 4) == 0);
  CHECK(bsa_plan_buffer_bytes(1 << 11, 1 << 10, 1 << 10) == 0);
  const size_t n = bsa_plan_buffer_bytes(2, 4, 4);
  CHECK(n > 0 && n % 256 == 0);
  size_t offs[4], pairs[4];
  CHECK(bsa_plan_sections(32, 256, 256, offs) == BSA_OK);
  CHECK(bsa_plan_pair_sections(32, 256, 256, pairs) == BSA_OK);
  CHECK(offs[0] == 0 && offs[3] > offs[2] && pairs[0] > offs[3] && pairs[3] > pairs[2]);
  CHECK(bsa_plan_buffer_bytes(32, 256, 256) >= pairs[3] + (size_t)32 * 128 * 256 * 4);
  CHECK(bsa_plan_sections(2, 0, 4, offs) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_plan_pair_sections(2, 4, 4, nullptr) == BSA_ERR_INVALID_ARG);
  bsa_plan_t out;
  const int32_t *lay = static_cast<const int32_t *>(fake(0x10000));
  CHECK(bsa_plan(nullptr, 2, 4, 4, fake(0x10000), n, &out, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_plan(lay, 2, 4, 4, nullptr, n, &out, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_plan(lay, 2, 4, 4, fake(0x10000), n, nullptr, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_plan(lay, 0, 4, 4, fake(0x10000), n, &out, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_plan(lay, 2, 4, 20000, fake(0x10000), (size_t)1 << 30, &out, nullptr) ==
        BSA_ERR_UNSUPPORTED);
  CHECK(bsa_plan(lay, 2, 4, 4, fake(0x10010), n, &out, nullptr) == BSA_ERR_MISALIGNED);
  CHECK(bsa_plan(lay, 2, 4, 4, fake(0x10000), n - 1, &out, nullptr) == BSA_ERR_BUFFER_TOO_SMALL);
  CHECK(std::strstr(bsa_last_error(), "buffer") != nullptr);
  int64_t nnz = 0;
  CHECK(bsa_plan_nnz(nullptr, &nnz, nullptr) == BSA_ERR_INVALID_ARG);
}

static void forward_checks() {
  const size_t n = bsa_plan_buffer_bytes(2, 4, 4);
  bsa_plan_t p = plan_of(2, 4, 4, 0x100000, n);
  void *f = fake(0x10000);
  auto call = [&](const void *q, const bsa_plan_t *pl, int32_t B, int32_t H, int32_t Sq,
                  int32_t Sk, int32_t bs, int32_t d, int dtype, float scale, float *lse) {
    return bsa_forward(q, f, f, pl, B, H, Sq, Sk, bs, d, (bsa_dtype_t)dtype, scale, f, lse,
                       nullptr);
  };
  CHECK(call(nullptr, &p, 1, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, nullptr, 1, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, &p, 0, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, &p, 1, 3, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_PLAN_MISMATCH);
  CHECK(call(f, &p, 1, 2, 128, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_PLAN_MISMATCH);
  CHECK(call(f, &p, 1, 2, 64, 64, 16, 32, 0, 0.f, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, &p, 1, 2, 64, 64, 16, 32, 0, std::numeric_limits<float>::quiet_NaN(), nullptr) ==
        BSA_ERR_INVALID_ARG);
  CHECK(call(f, &p, 1, 2, 64, 64, 16, 32, 7, 0.5f, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, &p, 1, 2, 64, 64, 16, 48, 0, 0.5f, nullptr) == BSA_ERR_UNSUPPORTED);
  CHECK(call(f, &p, 1, 2, 32, 32, 8, 32, 0, 0.5f, nullptr) == BSA_ERR_UNSUPPORTED);
  CHECK(call(fake(0x10008), &p, 1, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_MISALIGNED);
  CHECK(call(f, &p, 1, 2, 64, 64, 16, 32, 0, 0.5f, static_cast<float *>(fake(0x10002))) ==
        BSA_ERR_MISALIGNED);
  bsa_plan_t small = plan_of(2, 4, 4, 0x100000, 64);
  CHECK(call(f, &small, 1, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_BUFFER_TOO_SMALL);
  bsa_plan_t nobuf = plan_of(2, 4, 4, 0, n);
  CHECK(call(f, &nobuf, 1, 2, 64, 64, 16, 32, 0, 0.5f, nullptr) == BSA_ERR_INVALID_ARG);
  // options
  bsa_forward_opts_t o;
  std::memset(&o, 0, sizeof(o));
  auto callx = [&](const bsa_forward_opts_t *opts, int32_t H) {
    return bsa_forward_ex(f, f, f, &p, 1, H, 64, 64, 16, 32, BSA_BF16, 0.5f, opts, f, nullptr,
                          nullptr);
  };
  o.kv_heads = 3;
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.kv_heads = -1;
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.kv_heads = 0;
  o.soft_cap = -1.f;
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.soft_cap = std::numeric_limits<float>::infinity();
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.soft_cap = 1e-44f;
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.soft_cap = 0.f;
  o.attn_sink = static_cast<const float *>(fake(0x10002));
  CHECK(callx(&o, 2) == BSA_ERR_MISALIGNED);
  o.attn_sink = nullptr;
  o.q_segment_ids = static_cast<const int32_t *>(fake(0x10000));
  CHECK(callx(&o, 2) == BSA_ERR_INVALID_ARG);
  o.kv_segment_ids = static_cast<const int32_t *>(fake(0x10002));
  CHECK(callx(&o, 2) == BSA_ERR_MISALIGNED);
}

static void backward_checks() {
  const size_t n = bsa_plan_buffer_bytes(2, 4, 4);
  bsa_plan_t p = plan_of(2, 4, 4, 0x100000, n);
  bsa_plan_cols_t pc;
  std::memset(&pc, 0, sizeof(pc));
  pc.H = 2;
  pc.Hkv = 2;
  pc.Mb = 4;
  pc.Nb = 4;
  pc.dev_buf = fake(0x200000);
  pc.dev_bytes = bsa_plan_cols_buffer_bytes(2, 2, 4, 4);
  void *f = fake(0x10000);
  const float *lse = static_cast<const float *>(f);
  CHECK(bsa_backward_workspace_bytes(1, 2, 64) == 2u * 2 * 64 * 4);
  CHECK(bsa_backward(f, f, f, f, f, lse, &p, &pc, 1, 2, 64, 64, 16, 32, BSA_BF16, 0.5f, nullptr,
                     nullptr, 0, f, f, f, nullptr, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_backward(f, f, f, f, f, lse, &p, &pc, 1, 2, 64, 64, 16, 32, BSA_BF16, 0.5f, nullptr,
                     f, 16, f, f, f, nullptr, nullptr) == BSA_ERR_BUFFER_TOO_SMALL);
  pc.Hkv = 1;
  CHECK(bsa_backward(f, f, f, f, f, lse, &p, &pc, 1, 2, 64, 64, 16, 32, BSA_BF16, 0.5f, nullptr,
                     f, 1 << 20, f, f, f, nullptr, nullptr) != BSA_OK);
  pc.Hkv = 2;
  // the no-allocation form: same checks, and a limit of 2^21 query rows
  CHECK(bsa_backward_noalloc_max_rows() == (size_t)1 << 21);
  CHECK(bsa_backward_noalloc(f, f, f, f, f, lse, &p, &pc, 1, 2, 64, 64, 16, 32, BSA_BF16, 0.5f,
                             nullptr, nullptr, f, f, nullptr, nullptr) == BSA_ERR_INVALID_ARG);
  CHECK(bsa_backward_noalloc(f, f, f, f, f, lse, &p, &pc, 1, 2, 64, 64, 16, 48, BSA_BF16, 0.5f,
                             nullptr, f, f, f, nullptr, nullptr) == BSA_ERR_UNSUPPORTED);
  const int32_t nb = 8;  // 65 batch items x 32 heads x 1024 tokens = 2^21 + 2^15 rows
  bsa_plan_t pb = plan_of(32, nb, nb, 0x100000, bsa_plan_buffer_bytes(32, nb, nb));
  bsa_plan_cols_t pcb = pc;
  pcb.H = pcb.Hkv = 32;
  pcb.Mb = pcb.Nb = nb;
  pcb.dev_bytes = bsa_plan_cols_buffer_bytes(32, 32, nb, nb);
  CHECK(bsa_backward_noalloc(f, f, f, f, f, lse, &pb, &pcb, 65, 32, 1024, 1024, 128, 128,
                             BSA_BF16, 0.5f, nullptr, f, f, f, nullptr, nullptr) ==
        BSA_ERR_UNSUPPORTED);
  CHECK(std::strstr(bsa_last_error(), "static scratch") != nullptr);
}

static void topk_checks() {
  void *f = fake(0x10000);
  const int32_t *idx = static_cast<const int32_t *>(f);
  auto call = [&](const void *q, const float *sink, int32_t N, int32_t H, int32_t d,
                  int32_t topk, float scale) {
    return topk_sparse_attn(q, f, idx, sink, 1, 4, N, H, d, topk, scale, f, nullptr);
  };
  CHECK(call(nullptr, nullptr, 16, 8, 512, 8, 0.1f) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, nullptr, 16, 8, 512, 0, 0.1f) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, nullptr, -1, 8, 512, 8, 0.1f) == BSA_ERR_INVALID_ARG);
  CHECK(call(f, nullptr, 16, 8, 512, 8, std::numeric_limits<float>::infinity()) ==
        BSA_ERR_INVALID_ARG);
  CHECK(call(f, nullptr, 16, 64 * 65535 + 1, 512, 8, 0.1f) == BSA_ERR_UNSUPPORTED);
  CHECK(call(f, nullptr, 16, 8, 192, 8, 0.1f) == BSA_ERR_UNSUPPORTED);
  CHECK(call(f, static_cast<const float *>(fake(0x10001)), 16, 8, 512, 8, 0.1f) ==
        BSA_ERR_MISALIGNED);
  CHECK(call(f, nullptr, 1 << 22, 8, 512, 8, 0.1f) == BSA_ERR_UNSUPPORTED);
}

// The host plan checks read every section of a copied plan through counts
// and offsets taken from that same copy: over buffers of garbage they must
// report an inconsistency and stay inside the buffer.
static void plan_content_checks() {
  uint32_t x = 12345u;
  auto next = [&x]() {  // xorshift32
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  };
  const int dims[][4] = {{1, 1, 1, 1}, {2, 5, 7, 1}, {3, 8, 4, 3}, {4, 3, 9, 2}};
  for (const auto &d : dims) {
    const int H = d[0], Mb = d[1], Nb = d[2], Hkv = d[3];
    std::vector<int32_t> rows(bsa_plan_buffer_bytes(H, Mb, Nb) / 4);
    std::vector<int32_t> cols(bsa_plan_cols_buffer_bytes(H, Hkv, Mb, Nb) / 4);
    for (int trial = 0; trial < 50; ++trial) {
      for (auto &v : rows) v = (int32_t)(next() % 64) - 8;   // mostly small values
      for (auto &v : cols) v = (trial % 2) ? (int32_t)next() : (int32_t)(next() % 16);
      const int st = bsa_plan_check_host(rows.data(), rows.size() * 4, cols.data(),
                                         cols.size() * 4, H, Hkv, Mb, Nb);
      CHECK(st == BSA_ERR_BAD_PLAN || st == BSA_OK);
      CHECK(bsa_plan_check_host(nullptr, 0, cols.data(), cols.size() * 4, H, Hkv, Mb, Nb) <= 0);
    }
    // The empty layout's plan: all counts zero, identity orders.
    std::fill(rows.begin(), rows.end(), 0);
    std::fill(cols.begin(), cols.end(), 0);
    size_t ro[4], pr[4], co[4];
    CHECK(bsa_plan_sections(H, Mb, Nb, ro) == BSA_OK);
    CHECK(bsa_plan_pair_sections(H, Mb, Nb, pr) == BSA_OK);
    CHECK(bsa_plan_cols_sections(H, Hkv, Mb, Nb, co) == BSA_OK);
    for (int i = 0; i < H * Mb; ++i) rows[ro[1] / 4 + i] = i;
    for (int i = 0; i < H * ((Mb + 1) / 2); ++i) rows[pr[1] / 4 + i] = i;
    for (int i = 0; i < Hkv * Nb; ++i) cols[co[1] / 4 + i] = i;
    CHECK(bsa_plan_check_host(rows.data(), rows.size() * 4, cols.data(), cols.size() * 4, H, Hkv,
                              Mb, Nb) == BSA_OK);
    CHECK(bsa_plan_check_host(rows.data(), rows.size() * 4 - 4, nullptr, 0, H, Hkv, Mb, Nb) ==
          BSA_ERR_BUFFER_TOO_SMALL);
  }
  CHECK(bsa_plan_check(nullptr, nullptr, nullptr) == BSA_ERR_INVALID_ARG);
}

static void status_checks() {
  for (int code = 1; code >= -8; --code) CHECK(bsa_status_string(code) != nullptr);
  CHECK(bsa_last_error() != nullptr);
}

int main() {
  plan_checks();
  forward_checks();
  backward_checks();
  topk_checks();
  plan_content_checks();
  status_checks();
  if (g_failed) {
    std::fprintf(stderr, "%d checks failed\n", g_failed);
    return 1;
  }
  std::printf("abi host checks ok\n");
  return 0;
}
