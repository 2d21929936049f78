// Top-k gathered sparse attention forward with a per-head attention sink
// (gfx950).
//
// Semantics follow the DeepSeek-V4.1 "Sparse attention / Weighted row sum"
// page (sparse_attn_kernel): for each (batch, query position) the listed KV
// rows are gathered -- the same rows serve every head, only the queries
// differ -- the scaled scores of all gathered rows share one softmax whose
// denominator also holds exp(sink_h), and the output is the weighted sum of
// the same rows.  Slots holding -1 (and, for memory safety, any index outside
// [0, N)) contribute nothing; the running maximum starts at a finite floor so
// a position without a valid slot produces zeros instead of NaN.
//
// Work item = (batch, position); one workgroup of four waves.  Wave w owns
// heads 16w .. 16w+15.  Slots are processed in chunks of 64: each wave
// gathers 16 of the chunk's rows (one 1 KiB row per wave instruction) into a
// register prefetch buffer one chunk ahead; the chunk is then staged
// row-major in LDS and every wave computes
//   S^T = KV Q^T       (16x16x32 MFMA, Q^T resident in registers)
//   online softmax     (lane owns one head column)
//   O^T += KV^T P^T    (16x16x32 MFMA, KV^T by LDS transpose reads)
// so the one gather serves all heads of the position.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxFloor = -1e30f;

template <int D>
__global__ void __launch_bounds__(256)
topk_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv,
            const int32_t *__restrict__ idx, const float *__restrict__ sink, int32_t M,
            int32_t N, int32_t H, int32_t topk, float scale_log2, __bf16 *__restrict__ out) {
  constexpr int T = 64;               // slots per chunk
  constexpr int STR = D + 16;         // LDS row stride (elements)
  constexpr int RPW = T / 4;          // rows gathered per wave per chunk
  constexpr int LPR = D / 8;          // lanes per row (16-byte pieces)
  constexpr int RPI = 64 / LPR;       // rows per wave instruction
  constexpr int CPT = RPW / RPI;      // 16-byte pieces per thread per chunk
  constexpr int QC = D / 32;
  constexpr int DT = D / 16;
  static_assert(LPR <= 64 && 64 % LPR == 0 && RPW % RPI == 0, "row split");

  __shared__ __attribute__((aligned(16))) __bf16 KVs[T * STR];

  const int64_t pos = blockIdx.x;  // b * M + m
  const int64_t b = pos / M;
  const int tid = threadIdx.x, wid = tid / 64, lane = tid % 64;
  const int G = lane / 16, li = lane % 16;
  const int h = 16 * wid + li;
  const bool wave_active = 16 * wid < H;

  const __bf16 *kvb = kv + b * (int64_t)N * D;
  const int32_t *ib = idx + pos * (int64_t)topk;

  // Q^T fragments for this lane's head (zero for heads >= H).
  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    if (h < H)
      qf[c] = *reinterpret_cast<const bf16x8 *>(q + (pos * H + h) * (int64_t)D + 32 * c + 8 * G);
    else
      qf[c] = bf16x8{};
  }

  // Gather of one chunk into registers: wave wid fetches rows wid*RPW ..
  // (wid+1)*RPW-1 of the chunk; invalid slots load zeros.
  bf16x8 gr[CPT];
  uint64_t vmask_next = 0;
  auto gather = [&](int t0) -> uint64_t {
    const int slot = t0 + lane;
    int my = -1;
    if (slot < topk) my = ib[slot];
    const bool valid = slot < topk && my >= 0 && my < N;
    const uint64_t vm = __ballot(valid);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int row = wid * RPW + c * RPI + lane / LPR;
      const int src = __shfl(my, row, 64);
      const bool ok = (vm >> row) & 1ull;
      if (ok)
        gr[c] = *reinterpret_cast<const bf16x8 *>(kvb + (int64_t)src * D + (lane % LPR) * 8);
      else
        gr[c] = bf16x8{};
    }
    return vm;
  };
  auto stage = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int row = wid * RPW + c * RPI + lane / LPR;
      *reinterpret_cast<bf16x8 *>(&KVs[row * STR + (lane % LPR) * 8]) = gr[c];
    }
  };

  float m_run = kMaxFloor, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (topk + T - 1) / T;
  vmask_next = gather(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    const uint64_t vmask = vmask_next;
    __syncthreads();
    stage();
    __syncthreads();
    if (ch + 1 < nchunks) vmask_next = gather((ch + 1) * T);
    if (!wave_active) continue;

    f32x4 s[T / 16];
#pragma unroll
    for (int jt = 0; jt < T / 16; ++jt) {
      s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&KVs[(16 * jt + li) * STR + 32 * c + 8 * G]);
        s[jt] = mfma16(a, qf[c], s[jt]);
      }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < T / 16; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * G + e;
        if (!((vmask >> j) & 1ull)) s[jt][e] = -__builtin_inff();
        mx = fmaxf(mx, s[jt][e]);
      }
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < T / 16; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[jt][e], scale_log2, -m_new));
        s[jt][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;

    bf16x8 pf[T / 32];
#pragma unroll
    for (int kc = 0; kc < T / 32; ++kc)
      pf[kc] = to_bf16x8(s[2 * kc][0], s[2 * kc][1], s[2 * kc][2], s[2 * kc][3],
                         s[2 * kc + 1][0], s[2 * kc + 1][1], s[2 * kc + 1][2], s[2 * kc + 1][3]);
    const int e_src = li / 4, c_src = li % 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kc = 0; kc < T / 32; ++kc) {
        const __bf16 *src = &KVs[(32 * kc + 4 * G + e_src) * STR + 16 * dt + 4 * c_src];
        const bf16x8 a = cat4(lds_read_tr4(src), lds_read_tr4(src + 16 * STR));
        acc[dt] = mfma16(a, pf[kc], acc[dt]);
      }
  }
  if (!wave_active) return;

  float l_tot = sum_xor32(sum_xor16(l_run));
  if (sink != nullptr && h < H) l_tot += fast_exp2(fmaf(sink[h], kLog2e, -m_run));
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (h < H) {
    __bf16 *oh = out + (pos * H + h) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 x = acc[dt] * inv;
      bf16x4 r4;
      r4[0] = (__bf16)x[0]; r4[1] = (__bf16)x[1]; r4[2] = (__bf16)x[2]; r4[3] = (__bf16)x[3];
      *reinterpret_cast<bf16x4 *>(oh + 16 * dt + 4 * G) = r4;
    }
  }
}

}  // namespace

bool topk_supported(int32_t H, int32_t d) { return H >= 1 && H <= 64 && d == 512; }

hipError_t launch_topk(const void *q, const void *kv, const int32_t *idx, const float *sink,
                       int32_t B, int32_t M, int32_t N, int32_t H, int32_t d, int32_t topk,
                       float scale, void *out, hipStream_t stream) {
  if (!topk_supported(H, d)) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)B * M;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel<512>, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const __bf16 *)q, (const __bf16 *)kv, idx, sink, M, N, H, topk,
                     scale * kLog2e, (__bf16 *)out);
  return hipGetLastError();
}

}  // namespace bsa
