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
// Work item = (batch, position); one workgroup of four waves, wave w owning
// heads 16w .. 16w+15 over all of d.  Slots are processed in chunks of 32
// whose rows are copied straight from HBM into LDS (at d = 512 one
// buffer_load_dwordx4 ... lds per 1 KiB row; at d = 128 and 256 one or two
// buffer_load_dword ... lds of 256 bytes, so that every row keeps its
// padding; slots without a valid index get a zero row), one chunk ahead into
// the other of two buffers, so the one gather serves all heads of the
// position.  The page's kernel takes d as a parameter; d_h = 512 is the size
// its shapes show.  Every wave computes
//   S^T = KV Q^T       (16x16x32 MFMA, Q^T resident in registers)
//   online softmax     (lane owns one head column; the running maximum may
//                      lag the true one by a bounded amount before the
//                      accumulator is rescaled)
//   O^T += KV^T P^T    (16x16x32 MFMA, KV^T by LDS transpose reads)
// The two buffers (2 x 33 KiB with rows padded by 32 bytes against bank
// conflicts) let two workgroups share a CU, so each SIMD interleaves the
// waves of two positions.  The buffers are distinct LDS objects and the
// chunk loop is unrolled by two, so the compiler never waits for a copy
// into the buffer it is not reading.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxFloor = -1e30f;
constexpr float kLazy = 8.0f;  // tolerated staleness of the running max (log2 units)
constexpr int kReadAheadS = 6;   // KV row reads issued before the first score MFMA
constexpr int kReadAheadV = 12;  // KV transpose reads issued before the first PV MFMA

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
topk_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv,
            const int32_t *__restrict__ idx, const float *__restrict__ sink, int32_t M,
            int32_t N, int32_t H, int32_t topk, float scale_log2, __bf16 *__restrict__ out) {
  constexpr int T = 32;               // slots per chunk
  constexpr int STR = D + 16;         // LDS row stride (elements)
  constexpr int RPW = T / 4;          // rows gathered per wave per chunk
  constexpr int QC = D / 32;          // 32-wide k steps of S^T
  constexpr int DT = D / 16;          // 16-wide d tiles of O^T
  static_assert(D == 512 || D == 256 || D == 128, "row copies: one 1 KiB or D/128 256-byte pieces");

  __shared__ __attribute__((aligned(16))) __bf16 C0[T * STR];
  __shared__ __attribute__((aligned(16))) __bf16 C1[T * STR];

  const int64_t pos = blockIdx.x;  // b * M + m
  const int64_t b = pos / M;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, kept in SGPRs
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

  // Lane j < 32 loads slot j of chunk ch (-1 past the end); `valid` maps an
  // entry to its row, or to -1 when it names no row.  The two are kept apart
  // so that the load of a later chunk's indices is not waited for (which
  // would also wait for the row copies issued before it) until it is used.
  auto chunk_idx = [&](int ch) -> int {
    const int slot = ch * T + lane;
    return (lane < T && slot < topk) ? ib[slot] : -1;
  };
  auto valid = [&](int my) -> int { return (my >= 0 && my < N) ? my : -1; };
  // Copy rows wid*RPW .. wid*RPW+RPW-1 of a chunk into `dst`.
  const __amdgpu_buffer_rsrc_t kv_rs = make_rsrc(kvb, (uint32_t)((int64_t)N * D * 2));
  auto gather = [&](int my, __bf16 *dst) {
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int row = wid * RPW + j;
      const int src = __builtin_amdgcn_readlane(my, row);
      if (src >= 0) {
        if constexpr (D == 512) {
          copy16_to_lds(kv_rs, dst + row * STR, (uint32_t)(lane * 16), (uint32_t)src * (uint32_t)(D * 2));
        } else {
#pragma unroll
          for (int p = 0; p < D / 128; ++p)
            copy4_to_lds(kv_rs, dst + row * STR + 128 * p, (uint32_t)(lane * 4 + 256 * p),
                         (uint32_t)src * (uint32_t)(D * 2));
        }
      } else if (lane < D / 8) {
        *reinterpret_cast<bf16x8 *>(dst + row * STR + lane * 8) = bf16x8{};
      }
    }
  };

  float m_run = kMaxFloor, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int e_src = li / 4, c_src = li % 4;
  auto compute = [&](const __bf16 *kb, uint64_t vmask) {
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + (16 * jt + li) * STR + 32 * c + 8 * G);
        s[jt] = mfma16(a, qf[c], s[jt]);
      }
    sched_interleave<2 * QC, 2 * QC, kReadAheadS, 0>();
    float mx = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * G + e;
        if (!((vmask >> j) & 1ull)) s[jt][e] = -__builtin_inff();
        mx = fmaxf(mx, s[jt][e]);
      }
    mx = max_xor32(max_xor16(mx)) * scale_log2;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[jt][e], scale_log2, -m_run));
        s[jt][e] = p;
        psum += p;
      }
    l_run += psum;
    // k order of P^T: slots 4G+e (e < 4) then 16+4G+e, matching the rows of
    // the two transpose reads below.
    const bf16x8 pf = to_bf16x8(s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]);
    const __bf16 *rows = kb + (4 * G + e_src) * STR + 4 * c_src;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8 a = cat4(lds_read_tr4(rows + 16 * dt), lds_read_tr4(rows + 16 * STR + 16 * dt));
      acc[dt] = mfma16(a, pf, acc[dt]);
    }
    sched_interleave<DT, 2 * DT, kReadAheadV, 0>();
  };
  // my_cur: validated rows of chunk ch; raw_next: unvalidated entries of
  // chunk ch + 1.
  auto step = [&](int ch, int nchunks, int &my_cur, int &raw_next, const __bf16 *cur, __bf16 *nxt) {
    const uint64_t vmask = __ballot(my_cur >= 0);
    int my_following = -1;
    if (ch + 1 < nchunks) {
      my_following = valid(raw_next);
      gather(my_following, nxt);
      if (ch + 2 < nchunks) raw_next = chunk_idx(ch + 2);
    }
    if (wave_active && vmask != 0) compute(cur, vmask);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next chunk visible; this chunk's buffer free
    my_cur = my_following;
  };

  const int nchunks = (topk + T - 1) / T;
  int my_cur = valid(chunk_idx(0));
  gather(my_cur, C0);
  int my_next = nchunks > 1 ? chunk_idx(1) : -1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ch += 2) {
    step(ch, nchunks, my_cur, my_next, C0, C1);
    if (ch + 1 < nchunks) step(ch + 1, nchunks, my_cur, my_next, C1, C0);
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

bool topk_supported(int32_t H, int32_t d) {
  return H >= 1 && H <= 64 && (d == 128 || d == 256 || d == 512);
}

hipError_t launch_topk(const void *q, const void *kv, const int32_t *idx, const float *sink,
                       int32_t B, int32_t M, int32_t N, int32_t H, int32_t d, int32_t topk,
                       float scale, void *out, hipStream_t stream) {
  if (!topk_supported(H, d)) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)B * M;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
#define BSA_TOPK_LAUNCH(D_)                                                                    \
  hipLaunchKernelGGL(topk_kernel<D_>, dim3((unsigned)grid), dim3(256), 0, stream,              \
                     (const __bf16 *)q, (const __bf16 *)kv, idx, sink, M, N, H, topk,           \
                     scale * kLog2e, (__bf16 *)out)
  if (d == 512) BSA_TOPK_LAUNCH(512);
  else if (d == 256) BSA_TOPK_LAUNCH(256);
  else BSA_TOPK_LAUNCH(128);
#undef BSA_TOPK_LAUNCH
  return hipGetLastError();
}

}  // namespace bsa
