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
// Work item = (batch, position); one workgroup of four waves.  With topk up
// to 2048 the position's valid indices are first compacted into an LDS list,
// grouped by table range (slot order within a range), so that slots holding
// -1 cost nothing and the workgroups on an XCD gather from one range of the
// table at a time; longer lists are read in place.  Slots (list entries) are processed in chunks of 32 whose
// rows are copied straight from HBM into LDS
// (at d = 512 one buffer_load_dwordx4 ... lds per 1 KiB row; at d = 128 and
// 256 one or two buffer_load_dword ... lds of 256 bytes, so that every row
// keeps its padding; a slot without a valid index reads as a zero row), one
// chunk ahead into the other of two buffers, so the one gather serves all
// heads of the position.  The page's kernel takes d as a parameter; d_h = 512
// is the size its shapes show.  Wave w
//   forms S^T = KV Q^T for heads 16w .. 16w+15 over all of d (16x16x32 MFMA,
//     Q^T resident in registers) and their online softmax (a lane owns one
//     head column; the running maximum may lag the true one by a bounded
//     amount before the output is rescaled), writing the bf16 weights P and
//     each head's rescale factor to LDS;
//   after a block barrier, accumulates O^T += KV^T P^T for d columns
//     w*d/4 .. (w+1)*d/4 - 1 of all 64 heads (32x32x16 MFMA, KV^T by LDS
//     transpose reads of its quarter of the chunk only).
// A workgroup serves 64 heads; with more heads the grid's second dimension
// runs over groups of 64 (heads 64g .. 64g+63), each gathering the
// position's rows for its own heads.
// Splitting the output product over d rather than heads transposes each
// gathered element once per workgroup instead of once per wave; the LDS
// transpose reads were what bounded the head-split form.  The two chunk
// buffers (2 x 33 KiB, rows padded by 32 bytes against bank conflicts) plus
// P (5 KiB) and the index list (8 KiB) let two workgroups share a CU, so
// each SIMD interleaves the waves of two positions.  The buffers are
// distinct LDS objects and the chunk loop is unrolled by two, so the
// compiler never waits for a copy into the buffer it is not reading.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxFloor = -1e30f;
constexpr float kLazy = 8.0f;  // tolerated staleness of the running max (log2 units)
// KV row reads issued before the first score MFMA
template <int D> constexpr int kReadAheadS = D == 512 ? 6 : 3;
// Largest topk whose valid indices are compacted into LDS (4 bytes each)
constexpr int kWindow = 2048;
// The compacted list groups the valid indices by index range (in slot order
// within a range): a range spans 2^shift table rows, about 2 MiB at this d,
// at most kMaxRanges ranges (wider ones for larger tables).  Workgroups that
// run together then gather from the same range at the same time, which
// stays in an XCD's 4 MB L2, instead of from the whole table.
template <int D> constexpr int kRangeShift = D == 512 ? 11 : D == 256 ? 12 : 13;
constexpr int kMaxRanges = 8;

template <int D, bool COMPACT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
topk_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kv,
            const int32_t *__restrict__ idx, const float *__restrict__ sink, int32_t M,
            int32_t N, int32_t H, int32_t topk, float scale_log2,
            __bf16 *__restrict__ out) {
  constexpr int T = 32;               // slots per chunk
  constexpr int STR = D + 16;         // LDS row stride (elements)
  constexpr int RPW = T / 4;          // rows gathered per wave per chunk
  constexpr int QC = D / 32;          // 32-wide k steps of S^T
  constexpr int DW = D / 4;           // output columns per wave
  constexpr int DTW = DW / 32;        // 32-wide d tiles per wave
  constexpr int PSTR = T + 8;         // row stride of P (elements per head)
  static_assert(D == 512 || D == 256 || D == 128, "row copies: one 1 KiB or D/128 256-byte pieces");
  static_assert(DTW >= 1, "each wave owns at least one 32-wide d tile");

  __shared__ __attribute__((aligned(16))) __bf16 C0[T * STR];
  __shared__ __attribute__((aligned(16))) __bf16 C1[T * STR];
  __shared__ __attribute__((aligned(16))) __bf16 Ps[64 * PSTR];  // P of every head, [head][slot]
  __shared__ float As[64];  // per-head rescale factor of the chunk; 1/l at the end
  // COMPACT instances (topk <= kWindow): the valid indices of the slots, in
  // slot order; chunks take T of them at a time, so slots without a valid
  // index cost no products.  (The other instances read the slots in place.)
  __shared__ __attribute__((aligned(16))) int32_t LST[COMPACT ? kWindow : 1];
  __shared__ int32_t WCNT[4 * kMaxRanges];  // [range][wave] counts

  const int64_t pos = blockIdx.x;  // b * M + m
  const int64_t b = pos / M;
  const int hb = 64 * blockIdx.y;  // first head of this workgroup's group
  const int tid = threadIdx.x, lane = tid % 64;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, kept in SGPRs
  const int G = lane / 16, li = lane % 16;
  const int h2 = lane / 32, l32 = lane % 32;
  const int h = 16 * wid + li;          // head inside the group (LDS rows of P, factors)
  const int hg = hb + h;                // head index in q, out and sink
  const bool wave_active = hb + 16 * wid < H;
  const int d0 = wid * DW;

  const __bf16 *kvb = kv + b * (int64_t)N * D;
  const int32_t *ib = idx + pos * (int64_t)topk;

  // P rows of heads no wave writes stay zero, their factors one.
  for (int i = tid; i < 64 * PSTR / 8; i += 256) *reinterpret_cast<bf16x8 *>(Ps + 8 * i) = bf16x8{};
  if (tid < 64) As[tid] = 1.f;

  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    if (hg < H)
      qf[c] = *reinterpret_cast<const bf16x8 *>(q + (pos * H + hg) * (int64_t)D + 32 * c + 8 * G);
    else
      qf[c] = bf16x8{};
  }

  auto valid = [&](int my) -> int { return (my >= 0 && my < N) ? my : -1; };
  // COMPACT: slots [w0, w1) (at most kWindow): each wave takes a quarter of
  // them, 64 per load.  Per index range, the waves' counts give each wave
  // its offset in LST, after the earlier ranges; ballots with mbcnt give
  // each lane its place, so the list is the same on every run.  Returns the
  // number of valid indices.
  int rshift = kRangeShift<D>;
  while (((N - 1) >> rshift) >= kMaxRanges) ++rshift;
  const int nranges = N > 0 ? ((N - 1) >> rshift) + 1 : 1;
  auto compact_window = [&](int w0, int w1) -> int {
    constexpr int PERW = kWindow / 4 / 64;
    int raw[PERW], rng[PERW];  // index; its range, -1 for an invalid slot
#pragma unroll
    for (int j = 0; j < PERW; ++j) {
      const int slot = w0 + (wid * PERW + j) * 64 + lane;
      raw[j] = slot < w1 ? ib[slot] : -1;
    }
#pragma unroll
    for (int j = 0; j < PERW; ++j) rng[j] = (raw[j] >= 0 && raw[j] < N) ? raw[j] >> rshift : -1;
    for (int r = 0; r < nranges; ++r) {
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < PERW; ++j) cnt += __popcll(__ballot(rng[j] == r));
      if (lane == 0) WCNT[4 * r + wid] = cnt;
    }
    __syncthreads();
    int tot = 0;
    for (int r = 0; r < nranges; ++r) {
      int off = tot;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c = WCNT[4 * r + w];
        off += w < wid ? c : 0;
        tot += c;
      }
#pragma unroll
      for (int j = 0; j < PERW; ++j) {
        const uint64_t vm = __ballot(rng[j] == r);
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(vm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)vm, 0u));
        if (rng[j] == r) LST[off + below] = raw[j];
        off += __popcll(vm);
      }
    }
    __syncthreads();
    return tot;
  };
  const __amdgpu_buffer_rsrc_t kv_rs = make_rsrc(kvb, (uint32_t)((int64_t)N * D * 2));
  // The row offset rides in the per-lane offset, which is what the buffer
  // range check covers: an invalid slot (-1) wraps it past the end of the
  // table (the caller keeps N*d*2 <= 2^32 - 1024), so its row reads as zeros.
  auto gather = [&](int my, __bf16 *dst) {
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int row = wid * RPW + j;
      const uint32_t roff = (uint32_t)__builtin_amdgcn_readlane(my, row) * (uint32_t)(D * 2);
      if constexpr (D == 512) {
        copy16_to_lds(kv_rs, dst + row * STR, roff + (uint32_t)(lane * 16), 0u);
      } else {
#pragma unroll
        for (int p = 0; p < D / 128; ++p)
          copy4_to_lds(kv_rs, dst + row * STR + 128 * p, roff + (uint32_t)(lane * 4 + 256 * p), 0u);
      }
    }
  };

  float m_run = kMaxFloor, l_run = 0.f;
  f32x16 o[DTW][2];
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) o[dt][0] = o[dt][1] = f32x16{};

  // Scores and softmax of this wave's 16 heads; P (bf16) and the rescale
  // factor go to LDS.  P is stored per head in the k order of the output
  // product: within each 16-slot block, slot 4a' + e (a' = 0..3) sits at
  // 8 * (a' % 2) + 4 * (a' / 2) + e.
  auto scores = [&](const __bf16 *kb, uint64_t vmask) {
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + (16 * jt + li) * STR + 32 * c + 8 * G);
        s[jt] = mfma16(a, qf[c], s[jt]);
      }
    sched_interleave<2 * QC, 2 * QC, kReadAheadS<D>, 0>();
    // validity of this lane's slots 4G + e (bits 0..3) and 16 + 4G + e (bits 16..19)
    const uint32_t vbits = (uint32_t)(vmask >> (4 * G));
    float mx = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!((vbits >> (16 * jt + e)) & 1u)) s[jt][e] = -__builtin_inff();
        mx = fmaxf(mx, s[jt][e]);
      }
    mx = max_xor32(max_xor16(mx)) * scale_log2;
    float alpha = 1.f;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(fmaf(s[jt][e], scale_log2, -m_run));
        psum += p[e];
      }
      bf16x4 p4;
      p4[0] = (__bf16)p[0]; p4[1] = (__bf16)p[1]; p4[2] = (__bf16)p[2]; p4[3] = (__bf16)p[3];
      *reinterpret_cast<bf16x4 *>(Ps + h * PSTR + 16 * jt + 8 * (G % 2) + 4 * (G / 2)) = p4;
    }
    l_run += psum;
    if (G == 0) As[h] = alpha;
  };
  // O^T[d0 .. d0+DW) x 64 heads += KV^T P^T for one chunk.
  const int e_src = li / 4, c_src = li % 4;
  auto outprod = [&](const __bf16 *kb) {
    const float a0 = As[l32], a1 = As[32 + l32];
    if (__any(a0 != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) o[dt][0] *= a0;
    }
    if (__any(a1 != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) o[dt][1] *= a1;
    }
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const bf16x8 p0 = *reinterpret_cast<const bf16x8 *>(Ps + l32 * PSTR + 16 * kq + 8 * h2);
      const bf16x8 p1 = *reinterpret_cast<const bf16x8 *>(Ps + (32 + l32) * PSTR + 16 * kq + 8 * h2);
      // rows 16kq + 4h2 + e and 16kq + 8 + 4h2 + e, column d0 + 32dt + l32
      const int col = d0 + 16 * (G % 2) + 4 * c_src;
      const __bf16 *rlo = kb + (16 * kq + 4 * h2 + e_src) * STR + col;
      const __bf16 *rhi = kb + (16 * kq + 8 + 4 * h2 + e_src) * STR + col;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        const bf16x8 a = cat4(lds_read_tr4(rlo + 32 * dt), lds_read_tr4(rhi + 32 * dt));
        o[dt][0] = mfma32(a, p0, o[dt][0]);
        o[dt][1] = mfma32(a, p1, o[dt][1]);
      }
    }
  };
  // Block barrier that waits for this wave's LDS writes but leaves the row
  // copies in flight (vmcnt stays at its maximum).
  auto lds_barrier = []() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
  };
  int nv = 0;  // COMPACT: valid indices in LST
  // Raw index of this lane's slot of chunk ch (lanes T.. and slots past the
  // end: -1); it is validated only in the step that uses it, since testing a
  // fresh load would make the compiler wait for it and for every row copy
  // issued before it.
  auto chunk_idx = [&](int ch) -> int {
    const int i = ch * T + lane;
    if constexpr (COMPACT) return (lane < T && i < nv) ? LST[i] : -1;
    return (lane < T && i < topk) ? ib[i] : -1;
  };
  auto step = [&](int ch, int nchunks, int &my_cur, int &raw_next, const __bf16 *cur, __bf16 *nxt) {
    const uint64_t vmask = __ballot(my_cur >= 0);
    int my_following = -1;
    if (ch + 1 < nchunks) {
      my_following = valid(raw_next);
      gather(my_following, nxt);
      if (ch + 2 < nchunks) raw_next = chunk_idx(ch + 2);
    }
    if (wave_active && vmask != 0) scores(cur, vmask);
    lds_barrier();  // P and the factors of this chunk visible
    if (vmask != 0) outprod(cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next chunk visible; this chunk's buffer, P and factors free
    my_cur = my_following;
  };

  if constexpr (COMPACT) nv = compact_window(0, topk);
  const int nchunks = COMPACT ? max(1, (nv + T - 1) / T) : (topk + T - 1) / T;
  int my_cur = valid(chunk_idx(0));
  gather(my_cur, C0);
  int my_next = nchunks > 1 ? chunk_idx(1) : -1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ch += 2) {
    step(ch, nchunks, my_cur, my_next, C0, C1);
    if (ch + 1 < nchunks) step(ch + 1, nchunks, my_cur, my_next, C1, C0);
  }

  // 1/l of each head (with the sink) through As, then each wave writes its
  // d columns of every head.
  float l_tot = sum_xor32(sum_xor16(l_run));
  if (sink != nullptr && hg < H) l_tot += fast_exp2(fmaf(sink[hg], kLog2e, -m_run));
  if (wave_active && G == 0) As[h] = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __syncthreads();
  const float inv[2] = {As[l32], As[32 + l32]};
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = hb + 32 * ht + l32;
    if (head >= H) continue;
    __bf16 *oh = out + (pos * H + head) * (int64_t)D + d0 + 4 * h2;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 r4;
#pragma unroll
        for (int i = 0; i < 4; ++i) r4[i] = (__bf16)(o[dt][ht][4 * a + i] * inv[ht]);
        *reinterpret_cast<bf16x4 *>(oh + 32 * dt + 8 * a) = r4;
      }
  }
}

}  // namespace

bool topk_supported(int32_t H, int32_t d) {
  return H >= 1 && (d == 128 || d == 256 || d == 512);
}

hipError_t launch_topk(const void *q, const void *kv, const int32_t *idx, const float *sink,
                       int32_t B, int32_t M, int32_t N, int32_t H, int32_t d, int32_t topk,
                       float scale, void *out, hipStream_t stream) {
  if (!topk_supported(H, d)) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)B * M;
  const int64_t groups = ((int64_t)H + 63) / 64;  // 64 heads per workgroup
  if (grid > 0x7fffffff || groups > 65535) return hipErrorInvalidValue;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid, (unsigned)groups), dim3(256), 0, stream,
                       (const __bf16 *)q, (const __bf16 *)kv, idx, sink, M, N, H, topk,
                       scale * kLog2e, (__bf16 *)out);
  };
  const bool compact = topk <= kWindow;
  if (d == 512) {
    if (compact) launch(topk_kernel<512, true>); else launch(topk_kernel<512, false>);
  } else if (d == 256) {
    if (compact) launch(topk_kernel<256, true>); else launch(topk_kernel<256, false>);
  } else {
    if (compact) launch(topk_kernel<128, true>); else launch(topk_kernel<128, false>);
  }
  return hipGetLastError();
}

}  // namespace bsa
