// Fused block-sparse attention forward (gfx950).
//
// Computes, for every query row, softmax(scale * q K^T) V over the key tokens
// of the live tiles of its block row only (scaled dot-product attention of
// the next.gr "Block Sparse Attention Techniques" tutorial with -inf outside
// the pattern; each live tile is a dense b x b piece of work as in the
// Language AI Handbook's "Block Structure").  The softmax is evaluated online
// over the live tiles with a running maximum and sum, the streaming form the
// DeepSeek-V4.1 "Weighted row sum" kernel uses, including its finite start
// value for the running maximum.
//
// Work item = (batch b, head h, query block m).  Work items follow the plan's
// row order (head-major, heaviest rows first) and are laid out so that each of
// the eight XCDs receives one contiguous stretch of that order: consecutive
// workgroup ids go round-robin over the XCDs, so item = (id % 8) * per + id / 8.
//
// Every variant computes, per live tile, S^T = K Q^T with Q^T resident in
// registers as the MFMA B operand, an online softmax in which each lane owns
// one query column (exp2 with scale*log2(e) folded into one multiply-add),
// and O^T += V^T P^T with P^T taken straight from the S^T accumulators (the
// k-slot order of the accumulator layout is the contraction order) and V^T
// read from a row-major V tile by LDS transpose reads.  No score matrix ever
// leaves registers.  Variants:
//   bsa_fwd_kernel      bs = 16: 16 query rows per wave, 16x16x32 MFMA
//   bsa_fwd32_kernel    bs = 32 and fp32 I/O: 32 rows per wave, 32x32x16 MFMA,
//                       register-staged tiles, two key halves per row group
//                       when bs >= 64
//   bsa_fwd_dma_kernel  bf16, bs >= 64: one wave per 32-row group, each live
//                       tile streamed as two pieces of bs/2 keys copied from
//                       HBM straight into double-buffered, XOR-swizzled LDS
//                       (two workgroups per CU)
//
// Optional terms, from the arguments of the ejkernel BlockSparseAttention
// operation: grouped K/V heads (query head h reads K/V head h / kv_group), a
// per-head sink logit folded into the denominator after the loop, and -- in
// instances of their own, so that the plain instances keep their code -- a
// tanh cap on the scaled scores and an element-level causal mask on tiles
// that reach past the diagonal.  The bf16 copy-staged kernel (bs >= 64) has
// two plain-copy option instances for whole blocks without segment ids: the
// causal mask alone, and the cap compiled in (with or without the causal
// mask); every other option set runs the MASK instance.
#include <type_traits>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxFloor = -1e30f;
constexpr float kLazy = 8.0f;  // tolerated staleness of the running max (log2 units)
#ifndef BSA_DMA_KEY_SPLIT
#define BSA_DMA_KEY_SPLIT 2
#endif
constexpr int kDmaKeySplit = BSA_DMA_KEY_SPLIT;  // waves per 32-row group in the bf16 bs=128 kernel
#ifndef BSA_DMA_PIECES
#define BSA_DMA_PIECES 2
#endif
// pieces per tile in the bf16 bs=128 kernel with one wave per 32-row group
constexpr int kDmaPieces = BSA_DMA_PIECES;
#ifndef BSA_DMA_PIECES64
#define BSA_DMA_PIECES64 2
#endif
constexpr int kDmaPieces64 = BSA_DMA_PIECES64;  // the same for bs=64
#ifndef BSA_READ_AHEAD_K
#define BSA_READ_AHEAD_K 4
#endif
#ifndef BSA_READ_AHEAD_V
#define BSA_READ_AHEAD_V 6
#endif
#ifndef BSA_PAIR_FORM
#define BSA_PAIR_FORM 1
#endif
// 1: bf16 bs = 64 forwards use the plan's pairs of block rows when its flag is set
constexpr bool kPairForm = BSA_PAIR_FORM != 0;
// Live tiles per block row up to which the segment-id instances filter the
// row's list into LDS (12 bytes each: the column and one id per piece)
constexpr int kSegList = 512;
// List entries: the column in the low bits; bit 30 + h set when every key of
// piece h of the tile carries one segment id (kept in LSEG)
constexpr int kColBits = 0x3fffffff;

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
constexpr int kReadAheadK = BSA_READ_AHEAD_K;  // K operand reads issued before the first QK MFMA
constexpr int kReadAheadV = BSA_READ_AHEAD_V;  // V transpose reads issued before the first PV MFMA

template <typename T> struct Io;
template <> struct Io<__bf16> {
  // 8 consecutive elements -> bf16x8
  static __device__ __forceinline__ bf16x8 load8(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
  }
  static __device__ __forceinline__ void store4(__bf16 *p, f32x4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    *reinterpret_cast<bf16x4 *>(p) = r;
  }
  static __device__ __forceinline__ void store_zero4(__bf16 *p) {
    *reinterpret_cast<uint64_t *>(p) = 0ull;
  }
};
template <> struct Io<float> {
  static __device__ __forceinline__ bf16x8 load8(const float *p) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    return to_bf16x8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
  }
  static __device__ __forceinline__ void store4(float *p, f32x4 x) {
    *reinterpret_cast<f32x4 *>(p) = x;
  }
  static __device__ __forceinline__ void store_zero4(float *p) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

template <int BS, int D, typename T, bool MASK>
__global__ void __launch_bounds__(BS * 4)
bsa_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
               const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
               const int32_t *__restrict__ row_order, int32_t B, int32_t H, int32_t Mb,
               int32_t Nb, float scale_log2, T *__restrict__ out, float *__restrict__ lse, const FwdOptions opt) {
  constexpr int NW = BS / 16;            // waves per workgroup
  constexpr int NT = NW * 64;            // threads per workgroup
  constexpr int KSTR = D + 8;            // LDS row stride (elements) of the K tile
  constexpr int VSTR = D + 16;           // LDS row stride of the V tile
  constexpr int CPT = (BS * D / 8) / NT; // 8-element chunks per thread per tile
  constexpr int QC = D / 32;             // 32-wide k chunks of the QK^T contraction
  constexpr int JT = BS / 16;            // 16-key sub-tiles of a tile
  constexpr int DT = D / 16;             // 16-wide d sub-tiles of the output
  static_assert(CPT * NT * 8 == BS * D, "tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) __bf16 Ks[BS * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[BS * VSTR];

  const int64_t W = (int64_t)B * H * Mb;
  const int64_t per = (W + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= W) return;
  const int64_t HM = (int64_t)H * Mb;
  const int b = (int)(w / HM);
  const int r = row_order[w % HM];
  const int h = r / Mb;
  const int m = r % Mb;
  const int beg = row_ptr[r];
  const int end = row_ptr[r + 1];

  const int tid = threadIdx.x;
  const int wid = tid / 64;
  const int lane = tid % 64;
  const int G = lane / 16;   // lane group
  const int li = lane % 16;  // query column owned by this lane

  const int64_t bh = (int64_t)b * H + h;
  const int64_t Sq = opt.sq, Sk = opt.sk;
  const T *qh = q + bh * Sq * D;
  const int64_t bkv = (int64_t)b * (H / opt.kv_group) + h / opt.kv_group;  // K/V head
  const T *kh = k + bkv * Sk * D;
  const T *vh = v + bkv * Sk * D;
  T *oh = out + bh * Sq * D;
  float *lh = lse ? lse + bh * Sq : nullptr;
  const int64_t i_row = (int64_t)m * BS + 16 * wid + li;  // this lane's query row
  const bool q_ok = !MASK || i_row < Sq;                  // rows past a cut last block
  const int qsg = (MASK && opt.qseg && q_ok) ? opt.qseg[(int64_t)b * Sq + i_row] : 0;

  if (beg == end) {  // no live tile: zero output, lse = -inf (the sink logit with a sink)
    if (!q_ok) return;
    for (int dt = 0; dt < DT; ++dt) Io<T>::store_zero4(oh + i_row * D + 16 * dt + 4 * G);
    if (lh && G == 0) lh[i_row] = opt.sink ? opt.sink[h] : -__builtin_inff();
    return;
  }

  // Q^T fragments (B operand of S^T = K Q^T): column = query row, k = d.
  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) qf[c] = q_ok ? Io<T>::load8(qh + i_row * D + 32 * c + 8 * G) : bf16x8{};

  // Register prefetch of one K/V tile.
  bf16x8 kr[CPT], vr[CPT];
  auto load_tile = [&](int n) {
    const T *kt = kh + (int64_t)n * BS * D;
    const T *vt = vh + (int64_t)n * BS * D;
    const int kval = MASK ? (int)min((int64_t)BS, Sk - (int64_t)n * BS) : BS;  // rows that exist
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      const int row = qid / (D / 8), col = (qid % (D / 8)) * 8;
      const bool ok = !MASK || row < kval;
      kr[c] = ok ? Io<T>::load8(kt + row * D + col) : bf16x8{};
      vr[c] = ok ? Io<T>::load8(vt + row * D + col) : bf16x8{};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      const int row = qid / (D / 8), col = (qid % (D / 8)) * 8;
      *reinterpret_cast<bf16x8 *>(&Ks[row * KSTR + col]) = kr[c];
      *reinterpret_cast<bf16x8 *>(&Vs[row * VSTR + col]) = vr[c];
    }
  };

  float m_run = kMaxFloor;  // running max of scale*log2(e)*s
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(col_idx[beg]);
  for (int t = beg; t < end; ++t) {
    __syncthreads();  // all waves are done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < end) load_tile(col_idx[t + 1]);

    // S^T[j][i] for j in the tile (rows), i = this wave's 16 query rows.
    f32x4 s[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&Ks[(16 * jt + li) * KSTR + 32 * c + 8 * G]);
        s[jt] = mfma16(a, qf[c], s[jt]);
      }
    }
    // Options (MASK instances only): tanh logit cap, then the causal mask on
    // tiles that reach past the diagonal (key row 16jt + 4G + e, query row
    // 16 wid + li).
    if (MASK && opt.cap_k != 0.f) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[jt][e] = capped_score(s[jt][e], opt.cap_k, opt.cap_b);
    }
    if (MASK && opt.causal && col_idx[t] >= m) {
      const int dq = (m - col_idx[t]) * BS + 16 * wid + li;  // query minus key offset
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * jt + 4 * G + e > dq) s[jt][e] = -__builtin_inff();
    }
    if (MASK && (int64_t)(col_idx[t] + 1) * BS > Sk) {  // keys past a cut last block
      const int kv = (int)(Sk - (int64_t)col_idx[t] * BS);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * jt + 4 * G + e >= kv) s[jt][e] = -__builtin_inff();
    }
    if (MASK && opt.qseg) {  // packed sequences: only keys of the query's segment
      const int64_t k0 = (int64_t)col_idx[t] * BS;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t key = k0 + 16 * jt + 4 * G + e;
          if (key < Sk && opt.kseg[(int64_t)b * Sk + key] != qsg) s[jt][e] = -__builtin_inff();
        }
    }
    // Online softmax over this tile's keys for query column li.
    float mx = s[0][0];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[jt][e]);
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[jt][e], scale_log2, -m_new));
        s[jt][e] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;

    // O^T[d][i] += sum_j V[j][d] P^T[j][i]
    const int e_src = li / 4, c_src = li % 4;  // transpose-read source coordinates
    if constexpr (BS == 16) {
      const bf16x4 pf = bf16x4{(__bf16)s[0][0], (__bf16)s[0][1], (__bf16)s[0][2], (__bf16)s[0][3]};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 a = lds_read_tr4(&Vs[(4 * G + e_src) * VSTR + 16 * dt + 4 * c_src]);
        acc[dt] = mfma16k16(a, pf, acc[dt]);
      }
    } else {
      constexpr int KC = BS / 32;
      bf16x8 pf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        pf[kc] = to_bf16x8(s[2 * kc][0], s[2 * kc][1], s[2 * kc][2], s[2 * kc][3],
                           s[2 * kc + 1][0], s[2 * kc + 1][1], s[2 * kc + 1][2], s[2 * kc + 1][3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          // k-slots of lane group G: keys 32kc + 4G + e and 32kc + 16 + 4G + e
          const __bf16 *src = &Vs[(32 * kc + 4 * G + e_src) * VSTR + 16 * dt + 4 * c_src];
          const bf16x8 a = cat4(lds_read_tr4(src), lds_read_tr4(src + 16 * VSTR));
          acc[dt] = mfma16(a, pf[kc], acc[dt]);
        }
    }
  }

  float l_tot = sum_xor32(sum_xor16(l_run));
  float o_scale = 1.f;
  if (opt.sink) o_scale = fold_sink(m_run, l_tot, opt.sink[h] * kLog2e);
  const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
  if (!q_ok) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) Io<T>::store4(oh + i_row * D + 16 * dt + 4 * G, acc[dt] * inv);
  if (lh && G == 0) lh[i_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}


// Variant for bs >= 32: each wave owns 32 query rows and uses the 32x32x16
// MFMA, which halves the LDS operand traffic per FLOP of the 16-row layout.
// With KSPLIT = 2 (bs >= 64) the workgroup holds two waves per 32-row group:
// wave (g, s) handles keys [s*bs/2, (s+1)*bs/2) of every live tile for rows
// 32g .. 32g+31 with its own running max / sum / output, and the two partial
// results are merged once at the end (the split-softmax identity
// O = (a1 O1 + a2 O2) / (a1 l1 + a2 l2), a_k = exp(m_k - max(m1, m2))).  Two
// waves per SIMD let one wave's softmax overlap the other's MFMA work.
//   S^T[j][i]: lane column i = lane%32; key rows 8*(r/4) + 4*(lane/32) + r%4
//   P^T operand for 16 keys: registers r = 8c .. 8c+7 of one 32-key block
//   O^T[d][i]: the same result layout over d
template <int BS, int D, typename T, int KSPLIT, bool MASK>
__global__ void __launch_bounds__(BS * 2 * KSPLIT) __attribute__((amdgpu_waves_per_eu(2)))
bsa_fwd32_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                 const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                 const int32_t *__restrict__ row_order, int32_t B, int32_t H, int32_t Mb,
                 int32_t Nb, float scale_log2, T *__restrict__ out, float *__restrict__ lse, const FwdOptions opt) {
  constexpr int NRG = BS / 32;           // 32-row groups
  constexpr int NW = NRG * KSPLIT;       // waves per workgroup
  constexpr int NT = NW * 64;            // threads per workgroup
  constexpr int KW = BS / KSPLIT;        // keys per wave per tile
  constexpr int KSTR = D + 8;            // LDS row stride (elements) of the K tile
  constexpr int VSTR = D + 16;           // LDS row stride of the V tile
  constexpr int CPT = (BS * D / 8) / NT; // 8-element chunks per thread per tile
  constexpr int QC = D / 16;             // 16-wide k chunks of the QK^T contraction
  constexpr int JT = KW / 32;            // 32-key blocks per wave per tile
  constexpr int DT = D / 32;             // 32-wide d blocks of the output
  static_assert(CPT * NT * 8 == BS * D, "tile must split evenly over threads");
  static_assert(JT >= 1, "each wave needs at least 32 keys per tile");
  // merge scratch (fp32): per row group DT*16*64 output values + 2*64 (m, l)
  constexpr int MRG = DT * 16 * 64 + 128;
  static_assert(KSPLIT == 1 || (size_t)NRG * MRG * 4 <= (size_t)BS * (KSTR + VSTR) * 4,
                "merge scratch must fit in the tile buffers");

  // one LDS block: two K tiles, then two V tiles; reused as merge scratch
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * BS * (KSTR + VSTR)];
  // segment ids of the two K tiles' keys (MASK instances with segment ids)
  __shared__ __attribute__((aligned(16))) int32_t kseg_s[MASK ? 2 * BS : 4];
  __bf16 *const Kbuf0 = smem;
  __bf16 *const Vbuf0 = smem + 2 * BS * KSTR;

  const int64_t W = (int64_t)B * H * Mb;
  const int64_t per = (W + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= W) return;
  const int64_t HM = (int64_t)H * Mb;
  const int b = (int)(w / HM);
  const int r = row_order[w % HM];
  const int h = r / Mb;
  const int m = r % Mb;
  const int beg = row_ptr[r];
  const int end = row_ptr[r + 1];

  const int tid = threadIdx.x;
  const int wid = tid / 64;
  const int rg = wid % NRG;     // row group
  const int ks = wid / NRG;     // key half
  const int lane = tid % 64;
  const int h2 = lane / 32;     // half of the wave: selects k-slots 8*h2 .. 8*h2+7
  const int l32 = lane % 32;    // query column owned by this lane
  const int G = lane / 16;      // 16-lane group (transpose reads)
  const int l16 = lane % 16;

  const int64_t bh = (int64_t)b * H + h;
  const int64_t Sq = opt.sq, Sk = opt.sk;
  const T *qh = q + bh * Sq * D;
  const int64_t bkv = (int64_t)b * (H / opt.kv_group) + h / opt.kv_group;  // K/V head
  const T *kh = k + bkv * Sk * D;
  const T *vh = v + bkv * Sk * D;
  T *oh = out + bh * Sq * D;
  float *lh = lse ? lse + bh * Sq : nullptr;
  const int64_t i_row = (int64_t)m * BS + 32 * rg + l32;
  const bool q_ok = !MASK || i_row < Sq;  // rows past a cut last block
  const int qsg = (MASK && opt.qseg && q_ok) ? opt.qseg[(int64_t)b * Sq + i_row] : 0;

  if (beg == end) {
    if (ks == 0 && q_ok) {
      for (int dt = 0; dt < DT; ++dt)
        for (int a = 0; a < 4; ++a) Io<T>::store_zero4(oh + i_row * D + 32 * dt + 8 * a + 4 * h2);
      if (lh && h2 == 0) lh[i_row] = opt.sink ? opt.sink[h] : -__builtin_inff();
    }
    return;
  }

  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) qf[c] = q_ok ? Io<T>::load8(qh + i_row * D + 16 * c + 8 * h2) : bf16x8{};

  // Register staging of one K tile and one V tile (16-byte pieces).
  bf16x8 kr[CPT], vr[CPT];
  // (MASK instances: rows past a cut last block load zeros)
  auto kval_of = [&](int n) { return MASK ? (int)min((int64_t)BS, Sk - (int64_t)n * BS) : BS; };
  int ksr = 0;   // staged segment id of key `tid` of the next K tile
  auto load_k = [&](int n) {
    const T *src = kh + (int64_t)n * BS * D;
    const int kval = kval_of(n);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      kr[c] = (!MASK || qid / (D / 8) < kval)
                  ? Io<T>::load8(src + (qid / (D / 8)) * D + (qid % (D / 8)) * 8) : bf16x8{};
    }
    if (MASK && opt.qseg && tid < BS)
      ksr = tid < kval ? opt.kseg[(int64_t)b * Sk + (int64_t)n * BS + tid] : 0;
  };
  auto load_v = [&](int n) {
    const T *src = vh + (int64_t)n * BS * D;
    const int kval = kval_of(n);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      vr[c] = (!MASK || qid / (D / 8) < kval)
                  ? Io<T>::load8(src + (qid / (D / 8)) * D + (qid % (D / 8)) * 8) : bf16x8{};
    }
  };
  auto store_k = [&](int buf) {
    __bf16 *dst = Kbuf0 + buf * BS * KSTR;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      *reinterpret_cast<bf16x8 *>(&dst[(qid / (D / 8)) * KSTR + (qid % (D / 8)) * 8]) = kr[c];
    }
    if (MASK && opt.qseg && tid < BS) kseg_s[buf * BS + tid] = ksr;
  };
  auto store_v = [&](int buf) {
    __bf16 *dst = Vbuf0 + buf * BS * VSTR;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      *reinterpret_cast<bf16x8 *>(&dst[(qid / (D / 8)) * VSTR + (qid % (D / 8)) * 8]) = vr[c];
    }
  };

  const int key0 = ks * KW;
  const int e_src = l16 / 4, c_src = l16 % 4;
  const int koff = (key0 + l32) * KSTR + 8 * h2;
  const int voff = (key0 + 4 * h2 + e_src) * VSTR + 16 * (G % 2) + 4 * c_src;

  // S^T of this wave's keys of the tile held in K buffer `buf`.
  auto qk = [&](int buf, f32x16 (&s)[JT]) {
    const __bf16 *ksrc = Kbuf0 + buf * BS * KSTR + koff;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      s[jt] = f32x16{};
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ksrc + 32 * jt * KSTR + 16 * c);
        s[jt] = mfma32(a, qf[c], s[jt]);
      }
    }
  };

  // Options on a fresh score tile of column ncol (MASK instances; CAUSAL
  // instances the causal mask alone): tanh logit cap, then the causal mask
  // when the tile reaches past the diagonal
  // (key row key0 + 32jt + 8(e/4) + 4h2 + e%4, query row 32rg + l32).
  auto apply_opts = [&](f32x16 (&s)[JT], int ncol, int buf) {
    if constexpr (!MASK) return;
    if (opt.cap_k != 0.f) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[jt][e] = capped_score(s[jt][e], opt.cap_k, opt.cap_b);
    }
    if (opt.causal && ncol >= m) {
      const int dq = (m - ncol) * BS + 32 * rg + l32 - key0 - 4 * h2;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * jt + 8 * (e / 4) + (e % 4) > dq) s[jt][e] = -__builtin_inff();
    }
    if (MASK && (int64_t)(ncol + 1) * BS > Sk) {  // keys past a cut last block
      const int kv = (int)(Sk - (int64_t)ncol * BS) - key0 - 4 * h2;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * jt + 8 * (e / 4) + (e % 4) >= kv) s[jt][e] = -__builtin_inff();
    }
    if (opt.qseg) {  // packed sequences: only keys of the query's segment (ids staged in LDS)
      const int32_t *kst = kseg_s + buf * BS + key0 + 4 * h2;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const i32x4 ids = *reinterpret_cast<const i32x4 *>(kst + 32 * jt + 8 * a4);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (ids[i] != qsg) s[jt][4 * a4 + i] = -__builtin_inff();
        }
    }
  };

  float m_run = kMaxFloor;  // running max (log2 units); may lag the true max by < kLazy
  float l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

  // Online softmax of one tile's scores and the P V product from V buffer
  // `buf`.  The running max is raised only when a score exceeds it by more
  // than kLazy (log2 units): the shift cancels in out = O / l, so a stale max
  // is exact, and the rescale of O is skipped for most tiles.
  auto softmax_pv = [&](f32x16 (&s)[JT], int buf) {
    float mx = s[0][0];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jt][e]);
    mx = max_xor32(mx) * scale_log2;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(s[jt][e], scale_log2, -m_run));
        s[jt][e] = pe;
        psum += pe;
      }
    l_run += psum;
    const __bf16 *vsrc = Vbuf0 + buf * BS * VSTR + voff;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 pf = to_bf16x8(s[jt][8 * c2 + 0], s[jt][8 * c2 + 1], s[jt][8 * c2 + 2],
                                    s[jt][8 * c2 + 3], s[jt][8 * c2 + 4], s[jt][8 * c2 + 5],
                                    s[jt][8 * c2 + 6], s[jt][8 * c2 + 7]);
        // k-slots: keys 32jt + 16c2 + 4*h2 + e and 32jt + 16c2 + 8 + 4*h2 + e
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const __bf16 *src = vsrc + (32 * jt + 16 * c2) * VSTR + 32 * dt;
          const bf16x8 a = cat4(lds_read_tr4(src), lds_read_tr4(src + 8 * VSTR));
          o[dt] = mfma32(a, pf, o[dt]);
        }
      }
  };

  // Software pipeline over the row's live tiles u = 0 .. n-1 (tile u is
  // column col_idx[beg + u]).  Tile u's K sits in K buffer u % 2, its V in V
  // buffer u % 2.  At the top of iteration t: K_{t+1} and V_t are in LDS,
  // S_t is in registers, K_{t+2} and V_{t+1} are in the staging registers.
  // One barrier per tile; the QK^T of tile t+1 is independent of the
  // softmax of tile t, so their MFMA and VALU work can interleave.
  const int n = end - beg;
  const int32_t *cols = col_idx + beg;
  f32x16 s_cur[JT], s_next[JT];
  load_k(cols[0]);
  load_v(cols[0]);
  store_k(0);
  store_v(0);
  if (n > 1) {
    load_k(cols[1]);
    store_k(1);
  }
  __syncthreads();
  qk(0, s_cur);
  apply_opts(s_cur, cols[0], 0);
  if (n > 2) load_k(cols[2]);
  if (n > 1) load_v(cols[1]);
  // Steady state without branches: staging of tiles past the end re-loads
  // the last tile into a buffer that is never read again, which keeps the
  // QK^T of the next tile and the softmax of this one in one basic block.
  for (int t = 0; t + 1 < n; ++t) {
    __syncthreads();  // iteration t-1 is done with K buffer t%2 and V buffer (t+1)%2
    store_k(t & 1);
    store_v((t + 1) & 1);
    load_k(cols[min(t + 3, n - 1)]);
    load_v(cols[min(t + 2, n - 1)]);
    qk((t + 1) & 1, s_next);
    apply_opts(s_next, cols[t + 1], (t + 1) & 1);
    softmax_pv(s_cur, t & 1);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) s_cur[jt] = s_next[jt];
  }
  __syncthreads();
  softmax_pv(s_cur, (n - 1) & 1);

  float l_tot = sum_xor32(l_run);
  if constexpr (KSPLIT == 2) {
    // Merge the two key halves of each row group through LDS.
    float *mrg = reinterpret_cast<float *>(smem) + rg * MRG;
    __syncthreads();  // every wave is done with the tile buffers
    if (ks == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mrg[(dt * 16 + e) * 64 + lane] = o[dt][e];
      mrg[DT * 16 * 64 + lane] = m_run;
      mrg[DT * 16 * 64 + 64 + lane] = l_tot;
    }
    __syncthreads();
    if (ks == 1) return;
    const float m2 = mrg[DT * 16 * 64 + lane];
    const float l2 = mrg[DT * 16 * 64 + 64 + lane];
    const float mm = fmaxf(m_run, m2);
    const float a1 = fast_exp2(m_run - mm), a2 = fast_exp2(m2 - mm);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = o[dt][e] * a1 + mrg[(dt * 16 + e) * 64 + lane] * a2;
    l_tot = l_tot * a1 + l2 * a2;
    m_run = mm;
  }
  float o_scale = 1.f;
  if (opt.sink) o_scale = fold_sink(m_run, l_tot, opt.sink[h] * kLog2e);
  const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
  if (!q_ok) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      Io<T>::store4(oh + i_row * D + 32 * dt + 8 * a + 4 * h2,
                    f32x4{o[dt][4 * a], o[dt][4 * a + 1], o[dt][4 * a + 2], o[dt][4 * a + 3]} * inv);
  if (lh && h2 == 0) lh[i_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}

// bf16 variant for bs >= 64 whose K and V tiles travel from global memory
// straight into LDS (buffer_load_dwordx4 ... lds: lane l of a wave
// instruction writes bytes 16l .. 16l+15 of a 1 KiB LDS span), so no staging
// registers or LDS store instructions sit in the loop.  Rows are unpadded;
// 16-byte chunks are XOR-swizzled per row so that both read patterns are
// free of bank conflicts:
//   K (b128 reads, 16 consecutive rows per phase): chunk ^ (row % CPR)
//   V (transpose reads, 4 rows x 64 B per half-wave): chunk ^ 4*f(row)
// The work split and MFMA layouts match bsa_fwd32_kernel; the pipeline (two
// phases per tile, each copy given one and a half tiles to land) and the
// instruction schedule are described at the loop.
template <int D> struct VSwz {
  static __device__ __forceinline__ int f(int row) {
    if constexpr (D == 128) return 4 * (row & 3);
    else if constexpr (D == 64) return 4 * ((row >> 1) & 1);
    else return 0;
  }
};

// GROUP instances serve the pairs of neighbouring block rows of a layout
// with bs = BS / 2 (the plan's pair lists): a work item is pair p of head h,
// i.e. query rows p*BS .. p*BS + BS - 1 (block rows 2p and 2p+1), and each
// list entry names one key block of BS / 2 keys -- one piece -- together with
// the rows that list it (bits 24 and 25).  The row groups of the block row
// that does not list a piece give its scores -inf, so its weights are exactly
// zero: every shared tile is loaded once for both rows.
// sel / sel_want: with sel set, a launch whose *sel differs from sel_want
// returns at once (the pair and row forms are launched together and the
// plan's flag picks one).
template <int BS, int D, int KSPLIT, int PIECES, bool MASK, bool SEG = false, bool GROUP = false,
          bool CAUSAL = false, bool CAP = false>
__global__ void __launch_bounds__(BS * 2 * KSPLIT)
__attribute__((amdgpu_waves_per_eu(KSPLIT * PIECES)))
bsa_fwd_dma_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                   const __bf16 *__restrict__ v, const int32_t *__restrict__ row_ptr,
                   const int32_t *__restrict__ col_idx, const int32_t *__restrict__ row_order,
                   int32_t B, int32_t H, int32_t Mb, int32_t Nb, float scale_log2,
                   __bf16 *__restrict__ out, float *__restrict__ lse, const FwdOptions opt,
                   const int32_t *__restrict__ sel, int32_t sel_want) {
  constexpr int NRG = BS / 32;           // 32-row groups
  constexpr int NW = NRG * KSPLIT;       // waves per workgroup
  constexpr int PB = BS / PIECES;        // keys per piece (a tile is streamed in PIECES pieces)
  constexpr int KW = PB / KSPLIT;        // keys per wave per piece
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int TILE = PB * D;           // elements per K or V buffer (one piece)
  constexpr int NI = TILE * 2 / 1024;    // 1 KiB load instructions per tile
  constexpr int IPW = NI / NW;           // load instructions per wave per tile
  constexpr int RPI = 64 / CPR;          // rows per load instruction
  constexpr int QC = D / 16;
  constexpr int JT = KW / 32;
  constexpr int DT = D / 32;
  constexpr int HALF = DT * 8 * 64;      // merge floats per row group and buffer
  static_assert(NI % NW == 0 && IPW >= 1, "tile loads must split evenly over waves");
  static_assert(KSPLIT == 1 || NRG * HALF * 4 == TILE * 2, "merge halves fill one tile buffer each");
  static_assert(KSPLIT == 1 || PIECES == 1, "the key split merges whole tiles");
  // The K swizzle of the rows a lane copies repeats every NSW copy
  // instructions of its wave (NSW = 1 when RPI * NW is a multiple of CPR).
  constexpr int NSW = (RPI * NW) % CPR == 0 ? 1 : CPR / ((RPI * NW) % CPR);
  static_assert((RPI * NW * NSW) % CPR == 0 && IPW % NSW == 0, "K swizzle pattern must repeat");
  static_assert(!CAUSAL || (!MASK && !GROUP), "the plain-copy option instances have plain rows");
  static_assert(!CAP || CAUSAL, "the cap is compiled into the plain-copy option instance only");
  static_assert(!GROUP || (!MASK && KSPLIT == 1 && NRG == 4 && PIECES == 2),
                "pairs: four row groups (two per block row), plain scores");
  constexpr int PPE = GROUP ? 1 : PIECES;  // pieces per plan entry
  constexpr int KBLK = GROUP ? PB : BS;    // keys per layout block column
  if (sel != nullptr && *sel != sel_want) return;

  // Four distinct LDS objects, so that the compiler can tell the piece being
  // read from the piece being filled and need not wait for the copy in flight.
  __shared__ __attribute__((aligned(1024))) __bf16 K0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 K1[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V0[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 V1[TILE];
  static_assert(MASK || !SEG, "segment ids come with the other masks");

  const int64_t W = (int64_t)B * H * Mb;
  const int64_t per = (W + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= W) return;
  const int64_t HM = (int64_t)H * Mb;
  const int b = (int)(w / HM);
  const int r = row_order[w % HM];
  const int h = r / Mb;
  const int m = r % Mb;
  const int beg = row_ptr[r];
  const int end = row_ptr[r + 1];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, kept in SGPRs
  const int rg = wid % NRG;
  const int ks = wid / NRG;
  const int lane = tid % 64;
  const int h2 = lane / 32;
  const int l32 = lane % 32;
  const int G = lane / 16;
  const int l16 = lane % 16;

  const int64_t bh = (int64_t)b * H + h;
  const int64_t Sq = opt.sq, Sk = opt.sk;

  // SEG instances drop, before the pipeline starts, the live tiles whose key
  // segment ids cannot meet those of the block row's queries: when the
  // [min, max] ranges of the two sets of ids are disjoint, every score of
  // the tile is masked and its weights are exactly zero, so neither its
  // copies nor its products are needed.  (Ranges only ever keep a tile too
  // many; the element masks below still decide every score.)  The kept
  // columns go to LDS, each with a flag per piece whose keys all carry one
  // id (that id in LSEG): the element mask of such a piece is one compare
  // per query.  Each wave computes the same list on its own, so no barrier
  // orders the writes.  A row with more than kSegList live tiles walks the
  // plan's list unfiltered.
  static_assert(!SEG || PIECES == 2, "the list holds two pieces per tile");
  __shared__ int32_t LST[SEG ? kSegList : 1];
  __shared__ int32_t LSEG[SEG ? 2 * kSegList : 1];
  int n_live = end - beg;
  bool use_list = false;
  if constexpr (SEG) {
    if (n_live <= kSegList) {
      use_list = true;
      int qlo = INT32_MAX, qhi = INT32_MIN;
      for (int i = lane; i < KBLK; i += 64) {
        const int64_t qi = (int64_t)m * KBLK + i;
        if (qi < Sq) {
          const int sg = opt.qseg[(int64_t)b * Sq + qi];
          qlo = min(qlo, sg);
          qhi = max(qhi, sg);
        }
      }
      qlo = wave_min(qlo);
      qhi = wave_max(qhi);
      // 16 lanes per tile, four tiles per pass, four passes per round: lane
      // (g, sub) reads ids sub*IPL .. of tile 4p + g, so the first eight
      // lanes of a group cover piece 0 and the last eight piece 1.
      constexpr int IPL = KBLK / 16;
      const int g = lane / 16, sub = lane % 16;
      int kept = 0;
      for (int t0 = 0; t0 < n_live; t0 += 16) {
        int lo[4], hi[4], colv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int t = t0 + 4 * p + g;
          lo[p] = INT32_MAX;
          hi[p] = INT32_MIN;
          colv[p] = t < n_live ? col_idx[beg + t] : 0;
          const int64_t kb = (int64_t)colv[p] * KBLK + sub * IPL;
          const int32_t *kg = opt.kseg + (int64_t)b * Sk + kb;
#pragma unroll
          for (int i = 0; i < IPL; ++i) {
            if (t < n_live && kb + i < Sk) {
              const int sg = kg[i];
              lo[p] = min(lo[p], sg);
              hi[p] = max(hi[p], sg);
            }
          }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
          for (int o = 1; o < 8; o <<= 1) {
            lo[p] = min(lo[p], __shfl_xor(lo[p], o));
            hi[p] = max(hi[p], __shfl_xor(hi[p], o));
          }
          // lane sub = 0 holds piece 0's range, and receives piece 1's
          const int lo1 = __shfl_xor(lo[p], 8), hi1 = __shfl_xor(hi[p], 8);
          const int t = t0 + 4 * p + g;
          const bool keep = sub == 0 && t < n_live && min(lo[p], lo1) <= qhi && max(hi[p], hi1) >= qlo;
          const uint64_t mask = __ballot(keep);
          if (keep) {
            // a piece with no key before Sk counts as one id: its scores are masked anyway
            const int flags = (lo[p] >= hi[p] ? 1 << 30 : 0) | (lo1 >= hi1 ? 1 << 31 : 0);
            const int pos = kept + __popcll(mask & ((1ull << lane) - 1ull));
            LST[pos] = colv[p] | flags;
            LSEG[2 * pos] = lo[p];
            LSEG[2 * pos + 1] = lo1;
          }
          kept += __popcll(mask);
        }
      }
      n_live = kept;
    }
  }
  const __bf16 *qh = q + bh * Sq * D;
  const int64_t bkv = (int64_t)b * (H / opt.kv_group) + h / opt.kv_group;  // K/V head
  const __bf16 *kh = k + bkv * Sk * D;
  const __bf16 *vh = v + bkv * Sk * D;
  __bf16 *oh = out + bh * Sq * D;
  float *lh = lse ? lse + bh * Sq : nullptr;
  const int64_t i_row = (int64_t)m * BS + 32 * rg + l32;
  // rows past a cut last block, or the absent second row of a last pair
  const bool q_ok = !(MASK || GROUP) || i_row < Sq;
  const int qsg = (SEG && q_ok) ? opt.qseg[(int64_t)b * Sq + i_row] : 0;

  if (n_live == 0) {
    if (ks == 0 && q_ok) {
      for (int dt = 0; dt < DT; ++dt)
        for (int a = 0; a < 4; ++a) Io<__bf16>::store_zero4(oh + i_row * D + 32 * dt + 8 * a + 4 * h2);
      if (lh && h2 == 0) lh[i_row] = opt.sink ? opt.sink[h] : -__builtin_inff();
    }
    return;
  }

  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c)
    qf[c] = q_ok ? Io<__bf16>::load8(qh + i_row * D + 16 * c + 8 * h2) : bf16x8{};

  // Load instruction j of this wave covers tile rows RPI*(wid + NW*j) ..;
  // lane l writes physical chunk l % CPR of row RPI*i + l / CPR.
  const int lrow = lane / CPR, lph = lane % CPR;
  const int row0 = RPI * wid + lrow;  // f(row) of the V swizzle is the same for every j
  int k_src[NSW];                     // row % CPR repeats every NSW instructions
#pragma unroll
  for (int p = 0; p < NSW; ++p)
    k_src[p] = lrow * D + (lph ^ ((row0 + RPI * NW * p) & (CPR - 1))) * 8;
  const int v_src = lrow * D + (lph ^ VSwz<D>::f(row0)) * 8;
  // (MASK instances: a cut last tile's resource ends at the sequence end, so
  // the rows past it read as zeros.  The range check of a raw buffer load
  // covers the per-lane offset, not the scalar one, so those instances carry
  // the row offset per lane.)
  auto dma = [&](const __bf16 *src_tile, auto src_off_of, __bf16 *dst_tile, uint32_t bytes) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src_tile, bytes);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int i = wid + NW * j;
      const int src_off = src_off_of(j);
      if constexpr (MASK)
        copy16_to_lds(rs, dst_tile + i * 512, (uint32_t)(src_off * 2 + i * RPI * D * 2), 0u);
      else
        copy16_to_lds(rs, dst_tile + i * 512, (uint32_t)(src_off * 2), (uint32_t)(i * RPI * D * 2));
    }
  };
  // piece `half` of tile n: keys n*BS + half*PB .. + PB - 1 (rows past Sk read as zeros);
  // GROUP: key block n of PB keys (plan entries carry row bits above bit 24)
  auto tile_bytes = [&](int n, int half) -> uint32_t {
    return MASK ? (uint32_t)(max((int64_t)0, min((int64_t)PB, Sk - (int64_t)n * BS - half * PB)) * D * 2)
                : (uint32_t)(TILE * 2);
  };
  auto piece_src = [&](const __bf16 *base, int n, int half) {
    if constexpr (GROUP) n &= 0xffffff;
    return base + (int64_t)n * KBLK * D + (int64_t)half * PB * D;
  };
  auto load_k = [&](int n, int half, __bf16 *dst) {
    dma(piece_src(kh, n, half), [&](int j) { return k_src[j % NSW]; }, dst, tile_bytes(n, half));
  };
  auto load_v = [&](int n, int half, __bf16 *dst) {
    dma(piece_src(vh, n, half), [&](int) { return v_src; }, dst, tile_bytes(n, half));
  };

  // Per-lane element offsets of the K operand reads (one per k chunk).
  const int key0 = ks * KW;
  int koff[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c)
    koff[c] = (key0 + l32) * D + (((2 * c + h2) ^ (l32 & (CPR - 1))) * 8);
  // V^T operand: transpose-read source row and chunk of this lane
  const int e_src = l16 / 4, c_src = l16 % 4;
  const int vrow = key0 + 4 * h2 + e_src;   // + 32jt + 16c2 (+8) leaves f(row) unchanged
  const int vsw = VSwz<D>::f(vrow);

  auto qk = [&](const __bf16 *kb, f32x16 (&s)[JT]) {
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) s[jt] = f32x16{};
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + koff[c] + 32 * jt * D);
        s[jt] = mfma32(a, qf[c], s[jt]);
      }
  };

  // Options on a fresh score tile of column ncol (MASK instances; CAUSAL
  // instances the causal mask, with the cap when CAP): tanh logit cap, then
  // the causal mask when the tile reaches past the diagonal
  // (key row key0 + 32jt + 8(e/4) + 4h2 + e%4, query row 32rg + l32).
  // Bit 16 jt + e set: score e of block jt belongs to a key of another
  // segment.  ent is the list entry of piece u's tile: a piece whose keys
  // carry one id needs one compare; the others (segment boundaries, and
  // every piece of an unfiltered row) read this lane's key ids from memory.
  // u is an existing piece of the row, sid its id if it has only one.
  auto seg_bits = [&](int u, int ent, int sid) -> uint32_t {
    uint32_t bits = 0;
    if constexpr (SEG) {
      const int hf = u % PPE;
      if ((ent >> (30 + hf)) & 1) {
        bits = sid != qsg ? 0xffffffffu : 0u;
      } else {
        const int64_t kp = (int64_t)(ent & kColBits) * BS + hf * PB + key0 + 4 * h2;
        const int32_t *kg = opt.kseg + (int64_t)b * Sk;
#pragma unroll 1
        for (int x = 0; x < 16 * JT; ++x) {
          const int64_t key = kp + 32 * (x / 16) + 8 * ((x % 16) / 4) + (x % 4);
          bits |= (uint32_t)(key >= Sk || kg[key] != qsg) << x;
        }
      }
    }
    return bits;
  };
  auto apply_opts = [&](f32x16 (&s)[JT], int ncol, int half, uint32_t segbits) {
    if constexpr (GROUP) {  // a piece the wave's block row does not list: weights zero
      if (!((ncol >> (24 + rg / 2)) & 1)) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) s[jt] = f32x16{} - __builtin_inff();
      }
    }
    if constexpr (!MASK && !CAUSAL) return;
    const int kb0 = key0 + half * PB;   // this wave's first key inside the tile
    if (CAP || (MASK && opt.cap_k != 0.f)) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[jt][e] = capped_score(s[jt][e], opt.cap_k, opt.cap_b);
    }
    if (opt.causal && ncol >= m) {
      const int dq = (m - ncol) * BS + 32 * rg + l32 - kb0 - 4 * h2;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * jt + 8 * (e / 4) + (e % 4) > dq) s[jt][e] = -__builtin_inff();
    }
    if (MASK && (int64_t)(ncol + 1) * BS > Sk) {  // keys past a cut last block
      const int kv = (int)(Sk - (int64_t)ncol * BS) - kb0 - 4 * h2;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * jt + 8 * (e / 4) + (e % 4) >= kv) s[jt][e] = -__builtin_inff();
    }
    if constexpr (SEG) {  // packed sequences: only keys of the query's segment
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((segbits >> (16 * jt + e)) & 1u) s[jt][e] = -__builtin_inff();
    }
  };

  float m_run = kMaxFloor;  // running max (log2 units)
  float l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

  // This lane's maximum of a raw score tile.  The cross-lane step of the row
  // maximum is only needed when the running max moves, so it sits inside
  // the rescale branch; the test itself is a wave vote.
  auto tile_max = [&](const f32x16 (&s)[JT]) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[jt][e]);
    return mx;
  };
  // The running max moves only when some score of a tile exceeds it by more
  // than kLazy (log2 units); O and l are rescaled on those (rare) tiles alone.
  // The first tile always moves it off the finite floor (alpha = 0 there).
  auto rescale = [&](float mx) {
    if (__any(mx * scale_log2 > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, max_xor32(mx) * scale_log2);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
  };
  auto exp_pack = [&](const f32x16 (&s)[JT], bf16x8 (&pf)[2 * JT]) {
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s[jt][8 * c2 + e], scale_log2, -m_run));
        pf[2 * jt + c2] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        // the denominator sums the fp32 weights, so lse carries no bf16 rounding
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[e % 4] += p[e];
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  auto pv = [&](const bf16x8 (&pf)[2 * JT], const __bf16 *vb) {
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int row = vrow + 32 * jt + 16 * c2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // logical 8-byte piece (dt, G%2, c_src) of rows `row` and `row + 8`
          const int lc = 4 * dt + 2 * (G % 2) + c_src / 2;  // 16-byte chunk
          const __bf16 *src = vb + row * D + (lc ^ vsw) * 8 + 4 * (c_src % 2);
          const bf16x8 a = cat4(lds_read_tr4(src), lds_read_tr4(src + 8 * D));
          o[dt] = mfma32(a, pf[2 * jt + c2], o[dt]);
        }
      }
  };
  // Software pipeline over the row's pieces u = 0 .. n-1 (the live tiles'
  // pieces in order): piece u's K sits in K0 (u even) or K1 (u odd), its V
  // likewise in V0 / V1.  Step t has two phases separated by block barriers:
  //   S_t: K_{t+1} has landed; copy V_{t+1} into the V buffer PV(t-1) freed;
  //        then QK^T of piece t+1 beside the exponentials of piece t.
  //   M_t: V_t has landed; copy K_{t+3} into the K buffer QK(t+1) freed;
  //        then PV of piece t beside the row max of piece t+1.
  // Each copy thus has one and a half steps to land.  Every phase issues
  // IPW copies -- indices past
  // the row's end are clamped, so the last copies are redundant but
  // harmless -- and S_t also a column fetch, so the copy a phase needs is
  // followed by kVmInFlight copies and at most two fetches: waiting until at
  // most kVmInFlight vector-memory loads are in flight proves it has landed,
  // since loads complete in issue order.  (The count leaves the fetches out
  // because the compiler deletes those whose result is dead, in a row's last
  // steps; a spill store in between cannot loosen the wait, as it only adds
  // to the count.)  Column indices come from a vector load two steps ahead
  // (lane 0: K column for M_{t+2}, lane 1: V column for S_{t+2}); a scalar
  // load in flight would force every LDS wait in between to drain
  // completely.
  // Piece u = 0 .. n-1 is piece u % PIECES of live tile u / PIECES.
  const int n = n_live * PPE;
  const int32_t *cols = col_idx + beg;
  // SEG: the raw list entry (column and piece flags); col_at masks the flags
  auto entry_at = [&](int u) -> int {
    const int e = min(u, n - 1) / PPE;
    if constexpr (SEG) {
      // both loads are issued and the value selected: a selected pointer
      // would become a flat load, which the copy waits cannot count
      const int from_list = LST[min(e, kSegList - 1)];
      const int from_plan = cols[e];
      return use_list ? from_list : from_plan;
    }
    return cols[e];
  };
  auto col_at = [&](int u) -> int { return SEG ? entry_at(u) & kColBits : entry_at(u); };
  auto half_at = [&](int u) -> int { return min(u, n - 1) % PPE; };
  // SEG: lane 2 fetches the one segment id of piece vpos (meaningful when
  // its entry's flag says so)
  auto seg_id_at = [&](int u) -> int {
    const int uc = min(u, n - 1);
    return LSEG[min(2 * (uc / PPE) + uc % PPE, 2 * kSegList - 1)];
  };
  auto fetch_cols = [&](int kpos, int vpos) -> int {
    const int e = entry_at(lane == 0 ? kpos : vpos);
    if constexpr (SEG) {
      const int sid = seg_id_at(vpos);
      return lane == 2 ? sid : e;
    }
    return e;
  };
  constexpr int kVmInFlight = 2 * IPW;
  constexpr int kVmWait = (kVmInFlight & 15) | (7 << 4) | (15 << 8) | ((kVmInFlight >> 4) << 14);
  static_assert(kVmInFlight < 64, "vmcnt holds 6 bits");
  // Block barrier without the release fence of __syncthreads(), which would
  // drain every copy in flight; the explicit vmcnt waits above provide the
  // ordering, and the memory clobber keeps LDS accesses on their side.
  auto block_barrier = []() { asm volatile("s_barrier" ::: "memory"); };

  f32x16 s_a[JT], s_b[JT];
  float mx_a = 0.f, mx_b = 0.f;
  int cv0 = fetch_cols(3, 1);  // for S_0 / M_0
  int cv1 = fetch_cols(4, 2);  // for S_1 / M_1
  load_k(col_at(0), half_at(0), K0);
  load_v(col_at(0), half_at(0), V0);
  load_k(col_at(1), half_at(1), K1);
  const int k2 = col_at(2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  qk(K0, s_a);
  apply_opts(s_a, col_at(0), half_at(0), SEG ? seg_bits(0, entry_at(0), seg_id_at(0)) : 0u);
  mx_a = tile_max(s_a);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // M_{-1}: K0 free
  load_k(k2, half_at(2), K0);

  // One step; Kq is K[(t+1)%2], Vn is V[(t+1)%2], Vc is V[t%2].  MORE:
  // piece t+1 exists (every step but the row's last).
  auto step = [&](auto more_tag, int t, __bf16 *Kq, __bf16 *Vn, const __bf16 *Vc,
                  f32x16 (&s_cur)[JT], f32x16 (&s_nxt)[JT], float &mx_cur, float &mx_nxt,
                  int &cv) {
    constexpr bool MORE = decltype(more_tag)::value;
    __builtin_amdgcn_s_waitcnt(kVmWait);  // K_{t+1} landed (this wave's part)
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    const int kent = __builtin_amdgcn_readlane(cv, 0);  // column of piece t+3's tile
    const int vent = __builtin_amdgcn_readlane(cv, 1);  // column of piece t+1's tile
    const int kcol = SEG ? kent & kColBits : kent;
    const int vcol = SEG ? vent & kColBits : vent;
    const int vsid = SEG ? __builtin_amdgcn_readlane(cv, 2) : 0;  // its one segment id, if any
    cv = fetch_cols(t + 5, t + 3);
    load_v(vcol, half_at(t + 1), Vn);
    rescale(mx_cur);
    bf16x8 pf[2 * JT];
    if constexpr (MORE) qk(Kq, s_nxt);
    exp_pack(s_cur, pf);
    if constexpr (MORE) sched_interleave<JT * QC, JT * QC, kReadAheadK, 3 * 16 * JT / (JT * QC)>();
    __builtin_amdgcn_s_waitcnt(kVmWait);  // V_t landed
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    load_k(kcol, half_at(t + 3), Kq);
    uint32_t segbits = 0u;
    if constexpr (SEG && MORE) segbits = seg_bits(t + 1, vent, vsid);
    pv(pf, Vc);
    if constexpr (MORE) {
      apply_opts(s_nxt, vcol, half_at(t + 1), segbits);
      mx_nxt = tile_max(s_nxt);
      sched_interleave<JT * 2 * DT, 4 * JT * DT, kReadAheadV, 1>();
    } else {
      sched_interleave<JT * 2 * DT, 4 * JT * DT, kReadAheadV, 0>();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using More = std::true_type;
  using Last = std::false_type;
  int t = 0;
  for (; t + 2 < n; t += 2) {
    step(More{}, t, K1, V1, V0, s_a, s_b, mx_a, mx_b, cv0);
    step(More{}, t + 1, K0, V0, V1, s_b, s_a, mx_b, mx_a, cv1);
  }
  if (t + 1 < n) {
    step(More{}, t, K1, V1, V0, s_a, s_b, mx_a, mx_b, cv0);
    step(Last{}, t + 1, K0, V0, V1, s_b, s_a, mx_b, mx_a, cv1);
  } else {
    step(Last{}, t, K1, V1, V0, s_a, s_b, mx_a, mx_b, cv0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy may still be landing in the buffers reused below

  float l_tot = sum_xor32(l_run);
  if constexpr (KSPLIT == 2) {
    // merge the two key halves: O halves through K0 / K1, (m, l) through V0
    float *h0 = reinterpret_cast<float *>(K0) + rg * HALF;
    float *h1 = reinterpret_cast<float *>(K1) + rg * HALF;
    float *ml = reinterpret_cast<float *>(V0) + rg * 128;
    __syncthreads();
    if (ks == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int f = (dt * 16 + e) * 64 + lane;
          if (f < HALF) h0[f] = o[dt][e]; else h1[f - HALF] = o[dt][e];
        }
      ml[lane] = m_run;
      ml[64 + lane] = l_tot;
    }
    __syncthreads();
    if (ks == 1) return;
    const float m2 = ml[lane];
    const float l2 = ml[64 + lane];
    const float mm = fmaxf(m_run, m2);
    const float a1 = fast_exp2(m_run - mm), a2 = fast_exp2(m2 - mm);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int f = (dt * 16 + e) * 64 + lane;
        const float other = f < HALF ? h0[f] : h1[f - HALF];
        o[dt][e] = o[dt][e] * a1 + other * a2;
      }
    l_tot = l_tot * a1 + l2 * a2;
    m_run = mm;
  }
  float o_scale = 1.f;
  if (opt.sink) o_scale = fold_sink(m_run, l_tot, opt.sink[h] * kLog2e);
  const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
  if (!q_ok) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      Io<__bf16>::store4(oh + i_row * D + 32 * dt + 8 * a + 4 * h2,
                         f32x4{o[dt][4 * a], o[dt][4 * a + 1], o[dt][4 * a + 2], o[dt][4 * a + 3]} * inv);
  if (lh && h2 == 0) lh[i_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}

// Workgroups for W work items: a multiple of 8, so that the XCD mapping of
// the kernels (item = (id % 8) * per + id / 8) covers them.
int64_t grid_for(int64_t W) { return ((W + 7) / 8) * 8; }

template <int BS, int D, typename T, bool MASK, bool CAUSAL = false, bool CAP = false>
hipError_t launch_one(const void *q, const void *k, const void *v, const PlanArrays &pa, int32_t B,
                      int32_t H, int32_t Mb, int32_t Nb, float scale, const FwdOptions &opt,
                      void *out, float *lse, hipStream_t stream) {
  const int32_t *row_ptr = pa.row_ptr, *col_idx = pa.col_idx, *row_order = pa.row_order;
  const int64_t grid = grid_for((int64_t)B * H * Mb);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (BS == 16) {
    hipLaunchKernelGGL((bsa_fwd_kernel<BS, D, T, MASK>), dim3((unsigned)grid), dim3(BS * 4), 0,
                       stream, (const T *)q, (const T *)k, (const T *)v, row_ptr, col_idx,
                       row_order, B, H, Mb, Nb, scale * kLog2e, (T *)out, lse, opt);
  } else if constexpr (BS >= 64 && std::is_same<T, __bf16>::value) {
    constexpr int PC = BS == 128 ? kDmaPieces : kDmaPieces64;
    constexpr int KS = PC == 2 ? 1 : BS == 128 ? kDmaKeySplit : 2;
    const int32_t *sel = nullptr;
    if constexpr (kPairForm && BS == 64 && !MASK && !CAUSAL && PC == 2 && KS == 1) {
      // Pairs of block rows when the plan's flag says so (the unions of
      // neighbouring rows hold at most 3/4 of the tiles); both forms are
      // launched and the one the flag does not pick returns at once.
      if (pa.pair_info != nullptr && opt.qseg == nullptr) {
        sel = pa.pair_info + 1;
        const int32_t Mp = (Mb + 1) / 2;
        const int64_t pgrid = grid_for((int64_t)B * H * Mp);
        hipLaunchKernelGGL((bsa_fwd_dma_kernel<128, D, 1, 2, false, false, true>),
                           dim3((unsigned)pgrid), dim3(256), 0, stream, (const __bf16 *)q,
                           (const __bf16 *)k, (const __bf16 *)v, pa.pair_ptr, pa.pair_cols,
                           pa.pair_order, B, H, Mp, Nb, scale * kLog2e, (__bf16 *)out, lse, opt,
                           sel, 1);
      }
    }
    if constexpr (CAUSAL) {
      hipLaunchKernelGGL((bsa_fwd_dma_kernel<BS, D, KS, PC, false, false, false, true, CAP>),
                         dim3((unsigned)grid), dim3(BS * 2 * KS), 0, stream, (const __bf16 *)q,
                         (const __bf16 *)k, (const __bf16 *)v, row_ptr, col_idx, row_order, B, H,
                         Mb, Nb, scale * kLog2e, (__bf16 *)out, lse, opt, nullptr, 0);
    } else if (opt.qseg == nullptr) {
      hipLaunchKernelGGL((bsa_fwd_dma_kernel<BS, D, KS, PC, MASK>), dim3((unsigned)grid),
                         dim3(BS * 2 * KS), 0, stream, (const __bf16 *)q, (const __bf16 *)k,
                         (const __bf16 *)v, row_ptr, col_idx, row_order, B, H, Mb, Nb,
                         scale * kLog2e, (__bf16 *)out, lse, opt, sel, 0);
    } else {  // segment ids: the instance that filters each row's tiles by segment
      hipLaunchKernelGGL((bsa_fwd_dma_kernel<BS, D, KS, PC, true, true>), dim3((unsigned)grid),
                         dim3(BS * 2 * KS), 0, stream, (const __bf16 *)q, (const __bf16 *)k,
                         (const __bf16 *)v, row_ptr, col_idx, row_order, B, H, Mb, Nb,
                         scale * kLog2e, (__bf16 *)out, lse, opt, nullptr, 0);
    }
  } else {
    constexpr int KSPLIT = BS >= 64 ? 2 : 1;
    hipLaunchKernelGGL((bsa_fwd32_kernel<BS, D, T, KSPLIT, MASK>), dim3((unsigned)grid),
                       dim3(BS * 2 * KSPLIT), 0, stream, (const T *)q, (const T *)k, (const T *)v,
                       row_ptr, col_idx, row_order, B, H, Mb, Nb, scale * kLog2e, (T *)out, lse, opt);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(int32_t bs, int32_t d, const void *q, const void *k, const void *v,
                    const PlanArrays &pa, int32_t B, int32_t H, int32_t Mb, int32_t Nb,
                    float scale, const FwdOptions &opt, void *out, float *lse, hipStream_t s) {
  // Score-changing options (cap, causal) and cut last blocks select their own
  // kernel instances, so the plain forward keeps the code it has without them.
  const bool mask = opt.cap_k != 0.f || opt.causal != 0 || opt.sq % bs != 0 || opt.sk % bs != 0 ||
                    opt.qseg != nullptr;
  // Whole blocks without segment ids keep plain copies in the bf16
  // copy-staged kernel: the causal mask alone has one instance, and the cap
  // (with or without the causal mask) one with the cap compiled in, which
  // spares its per-tile branch (cap 1.30 -> 1.24 ms on the 32-head 32K
  // workload, outputs bit-identical).
  const bool plain_copies = opt.sq % bs == 0 && opt.sk % bs == 0 && opt.qseg == nullptr &&
                            std::is_same<T, __bf16>::value && bs >= 64;
  const bool causal_only = opt.causal != 0 && opt.cap_k == 0.f && plain_copies;
  const bool cap_plain = opt.cap_k != 0.f && plain_copies;
#define BSA_CASE(BS_, D_)                                                                     \
  if (bs == BS_ && d == D_)                                                                   \
    return cap_plain ? launch_one<BS_, D_, T, false, true, true>(q, k, v, pa, B, H, Mb, Nb,   \
                                                                 scale, opt, out, lse, s)     \
         : causal_only ? launch_one<BS_, D_, T, false, true>(q, k, v, pa, B, H, Mb, Nb, scale, \
                                                             opt, out, lse, s)                \
         : mask ? launch_one<BS_, D_, T, true>(q, k, v, pa, B, H, Mb, Nb, scale, opt, out, lse, \
                                               s)                                             \
                : launch_one<BS_, D_, T, false>(q, k, v, pa, B, H, Mb, Nb, scale, opt, out,     \
                                                lse, s);
  BSA_CASE(16, 32) BSA_CASE(16, 64) BSA_CASE(16, 128)
  BSA_CASE(32, 32) BSA_CASE(32, 64) BSA_CASE(32, 128)
  BSA_CASE(64, 32) BSA_CASE(64, 64) BSA_CASE(64, 128)
  BSA_CASE(128, 32) BSA_CASE(128, 64) BSA_CASE(128, 128)
#undef BSA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool forward_supported(int32_t bs, int32_t d) {
  return (bs == 16 || bs == 32 || bs == 64 || bs == 128) && (d == 32 || d == 64 || d == 128);
}

hipError_t launch_forward(const void *q, const void *k, const void *v, const PlanArrays &pa,
                          int32_t B, int32_t H, int32_t Mb, int32_t Nb, int32_t bs, int32_t d,
                          bool f32, float scale, const FwdOptions &opt, void *out, float *lse,
                          hipStream_t stream) {
  if (opt.kv_group < 1 || H % opt.kv_group != 0) return hipErrorInvalidValue;
  if (f32) return dispatch<float>(bs, d, q, k, v, pa, B, H, Mb, Nb, scale, opt, out, lse, stream);
  return dispatch<__bf16>(bs, d, q, k, v, pa, B, H, Mb, Nb, scale, opt, out, lse, stream);
}

}  // namespace bsa
