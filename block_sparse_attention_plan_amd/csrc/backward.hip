// Block-sparse attention backward (gfx950).
//
// Gradients of the forward in forward.hip for an upstream gradient dO.  The
// next.gr "Block Sparse Attention Techniques" tutorial ("Gradient Propagation
// in Block Sparse Attention") fixes that gradients flow through the live
// blocks only: dQ of query block m sums over the live tiles of its block row,
// dK and dV of key block n over the live tiles of its block column.  With the
// forward's lse saved, every tile is recomputed independently:
//   P   = exp(c(scale * Q K^T) - lse)      (c: optional tanh cap, masks -> 0)
//   dP  = dO V^T,   D_i = dO_i . out_i
//   dS  = P * (dP - D) * c'(.)
//   dQ  = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
//   dsink_h = -sum_i exp(sink_h - lse_i) D_i
//
// Three kernels (four at bs = 16), none with atomics, so every gradient is
// bit-for-bit repeatable:
//   bwd_dq_kernel    work item (b, h, query block m) over the row plan; the
//                    wave owning 32 query rows first forms its rows' D_i and
//                    lse_i * log2(e) (written to the workspace for the two
//                    kernels after it), keeps Q^T and dO^T in registers and
//                    computes S^T = K Q^T, dP^T = V dO^T and
//                    dQ^T += K^T dS^T (dS^T straight from the accumulators as
//                    the B operand, K^T by LDS transpose reads)
//   bwd_dkdv_kernel  work item (b, K/V head, key block n) over the column plan
//                    (the query heads of a group one after another); the wave
//                    owning 32 key rows keeps K^T and V^T in registers and
//                    computes S = Q K^T, dP = dO V^T, dV^T += dO^T P and
//                    dK^T += Q^T dS
//   bwd_dsink_kernel one workgroup per head, fixed-order reduction
// (bs = 16 runs bwd_pre_kernel for D and lse2, then one-wave kernels below.)
// Tiles travel from HBM straight into LDS (buffer_load_dwordx4 ... lds); each
// tile is read both row-wise (16-byte reads) and transposed
// (ds_read_b64_tr_b16), so its 16-byte chunks are XOR-swizzled per row with a
// pattern that keeps both read shapes free of bank conflicts.
// Instances of the bs >= 32 kernels by option set: plain; LITE (bf16) for the
// causal mask, cut last blocks and the cap, each decided per tile or at
// compile time so that no per-score test on an option remains; MASK + SEG
// for segment ids; MASK for fp32 I/O with any option.
#include <type_traits>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Packed sequences: a tile whose query and key segment ids have disjoint
// [min, max] ranges has only masked scores, so its weights are exactly zero
// and it adds nothing to any gradient; the bs >= 32 kernels skip it, copies
// included.  (Ranges only ever keep a tile too many; the element masks still
// decide every score.)

// [lo, hi] of the n ids at ids[0 ..], over one wave (lo > hi: none).
__device__ __forceinline__ void wave_id_range(const int32_t *ids, int n, int &lo, int &hi) {
  lo = INT32_MAX;
  hi = INT32_MIN;
  for (int i = __lane_id(); i < n; i += 64) {
    const int v = ids[i];
    lo = min(lo, v);
    hi = max(hi, v);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
}

// Bit i (i < 16, i < nblocks) set when id block i holds an id in [lo, hi].
// block(i, ids, len) names block i's ids; 16 lanes read each block (IPL ids
// per lane), four blocks per pass, the four passes' loads in flight
// together.  Every wave of a workgroup computes the same bits.
template <int IPL, typename F>
__device__ __forceinline__ uint32_t keep_bits16(F block, int nblocks, int lo, int hi) {
  const int lane = __lane_id();
  const int g = lane / 16, sub = lane % 16;
  int mn[4], mx[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    mn[p] = INT32_MAX;
    mx[p] = INT32_MIN;
    const int i = 4 * p + g;
    if (i < nblocks) {
      const int32_t *ids;
      int len;
      block(i, ids, len);
#pragma unroll
      for (int k = 0; k < IPL; ++k) {
        const int e = sub * IPL + k;
        if (e < len) {
          const int v = ids[e];
          mn[p] = min(mn[p], v);
          mx[p] = max(mx[p], v);
        }
      }
    }
  }
  uint32_t bits = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      mn[p] = min(mn[p], __shfl_xor(mn[p], o));
      mx[p] = max(mx[p], __shfl_xor(mx[p], o));
    }
    const uint64_t ball = __ballot(sub == 0 && mn[p] <= hi && mx[p] >= lo);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) bits |= (uint32_t)((ball >> (16 * gg)) & 1u) << (4 * p + gg);
  }
  return bits;
}

// Chunk c of tile row r sits at chunk c ^ f(r).  Row reads touch 16
// consecutive rows at one logical chunk (f is a bijection on r % 16 among the
// rows that share LDS banks); transpose reads touch 4 aligned rows at 4
// aligned chunks (f moves each of those rows to a different 64-byte bank
// group).  f depends on r % 16 only.
template <int D> struct BSwz {
  static __device__ __forceinline__ int f(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
  }
};

// Copy a contiguous BS x D bf16 tile into LDS with the swizzle; the NW waves
// of the workgroup share its 1 KiB copy instructions.  Only the first `bytes`
// bytes exist (a block cut at the sequence end): the rest read as zeros (the
// whole offset is per lane, where the buffer range check applies).
//
// A wave's successive copies are STEP rows apart, and the swizzle depends on
// the row modulo 16 only, so the per-lane offsets repeat with period P; copy
// j reuses the offset of copy j % P and moves the (scalar) buffer base by the
// whole periods instead, which keeps P vector registers live, not NI / NW.
template <int BS, int D, int NW>
__device__ __forceinline__ void copy_tile(const __bf16 *src, __bf16 *dst, int wid, int lane,
                                          uint32_t bytes = BS * D * 2) {
  constexpr int CPR = D / 8;
  constexpr int NI = BS * D * 2 / 1024;
  constexpr int RPI = 64 / CPR;
  constexpr int STEP = RPI * NW;
  constexpr int P0 = STEP % 16 == 0 ? 1 : STEP % 8 == 0 ? 2 : STEP % 4 == 0 ? 4
                   : STEP % 2 == 0 ? 8 : 16;
  constexpr int P = P0 < NI / NW ? P0 : NI / NW;
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  uint32_t voff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int row = RPI * (wid + NW * p) + lane / CPR;
    voff[p] = (uint32_t)((row * D + (((lane % CPR) ^ BSwz<D>::f(row)) << 3)) * 2);
  }
#pragma unroll
  for (int j = 0; j < NI / NW; ++j) {
    const uint32_t shift = (uint32_t)((j - j % P) * STEP * D * 2);   // bytes
    // the bytes left past `shift`, formed with scalar-capable signed max (a
    // saturating unsigned subtract exists only as a vector instruction, and a
    // descriptor built from a vector register makes the compiler wrap the
    // copy in a loop over its distinct values)
    const uint32_t left = (uint32_t)max((int)bytes - (int)shift, 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(src) + shift, left);
    copy16_to_lds(rs, dst + (wid + NW * j) * 512, voff[j % P], 0u);
  }
}

// Row operand: 8 elements of tile row `row`, logical chunk `chunk`
// (sw = f(row)).
template <int D>
__device__ __forceinline__ bf16x8 row_read(const __bf16 *tile, int row, int chunk, int sw) {
  return *reinterpret_cast<const bf16x8 *>(tile + row * D + ((chunk ^ sw) << 3));
}

// Transposed operand X^T (rows of X are the contraction index) for the 32
// columns of block dt and the 16 rows starting at r16 (a multiple of 16):
// this lane reads rows r16 + tr_r and r16 + tr_r + 8, columns
// 32 dt + 16 (G % 2) + 4 c_src .. +3 (the k-slot order of the 32x32x16
// accumulator layout).
template <int D>
__device__ __forceinline__ bf16x8 tr_read(const __bf16 *tile, int r16, int dt, int tr_r, int lc_off,
                                          int pc, int sw0, int sw8) {
  const int lc = 4 * dt + lc_off;
  const __bf16 *p0 = tile + (r16 + tr_r) * D + ((lc ^ sw0) << 3) + pc;
  const __bf16 *p8 = tile + (r16 + tr_r + 8) * D + ((lc ^ sw8) << 3) + pc;
  return cat4(lds_read_tr4(p0), lds_read_tr4(p8));
}

__device__ __forceinline__ void store4_bf16(__bf16 *p, float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
  *reinterpret_cast<bf16x4 *>(p) = r;
}

// The two I/O types: 8 consecutive elements as a bf16 MFMA operand (fp32
// rounds to nearest even, as the forward does), as floats, and 4 results
// stored in the I/O type.
template <typename T> struct BIo;
template <> struct BIo<__bf16> {
  static __device__ __forceinline__ bf16x8 load8(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
  }
  static __device__ __forceinline__ void load8f(const __bf16 *p, float (&x)[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  static __device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d) {
    store4_bf16(p, a, b, c, d);
  }
};
template <> struct BIo<float> {
  static __device__ __forceinline__ bf16x8 load8(const float *p) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    return to_bf16x8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
  }
  static __device__ __forceinline__ void load8f(const float *p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
  }
};

// One tile into the swizzled bf16 LDS layout: bf16 tiles by LDS copies, fp32
// tiles through registers (rounded to bf16).  Rows at or past `rows` (a block
// cut at the sequence end) become zeros.
template <int BS, int D, int NW, typename T>
__device__ __forceinline__ void stage_tile(const T *src, __bf16 *dst, int wid, int lane, int rows) {
  if constexpr (std::is_same<T, __bf16>::value) {
    copy_tile<BS, D, NW>(src, dst, wid, lane, (uint32_t)(rows * D * 2));
  } else {
    constexpr int CPR = D / 8;
    const int tid = wid * 64 + lane;
    for (int i = tid; i < BS * CPR; i += NW * 64) {
      const int row = i / CPR, ch = i % CPR;
      const bf16x8 x = row < rows ? BIo<T>::load8(src + row * D + ch * 8) : bf16x8{};
      *reinterpret_cast<bf16x8 *>(dst + row * D + ((ch ^ BSwz<D>::f(row)) << 3)) = x;
    }
  }
}

// D_i = dO_i . out_i (fp32 over bf16 products) and lse_i * log2(e), with
// +inf for a row without a live key (lse = -inf), so that its weights
// exp2(s - lse2) vanish.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const T *__restrict__ out,
                                                      const T *__restrict__ dout,
                                                      const float *__restrict__ lse, int64_t rows,
                                                      float *__restrict__ Dv,
                                                      float *__restrict__ lse2) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per workgroup pass
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < rows; r0 += (int64_t)gridDim.x * RPB) {
    const int64_t r = r0 + tid / LPR;
    float acc = 0.f;
    if (r < rows) {
      float a[8], g[8];
      BIo<T>::load8f(out + r * D + sub * 8, a);
      BIo<T>::load8f(dout + r * D + sub * 8, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(a[i], g[i], acc);
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (r < rows && sub == 0) {
      Dv[r] = acc;
      const float l = lse[r];
      lse2[r] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
    }
  }
}

// dsink_h = -sum over batch items and rows of exp2(sink_h log2 e - lse2) D.
__global__ void __launch_bounds__(256) bwd_dsink_kernel(const float *__restrict__ lse2,
                                                        const float *__restrict__ Dv,
                                                        const float *__restrict__ sink, int32_t B,
                                                        int32_t H, int64_t Sq,
                                                        float *__restrict__ dsink) {
  __shared__ float part[256];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const float s2 = sink[h] * kLog2e;
  float acc = 0.f;
  for (int b = 0; b < B; ++b) {
    const int64_t base = ((int64_t)b * H + h) * Sq;
    for (int64_t i = tid; i < Sq; i += 256) acc += fast_exp2(s2 - lse2[base + i]) * Dv[base + i];
  }
  part[tid] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) dsink[h] = -part[0];
}

// Options on one score of a recomputed tile (MASK instances): the tanh cap
// and its slope, then the weight exp2(c * scale_log2 - lse2).
struct Weight {
  float p, slope;
};
template <bool MASK>
__device__ __forceinline__ Weight weight(float s, float scale_log2, float l2, const FwdOptions &opt) {
  float slope = 1.f;
  if (MASK && opt.cap_k != 0.f) {
    // the forward's capped score b * tanh, with the tanh kept for the slope:
    // tanh(y) = 1 - 2 / (e^(2y) + 1), e^(2y) = exp2(s * k2)
    const float t = fmaf(-2.f, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s * opt.cap_k) + 1.f), 1.f);
    s = opt.cap_b * t;
    slope = fmaf(-t, t, 1.f);
  }
  return Weight{fast_exp2(fmaf(s, scale_log2, -l2)), slope};
}

// The capped weight of the LITE = 3 instances, the cap decided at compile
// time (the same operations as weight<true> with a cap).
__device__ __forceinline__ Weight weight_cap(float s, float scale_log2, float l2,
                                             const FwdOptions &opt) {
  const float t = fmaf(-2.f, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s * opt.cap_k) + 1.f), 1.f);
  return Weight{fast_exp2(fmaf(opt.cap_b * t, scale_log2, -l2)), fmaf(-t, t, 1.f)};
}

// SEG instances (calls with segment ids) also skip the tiles whose ids
// cannot meet.  LITE instances serve the causal mask and cut last blocks
// without cap or segment ids: the plain code, with the keys after each query
// (diagonal tiles) and the keys past a cut end (the last key tile) set to
// -inf before the weights, under one uniform branch per tile each.  Rows
// past a cut end weigh nothing through their lse2 of +inf.  LITE = 1: the
// causal mask on whole blocks; LITE = 2: cut last blocks, with or without
// the causal mask; LITE = 3: the tanh cap, with or without the causal mask
// and cut last blocks -- the cap decided at compile time, and the masked
// weights set to zero after it by one compare and select per score (a
// capped score of -inf would still be finite).
template <int BS, int D, typename T, bool MASK, bool SEG = false, int LITE = 0>
__global__ void __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(const T *__restrict__ q, const T *__restrict__ k,
              const T *__restrict__ v, const T *__restrict__ dout,
              const T *__restrict__ out, const float *__restrict__ lse,
              float *__restrict__ lse2, float *__restrict__ Dv,
              const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
              const int32_t *__restrict__ row_order, int32_t B, int32_t H, int32_t Mb, int32_t Nb,
              float scale_log2, float scale, const FwdOptions opt, T *__restrict__ dq) {
  constexpr int NW = BS / 32;
  constexpr int TILE = BS * D;
  constexpr int QC = D / 16;
  constexpr int JT = BS / 32;
  constexpr int DT = D / 32;

  __shared__ __attribute__((aligned(1024))) __bf16 Ks[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[TILE];
  __shared__ __attribute__((aligned(16))) int32_t Gk[SEG ? BS : 4];  // segment ids of the tile's keys

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
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int h2 = lane / 32, l32 = lane % 32;
  const int G = lane / 16, l16 = lane % 16;

  const int64_t bh = (int64_t)b * H + h;
  const int64_t Sq = opt.sq, Sk = opt.sk;
  const int64_t bkv = (int64_t)b * (H / opt.kv_group) + h / opt.kv_group;
  const T *kh = k + bkv * Sk * D;
  const T *vh = v + bkv * Sk * D;
  const int qrow = 32 * wid + l32;            // query row inside the block
  const int64_t i_row = (int64_t)m * BS + qrow;
  constexpr bool CUT = MASK || LITE >= 2;      // lengths may end inside a block
  const bool q_ok = !CUT || i_row < Sq;        // rows past a cut last block
  const int qsg = (MASK && opt.qseg && q_ok) ? opt.qseg[(int64_t)b * Sq + i_row] : 0;

  // D_i = dO_i . out_i (fp32 over the I/O values) and lse_i log2 e of this
  // lane's row (+inf for a row without a live key, so that its weights
  // vanish); lane l and l + 32 each hold half of the row.  Written to the
  // workspace for the dK/dV and d sink kernels, which run after this one.
  float dd = 0.f, l2 = __builtin_inff();
  {
    float part = 0.f;
    if (q_ok) {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        float o8[8], g8[8];
        BIo<T>::load8f(out + (bh * Sq + i_row) * D + 16 * c + 8 * h2, o8);
        BIo<T>::load8f(dout + (bh * Sq + i_row) * D + 16 * c + 8 * h2, g8);
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf(o8[i], g8[i], part);
      }
      const float l = lse[bh * Sq + i_row];
      l2 = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
    }
    dd = sum_xor32(part);
    if (q_ok && h2 == 0) {
      Dv[bh * Sq + i_row] = dd;
      lse2[bh * Sq + i_row] = l2;
    }
  }
  bf16x8 qf[QC], gf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    qf[c] = q_ok ? BIo<T>::load8(q + (bh * Sq + i_row) * D + 16 * c + 8 * h2) : bf16x8{};
    gf[c] = q_ok ? BIo<T>::load8(dout + (bh * Sq + i_row) * D + 16 * c + 8 * h2) : bf16x8{};
  }
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  const int sw_row = BSwz<D>::f(l32);
  const int tr_r = 4 * h2 + l16 / 4;
  const int c_src = l16 % 4;
  const int lc_off = 2 * (G % 2) + c_src / 2, pc = 4 * (c_src % 2);
  const int sw0 = BSwz<D>::f(tr_r), sw8 = BSwz<D>::f(tr_r + 8);

  // segment ids: the block row's query id range, and keep bits for the
  // row's tiles, 16 at a time
  int qlo = 0, qhi = 0;
  uint32_t keep = 0;
  if constexpr (SEG)
    wave_id_range(opt.qseg + (int64_t)b * Sq + (int64_t)m * BS,
                  (int)min((int64_t)BS, Sq - (int64_t)m * BS), qlo, qhi);
  for (int t = beg; t < end; ++t) {
    if constexpr (SEG) {
      if ((t - beg) % 16 == 0)
        keep = keep_bits16<BS / 16>(
            [&](int i, const int32_t *&ids, int &len) {
              const int64_t k0 = (int64_t)col_idx[t + i] * BS;
              ids = opt.kseg + (int64_t)b * Sk + k0;
              len = (int)min((int64_t)BS, Sk - k0);
            },
            min(16, end - t), qlo, qhi);
      if (!((keep >> ((t - beg) % 16)) & 1u)) continue;   // no key shares a segment
    }
    const int ncol = col_idx[t];
    if ((MASK || LITE != 0) && opt.causal && ncol > m) continue;  // every key after every query
    __syncthreads();                                // previous tile fully read
    const int kv = CUT ? (int)min((int64_t)BS, Sk - (int64_t)ncol * BS) : BS;  // keys that exist
    stage_tile<BS, D, NW, T>(kh + (int64_t)ncol * TILE, Ks, wid, lane, kv);
    stage_tile<BS, D, NW, T>(vh + (int64_t)ncol * TILE, Vs, wid, lane, kv);
    if constexpr (SEG)
      if (tid < BS) Gk[tid] = tid < kv ? opt.kseg[(int64_t)b * Sk + (int64_t)ncol * BS + tid] : 0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool diag = MASK && opt.causal && ncol == m;
    int limit = BS;   // LITE = 3: keys at or past it weigh nothing
    if constexpr (LITE == 3) {
      if (opt.causal && ncol == m) limit = qrow + 1;
      limit = min(limit, kv);
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        s = mfma32(row_read<D>(Ks, 32 * jt + l32, 2 * c + h2, sw_row), qf[c], s);
        dp = mfma32(row_read<D>(Vs, 32 * jt + l32, 2 * c + h2, sw_row), gf[c], dp);
      }
      if constexpr (LITE == 1 || LITE == 2) {
        if ((LITE == 1 || opt.causal) && ncol == m) {  // the diagonal tile: keys after the query weigh nothing
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * jt + 8 * (e / 4) + 4 * h2 + (e % 4) > qrow) s[e] = -__builtin_inff();
        }
        if (LITE == 2 && kv < BS) {  // the cut last key tile: keys past the end weigh nothing
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * jt + 8 * (e / 4) + 4 * h2 + (e % 4) >= kv) s[e] = -__builtin_inff();
        }
      }
      // S^T[key][query]: key 32jt + 8(e/4) + 4h2 + e%4, query qrow
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const Weight wt = LITE == 3 ? weight_cap(s[e], scale_log2, l2, opt)
                                    : weight<MASK>(s[e], scale_log2, l2, opt);
        float p = wt.p;
        if constexpr (LITE == 3) p = 32 * jt + 8 * (e / 4) + 4 * h2 + (e % 4) >= limit ? 0.f : p;
        if (diag && 32 * jt + 8 * (e / 4) + 4 * h2 + (e % 4) > qrow) p = 0.f;
        if (MASK && 32 * jt + 8 * (e / 4) + 4 * h2 + (e % 4) >= kv) p = 0.f;
        if constexpr (SEG) {  // packed sequences: only keys of the query's segment
          // the 4 keys 32jt + 8(e/4) + 4h2 + 0..3 are consecutive: one 16-byte read
          const int4 g4 = *reinterpret_cast<const int4 *>(&Gk[32 * jt + 8 * (e / 4) + 4 * h2]);
          const int kid = (e % 4) == 0 ? g4.x : (e % 4) == 1 ? g4.y : (e % 4) == 2 ? g4.z : g4.w;
          if (kid != qsg) p = 0.f;
        }
        s[e] = p * (dp[e] - dd) * wt.slope;
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 dsf = to_bf16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                                     s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = mfma32(tr_read<D>(Ks, 32 * jt + 16 * c2, dt, tr_r, lc_off, pc, sw0, sw8), dsf,
                           acc[dt]);
      }
      if constexpr (!MASK && (LITE == 0 || LITE == 3)) {
        // S and dP: four row reads ahead, then one per product; dQ: two
        // transpose reads per product (blocks without branches only)
        sched_interleave<2 * QC, 2 * QC, 4, 0>();
        sched_steps<0, 2 * DT, 2, 0>();
      }
    }
  }
  if (!q_ok) return;
  T *dqh = dq + (bh * Sq + i_row) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      BIo<T>::store4(dqh + 32 * dt + 8 * a + 4 * h2, scale * acc[dt][4 * a],
                     scale * acc[dt][4 * a + 1], scale * acc[dt][4 * a + 2],
                     scale * acc[dt][4 * a + 3]);
}

template <int BS, int D, typename T, bool MASK, bool SEG = false, int LITE = 0>
__global__ void __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkdv_kernel(const T *__restrict__ q, const T *__restrict__ k,
                const T *__restrict__ v, const T *__restrict__ dout,
                const float *__restrict__ lse2, const float *__restrict__ Dv,
                const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ row_idx,
                const int32_t *__restrict__ col_order, int32_t B, int32_t H, int32_t Hkv,
                int32_t Mb, int32_t Nb, float scale_log2, float scale, const FwdOptions opt,
                T *__restrict__ dk, T *__restrict__ dv) {
  constexpr int NW = BS / 32;
  constexpr int TILE = BS * D;
  constexpr int QC = D / 16;
  constexpr int JT = BS / 32;
  constexpr int DT = D / 32;

  __shared__ __attribute__((aligned(1024))) __bf16 Qs[TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 Gs[TILE];   // dO tile
  __shared__ __attribute__((aligned(16))) float Ls[BS];         // lse2 of the tile's rows
  __shared__ __attribute__((aligned(16))) float Ds[BS];         // D of the tile's rows
  __shared__ __attribute__((aligned(16))) int32_t Gq[BS];       // segment ids of the tile's rows

  const int64_t W = (int64_t)B * Hkv * Nb;
  const int64_t per = (W + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= W) return;
  const int64_t KN = (int64_t)Hkv * Nb;
  const int b = (int)(w / KN);
  const int item = col_order[w % KN];
  const int kvh = item / Nb;
  const int n = item % Nb;
  const int g = H / Hkv;

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int h2 = lane / 32, l32 = lane % 32;
  const int G = lane / 16, l16 = lane % 16;

  const int64_t Sq = opt.sq, Sk = opt.sk;
  const int64_t bkv = (int64_t)b * Hkv + kvh;
  const int krow = 32 * wid + l32;            // key row inside the block
  const int64_t j_row = (int64_t)n * BS + krow;
  constexpr bool CUT = MASK || LITE >= 2;      // lengths may end inside a block
  const bool k_ok = !CUT || j_row < Sk;        // keys past a cut last block
  const int ksg = (MASK && opt.kseg && k_ok) ? opt.kseg[(int64_t)b * Sk + j_row] : 0;

  bf16x8 kf[QC], vf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    kf[c] = k_ok ? BIo<T>::load8(k + (bkv * Sk + j_row) * D + 16 * c + 8 * h2) : bf16x8{};
    vf[c] = k_ok ? BIo<T>::load8(v + (bkv * Sk + j_row) * D + 16 * c + 8 * h2) : bf16x8{};
  }
  f32x16 ak[DT], av[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    ak[dt] = f32x16{};
    av[dt] = f32x16{};
  }

  const int sw_row = BSwz<D>::f(l32);
  const int tr_r = 4 * h2 + l16 / 4;
  const int c_src = l16 % 4;
  const int lc_off = 2 * (G % 2) + c_src / 2, pc = 4 * (c_src % 2);
  const int sw0 = BSwz<D>::f(tr_r), sw8 = BSwz<D>::f(tr_r + 8);

  // segment ids: the key block's id range, and keep bits for the visited
  // tiles of each query head, 16 at a time
  int klo = 0, khi = 0;
  uint32_t keep = 0;
  if constexpr (SEG)
    wave_id_range(opt.kseg + (int64_t)b * Sk + (int64_t)n * BS,
                  (int)min((int64_t)BS, Sk - (int64_t)n * BS), klo, khi);
  for (int hh = 0; hh < g; ++hh) {
    const int h = kvh * g + hh;
    const int64_t bh = (int64_t)b * H + h;
    const int beg = col_ptr[h * Nb + n];
    const int end = col_ptr[h * Nb + n + 1];
    for (int t = beg; t < end; ++t) {
      if constexpr (SEG) {
        if ((t - beg) % 16 == 0)
          keep = keep_bits16<BS / 16>(
              [&](int i, const int32_t *&ids, int &len) {
                const int64_t q0 = (int64_t)row_idx[t + i] * BS;
                ids = opt.qseg + (int64_t)b * Sq + q0;
                len = (int)min((int64_t)BS, Sq - q0);
              },
              min(16, end - t), klo, khi);
        if (!((keep >> ((t - beg) % 16)) & 1u)) continue;   // no query shares a segment
      }
      const int m = row_idx[t];
      if ((MASK || LITE != 0) && opt.causal && m < n) continue;  // every key after every query
      __syncthreads();                              // previous tile fully read
      const int qv = CUT ? (int)min((int64_t)BS, Sq - (int64_t)m * BS) : BS;  // rows that exist
      stage_tile<BS, D, NW, T>(q + (bh * Sq + (int64_t)m * BS) * D, Qs, wid, lane, qv);
      stage_tile<BS, D, NW, T>(dout + (bh * Sq + (int64_t)m * BS) * D, Gs, wid, lane, qv);
      if (tid < BS) {
        // rows past a cut last block: weight exp2(s - inf) = 0
        Ls[tid] = tid < qv ? lse2[bh * Sq + (int64_t)m * BS + tid] : __builtin_inff();
        Ds[tid] = tid < qv ? Dv[bh * Sq + (int64_t)m * BS + tid] : 0.f;
        if (MASK && opt.qseg) Gq[tid] = tid < qv ? opt.qseg[(int64_t)b * Sq + (int64_t)m * BS + tid] : 0;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool diag = MASK && opt.causal && m == n;
      int qlim = 0;   // LITE = 3: queries before it weigh nothing (diagonal tile)
      if constexpr (LITE == 3)
        if (opt.causal && m == n) qlim = krow;
      // One 32-query chunk at a time: K^T, V^T and both accumulators stay
      // live across the loop, so the chunks are not unrolled into each other,
      // and each chunk runs in phases (fenced against the scheduler) that keep
      // at most one fp32 score block live besides them:
      //   S = Q K^T -> P (bf16, and P * cap slope for the MASK instances)
      //   dV^T += dO^T P beside dP = dO V^T
      //   dS = P (dP - D) from the bf16 P -> dK^T += Q^T dS
#pragma unroll 1
      for (int jq = 0; jq < JT; ++jq) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int c = 0; c < QC; ++c)
          s = mfma32(row_read<D>(Qs, 32 * jq + l32, 2 * c + h2, sw_row), kf[c], s);
        // (LITE: rows past a cut end weigh nothing through lse2 = +inf, and a
        // key past it only feeds its own dK and dV rows, which are not stored)
        if constexpr (LITE == 1 || LITE == 2) {
          if ((LITE == 1 || opt.causal) && m == n) {  // the diagonal tile: this key weighs nothing for earlier queries
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (krow > 32 * jq + 8 * (e / 4) + 4 * h2 + (e % 4)) s[e] = -__builtin_inff();
          }
        }
        // S[query][key]: query 32jq + 8(e/4) + 4h2 + e%4, key krow
        constexpr bool SLOPE = MASK || LITE == 3;   // weights carry a cap slope
        f32x16 w;   // P times the cap slope (SLOPE instances)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&Ls[32 * jq + 8 * a + 4 * h2]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * a + i;
            const Weight wt = LITE == 3 ? weight_cap(s[e], scale_log2, l4[i], opt)
                                        : weight<MASK>(s[e], scale_log2, l4[i], opt);
            float p = wt.p;
            if constexpr (LITE == 3) p = 32 * jq + 8 * a + 4 * h2 + i < qlim ? 0.f : p;
            if (diag && krow > 32 * jq + 8 * a + 4 * h2 + i) p = 0.f;
            if (!k_ok) p = 0.f;
            if (MASK && opt.qseg && Gq[32 * jq + 8 * a + 4 * h2 + i] != ksg) p = 0.f;
            s[e] = p;
            if constexpr (SLOPE) w[e] = p * wt.slope;
          }
        }
        bf16x8 pf[2], wf[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          pf[c2] = to_bf16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                             s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
          if constexpr (SLOPE)
            wf[c2] = to_bf16x8(w[8 * c2 + 0], w[8 * c2 + 1], w[8 * c2 + 2], w[8 * c2 + 3],
                               w[8 * c2 + 4], w[8 * c2 + 5], w[8 * c2 + 6], w[8 * c2 + 7]);
          else
            wf[c2] = pf[c2];
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 dp = f32x16{};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            av[dt] = mfma32(tr_read<D>(Gs, 32 * jq + 16 * c2, dt, tr_r, lc_off, pc, sw0, sw8),
                            pf[c2], av[dt]);
#pragma unroll
        for (int c = 0; c < QC; ++c)
          dp = mfma32(row_read<D>(Gs, 32 * jq + l32, 2 * c + h2, sw_row), vf[c], dp);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&Ds[32 * jq + 8 * a + 4 * h2]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * a + i;
            dp[e] = (float)wf[e / 8][e % 8] * (dp[e] - d4[i]);
          }
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16x8 dsf = to_bf16x8(dp[8 * c2 + 0], dp[8 * c2 + 1], dp[8 * c2 + 2],
                                       dp[8 * c2 + 3], dp[8 * c2 + 4], dp[8 * c2 + 5],
                                       dp[8 * c2 + 6], dp[8 * c2 + 7]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            ak[dt] = mfma32(tr_read<D>(Qs, 32 * jq + 16 * c2, dt, tr_r, lc_off, pc, sw0, sw8), dsf,
                            ak[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!k_ok) return;
  T *dkr = dk + (bkv * Sk + j_row) * D;
  T *dvr = dv + (bkv * Sk + j_row) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      BIo<T>::store4(dkr + 32 * dt + 8 * a + 4 * h2, scale * ak[dt][4 * a],
                     scale * ak[dt][4 * a + 1], scale * ak[dt][4 * a + 2],
                     scale * ak[dt][4 * a + 3]);
      BIo<T>::store4(dvr + 32 * dt + 8 * a + 4 * h2, av[dt][4 * a], av[dt][4 * a + 1],
                     av[dt][4 * a + 2], av[dt][4 * a + 3]);
    }
}

// Block size 16: one wave per work item and 16x16 tiles.
//   bwd_dq16_kernel    S^T = K Q^T and dP^T = V dO^T (16x16x32; K and V rows
//                      from LDS, Q^T and dO^T in registers), then
//                      dQ^T += K^T dS^T (16x16x16; K^T by transpose reads,
//                      dS^T straight from the accumulators as the B operand)
//   bwd_dkdv16_kernel  S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//                      dK^T += Q^T dS the same way
// Tiles sit in LDS row-major with rows padded by 16 bytes.
template <int D> constexpr int kStr16 = D + 8;

// A 16 x D tile into LDS (rows at or past `rows` become zeros); one wave.
template <int D, typename T>
__device__ __forceinline__ void stage16(const T *src, __bf16 *dst, int lane, int rows) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = lane; i < 16 * CPR; i += 64) {
    const int row = i / CPR, ch = i % CPR;
    const bf16x8 x = row < rows ? BIo<T>::load8(src + row * D + ch * 8) : bf16x8{};
    *reinterpret_cast<bf16x8 *>(dst + row * kStr16<D> + ch * 8) = x;
  }
}

// Row operand of a 16x16x32 product: tile row `row`, elements 32 c + 8 G ..
template <int D>
__device__ __forceinline__ bf16x8 row16(const __bf16 *tile, int row, int c, int G) {
  return *reinterpret_cast<const bf16x8 *>(tile + row * kStr16<D> + 32 * c + 8 * G);
}

// Transposed operand of a 16x16x16 product: tile rows 4G .. 4G+3 (the
// contraction index) of column d0 + l16.
template <int D>
__device__ __forceinline__ bf16x4 tr16(const __bf16 *tile, int d0, int G, int l16) {
  return lds_read_tr4(tile + (4 * G + l16 / 4) * kStr16<D> + d0 + 4 * (l16 % 4));
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
  return r;
}

template <int D, typename T, bool MASK>
__global__ void __launch_bounds__(64)
bwd_dq16_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                const T *__restrict__ dout, const float *__restrict__ lse2,
                const float *__restrict__ Dv, const int32_t *__restrict__ row_ptr,
                const int32_t *__restrict__ col_idx, const int32_t *__restrict__ row_order,
                int32_t B, int32_t H, int32_t Mb, int32_t Nb, float scale_log2, float scale,
                const FwdOptions opt, T *__restrict__ dq) {
  constexpr int QC = D / 32;   // 32-wide k steps of the score products
  constexpr int DT = D / 16;   // 16-wide d tiles of dQ^T
  __shared__ __attribute__((aligned(16))) __bf16 Ks[16 * kStr16<D>];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[16 * kStr16<D>];

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

  const int lane = threadIdx.x;
  const int G = lane / 16, l16 = lane % 16;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t Sq = opt.sq, Sk = opt.sk;
  const int64_t bkv = (int64_t)b * (H / opt.kv_group) + h / opt.kv_group;
  const T *kh = k + bkv * Sk * D;
  const T *vh = v + bkv * Sk * D;
  const int64_t i_row = (int64_t)m * 16 + l16;   // this lane's query (a column of S^T)
  const bool q_ok = !MASK || i_row < Sq;
  const int qsg = (MASK && opt.qseg && q_ok) ? opt.qseg[(int64_t)b * Sq + i_row] : 0;
  const float l2 = q_ok ? lse2[bh * Sq + i_row] : __builtin_inff();
  const float dd = q_ok ? Dv[bh * Sq + i_row] : 0.f;

  bf16x8 qf[QC], gf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    qf[c] = q_ok ? BIo<T>::load8(q + (bh * Sq + i_row) * D + 32 * c + 8 * G) : bf16x8{};
    gf[c] = q_ok ? BIo<T>::load8(dout + (bh * Sq + i_row) * D + 32 * c + 8 * G) : bf16x8{};
  }
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = beg; t < end; ++t) {
    const int ncol = col_idx[t];
    if (MASK && opt.causal && ncol > m) continue;   // every key after every query
    __syncthreads();                                // previous tile fully read
    const int kv = MASK ? (int)min((int64_t)16, Sk - (int64_t)ncol * 16) : 16;  // keys that exist
    stage16<D, T>(kh + (int64_t)ncol * 16 * D, Ks, lane, kv);
    stage16<D, T>(vh + (int64_t)ncol * 16 * D, Vs, lane, kv);
    __syncthreads();
    const bool diag = MASK && opt.causal && ncol == m;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      s = mfma16(row16<D>(Ks, l16, c, G), qf[c], s);
      dp = mfma16(row16<D>(Vs, l16, c, G), gf[c], dp);
    }
    // S^T[key][query]: key 4G + e, query l16
    float ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 4 * G + e;
      const Weight wt = weight<MASK>(s[e], scale_log2, l2, opt);
      float p = wt.p;
      if (diag && key > l16) p = 0.f;
      if (MASK && key >= kv) p = 0.f;
      if (MASK && opt.qseg && key < kv &&
          opt.kseg[(int64_t)b * Sk + (int64_t)ncol * 16 + key] != qsg)
        p = 0.f;
      ds[e] = p * (dp[e] - dd) * wt.slope;
    }
    const bf16x4 dsb = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma16k16(tr16<D>(Ks, 16 * dt, G, l16), dsb, acc[dt]);
  }
  if (!q_ok) return;
  T *dqh = dq + (bh * Sq + i_row) * D + 4 * G;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    BIo<T>::store4(dqh + 16 * dt, scale * acc[dt][0], scale * acc[dt][1], scale * acc[dt][2],
                   scale * acc[dt][3]);
}

template <int D, typename T, bool MASK>
__global__ void __launch_bounds__(64)
bwd_dkdv16_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                  const T *__restrict__ dout, const float *__restrict__ lse2,
                  const float *__restrict__ Dv, const int32_t *__restrict__ col_ptr,
                  const int32_t *__restrict__ row_idx, const int32_t *__restrict__ col_order,
                  int32_t B, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, float scale_log2,
                  float scale, const FwdOptions opt, T *__restrict__ dk, T *__restrict__ dv) {
  constexpr int QC = D / 32;
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 Qs[16 * kStr16<D>];
  __shared__ __attribute__((aligned(16))) __bf16 Gs[16 * kStr16<D>];   // dO tile
  __shared__ float Ls[16], Ds[16];
  __shared__ int32_t Gq[16];

  const int64_t W = (int64_t)B * Hkv * Nb;
  const int64_t per = (W + 7) / 8;
  const int64_t w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (w >= W) return;
  const int64_t KN = (int64_t)Hkv * Nb;
  const int b = (int)(w / KN);
  const int item = col_order[w % KN];
  const int kvh = item / Nb;
  const int n = item % Nb;
  const int g = H / Hkv;

  const int lane = threadIdx.x;
  const int G = lane / 16, l16 = lane % 16;
  const int64_t Sq = opt.sq, Sk = opt.sk;
  const int64_t bkv = (int64_t)b * Hkv + kvh;
  const int64_t j_row = (int64_t)n * 16 + l16;   // this lane's key (a column of S)
  const bool k_ok = !MASK || j_row < Sk;
  const int ksg = (MASK && opt.kseg && k_ok) ? opt.kseg[(int64_t)b * Sk + j_row] : 0;

  bf16x8 kf[QC], vf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    kf[c] = k_ok ? BIo<T>::load8(k + (bkv * Sk + j_row) * D + 32 * c + 8 * G) : bf16x8{};
    vf[c] = k_ok ? BIo<T>::load8(v + (bkv * Sk + j_row) * D + 32 * c + 8 * G) : bf16x8{};
  }
  f32x4 ak[DT], av[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) ak[dt] = av[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int hh = 0; hh < g; ++hh) {
    const int h = kvh * g + hh;
    const int64_t bh = (int64_t)b * H + h;
    const int beg = col_ptr[h * Nb + n];
    const int end = col_ptr[h * Nb + n + 1];
    for (int t = beg; t < end; ++t) {
      const int m = row_idx[t];
      if (MASK && opt.causal && m < n) continue;    // every key after every query
      __syncthreads();                              // previous tile fully read
      const int qv = MASK ? (int)min((int64_t)16, Sq - (int64_t)m * 16) : 16;  // rows that exist
      stage16<D, T>(q + (bh * Sq + (int64_t)m * 16) * D, Qs, lane, qv);
      stage16<D, T>(dout + (bh * Sq + (int64_t)m * 16) * D, Gs, lane, qv);
      if (lane < 16) {
        // rows past a cut last block: weight exp2(s - inf) = 0
        Ls[lane] = lane < qv ? lse2[bh * Sq + (int64_t)m * 16 + lane] : __builtin_inff();
        Ds[lane] = lane < qv ? Dv[bh * Sq + (int64_t)m * 16 + lane] : 0.f;
        if (MASK && opt.qseg) Gq[lane] = lane < qv ? opt.qseg[(int64_t)b * Sq + (int64_t)m * 16 + lane] : 0;
      }
      __syncthreads();
      const bool diag = MASK && opt.causal && m == n;
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        s = mfma16(row16<D>(Qs, l16, c, G), kf[c], s);
        dp = mfma16(row16<D>(Gs, l16, c, G), vf[c], dp);
      }
      // S[query][key]: query 4G + e, key l16
      float pw[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int qr = 4 * G + e;
        const Weight wt = weight<MASK>(s[e], scale_log2, Ls[qr], opt);
        float p = wt.p;
        if (diag && l16 > qr) p = 0.f;
        if (!k_ok) p = 0.f;
        if (MASK && opt.qseg && Gq[qr] != ksg) p = 0.f;
        pw[e] = p;
        ds[e] = p * (dp[e] - Ds[qr]) * wt.slope;
      }
      const bf16x4 pb = to_bf16x4(pw[0], pw[1], pw[2], pw[3]);
      const bf16x4 dsb = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        av[dt] = mfma16k16(tr16<D>(Gs, 16 * dt, G, l16), pb, av[dt]);
        ak[dt] = mfma16k16(tr16<D>(Qs, 16 * dt, G, l16), dsb, ak[dt]);
      }
    }
  }
  if (!k_ok) return;
  T *dkr = dk + (bkv * Sk + j_row) * D + 4 * G;
  T *dvr = dv + (bkv * Sk + j_row) * D + 4 * G;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    BIo<T>::store4(dkr + 16 * dt, scale * ak[dt][0], scale * ak[dt][1], scale * ak[dt][2],
                   scale * ak[dt][3]);
    BIo<T>::store4(dvr + 16 * dt, av[dt][0], av[dt][1], av[dt][2], av[dt][3]);
  }
}

template <int D, typename T, bool MASK>
hipError_t launch_grads16(const BwdArgs &a, hipStream_t stream) {
  const float scale_log2 = a.scale * kLog2e;
  {
    const int64_t W = (int64_t)a.B * a.H * a.Mb;
    const int64_t grid = (W + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq16_kernel<D, T, MASK>), dim3((unsigned)grid), dim3(64), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.dout, a.lse2,
                       a.Dv, a.row_ptr, a.col_idx, a.row_order, a.B, a.H, a.Mb, a.Nb, scale_log2,
                       a.scale, a.opt, (T *)a.dq);
  }
  {
    const int32_t Hkv = a.H / a.opt.kv_group;
    const int64_t W = (int64_t)a.B * Hkv * a.Nb;
    const int64_t grid = (W + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv16_kernel<D, T, MASK>), dim3((unsigned)grid), dim3(64), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.dout, a.lse2,
                       a.Dv, a.col_ptr, a.row_idx, a.col_order, a.B, a.H, Hkv, a.Mb, a.Nb,
                       scale_log2, a.scale, a.opt, (T *)a.dk, (T *)a.dv);
  }
  return hipGetLastError();
}

template <int BS, int D, typename T, bool MASK, bool SEG = false, int LITE = 0>
hipError_t launch_grads(const BwdArgs &a, hipStream_t stream) {
  const float scale_log2 = a.scale * kLog2e;
  {
    const int64_t W = (int64_t)a.B * a.H * a.Mb;
    const int64_t grid = (W + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<BS, D, T, MASK, SEG, LITE>), dim3((unsigned)grid), dim3(BS * 2), 0,
                       stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v,
                       (const T *)a.dout, (const T *)a.out, a.lse, a.lse2, a.Dv, a.row_ptr,
                       a.col_idx, a.row_order,
                       a.B, a.H, a.Mb, a.Nb, scale_log2, a.scale, a.opt, (T *)a.dq);
  }
  {
    const int32_t Hkv = a.H / a.opt.kv_group;
    const int64_t W = (int64_t)a.B * Hkv * a.Nb;
    const int64_t grid = (W + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<BS, D, T, MASK, SEG, LITE>), dim3((unsigned)grid), dim3(BS * 2),
                       0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v,
                       (const T *)a.dout, a.lse2, a.Dv, a.col_ptr, a.row_idx, a.col_order,
                       a.B, a.H, Hkv, a.Mb, a.Nb, scale_log2, a.scale, a.opt, (T *)a.dk,
                       (T *)a.dv);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_pre(const BwdArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.opt.sq;
  const int64_t rpb = 256 / (D / 8);
  int64_t grid = (rows + rpb - 1) / rpb;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const T *)a.out, (const T *)a.dout, a.lse, rows, a.Dv, a.lse2);
  return hipGetLastError();
}

}  // namespace

bool backward_supported(int32_t bs, int32_t d) {
  return (bs == 16 || bs == 32 || bs == 64 || bs == 128) && (d == 32 || d == 64 || d == 128);
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t stream) {
  if (!backward_supported(a.bs, a.d)) return hipErrorInvalidValue;
  if (a.opt.kv_group < 1 || a.H % a.opt.kv_group != 0) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  // bs = 16: D and lse2 by their own pass; larger blocks: by the dQ kernel
  if (a.bs == 16) {
    if (a.f32)
      e = a.d == 32 ? launch_pre<float, 32>(a, stream)
        : a.d == 64 ? launch_pre<float, 64>(a, stream)
                    : launch_pre<float, 128>(a, stream);
    else
      e = a.d == 32 ? launch_pre<__bf16, 32>(a, stream)
        : a.d == 64 ? launch_pre<__bf16, 64>(a, stream)
                    : launch_pre<__bf16, 128>(a, stream);
    if (e != hipSuccess) return e;
  }
  const bool mask = a.opt.cap_k != 0.f || a.opt.causal != 0 || a.opt.sq % a.bs != 0 ||
                    a.opt.sk % a.bs != 0 || a.opt.qseg != nullptr;
  const bool seg = a.opt.qseg != nullptr;
  // the causal mask and cut last blocks without cap or segment ids (bf16)
  // have instances of their own that mask the diagonal and last tiles only
  const bool lite = mask && a.opt.cap_k == 0.f && a.opt.qseg == nullptr;
  const bool whole = a.opt.sq % a.bs == 0 && a.opt.sk % a.bs == 0;
  // the cap without segment ids (bf16) likewise: the cap decided at compile
  // time, the masks by a select per score.  (Every other bf16 call with a
  // mask has segment ids, so the bf16 MASK instances are the SEG ones.)
  const bool capped = a.opt.cap_k != 0.f && a.opt.qseg == nullptr;
#define BSA_BWD_CASE(BS_, D_)                                                                  \
  if (a.bs == BS_ && a.d == D_)                                                               \
    e = a.f32 ? (seg    ? launch_grads<BS_, D_, float, true, true>(a, stream)                 \
                 : mask ? launch_grads<BS_, D_, float, true>(a, stream)                       \
                        : launch_grads<BS_, D_, float, false>(a, stream))                     \
              : (seg      ? launch_grads<BS_, D_, __bf16, true, true>(a, stream)              \
                 : lite   ? (whole ? launch_grads<BS_, D_, __bf16, false, false, 1>(a, stream) \
                                   : launch_grads<BS_, D_, __bf16, false, false, 2>(a, stream))\
                 : capped ? launch_grads<BS_, D_, __bf16, false, false, 3>(a, stream)         \
                          : launch_grads<BS_, D_, __bf16, false>(a, stream));
#define BSA_BWD16_CASE(D_)                                                                     \
  if (a.bs == 16 && a.d == D_)                                                                \
    e = a.f32 ? (mask ? launch_grads16<D_, float, true>(a, stream)                            \
                      : launch_grads16<D_, float, false>(a, stream))                          \
              : (mask ? launch_grads16<D_, __bf16, true>(a, stream)                           \
                      : launch_grads16<D_, __bf16, false>(a, stream));
  BSA_BWD16_CASE(32) BSA_BWD16_CASE(64) BSA_BWD16_CASE(128)
#undef BSA_BWD16_CASE
  BSA_BWD_CASE(32, 32) BSA_BWD_CASE(32, 64) BSA_BWD_CASE(32, 128)
  BSA_BWD_CASE(64, 32) BSA_BWD_CASE(64, 64) BSA_BWD_CASE(64, 128)
  BSA_BWD_CASE(128, 32) BSA_BWD_CASE(128, 64) BSA_BWD_CASE(128, 128)
#undef BSA_BWD_CASE
  if (e != hipSuccess) return e;
  if (a.opt.sink != nullptr && a.dsink != nullptr) {
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(a.H), dim3(256), 0, stream, (const float *)a.lse2,
                       (const float *)a.Dv, a.opt.sink, a.B, a.H, (int64_t)a.opt.sq, a.dsink);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace bsa
