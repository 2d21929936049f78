// Content-adaptive block layout (gfx950).
//
// The next.gr "Block Sparse Attention Techniques" tutorial ("Fixed vs.
// Adaptive Block Sparsity") marks a block pair live when the similarity of
// its queries and keys reaches a threshold tau, naming cosine similarity;
// the Language AI Handbook scores such candidates at a coarser granularity
// than tokens.  Here a block is represented by the mean of its rows, so for
// one batch item
//   live(h, m, n) = cos(mean q[h, block m], mean k[h / g, block n]) >= tau
// with optional causal (n <= m only) and forced-diagonal (n == m always)
// rules.  Two kernels:
//   pool   one wave per (head, block): fp32 sum of the block's rows in a
//          fixed order, then the unit vector (zero for a zero sum) into the
//          workspace.  Reads q and k once: bound by HBM.
//   score  one workgroup per (head, 64 block rows, 64 block columns): the
//          unit vectors staged in LDS with 16-byte copies (rows padded by
//          four floats), each thread 4 x 4 fp32 dot products from 16-byte
//          reads (eight reads feed 64 FMAs), the threshold, and optionally
//          the scores themselves.  Under the causal rule, a tile wholly
//          above the diagonal only writes zeros when no scores are asked
//          for.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

template <typename T> __device__ __forceinline__ void load8f(const T *p, float (&x)[8]);
template <> __device__ __forceinline__ void load8f<__bf16>(const __bf16 *p, float (&x)[8]) {
  const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
template <> __device__ __forceinline__ void load8f<float>(const float *p, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// Unit block means: item i < nq is query block (h, m) = (i / Mb, i % Mb) of
// q, otherwise key block (i - nq) of k (K/V head, n).  Lanes split a row into
// D/8 pieces of 8 elements; 64 / (D/8) rows are summed side by side and then
// folded together, so the order of every sum is fixed.
template <typename T, int D>
__global__ void __launch_bounds__(256) adaptive_pool_kernel(const T *__restrict__ q,
                                                            const T *__restrict__ k, int32_t nq,
                                                            int32_t nitems, int32_t bs,
                                                            float *__restrict__ unit) {
  constexpr int LPR = D / 8;        // lanes per row
  constexpr int RPI = 64 / LPR;     // rows side by side
  const int lane = threadIdx.x % 64;
  const int64_t item = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (item >= nitems) return;
  const T *src = item < nq ? q + item * bs * D : k + (item - nq) * bs * D;
  const int piece = lane % LPR, r0 = lane / LPR;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // bs is a multiple of 16 and RPI <= 16, so the trip count is a multiple of
  // 16 / RPI; unrolling keeps several row loads in flight per lane.
#pragma unroll 8
  for (int r = r0; r < bs; r += RPI) {
    float x[8];
    load8f<T>(src + (int64_t)r * D + piece * 8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += x[i];
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o, 64);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(acc[i], acc[i], ss);
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  if (lane < LPR) {
    float *dst = unit + item * D + piece * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[i] * inv;
  }
}

constexpr int kTileM = 64, kTileN = 64;

template <int D>
__global__ void __launch_bounds__(256) adaptive_score_kernel(const float *__restrict__ unit,
                                                             int32_t H, int32_t g, int32_t Mb,
                                                             int32_t Nb, float tau, int32_t causal,
                                                             int32_t keep_diagonal,
                                                             int32_t *__restrict__ layout,
                                                             float *__restrict__ scores) {
  constexpr int STR = D + 4;   // rows 16-byte aligned; 4 floats of padding keep reads conflict-free
  __shared__ __attribute__((aligned(16))) float qs[kTileM * STR];
  __shared__ __attribute__((aligned(16))) float ks[kTileN * STR];
  const int h = blockIdx.z;
  const int m0 = blockIdx.y * kTileM, n0 = blockIdx.x * kTileN;
  const int tid = threadIdx.x;
  if (causal && scores == nullptr && n0 > m0 + kTileM - 1) {
    // every pair of the tile lies above the diagonal: no score is needed
    for (int i = tid; i < kTileM * kTileN; i += 256) {
      const int m = m0 + i / kTileN, n = n0 + i % kTileN;
      if (m < Mb && n < Nb) layout[((int64_t)h * Mb + m) * Nb + n] = 0;
    }
    return;
  }
  const float *qu = unit + ((int64_t)h * Mb) * D;
  const float *ku = unit + ((int64_t)H * Mb + (int64_t)(h / g) * Nb) * D;
  for (int i = tid; i < kTileM * D / 4; i += 256) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    *reinterpret_cast<f32x4 *>(&qs[r * STR + 4 * c4]) =
        m0 + r < Mb ? *reinterpret_cast<const f32x4 *>(&qu[(int64_t)(m0 + r) * D + 4 * c4]) : f32x4{};
  }
  for (int i = tid; i < kTileN * D / 4; i += 256) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    *reinterpret_cast<f32x4 *>(&ks[r * STR + 4 * c4]) =
        n0 + r < Nb ? *reinterpret_cast<const f32x4 *>(&ku[(int64_t)(n0 + r) * D + 4 * c4]) : f32x4{};
  }
  __syncthreads();
  // thread: block rows rg + 16i and block columns cg + 16j of the tile
  // (i, j < 4); the 16 lanes of a row group read one q row (broadcast) and
  // 16 k rows 528 bytes apart (distinct banks)
  const int cg = tid % 16, rg = tid / 16;
  float dots[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) dots[i][j] = 0.f;
#pragma unroll 2
  for (int c4 = 0; c4 < D / 4; ++c4) {
    f32x4 qv[4], kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] = *reinterpret_cast<const f32x4 *>(&qs[(rg + 16 * i) * STR + 4 * c4]);
      kv[i] = *reinterpret_cast<const f32x4 *>(&ks[(cg + 16 * i) * STR + 4 * c4]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dots[i][j] = fmaf(qv[i][e], kv[j][e], dots[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + rg + 16 * i, n = n0 + cg + 16 * j;
      if (m >= Mb || n >= Nb) continue;
      const float dot = dots[i][j];
      bool live = dot >= tau;
      if (causal && n > m) live = false;
      if (keep_diagonal && n == m) live = true;
      const int64_t o = ((int64_t)h * Mb + m) * Nb + n;
      layout[o] = live ? 1 : 0;
      if (scores) scores[o] = dot;
    }
}

template <typename T, int D>
hipError_t launch_adaptive_t(const void *q, const void *k, int32_t H, int32_t Hkv, int32_t Mb,
                             int32_t Nb, int32_t bs, float tau, int32_t causal,
                             int32_t keep_diagonal, float *unit, int32_t *layout, float *scores,
                             hipStream_t stream) {
  const int32_t nq = H * Mb, nitems = H * Mb + Hkv * Nb;
  hipLaunchKernelGGL((adaptive_pool_kernel<T, D>), dim3((nitems + 3) / 4), dim3(256), 0, stream,
                     (const T *)q, (const T *)k, nq, nitems, bs, unit);
  const dim3 grid((Nb + kTileN - 1) / kTileN, (Mb + kTileM - 1) / kTileM, H);
  hipLaunchKernelGGL((adaptive_score_kernel<D>), grid, dim3(256), 0, stream, (const float *)unit,
                     H, H / Hkv, Mb, Nb, tau, causal, keep_diagonal, layout, scores);
  return hipGetLastError();
}

}  // namespace

bool adaptive_supported(int32_t bs, int32_t d) {
  return bs >= 16 && bs % 16 == 0 && (d == 32 || d == 64 || d == 128);
}

hipError_t launch_adaptive(const void *q, const void *k, int32_t H, int32_t Hkv, int32_t Mb,
                           int32_t Nb, int32_t bs, int32_t d, bool f32, float tau, int32_t causal,
                           int32_t keep_diagonal, float *unit, int32_t *layout, float *scores,
                           hipStream_t stream) {
#define BSA_AD_CASE(D_)                                                                        \
  if (d == D_)                                                                                 \
    return f32 ? launch_adaptive_t<float, D_>(q, k, H, Hkv, Mb, Nb, bs, tau, causal,            \
                                              keep_diagonal, unit, layout, scores, stream)      \
               : launch_adaptive_t<__bf16, D_>(q, k, H, Hkv, Mb, Nb, bs, tau, causal,           \
                                               keep_diagonal, unit, layout, scores, stream);
  BSA_AD_CASE(32) BSA_AD_CASE(64) BSA_AD_CASE(128)
#undef BSA_AD_CASE
  return hipErrorInvalidValue;
}

}  // namespace bsa
