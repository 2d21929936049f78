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
// Inside a workgroup of bs/16 waves, wave w owns query rows 16w .. 16w+15 of
// the block.  For each live tile the K and V tiles are staged row-major in LDS
// (prefetched into registers one tile ahead), then every wave computes
//   S^T = K Q^T        (16x16x32 MFMA; Q^T stays in registers)
//   online softmax     (lane owns one query column; exp2 with the scale and
//                       log2(e) folded into one multiply-add)
//   O^T += V^T P^T     (16x16x32 MFMA; P^T straight from the S^T registers,
//                       V^T read from the row-major V tile by LDS transpose
//                       reads)
// so no score matrix ever leaves registers.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxFloor = -1e30f;

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

template <int BS, int D, typename T>
__global__ void __launch_bounds__(BS * 4)
bsa_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
               const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
               const int32_t *__restrict__ row_order, int32_t B, int32_t H, int32_t Mb,
               int32_t Nb, float scale_log2, T *__restrict__ out, float *__restrict__ lse) {
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
  const int64_t Sq = (int64_t)Mb * BS, Sk = (int64_t)Nb * BS;
  const T *qh = q + bh * Sq * D;
  const T *kh = k + bh * Sk * D;
  const T *vh = v + bh * Sk * D;
  T *oh = out + bh * Sq * D;
  float *lh = lse ? lse + bh * Sq : nullptr;
  const int64_t i_row = (int64_t)m * BS + 16 * wid + li;  // this lane's query row

  if (beg == end) {  // no live tile: zero output, lse = -inf
    for (int dt = 0; dt < DT; ++dt) Io<T>::store_zero4(oh + i_row * D + 16 * dt + 4 * G);
    if (lh && G == 0) lh[i_row] = -__builtin_inff();
    return;
  }

  // Q^T fragments (B operand of S^T = K Q^T): column = query row, k = d.
  bf16x8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) qf[c] = Io<T>::load8(qh + i_row * D + 32 * c + 8 * G);

  // Register prefetch of one K/V tile.
  bf16x8 kr[CPT], vr[CPT];
  auto load_tile = [&](int n) {
    const T *kt = kh + (int64_t)n * BS * D;
    const T *vt = vh + (int64_t)n * BS * D;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int qid = c * NT + tid;
      const int row = qid / (D / 8), col = (qid % (D / 8)) * 8;
      kr[c] = Io<T>::load8(kt + row * D + col);
      vr[c] = Io<T>::load8(vt + row * D + col);
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

  const float l_tot = sum_xor32(sum_xor16(l_run));
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) Io<T>::store4(oh + i_row * D + 16 * dt + 4 * G, acc[dt] * inv);
  if (lh && G == 0) lh[i_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}

template <int BS, int D, typename T>
hipError_t launch_one(const void *q, const void *k, const void *v, const int32_t *row_ptr,
                      const int32_t *col_idx, const int32_t *row_order, int32_t B, int32_t H,
                      int32_t Mb, int32_t Nb, float scale, void *out, float *lse,
                      hipStream_t stream) {
  const int64_t W = (int64_t)B * H * Mb;
  const int64_t per = (W + 7) / 8;
  const int64_t grid = per * 8;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bsa_fwd_kernel<BS, D, T>), dim3((unsigned)grid), dim3(BS * 4), 0, stream,
                     (const T *)q, (const T *)k, (const T *)v, row_ptr, col_idx, row_order, B, H,
                     Mb, Nb, scale * kLog2e, (T *)out, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(int32_t bs, int32_t d, const void *q, const void *k, const void *v,
                    const int32_t *rp, const int32_t *ci, const int32_t *ro, int32_t B, int32_t H,
                    int32_t Mb, int32_t Nb, float scale, void *out, float *lse, hipStream_t s) {
#define BSA_CASE(BS_, D_)                                                                   \
  if (bs == BS_ && d == D_)                                                                 \
    return launch_one<BS_, D_, T>(q, k, v, rp, ci, ro, B, H, Mb, Nb, scale, out, lse, s);
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

hipError_t launch_forward(const void *q, const void *k, const void *v, const int32_t *row_ptr,
                          const int32_t *col_idx, const int32_t *row_order, int32_t B, int32_t H,
                          int32_t Mb, int32_t Nb, int32_t bs, int32_t d, bool f32, float scale,
                          void *out, float *lse, hipStream_t stream) {
  if (f32)
    return dispatch<float>(bs, d, q, k, v, row_ptr, col_idx, row_order, B, H, Mb, Nb, scale, out,
                           lse, stream);
  return dispatch<__bf16>(bs, d, q, k, v, row_ptr, col_idx, row_order, B, H, Mb, Nb, scale, out,
                          lse, stream);
}

}  // namespace bsa
