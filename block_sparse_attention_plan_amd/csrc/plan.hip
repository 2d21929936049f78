// Layout -> per-row CSR planner (gfx950).
//
// The layout is an int32 [H, Mb, Nb] tensor whose non-zero entries mark live
// tiles (DeepSpeed sparse-attention utils page, "I/O Contract").  The plan keeps
// only the live tiles with their column indices, the CSR form of the next.gr
// "Block Sparse Attention Techniques" tutorial (section 3.2), and adds a
// load-balance order of the rows.  Rows are r = h * Mb + m.
//
// Four kernels, all stream-ordered:
//   count  one wave per row: live count by ballot + popcount -> row_ptr[r+1]
//   scan   one workgroup: in-place inclusive scan of row_ptr[1..R] built from
//          wavefront prefix scans; writes nnz_total
//   fill   one wave per row: ballot + mbcnt compaction of the live columns
//   order  one workgroup per head: stable counting sort of the head's rows by
//          live count, descending; ties keep m ascending
//
// The backward's column plan is the same construction on the transposed
// layout (columns c = h * Nb + n, the live query blocks m of each column in
// ascending order), built by a column count and a column fill kernel (one
// lane per column, walking m; neighbouring lanes read neighbouring words),
// the same scan, and the same counting sort over the key-block work items
// (K/V head, n), whose key is the live count summed over the query heads of
// the K/V head's group.
// Every step is integer work with no atomics whose order matters, so the plan
// is bit-for-bit deterministic.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele
// over lane shifts).
__device__ __forceinline__ int wave_incl_scan(int x) {
  int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (l >= d) x += y;
  }
  return x;
}

__global__ void __launch_bounds__(256) plan_count_kernel(const int32_t *__restrict__ layout,
                                                         int32_t R, int32_t Nb,
                                                         int32_t *__restrict__ row_ptr) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  if (r == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (r >= R) return;
  const int32_t *row = layout + r * (int64_t)Nb;
  int cnt = 0;
  for (int n0 = 0; n0 < Nb; n0 += kWave) {
    const int n = n0 + lane;
    const bool live = n < Nb && row[n] != 0;
    cnt += __popcll(__ballot(live));
  }
  if (lane == 0) row_ptr[r + 1] = cnt;
}

// In-place inclusive scan of row_ptr[1..R] by one workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) plan_scan_kernel(int32_t R, int32_t *__restrict__ row_ptr,
                                                         int32_t *__restrict__ nnz_total) {
  __shared__ int wave_tot[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = lane_id();
  if (tid == 0) carry_s = 0;
  __syncthreads();
  int32_t *a = row_ptr + 1;
  for (int64_t base = 0; base < R; base += 1024) {
    const int64_t i = base + tid;
    const int x = i < R ? a[i] : 0;
    const int incl = wave_incl_scan(x);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += wave_tot[w];
    const int carry = carry_s;
    if (i < R) a[i] = carry + wave_off + incl;
    __syncthreads();
    if (tid == 1023) carry_s = carry + wave_off + incl;
    __syncthreads();
  }
  if (tid == 0) *nnz_total = carry_s;
}

__global__ void __launch_bounds__(256) plan_fill_kernel(const int32_t *__restrict__ layout,
                                                        int32_t R, int32_t Nb,
                                                        const int32_t *__restrict__ row_ptr,
                                                        int32_t *__restrict__ col_idx) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  if (r >= R) return;
  const int32_t *row = layout + r * (int64_t)Nb;
  int pos = row_ptr[r];
  const uint64_t lt = lanemask_lt();
  for (int n0 = 0; n0 < Nb; n0 += kWave) {
    const int n = n0 + lane;
    const bool live = n < Nb && row[n] != 0;
    const uint64_t bal = __ballot(live);
    if (live) col_idx[pos + __popcll(bal & lt)] = n;
    pos += __popcll(bal);
  }
}

// Stable counting sort of one segment's items by key, descending.  Segment
// s holds items i = 0 .. items-1; the key of item i is the sum over j < g of
// the extent ptr[(s g + j) items + i + 1] - ptr[(s g + j) items + i] (the live
// count of a row for g = 1, of a key block summed over a head group for the
// column plan).  Writes order[s items + rank] = s items + i.
// Dynamic LDS: start[max_key+1] (bucket start, then running position) as int.
__global__ void __launch_bounds__(256) plan_order_kernel(int32_t items, int32_t max_key, int32_t g,
                                                         const int32_t *__restrict__ ptr,
                                                         int32_t *__restrict__ order) {
  extern __shared__ int start[];
  const int seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int nkeys = max_key + 1;
  const int32_t *sp = ptr + (int64_t)seg * g * items;
  auto key_of = [&](int i) {
    int key = 0;
    for (int j = 0; j < g; ++j) key += sp[(int64_t)j * items + i + 1] - sp[(int64_t)j * items + i];
    return key;
  };
  for (int k = tid; k < nkeys; k += blockDim.x) start[k] = 0;
  __syncthreads();
  // histogram of keys (integer increments: order does not matter)
  for (int i = tid; i < items; i += blockDim.x) atomicAdd(&start[key_of(i)], 1);
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    // start[k] = number of rows whose count exceeds k: a reverse exclusive
    // scan, walked from the largest key down in chunks of 64.
    int carry = 0;
    for (int top = nkeys - 1; top >= 0; top -= kWave) {
      const int k = top - lane;
      const int x = k >= 0 ? start[k] : 0;
      const int incl = wave_incl_scan(x);
      if (k >= 0) start[k] = carry + incl - x;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    // place items in index order, 64 at a time; equal keys inside a chunk
    // are ranked by lane order, which keeps the sort stable.
    int nbits = 1;
    while ((1 << nbits) <= max_key) ++nbits;
    const uint64_t lt = lanemask_lt();
    for (int i0 = 0; i0 < items; i0 += kWave) {
      const int i = i0 + lane;
      const bool act = i < items;
      const int key = act ? key_of(i) : 0;
      uint64_t same = __ballot(act);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        same &= bit ? bb : ~bb;
      }
      const int rank = __popcll(same & lt);
      const int base = act ? start[key] : 0;
      if (act) order[(int64_t)seg * items + base + rank] = seg * items + i;
      // the lowest lane of each key group advances that key's position
      const bool leader = act && (same & lt) == 0;
      __builtin_amdgcn_wave_barrier();
      if (leader) start[key] = base + __popcll(same);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Live count of each column c = h * Nb + n (one lane per column).
__global__ void __launch_bounds__(256) plan_col_count_kernel(const int32_t *__restrict__ layout,
                                                             int32_t H, int32_t Mb, int32_t Nb,
                                                             int32_t *__restrict__ col_ptr) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c == 0) col_ptr[0] = 0;
  if (c >= (int64_t)H * Nb) return;
  const int64_t h = c / Nb, n = c % Nb;
  const int32_t *col = layout + h * Mb * Nb + n;
  int cnt = 0;
#pragma unroll 8
  for (int m = 0; m < Mb; ++m) cnt += col[(int64_t)m * Nb] != 0;
  col_ptr[c + 1] = cnt;
}

// Query blocks of each column in ascending order.
__global__ void __launch_bounds__(256) plan_col_fill_kernel(const int32_t *__restrict__ layout,
                                                            int32_t H, int32_t Mb, int32_t Nb,
                                                            const int32_t *__restrict__ col_ptr,
                                                            int32_t *__restrict__ row_idx) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= (int64_t)H * Nb) return;
  const int64_t h = c / Nb, n = c % Nb;
  const int32_t *col = layout + h * Mb * Nb + n;
  int pos = col_ptr[c];
  for (int m = 0; m < Mb; ++m)
    if (col[(int64_t)m * Nb] != 0) row_idx[pos++] = m;
}

hipError_t launch_order(int32_t segs, int32_t items, int32_t max_key, int32_t g,
                        const int32_t *ptr, int32_t *order, hipStream_t stream) {
  const size_t lds = (size_t)(max_key + 1) * sizeof(int);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void *)plan_order_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_order_kernel, dim3(segs), dim3(256), lds, stream, items, max_key, g,
                     ptr, order);
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool plan_geometry(int32_t H, int32_t Mb, int32_t Nb, PlanGeometry *g) {
  if (H <= 0 || Mb <= 0 || Nb <= 0) return false;
  const int64_t tiles = (int64_t)H * Mb * Nb;
  if (tiles >= (int64_t(1) << 31)) return false;
  const size_t R = (size_t)H * Mb;
  g->off_row_ptr = 0;
  g->off_row_order = align256(g->off_row_ptr + (R + 1) * 4);
  g->off_nnz = align256(g->off_row_order + R * 4);
  g->off_col_idx = align256(g->off_nnz + 4);
  g->total = align256(g->off_col_idx + (size_t)tiles * 4);
  return true;
}

hipError_t launch_plan(const int32_t *layout, int32_t H, int32_t Mb, int32_t Nb,
                       int32_t *row_ptr, int32_t *row_order, int32_t *nnz_total,
                       int32_t *col_idx, hipStream_t stream) {
  const int32_t R = H * Mb;
  const int rows_per_block = 256 / kWave;
  const int nblk = (R + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(plan_count_kernel, dim3(nblk), dim3(256), 0, stream, layout, R, Nb, row_ptr);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, R, row_ptr, nnz_total);
  hipLaunchKernelGGL(plan_fill_kernel, dim3(nblk), dim3(256), 0, stream, layout, R, Nb,
                     (const int32_t *)row_ptr, col_idx);
  return launch_order(H, Mb, Nb, 1, row_ptr, row_order, stream);
}

bool plan_cols_geometry(int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb, PlanColsGeometry *g) {
  if (H <= 0 || Hkv <= 0 || Mb <= 0 || Nb <= 0 || H % Hkv != 0) return false;
  const int64_t tiles = (int64_t)H * Mb * Nb;
  if (tiles >= (int64_t(1) << 31)) return false;
  const size_t C = (size_t)H * Nb;
  g->off_col_ptr = 0;
  g->off_col_order = align256(g->off_col_ptr + (C + 1) * 4);
  g->off_nnz = align256(g->off_col_order + (size_t)Hkv * Nb * 4);
  g->off_row_idx = align256(g->off_nnz + 4);
  g->total = align256(g->off_row_idx + (size_t)tiles * 4);
  return true;
}

hipError_t launch_plan_cols(const int32_t *layout, int32_t H, int32_t Hkv, int32_t Mb, int32_t Nb,
                            int32_t *col_ptr, int32_t *col_order, int32_t *nnz_total,
                            int32_t *row_idx, hipStream_t stream) {
  const int32_t C = H * Nb;
  const int nblk = (C + 255) / 256;
  hipLaunchKernelGGL(plan_col_count_kernel, dim3(nblk), dim3(256), 0, stream, layout, H, Mb, Nb,
                     col_ptr);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, C, col_ptr, nnz_total);
  hipLaunchKernelGGL(plan_col_fill_kernel, dim3(nblk), dim3(256), 0, stream, layout, H, Mb, Nb,
                     (const int32_t *)col_ptr, row_idx);
  const int32_t g = H / Hkv;
  return launch_order(Hkv, Nb, g * Mb, g, col_ptr, col_order, stream);
}

}  // namespace bsa
