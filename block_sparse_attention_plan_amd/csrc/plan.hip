// Layout -> per-row CSR planner (gfx950).
//
// The layout is an int32 [H, Mb, Nb] tensor whose non-zero entries mark live
// tiles (DeepSpeed sparse-attention utils page, "I/O Contract").  The plan keeps
// only the live tiles with their column indices, the CSR form of the next.gr
// "Block Sparse Attention Techniques" tutorial (section 3.2), and adds a
// load-balance order of the rows.  Rows are r = h * Mb + m.
//
// Beside the rows, the plan holds the pairs of neighbouring block rows
// (2p, 2p+1) of each head: for pair q = h * Mp + p the union of the two rows'
// live columns, ascending, each entry tagged with which of the two rows lists
// it (n | mask << 24).  Layouts built from local windows, global columns and
// strides repeat most columns from one block row to the next, so a forward
// work item that covers a pair loads each shared tile once.  A flag records
// whether the unions hold at most three quarters of the live tiles, which is
// when the forward uses the pairs.
//
// Four steps in three launches, all stream-ordered (fill and order share the
// last launch, as both need only the scanned counts):
//   count  one wave per pair of rows: live counts of both rows and of their
//          union by ballot + popcount -> row_ptr[r+1], pair_ptr[q+1]
//   scan   one workgroup per array: in-place inclusive scans of row_ptr[1..R]
//          and pair_ptr[1..Q], 8192 entries per round (8 per thread in
//          registers, then wavefront prefix scans); writes nnz_total and
//          pair_total
//   fill   one wave per pair of rows: ballot + mbcnt compaction of each row's
//          live columns and of the union with its row tags
//   order  one workgroup per head and array: stable counting sort of the
//          head's rows (pairs) by live (union) count, descending; ties keep m
//          (p) ascending; then the pair flag
//
// The backward's column plan is the same construction on the transposed
// layout (columns c = h * Nb + n, the live query blocks m of each column in
// ascending order), built by a column count and a column fill kernel (one
// lane per column, neighbouring lanes reading neighbouring words, and eight
// waves per 64 columns, each walking one stretch of m),
// the same scan, and the same counting sort over the key-block work items
// (K/V head, n), whose key is the live count summed over the query heads of
// the K/V head's group.
// Every step is integer work with no atomics whose order matters, so the plan
// is bit-for-bit deterministic.
#include <algorithm>

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

// One wave per pair q = h * Mp + p: rows r0 = h * Mb + 2p and r0 + 1 (the
// second absent when 2p + 1 == Mb).
__global__ void __launch_bounds__(256) plan_count_kernel(const int32_t *__restrict__ layout,
                                                         int32_t H, int32_t Mb, int32_t Nb,
                                                         int32_t *__restrict__ row_ptr,
                                                         int32_t *__restrict__ pair_ptr) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int Mp = (Mb + 1) / 2;
  const int64_t q = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave;
  if (q == 0 && threadIdx.x == 0) {
    row_ptr[0] = 0;
    pair_ptr[0] = 0;
  }
  if (q >= (int64_t)H * Mp) return;
  const int64_t h = q / Mp, p = q % Mp;
  const int64_t r0 = h * Mb + 2 * p;
  const bool two = 2 * p + 1 < Mb;
  const int32_t *row0 = layout + r0 * (int64_t)Nb;
  const int32_t *row1 = row0 + Nb;
  int c0 = 0, c1 = 0, cu = 0;
  for (int n0 = 0; n0 < Nb; n0 += kWave) {
    const int n = n0 + lane;
    const bool a = n < Nb && row0[n] != 0;
    const bool b = two && n < Nb && row1[n] != 0;
    c0 += __popcll(__ballot(a));
    c1 += __popcll(__ballot(b));
    cu += __popcll(__ballot(a || b));
  }
  if (lane == 0) {
    row_ptr[r0 + 1] = c0;
    if (two) row_ptr[r0 + 2] = c1;
    pair_ptr[q + 1] = cu;
  }
}

// In-place inclusive scan of ptr[1..n]; the total goes to *total.
struct ScanJob {
  int32_t n;
  int32_t *ptr;
  int32_t *total;
};

// One workgroup of 1024 threads per job (blockIdx.x selects the job).  Each
// round covers 8192 entries: a thread loads 8 consecutive ones (all loads in
// flight at once) and scans them in registers; the threads' totals are
// scanned across the wavefront and the 16 wavefronts through LDS.
__global__ void __launch_bounds__(1024) plan_scan_kernel(ScanJob j0, ScanJob j1) {
  constexpr int PER = 8;
  __shared__ int wave_tot[16];
  const ScanJob job = blockIdx.x == 0 ? j0 : j1;
  const int64_t R = job.n;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = lane_id();
  int32_t *a = job.ptr + 1;
  int carry = 0;
  for (int64_t base = 0; base < R; base += 1024 * PER) {
    const int64_t i0 = base + (int64_t)tid * PER;
    int x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) x[k] = i0 + k < R ? a[i0 + k] : 0;
#pragma unroll
    for (int k = 1; k < PER; ++k) x[k] += x[k - 1];
    const int incl = wave_incl_scan(x[PER - 1]);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int wave_off = 0, round = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int t = wave_tot[w];
      wave_off += w < wave ? t : 0;
      round += t;
    }
    const int off = carry + wave_off + incl - x[PER - 1];
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (i0 + k < R) a[i0 + k] = off + x[k];
    carry += round;
    __syncthreads();  // wave_tot is rewritten by the next round
  }
  if (tid == 0) *job.total = carry;
}

// One wave per pair, as the count kernel: each row's live columns, and the
// union with bit 24 (row 2p) and bit 25 (row 2p + 1) set per column.
// (A body run by the first blocks of the fill-and-order launch.)
__device__ __forceinline__ void plan_fill_body(int block, const int32_t *__restrict__ layout,
                                               int32_t H, int32_t Mb, int32_t Nb,
                                               const int32_t *__restrict__ row_ptr,
                                               int32_t *__restrict__ col_idx,
                                               const int32_t *__restrict__ pair_ptr,
                                               int32_t *__restrict__ pair_cols) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int Mp = (Mb + 1) / 2;
  const int64_t q = (int64_t)block * (blockDim.x / kWave) + wave;
  if (q >= (int64_t)H * Mp) return;
  const int64_t h = q / Mp, p = q % Mp;
  const int64_t r0 = h * Mb + 2 * p;
  const bool two = 2 * p + 1 < Mb;
  const int32_t *row0 = layout + r0 * (int64_t)Nb;
  const int32_t *row1 = row0 + Nb;
  int pos0 = row_ptr[r0];
  int pos1 = two ? row_ptr[r0 + 1] : 0;
  int posu = pair_ptr[q];
  const uint64_t lt = lanemask_lt();
  for (int n0 = 0; n0 < Nb; n0 += kWave) {
    const int n = n0 + lane;
    const bool a = n < Nb && row0[n] != 0;
    const bool b = two && n < Nb && row1[n] != 0;
    const uint64_t ba = __ballot(a), bb = __ballot(b), bu = __ballot(a || b);
    if (a) col_idx[pos0 + __popcll(ba & lt)] = n;
    if (b) col_idx[pos1 + __popcll(bb & lt)] = n;
    if (a || b) pair_cols[posu + __popcll(bu & lt)] = n | ((a ? 1 : 0) << 24) | ((b ? 1 : 0) << 25);
    pos0 += __popcll(ba);
    pos1 += __popcll(bb);
    posu += __popcll(bu);
  }
}

// Stable counting sort of one segment's items by key, descending.  Segment
// s holds items i = 0 .. items-1; the key of item i is the sum over j < g of
// the extent ptr[(s g + j) items + i + 1] - ptr[(s g + j) items + i] (the live
// count of a row for g = 1, of a key block summed over a head group for the
// column plan).  Writes order[s items + rank] = s items + i.
struct OrderJob {
  int32_t segs, items, max_key, g;
  const int32_t *ptr;
  int32_t *order;
};

// The use-pairs flag: 1 when 4 * pair_total <= 3 * nnz_total.
struct PairFlag {
  const int32_t *nnz_total, *pair_total;
  int32_t *flag;  // nullptr: no flag to write
};

// One workgroup per segment of job 0, then per segment of job 1 (block =
// the workgroup's index among them).  start[max_key+1] in LDS (bucket
// start, then running position).
__device__ __forceinline__ void plan_order_body(int block, int *start, OrderJob j0, OrderJob j1,
                                                PairFlag pf) {
  const bool first = block < j0.segs;
  const OrderJob job = first ? j0 : j1;
  const int seg = first ? block : block - j0.segs;
  const int items = job.items, max_key = job.max_key, g = job.g;
  const int tid = threadIdx.x;
  if (block == 0 && tid == 0 && pf.flag != nullptr)
    *pf.flag = 4 * (int64_t)*pf.pair_total <= 3 * (int64_t)*pf.nnz_total ? 1 : 0;
  const int nkeys = max_key + 1;
  const int32_t *sp = job.ptr + (int64_t)seg * g * items;
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
      if (act) job.order[(int64_t)seg * items + base + rank] = seg * items + i;
      // the lowest lane of each key group advances that key's position
      const bool leader = act && (same & lt) == 0;
      __builtin_amdgcn_wave_barrier();
      if (leader) start[key] = base + __popcll(same);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Dynamic LDS: the order body's start[].
__global__ void __launch_bounds__(256) plan_order_kernel(OrderJob j0, OrderJob j1, PairFlag pf) {
  extern __shared__ int start[];
  plan_order_body(blockIdx.x, start, j0, j1, pf);
}

// The row plan's fill and order in one launch (both need only the scanned
// counts): blocks 0 .. nfill-1 fill, the rest order.
__global__ void __launch_bounds__(256) plan_fill_order_kernel(
    int32_t nfill, const int32_t *__restrict__ layout, int32_t H, int32_t Mb, int32_t Nb,
    const int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx,
    const int32_t *__restrict__ pair_ptr, int32_t *__restrict__ pair_cols, OrderJob j0,
    OrderJob j1, PairFlag pf) {
  extern __shared__ int start[];
  if ((int)blockIdx.x < nfill)
    plan_fill_body(blockIdx.x, layout, H, Mb, Nb, row_ptr, col_idx, pair_ptr, pair_cols);
  else
    plan_order_body((int)blockIdx.x - nfill, start, j0, j1, pf);
}

// Column kernels: one workgroup per 64 columns c = h * Nb + n (lane = column,
// so neighbouring lanes read neighbouring layout words) and kColWaves
// waves, wave s walking the contiguous stretch of query blocks
// [s * seg, (s + 1) * seg), seg = ceil(Mb / kColWaves).  The waves' counts
// meet in LDS.
constexpr int kColWaves = 8;

__device__ __forceinline__ int col_count_stretch(const int32_t *col, int64_t stride, int m0,
                                                 int m1) {
  int cnt = 0;
#pragma unroll 8
  for (int m = m0; m < m1; ++m) cnt += col[(int64_t)m * stride] != 0;
  return cnt;
}

// Live count of each column.
__global__ void __launch_bounds__(64 * kColWaves) plan_col_count_kernel(
    const int32_t *__restrict__ layout, int32_t H, int32_t Mb, int32_t Nb,
    int32_t *__restrict__ col_ptr) {
  __shared__ int part[kColWaves][64];
  const int lane = threadIdx.x % 64, s = threadIdx.x / 64;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  if (blockIdx.x == 0 && threadIdx.x == 0) col_ptr[0] = 0;
  const bool ok = c < (int64_t)H * Nb;
  const int seg = (Mb + kColWaves - 1) / kColWaves;
  const int m0 = min(Mb, s * seg), m1 = min(Mb, (s + 1) * seg);
  const int64_t h = c / Nb, n = c % Nb;
  part[s][lane] = ok ? col_count_stretch(layout + h * Mb * Nb + n, Nb, m0, m1) : 0;
  __syncthreads();
  if (s == 0 && ok) {
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kColWaves; ++w) cnt += part[w][lane];
    col_ptr[c + 1] = cnt;
  }
}

// Query blocks of each column in ascending order: each wave counts its
// stretch, the counts of the stretches before it give its first slot.
__global__ void __launch_bounds__(64 * kColWaves) plan_col_fill_kernel(
    const int32_t *__restrict__ layout, int32_t H, int32_t Mb, int32_t Nb,
    const int32_t *__restrict__ col_ptr, int32_t *__restrict__ row_idx) {
  __shared__ int part[kColWaves][64];
  const int lane = threadIdx.x % 64, s = threadIdx.x / 64;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const bool ok = c < (int64_t)H * Nb;
  const int seg = (Mb + kColWaves - 1) / kColWaves;
  const int m0 = min(Mb, s * seg), m1 = min(Mb, (s + 1) * seg);
  const int64_t h = c / Nb, n = c % Nb;
  const int32_t *col = layout + h * Mb * Nb + n;
  part[s][lane] = ok ? col_count_stretch(col, Nb, m0, m1) : 0;
  __syncthreads();
  if (!ok) return;
  int pos = col_ptr[c];
  for (int w = 0; w < s; ++w) pos += part[w][lane];
  for (int m = m0; m < m1; ++m)
    if (col[(int64_t)m * Nb] != 0) row_idx[pos++] = m;
}

size_t order_lds(const OrderJob &j0, const OrderJob &j1) {
  return (size_t)(std::max(j0.max_key, j1.max_key) + 1) * sizeof(int);
}

hipError_t allow_lds(const void *kernel, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_order(const OrderJob &j0, const OrderJob &j1, const PairFlag &pf,
                        hipStream_t stream) {
  const size_t lds = order_lds(j0, j1);
  hipError_t e = allow_lds((const void *)plan_order_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_order_kernel, dim3(j0.segs + j1.segs), dim3(256), lds, stream, j0, j1,
                     pf);
  return hipGetLastError();
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool plan_geometry(int32_t H, int32_t Mb, int32_t Nb, PlanGeometry *g) {
  if (H <= 0 || Mb <= 0 || Nb <= 0) return false;
  const int64_t tiles = (int64_t)H * Mb * Nb;
  if (tiles >= (int64_t(1) << 31)) return false;
  const size_t R = (size_t)H * Mb;
  const size_t Q = (size_t)H * ((Mb + 1) / 2);
  g->off_row_ptr = 0;
  g->off_row_order = align256(g->off_row_ptr + (R + 1) * 4);
  g->off_nnz = align256(g->off_row_order + R * 4);
  g->off_col_idx = align256(g->off_nnz + 4);
  g->off_pair_ptr = align256(g->off_col_idx + (size_t)tiles * 4);
  g->off_pair_order = align256(g->off_pair_ptr + (Q + 1) * 4);
  g->off_pair_info = align256(g->off_pair_order + Q * 4);
  g->off_pair_cols = align256(g->off_pair_info + 8);
  g->total = align256(g->off_pair_cols + Q * (size_t)Nb * 4);
  return true;
}

hipError_t launch_plan(const int32_t *layout, int32_t H, int32_t Mb, int32_t Nb,
                       int32_t *row_ptr, int32_t *row_order, int32_t *nnz_total,
                       int32_t *col_idx, int32_t *pair_ptr, int32_t *pair_order,
                       int32_t *pair_info, int32_t *pair_cols, hipStream_t stream) {
  const int32_t R = H * Mb;
  const int32_t Mp = (Mb + 1) / 2;
  const int32_t Q = H * Mp;
  const int pairs_per_block = 256 / kWave;
  const int nblk = (Q + pairs_per_block - 1) / pairs_per_block;
  hipLaunchKernelGGL(plan_count_kernel, dim3(nblk), dim3(256), 0, stream, layout, H, Mb, Nb,
                     row_ptr, pair_ptr);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(2), dim3(1024), 0, stream,
                     ScanJob{R, row_ptr, nnz_total}, ScanJob{Q, pair_ptr, pair_info});
  const OrderJob j0{H, Mb, Nb, 1, row_ptr, row_order}, j1{H, Mp, Nb, 1, pair_ptr, pair_order};
  const size_t lds = order_lds(j0, j1);
  hipError_t e = allow_lds((const void *)plan_fill_order_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_fill_order_kernel, dim3(nblk + j0.segs + j1.segs), dim3(256), lds, stream,
                     nblk, layout, H, Mb, Nb, (const int32_t *)row_ptr, col_idx,
                     (const int32_t *)pair_ptr, pair_cols, j0, j1,
                     PairFlag{nnz_total, pair_info, pair_info + 1});
  return hipGetLastError();
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
  const int nblk = (C + 63) / 64;
  hipLaunchKernelGGL(plan_col_count_kernel, dim3(nblk), dim3(64 * kColWaves), 0, stream, layout,
                     H, Mb, Nb, col_ptr);
  const ScanJob scan{C, col_ptr, nnz_total};
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, scan, scan);
  hipLaunchKernelGGL(plan_col_fill_kernel, dim3(nblk), dim3(64 * kColWaves), 0, stream, layout,
                     H, Mb, Nb, (const int32_t *)col_ptr, row_idx);
  const int32_t g = H / Hkv;
  const OrderJob order{Hkv, Nb, g * Mb, g, col_ptr, col_order};
  return launch_order(order, OrderJob{0, 0, 0, 1, nullptr, nullptr}, PairFlag{nullptr, nullptr, nullptr},
                      stream);
}

}  // namespace bsa
