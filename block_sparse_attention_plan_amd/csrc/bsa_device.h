// Device-side building blocks shared by the gfx950 kernels of libbsa:
// vector types, MFMA wrappers, bf16 packing, cross-lane reductions and the
// LDS transpose read.  Lane layouts below were measured on gfx950.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define BSA_LDS __attribute__((address_space(3)))

// D = A * B + C with 16x16x32 bf16 operands.
// Operand layout: lane l holds row (A) / column (B) l%16 and the 8 k-values
// 8*(l/16) .. 8*(l/16)+7.  Result: lane l holds column l%16, rows
// 4*(l/16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C with 32x32x16 bf16 operands.
// Operand layout: lane l holds row (A) / column (B) l%32 and k-values
// 8*(l/32) .. +7.  Result: lane l holds column l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even float -> bf16 conversion of 8 floats.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Value of lane l ^ 16 and lane l ^ 32 combined through permlane swaps: with
// x passed as both operands, the two results hold x of lanes {l, l^16}
// (resp. {l, l^32}) in some order, so op(r0, r1) is the pair reduction.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The tanh logit cap applied to a raw score s (before scaling): returns
// s' with scale * s' = cap * tanh(scale * s / cap), given k2 =
// 2 * scale * log2(e) / cap and b = cap / scale; tanh(y) = 1 - 2 / (e^(2y) + 1)
// saturates cleanly at +-1 when e^(2y) over- or underflows.
__device__ __forceinline__ float capped_score(float s, float k2, float b) {
  const float e = __builtin_amdgcn_exp2f(s * k2);
  return b * fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
}

// Folds a sink logit (log2 units) into a row's running max m and sum l and
// returns the factor by which the row's unnormalised output must be scaled.
__device__ __forceinline__ float fold_sink(float &m, float &l, float sink_l2) {
  const float mm = fmaxf(m, sink_l2);
  const float a = __builtin_amdgcn_exp2f(m - mm);
  l = l * a + __builtin_amdgcn_exp2f(sink_l2 - mm);
  m = mm;
  return a;
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 untyped access);
// reads at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Copy 16 bytes per lane from rsrc + voff + soff straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds; lds_base is
// wave-uniform).  Unlike the global_load_lds form, the compiler accounts
// for this copy on the vector-memory counter alone, so LDS reads issued
// while it is in flight can be waited for one by one.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rs, void *lds_base,
                                              uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (BSA_LDS void *)lds_base, 16, voff, soff, 0, 0);
}

// The same with 4 bytes per lane (buffer_load_dword ... lds): one wave
// instruction fills 256 contiguous LDS bytes at lds_base + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(__amdgpu_buffer_rsrc_t rs, void *lds_base,
                                             uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (BSA_LDS void *)lds_base, 4, voff, soff, 0, 0);
}

// LDS transpose read of 4 bf16 values.  Inside each group of 16 lanes, lane
// s supplies the address of a 4-element (8-byte) chunk; lane t receives
// element t%4 of the chunks supplied by lanes 4e + t/4 (e = 0..3) of its
// group.  With lane s = 4e' + c pointing at row (k0 + e') and columns
// (n0 + 4c .. n0 + 4c + 3) of a row-major [k][n] tile, lane t receives
// tile[k0 + e][n0 + t] for e = 0..3: four consecutive k of column t.
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16 *lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BSA_LDS i16x4 *)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// D = A * B + C with 16x16x16 bf16 operands (4 k-values per lane, lane l
// holds k = 4*(l/16) .. +3); result layout as for mfma16.
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// Schedule pattern for one straight-line region: N MFMAs, each followed by
// V VALU instructions and R LDS reads, with P reads issued ahead of the
// first MFMA (reads beyond the total are simply not matched).
template <int I, int N, int R, int V>
__device__ __forceinline__ void sched_steps() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
    if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // LDS read
    sched_steps<I + 1, N, R, V>();
  }
}
template <int N, int TOTAL_READS, int P, int V>
__device__ __forceinline__ void sched_interleave() {
  constexpr int R = (TOTAL_READS + N - 1) / N;
  if constexpr (P > 0) __builtin_amdgcn_sched_group_barrier(0x100, P, 0);
  sched_steps<0, N, R, V>();
}

}  // namespace bsa
