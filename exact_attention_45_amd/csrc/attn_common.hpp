// Device helpers shared by the attention kernels (gfx950, wave64).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16):
//   D[32x32] += A[32x16] * B[16x32], fp32 accumulate.
//   lane l, half h = l / 32, c = l % 32:
//     A operand: row c, k = 8h .. 8h+7      (8 bf16 in 4 VGPRs)
//     B operand: col c, k = 8h .. 8h+7
//     D/C: 16 floats; element v holds row 8*(v/4) + 4h + (v%4), col c.
//
// Both attention GEMMs are issued transposed so that one lane owns one query
// column of every accumulator:
//   S^T[key][query]  = K[key][d]   * Q^T[d][query]
//   O^T[d][query]   += V^T[d][key] * P^T[key][query]
// The softmax statistics of a query then live in a single lane (plus its
// partner lane l ^ 32, which holds the other half of the keys), so the row
// max needs one cross-half exchange and the row sum none until the epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (l ^ 32). ds_bpermute based; well defined for every lane.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ bf16x4 cvt4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  r[2] = (__bf16)c;
  r[3] = (__bf16)d;
  return r;
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = lo[i];
    r[i + 4] = hi[i];
  }
  return r;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)0.0f;
  return r;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = 0.0f;
  return r;
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lanes 4e..4e+3 each point at four consecutive 16-bit elements of "row" e
// (e = 0..3); lane i of the group receives element i of rows 0..3. With V
// row-major (key, dim) in LDS and lane j pointing at key j/4, dims 4*(j%4),
// lane i gets dim i of four consecutive keys: an MFMA operand fragment whose
// contraction index is the key. (Semantics measured on gfx950.)
__device__ __forceinline__ bf16x4 ds_read_tr16(const __bf16* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt = 0), not for outstanding global loads: register prefetches for
// later tiles stay in flight across it. (__syncthreads also waits vmcnt = 0.)
// s_waitcnt encoding (gfx9): vmcnt[3:0]|expcnt[6:4]|lgkmcnt[11:8]|vmcnt_hi[15:14];
// 0xC07F = vmcnt 63, expcnt 7, lgkmcnt 0.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

// 16-byte global load / store of raw bits.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace mi_attn
