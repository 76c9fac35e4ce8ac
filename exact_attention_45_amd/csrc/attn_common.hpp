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
// Reductions over the lane pair (l, l ^ 32) without LDS traffic:
// v_permlane32_swap with both operands x leaves, in every lane l, x of lane
// l % 32 in the first result and x of lane l % 32 + 32 in the second (both
// halves then combine the same two values in the same order).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// IEEE 754-2019 maximum (NaN-propagating). gfx950 has it as v_maximum3_f32,
// which needs no input quieting; fmaxf lowers in IEEE mode with a
// canonicalising v_max_f32 in front of every input that is not the result of
// ordinary arithmetic (MFMA outputs, lane shuffles), doubling the max cost.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// Masking without vector compares (each compare result takes a scalar
// register pair, and unrolled over a tile they exhaust the scalar file).
// vis64 sets bit l for the local key offsets l in [r0, r1] of a 64-key
// window; mask_by_bit keeps x when bit `bit` of `word` is set and otherwise
// returns -inf, as min(x, +inf) or min(x, -inf).
__device__ __forceinline__ uint64_t vis64(int r0, int r1) {
  const int a0 = r0 < 0 ? 0 : r0;
  const int a1 = r1 > 63 ? 63 : r1;
  if (a0 > a1) return 0;
  return (~0ull >> (63 - a1)) & (~0ull << a0);
}
__device__ __forceinline__ float mask_by_bit(float x, uint32_t word, int bit) {
  const uint32_t keep = (word >> bit) & 1u;
  return vmin(x, __uint_as_float(0xFF800000u ^ (keep << 31)));
}

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
//
// Fragment orders used by the P V product (O^T += V^T P^T), 16 keys per MFMA:
//   * V^T fragment (A operand): two transposing reads. 16-lane group g reads
//     4 keys x 16 dims; lane j points at key 4*half + j/4 (+16t for MFMA t,
//     +8 for the second read), dims 16*(g&1) + 4*(j&3) of d-block db, i.e.
//     16-byte chunk 4*db + 2*(g&1) + (j&3)/2 of that key row, which sits at
//     8*(db>>1) + ((4*(db&1) + chunk%4) ^ swz_key(key)) in the swizzled tile:
//     two lane patterns (db even / odd) plus immediates.
//   * P^T fragment (B operand): MFMA t covers keys 16t..16t+15 of the tile;
//     lane half h supplies keys {16t+4h+j, 16t+8+4h+j : j<4}, the key order of
//     the V^T fragment above, taken from S^T accumulator registers
//     8*(t&1) .. 8*(t&1)+7 of key block t>>1. The contraction is over the
//     same 16 keys in the same order on both sides, so the product is exact.
__device__ __forceinline__ bf16x4 ds_read_tr16(const __bf16* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Learnable sink (interface page, `learnable_sink`, one logit per query
// head), read as one more term of the softmax denominator that carries no
// value. Given a row's log-sum-exp over its keys, lse_keys (-inf when it has
// none), returns the row's LSE with the sink, log(exp(lse_keys) +
// exp(sink)), and sets *w = exp(lse_keys - that), the factor that rescales
// the row's normalised output (0 when the row has no key).
__device__ __forceinline__ float merge_sink(float lse_keys, float sink, float* w) {
  if (sink == kNegInf) {  // no sink term
    *w = 1.0f;
    return lse_keys;
  }
  const float hi = vmax(lse_keys, sink);
  const float lse = hi + __logf(__expf(lse_keys - hi) + __expf(sink - hi));
  *w = lse_keys == kNegInf ? 0.0f : __expf(lse_keys - lse);
  return lse;
}

// Logit soft-capping in raw score units. With the scaled score x = scale * s
// capped to cap * tanh(x / cap), the raw score becomes
// k2 * tanh(k1 * s), k1 = scale / cap, k2 = cap / scale, so the exp2-domain
// softmax after it is unchanged. Here k1x = 2 k1 log2(e) and
// tanh(y) = 1 - 2 / (exp(2y) + 1), whose limits are exact: exp2 overflows to
// +inf (rcp gives 0, tanh 1) or underflows to 0 (tanh -1).
__device__ __forceinline__ float softcap_raw(float s, float k1x, float k2) {
  const float e = fast_exp2(s * k1x);
  return k2 * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt = 0), not for outstanding global loads: register prefetches for
// later tiles stay in flight across it. (__syncthreads also waits vmcnt = 0.)
// s_waitcnt encoding (gfx9): vmcnt[3:0]|expcnt[6:4]|lgkmcnt[11:8]|vmcnt_hi[15:14];
// 0xC07F = vmcnt 63, expcnt 7, lgkmcnt 0.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier (the barrier intrinsic itself is declared not to touch
// memory); they emit no instructions.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A wave-uniform int the compiler computed in vector registers (e.g. after a
// division), moved to a scalar register so loop counters and addresses
// derived from it stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// LDS tile layout shared by the kernels: rows of head_dim bf16 (16-byte
// chunks), chunk c of row `key` stored at chunk position c ^ swz_key(key).
// swz_key maps key & 7 onto 0,2,4,6,1,3,5,7: eight consecutive keys reading
// the same chunk hit eight different 16-byte bank groups (16-byte fragment
// reads), while the four keys of a transposing read, 4h..4h+3, keep each
// 32-byte chunk pair together and spread over four pair slots.
__device__ __forceinline__ int swz_key(int key) { return ((key & 3) << 1) | ((key >> 2) & 1); }

// Buffer resource over [base, base + num_bytes): raw buffer loads whose byte
// offset falls outside return zero instead of touching memory. The third
// descriptor dword 0x00020000 selects the 32-bit data format gfx9-family raw
// buffer loads use.
// Arguments must be wave-uniform; readfirstlane states that to the compiler
// (otherwise it wraps each load in a loop over distinct descriptor values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(num_bytes);
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Same, marked non-temporal (data read once, e.g. a decode step's KV cache
// stream).
__device__ __forceinline__ uint4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// LDS byte address (offset within the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global-to-LDS load (gfx950 buffer_load_dwordx4 ... lds): lane i's 16
// bytes at buffer offset voff land at LDS address lds_base + 16 * i, with
// lds_base wave-uniform (it goes through M0). No registers are staged.
// Issued as inline asm: the compiler cannot tell which LDS buffer such a load
// writes when buffers rotate at run time, and for its own builtin it would
// then wait for every outstanding load before each later LDS read. Loads the
// compiler does not count only make its own vmcnt waits stricter; the caller
// waits for these itself (vmcnt_wait, then a barrier for other waves' loads).
// The kernels keep nothing in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(lds_base)
      : "memory", "m0");
}
// Same load without touching M0 (it must still hold the LDS base of an
// earlier dma16): the immediate OFF shifts both the LDS destination and the
// global offset; soff (wave-uniform) adds to the global offset only.
template <int OFF>
__device__ __forceinline__ void dma16_same_m0(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "i"(OFF)
               : "memory");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt at their no-wait maxima).
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

// 16-byte global load / store of raw bits.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8_nt(const void* p) {
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Four OCP fp8 bytes (little-endian in w; e4m3, or e5m2 when E5M2) -> four
// bf16 values, exact: one hardware conversion per byte pair goes straight to
// bf16 with a scale of 1.0, so each result is the format's value itself, and
// every e4m3 and e5m2 value is a bf16 value.
template <bool E5M2>
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __bf16 b16x2;
  b16x2 lo, hi;
  if constexpr (E5M2) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true);
  } else {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  }
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

}  // namespace mi_attn
