// Internal launch interface between the C ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

// Prefill forward arguments. Strides in elements; masks already normalised
// (causal folded into window_right = 0; negative = unbounded).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t q_bs, q_rs, q_hs;
  int64_t k_bs, k_rs, k_hs;
  int64_t v_bs, v_rs, v_hs;
  int64_t o_bs, o_rs, o_hs;
  const int32_t* cu_q;  // NULL for dense batches
  const int32_t* cu_k;
  int32_t batch, seqlen_q, seqlen_k;
  int32_t hq, hkv, group;  // group = hq / hkv
  int32_t total_q;
  int32_t max_rows;        // max_seqlen_q * group (packed rows of the longest sequence)
  int32_t num_m_blocks;    // set by each launcher: ceil(max_rows / its BLOCK_M)
  float scale;             // softmax_scale
  float scale_log2;        // softmax_scale * log2(e)
  int32_t wl, wr;
};

// Paged split-KV decode arguments.
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* page_table;
  const int32_t* seqused_k;  // may be NULL
  float* o_part;             // [batch*hq][splits][d]
  float* lse_part;           // [batch*hq][splits]
  int64_t q_bs, q_hs;
  int32_t batch, hq, hkv, group;
  int32_t page_size, num_pages, max_pages;
  int32_t num_splits;
  int32_t row_blocks;        // ceil(group / 32)
  float scale;
  float scale_log2;
  int32_t wl;                // < 0 unbounded
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  void* out;
  int64_t out_row_stride;
  float* lse;
  int32_t rows, num_splits;
};

constexpr int kFwdBlockM = 128;   // packed query rows per workgroup (4 waves x 32), D = 256
constexpr int kFwdPPBlockM = 256; // ping-pong kernel, D = 64/128 (8 waves x 32)
constexpr int kFwdBlockN = 64;    // keys per K/V tile
constexpr int kDecBlockN = 128;   // keys per decode tile (4 waves x 32)

// The per-wave streaming decode kernel serves head_dim <= 128 when every
// aligned 32-key slice lies in one page; the tile kernel serves the rest.
constexpr bool decode_streams(int head_dim, int page_size) {
  return head_dim <= 128 && page_size % 32 == 0;
}

template <int D> hipError_t launch_fwd(const FwdArgs& a, hipStream_t s);
template <int D> hipError_t launch_fwd_pp(const FwdArgs& a, hipStream_t s);
template <int D> hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
template <int D> hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t s);
template <int D> hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace mi_attn
