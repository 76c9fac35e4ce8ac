// Internal launch interface of the backward pass (api.hip -> bwd_kernel.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

// Backward arguments. Strides in elements; masks already normalised (causal
// folded into window_right = 0; negative = unbounded). out/dout/dq use the
// query layout, dk/dv the key layout, lse and dpsum the forward LSE layout:
// [batch, hq, seqlen_q] for dense batches, [hq, total_q] with cu_q.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dpsum;     // workspace: row sums of O * dO
  float* lse_log2;  // workspace: LSE * log2(e), +inf where LSE = -inf
  // workspace when splits > 1: float32 dK / dV partials of each split,
  // [splits][batch][seqlen_k][hkv][2][head_dim] (seqlen_k: the maximum)
  float* dkv_part;
  int32_t splits;  // workgroups sharing one key block's walk over the queries
  int64_t q_bs, q_rs, q_hs;
  int64_t k_bs, k_rs, k_hs;
  int64_t v_bs, v_rs, v_hs;
  int64_t o_bs, o_rs, o_hs;
  int64_t do_bs, do_rs, do_hs;
  int64_t dq_bs, dq_rs, dq_hs;
  int64_t dk_bs, dk_rs, dk_hs;
  int64_t dv_bs, dv_rs, dv_hs;
  const int32_t* cu_q;  // NULL for dense batches
  const int32_t* cu_k;
  int32_t batch, seqlen_q, seqlen_k;  // dense: the lengths; varlen: max_seqlen_q / _k
  int32_t hq, hkv, group;
  int32_t total_q;
  float scale;       // softmax_scale
  float scale_log2;  // softmax_scale * log2(e)
  int32_t wl, wr;
};

constexpr int kBwdBlockM = 128;   // dQ kernel: packed query rows per workgroup
constexpr int kBwdBlockN = 128;   // dK/dV kernel: keys per workgroup (32 per wave)
constexpr int kBwdBlockNPair = 64;  // paired dK/dV kernel (head_dim 192, 256): keys per workgroup
constexpr int kBwdTileM = 64;     // dK/dV kernel: queries per step
constexpr int kBwdTileN = 64;     // dQ kernel: keys per step

// Keys per dK/dV workgroup at a head dimension: head_dim 192 and 256 run the
// paired kernel, whose two waves per 32 keys each hold one of the dK, dV
// accumulators.
inline int bwd_block_n(int head_dim) { return head_dim > 128 ? kBwdBlockNPair : kBwdBlockN; }

// Elements of the dpsum workspace (float32) for a; lse_log2 has as many.
inline int64_t bwd_dpsum_elems(const BwdArgs& a) {
  return a.cu_q != nullptr ? (int64_t)a.hq * a.total_q
                           : (int64_t)a.batch * a.hq * a.seqlen_q;
}

// Splits of the dK/dV walk: enough workgroups for about two per compute
// unit of a 256-unit device, at most four (each split adds a float32 partial
// of dK and dV to write and reduce).
inline int bwd_splits(const BwdArgs& a, int head_dim) {
  const int bn = bwd_block_n(head_dim);
  const int64_t nblocks = ((int64_t)a.seqlen_k + bn - 1) / bn;
  const int64_t wg = nblocks * a.hkv * a.batch;
  if (wg <= 0 || a.batch > 16383) return 1;
  const int64_t s = (512 + wg - 1) / wg;
  return (int)(s < 1 ? 1 : (s > 4 ? 4 : s));
}

inline int64_t bwd_part_elems(const BwdArgs& a, int splits, int head_dim) {
  return splits > 1 ? (int64_t)splits * a.batch * a.seqlen_k * a.hkv * 2 * head_dim : 0;
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s);

}  // namespace mi_attn
