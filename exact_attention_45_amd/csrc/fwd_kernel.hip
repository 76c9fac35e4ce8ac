// Prefill forward: fused exact attention, one workgroup per (128 packed query
// rows, KV head, sequence).
//
// Method (mslk flash_attn interface.py page, `_flash_attn_fwd`; the online
// softmax in the exp2 domain with scale*log2(e) folded into one FMA, as the
// flash_bwd_sm100.py page's P = exp2(S*scale_log2 - LSE*log2e) recompute):
//   for each K/V tile of 64 keys in the workgroup's visible range:
//     S^T  = K * Q^T                         (bf16 MFMA, fp32 accumulate)
//     mask keys outside [i+off-wl, i+off+wr] and beyond seqlen_k (edge tiles)
//     m'   = max(m, rowmax S);  alpha = exp2((m - m') * c);  c = scale*log2e
//     P    = exp2(S*c - m'*c)                (rounded to bf16 for the MFMA)
//     l    = alpha*l + rowsum P;  O = alpha*O + P*V
//   O /= l;  LSE = m*scale + ln(l);  rows with no visible key: O = 0, LSE = -inf.
//
// MI355X mapping:
//   * 4 waves x 32 query rows. Rows are "packed": the r = Hq/Hkv query heads
//     that share a KV head are folded into the row index (row = pos*r + head
//     offset), so one K/V tile serves all of them (GQA packing, interface
//     page `pack_gqa`; the sm_120 PR page's qhead-into-seqlen fold).
//   * Both GEMMs are transposed (see attn_common.hpp) so each lane owns one
//     query: row max needs one exchange with lane ^ 32, row sum none.
//   * K tile row-major and V tile transposed in LDS; the next tile's global
//     loads are issued into registers before the current tile's math.
//   * Tiles wholly outside the causal/window band are never visited; only
//     edge tiles pay for per-element masking.
//   * Launch order: heaviest (latest) query blocks first, KV head fastest, so
//     the 8 XCDs (round-robin workgroup placement) each keep a fixed subset
//     of KV heads hot in their L2.
#include <climits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

template <int D>
struct FwdTile {
  static constexpr int BM = kFwdBlockM;
  static constexpr int BN = kFwdBlockN;
  static constexpr int KS = D + 8;        // K tile row stride (elements)
  static constexpr int VS = BN + 4;       // V^T tile row stride (elements)
  static constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  static constexpr int NCH = BN * CPR / 256;  // chunks per thread per tensor
  static_assert(NCH * 256 == BN * CPR, "tile must split evenly over 256 threads");
};

template <int D>
__global__ __launch_bounds__(256) void fwd_kernel(const FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int BM = T::BM, BN = T::BN, KS = T::KS, VS = T::VS, CPR = T::CPR, NCH = T::NCH;
  __shared__ __attribute__((aligned(16))) __bf16 sK[BN * KS];
  __shared__ __attribute__((aligned(16))) __bf16 sV[D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: heavy query blocks first, (KV head, sequence) fastest
  const int nhb = a.hkv * a.batch;
  const int lin = blockIdx.x;
  const int hb = lin % nhb;
  const int mb = a.num_m_blocks - 1 - lin / nhb;
  const int hk = hb % a.hkv;
  const int b = hb / a.hkv;

  int sq = a.seqlen_q, sk = a.seqlen_k;
  int64_t q_base, k_base, v_base, o_base;
  int q_tok0 = 0;
  if (a.cu_q != nullptr) {
    q_tok0 = a.cu_q[b];
    sq = a.cu_q[b + 1] - q_tok0;
    const int k_tok0 = a.cu_k[b];
    sk = a.cu_k[b + 1] - k_tok0;
    q_base = (int64_t)q_tok0 * a.q_rs;
    o_base = (int64_t)q_tok0 * a.o_rs;
    k_base = (int64_t)k_tok0 * a.k_rs;
    v_base = (int64_t)k_tok0 * a.v_rs;
  } else {
    q_base = (int64_t)b * a.q_bs;
    o_base = (int64_t)b * a.o_bs;
    k_base = (int64_t)b * a.k_bs;
    v_base = (int64_t)b * a.v_bs;
  }
  const int r = a.group;
  const int rows = sq * r;
  const int row0 = mb * BM;
  if (row0 >= rows) return;  // uniform over the workgroup

  // ---- this lane's query row
  const int prow = row0 + wave * 32 + c32;
  const bool valid = prow < rows;
  const int pos = valid ? prow / r : 0;
  const int hq = hk * r + (valid ? prow - (prow / r) * r : 0);

  const int off = sk - sq;  // bottom-right alignment
  const int lo = a.wl >= 0 ? pos + off - a.wl : INT_MIN / 2;
  const int hi = min(a.wr >= 0 ? pos + off + a.wr : INT_MAX / 2, sk - 1);

  // workgroup-wide visible key range
  const int pos_min = row0 / r;
  const int pos_max = (min(row0 + BM, rows) - 1) / r;
  const int kv_lo = a.wl >= 0 ? max(0, pos_min + off - a.wl) : 0;
  const int kv_hi = a.wr >= 0 ? min(sk, pos_max + off + a.wr + 1) : sk;  // exclusive
  const int n_begin = kv_lo / BN;
  const int n_end = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : n_begin;
  // a tile [n0, n0+BN) is fully visible to every row iff
  //   n0 + BN <= sk, n0 + BN - 1 <= pos_min + off + wr, n0 >= pos_max + off - wl
  const int full_hi = a.wr >= 0 ? pos_min + off + a.wr : INT_MAX / 2;
  const int full_lo = a.wl >= 0 ? pos_max + off - a.wl : INT_MIN / 2;

  // ---- Q^T fragments (B operand), kept in registers for the whole loop
  const __bf16* qp = static_cast<const __bf16*>(a.q) + q_base + (int64_t)pos * a.q_rs +
                     (int64_t)hq * a.q_hs;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = valid ? as_bf16x8(ld16(qp + 16 * c + 8 * half)) : zero_bf16x8();

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.0f;

  // ---- K/V tile staging: each wave instruction moves 32 rows x 2 chunks
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  uint4 kreg[NCH], vreg[NCH];

  auto chunk_row = [&](int u) { return ((u * 4 + wave) & 1) * 32 + c32; };
  auto chunk_col = [&](int u) { return (((u * 4 + wave) >> 1) * 2 + half) * 8; };

  auto load_tile = [&](int n0) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int key = n0 + chunk_row(u);
      const int col = chunk_col(u);
      if (key < sk) {
        kreg[u] = ld16(kp + (int64_t)key * a.k_rs + col);
        vreg[u] = ld16(vp + (int64_t)key * a.v_rs + col);
      } else {
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int row = chunk_row(u);
      const int col = chunk_col(u);
      *reinterpret_cast<uint4*>(&sK[row * KS + col]) = kreg[u];
      const bf16x8 vv = as_bf16x8(vreg[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sV[(col + e) * VS + row] = vv[e];
    }
  };

  const float c = a.scale_log2;
  if (n_begin < n_end) load_tile(n_begin * BN);

  for (int nb = n_begin; nb < n_end; ++nb) {
    const int n0 = nb * BN;
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (nb + 1 < n_end) load_tile(n0 + BN);

    // S^T = K Q^T: two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
      const __bf16* krow = &sK[(kb * 32 + c32) * KS + 8 * half];
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * cc);
        s[kb] = mfma32(kf, qf[cc], s[kb]);
      }
    }

    const bool full = (n0 + BN <= sk) && (n0 + BN - 1 <= full_hi) && (n0 >= full_lo);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = n0 + kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (key < lo || key > hi) s[kb][v] = kNegInf;
        }
    }

    // online softmax (exp2 domain)
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[kb][v]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt);
    const float ms = (m_new == kNegInf) ? 0.0f : m_new * c;
    // exactly 1 when the max did not move (m_run - m_new == 0), exactly 0
    // when nothing was visible before (m_run = -inf)
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2((m_run - m_new) * c);
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s[kb][v], c, -ms));
        s[kb][v] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

    // P^T fragments: MFMA t covers keys 16t..16t+15 of the tile. Lane half h
    // supplies keys {16t+4h+j, 16t+8+4h+j : j<4}; the V^T fragment below
    // uses the same key order, so the contraction is unchanged.
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1;
      const int i0 = 2 * (t & 1);
      pf[t] = cat(cvt4(s[kb][4 * i0 + 0], s[kb][4 * i0 + 1], s[kb][4 * i0 + 2], s[kb][4 * i0 + 3]),
                  cvt4(s[kb][4 * i0 + 4], s[kb][4 * i0 + 5], s[kb][4 * i0 + 6], s[kb][4 * i0 + 7]));
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const __bf16* vrow = &sV[(db * 32 + c32) * VS + 4 * half];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 16 * t);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 16 * t + 8);
        o[db] = mfma32(cat(v0, v1), pf[t], o[db]);
      }
    }
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (valid) {
    __bf16* op = static_cast<__bf16*>(a.out) + o_base + (int64_t)pos * a.o_rs +
                 (int64_t)hq * a.o_hs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<bf16x4*>(op + d0) =
            cvt4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                 o[db][4 * i + 3] * inv);
      }
    if (half == 0 && a.lse != nullptr) {
      const float lse = l_tot > 0.0f ? m_run * a.scale + __logf(l_tot) : kNegInf;
      const int64_t li = a.cu_q != nullptr
                             ? (int64_t)hq * a.total_q + q_tok0 + pos
                             : ((int64_t)b * a.hq + hq) * sq + pos;
      a.lse[li] = lse;
    }
  }
}

template <int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.num_m_blocks * a.hkv * a.batch;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_kernel<D>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_fwd<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<128>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<256>(const FwdArgs&, hipStream_t);

}  // namespace mi_attn
