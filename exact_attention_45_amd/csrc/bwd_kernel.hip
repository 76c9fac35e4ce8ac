// Attention backward for head_dim 64/128: dQ, dK, dV of exact attention.
//
// Method (Blackwell backward page flash_bwd_sm100.py: P is recomputed from
// the scores and the forward LSE in the exp2 domain, dV = P^T dO,
// dP = dO V^T, dS = P (dP - dPsum), dQ = scale dS K, dK = scale dS^T Q; the
// interface page's backward preprocess computes dPsum as the row sum of
// O * dO, and its postprocess scales and, with GQA, sums dK/dV over the
// query heads of a KV head).
//
// Three launches, no atomics, deterministic:
//   bwd_pre_kernel   dPsum[row] = sum_d O[row, d] dO[row, d]  (float32 workspace)
//   bwd_dq_kernel    one workgroup per 128 packed query rows (as the forward
//                    packs GQA heads): walks the visible 64-key tiles, per
//                    tile S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - dPsum),
//                    dQ^T += K^T dS^T; dQ is written once, scaled
//   bwd_dkdv_kernel  one workgroup per 128 keys of a KV head: walks every
//                    query head of the group and its visible 64-query tiles,
//                    per tile S = Q K^T, dP = dO V^T, dS = P (dP - dPsum),
//                    dV^T += dO^T P, dK^T += Q^T dS; dK (scaled) and dV are
//                    written once, already summed over the group
// S and dP are recomputed in both kernels (seven tile products per score
// tile instead of five) in exchange for no dQ accumulation buffer and no
// atomic traffic.
//
// Every product is v_mfma_f32_32x32x16_bf16 in the orientation of the
// forward kernels: the operand that stays fixed for the whole walk (the
// lane's query rows, or the lane's keys) is the B operand held in registers,
// the streamed tile is read from LDS as row fragments (A of S and dP) and,
// by transposing reads, as the A operand of the accumulating products, whose
// B operand (P, dS) comes straight from the score accumulators in the
// matching contraction order (attn_common.hpp). Tiles are staged through
// registers: the next tile's loads are in flight while the current one is
// computed.
#include <climits>

#include "attn_common.hpp"
#include "bwd.hpp"

namespace mi_attn {

// ---------------------------------------------------------------- dPsum ----

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdArgs a) {
  constexpr int CPR = D / 8;         // lanes per (token, head) row, 8 elements each
  constexpr int RPB = 256 / CPR;     // rows per workgroup
  const int64_t ntok = a.cu_q != nullptr ? (int64_t)a.total_q : (int64_t)a.batch * a.seqlen_q;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  const bool ok = row < ntok * a.hq;
  const int64_t t = ok ? row / a.hq : 0;
  const int h = ok ? (int)(row - t * a.hq) : 0;
  int64_t o_off, do_off, out_idx;
  if (a.cu_q != nullptr) {
    o_off = t * a.o_rs + (int64_t)h * a.o_hs;
    do_off = t * a.do_rs + (int64_t)h * a.do_hs;
    out_idx = (int64_t)h * a.total_q + t;
  } else {
    const int64_t b = t / a.seqlen_q, pos = t - b * a.seqlen_q;
    o_off = b * a.o_bs + pos * a.o_rs + (int64_t)h * a.o_hs;
    do_off = b * a.do_bs + pos * a.do_rs + (int64_t)h * a.do_hs;
    out_idx = (b * a.hq + h) * a.seqlen_q + pos;
  }
  float acc = 0.0f;
  if (ok) {
    const bf16x8 o = as_bf16x8(ld16(static_cast<const __bf16*>(a.o) + o_off + 8 * c));
    const bf16x8 g = as_bf16x8(ld16(static_cast<const __bf16*>(a.dout) + do_off + 8 * c));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)g[i], acc);
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, CPR);
  if (ok && c == 0) a.dpsum[out_idx] = acc;
}

// ----------------------------------------------------------- shared bits ----

// Logical chunk ch of tile row `row` sits at chunk position ch ^ swz_key(row)
// (attn_common.hpp). Row fragments: lane (c32, half) reads chunk
// 2*cc + half of row c32 (+32 per 32-row block; same swizzle).
template <int D>
struct BwdTile {
  static constexpr int ROW_B = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int ROWS = 64;
  static constexpr int TILE_B = ROWS * ROW_B;
  static constexpr int NL = ROWS * CPR / 256;  // 16-byte chunks per thread per tile
  static_assert(NL * 256 == ROWS * CPR, "a tile splits evenly over 256 threads");
};

// Transposing-read offsets of a 64-row tile (the V^T fragment pattern of
// attn_common.hpp): fragment (t, db) covers rows 16t..16t+15 and columns
// 32db..32db+31.
__device__ __forceinline__ void tr_offsets(int lane, int row_b, int tr[2]) {
  const int half = lane >> 5;
  const int g = lane >> 4, j = lane & 15;
  const int row = 4 * half + (j >> 2);
  const int c = (g & 1) * 2 + ((j & 3) >> 1);
  const int f = swz_key(row);
#pragma unroll
  for (int i = 0; i < 2; ++i) tr[i] = row * row_b + (((4 * i + c) ^ f) * 16) + (j & 1) * 8;
}

template <int ROW_B>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, const int tr[2], int t, int db) {
  const char* p = tile + (16 * t) * ROW_B + (db >> 1) * 128 + tr[db & 1];
  const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(p));
  const bf16x4 v1 = ds_read_tr16(reinterpret_cast<const __bf16*>(p + 8 * ROW_B));
  return cat(v0, v1);
}

// B-operand fragments (contraction over the 64 rows of a tile) from two
// 32x32 accumulators, in the order the transposing reads deliver.
__device__ __forceinline__ void acc_to_frags(const f32x16 x[2], bf16x8 f[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kb = t >> 1, i0 = 8 * (t & 1);
    f[t] = cat(cvt4(x[kb][i0 + 0], x[kb][i0 + 1], x[kb][i0 + 2], x[kb][i0 + 3]),
               cvt4(x[kb][i0 + 4], x[kb][i0 + 5], x[kb][i0 + 6], x[kb][i0 + 7]));
  }
}

// ------------------------------------------------------------------- dQ ----

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int ROW_B = T::ROW_B, CPR = T::CPR, TILE_B = T::TILE_B, NL = T::NL;
  constexpr int BM = kBwdBlockM, BN = kBwdTileN;
  static_assert(BN == T::ROWS, "one staged tile per key step");
  __shared__ __attribute__((aligned(16))) char smem[2 * TILE_B];  // K tile, V tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, half = lane >> 5;
  const int mb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;

  int sq = a.seqlen_q, sk = a.seqlen_k, q_tok0 = 0;
  int64_t q_base, do_base, dq_base, k_base, v_base;
  if (a.cu_q != nullptr) {
    q_tok0 = a.cu_q[b];
    sq = a.cu_q[b + 1] - q_tok0;
    q_base = (int64_t)q_tok0 * a.q_rs;
    do_base = (int64_t)q_tok0 * a.do_rs;
    dq_base = (int64_t)q_tok0 * a.dq_rs;
  } else {
    q_base = (int64_t)b * a.q_bs;
    do_base = (int64_t)b * a.do_bs;
    dq_base = (int64_t)b * a.dq_bs;
  }
  if (a.cu_k != nullptr) {
    const int k0 = a.cu_k[b];
    sk = a.cu_k[b + 1] - k0;
    k_base = (int64_t)k0 * a.k_rs;
    v_base = (int64_t)k0 * a.v_rs;
  } else {
    k_base = (int64_t)b * a.k_bs;
    v_base = (int64_t)b * a.v_bs;
  }
  sq = uniform(sq);
  sk = uniform(sk);
  const int r = a.group;
  const int rows = sq * r;
  const int row0 = mb * BM;
  if (row0 >= rows) return;  // uniform over the workgroup

  const int prow = row0 + wave * 32 + c32;
  const bool valid = prow < rows;
  const int pos = valid ? prow / r : 0;
  const int hq = hk * r + (valid ? prow - (prow / r) * r : 0);
  const int off = sk - sq;
  const int lo = a.wl >= 0 ? pos + off - a.wl : INT_MIN / 2;
  const int hi = min(a.wr >= 0 ? pos + off + a.wr : INT_MAX / 2, sk - 1);
  const int pos_min = uniform(row0 / r);
  const int pos_max = uniform((min(row0 + BM, rows) - 1) / r);
  const int kv_lo = a.wl >= 0 ? max(0, pos_min + off - a.wl) : 0;
  const int kv_hi = a.wr >= 0 ? min(sk, pos_max + off + a.wr + 1) : sk;  // exclusive
  const int n_begin = uniform(kv_lo / BN);
  const int n_end = uniform(kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : n_begin);

  // this lane's row: Q^T and dO^T fragments (B operands), LSE, dPsum
  const __bf16* qp = static_cast<const __bf16*>(a.q) + q_base + (int64_t)pos * a.q_rs +
                     (int64_t)hq * a.q_hs;
  const __bf16* gp = static_cast<const __bf16*>(a.dout) + do_base + (int64_t)pos * a.do_rs +
                     (int64_t)hq * a.do_hs;
  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    const bf16x8 x = as_bf16x8(ld16(qp + 16 * cc + 8 * half));
    const bf16x8 y = as_bf16x8(ld16(gp + 16 * cc + 8 * half));
    qf[cc] = valid ? x : zero_bf16x8();
    gf[cc] = valid ? y : zero_bf16x8();
  }
  const int64_t li = a.cu_q != nullptr ? (int64_t)hq * a.total_q + q_tok0 + pos
                                       : ((int64_t)b * a.hq + hq) * sq + pos;
  const float lse = valid ? a.lse[li] : kNegInf;
  const float dps = valid ? a.dpsum[li] : 0.0f;
  // a row with no visible key (LSE = -inf) gets P = exp2(x - inf) = 0
  const float lse2 = lse == kNegInf ? __builtin_huge_valf() : lse * kLog2e;
  const float c = a.scale_log2;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqa[i] = zero_f32x16();

  // staging: thread chunk e = tid + 256 i -> tile row e / CPR, chunk e % CPR
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  uint32_t gk[NL], gv[NL], sl[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + 256 * i, row = e / CPR, ch = e % CPR;
    gk[i] = (uint32_t)(row * a.k_rs * 2 + ch * 16);
    gv[i] = (uint32_t)(row * a.v_rs * 2 + ch * 16);
    sl[i] = (uint32_t)(row * ROW_B + ((ch ^ swz_key(row)) * 16));
  }
  uint4 kreg[NL], vreg[NL];
  auto load = [&](int n0) __attribute__((always_inline)) {
    const int nrows = min(sk - n0, BN);  // >= 1
    const auto kr = make_rsrc(kp + (int64_t)n0 * a.k_rs, (uint32_t)((nrows - 1) * a.k_rs * 2 + ROW_B));
    const auto vr = make_rsrc(vp + (int64_t)n0 * a.v_rs, (uint32_t)((nrows - 1) * a.v_rs * 2 + ROW_B));
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kreg[i] = buf_ld16(kr, gk[i]);
      vreg[i] = buf_ld16(vr, gv[i]);
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      *reinterpret_cast<uint4*>(smem + sl[i]) = kreg[i];
      *reinterpret_cast<uint4*>(smem + TILE_B + sl[i]) = vreg[i];
    }
  };

  int rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ swz_key(c32)) * 16);
  int tr[2];
  tr_offsets(lane, ROW_B, tr);

  auto compute = [&](int n0) __attribute__((always_inline)) {
    const char* kt = smem;
    const char* vt = smem + TILE_B;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
      dp[kb] = zero_f32x16();
    }
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int ro = kb * 32 * ROW_B + rd[cc];
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(kt + ro), qf[cc], s[kb]);
        dp[kb] = mfma32(*reinterpret_cast<const bf16x8*>(vt + ro), gf[cc], dp[kb]);
      }
    // element (kb, v) holds key n0 + 4*half + 32*kb + 8*(v>>2) + (v&3)
    const uint64_t vis = vis64(lo - n0 - 4 * half, hi - n0 - 4 * half);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t w = (uint32_t)(vis >> (32 * kb));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = mask_by_bit(s[kb][v], w, 8 * (v >> 2) + (v & 3));
        const float p = fast_exp2(fmaf(x, c, -lse2));
        s[kb][v] = p * (dp[kb][v] - dps);  // dS^T
      }
    }
    bf16x8 dsf[4];
    acc_to_frags(s, dsf);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dqa[db] = mfma32(tr_frag<ROW_B>(kt, tr, t, db), dsf[t], dqa[db]);
  };

  if (n_end > n_begin) {
    load(n_begin * BN);
    for (int n = n_begin; n < n_end; ++n) {
      __syncthreads();  // every wave is done with the previous tile
      store();
      __syncthreads();
      if (n + 1 < n_end) load((n + 1) * BN);
      compute(n * BN);
    }
  }

  if (valid) {
    __bf16* dqp = static_cast<__bf16*>(a.dq) + dq_base + (int64_t)pos * a.dq_rs +
                  (int64_t)hq * a.dq_hs;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<bf16x4*>(dqp + d0) =
            cvt4(dqa[db][4 * i] * sc, dqa[db][4 * i + 1] * sc, dqa[db][4 * i + 2] * sc,
                 dqa[db][4 * i + 3] * sc);
      }
  }
}

// ---------------------------------------------------------------- dK dV ----

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(const BwdArgs a) {
  using T = BwdTile<D>;
  constexpr int ROW_B = T::ROW_B, CPR = T::CPR, TILE_B = T::TILE_B, NL = T::NL;
  constexpr int BNK = kBwdBlockN, BM = kBwdTileM;
  static_assert(BM == T::ROWS, "one staged tile per query step");
  // Q tile, dO tile, then LSE*log2e and dPsum of the tile's 64 queries
  __shared__ __attribute__((aligned(16))) char smem[2 * TILE_B + 2 * BM * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, half = lane >> 5;
  const int nb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;

  int sq = a.seqlen_q, sk = a.seqlen_k, q_tok0 = 0;
  int64_t q_base, do_base, k_base, v_base, dk_base, dv_base;
  if (a.cu_q != nullptr) {
    q_tok0 = a.cu_q[b];
    sq = a.cu_q[b + 1] - q_tok0;
    q_base = (int64_t)q_tok0 * a.q_rs;
    do_base = (int64_t)q_tok0 * a.do_rs;
  } else {
    q_base = (int64_t)b * a.q_bs;
    do_base = (int64_t)b * a.do_bs;
  }
  if (a.cu_k != nullptr) {
    const int k0 = a.cu_k[b];
    sk = a.cu_k[b + 1] - k0;
    k_base = (int64_t)k0 * a.k_rs;
    v_base = (int64_t)k0 * a.v_rs;
    dk_base = (int64_t)k0 * a.dk_rs;
    dv_base = (int64_t)k0 * a.dv_rs;
  } else {
    k_base = (int64_t)b * a.k_bs;
    v_base = (int64_t)b * a.v_bs;
    dk_base = (int64_t)b * a.dk_bs;
    dv_base = (int64_t)b * a.dv_bs;
  }
  sq = uniform(sq);
  sk = uniform(sk);
  const int j0 = nb * BNK;
  if (j0 >= sk) return;  // uniform over the workgroup

  const int key = j0 + wave * 32 + c32;
  const bool kvalid = key < sk;
  const int kk = kvalid ? key : 0;
  const int r = a.group;
  const int off = sk - sq;
  // queries that see key j: j - off - wr <= i <= j - off + wl, 0 <= i < sq
  int qlo = a.wr >= 0 ? max(0, kk - off - a.wr) : 0;
  int qhi = a.wl >= 0 ? min(sq - 1, kk - off + a.wl) : sq - 1;
  if (!kvalid) qhi = qlo - 1;
  const int j1 = min(sk, j0 + BNK) - 1;
  const int i_lo = uniform(a.wr >= 0 ? max(0, j0 - off - a.wr) : 0);
  const int i_hi = uniform(a.wl >= 0 ? min(sq - 1, j1 - off + a.wl) : sq - 1);
  const int m_begin = i_lo / BM;
  const int nm = i_hi >= i_lo ? i_hi / BM - m_begin + 1 : 0;
  const int n_it = uniform(nm * r);

  // this lane's key: K^T and V^T fragments (B operands)
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)kk * a.k_rs +
                     (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)kk * a.v_rs +
                     (int64_t)hk * a.v_hs;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    const bf16x8 x = as_bf16x8(ld16(kp + 16 * cc + 8 * half));
    const bf16x8 y = as_bf16x8(ld16(vp + 16 * cc + 8 * half));
    kf[cc] = kvalid ? x : zero_bf16x8();
    vf[cc] = kvalid ? y : zero_bf16x8();
  }
  const float c = a.scale_log2;

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dka[i] = zero_f32x16();
    dva[i] = zero_f32x16();
  }

  uint32_t gq[NL], gd[NL], sl[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + 256 * i, row = e / CPR, ch = e % CPR;
    gq[i] = (uint32_t)(row * a.q_rs * 2 + ch * 16);
    gd[i] = (uint32_t)(row * a.do_rs * 2 + ch * 16);
    sl[i] = (uint32_t)(row * ROW_B + ((ch ^ swz_key(row)) * 16));
  }
  uint4 qreg[NL], dreg[NL];
  float sreg = 0.0f;  // threads 0..63: LSE*log2e of query m0+tid; 64..127: dPsum of m0+tid-64
  // iteration it: query head hk*r + it / nm, query tile m_begin + it % nm
  auto load = [&](int it) __attribute__((always_inline)) {
    const int h = uniform(hk * r + it / nm);
    const int m0 = uniform((m_begin + it % nm) * BM);
    const int nrows = min(sq - m0, BM);  // >= 1
    const __bf16* q0 = static_cast<const __bf16*>(a.q) + q_base + (int64_t)m0 * a.q_rs +
                       (int64_t)h * a.q_hs;
    const __bf16* g0 = static_cast<const __bf16*>(a.dout) + do_base + (int64_t)m0 * a.do_rs +
                       (int64_t)h * a.do_hs;
    const auto qr = make_rsrc(q0, (uint32_t)((nrows - 1) * a.q_rs * 2 + ROW_B));
    const auto gr = make_rsrc(g0, (uint32_t)((nrows - 1) * a.do_rs * 2 + ROW_B));
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      qreg[i] = buf_ld16(qr, gq[i]);
      dreg[i] = buf_ld16(gr, gd[i]);
    }
    if (tid < 2 * BM) {
      const int qi = m0 + (tid & (BM - 1));
      const int64_t li = a.cu_q != nullptr ? (int64_t)h * a.total_q + q_tok0 + qi
                                           : ((int64_t)b * a.hq + h) * sq + qi;
      if (tid < BM) {
        const float l = qi < sq ? a.lse[li] : kNegInf;
        sreg = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
      } else {
        sreg = qi < sq ? a.dpsum[li] : 0.0f;
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      *reinterpret_cast<uint4*>(smem + sl[i]) = qreg[i];
      *reinterpret_cast<uint4*>(smem + TILE_B + sl[i]) = dreg[i];
    }
    if (tid < 2 * BM) reinterpret_cast<float*>(smem + 2 * TILE_B)[tid] = sreg;
  };

  int rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ swz_key(c32)) * 16);
  int tr[2];
  tr_offsets(lane, ROW_B, tr);

  auto compute = [&](int m0) __attribute__((always_inline)) {
    const char* qt = smem;
    const char* gt = smem + TILE_B;
    const float* l2s = reinterpret_cast<const float*>(smem + 2 * TILE_B);
    const float* dss = l2s + BM;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = zero_f32x16();
      dp[qb] = zero_f32x16();
    }
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int ro = qb * 32 * ROW_B + rd[cc];
        s[qb] = mfma32(*reinterpret_cast<const bf16x8*>(qt + ro), kf[cc], s[qb]);
        dp[qb] = mfma32(*reinterpret_cast<const bf16x8*>(gt + ro), vf[cc], dp[qb]);
      }
    // element (qb, v) holds query m0 + 4*half + 32*qb + 8*(v>>2) + (v&3), key `key`
    const uint64_t vis = vis64(qlo - m0 - 4 * half, qhi - m0 - 4 * half);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const uint32_t w = (uint32_t)(vis >> (32 * qb));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qo = 32 * qb + 8 * i + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dss + qo);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * i + j;
          const float x = mask_by_bit(s[qb][v], w, 8 * i + j);
          const float p = fast_exp2(fmaf(x, c, -l4[j]));
          s[qb][v] = p;
          dp[qb][v] = p * (dp[qb][v] - d4[j]);  // dS
        }
      }
    }
    bf16x8 pf[4], dsf[4];
    acc_to_frags(s, pf);
    acc_to_frags(dp, dsf);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        dva[db] = mfma32(tr_frag<ROW_B>(gt, tr, t, db), pf[t], dva[db]);
        dka[db] = mfma32(tr_frag<ROW_B>(qt, tr, t, db), dsf[t], dka[db]);
      }
  };

  if (n_it > 0) {
    load(0);
    for (int it = 0; it < n_it; ++it) {
      __syncthreads();  // every wave is done with the previous tile
      store();
      __syncthreads();
      const int m0 = uniform((m_begin + it % nm) * BM);
      if (it + 1 < n_it) load(it + 1);
      compute(m0);
    }
  }

  if (kvalid) {
    __bf16* dkp = static_cast<__bf16*>(a.dk) + dk_base + (int64_t)key * a.dk_rs +
                  (int64_t)hk * a.dk_hs;
    __bf16* dvp = static_cast<__bf16*>(a.dv) + dv_base + (int64_t)key * a.dv_rs +
                  (int64_t)hk * a.dv_hs;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<bf16x4*>(dkp + d0) =
            cvt4(dka[db][4 * i] * sc, dka[db][4 * i + 1] * sc, dka[db][4 * i + 2] * sc,
                 dka[db][4 * i + 3] * sc);
        *reinterpret_cast<bf16x4*>(dvp + d0) =
            cvt4(dva[db][4 * i], dva[db][4 * i + 1], dva[db][4 * i + 2], dva[db][4 * i + 3]);
      }
  }
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  const int64_t ntok = a.cu_q != nullptr ? (int64_t)a.total_q : (int64_t)a.batch * a.seqlen_q;
  const int64_t pre_rows = ntok * a.hq;
  if (pre_rows > 0) {
    const int64_t rpb = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((pre_rows + rpb - 1) / rpb)),
                       dim3(256), 0, s, a);
  }
  const int64_t mblocks = ((int64_t)a.seqlen_q * a.group + kBwdBlockM - 1) / kBwdBlockM;
  if (mblocks > 0 && a.batch > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)mblocks, a.hkv, a.batch), dim3(256), 0,
                       s, a);
  const int64_t nblocks = ((int64_t)a.seqlen_k + kBwdBlockN - 1) / kBwdBlockN;
  if (nblocks > 0 && a.batch > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)nblocks, a.hkv, a.batch), dim3(256),
                       0, s, a);
  return hipGetLastError();
}

template hipError_t launch_bwd<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd<128>(const BwdArgs&, hipStream_t);

}  // namespace mi_attn
