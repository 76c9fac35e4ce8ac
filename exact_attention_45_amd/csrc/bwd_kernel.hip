// Attention backward for head_dim 64/96/128/192/256: dQ, dK, dV of exact
// attention.
//
// Method (Blackwell backward page flash_bwd_sm100.py: P is recomputed from
// the scores and the forward LSE in the exp2 domain, dV = P^T dO,
// dP = dO V^T, dS = P (dP - dPsum), dQ = scale dS K, dK = scale dS^T Q; the
// interface page's backward preprocess computes dPsum as the row sum of
// O * dO, and its postprocess scales and, with GQA, sums dK/dV over the
// query heads of a KV head).
//
// Three or four launches, no atomics, deterministic:
//   bwd_pre_kernel   dPsum[row] = sum_d O[row, d] dO[row, d] and LSE[row] log2 e
//                    (float32 workspace; +inf for LSE = -inf, so that the
//                    probabilities exp2(S c - LSE log2 e) of such a row are 0)
//   bwd_dq_kernel    one workgroup per 128 packed query rows (as the forward
//                    packs GQA heads): walks the visible 64-key tiles, per
//                    tile S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - dPsum),
//                    dQ^T += K^T dS^T; dQ is written once, scaled
//   bwd_dkdv_kernel  one workgroup per 128 keys of a KV head (32 per wave)
//                    and split: walks its part of (query head of the group,
//                    visible 64-query tile), per tile S = Q K^T, dP = dO V^T,
//                    dS = P (dP - dPsum), dV^T += dO^T P, dK^T += Q^T dS;
//                    with one split dK (scaled) and dV are written once,
//                    already summed over the group; with several, float32
//                    partials go to the workspace and
//   bwd_dkv_reduce_kernel  sums them in split order (deterministic)
// At head_dim 192 and 256 bwd_dkdv_pair_kernel takes the dK/dV walk: 64 keys per
// workgroup, each 32-key column served by two waves, one computing P and
// dV, the other dP, dS and dK (P of half the tile's queries and the raw
// scores of the other half pass between them through LDS).
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

// Head dims 96 and 192 run in the layouts of 128 and 256 (bwd_width): LDS
// tile rows, lane groups and swizzles have the wider shape, every product
// loops over the real head_dim only, and tile descriptors end at the real
// row, so the padding columns are never read.
template <int D>
constexpr int bwd_width() {
  return D == 96 ? 128 : (D == 192 ? 256 : D);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdArgs a) {
  constexpr int CPR = bwd_width<D>() / 8;  // lanes per (token, head) row, 8 elements each
  constexpr int RPB = 256 / CPR;           // rows per workgroup
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
  if (ok && c < D / 8) {  // lanes past the row (D = 96, 192) add nothing
    const bf16x8 o = as_bf16x8(ld16(static_cast<const __bf16*>(a.o) + o_off + 8 * c));
    const bf16x8 g = as_bf16x8(ld16(static_cast<const __bf16*>(a.dout) + do_off + 8 * c));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)o[i], (float)g[i], acc);
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, CPR);
  if (ok && c == 0) {
    a.dpsum[out_idx] = acc;
    const float l = a.lse[out_idx];
    a.lse_log2[out_idx] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
  }
}

// ----------------------------------------------------------- shared bits ----

// Logical chunk ch of tile row `row` sits at chunk position ch ^ tswz<D>(row).
// tswz extends swz_key (attn_common.hpp) for D >= 128 by key bit 3 into
// chunk bit 3, as the forward does for its K tiles: the 16 lanes an LDS
// cycle serves, reading one logical chunk of 16 consecutive rows, then hit
// 16 different chunk positions (row fragments conflict-free), while each
// transposing read (8 rows with the same bit 3) sees swz_key alone, shifted
// by 128 bytes within its 256-byte quarter. Row fragments: lane (c32, half)
// reads chunk 2*cc + half of row c32 (+32 per 32-row block; same swizzle).
template <int D>
__device__ __forceinline__ int tswz(int row) {
  return D >= 128 ? (swz_key(row) | (((row >> 3) & 1) << 3)) : swz_key(row);
}
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

// The second read covers rows with bit 3 set: under tswz<D> (D >= 128) its
// 128-byte segment is the other one of the 256-byte pair.
template <int ROW_B>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, const int tr[2], int t, int db) {
  constexpr int FLIP = ROW_B >= 256 ? 1 : 0;
  const char* p = tile + (16 * t) * ROW_B + tr[db & 1];
  const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(p + (db >> 1) * 128));
  const bf16x4 v1 = ds_read_tr16(
      reinterpret_cast<const __bf16*>(p + 8 * ROW_B + ((db >> 1) ^ FLIP) * 128));
  return cat(v0, v1);
}

// Direct global-to-LDS load of one dword per lane (buffer_load_dword ... lds):
// lane i's 4 bytes at buffer offset voff land at LDS address lds_base + 4 i;
// offsets past the descriptor's bound load zero, dword by dword. Same
// conventions as dma16 (attn_common.hpp): lds_base is wave-uniform and goes
// through M0, the caller waits for the load (vmcnt) and then barriers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

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

// At head_dim 256 the row's Q^T, dO^T fragments and the dQ accumulators
// alone take 256 registers: one wave per SIMD.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bwd_width<D>() == 256 ? 1 : 2)))
void bwd_dq_kernel(const BwdArgs a) {
  constexpr int DL = bwd_width<D>();  // layout head dim
  using T = BwdTile<DL>;
  constexpr int ROW_B = T::ROW_B, CPR = T::CPR, TILE_B = T::TILE_B;
  constexpr int BM = kBwdBlockM, BN = kBwdTileN;
  static_assert(BN == T::ROWS, "one staged tile per key step");
  constexpr int BUF_B = 2 * TILE_B;  // K tile, V tile
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF_B];  // two buffers

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, half = lane >> 5;
  // Work item: heavy (late) query blocks first, (KV head, sequence) fastest.
  // Workgroups are dispatched in linear order and dealt round-robin to the
  // XCDs, so consecutive ones take different KV heads: each XCD's L2 holds
  // the K/V of few heads, and the longest causal blocks start first.
  int mb, hk, b;
  {
    const int nhb = a.hkv * a.batch;
    const int lin = uniform((int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)));
    const int hb = uniform(lin % nhb);
    mb = uniform((int)gridDim.x - 1 - lin / nhb);
    hk = uniform(hb % a.hkv);
    b = uniform(hb / a.hkv);
  }

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

  // this lane's row: Q^T and dO^T fragments (B operands), LSE log2 e, dPsum
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
  // a row with no visible key (LSE = -inf) has +inf here: P = exp2(x - inf) = 0
  const float lse2 = valid ? a.lse_log2[li] : __builtin_huge_valf();
  const float dps = valid ? a.dpsum[li] : 0.0f;
  const float c = a.scale_log2;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqa[i] = zero_f32x16();

  // K/V tiles go global -> LDS directly (dma16), double-buffered: for each
  // tensor, instruction i of wave w fills tile rows RPI*(NI*w + i) ..
  // +RPI-1; lane j lands at row offset j / CPR, physical chunk j % CPR, so it
  // loads logical chunk (j % CPR) ^ tswz(row) of that row.
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  constexpr int RPI = 1024 / ROW_B;  // rows per instruction
  constexpr int NI = BN / RPI / 4;   // instructions per wave per tensor
  static_assert(NI * RPI * 4 == BN, "a tile splits evenly over four waves");
  uint32_t kdo[NI], vdo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (NI * wave + i) + lane / CPR;
    kdo[i] = (uint32_t)(row * a.k_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
    vdo[i] = (uint32_t)(row * a.v_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
  }
  const uint32_t lds_w = (uint32_t)uniform((int)(lds_addr(smem) + NI * wave * 1024));
  auto issue = [&](int n0, int buf) __attribute__((always_inline)) {
    const int nrows = min(sk - n0, BN);  // >= 1; rows past it read as zero
    const auto kr = make_rsrc(kp + (int64_t)n0 * a.k_rs, (uint32_t)((nrows - 1) * a.k_rs * 2 + D * 2));
    const auto vr = make_rsrc(vp + (int64_t)n0 * a.v_rs, (uint32_t)((nrows - 1) * a.v_rs * 2 + D * 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(kr, kdo[i], lds_w + (uint32_t)(buf * BUF_B + i * 1024));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(vr, vdo[i], lds_w + (uint32_t)(buf * BUF_B + TILE_B + i * 1024));
  };

  int rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ tswz<DL>(c32)) * 16);
  int tr[2];
  tr_offsets(lane, ROW_B, tr);

  // One step, software-pipelined over the two 32-key blocks kb of the tile
  // so that each block's dS arithmetic runs between matrix instructions:
  //   part 1: S^T, dP^T of block 0, then of block 1 with one block-0 dS
  //           slice after each MFMA
  //   part 2: dQ^T over the 16-key steps of block 0 with one block-1 dS
  //           slice after each MFMA, then over those of block 1
  auto compute = [&](int n0, const char* kt) __attribute__((always_inline)) {
    const char* vt = kt + TILE_B;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
      dp[kb] = zero_f32x16();
    }
    // element (kb, v) holds key n0 + 4*half + 32*kb + 8*(v>>2) + (v&3)
    const uint64_t vis = vis64(lo - n0 - 4 * half, hi - n0 - 4 * half);
    // the mask runs only on tiles where some lane of the wave has a key
    // outside its visible range (edge tiles; a wave-uniform branch)
    const bool edge = __builtin_amdgcn_ballot_w64(vis != ~0ull) != 0;
    auto mask = [&](int kb) __attribute__((always_inline)) {
      if (edge) {
        const uint32_t w = (uint32_t)(vis >> (32 * kb));
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = mask_by_bit(s[kb][v], w, 8 * (v >> 2) + (v & 3));
      }
    };
    // dS^T elements [e0, e1) of block kb, in place of S^T
    auto ds = [&](int kb, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
      for (int v = e0; v < e1; ++v) {
        const float p = fast_exp2(fmaf(s[kb][v], c, -lse2));
        s[kb][v] = p * (dp[kb][v] - dps);
      }
    };
    {
      // MFMA g: block g / NS, i = g % NS: contraction step i / 2; even i:
      // S^T from K rows, odd i: dP^T from V rows
      constexpr int NS = 2 * (D / 16), N = 2 * NS, LEAD = 6;
      auto rdf = [&](int g) __attribute__((always_inline)) {
        const int kb = g / NS, i = g % NS;
        return *reinterpret_cast<const bf16x8*>((i & 1 ? vt : kt) + kb * 32 * ROW_B + rd[i >> 1]);
      };
      bf16x8 ring[LEAD];
#pragma unroll
      for (int g = 0; g < LEAD; ++g) ring[g] = rdf(g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < N; ++g) {
        const bf16x8 f = ring[g % LEAD];
        if (g + LEAD < N) ring[g % LEAD] = rdf(g + LEAD);
        const int kb = g / NS, i = g % NS;
        if (i & 1)
          dp[kb] = mfma32(f, gf[i >> 1], dp[kb]);
        else
          s[kb] = mfma32(f, qf[i >> 1], s[kb]);
        if (kb == 1) {
          if (i == 0) mask(0);
          ds(0, 16 * i / NS, 16 * (i + 1) / NS);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mask(1);
    bf16x8 dsf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i0 = 8 * t;
      dsf[t] = cat(cvt4(s[0][i0], s[0][i0 + 1], s[0][i0 + 2], s[0][i0 + 3]),
                   cvt4(s[0][i0 + 4], s[0][i0 + 5], s[0][i0 + 6], s[0][i0 + 7]));
    }
    {
      // MFMA g: 16-key step g / NDB (steps 0, 1: block 0), d-block g % NDB
      constexpr int NDB = D / 32, NP = 2 * NDB, N = 4 * NDB, LEAD = 4;
      bf16x8 ring[LEAD];
#pragma unroll
      for (int g = 0; g < LEAD; ++g) ring[g] = tr_frag<ROW_B>(kt, tr, g / NDB, g % NDB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < N; ++g) {
        if (g == NP) {
#pragma unroll
          for (int t = 2; t < 4; ++t) {
            const int i0 = 8 * (t - 2);
            dsf[t] = cat(cvt4(s[1][i0], s[1][i0 + 1], s[1][i0 + 2], s[1][i0 + 3]),
                         cvt4(s[1][i0 + 4], s[1][i0 + 5], s[1][i0 + 6], s[1][i0 + 7]));
          }
        }
        const bf16x8 f = ring[g % LEAD];
        if (g + LEAD < N) ring[g % LEAD] = tr_frag<ROW_B>(kt, tr, (g + LEAD) / NDB, (g + LEAD) % NDB);
        dqa[g % NDB] = mfma32(f, dsf[g / NDB], dqa[g % NDB]);
        if (g < NP) ds(1, 16 * g / NP, 16 * (g + 1) / NP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (n_end > n_begin) {
    issue(n_begin * BN, 0);
    vmcnt_wait<0>();
    lds_barrier();
    for (int n = n_begin; n < n_end; ++n) {
      const int cur = (n - n_begin) & 1;
      // the other buffer's last readers finished before the previous barrier
      if (n + 1 < n_end) issue((n + 1) * BN, cur ^ 1);
      compute(n * BN, smem + cur * BUF_B);
      vmcnt_wait<0>();  // this wave's share of tile n+1 has landed
      lds_barrier();    // and every other wave's
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

// XCD-aware work order of the dK/dV grids. Consecutive workgroups go to the
// eight XCDs in turn, so workgroup L runs on XCD g = L % 8 as its slot
// s = L / 8 there. W items, numbered key block fastest (NB blocks), then
// (KV head, sequence, split): each XCD should hold whole (KV head,
// sequence) walks, whose workgroups read the same Q and dO rows and so
// share its L2, and an even share of the work. With P = W / 8 items per
// XCD:
//   - NB <= P: XCD g takes the contiguous items g*P .. g*P + P-1 (whole
//     walks of P / NB combinations);
//   - NB = q P with q dividing 8: the q XCDs g = c q .. c q + q-1 share
//     combination c, XCD c q + ph taking key blocks ph, ph + q, ...:
//     under a causal mask the walk length falls with the key block, and a
//     contiguous range of blocks per XCD would give the first XCD up to
//     seven times the work of another;
//   - otherwise (W not a multiple of 8, or no such q) the plain order.
__device__ __forceinline__ int64_t dkdv_item(int64_t L, int64_t W, int64_t NB) {
  if ((W & 7) != 0) return L;
  const int64_t P = W >> 3, g = L & 7, s = L >> 3;
  if (NB > P && NB % P == 0 && 8 % (NB / P) == 0) {
    const int64_t q = NB / P;
    return (g / q) * NB + s * q + (g % q);
  }
  if (NB > P) return L;
  return g * P + s;
}

// One workgroup per 128 keys of a KV head (32 per wave) and split: the walk
// over (query head of the group, 64-query tile) is cut into `splits`
// contiguous parts, one per workgroup; every wave reads the whole staged
// tile. With one split dK (scaled) and dV are written as bf16; otherwise
// each split writes float32 partials that bwd_dkv_reduce_kernel sums in
// split order.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int DL = bwd_width<D>();  // layout head dim
  constexpr int ROW_B = DL * 2, CPR = DL / 8;
  constexpr int BNK = kBwdBlockN, BM = kBwdTileM;
  static_assert(BNK == 128 && BM == 64, "four 32-key waves, 64-query tiles");
  constexpr int TILE_B = BM * ROW_B;
  // per buffer: Q tile, dO tile, then the tile's 64 LSE log2 e and 64 dPsum values
  constexpr int BUF_B = 2 * TILE_B + 2 * 256;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF_B];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, half = lane >> 5;
  const int S = a.splits;
  const int64_t NB = gridDim.x;
  const int64_t W = NB * gridDim.y * gridDim.z;
  const int64_t L = blockIdx.x + NB * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t w_item = dkdv_item(L, W, NB);
  const int nb = (int)(w_item % NB);
  const int64_t combo = w_item / NB;  // hk + hkv * (b * S + sp)
  const int hk = (int)(combo % gridDim.y);
  const int bs = (int)(combo / gridDim.y);
  const int b = bs / S, sp = bs - b * S;

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
  const int qlo = a.wr >= 0 ? max(0, kk - off - a.wr) : 0;
  const int qhi = kvalid ? (a.wl >= 0 ? min(sq - 1, kk - off + a.wl) : sq - 1) : qlo - 1;
  const int j1 = min(sk, j0 + BNK) - 1;
  const int i_lo = uniform(a.wr >= 0 ? max(0, j0 - off - a.wr) : 0);
  const int i_hi = uniform(a.wl >= 0 ? min(sq - 1, j1 - off + a.wl) : sq - 1);
  const int m_begin = i_lo / BM;
  const int nm = i_hi >= i_lo ? i_hi / BM - m_begin + 1 : 0;
  const int n_all = nm * r;
  const int it_begin = uniform((int)((int64_t)n_all * sp / S));
  const int it_end = uniform((int)((int64_t)n_all * (sp + 1) / S));

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

  // Q / dO tiles (and the tile's LSE log2 e and dPsum) go global -> LDS directly
  // (dma16), double-buffered. For each tensor, instruction i of wave w fills
  // tile rows RPI*(NI*w + i) .. +RPI-1; lane j lands at row offset j / CPR,
  // physical chunk j % CPR, so it loads logical chunk (j % CPR) ^ tswz(row).
  // Wave 0 loads the 64 LSE log2 e values, wave 1 the 64 dPsum values (one dword
  // per lane; rows past the sequence load zero).
  constexpr int RPI = 1024 / ROW_B;  // rows per instruction
  constexpr int NI = BM / RPI / 4;   // instructions per wave per tensor
  static_assert(NI * RPI * 4 == BM, "a tile splits evenly over four waves");
  uint32_t qdo[NI], gdo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (NI * wave + i) + lane / CPR;
    qdo[i] = (uint32_t)(row * a.q_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
    gdo[i] = (uint32_t)(row * a.do_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
  }
  const uint32_t lds_w = (uint32_t)uniform((int)(lds_addr(smem) + NI * wave * 1024));
  const uint32_t lds_s = (uint32_t)uniform((int)(lds_addr(smem) + 2 * TILE_B + (wave & 1) * 256));
  // iteration it: query head hk*r + it / nm, query tile m_begin + it % nm
  auto issue = [&](int it, int buf) __attribute__((always_inline)) {
    const int h = uniform(hk * r + it / nm);
    const int m0 = uniform((m_begin + it % nm) * BM);
    const int nrows = min(sq - m0, BM);  // >= 1; rows past it read as zero
    const __bf16* q0 = static_cast<const __bf16*>(a.q) + q_base + (int64_t)m0 * a.q_rs +
                       (int64_t)h * a.q_hs;
    const __bf16* g0 = static_cast<const __bf16*>(a.dout) + do_base + (int64_t)m0 * a.do_rs +
                       (int64_t)h * a.do_hs;
    const auto qr = make_rsrc(q0, (uint32_t)((nrows - 1) * a.q_rs * 2 + D * 2));
    const auto gr = make_rsrc(g0, (uint32_t)((nrows - 1) * a.do_rs * 2 + D * 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(qr, qdo[i], lds_w + (uint32_t)(buf * BUF_B + i * 1024));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(gr, gdo[i], lds_w + (uint32_t)(buf * BUF_B + TILE_B + i * 1024));
    if (wave < 2) {  // wave-uniform
      const int64_t li = a.cu_q != nullptr ? (int64_t)h * a.total_q + q_tok0 + m0
                                           : ((int64_t)b * a.hq + h) * sq + m0;
      const auto sr =
          make_rsrc(wave == 0 ? a.lse_log2 + li : a.dpsum + li, (uint32_t)(nrows * 4));
      dma4(sr, (uint32_t)(4 * lane), lds_s + (uint32_t)(buf * BUF_B));
    }
  };

  int rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ tswz<DL>(c32)) * 16);
  int tr[2];
  tr_offsets(lane, ROW_B, tr);

  // One step, software-pipelined over the two 32-query blocks qb of the
  // tile so that each block's exponentials run between matrix instructions
  // of the other block (a wave's VALU work proceeds while its earlier MFMAs
  // execute):
  //   part 1: S, dP of block 0 (MFMAs 0..NS-1), then S, dP of block 1, one
  //           block-0 softmax slice after each of those MFMAs
  //   part 2: dV, dK of block 0, one block-1 softmax slice after each of
  //           the first NP MFMAs; then dV, dK of block 1
  auto compute = [&](int m0, const char* qt) __attribute__((always_inline)) {
    const char* gt = qt + TILE_B;
    const float* l2s = reinterpret_cast<const float*>(qt + 2 * TILE_B);  // LSE log2 e
    const float* dss = l2s + BM;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = zero_f32x16();
      dp[qb] = zero_f32x16();
    }
    // element (qb, v) holds query m0 + 4*half + 32*qb + 8*(v>>2) + (v&3), key `key`
    const uint64_t vis = vis64(qlo - m0 - 4 * half, qhi - m0 - 4 * half);
    // row statistics of query block qb, read from LDS a few matrix
    // instructions before the block's softmax slices need them (so they are
    // not live through the other block's work)
    f32x4 l4[2][4], d4[2][4];
    auto load_stats = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qo = 32 * qb + 8 * i + 4 * half;
        // LSE log2 e (+inf for a row with no visible key, so P = 0; rows
        // past the sequence read 0 and are masked)
        l4[qb][i] = *reinterpret_cast<const f32x4*>(l2s + qo);
        d4[qb][i] = *reinterpret_cast<const f32x4*>(dss + qo);
      }
    };
    // the mask runs only on tiles where some lane of the wave has a query
    // outside its visible range (edge tiles; a wave-uniform branch)
    const bool edge = __builtin_amdgcn_ballot_w64(vis != ~0ull) != 0;
    auto mask = [&](int qb) __attribute__((always_inline)) {
      if (edge) {
        const uint32_t w = (uint32_t)(vis >> (32 * qb));
#pragma unroll
        for (int v = 0; v < 16; ++v) s[qb][v] = mask_by_bit(s[qb][v], w, 8 * (v >> 2) + (v & 3));
      }
    };
    // softmax elements [e0, e1) of block qb: P, then dS in place of dP
    auto sm = [&](int qb, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
      for (int v = e0; v < e1; ++v) {
        const float p = fast_exp2(fmaf(s[qb][v], c, -l4[qb][v >> 2][v & 3]));
        s[qb][v] = p;
        dp[qb][v] = p * (dp[qb][v] - d4[qb][v >> 2][v & 3]);
      }
    };
    {
      // MFMA g: block g / NS, i = g % NS: contraction step i / 2; even i: S
      // from Q rows, odd i: dP from dO rows
      constexpr int NS = 2 * (D / 16), N = 2 * NS, LEAD = 6;
      auto rdf = [&](int g) __attribute__((always_inline)) {
        const int qb = g / NS, i = g % NS;
        return *reinterpret_cast<const bf16x8*>((i & 1 ? gt : qt) + qb * 32 * ROW_B + rd[i >> 1]);
      };
      bf16x8 ring[LEAD];
#pragma unroll
      for (int g = 0; g < LEAD; ++g) ring[g] = rdf(g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < N; ++g) {
        const bf16x8 f = ring[g % LEAD];
        if (g + LEAD < N) ring[g % LEAD] = rdf(g + LEAD);
        const int qb = g / NS, i = g % NS;
        if (i & 1)
          dp[qb] = mfma32(f, vf[i >> 1], dp[qb]);
        else
          s[qb] = mfma32(f, kf[i >> 1], s[qb]);
        if (g == NS - 4) load_stats(0);
        if (g == N - 4) load_stats(1);
        if (qb == 1) {
          if (i == 0) mask(0);
          sm(0, 16 * i / NS, 16 * (i + 1) / NS);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mask(1);
    bf16x8 pf[4], dsf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i0 = 8 * t;
      pf[t] = cat(cvt4(s[0][i0], s[0][i0 + 1], s[0][i0 + 2], s[0][i0 + 3]),
                  cvt4(s[0][i0 + 4], s[0][i0 + 5], s[0][i0 + 6], s[0][i0 + 7]));
      dsf[t] = cat(cvt4(dp[0][i0], dp[0][i0 + 1], dp[0][i0 + 2], dp[0][i0 + 3]),
                   cvt4(dp[0][i0 + 4], dp[0][i0 + 5], dp[0][i0 + 6], dp[0][i0 + 7]));
    }
    {
      // MFMA g: fragment t = g / (2 NDB) (t < 2: block 0, else block 1),
      // d-block (g / 2) % NDB; even g: dV from dO^T, odd g: dK from Q^T
      constexpr int NDB = D / 32, NP = 4 * NDB, N = 2 * NP, LEAD = 4;
      auto rdf = [&](int g) __attribute__((always_inline)) {
        return tr_frag<ROW_B>(g & 1 ? qt : gt, tr, g / (2 * NDB), (g >> 1) % NDB);
      };
      bf16x8 ring[LEAD];
#pragma unroll
      for (int g = 0; g < LEAD; ++g) ring[g] = rdf(g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < N; ++g) {
        if (g == NP) {
#pragma unroll
          for (int t = 2; t < 4; ++t) {
            const int i0 = 8 * (t - 2);
            pf[t] = cat(cvt4(s[1][i0], s[1][i0 + 1], s[1][i0 + 2], s[1][i0 + 3]),
                        cvt4(s[1][i0 + 4], s[1][i0 + 5], s[1][i0 + 6], s[1][i0 + 7]));
            dsf[t] = cat(cvt4(dp[1][i0], dp[1][i0 + 1], dp[1][i0 + 2], dp[1][i0 + 3]),
                         cvt4(dp[1][i0 + 4], dp[1][i0 + 5], dp[1][i0 + 6], dp[1][i0 + 7]));
          }
        }
        const bf16x8 f = ring[g % LEAD];
        if (g + LEAD < N) ring[g % LEAD] = rdf(g + LEAD);
        const int t = g / (2 * NDB), db = (g >> 1) % NDB;
        if (g & 1)
          dka[db] = mfma32(f, dsf[t], dka[db]);
        else
          dva[db] = mfma32(f, pf[t], dva[db]);
        if (g < NP) sm(1, 16 * g / NP, 16 * (g + 1) / NP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (it_end > it_begin) {
    issue(it_begin, 0);
    vmcnt_wait<0>();
    lds_barrier();
    for (int it = it_begin; it < it_end; ++it) {
      const int cur = (it - it_begin) & 1;
      const int m0 = uniform((m_begin + it % nm) * BM);
      // the other buffer's last readers finished before the previous barrier
      if (it + 1 < it_end) issue(it + 1, cur ^ 1);
      compute(m0, smem + cur * BUF_B);
      vmcnt_wait<0>();  // this wave's share of the next tile has landed
      lds_barrier();    // and every other wave's
    }
  }

  if (!kvalid) return;
  if (S == 1) {
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
  } else if (key < a.seqlen_k) {
    // partial row (split, sequence, key, KV head): dK then dV, D floats each.
    // The partial buffer holds seqlen_k (the caller's max_seqlen_k) keys per
    // sequence; keys of a longer sequence (an understated maximum) are not
    // written anywhere.
    float* pp = a.dkv_part +
                ((((int64_t)sp * a.batch + b) * a.seqlen_k + key) * a.hkv + hk) * (2 * D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<f32x4*>(pp + d0) =
            f32x4{dka[db][4 * i], dka[db][4 * i + 1], dka[db][4 * i + 2], dka[db][4 * i + 3]};
        *reinterpret_cast<f32x4*>(pp + D + d0) =
            f32x4{dva[db][4 * i], dva[db][4 * i + 1], dva[db][4 * i + 2], dva[db][4 * i + 3]};
      }
  }
}

// ----------------------------------------------------- dK dV, paired waves ----

// The dK/dV walk for head_dim 256 (and 192, in its layout). Holding the
// lane's K and V fragments and
// both 32 x 256 accumulators (dK^T, dV^T) takes ~540 registers, past the
// 512 a wave can have, so each 32-key column is served by a pair of waves
// that split the four products without repeating any:
//   wave A (even): S = Q K^T, P = exp2(S c - LSE log2e), dV^T += dO^T P
//   wave B (odd):  dP = dO V^T, dS = P (dP - dPsum), dK^T += Q^T dS
// A hands P of the first 32 queries and the raw scores of the other 32
// (float32) to B through LDS; B recomputes P of the latter.
// Each wave holds one key fragment set (K or V, 64 registers) and one
// accumulator (128). One workgroup = two pairs = 64 keys; the Q / dO tile
// staging, the split of the walk and the XCD-aware order are those of
// bwd_dkdv_kernel.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_pair_kernel(const BwdArgs a) {
  constexpr int DL = bwd_width<D>();  // layout head dim
  constexpr int ROW_B = DL * 2, CPR = DL / 8;
  constexpr int BNK = kBwdBlockNPair, BM = kBwdTileM;
  static_assert(BNK == 64 && BM == 64, "two 32-key wave pairs, 64-query tiles");
  constexpr int TILE_B = BM * ROW_B;
  // per buffer: Q tile, dO tile, then the tile's 64 LSE log2 e and 64 dPsum values
  constexpr int BUF_B = 2 * TILE_B + 2 * 256;
  constexpr int PX_B = 64 * 32 * 4;  // one pair's P: 32 floats per lane
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF_B + 2 * PX_B];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, half = lane >> 5;
  const int role = wave & 1, pair = wave >> 1;  // role 0: A, 1: B
  const int S = a.splits;
  const int64_t NB = gridDim.x;
  const int64_t W = NB * gridDim.y * gridDim.z;
  const int64_t L = blockIdx.x + NB * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t w_item = dkdv_item(L, W, NB);
  const int nb = (int)(w_item % NB);
  const int64_t combo = w_item / NB;  // hk + hkv * (b * S + sp)
  const int hk = (int)(combo % gridDim.y);
  const int bs = (int)(combo / gridDim.y);
  const int b = bs / S, sp = bs - b * S;

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

  const int key = j0 + pair * 32 + c32;
  const bool kvalid = key < sk;
  const int kk = kvalid ? key : 0;
  const int r = a.group;
  const int off = sk - sq;
  // queries that see key j: j - off - wr <= i <= j - off + wl, 0 <= i < sq
  const int qlo = a.wr >= 0 ? max(0, kk - off - a.wr) : 0;
  const int qhi = kvalid ? (a.wl >= 0 ? min(sq - 1, kk - off + a.wl) : sq - 1) : qlo - 1;
  const int j1 = min(sk, j0 + BNK) - 1;
  const int i_lo = uniform(a.wr >= 0 ? max(0, j0 - off - a.wr) : 0);
  const int i_hi = uniform(a.wl >= 0 ? min(sq - 1, j1 - off + a.wl) : sq - 1);
  const int m_begin = i_lo / BM;
  const int nm = i_hi >= i_lo ? i_hi / BM - m_begin + 1 : 0;
  const int n_all = nm * r;
  const int it_begin = uniform((int)((int64_t)n_all * sp / S));
  const int it_end = uniform((int)((int64_t)n_all * (sp + 1) / S));

  // this lane's key: K^T (wave A) or V^T (wave B) fragments, the B operands
  // of S and dP
  const __bf16* kvp =
      role == 0 ? static_cast<const __bf16*>(a.k) + k_base + (int64_t)kk * a.k_rs +
                      (int64_t)hk * a.k_hs
                : static_cast<const __bf16*>(a.v) + v_base + (int64_t)kk * a.v_rs +
                      (int64_t)hk * a.v_hs;
  bf16x8 mf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    const bf16x8 x = as_bf16x8(ld16(kvp + 16 * cc + 8 * half));
    mf[cc] = kvalid ? x : zero_bf16x8();
  }
  const float c = a.scale_log2;

  f32x16 acc[D / 32];  // A: dV^T, B: dK^T (unscaled)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero_f32x16();

  // Q / dO tile staging as in bwd_dkdv_kernel: instruction i of wave w
  // fills tile rows RPI*(NI*w + i) .. +RPI-1; wave 0 loads the 64 LSE log2 e
  // values, wave 1 the 64 dPsum values.
  constexpr int RPI = 1024 / ROW_B;  // rows per instruction
  constexpr int NI = BM / RPI / 4;   // instructions per wave per tensor
  static_assert(NI * RPI * 4 == BM, "a tile splits evenly over four waves");
  uint32_t qdo[NI], gdo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (NI * wave + i) + lane / CPR;
    qdo[i] = (uint32_t)(row * a.q_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
    gdo[i] = (uint32_t)(row * a.do_rs * 2 + ((lane % CPR) ^ tswz<DL>(row)) * 16);
  }
  const uint32_t lds_w = (uint32_t)uniform((int)(lds_addr(smem) + NI * wave * 1024));
  const uint32_t lds_s = (uint32_t)uniform((int)(lds_addr(smem) + 2 * TILE_B + (wave & 1) * 256));
  // iteration it: query head hk*r + it / nm, query tile m_begin + it % nm
  auto issue = [&](int it, int buf) __attribute__((always_inline)) {
    const int h = uniform(hk * r + it / nm);
    const int m0 = uniform((m_begin + it % nm) * BM);
    const int nrows = min(sq - m0, BM);  // >= 1; rows past it read as zero
    const __bf16* q0 = static_cast<const __bf16*>(a.q) + q_base + (int64_t)m0 * a.q_rs +
                       (int64_t)h * a.q_hs;
    const __bf16* g0 = static_cast<const __bf16*>(a.dout) + do_base + (int64_t)m0 * a.do_rs +
                       (int64_t)h * a.do_hs;
    const auto qr = make_rsrc(q0, (uint32_t)((nrows - 1) * a.q_rs * 2 + D * 2));
    const auto gr = make_rsrc(g0, (uint32_t)((nrows - 1) * a.do_rs * 2 + D * 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(qr, qdo[i], lds_w + (uint32_t)(buf * BUF_B + i * 1024));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(gr, gdo[i], lds_w + (uint32_t)(buf * BUF_B + TILE_B + i * 1024));
    if (wave < 2) {  // wave-uniform
      const int64_t li = a.cu_q != nullptr ? (int64_t)h * a.total_q + q_tok0 + m0
                                           : ((int64_t)b * a.hq + h) * sq + m0;
      const auto sr =
          make_rsrc(wave == 0 ? a.lse_log2 + li : a.dpsum + li, (uint32_t)(nrows * 4));
      dma4(sr, (uint32_t)(4 * lane), lds_s + (uint32_t)(buf * BUF_B));
    }
  };

  int rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ tswz<DL>(c32)) * 16);
  int tr[2];
  tr_offsets(lane, ROW_B, tr);
  // this pair's P exchange: chunk i (4 floats) of lane l at 1024 i + 16 l
  char* px = smem + 2 * BUF_B + pair * PX_B + 16 * lane;

  // the S (A) or dP (B) products of both 32-query blocks, reading
  // Q (A) or dO (B) rows; MFMA g: block g / NK, contraction step g % NK
  auto rows_products = [&](const char* t, f32x16 x[2], auto&& between)
      __attribute__((always_inline)) {
    constexpr int NK = D / 16, N = 2 * NK, LEAD = 6;
    auto rdf = [&](int g) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(t + (g / NK) * 32 * ROW_B + rd[g % NK]);
    };
    bf16x8 ring[LEAD];
#pragma unroll
    for (int g = 0; g < LEAD; ++g) ring[g] = rdf(g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < N; ++g) {
      const bf16x8 f = ring[g % LEAD];
      if (g + LEAD < N) ring[g % LEAD] = rdf(g + LEAD);
      x[g / NK] = mfma32(f, mf[g % NK], x[g / NK]);
      between(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc^T += T^T F over the 32 queries of block qb, T read by transposing
  // reads; MFMA g: 16-query step 2 qb + g / NDB, d-block g % NDB
  auto trans_products = [&](const char* t, int qb, const bf16x8 fr[2], auto&& between)
      __attribute__((always_inline)) {
    constexpr int NDB = D / 32, N = 2 * NDB, LEAD = 4;
    bf16x8 ring[LEAD];
#pragma unroll
    for (int g = 0; g < LEAD; ++g) ring[g] = tr_frag<ROW_B>(t, tr, 2 * qb + g / NDB, g % NDB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < N; ++g) {
      const bf16x8 f = ring[g % LEAD];
      if (g + LEAD < N)
        ring[g % LEAD] = tr_frag<ROW_B>(t, tr, 2 * qb + (g + LEAD) / NDB, (g + LEAD) % NDB);
      acc[g % NDB] = mfma32(f, fr[g / NDB], acc[g % NDB]);
      between(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto to_frags = [&](const f32x16& x, bf16x8 f[2]) __attribute__((always_inline)) {
    f[0] = cat(cvt4(x[0], x[1], x[2], x[3]), cvt4(x[4], x[5], x[6], x[7]));
    f[1] = cat(cvt4(x[8], x[9], x[10], x[11]), cvt4(x[12], x[13], x[14], x[15]));
  };

  // One step over a 64-query tile, in two parts around a workgroup barrier
  // (the pairs run the same schedule):
  //   A: S of blocks 0, 1, block 0's P between block 1's MFMAs; out: P of
  //      block 0 and the raw scores of block 1
  //   B: dP of blocks 0, 1
  //   -- barrier
  //   A: dV from block 0 with block 1's P between its MFMAs, dV from block 1
  //   B: dS of block 0 (its second half between the first MFMAs), dK from
  //      block 0 with block 1's P and dS between its MFMAs, dK from block 1
  // B recomputing block 1's P keeps the exponentials off the part before
  // the barrier, which the MFMAs of both waves then fill evenly.
  // Element (qb, v) of a score accumulator holds query
  // m0 + 4*half + 32*qb + 8*(v>>2) + (v&3), key `key`. A tile that every
  // lane sees whole (most of a causal walk) skips the mask; both waves of a
  // pair hold the same keys and so take the same branch.
  auto step = [&](int m0, const char* qt) __attribute__((always_inline)) {
    const char* gt = qt + TILE_B;
    const float* lses = reinterpret_cast<const float*>(qt + 2 * TILE_B);  // LSE log2 e
    const float* dss = lses + BM;
    constexpr int NK = D / 16, NDB = D / 32;
    f32x16 x[2];
    x[0] = zero_f32x16();
    x[1] = zero_f32x16();
    bf16x8 fr[2][2];
    const uint64_t vis = vis64(qlo - m0 - 4 * half, qhi - m0 - 4 * half);
    // +inf for a row with no visible key, so P = 0; rows past the sequence
    // read 0 and are masked
    auto lse4 = [&](int qb, int i) __attribute__((always_inline)) {
      return *reinterpret_cast<const f32x4*>(lses + 32 * qb + 8 * i + 4 * half);
    };
    auto path = [&](auto wm) __attribute__((always_inline)) {
      // P of score s, element v of block qb
      auto prob = [&](float sv, int qb, int v, float l) __attribute__((always_inline)) {
        if constexpr (decltype(wm)::value)
          sv = mask_by_bit(sv, (uint32_t)(vis >> (32 * qb)), 8 * (v >> 2) + (v & 3));
        return fast_exp2(fmaf(sv, c, -l));
      };
      if (role == 0) {
        f32x4 l4[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) l4[qb][i] = lse4(qb, i);
        auto sm = [&](int qb, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
          for (int v = e0; v < e1; ++v) x[qb][v] = prob(x[qb][v], qb, v, l4[qb][v >> 2][v & 3]);
        };
        rows_products(qt, x, [&](int g) __attribute__((always_inline)) {
          if (g >= NK) sm(0, 16 * (g - NK) / NK, 16 * (g - NK + 1) / NK);
        });
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x16& xs = x[i >> 2];
          *reinterpret_cast<f32x4*>(px + 1024 * i) =
              f32x4{xs[4 * (i & 3)], xs[4 * (i & 3) + 1], xs[4 * (i & 3) + 2], xs[4 * (i & 3) + 3]};
        }
        to_frags(x[0], fr[0]);
        lds_barrier();  // P0 and S1 are in LDS
        trans_products(gt, 0, fr[0], [&](int g) __attribute__((always_inline)) {
          sm(1, 16 * g / (2 * NDB), 16 * (g + 1) / (2 * NDB));
        });
        to_frags(x[1], fr[1]);
        trans_products(gt, 1, fr[1], [](int) __attribute__((always_inline)) {});
      } else {
        f32x4 d4[2][4], l4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d4[0][i] = *reinterpret_cast<const f32x4*>(dss + 8 * i + 4 * half);
          d4[1][i] = *reinterpret_cast<const f32x4*>(dss + 32 + 8 * i + 4 * half);
          l4[i] = lse4(1, i);
        }
        rows_products(gt, x, [](int) __attribute__((always_inline)) {});
        lds_barrier();  // P0 and S1 are in LDS
        f32x4 pv[4], sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = *reinterpret_cast<const f32x4*>(px + 1024 * i);
          sv[i] = *reinterpret_cast<const f32x4*>(px + 1024 * (4 + i));
        }
        // dS = P (dP - dPsum), in place of dP
        auto ds0 = [&](int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
          for (int v = e0; v < e1; ++v)
            x[0][v] = pv[v >> 2][v & 3] * (x[0][v] - d4[0][v >> 2][v & 3]);
        };
        auto ds1 = [&](int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
          for (int v = e0; v < e1; ++v)
            x[1][v] = prob(sv[v >> 2][v & 3], 1, v, l4[v >> 2][v & 3]) *
                      (x[1][v] - d4[1][v >> 2][v & 3]);
        };
        ds0(0, 8);
        fr[0][0] = cat(cvt4(x[0][0], x[0][1], x[0][2], x[0][3]),
                       cvt4(x[0][4], x[0][5], x[0][6], x[0][7]));
        trans_products(qt, 0, fr[0], [&](int g) __attribute__((always_inline)) {
          if (g < NDB) {
            ds0(8 + 8 * g / NDB, 8 + 8 * (g + 1) / NDB);
            if (g == NDB - 1)
              fr[0][1] = cat(cvt4(x[0][8], x[0][9], x[0][10], x[0][11]),
                             cvt4(x[0][12], x[0][13], x[0][14], x[0][15]));
          } else {
            ds1(16 * (g - NDB) / NDB, 16 * (g - NDB + 1) / NDB);
          }
        });
        to_frags(x[1], fr[1]);
        trans_products(qt, 1, fr[1], [](int) __attribute__((always_inline)) {});
      }
    };
    if (__builtin_amdgcn_ballot_w64(vis != ~0ull) != 0)
      path(std::true_type{});
    else
      path(std::false_type{});
  };

  if (it_end > it_begin) {
    issue(it_begin, 0);
    vmcnt_wait<0>();
    lds_barrier();
    for (int it = it_begin; it < it_end; ++it) {
      const int cur = (it - it_begin) & 1;
      const int m0 = uniform((m_begin + it % nm) * BM);
      // the other buffer's last readers finished before the previous barrier
      if (it + 1 < it_end) issue(it + 1, cur ^ 1);
      step(m0, smem + cur * BUF_B);
      vmcnt_wait<0>();  // this wave's share of the next tile has landed
      lds_barrier();    // and every other wave's; B is done with this P
    }
  }

  if (!kvalid) return;
  if (S == 1) {
    __bf16* dst = role == 0 ? static_cast<__bf16*>(a.dv) + dv_base + (int64_t)key * a.dv_rs +
                                  (int64_t)hk * a.dv_hs
                            : static_cast<__bf16*>(a.dk) + dk_base + (int64_t)key * a.dk_rs +
                                  (int64_t)hk * a.dk_hs;
    const float sc = role == 0 ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<bf16x4*>(dst + d0) =
            cvt4(acc[db][4 * i] * sc, acc[db][4 * i + 1] * sc, acc[db][4 * i + 2] * sc,
                 acc[db][4 * i + 3] * sc);
      }
  } else if (key < a.seqlen_k) {
    // partial row (split, sequence, key, KV head): dK then dV, D floats each
    // (keys past the caller's max_seqlen_k are not written anywhere)
    float* pp = a.dkv_part +
                ((((int64_t)sp * a.batch + b) * a.seqlen_k + key) * a.hkv + hk) * (2 * D) +
                (role == 0 ? D : 0);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<f32x4*>(pp + d0) =
            f32x4{acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]};
      }
  }
}

// Sums the splits' float32 partials in split order (deterministic), scales
// dK, and writes dK and dV as bf16. One thread per 4 floats of a partial row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(const BwdArgs a) {
  constexpr int CH = D / 2;  // float4 chunks per partial row (dK then dV)
  const int64_t rows = (int64_t)a.batch * a.seqlen_k * a.hkv;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * CH) return;
  const int64_t row = e / CH;
  const int cidx = (int)(e - row * CH);
  const int hk = (int)(row % a.hkv);
  const int64_t bk = row / a.hkv;
  const int key = (int)(bk % a.seqlen_k);
  const int b = (int)(bk / a.seqlen_k);
  int sk = a.seqlen_k;
  int64_t kb;
  const bool is_v = cidx >= CH / 2;
  const int d0 = 4 * (cidx - (is_v ? CH / 2 : 0));
  if (a.cu_k != nullptr) {
    sk = a.cu_k[b + 1] - a.cu_k[b];
    kb = (int64_t)(a.cu_k[b] + key) * (is_v ? a.dv_rs : a.dk_rs);
  } else {
    kb = (int64_t)b * (is_v ? a.dv_bs : a.dk_bs) + (int64_t)key * (is_v ? a.dv_rs : a.dk_rs);
  }
  if (key >= sk) return;
  const int64_t stride = (int64_t)a.batch * a.seqlen_k * a.hkv * (2 * D);
  const float* src = a.dkv_part + row * (2 * D) + (is_v ? D : 0) + d0;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int s = 1; s < a.splits; ++s) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + s * stride);
    acc += x;
  }
  const float sc = is_v ? 1.0f : a.scale;
  __bf16* dst = static_cast<__bf16*>(is_v ? a.dv : a.dk) + kb +
                (int64_t)hk * (is_v ? a.dv_hs : a.dk_hs) + d0;
  *reinterpret_cast<bf16x4*>(dst) = cvt4(acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc);
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  const int64_t ntok = a.cu_q != nullptr ? (int64_t)a.total_q : (int64_t)a.batch * a.seqlen_q;
  const int64_t pre_rows = ntok * a.hq;
  constexpr int DL = bwd_width<D>();
  if (pre_rows > 0) {
    const int64_t rpb = 256 / (DL / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((pre_rows + rpb - 1) / rpb)),
                       dim3(256), 0, s, a);
  }
  const int64_t mblocks = ((int64_t)a.seqlen_q * a.group + kBwdBlockM - 1) / kBwdBlockM;
  if (mblocks > 0 && a.batch > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)mblocks, a.hkv, a.batch), dim3(256), 0,
                       s, a);
  constexpr int BN = DL == 256 ? kBwdBlockNPair : kBwdBlockN;
  const int64_t nblocks = ((int64_t)a.seqlen_k + BN - 1) / BN;
  if (nblocks > 0 && a.batch > 0) {
    if constexpr (DL == 256)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D>),
                         dim3((unsigned)nblocks, a.hkv, a.batch * a.splits), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)nblocks, a.hkv, a.batch * a.splits),
                         dim3(256), 0, s, a);
    if (a.splits > 1) {
      const int64_t chunks = (int64_t)a.batch * a.seqlen_k * a.hkv * (D / 2);
      hipLaunchKernelGGL((bwd_dkv_reduce_kernel<D>), dim3((unsigned)((chunks + 255) / 256)),
                         dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

template hipError_t launch_bwd<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd<96>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd<192>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd<256>(const BwdArgs&, hipStream_t);

}  // namespace mi_attn
