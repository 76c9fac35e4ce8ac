// Prefill forward for head_dim 64/128: eight waves in two ping-pong groups.
//
// Same method as launch_fwd in kernels.hpp (mslk flash_attn interface.py page,
// `_flash_attn_fwd`: exact attention with online softmax in the exp2 domain
// and a natural-log LSE; lazily updated running max). What differs is the
// schedule. A workgroup owns 256 packed query rows: group A = waves 0-3
// (rows 0-127), group B = waves 4-7 (rows 128-255). Wave w and wave w+4
// share SIMD w, and the two groups run the same per-tile work offset by half
// a tile:
//
//   iteration k, group A: MFMA item k, then softmax of tile k
//   iteration k, group B: softmax of tile k-1, then MFMA item k
//   MFMA item k = O += P(k-1) V(k-1)  and  S(k) = K(k) Q^T   (32 MFMAs)
//
// so on every SIMD one wave keeps the matrix cores busy while the other runs
// its exponentials. One workgroup barrier per iteration (the tile hand-over
// below) is the only synchronisation: inside an iteration the two phases of a
// SIMD's waves float against each other, the matrix wave at raised priority.
// (A second barrier between the phases, forcing them into lock step, cost
// 3.5% on the causal S4096 D128 workload.)
//
// K/V tiles (64 keys) rotate through four LDS buffers and go there straight
// from global memory (direct-to-LDS buffer loads, nothing staged in
// registers). Tile k is read in iterations k and k+1; tile k+2 is requested
// during iteration k into the buffer tile k-2 vacated (each group issues its
// share spread over the S MFMAs of its matrix phase), and an explicit
// load-count wait plus a barrier at the end of iteration k make tile k+1
// visible. Every request is issued unconditionally (tiles past the end get
// zero-length descriptors and load nothing), which keeps the wait counts
// static.
#include <climits>
#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

// Head dim 96 uses the head-dim-128 LDS layout (rows of 256 bytes): tiles
// load whole 256-byte row slots (the last 64 bytes of a row slot hold the
// next row's first values, or zeros past the end of the tensor) and every
// product reads only the first 96 columns.
template <int D>
struct PPCfg {
  static constexpr int DL = D == 96 ? 128 : D;  // layout head dim
  static constexpr int BM = kFwdPPBlockM;      // 256 packed rows
  static constexpr int BN = kFwdBlockN;        // 64 keys
  static constexpr int NT = 512;               // 8 waves
  static constexpr int CPR = DL / 8;           // 16-byte chunks per LDS row
  static constexpr int TILE_B = BN * DL * 2;   // bytes per K (or V) tile
  static constexpr int NBUF = 4;
  static constexpr float RESCALE_LOG2 = 8.0f;
  static_assert(BN == 64 && (CPR == 8 || CPR == 16), "staging assumes 64-key tiles, D 64/128");
};

template <int D, bool PAGED, bool SC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pp_kernel(const FwdArgs a) {
  using C = PPCfg<D>;
  constexpr int BM = C::BM, BN = C::BN, CPR = C::CPR;
  constexpr int TILE_B = C::TILE_B;
  constexpr int ROW_B = C::DL * 2;  // LDS row bytes
  constexpr int BUF_B = 2 * TILE_B;  // K then V
  __shared__ __attribute__((aligned(16))) char smem[C::NBUF * BUF_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int wig = wave & 3;   // wave in group
  const int c32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item (heavy query blocks first; see fwd_work_item)
  int hk, b, mb;
  FwdSeq seq;
  if (!fwd_work_item<BM>(a, hk, b, mb, seq)) return;

  int sq = a.seqlen_q, sk = a.seqlen_k;
  int64_t q_base, k_base, v_base, o_base;
  int q_tok0 = 0;
  if (a.cu_q != nullptr) {
    q_tok0 = seq.q0;
    sq = seq.q1 - seq.q0;
    q_base = (int64_t)q_tok0 * a.q_rs;
    o_base = (int64_t)q_tok0 * a.o_rs;
  } else {
    q_base = (int64_t)b * a.q_bs;
    o_base = (int64_t)b * a.o_bs;
  }
  fwd_kv_extent<PAGED>(a, b, seq, sk, k_base, v_base);
  sq = uniform(sq);
  sk = uniform(sk);
  const int r = a.group;
  const int rows = sq * r;
  const int row0 = mb * BM;
  if (row0 >= rows) return;  // uniform over the workgroup

  // ---- this lane's query row
  const int prow = row0 + grp * 128 + wig * 32 + c32;
  const bool valid = prow < rows;
  const int pos = valid ? prow / r : 0;
  const int hq = hk * r + (valid ? prow - (prow / r) * r : 0);

  const int off = sk - sq;  // bottom-right alignment
  const int lo = a.wl >= 0 ? pos + off - a.wl : INT_MIN / 2;
  const int hi = min(a.wr >= 0 ? pos + off + a.wr : INT_MAX / 2, sk - 1);

  // workgroup-wide visible key range (both groups walk the same tiles)
  const int pos_min = uniform(row0 / r);
  const int pos_max = uniform((min(row0 + BM, rows) - 1) / r);
  const int kv_lo = a.wl >= 0 ? max(0, pos_min + off - a.wl) : 0;
  const int kv_hi = a.wr >= 0 ? min(sk, pos_max + off + a.wr + 1) : sk;  // exclusive
  const int n_begin = uniform(kv_lo / BN);
  const int n_end = uniform(kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : n_begin);
  int T = n_end - n_begin;
  // a paged cache with a page id outside [0, num_pages) in this range: no
  // tile is read and every row of the workgroup gets NaN
  const bool poison = fwd_bad_pages<PAGED>(a, b, n_begin * BN, min(sk, n_end * BN), lane);
  if (poison) T = 0;
  // per-group "tile fully visible" bounds (group rows [g0, g1))
  const int g0 = min(row0 + grp * 128, rows - 1);
  const int g1 = min(row0 + grp * 128 + 128, rows) - 1;
  const int gpos_min = uniform(g0 / r);
  const int gpos_max = uniform(max(g0, g1) / r);
  const int full_hi = a.wr >= 0 ? gpos_min + off + a.wr : INT_MAX / 2;
  const int full_lo = a.wl >= 0 ? gpos_max + off - a.wl : INT_MIN / 2;

  // ---- Q^T fragments (B operand). Branch-free: invalid lanes read row 0 of
  // head hk*r and zero it (a load under a divergent branch makes later waits
  // drain every outstanding load).
  const __bf16* qp = static_cast<const __bf16*>(a.q) + q_base + (int64_t)pos * a.q_rs +
                     (int64_t)hq * a.q_hs;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const bf16x8 x = as_bf16x8(ld16(qp + 16 * c + 8 * half));
    qf[c] = valid ? x : zero_bf16x8();
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.0f;

  // ---- K/V tiles go global -> LDS directly (dma16), 1 KB per wave
  // instruction, nothing staged in registers. For each tensor, instruction i
  // of wave w fills LDS rows RPI*(NI*w + i) .. +RPI-1: lane j lands at row
  // offset j / CPR, physical chunk j % CPR, so it loads the logical chunk
  // (j % CPR) ^ swizzle(row) of that row.
  // K has its own swizzle, conflict-free for the 16-byte fragment reads (the
  // 16 lanes an LDS cycle serves read one logical chunk of 16 consecutive
  // keys): D = 128 (16 chunks per 256-byte row): kswz(key) = swz_key(key)
  // with bit 3 = key bit 3, covering all 16 positions; D = 64 (two 128-byte
  // rows per bank window): kswz(key) = (key >> 1) & 7. V keeps swz_key for
  // its transposing reads.
  constexpr int RPI = 1024 / ROW_B;  // rows per DMA instruction
  constexpr int NI = BN / RPI / 8;   // DMA instructions per wave per tensor
  static_assert(NI * RPI * 8 == BN, "a tile splits evenly over eight waves");
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  auto kswz = [](int key) {
    return C::DL == 128 ? (swz_key(key) | (((key >> 3) & 1) << 3)) : ((key >> 1) & 7);
  };
  uint32_t kdo[NI], vdo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (NI * wave + i) + lane / CPR;
    kdo[i] = (uint32_t)(row * a.k_rs * 2 + ((lane % CPR) ^ kswz(row)) * 16);
    vdo[i] = (uint32_t)(row * a.v_rs * 2 + ((lane % CPR) ^ swz_key(row)) * 16);
  }
  const uint32_t lds_w = (uint32_t)uniform((int)(lds_addr(smem) + NI * wave * 1024));

  // One buffer descriptor per tensor per tile, ending at the last row before
  // seqlen_k (rows past it read as zero); its base is the tile's first row,
  // ko / vo elements from the sequence's K / V base (contiguous, or in the
  // page that holds it). Tile j >= T (the loop requests two tiles ahead)
  // gets zero-length descriptors: its loads touch no memory and only write
  // zeros into a buffer nothing reads again, so every iteration issues the
  // same number of loads and the load-count waits stay static.
  struct TileDesc {
    __amdgpu_buffer_rsrc_t k, v;
    int buf;
  };
  auto tile_desc = [&](int j) __attribute__((always_inline)) {
    const int jj = min(j, T - 1);
    const int n0 = (n_begin + jj) * BN;
    int64_t ko, vo;
    fwd_tile_rows<PAGED>(a, b, n0, ko, vo);
    const int nrows = min(sk - n0, BN);  // >= 1
    TileDesc t;
    t.k = make_rsrc(kp + ko, j < T ? (uint32_t)((nrows - 1) * a.k_rs * 2 + D * 2) : 0u);
    t.v = make_rsrc(vp + vo, j < T ? (uint32_t)((nrows - 1) * a.v_rs * 2 + D * 2) : 0u);
    t.buf = j & 3;
    return t;
  };
  // this wave's load p of a tile: K parts p = 0..NI-1, then V parts
  auto dma_part = [&](const TileDesc& t, int p) __attribute__((always_inline)) {
    if (p < NI)
      dma16(t.k, kdo[p], lds_w + (uint32_t)(t.buf * BUF_B + p * 1024));
    else
      dma16(t.v, vdo[p - NI], lds_w + (uint32_t)(t.buf * BUF_B + TILE_B + (p - NI) * 1024));
  };

  // ---- fragment read offsets. K: lane (c32, half) reads logical chunk
  // 2*cc + half of key c32 (+32 for the second key block, which has the same
  // swizzle). V: per-lane constant + immediate (the two transposing-read patterns
  // of attn_common.hpp).
  const int fk = kswz(c32);
  int k_rd[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) k_rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ fk) * 16);
  const int tr_g = lane >> 4;
  const int tr_j = lane & 15;
  const int tr_row = 4 * half + (tr_j >> 2);
  const int tr_c = (tr_g & 1) * 2 + ((tr_j & 3) >> 1);
  const int fv = swz_key(tr_row);
  int v_rd[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    v_rd[i] = tr_row * ROW_B + (((4 * i + tr_c) ^ fv) * 16) + (tr_j & 1) * 8;

  const float c = a.scale_log2;
  const float rescale_raw = C::RESCALE_LOG2 / fmaxf(c, 1e-30f);

  f32x16 s[2];
  bf16x8 pf[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pf[t] = zero_bf16x8();

  // Both parts of a matrix phase are written in issue order: a ring of LDS
  // fragments read LEAD MFMAs ahead, consecutive MFMAs on different
  // accumulators, and scheduling barriers between the {read i + LEAD,
  // MFMA i} groups so the compiler keeps that order.
  constexpr int LEAD = 4;
  // S(k) = K(k) Q^T into s[]; MFMA i: contraction step i / 2, key block i % 2.
  // This wave's 2 * NI loads of the tile two ahead (descriptor nx) go out
  // spread over the MFMAs: issued in one burst by the four waves of a group,
  // 16 direct-to-LDS loads of 1 KB queue in the CU's load path for several
  // hundred cycles, and the issuing waves stall with them.
  auto s_part = [&](int k, const TileDesc& nx) __attribute__((always_inline)) {
    const char* kb0 = smem + (k & 3) * BUF_B;
    constexpr int N = 2 * (D / 16);  // i -> cc = i / 2, kb = i % 2
    auto rd = [&](int i) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kb0 + (i & 1) * 32 * ROW_B + k_rd[i >> 1]);
    };
    bf16x8 ring[LEAD];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) ring[i] = rd(i);
    s[0] = zero_f32x16();
    s[1] = zero_f32x16();
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NP = 2 * NI;  // loads per wave per tile
    static_assert(N % NP == 0, "loads spread evenly over the MFMAs");
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 kf = ring[i % LEAD];
      if (i + LEAD < N) ring[i % LEAD] = rd(i + LEAD);
      s[i & 1] = mfma32(kf, qf[i >> 1], s[i & 1]);
      if (i % (N / NP) == 1 % (N / NP)) dma_part(nx, i / (N / NP));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O += P(k) V(k); V^T fragments from row-major V by transposing reads;
  // MFMA i: 16-key step i / NDB, d-block i % NDB
  auto pv_part = [&](int k) __attribute__((always_inline)) {
    const char* vb = smem + (k & 3) * BUF_B + TILE_B;
    constexpr int NDB = D / 32, N = 4 * NDB;  // i -> t = i / NDB, db = i % NDB
    auto rd = [&](int i) __attribute__((always_inline)) {
      const int t = i / NDB, db = i % NDB;
      const char* p = vb + (16 * t) * ROW_B + (db >> 1) * 128 + v_rd[db & 1];
      const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(p));
      const bf16x4 v1 = ds_read_tr16(reinterpret_cast<const __bf16*>(p + 8 * ROW_B));
      return cat(v0, v1);
    };
    bf16x8 ring[LEAD];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) ring[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 vf = ring[i % LEAD];
      if (i + LEAD < N) ring[i % LEAD] = rd(i + LEAD);
      o[i % NDB] = mfma32(vf, pf[i / NDB], o[i % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // MFMA item k: O += P(k-1) V(k-1) (k >= 1), then S(k) = K(k) Q^T (k < T)
  // with the loads of tile k + 2
  auto mfma_item = [&](int k) {
    if (k >= 1) pv_part(k - 1);
    if (k < T) s_part(k, tile_desc(k + 2));
  };

  // softmax of S(k) into P(k): mask edge tiles, lazy running max, exp2
  auto sm_item = [&](int k) {
    const int n0 = (n_begin + k) * BN;
    const bool full = (n0 + BN <= sk) && (n0 + BN - 1 <= full_hi) && (n0 >= full_lo);
    if constexpr (SC) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = softcap_raw(s[kb][v], a.sc_k1x, a.sc_k2);
    }
    if (!full) {
      // element (kb, v) holds key n0 + 4*half + l, l = 32*kb + 8*(v>>2) + (v&3)
      const uint64_t vis = vis64(lo - n0 - 4 * half, hi - n0 - 4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t w = (uint32_t)(vis >> (32 * kb));
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = mask_by_bit(s[kb][v], w, 8 * (v >> 2) + (v & 3));
      }
    }
    // two independent max chains (one per 32-key half), then the lane pair
    float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      m0 = vmax3(m0, s[0][v], s[0][v + 1]);
      m1 = vmax3(m1, s[1][v], s[1][v + 1]);
    }
    const float mt = pair_max(vmax(m0, m1));
    const bool grow = (m_run == kNegInf) ? (mt != kNegInf) : (mt - m_run > rescale_raw);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_run;
      const float alpha = grow ? ((m_run == kNegInf) ? 0.0f : fast_exp2((m_run - m_new) * c))
                               : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    const float ms = (m_run == kNegInf) ? 0.0f : m_run * c;
    // four partial row sums keep the adds off one serial chain
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s[kb][v], c, -ms));
        s[kb][v] = p;
        rs[v & 3] += p;
      }
    }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // P^T fragments in the key order of the V^T fragments (attn_common.hpp)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1;
      const int i0 = 2 * (t & 1);
      pf[t] = cat(cvt4(s[kb][4 * i0 + 0], s[kb][4 * i0 + 1], s[kb][4 * i0 + 2], s[kb][4 * i0 + 3]),
                  cvt4(s[kb][4 * i0 + 4], s[kb][4 * i0 + 5], s[kb][4 * i0 + 6], s[kb][4 * i0 + 7]));
    }
  };

  if (T > 0) {
    // prologue: tiles 0 and 1 requested (tile 1 loads nothing when T == 1);
    // wait for tile 0 (this wave's part), then the barrier makes all parts
    // visible
    {
      const TileDesc t0 = tile_desc(0), t1 = tile_desc(1);
#pragma unroll
      for (int p = 0; p < 2 * NI; ++p) dma_part(t0, p);
#pragma unroll
      for (int p = 0; p < 2 * NI; ++p) dma_part(t1, p);
    }
    vmcnt_wait<2 * NI>();
    lds_barrier();
    for (int k = 0; k < T; ++k) {
      // Tile k+2 goes into the buffer tile k-2 left (its last reader, the
      // P V product of matrix phase k-1, finished before the previous
      // barrier); each group requests its share during its own matrix phase,
      // spread over the S MFMAs.
      // first phase: A matrix work, B softmax
      if (grp == 0) {
        __builtin_amdgcn_s_setprio(1);
        mfma_item(k);
        __builtin_amdgcn_s_setprio(0);
      } else if (k >= 1) {
        sm_item(k - 1);
      }
      // second phase: A softmax, B matrix work; then tile k+1 must have
      // landed (only tile k+2's loads may still be in flight)
      if (grp == 0) {
        sm_item(k);
      } else {
        __builtin_amdgcn_s_setprio(1);
        mfma_item(k);
        __builtin_amdgcn_s_setprio(0);
      }
      vmcnt_wait<2 * NI>();
      lds_barrier();
    }
    // tail: the last P V products
    if (grp == 0) {
      mfma_item(T);
    } else {
      sm_item(T - 1);
    }
    if (grp == 1) mfma_item(T);
    // the last (zero-length) requests must land before the workgroup's LDS
    // is released
    vmcnt_wait<0>();
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store.
  // O leaves through LDS, free once every wave is past the loop: each wave
  // writes its 32 normalised rows there, then stores them as whole rows of
  // 16-byte chunks, so each output line is written in full by one
  // instruction. (Stored in place, 8 bytes per lane, the lines were written
  // in pieces and the write counter read up to 1.4x the output bytes.)
  const float l_tot = pair_sum(l_run);
  float inv = poison ? __builtin_nanf("") : (l_tot > 0.0f ? 1.0f / l_tot : 0.0f);
  float lse_row = l_tot > 0.0f ? m_run * a.scale + __logf(l_tot) : kNegInf;
  if (a.sink != nullptr) {
    float w;
    lse_row = merge_sink(lse_row, (float)a.sink[hq], &w);
    inv *= w;
  }
  constexpr int OS = 2 * D + 16;  // LDS row stride of the staged O, bytes
  static_assert(8 * 32 * OS <= C::NBUF * BUF_B, "staged O fits the tile buffers");
  char* so = smem + wave * 32 * OS;
  lds_barrier();  // every wave is done with the K/V tiles (and its loads landed)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + 8 * i + 4 * half;
      *reinterpret_cast<bf16x4*>(so + c32 * OS + 2 * d0) =
          cvt4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
               o[db][4 * i + 3] * inv);
    }
  // the lanes read chunks other lanes of this wave wrote: a wave's LDS
  // accesses complete in order, and the empty asm keeps the compiler's order
  asm volatile("" ::: "memory");
  {
    constexpr int CH = D / 8;                 // 16-byte chunks per row
    constexpr int NST = (32 * CH + 63) / 64;  // store instructions per wave
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int ci = k * 64 + lane;
      const int rr = ci / CH, cc = ci - rr * CH;
      const int prow_r = row0 + grp * 128 + wig * 32 + rr;
      if (rr < 32 && prow_r < rows) {
        const int pos_r = prow_r / r;
        const int hq_r = hk * r + (prow_r - pos_r * r);
        const uint4 val = *reinterpret_cast<const uint4*>(so + rr * OS + 16 * cc);
        *reinterpret_cast<uint4*>(static_cast<__bf16*>(a.out) + o_base + (int64_t)pos_r * a.o_rs +
                                  (int64_t)hq_r * a.o_hs + 8 * cc) = val;
      }
    }
  }
  if (valid) {
    if (half == 0 && a.lse != nullptr) {
      const float lse = poison ? __builtin_nanf("") : lse_row;
      const int64_t li = a.cu_q != nullptr
                             ? (int64_t)hq * a.total_q + q_tok0 + pos
                             : ((int64_t)b * a.hq + hq) * sq + pos;
      a.lse[li] = lse;
    }
  }
}

template <int D>
hipError_t launch_fwd_pp(const FwdArgs& args, hipStream_t s) {
  FwdArgs a = args;
  a.num_m_blocks = (int)(((int64_t)a.max_rows + kFwdPPBlockM - 1) / kFwdPPBlockM);
  const int64_t grid = fwd_blocks_per_head(a, kFwdPPBlockM) * a.hkv;
  if (grid <= 0) return hipSuccess;
  const bool sc = a.softcap > 0.0f;
  if (a.page_table != nullptr) {
    if (sc)
      hipLaunchKernelGGL((fwd_pp_kernel<D, true, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_pp_kernel<D, true, false>), dim3((unsigned)grid), dim3(512), 0, s, a);
  } else {
    if (sc)
      hipLaunchKernelGGL((fwd_pp_kernel<D, false, true>), dim3((unsigned)grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_pp_kernel<D, false, false>), dim3((unsigned)grid), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

template hipError_t launch_fwd_pp<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_pp<96>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_pp<128>(const FwdArgs&, hipStream_t);

}  // namespace mi_attn
