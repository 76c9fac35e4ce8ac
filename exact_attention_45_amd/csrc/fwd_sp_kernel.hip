// Prefill forward with one wave per SIMD and software pipelining inside the
// wave: the matrix cores compute the next tile's scores while the same wave
// runs the current tile's exponentials. Serves head_dim 256, whose O
// accumulators alone take 128 registers per lane.
//
// Method as launch_fwd in kernels.hpp (mslk flash_attn interface.py page,
// `_flash_attn_fwd`): exact attention, online softmax in the exp2 domain with
// a lazily updated running max, natural-log LSE, empty rows O = 0 and
// LSE = -inf. Same MFMA conventions (attn_common.hpp: both GEMMs transposed so
// a lane owns one query), the same packed GQA rows, tile skipping, edge masks
// and grid order.
//
// Schedule. A workgroup is four waves, one per SIMD, each with the whole
// 512-entry register file; wave w owns 32*QB consecutive packed rows (QB query
// blocks of 32 MFMA columns), so every K or V fragment read from LDS feeds QB
// MFMAs. Iteration k of the key-tile loop:
//   top     : wait until K(k+1) has landed, barrier
//   softmax : lazy rescale of O (the row max of S(k) is already known)
//   phase 1 : S(k+1) = K(k+1) Q^T on the matrix cores, each MFMA issued
//             together with exponentials, row-sum adds and bf16 packing of
//             key block 0 of P(k) (one element every other MFMA), K
//             fragment reads a few MFMAs ahead; V(k+1) requested straight
//             into LDS (direct-to-LDS buffer loads), one load every few MFMAs
//   mid     : wait until V(k) has landed, barrier
//   phase 2 : O += P(k) V(k), the transposing V reads issued several MFMAs
//             ahead; K(k+3) requested the same way; the exponentials of key
//             block 1 of P(k) between the MFMAs of key block 0 (which do not
//             use them), the edge mask and the row max of S(k+1) between the
//             later ones
// Both phases are written in the intended issue order and held there by
// scheduling barriers. Each tile is requested about one and a half
// iterations before its use, and no wave ever issues its loads in a burst.
// K and V each have two LDS buffers (tile j in buffer j & 1). The loop is
// unrolled by two so buffer offsets and the two score register sets are
// fixed at compile time.
//
// With one wave per SIMD nothing hides LDS latency but the wave's own
// read-ahead: with each read issued just before its MFMA (the compiler's
// choice when left alone) the long-context D256 workload ran 2.85 ms; with
// six MFMAs of read-ahead in phase 2, 2.35 ms; with phase 1 also written out
// group by group, 2.07 ms. Moving half of each tile's exponentials from
// phase 1 into phase 2 took another 2% (1.86 vs 1.90 ms on one box).
//
// Register classes: this source is compiled with MFMA results in vector
// registers (the build's per-file flag), so O and S stay where the softmax
// and the rescale read them, and the Q fragments, which are only MFMA
// operands, are placed in the accumulation registers.
#include <climits>
#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

// Head dim 192 uses the head-dim-256 LDS layout (rows of 512 bytes): tiles
// load whole 512-byte row slots (the last 128 bytes of a row slot hold the
// next row's first values, or zeros past the end of the tensor) and every
// product reads only the first 192 columns.
template <int D, int QB>
struct SPCfg {
  static constexpr int DL = D == 192 ? 256 : D;  // layout head dim
  static constexpr int BM = 128 * QB;          // packed rows per workgroup
  static constexpr int BN = kFwdBlockN;        // 64 keys per tile
  static constexpr int ROW_B = DL * 2;         // bytes per K/V LDS row
  static constexpr int CPR = DL / 8;           // 16-byte chunks per LDS row
  static constexpr int TILE_B = BN * ROW_B;    // bytes per K (or V) tile
  static constexpr int RPI = 1024 / ROW_B;     // rows per direct-to-LDS wave instruction
  static constexpr int NI = BN / RPI / 4;      // such instructions per wave per tensor
  static constexpr float RESCALE_LOG2 = 8.0f;  // lazy-rescale threshold
  static_assert(NI * RPI * 4 == BN, "a tile splits evenly over four waves");
  static_assert(DL == 128 || DL == 256, "16-byte-chunk swizzles assume 256- or 512-byte rows");
};

// K tile swizzle: chunk c of key row `key` sits at chunk c ^ kswz16(key). The
// 16 lanes an LDS cycle serves read one logical chunk of 16 consecutive keys;
// kswz16 takes 16 distinct values over any 16 consecutive keys, and rows are a
// multiple of 256 bytes, so those reads hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kswz16(int key) { return swz_key(key) | (((key >> 3) & 1) << 3); }

template <int D, int QB, bool PAGED, bool SC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_sp_kernel(const FwdArgs a) {
  using C = SPCfg<D, QB>;
  constexpr int BM = C::BM, BN = C::BN, ROW_B = C::ROW_B, CPR = C::CPR, TILE_B = C::TILE_B;
  constexpr int RPI = C::RPI, NI = C::NI;
  constexpr int NKC = D / 16;  // 16-deep contraction steps of S over head_dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  // K0 K1 V0 V1
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- this lane's query rows, one per query block
  const int off = sk - sq;  // bottom-right alignment
  bool valid[QB];
  int pos[QB], hq[QB], lo[QB], hi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int prow = row0 + wave * 32 * QB + qb * 32 + c32;
    valid[qb] = prow < rows;
    pos[qb] = valid[qb] ? prow / r : 0;
    hq[qb] = hk * r + (valid[qb] ? prow - (prow / r) * r : 0);
    lo[qb] = a.wl >= 0 ? pos[qb] + off - a.wl : INT_MIN / 2;
    hi[qb] = min(a.wr >= 0 ? pos[qb] + off + a.wr : INT_MAX / 2, sk - 1);
  }

  // workgroup-wide visible key range and "tile fully visible" bounds
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
  const int full_hi = a.wr >= 0 ? pos_min + off + a.wr : INT_MAX / 2;
  const int full_lo = a.wl >= 0 ? pos_max + off - a.wl : INT_MIN / 2;

  // ---- Q^T fragments (B operand of S), in registers for the whole loop.
  // Branch-free: invalid lanes read a valid row and zero it.
  bf16x8 qf[QB][NKC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + q_base + (int64_t)pos[qb] * a.q_rs +
                       (int64_t)hq[qb] * a.q_hs;
#pragma unroll
    for (int cc = 0; cc < NKC; ++cc) {
      const bf16x8 x = as_bf16x8(ld16(qp + 16 * cc + 8 * half));
      qf[qb][cc] = valid[qb] ? x : zero_bf16x8();
    }
  }
  // Register classes: the Q fragments are only ever MFMA operands, so they
  // can live in accumulation registers; O is rescaled by vector
  // instructions, which read only vector registers. Left to itself the
  // allocator keeps O in accumulation registers and copies all of it out at
  // every loop iteration for the (rarely taken) rescale. The empty asm
  // statements state the intended classes and emit no instructions.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cc = 0; cc < NKC; ++cc) asm volatile("" : "+a"(qf[qb][cc]));

  f32x16 o[NDB][QB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[db][qb] = zero_f32x16();
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.0f;
  }

  // ---- K/V tiles go global -> LDS directly, 1 KB per wave instruction.
  // Instruction i of wave w fills tile rows RPI*(NI*w + i) .. +RPI-1: lane j
  // lands at row offset j / CPR, physical chunk j % CPR, so it loads logical
  // chunk (j % CPR) ^ swizzle(row). K uses kswz16, V swz_key (the pattern its
  // transposing reads need).
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  uint32_t kdo[NI], vdo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * (NI * wave + i) + lane / CPR;
    kdo[i] = (uint32_t)(row * a.k_rs * 2 + ((lane % CPR) ^ kswz16(row)) * 16);
    vdo[i] = (uint32_t)(row * a.v_rs * 2 + ((lane % CPR) ^ swz_key(row)) * 16);
  }
  const uint32_t lds_w = (uint32_t)uniform((int)(lds_addr(smem) + NI * wave * 1024));
  // Buffer descriptor of K (V) tile j: based at the tile's first row (ko / vo
  // elements from the sequence's K / V base: contiguous, or in the page that
  // holds it), ending at the last row before seqlen_k (rows past it read as
  // zero). A tile j >= T gets a zero-length descriptor: its loads touch no
  // memory (they only write zeros into a buffer nothing reads again), so
  // every iteration issues the same number of loads and the load-count waits
  // stay static.
  auto k_rsrc = [&](int j) __attribute__((always_inline)) {
    const int jj = min(j, T - 1);
    int64_t ko, vo;
    fwd_tile_rows<PAGED>(a, b, (n_begin + jj) * BN, ko, vo);
    const int nrows = min(sk - (n_begin + jj) * BN, BN);  // >= 1
    return make_rsrc(kp + ko, j < T ? (uint32_t)((nrows - 1) * a.k_rs * 2 + D * 2) : 0u);
  };
  auto v_rsrc = [&](int j) __attribute__((always_inline)) {
    const int jj = min(j, T - 1);
    int64_t ko, vo;
    fwd_tile_rows<PAGED>(a, b, (n_begin + jj) * BN, ko, vo);
    const int nrows = min(sk - (n_begin + jj) * BN, BN);
    return make_rsrc(vp + vo, j < T ? (uint32_t)((nrows - 1) * a.v_rs * 2 + D * 2) : 0u);
  };
  // this wave's part i (of NI) of a K tile into K buffer kbuf, of a V tile
  // into V buffer vbuf
  auto dma_k = [&](__amdgpu_buffer_rsrc_t r, int kbuf, int i) __attribute__((always_inline)) {
    dma16(r, kdo[i], lds_w + (uint32_t)(kbuf * TILE_B + i * 1024));
  };
  auto dma_v = [&](__amdgpu_buffer_rsrc_t r, int vbuf, int i) __attribute__((always_inline)) {
    dma16(r, vdo[i], lds_w + (uint32_t)((2 + vbuf) * TILE_B + i * 1024));
  };

  // ---- fragment read offsets. K: lane (c32, half) reads logical chunk
  // 2*cc + half of key c32 (+32 for the second key block, same swizzle); for
  // cc >= 8 (D = 256) the chunk lies 16 chunks = 256 bytes further. V: the
  // transposing-read pattern of attn_common.hpp.
  const int fk = kswz16(c32);
  int k_rd[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) k_rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ fk) * 16);
  const int tr_g = lane >> 4;
  const int tr_j = lane & 15;
  const int tr_row = 4 * half + (tr_j >> 2);
  const int tr_c = (tr_g & 1) * 2 + ((tr_j & 3) >> 1);
  const int fv = swz_key(tr_row);
  int v_rd[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    v_rd[i] = 2 * TILE_B + tr_row * ROW_B + (((4 * i + tr_c) ^ fv) * 16) + (tr_j & 1) * 8;

  const float c = a.scale_log2;
  const float rescale_raw = C::RESCALE_LOG2 / fmaxf(c, 1e-30f);

  typedef f32x16 STile[2][QB];  // S^T accumulators: key block x query block
  bf16x8 pf[QB][4];             // P^T fragments of the current tile
  float ms[QB];                 // running max in exp2 units, per query block

  // S = K(tile in buffer buf) Q^T. Contraction step outermost, so consecutive
  // MFMAs accumulate into different registers.
  auto s_tile = [&](auto buf_c, STile& s) {
    constexpr int buf = decltype(buf_c)::value;
    const char* kb0 = smem + buf * TILE_B;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = zero_f32x16();
#pragma unroll
    for (int cc = 0; cc < NKC; ++cc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb0 + kb * 32 * ROW_B + (cc >> 3) * 256 +
                                                           k_rd[cc & 7]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(kf, qf[qb][cc], s[kb][qb]);
      }
    }
  };

  // Softmax statistics of a score tile are taken in two steps: sm_edge
  // (soft-capping, the edge-tile mask) and the tile's row max with the
  // rescale decision, normally interleaved with the P V MFMAs of the previous
  // tile (pv_tile) so the matrix cores keep working; then sm_apply at the top
  // of the tile's own iteration, once O holds the previous tile's products:
  // the (rare) lazy rescale of O and l, and the exp2 offset.
  float mt_n[QB];   // row max of the next tile's scores (raw units)
  bool grow_n[QB];  // whether it moves the running max
  auto sm_edge = [&](STile& s, int j) __attribute__((always_inline)) {
    const int n0 = (n_begin + j) * BN;
    const bool full = (n0 + BN <= sk) && (n0 + BN - 1 <= full_hi) && (n0 >= full_lo);
    if constexpr (SC) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[kb][qb][v] = softcap_raw(s[kb][qb][v], a.sc_k1x, a.sc_k2);
    }
    if (!full) {
      // element (kb, v) holds key n0 + 4*half + l, l = 32*kb + 8*(v>>2) + (v&3)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const uint64_t vis = vis64(lo[qb] - n0 - 4 * half, hi[qb] - n0 - 4 * half);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t w = (uint32_t)(vis >> (32 * kb));
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[kb][qb][v] = mask_by_bit(s[kb][qb][v], w, 8 * (v >> 2) + (v & 3));
        }
      }
    }
  };
  // row max of a tile (two independent chains, then the lane pair) and the
  // rescale decision against the running max
  auto max_grow = [&](float m0, float m1, int qb) __attribute__((always_inline)) {
    mt_n[qb] = pair_max(vmax(m0, m1));
    grow_n[qb] = (m_run[qb] == kNegInf) ? (mt_n[qb] != kNegInf) : (mt_n[qb] - m_run[qb] > rescale_raw);
  };
  auto sm_max = [&](STile& s) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        m0 = vmax3(m0, s[0][qb][v], s[0][qb][v + 1]);
        m1 = vmax3(m1, s[1][qb][v], s[1][qb][v + 1]);
      }
      max_grow(m0, m1, qb);
    }
  };
  auto sm_apply = [&]() __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) any = any || grow_n[qb];
    if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = grow_n[qb] ? mt_n[qb] : m_run[qb];
        const float alpha = grow_n[qb]
                                ? ((m_run[qb] == kNegInf) ? 0.0f : fast_exp2((m_run[qb] - m_new) * c))
                                : 1.0f;
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][qb][v] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ms[qb] = (m_run[qb] == kNegInf) ? 0.0f : m_run[qb] * c;
  };

  // P = exp2(S*c - m*c) of key block 0, row sums, P^T fragments 0 and 1 in
  // the key order of the V^T fragments (attn_common.hpp): phase 1's share at
  // the last tile (the P V phase does key block 1)
  auto sm_exp = [&](STile& s) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 1; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(s[kb][qb][v], c, -ms[qb]));
          s[kb][qb][v] = p;
          rs[v & 3] += p;
        }
      }
      l_run[qb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kb = t >> 1;
        const int i0 = 2 * (t & 1);
        pf[qb][t] = cat(cvt4(s[kb][qb][4 * i0 + 0], s[kb][qb][4 * i0 + 1], s[kb][qb][4 * i0 + 2],
                             s[kb][qb][4 * i0 + 3]),
                        cvt4(s[kb][qb][4 * i0 + 4], s[kb][qb][4 * i0 + 5], s[kb][qb][4 * i0 + 6],
                             s[kb][qb][4 * i0 + 7]));
      }
    }
  };

  // Phase 1 for one query block per wave: S(next) = K(tile in buffer buf)
  // Q^T fused with the exponentials of key block 0 of S(cur). MFMA i
  // (contraction step i / 2, key block i % 2) is issued with the K fragment
  // read LEAD1 MFMAs ahead and with the exponentials, row-sum adds and bf16
  // packing of 16 / N score elements (elements 16 i / N .. 16 (i + 1) / N - 1
  // with MFMA i), in that source order, held by scheduling barriers between
  // the groups.
  // This wave's NI loads of the next V tile (descriptor vr, V buffer vbuf)
  // go out spread over the MFMAs, one every N / NI: issued in one burst by all
  // four waves, 64 direct-to-LDS loads of 1 KB queue in the CU's load path
  // for about a thousand cycles, and the issuing waves stall with them.
  auto phase1 = [&](auto buf_c, STile& cur, STile& nxt, __amdgpu_buffer_rsrc_t vr, int vbuf)
      __attribute__((always_inline)) {
    static_assert(QB == 1, "fused phase 1 handles one query block per wave");
    constexpr int buf = decltype(buf_c)::value;
    constexpr int N = 2 * NKC;   // MFMAs and K fragment reads
    static_assert(N <= 32, "at least one score element per MFMA");
    static_assert(N % NI == 0, "loads spread evenly over the MFMAs");
    constexpr int L1 = 4;
    auto kread = [&](int i) __attribute__((always_inline)) {
      const int cc = i >> 1, kb = i & 1;
      return *reinterpret_cast<const bf16x8*>(smem + k_rd[cc & 7] +
                                              (buf * TILE_B + kb * 32 * ROW_B + (cc >> 3) * 256));
    };
    bf16x8 ring[L1];
#pragma unroll
    for (int i = 0; i < L1; ++i) ring[i] = kread(i);
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int cc = i >> 1, kb = i & 1;
      const bf16x8 kf = ring[i % L1];
      if (i + L1 < N) ring[i % L1] = kread(i + L1);
      nxt[kb][0] = mfma32(kf, qf[0][cc], cc == 0 ? zero_f32x16() : nxt[kb][0]);
      if (i % (N / NI) == 0) dma_v(vr, vbuf, i / (N / NI));
#pragma unroll
      for (int j = 16 * i / N; j < 16 * (i + 1) / N; ++j) {
        // element j of key block 0 (block 1's follow in the P V phase)
        const int jb = 0, jv = j;
        const float x = fast_exp2(fmaf(cur[jb][0][jv], c, -ms[0]));
        cur[jb][0][jv] = x;
        rs[jv & 3] += x;
        if ((j & 7) == 7) {
          // P^T fragment t holds elements 8t .. 8t+7 (see sm_exp)
          const int t = j >> 3, tb = t >> 1, t0 = 8 * (t & 1);
          pf[0][t] = cat(cvt4(cur[tb][0][t0 + 0], cur[tb][0][t0 + 1], cur[tb][0][t0 + 2],
                              cur[tb][0][t0 + 3]),
                         cvt4(cur[tb][0][t0 + 4], cur[tb][0][t0 + 5], cur[tb][0][t0 + 6],
                              cur[tb][0][t0 + 7]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run[0] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  // O += P V(tile in buffer buf); MFMA i covers key step t = i / NDB and
  // d-block db = i % NDB (consecutive MFMAs use different accumulators). The
  // V^T fragments are read LEAD2 MFMAs ahead, in source order, and scheduling
  // barriers (nothing may cross them) between the {read i + LEAD2, MFMA i}
  // groups keep that order: left free, the scheduler issues each read right
  // before its MFMA, which then waits out the whole LDS latency.
  // The NI loads of a K tile (descriptor kr, K buffer kbuf) go out spread
  // over the MFMAs as in phase 1. The first 2 NDB MFMAs (key block 0, P^T
  // fragments 0 and 1) carry the exponentials of key block 1 of the current
  // tile's scores cu (fragments 2 and 3, first read by MFMA 2 NDB). With WM,
  // the next tile's scores nx (tile j) get their edge treatment before the
  // MFMAs and their row max during the nine MFMAs after those.
  auto pv_tile = [&](auto buf_c, __amdgpu_buffer_rsrc_t kr, int kbuf, auto wm_c, STile& cu,
                     STile& nx, int j) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool WM = decltype(wm_c)::value;
    static_assert(!WM || QB == 1, "interleaved row max handles one query block per wave");
    constexpr int N = 4 * NDB;
    static_assert(N >= 2 * NDB + 9, "row max spread over nine MFMAs of the second half");
    static_assert(N % NI == 0, "loads spread evenly over the MFMAs");
    constexpr int LEAD2 = 6;
    auto read = [&](int i) __attribute__((always_inline)) {
      const int t = i / NDB, db = i % NDB;
      const char* p = smem + v_rd[db & 1] + (buf * TILE_B + (16 * t) * ROW_B + (db >> 1) * 128);
      const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(p));
      const bf16x4 v1 = ds_read_tr16(reinterpret_cast<const __bf16*>(p + 8 * ROW_B));
      return cat(v0, v1);
    };
    bf16x8 ring[LEAD2];
#pragma unroll
    for (int i = 0; i < LEAD2; ++i) ring[i] = read(i);
    if constexpr (WM) sm_edge(nx, j);
    float m0 = kNegInf, m1 = kNegInf;
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int H = 2 * NDB;  // MFMAs of the first key block (P^T fragments 0, 1)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int t = i / NDB, db = i % NDB;
      const bf16x8 vf = ring[i % LEAD2];
      if (i + LEAD2 < N) ring[i % LEAD2] = read(i + LEAD2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma32(vf, pf[qb][t], o[db][qb]);
      if (i % (N / NI) == 0) dma_k(kr, kbuf, i / (N / NI));
      if (i < H) {
        // exponentials of key block 1 of the current tile (fragments 2, 3,
        // first used by MFMA H)
#pragma unroll
        for (int e = 16 * i / H; e < 16 * (i + 1) / H; ++e) {
          const float x = fast_exp2(fmaf(cu[1][0][e], c, -ms[0]));
          cu[1][0][e] = x;
          rs[e & 3] += x;
          if ((e & 7) == 7) {
            const int t0 = e - 7;
            pf[0][2 + (e >> 3)] = cat(cvt4(cu[1][0][t0 + 0], cu[1][0][t0 + 1], cu[1][0][t0 + 2],
                                           cu[1][0][t0 + 3]),
                                      cvt4(cu[1][0][t0 + 4], cu[1][0][t0 + 5], cu[1][0][t0 + 6],
                                           cu[1][0][t0 + 7]));
          }
        }
      }
      if constexpr (WM) {
        if (i >= H && i < H + 8) {
          const int r = i - H;
          m0 = vmax3(m0, nx[0][0][2 * r], nx[0][0][2 * r + 1]);
          m1 = vmax3(m1, nx[1][0][2 * r], nx[1][0][2 * r + 1]);
        } else if (i == H + 8) {
          max_grow(m0, m1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run[0] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };


  STile sA, sB;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Iteration k (cur holds S(k); nxt receives S(k+1); par = k & 1). Tile j
  // of K lives in K buffer j & 1, tile j of V in V buffer j & 1. Per wave the
  // loads go out in the order ..., V(k) in phase 1 of iteration k-1, K(k+2)
  // in its P V phase, V(k+1) in phase 1 of iteration k, K(k+3) in its P V
  // phase, ...:
  //   top: K(k+1) has landed once at most 2*NI loads (V(k), K(k+2)) are
  //        outstanding; the barrier also ends every wave's reads of V(k-1),
  //        whose buffer phase 1 refills with V(k+1)
  //   mid: V(k) has landed once at most 2*NI loads (K(k+2), V(k+1)) are
  //        outstanding; the barrier also ends every wave's reads of K(k+1),
  //        whose buffer the P V phase refills with K(k+3)
  // so each tile is requested about one and a half iterations before use.
  // The statistics of S(k) (row max, rescale decision) were taken during the
  // P V phase of iteration k-1 (for k = 0 in the prologue); sm_apply
  // rescales O and l, which then hold the products of tiles < k.
  auto step = [&](int k, auto par_c, STile& cur, STile& nxt) {
    constexpr int par = decltype(par_c)::value;
    using PN = std::integral_constant<int, par ^ 1>;
    vmcnt_wait<2 * NI>();
    lds_barrier();
    const auto vr = v_rsrc(k + 1);
    sm_apply();
    if (k + 1 < T) {
      phase1(PN{}, cur, nxt, vr, par ^ 1);
    } else {
      sm_exp(cur);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_v(vr, par ^ 1, i);  // zero-length: keeps the count
    }
    vmcnt_wait<2 * NI>();
    lds_barrier();
    // At the last tile nxt holds no scores; the statistics taken from it are
    // never used. (A second instantiation without them, selected by a branch,
    // makes the register allocator spill.)
    pv_tile(par_c, k_rsrc(k + 3), par ^ 1, std::true_type{}, cur, nxt, k + 1);
  };

  if (T > 0) {
    // prologue: K(0), K(1), V(0) requested (tiles past the last one load
    // nothing); wait for K(0), compute S(0); once every wave has read K(0),
    // K(2) goes into its buffer (the loop's waits assume K(2) after V(0))
    {
      const auto k0 = k_rsrc(0), k1 = k_rsrc(1), v0 = v_rsrc(0);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_k(k0, 0, i);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_k(k1, 1, i);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_v(v0, 0, i);
    }
    vmcnt_wait<2 * NI>();
    lds_barrier();
    s_tile(I0{}, sA);
    sm_edge(sA, 0);
    sm_max(sA);
    lds_barrier();
    {
      const auto k2 = k_rsrc(2);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_k(k2, 0, i);
    }
    for (int k = 0; k < T; k += 2) {
      step(k, I0{}, sA, sB);
      if (k + 1 < T) step(k + 1, I1{}, sB, sA);
    }
    // the last requests (zero-length) must land before the workgroup's LDS
    // is released
    vmcnt_wait<0>();
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store.
  // O leaves through LDS, free once every wave is past the loop: each wave
  // writes its normalised rows there, then stores them as whole rows of
  // 16-byte chunks, so each output line is written by one instruction.
  constexpr int OS = 2 * D + 16;  // LDS row stride of the staged O, bytes
  static_assert(4 * 32 * QB * OS <= 4 * TILE_B, "staged O fits the tile buffers");
  char* so = smem + wave * 32 * QB * OS;
  lds_barrier();  // every wave is done with the K/V tiles (and its loads landed)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    float inv = poison ? __builtin_nanf("") : (l_tot > 0.0f ? 1.0f / l_tot : 0.0f);
    float lse_row = l_tot > 0.0f ? m_run[qb] * a.scale + __logf(l_tot) : kNegInf;
    if (a.sink != nullptr) {
      float w;
      lse_row = merge_sink(lse_row, (float)a.sink[hq[qb]], &w);
      inv *= w;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<bf16x4*>(so + (qb * 32 + c32) * OS + 2 * d0) =
            cvt4(o[db][qb][4 * i] * inv, o[db][qb][4 * i + 1] * inv, o[db][qb][4 * i + 2] * inv,
                 o[db][qb][4 * i + 3] * inv);
      }
    if (valid[qb]) {
      if (half == 0 && a.lse != nullptr) {
        const float lse = poison ? __builtin_nanf("") : lse_row;
        const int64_t li = a.cu_q != nullptr
                               ? (int64_t)hq[qb] * a.total_q + q_tok0 + pos[qb]
                               : ((int64_t)b * a.hq + hq[qb]) * sq + pos[qb];
        a.lse[li] = lse;
      }
    }
  }
  // the lanes read chunks other lanes of this wave wrote: a wave's LDS
  // accesses complete in order, and the empty asm keeps the compiler's order
  asm volatile("" ::: "memory");
  {
    constexpr int CH = D / 8;                      // 16-byte chunks per row
    constexpr int NST = (32 * QB * CH + 63) / 64;  // store instructions per wave
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int ci = k * 64 + lane;
      const int rr = ci / CH, cc = ci - rr * CH;
      const int prow_r = row0 + wave * 32 * QB + rr;
      if (rr < 32 * QB && prow_r < rows) {
        const int pos_r = prow_r / r;
        const int hq_r = hk * r + (prow_r - pos_r * r);
        const uint4 val = *reinterpret_cast<const uint4*>(so + rr * OS + 16 * cc);
        *reinterpret_cast<uint4*>(static_cast<__bf16*>(a.out) + o_base + (int64_t)pos_r * a.o_rs +
                                  (int64_t)hq_r * a.o_hs + 8 * cc) = val;
      }
    }
  }
}

template <int D, int QB>
hipError_t launch_fwd_sp(const FwdArgs& args, hipStream_t s) {
  constexpr int BM = SPCfg<D, QB>::BM;
  FwdArgs a = args;
  a.num_m_blocks = (int)(((int64_t)a.max_rows + BM - 1) / BM);
  const int64_t grid = fwd_blocks_per_head(a, BM) * a.hkv;
  if (grid <= 0) return hipSuccess;
  const bool sc = a.softcap > 0.0f;
  if (a.page_table != nullptr) {
    if (sc)
      hipLaunchKernelGGL((fwd_sp_kernel<D, QB, true, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_sp_kernel<D, QB, true, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  } else {
    if (sc)
      hipLaunchKernelGGL((fwd_sp_kernel<D, QB, false, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_sp_kernel<D, QB, false, false>), dim3((unsigned)grid), dim3(256), 0,
                         s, a);
  }
  return hipGetLastError();
}

template hipError_t launch_fwd_sp<192, 1>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_sp<256, 1>(const FwdArgs&, hipStream_t);

}  // namespace mi_attn
