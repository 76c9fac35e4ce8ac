// Prefill forward: fused exact attention, one workgroup per (128 packed query
// rows, KV head, sequence).
//
// Method (mslk flash_attn interface.py page, `_flash_attn_fwd`; the online
// softmax in the exp2 domain with scale*log2(e) folded into one FMA, as the
// flash_bwd_sm100.py page's P = exp2(S*scale_log2 - LSE*log2e) recompute):
//   for each K/V tile of 64 keys in the workgroup's visible range:
//     S^T  = K * Q^T                         (bf16 MFMA, fp32 accumulate)
//     mask keys outside [i+off-wl, i+off+wr] and beyond seqlen_k (edge tiles)
//     m'   = max(m, rowmax S) when it grew by more than 2^8 in P units, else m
//     alpha = exp2((m - m') * c);  c = scale*log2e
//     P    = exp2(S*c - m'*c)                (rounded to bf16 for the MFMA)
//     l    = alpha*l + rowsum P;  O = alpha*O + P*V
//   O /= l;  LSE = m*scale + ln(l);  rows with no visible key: O = 0, LSE = -inf.
// Keeping a stale running max (the sm_120 PR page notes FA4's rescale
// threshold: the max may lag by a few log2 units) changes no result: O and l
// carry the same factor, and P stays below 2^8, far inside fp32/bf16 range.
//
// MI355X mapping:
//   * 4 waves x 32 packed query rows; rows fold the r = Hq/Hkv query heads of
//     one KV head into the row index (row = pos*r + head offset), so each K/V
//     tile serves all of them (interface page `pack_gqa`; sm_120 PR page's
//     qhead-into-seqlen fold).
//   * Both GEMMs transposed (attn_common.hpp): one lane owns one query.
//   * K and V tiles are row-major in LDS with 16-byte chunks XOR-swizzled by
//     key (swz_key); global loads are fully coalesced (16 lanes per 256-byte
//     row) and the 16-byte LDS stores, the K fragment reads and the
//     transposing V fragment reads (ds_read_b64_tr_b16) are bank-conflict
//     free.
//   * Double-buffered LDS, next tile prefetched into registers during the
//     current tile's math; one barrier per tile. D = 64/128 fit two waves per
//     SIMD (two workgroups per CU), so one wave's softmax overlaps another's
//     MFMAs.
//   * Few VALU instructions outside the softmax itself: the tile loop is
//     unrolled by two so both LDS buffers sit at compile-time offsets, every
//     fragment address is a per-lane constant plus an immediate, and K/V rows
//     are fetched with buffer loads whose descriptor ends at seqlen_k (rows
//     past it read as zero, no clamping).
//   * Tiles wholly outside the causal/window band are never visited.
//   * Grid order: heaviest (latest) query blocks first, KV head fastest, so
//     round-robin placement keeps each KV head's K/V in a fixed subset of the
//     8 XCD L2s.
#include <climits>
#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

template <int D>
struct FwdCfg {
  static constexpr int BM = kFwdBlockM;      // 128 rows, 4 waves
  static constexpr int BN = kFwdBlockN;      // 64 keys
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPL = 64 / CPR;       // rows one wave instruction covers
  static constexpr int NCH = BN * CPR / 256; // chunks per thread per tensor
  static constexpr int TILE_B = BN * D * 2;  // bytes per K (or V) tile
  static constexpr int WAVES_PER_EU = D <= 128 ? 2 : 1;
  static constexpr float RESCALE_LOG2 = 8.0f;  // lazy-rescale threshold
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WAVES_PER_EU)))
void fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int BM = C::BM, BN = C::BN, CPR = C::CPR, RPL = C::RPL, NCH = C::NCH;
  constexpr int TILE_B = C::TILE_B;
  constexpr int ROW_B = D * 2;  // bytes per tile row
  // K0 V0 K1 V1
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item (heavy query blocks first; see fwd_work_item)
  int hk, b, mb;
  if (!fwd_work_item<BM>(a, hk, b, mb)) return;

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
  sq = uniform(sq);
  sk = uniform(sk);
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
  const int pos_min = uniform(row0 / r);
  const int pos_max = uniform((min(row0 + BM, rows) - 1) / r);
  const int kv_lo = a.wl >= 0 ? max(0, pos_min + off - a.wl) : 0;
  const int kv_hi = a.wr >= 0 ? min(sk, pos_max + off + a.wr + 1) : sk;  // exclusive
  const int n_begin = uniform(kv_lo / BN);
  const int n_end = uniform(kv_hi > kv_lo ? (kv_hi + BN - 1) / BN : n_begin);
  // a tile [n0, n0+BN) is fully visible to every row iff
  //   n0 + BN <= sk, n0 + BN - 1 <= pos_min + off + wr, n0 >= pos_max + off - wl
  const int full_hi = a.wr >= 0 ? pos_min + off + a.wr : INT_MAX / 2;
  const int full_lo = a.wl >= 0 ? pos_max + off - a.wl : INT_MIN / 2;

  // ---- Q^T fragments (B operand), kept in registers for the whole loop.
  // Branch-free: invalid lanes read row 0 of head hk*r and zero it (a load
  // under a divergent branch makes later waits drain every outstanding load).
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

  // ---- K/V staging. Wave instruction u covers RPL whole rows, CPR lanes per
  // row (chunk ld_c = lane % CPR); row & 7 does not depend on u, so each
  // lane's LDS store offset is one constant plus an immediate per u.
  const __bf16* kp = static_cast<const __bf16*>(a.k) + k_base + (int64_t)hk * a.k_hs;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + v_base + (int64_t)hk * a.v_hs;
  const int ld_c = lane % CPR;
  const int ld_r = wave * RPL + lane / CPR;  // row within each 4*RPL-row slice u
  const uint32_t koff = (uint32_t)(ld_r * a.k_rs * 2 + ld_c * 16);
  const uint32_t voff = (uint32_t)(ld_r * a.v_rs * 2 + ld_c * 16);
  const int st_off = ld_r * ROW_B + ((ld_c ^ swz_key(ld_r)) * 16);
  uint4 kreg[NCH], vreg[NCH];

  // One buffer descriptor per slice u (rows n0 + 4*RPL*u ..), ending at the
  // last row before seqlen_k: rows past it read as zero. Descriptors live in
  // scalar registers; each lane keeps a single byte offset per tensor.
  auto load_tile = [&](int n0) {
    const int nrows = min(sk - n0, BN);  // >= 1
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int r0 = u * 4 * RPL;
      const int left = nrows - r0;
      const uint32_t kn = left > 0 ? (uint32_t)((left - 1) * a.k_rs * 2 + ROW_B) : 0u;
      const uint32_t vn = left > 0 ? (uint32_t)((left - 1) * a.v_rs * 2 + ROW_B) : 0u;
      kreg[u] = buf_ld16(make_rsrc(kp + (int64_t)(n0 + r0) * a.k_rs, kn), koff);
      vreg[u] = buf_ld16(make_rsrc(vp + (int64_t)(n0 + r0) * a.v_rs, vn), voff);
    }
  };
  auto store_tile = [&](auto buf_c) {
    constexpr int KB = decltype(buf_c)::value * 2 * TILE_B;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      *reinterpret_cast<uint4*>(smem + KB + st_off + u * 4 * RPL * ROW_B) = kreg[u];
      *reinterpret_cast<uint4*>(smem + KB + TILE_B + st_off + u * 4 * RPL * ROW_B) = vreg[u];
    }
  };

  // ---- fragment read offsets (bytes): a per-lane constant + an immediate.
  // K (A operand of S^T): row kb*32 + c32, chunk 2*cc + half. With f = swz
  // of the row (same for both 32-row blocks), the chunk lands at
  // 8*(cc>>2) + ((2*(cc&3) + half) ^ f): four lane patterns.
  const int fk = swz_key(c32);
  int k_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_rd[i] = c32 * ROW_B + (((2 * i + half) ^ fk) * 16);
  // V (A operand of O^T, transposing read): 16-lane group g reads 4 keys x 16
  // dims; lane j points at key 4*half + j/4 (+16t, +8 part), dims
  // 16*(g&1) + 4*(j&3) of d-block db: chunk 4*db + 2*(g&1) + (j&3)/2, lands
  // at 8*(db>>1) + ((4*(db&1) + chunk%4) ^ f): two lane patterns.
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

  // one tile: compute from LDS buffer `buf`, store the prefetched next tile
  // into the other buffer, barrier
  auto step = [&](int nb, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr int KB = buf * 2 * TILE_B;
    constexpr int VB = KB + TILE_B;
    const int n0 = nb * BN;
    const bool more = nb + 1 < n_end;
    if (more) load_tile(n0 + BN);

    // S^T = K Q^T: two 32-key blocks. Matrix phases run at raised wave
    // priority so the SIMD keeps issuing this wave's MFMAs while the other
    // resident wave's softmax fills the vector-ALU slots.
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            smem + KB + kb * 32 * ROW_B + (cc >> 2) * 128 + k_rd[cc & 3]);
        s[kb] = mfma32(kf, qf[cc], s[kb]);
      }
    }

    __builtin_amdgcn_s_setprio(0);
    const bool full = (n0 + BN <= sk) && (n0 + BN - 1 <= full_hi) && (n0 >= full_lo);
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

    // online softmax with a lazily updated running max; the max and the row
    // sum run on two and four independent chains
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
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s[kb][v], c, -ms));
        s[kb][v] = p;
        rs[v & 3] += p;
      }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);

    // P^T fragments: MFMA t covers keys 16t..16t+15 of the tile; lane half h
    // supplies keys {16t+4h+j, 16t+8+4h+j : j<4}; the V^T fragment below uses
    // the same key order, so the contraction is unchanged.
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1;
      const int i0 = 2 * (t & 1);
      pf[t] = cat(cvt4(s[kb][4 * i0 + 0], s[kb][4 * i0 + 1], s[kb][4 * i0 + 2], s[kb][4 * i0 + 3]),
                  cvt4(s[kb][4 * i0 + 4], s[kb][4 * i0 + 5], s[kb][4 * i0 + 6], s[kb][4 * i0 + 7]));
    }

    // O^T += V^T P^T, V^T fragments read transposed from row-major V
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const char* vb = smem + VB + (16 * t) * ROW_B + (db >> 1) * 128 + v_rd[db & 1];
        const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(vb));
        const bf16x4 v1 = ds_read_tr16(reinterpret_cast<const __bf16*>(vb + 8 * ROW_B));
        o[db] = mfma32(cat(v0, v1), pf[t], o[db]);
      }
    }

    __builtin_amdgcn_s_setprio(0);
    if (more) store_tile(std::integral_constant<int, buf ^ 1>{});
    lds_barrier();  // next buffer written; this buffer free for reuse
  };

  if (n_begin < n_end) {
    load_tile(n_begin * BN);
    store_tile(std::integral_constant<int, 0>{});
    lds_barrier();
  }
  for (int nb = n_begin; nb < n_end; nb += 2) {
    step(nb, std::integral_constant<int, 0>{});
    if (nb + 1 < n_end) step(nb + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store
  const float l_tot = pair_sum(l_run);
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

// head_dim 64/128 run the eight-wave ping-pong kernel (fwd_pp_kernel.hip);
// head_dim 256 needs all 512 registers of a lane for one wave's accumulators,
// so it runs this four-wave kernel at one wave per SIMD.
template <int D>
hipError_t launch_fwd(const FwdArgs& args, hipStream_t s) {
  if constexpr (D <= 128) {
    return launch_fwd_pp<D>(args, s);
  } else {
    return launch_fwd_sp<D, 1>(args, s);
  }
}

template hipError_t launch_fwd<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<128>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<256>(const FwdArgs&, hipStream_t);

}  // namespace mi_attn
