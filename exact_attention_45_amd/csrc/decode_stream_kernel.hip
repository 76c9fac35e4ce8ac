// Split-KV decode over a paged K/V cache: per-wave streaming variant, used
// when every aligned 32-key slice lies inside one page (page_size a multiple
// of 32), at every head dim (96 and 192 in the LDS layouts of 128 and 256).
//
// Same method as decode_kernel.hip (split-K decoding page, triton_splitk.py
// `FwOp.apply`; interface page, the num_splits path of `_flash_attn_fwd`):
// each split writes a normalised fp32 partial O_s and its LSE_s, and the
// combine kernel merges them by LSE weights. What differs is how the bytes
// move. Decode reads every K/V byte once, so the kernel is a streaming
// kernel whose speed is the number of bytes it keeps in flight:
//   * A workgroup (4 waves) owns one (sequence, 32-head row block, split)
//     for four consecutive KV heads, one head per wave. The heads of a token
//     share its cache row (Hkv x D x 2 bytes), so the four waves read whole
//     rows between them at about the same time. Each wave streams the whole
//     split for its head: the split's keys cut into 32-key slices aligned to
//     absolute key multiples of 32, one running (max, sum, O), and at the end
//     it writes its normalised partial straight from registers. The waves
//     never synchronise.
//   * K and V of a slice are loaded into registers with 16-byte loads in row
//     order, every lane a chunk of the cache (at D = 128 each instruction
//     reads four whole 256-byte rows: measured on
//     MI355X, reading a head's rows this way streams at ~6.5 TB/s, while the
//     MFMA-fragment order, 32 rows x 32 bytes per instruction, manages ~3.9).
//     Both go to a wave-private LDS slot just before use; K is read back as
//     MFMA fragments, V with transposing reads. NS register sets per wave: a
//     set is refilled with slice i+NS as soon as slice i has moved to LDS, so
//     NS slices (16 KB each at D = 128) stay requested while slice i is
//     computed (registers, not LDS, are the large buffer here: a wave may
//     hold 512 of them). The loads are marked non-temporal: the cache is
//     read once per step.
//   * The slot loop is unrolled NS times so every register set is named at
//     compile time and the compiler derives each load-count wait itself.
//   * A slice sits in one page, so its page id is one scalar load and its K
//     and V rows are reached through one buffer descriptor per tensor whose
//     bound ends at the last key before seqused_k: rows past it read as zero.
//   * A page id outside [0, num_pages), or a seqused_k outside [0, capacity],
//     is never dereferenced and turns the split's partial into NaN.
//   * fp8 cache (KV = 1 e4m3, 2 e5m2; sm_120 PR page, fp8 KV-cache decode:
//     OCP e4m3 / e5m2 K/V with a per-(batch, KV head) k_descale / v_descale and
//     bf16 compute):
//     a row is head_dim bytes, so a 16-byte load covers twice the keys and a
//     slice half the bytes. Staging converts each byte to bf16 (exact: e4m3
//     values are bf16 values) into the same LDS layout, so the fragment reads,
//     MFMAs and softmax are those of the bf16 path. k_descale multiplies the
//     score scale (S = scale * ks * q.k8); v_descale multiplies the
//     normalised partial (O = vs * sum p v8).
#include <climits>
#include <type_traits>
#include <utility>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

template <int D, int KV>
struct StreamCfg {
  static constexpr bool FP8 = KV != 0;
  // D = 96 and 192 keep LDS rows of 128 and 256 columns (the swizzles below
  // permute chunks within 256-byte windows); their padding columns are never
  // written or read: the loads cover only the cache's chunks, and the
  // fragment reads only the first D columns
  static constexpr int DL = D == 192 ? 256 : (D == 96 ? 128 : D);
  // K/V register sets per wave. fp8 slices carry half the bytes, yet more
  // fp8 sets in flight measured slower on the B16 Sk32768 workload (split +
  // combine: 2 sets 86.0-87.3 us, 3 sets 87.3-88.5, 4 sets 101, 5 sets 115);
  // bf16 measured the same with 2 or 3. A bf16 set at D = 256 is 128
  // registers (32 KB per slice), next to O's 128 and Q's 64: one set; at
  // D = 192 a second set (96 registers) spilled and ran 43% slower. At D = 96
  // a fourth set measured no faster than three.
  static constexpr int NS = DL == 256 ? 1 : (FP8 ? 2 : 3);
  static constexpr float RESCALE_LOG2 = 8.0f;   // lazy-rescale threshold
  static constexpr int SLICE = 32;              // keys per slice
  static constexpr int ROW_B = DL * 2;          // bytes per bf16 K/V row (LDS)
  static constexpr int SLICE_B = SLICE * ROW_B; // bytes per K (or V) slice in LDS
  static constexpr int GROW_B = FP8 ? D : D * 2; // bytes per K/V row in the cache
  static constexpr int CPR = GROW_B / 16;       // 16-byte chunks per cache row
  // loads: chunk f = 64 u + lane of the slice's SLICE x CPR chunks (row
  // f / CPR, chunk f % CPR) for instruction u; CPR is even, so NLD
  // instructions cover the slice exactly. The (row, chunk) pattern repeats
  // every P instructions (the odd part of CPR) shifted by R rows.
  static constexpr int NLD = SLICE * CPR / 64;  // load instructions per tensor per slice
  static constexpr int P = CPR / (CPR & -CPR);
  static constexpr int R = 64 / (CPR & -CPR);
  // the K swizzle is a function of key bits 0..3, the V swizzle of bits
  // 0..2: the staging addresses repeat every KP (VP) instructions, shifted by
  // KROWS (VROWS) rows
  static constexpr int KP = P * (R >= 16 ? 1 : 16 / R);
  static constexpr int VP = P * (R >= 8 ? 1 : 8 / R);
  static constexpr int KROWS = KP / P * R, VROWS = VP / P * R;
  static constexpr int SLOT_B = 4 * 2 * SLICE_B; // K and V slots of the four waves
  static constexpr int LDS_B = SLOT_B;
};

// LDS chunk position of logical 16-byte chunk c of V row `key`. The XOR
// spreads the eight keys of a transposing read over distinct bank groups; it
// is an involution, so it also maps a physical position back to its chunk.
template <int D>
__device__ __forceinline__ int vswz(int key, int c) {
  return D >= 128 ? (c ^ ((key & 7) << 1)) : (c ^ ((key & 3) << 1));
}

// The slot loop of one wave over its n_w slices with NS = sizeof...(J)
// register sets: request slices 0..NS-1, then per round, for each set J in
// order, move slice i+J to LDS, refill set J with slice i+J+NS and compute
// slice i+J; the last fewer-than-NS slices sit in sets 0, 1, ...
template <class Issue, class Stage, class Consume, int... J>
__device__ __forceinline__ void stream_slices(int n_w, Issue& issue, Stage& stage, Consume& consume,
                                              std::integer_sequence<int, J...>) {
  constexpr int NS = sizeof...(J);
  (issue(J, std::integral_constant<int, J>{}), ...);
  int i = 0;
  for (; i + NS <= n_w; i += NS)
    ((stage(std::integral_constant<int, J>{}), issue(i + NS + J, std::integral_constant<int, J>{}),
      consume(i + J)),
     ...);
  ((i + J < n_w ? (stage(std::integral_constant<int, J>{}), consume(i + J), 0) : 0), ...);
}

// KV: 0 = bf16 cache, 1 = fp8 e4m3, 2 = fp8 e5m2
template <int D, int KV, bool SC>
__global__ __launch_bounds__(256) void decode_stream_kernel(const DecodeArgs a) {
  constexpr bool FP8 = KV != 0;
  using C = StreamCfg<D, KV>;
  constexpr int NS = C::NS, ROW_B = C::ROW_B, SLICE_B = C::SLICE_B, CPR = C::CPR;
  constexpr int NLD = C::NLD, GROW_B = C::GROW_B, DL = C::DL, P = C::P, R = C::R;
  constexpr int KP = C::KP, VP = C::VP;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int c32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (sequence, 32-head row block, split) for four consecutive
  // KV heads, one per wave; split fastest
  const int n_hg = (a.hkv + 3) / 4;
  int lin = blockIdx.x;
  const int split = lin % a.num_splits;
  lin /= a.num_splits;
  const int hg = lin % n_hg;
  lin /= n_hg;
  const int rb = lin % a.row_blocks;
  const int b = lin / a.row_blocks;
  const int hk = hg * 4 + wave;
  if (hk >= a.hkv) return;  // wave-uniform; the waves never synchronise

  const int cap = a.max_pages * a.page_size;
  int sk = a.seqused_k != nullptr ? a.seqused_k[b] : cap;
  bool bad = sk < 0 || sk > cap;  // would index past the page-table row
  sk = uniform(min(max(sk, 0), cap));
  int t0, n;
  dec_tokens(a, b, t0, n);
  const int rows = n * a.group;
  if (rb * 32 >= rows) return;  // no (token, head) row in this block
  // this lane's row, and the block's first and last rows: their visible keys
  // bound the block's key range and the slices every row sees in full
  const DecRow row = dec_row(a, t0, n, sk, hk, rb, c32);
  const DecRow r_first = dec_row(a, t0, n, sk, hk, rb, 0);
  const DecRow r_last = dec_row(a, t0, n, sk, hk, rb, min(31, rows - 1 - rb * 32));
  const int kv_lo = uniform(r_first.lo);
  const int kv_hi = uniform(max(r_last.hi + 1, kv_lo));  // exclusive
  const int full_lo = uniform(r_last.lo);
  const int full_hi = uniform(r_first.hi);
  // this split's slices [m_lo, m_hi) of the visible ones
  const int m_first = kv_lo / 32;
  const int n_sl = kv_hi > kv_lo ? (kv_hi - 1) / 32 - m_first + 1 : 0;
  const int per = (n_sl + a.num_splits - 1) / a.num_splits;
  const int m_lo = uniform(m_first + min(n_sl, split * per));
  const int m_hi = uniform(m_first + min(n_sl, (split + 1) * per));
  // this wave's slices m_lo + i, i < n_w (all of the split, for its head)
  const int n_w = uniform(m_hi - m_lo);

  // ---- this lane's query row (MFMA B operand)
  const bool valid = row.valid;
  const __bf16* qp = static_cast<const __bf16*>(a.q) + row.token * a.q_bs + (int64_t)row.hq * a.q_hs;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    const bf16x8 x = as_bf16x8(ld16(qp + 16 * cc + 8 * half));
    qf[cc] = valid ? x : zero_bf16x8();
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.0f;
  // fp8: the key descale joins the score scale, the value descale the output
  float kds = 1.0f, vds = 1.0f;
  if constexpr (FP8) {
    if (a.k_descale != nullptr) kds = a.k_descale[(int64_t)b * a.hkv + hk];
    if (a.v_descale != nullptr) vds = a.v_descale[(int64_t)b * a.hkv + hk];
  }
  // a zero key descale makes every score 0 (uniform weights; the constant is
  // kept positive so masked -inf scores still give weight 0); a negative or
  // NaN one has no meaning for a cache scale: this wave's rows get NaN
  bad |= !(kds >= 0.0f);
  const float c = fmaxf(a.scale_log2 * kds, 1e-30f);
  const float rescale_raw = C::RESCALE_LOG2 / c;
  // soft-capping of scale * kds * s (a zero effective scale leaves all scores 0)
  const float sc_eff = a.scale * kds;
  const float sc_k1x = SC && sc_eff != 0.0f ? 2.0f * kLog2e * sc_eff / a.softcap : 0.0f;
  const float sc_k2 = SC && sc_eff != 0.0f ? a.softcap / sc_eff : 0.0f;

  // ---- slice addressing
  const int64_t ts2 = (int64_t)a.hkv * GROW_B;  // bytes between consecutive tokens
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)hk * GROW_B;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)hk * GROW_B;
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  // loads: instruction u = P q + p reads chunk ld_c[p] of slice row
  // ld_r[p] + R q (this lane's chunk f = 64 u + lane, see StreamCfg)
  int ld_r[P], ld_c[P];
  uint32_t ld_off[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    ld_r[p] = (64 * p + lane) / CPR;
    ld_c[p] = (64 * p + lane) % CPR;
    ld_off[p] = (uint32_t)(ld_r[p] * ts2 + ld_c[p] * 16);
  }
  // K slot: chunk c of row r at position c ^ kswz(r), conflict-free for the
  // fragment reads (16 lanes read one logical chunk of 16 consecutive keys:
  // 16 distinct positions within a 256-byte bank window at D >= 128, whose
  // rows are whole multiples of it); V slot: chunk c at vswz(r, c), for the
  // transposing reads
  auto kswz = [](int key) {
    return DL >= 128 ? (((key & 3) << 1) | ((key >> 2) & 1) | (((key >> 3) & 1) << 3)) : ((key >> 1) & 7);
  };
  char* kslot = smem + wave * 2 * SLICE_B;
  char* vslot = kslot + SLICE_B;
  // staging address of load u: k_st[u % KP] + (u / KP) KROWS rows, and
  // v_st[u % VP] + (u / VP) VROWS rows
  int k_st[KP], v_st[VP];
#pragma unroll
  for (int p = 0; p < KP; ++p) {
    const int row = ld_r[p % P] + R * (p / P);
    const int ch = ld_c[p % P];
    k_st[p] = row * ROW_B + ((ch ^ kswz(row)) * 16);
    if (p < VP) v_st[p] = row * ROW_B + vswz<DL>(row, ch) * 16;
  }
  const int fk = kswz(c32);
  // fragment cc reads chunk 2*cc + half; kswz only moves chunks within a
  // 256-byte window (16 chunks), so fragments cc and cc + 8 differ by 256
  // bytes and eight address registers serve D = 192 and 256
  constexpr int NKR = D / 16 < 8 ? D / 16 : 8;
  int k_rd[NKR];
#pragma unroll
  for (int cc = 0; cc < NKR; ++cc) k_rd[cc] = c32 * ROW_B + (((2 * cc + half) ^ fk) * 16);

  uint4 kreg[NS][NLD];
  uint4 vreg[NS][NLD];
  // request slice i of this wave into register set `slot` (compile time)
  auto issue = [&](int i, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int m = m_lo + i;
    const int key0 = 32 * m;
    const int nvalid = (i < n_w) ? min(32, sk - key0) : 0;
    const int pidx = min(key0 / a.page_size, a.max_pages - 1);
    int page = nvalid > 0 ? ptab[pidx] : 0;
    const bool ok = page >= 0 && page < a.num_pages;
    bad |= !ok;
    page = ok ? page : 0;
    const int64_t row0 = (int64_t)page * a.page_size + key0 % a.page_size;
    const uint32_t nrec = nvalid > 0 && ok ? (uint32_t)((nvalid - 1) * ts2 + GROW_B) : 0u;
    const auto kr = make_rsrc(kbase + row0 * ts2, nrec);
    const auto vr = make_rsrc(vbase + row0 * ts2, nrec);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      kreg[slot][u] = buf_ld16_nt(kr, ld_off[u % P] + (uint32_t)(R * (u / P) * ts2));
      vreg[slot][u] = buf_ld16_nt(vr, ld_off[u % P] + (uint32_t)(R * (u / P) * ts2));
    }
  };

  // transposing V reads: lane j of 16-lane group g points at key j/4
  const int tr_g = lane >> 4;
  const int tr_j = lane & 15;
  const int tr_key = tr_j >> 2;
  const int tr_c = (tr_g & 1) * 2 + ((tr_j & 3) >> 1);
  const int tr_e = (tr_j & 1) * 8;
  // a transposing read of keys k = 16 tt + v_key (+ 8) at chunk 4 db + tr_c:
  // vswz depends on key bits 0..2 only, which the offsets 16 tt and 8 keep,
  // and moves chunks within a 16-chunk window, so d-blocks db and db + 4
  // differ by 256 bytes: NVR address registers serve every (db, tt)
  const int v_key = 4 * half + tr_key;
  constexpr int NVR = D / 32 < 4 ? D / 32 : 4;
  int v_rd[NVR];
#pragma unroll
  for (int j = 0; j < NVR; ++j) v_rd[j] = v_key * ROW_B + vswz<DL>(v_key, 4 * j + tr_c) * 16 + tr_e;

  // K and V rows of register set `slot` into this wave's LDS slots (LDS
  // operations of one wave complete in order, so the previous slice's reads
  // are done first); the set is free for the next request afterwards
  auto stage = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    if constexpr (!FP8) {
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        *reinterpret_cast<uint4*>(kslot + k_st[u % KP] + (u / KP) * C::KROWS * ROW_B) = kreg[slot][u];
        *reinterpret_cast<uint4*>(vslot + v_st[u % VP] + (u / VP) * C::VROWS * ROW_B) = vreg[slot][u];
      }
    } else {
      // 16 fp8 values = dims 16 ch .. +15 of the load's row: bf16 chunks
      // 2 ch and 2 ch + 1 of that row, each at its swizzled place
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int row = ld_r[u % P] + R * (u / P);
        const int ch = ld_c[u % P];
        const uint4 kx = kreg[slot][u], vx = vreg[slot][u];
        const uint2 k0 = fp8x4_to_bf16x4<KV == 2>(kx.x), k1 = fp8x4_to_bf16x4<KV == 2>(kx.y);
        const uint2 k2 = fp8x4_to_bf16x4<KV == 2>(kx.z), k3 = fp8x4_to_bf16x4<KV == 2>(kx.w);
        const uint2 v0 = fp8x4_to_bf16x4<KV == 2>(vx.x), v1 = fp8x4_to_bf16x4<KV == 2>(vx.y);
        const uint2 v2 = fp8x4_to_bf16x4<KV == 2>(vx.z), v3 = fp8x4_to_bf16x4<KV == 2>(vx.w);
        char* kr = kslot + row * ROW_B;
        char* vr = vslot + row * ROW_B;
        *reinterpret_cast<uint4*>(kr + (((2 * ch) ^ kswz(row)) * 16)) = make_uint4(k0.x, k0.y, k1.x, k1.y);
        *reinterpret_cast<uint4*>(kr + (((2 * ch + 1) ^ kswz(row)) * 16)) = make_uint4(k2.x, k2.y, k3.x, k3.y);
        *reinterpret_cast<uint4*>(vr + vswz<DL>(row, 2 * ch) * 16) = make_uint4(v0.x, v0.y, v1.x, v1.y);
        *reinterpret_cast<uint4*>(vr + vswz<DL>(row, 2 * ch + 1) * 16) = make_uint4(v2.x, v2.y, v3.x, v3.y);
      }
    }
  };

  // compute slice i from the LDS slots
  auto consume = [&](int i) {
    const char* vs = vslot;
    f32x16 s = zero_f32x16();
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
      s = mfma32(*reinterpret_cast<const bf16x8*>(kslot + k_rd[cc % NKR] + (cc / NKR) * 256), qf[cc], s);
    if constexpr (SC) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = softcap_raw(s[v], sc_k1x, sc_k2);
    }
    // keys outside the row's [lo, hi] (first and last slices, and padding)
    const int key0 = 32 * (m_lo + i);
    if (i >= n_w || key0 < full_lo || key0 + 31 > full_hi) [[unlikely]] {
      const uint32_t w = (uint32_t)vis64(row.lo - key0 - 4 * half, row.hi - key0 - 4 * half);
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = mask_by_bit(s[v], i < n_w ? w : 0u, 8 * (v >> 2) + (v & 3));
    }
    float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
      m0 = vmax3(m0, s[v], s[v + 1]);
      m1 = vmax3(m1, s[v + 2], s[v + 3]);
    }
    const float mt = pair_max(vmax(m0, m1));
    // lazy rescale (as in the prefill kernels): the running max moves only
    // when a slice max exceeds it by more than 2^RESCALE_LOG2 in exp2 units,
    // so the O accumulators (which live in accumulation registers that vector
    // arithmetic must copy out and back) are rarely touched; alpha is exactly
    // 1 for lanes whose max stays
    const bool grow = (m_run == kNegInf) ? (mt != kNegInf) : (mt - m_run > rescale_raw);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_run;
      const float alpha = grow ? ((m_run == kNegInf) ? 0.0f : fast_exp2((m_run - m_new) * c)) : 1.0f;
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
    for (int v = 0; v < 16; ++v) {
      s[v] = fast_exp2(fmaf(s[v], c, -ms));
      rs[v & 3] += s[v];
    }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    bf16x8 pf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int i0 = 2 * tt;
      pf[tt] = cat(cvt4(s[4 * i0 + 0], s[4 * i0 + 1], s[4 * i0 + 2], s[4 * i0 + 3]),
                   cvt4(s[4 * i0 + 4], s[4 * i0 + 5], s[4 * i0 + 6], s[4 * i0 + 7]));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        // keys 16 tt + v_key and that + 8, chunk 4 db + tr_c (see v_rd)
        const char* p = vs + v_rd[db % NVR] + (db / NVR) * 256 + 16 * tt * ROW_B;
        const bf16x4 v0 = ds_read_tr16(reinterpret_cast<const __bf16*>(p));
        const bf16x4 v1 = ds_read_tr16(reinterpret_cast<const __bf16*>(p + 8 * ROW_B));
        o[db] = mfma32(cat(v0, v1), pf[tt], o[db]);
      }
    }
  };

  // NS slices stay requested while one is computed; requests past the last
  // slice load nothing (zero-length descriptor). The slot loop is unrolled NS
  // times (a fold over the slots) so every register set is named at compile
  // time.
  if (n_w > 0) stream_slices(n_w, issue, stage, consume, std::make_integer_sequence<int, NS>{});
  // the last requests (past the end, all-zero rows) must land before the
  // workgroup's registers and LDS are released
  __builtin_amdgcn_s_waitcnt(0);

  // ---- this wave owns its head's whole split: normalise and write the
  // partial straight from registers (lane: query column c32, head dims
  // 32*db + 8*i + 4*half .. +3)
  const float l_tot = pair_sum(l_run);
  if (valid) {
    const float inv = l_tot > 0.0f ? vds / l_tot : 0.0f;
    const float nan = __builtin_nanf("");
    const int64_t prow = row.prow;
    float* op = a.o_part + (prow * a.num_splits + split) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * half;
        *reinterpret_cast<float4*>(op + d0) =
            bad ? make_float4(nan, nan, nan, nan)
                : make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                              o[db][4 * i + 3] * inv);
      }
    if (half == 0) {
      const float lse = l_tot > 0.0f ? m_run * (a.scale * kds) + __logf(l_tot) : kNegInf;
      a.lse_part[prow * a.num_splits + split] = bad ? nan : lse;
    }
  }
}

template <int D, int KV>
hipError_t launch_stream(const DecodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.batch * ((a.hkv + 3) / 4) * a.row_blocks * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((decode_stream_kernel<D, KV, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<D, KV, false>), dim3((unsigned)grid), dim3(256), 0, s,
                       a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t s) {
  return launch_stream<D, 0>(a, s);
}
template <int D>
hipError_t launch_decode_stream_fp8(const DecodeArgs& a, hipStream_t s) {
  return a.kv_fp8 == 2 ? launch_stream<D, 2>(a, s) : launch_stream<D, 1>(a, s);
}

template hipError_t launch_decode_stream<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream<96>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream<128>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream<192>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream<256>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream_fp8<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream_fp8<96>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream_fp8<128>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream_fp8<192>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode_stream_fp8<256>(const DecodeArgs&, hipStream_t);

}  // namespace mi_attn
