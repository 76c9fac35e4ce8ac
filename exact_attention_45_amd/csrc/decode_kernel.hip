// Split-KV decode over a paged K/V cache, and the LSE-weighted combine.
//
// Method (split-K decoding page, triton_splitk.py `FwOp.apply`: fp32 split
// partials then `merge_attentions`; interface page, the num_splits path of
// `_flash_attn_fwd` followed by `_flash_attn_fwd_combine`):
//   split s of sequence b covers a contiguous key range; for it compute
//     O_s = softmax(scale * q K_s^T) V_s (normalised), LSE_s = log sum exp(...)
//   then combine: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
// An empty split has LSE_s = -inf and O_s = 0 and drops out of the combine.
//
// MI355X mapping of the split kernel (decode is HBM-bound: each K/V byte is
// used for r = Hq/Hkv query heads only):
//   * One workgroup per (sequence, KV head, 32-head row block, split). The r
//     query heads sharing the KV head are the MFMA's query columns (GQA
//     packing), padded to 32.
//   * 256 threads stream 128-key tiles through LDS with 16-byte loads,
//     prefetching the next tile into registers during the current tile's
//     math; each page row of one KV head is head_dim*2 contiguous bytes.
//   * Each wave takes its own 32 keys of the tile, keeps its own running
//     (max, sum, O), and the four waves merge through LDS at the end, so a
//     split writes exactly one normalised partial per query head.
//   * Page ids are looked up per key row; an id outside [0, num_pages) is
//     never dereferenced and turns the split's partial into NaN.
//   * fp8 caches (KV = 1 e4m3, 2 e5m2; sm_120 PR page, fp8 KV-cache decode):
//     each lane loads the 8 bytes of its 8-element chunk, and the register
//     set is widened to bf16 (exactly) when it is stored to LDS, so tiles,
//     fragments and MFMAs are the bf16 path's. k_descale joins the score
//     scale (S = scale * ks * q.k8), v_descale the normalised partial
//     (O = vs * sum p v8), as in the streaming kernel.
#include <climits>
#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

template <int D>
struct DecCfg {
  static constexpr int BN = kDecBlockN;              // 128 keys per tile, 32 per wave
  static constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  static constexpr int ROWS_PER_LD = 64 / CPR;       // rows one wave instruction covers
  static constexpr int NCH = BN * CPR / 256;         // chunks per thread per tensor
  static constexpr int TILE = BN * D;                // elements per K (or V) tile
  static constexpr int NBUF = D <= 128 ? 2 : 1;      // LDS tile buffers
  static constexpr int NSET = D <= 128 ? 2 : 1;      // register prefetch sets
  static constexpr int LDS_TILES = NBUF * 2 * TILE * 2;          // bytes
  static constexpr int LDS_MERGE = (4 * D * 32 + 4 * 64) * 4;    // bytes
  static constexpr int LDS_BYTES = LDS_TILES > LDS_MERGE ? LDS_TILES : LDS_MERGE;
};

template <int D>
__device__ __forceinline__ int dswz(int key, int c) {
  return D >= 128 ? (c ^ ((key & 7) << 1)) : (c ^ ((key & 3) << 1));
}

// Head dims 96 and 192 run at the next power-of-two width DP (128, 256):
// the LDS tiles, fragments and accumulators have DP columns, the chunks
// past D are zero (never loaded: their lanes re-read chunk 0 of the row,
// a line the same instruction fetches anyway, and drop it), so the scores
// and the first D output columns are those of width D; only those are
// stored.
template <int D>
constexpr int dec_width() {
  return D == 96 ? 128 : (D == 192 ? 256 : D);
}

template <int D, int KV>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a) {
  constexpr bool FP8 = KV != 0;
  using Raw = std::conditional_t<FP8, uint2, uint4>;  // one lane's chunk as loaded
  constexpr int DP = dec_width<D>();
  using C = DecCfg<DP>;
  constexpr int BN = C::BN, CPR = C::CPR, NCH = C::NCH, TILE = C::TILE;
  constexpr int NBUF = C::NBUF, NSET = C::NSET;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
  __bf16* tiles = reinterpret_cast<__bf16*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: split fastest, then row block, KV head, sequence
  int lin = blockIdx.x;
  const int split = lin % a.num_splits;
  lin /= a.num_splits;
  const int rb = lin % a.row_blocks;
  lin /= a.row_blocks;
  const int hk = lin % a.hkv;
  const int b = lin / a.hkv;

  const int cap = a.max_pages * a.page_size;
  int sk = a.seqused_k != nullptr ? a.seqused_k[b] : cap;
  // a length outside [0, capacity] would index past the page-table row
  bool bad_page = sk < 0 || sk > cap;
  sk = __builtin_amdgcn_readfirstlane(min(max(sk, 0), cap));
  int t0, n;
  dec_tokens(a, b, t0, n);
  const int rows = n * a.group;
  if (rb * 32 >= rows) return;  // no (token, head) row in this block (uniform)
  // this lane's row, and the block's first and last rows: their visible keys
  // bound the block's key range and the tiles every row sees in full
  const DecRow row = dec_row(a, t0, n, sk, hk, rb, c32);
  const DecRow r_first = dec_row(a, t0, n, sk, hk, rb, 0);
  const DecRow r_last = dec_row(a, t0, n, sk, hk, rb, min(31, rows - 1 - rb * 32));
  const int kv_lo = __builtin_amdgcn_readfirstlane(r_first.lo);
  const int kv_hi = __builtin_amdgcn_readfirstlane(max(r_last.hi + 1, kv_lo));  // exclusive
  const int full_lo = __builtin_amdgcn_readfirstlane(r_last.lo);
  const int full_hi = __builtin_amdgcn_readfirstlane(r_first.hi);
  const int span = max(0, kv_hi - kv_lo);
  int chunk = (span + a.num_splits - 1) / a.num_splits;
  chunk = (chunk + BN - 1) / BN * BN;
  const int k_begin = min(kv_hi, kv_lo + split * chunk);
  const int k_end = min(kv_hi, k_begin + chunk);
  const int n_tiles = (k_end - k_begin + BN - 1) / BN;

  // ---- this lane's query row
  const bool valid = row.valid;
  const __bf16* qp = static_cast<const __bf16*>(a.q) + row.token * a.q_bs + (int64_t)row.hq * a.q_hs;
  // branch-free: invalid lanes read head 0's row and zero it afterwards (a
  // load under a divergent branch makes every later wait drain all loads)
  bf16x8 qf[DP / 16];
#pragma unroll
  for (int c = 0; c < DP / 16; ++c) {
    const int e0 = 16 * c + 8 * half;  // columns past D (padding) are zero
    const bf16x8 x = as_bf16x8(ld16(qp + (e0 < D ? e0 : 0)));
    qf[c] = valid && e0 < D ? x : zero_bf16x8();
  }

  f32x16 o[DP / 32];
#pragma unroll
  for (int i = 0; i < DP / 32; ++i) o[i] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.0f;

  // element offsets; an element is 2 bytes (bf16) or 1 (fp8)
  constexpr int EB = FP8 ? 1 : 2;
  const char* kc = static_cast<const char*>(a.k_cache) + (int64_t)hk * D * EB;
  const char* vc = static_cast<const char*>(a.v_cache) + (int64_t)hk * D * EB;
  const int64_t tok_stride = (int64_t)a.hkv * D;
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int ld_c = lane % CPR;
  const int ld_r = lane / CPR;
  const bool ld_in = ld_c < D / 8;  // a chunk of the row (not padding)
  const int ld_off = (ld_in ? ld_c : 0) * 8;

  // Register prefetch sets. Page ids of tile t+1 are requested before the
  // K/V loads of tile t: load counters retire in issue order, so a page id
  // requested after a tile's loads could not be used until that tile landed.
  Raw kreg[NSET][NCH], vreg[NSET][NCH];
  int pid[2][NCH];  // by tile parity

  auto tile_row = [&](int u) { return (u * 4 + wave) * C::ROWS_PER_LD + ld_r; };
  // Loads are branch-free per lane (divergent branches around loads make the
  // compiler drain every outstanding load): a key past the split end is
  // clamped to the last key (its scores are masked), and a page id outside
  // the cache is replaced by page 0 and flags the split as NaN. Only the
  // wave-uniform `t < n_tiles` test skips work.
  // slot = t & 1 (compile-time at every call site). Requests for tiles past
  // the split's end are still issued, so every wait count in the loop is
  // static; their keys clamp to the split's last key (a cached row whose
  // page id its own tile already checks), and their scores are masked.
  auto fetch_pages = [&](int t, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int key = min(k_begin + t * BN + tile_row(u), k_end - 1);
      pid[slot][u] = ptab[key / a.page_size];
    }
  };
  auto load_tile = [&](int t, auto set_c, auto slot_c) {
    constexpr int set = decltype(set_c)::value;
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int key = min(k_begin + t * BN + tile_row(u), k_end - 1);
      const bool ok = pid[slot][u] >= 0 && pid[slot][u] < a.num_pages;
      bad_page |= !ok;
      const int page = ok ? pid[slot][u] : 0;
      const int64_t off =
          ((int64_t)page * a.page_size + key % a.page_size) * tok_stride + ld_off;
      // the cache is read once per step
      if constexpr (FP8) {
        const uint2 kx = ld8_nt(kc + off), vx = ld8_nt(vc + off);
        kreg[set][u] = ld_in ? kx : make_uint2(0u, 0u);
        vreg[set][u] = ld_in ? vx : make_uint2(0u, 0u);
      } else {
        const uint4 kx = ld16_nt(kc + 2 * off), vx = ld16_nt(vc + 2 * off);
        kreg[set][u] = ld_in ? kx : make_uint4(0u, 0u, 0u, 0u);
        vreg[set][u] = ld_in ? vx : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](auto set_c, int buf) {
    constexpr int set = decltype(set_c)::value;
    __bf16* sK = tiles + buf * 2 * TILE;
    __bf16* sV = sK + TILE;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int row = tile_row(u);
      const int p = row * DP + dswz<DP>(row, ld_c) * 8;
      if constexpr (FP8) {
        const uint2 k0 = fp8x4_to_bf16x4<KV == 2>(kreg[set][u].x);
        const uint2 k1 = fp8x4_to_bf16x4<KV == 2>(kreg[set][u].y);
        const uint2 v0 = fp8x4_to_bf16x4<KV == 2>(vreg[set][u].x);
        const uint2 v1 = fp8x4_to_bf16x4<KV == 2>(vreg[set][u].y);
        *reinterpret_cast<uint4*>(&sK[p]) = make_uint4(k0.x, k0.y, k1.x, k1.y);
        *reinterpret_cast<uint4*>(&sV[p]) = make_uint4(v0.x, v0.y, v1.x, v1.y);
      } else {
        *reinterpret_cast<uint4*>(&sK[p]) = kreg[set][u];
        *reinterpret_cast<uint4*>(&sV[p]) = vreg[set][u];
      }
    }
  };

  // transposing V fragment reads: lane j of 16-lane group g points at key j/4
  const int tr_g = lane >> 4;
  const int tr_j = lane & 15;
  const int tr_key = tr_j >> 2;
  const int tr_c = (tr_g & 1) * 2 + ((tr_j & 3) >> 1);
  const int tr_e = (tr_j & 1) * 4;
  // fp8: the key descale joins the score scale, the value descale the output;
  // a zero key descale makes every score 0 (uniform weights), a negative or
  // NaN one turns the split's partial into NaN
  float kds = 1.0f, vds = 1.0f;
  if constexpr (FP8) {
    if (a.k_descale != nullptr) kds = a.k_descale[(int64_t)b * a.hkv + hk];
    if (a.v_descale != nullptr) vds = a.v_descale[(int64_t)b * a.hkv + hk];
    bad_page |= !(kds >= 0.0f);
  }
  const float c = FP8 ? fmaxf(a.scale_log2 * kds, 1e-30f) : a.scale_log2;
  // soft-capping of scale * kds * s (a zero effective scale leaves all scores 0)
  const float sc_eff = a.scale * kds;
  const float sc_k1x = a.softcap > 0.0f && sc_eff != 0.0f ? 2.0f * kLog2e * sc_eff / a.softcap : 0.0f;
  const float sc_k2 = a.softcap > 0.0f && sc_eff != 0.0f ? a.softcap / sc_eff : 0.0f;

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, NSET == 2 ? 1 : 0>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using PN = std::integral_constant<int, NSET & 1>;         // slot of tile NSET
  using PN1 = std::integral_constant<int, (NSET + 1) & 1>;  // slot of tile NSET+1

  // Issue order: pages(t+1) before loads(t); loads(t) before store(t).
  // Prologue: tile 0 in LDS, tiles 1..NSET in flight.
  if (n_tiles > 0) {
    fetch_pages(0, P0{});
    fetch_pages(1, P1{});
    load_tile(0, S0{}, P0{});
    if (NSET == 2) {
      fetch_pages(2, P0{});
      load_tile(1, S1{}, P1{});
    }
    fetch_pages(NSET + 1, PN1{});
    store_tile(S0{}, 0);
    load_tile(NSET, S0{}, PN{});
    lds_barrier();
  }

  // one tile; `par` = t & 1 as a compile-time constant (register set and
  // LDS buffer of tile t when double-buffered)
  auto step = [&](int t, auto par_c) {
    constexpr int par = decltype(par_c)::value;
    using SetNext = std::integral_constant<int, NSET == 2 ? (par ^ 1) : 0>;
    using SlotLoad = std::integral_constant<int, (par + 1 + NSET) & 1>;   // tile t+1+NSET
    using SlotFetch = std::integral_constant<int, (par + NSET) & 1>;      // tile t+2+NSET
    const int buf = NBUF == 2 ? par : 0;
    const __bf16* sK = tiles + buf * 2 * TILE;
    const __bf16* sV = sK + TILE;
    const int n0 = k_begin + t * BN;

    // this wave's 32 keys: S^T = K Q^T
    f32x16 s = zero_f32x16();
    {
      const int key = wave * 32 + c32;
      const __bf16* krow = sK + key * DP;
#pragma unroll
      for (int cc = 0; cc < DP / 16; ++cc)
        s = mfma32(*reinterpret_cast<const bf16x8*>(krow + dswz<DP>(key, 2 * cc + half) * 8),
                   qf[cc], s);
    }
    if (a.softcap > 0.0f) {  // uniform
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = softcap_raw(s[v], sc_k1x, sc_k2);
    }
    // keys past the split's end or outside the row's [lo, hi]
    if (n0 + BN > k_end || n0 < full_lo || n0 + BN - 1 > full_hi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = n0 + wave * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (key >= k_end || key < row.lo || key > row.hi) s[v] = kNegInf;
      }
    }

    float mt = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; v += 2) mt = vmax3(mt, s[v], s[v + 1]);
    mt = pair_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float ms = (m_new == kNegInf) ? 0.0f : m_new * c;
    // exactly 1 when the max did not move, exactly 0 when nothing was seen
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2((m_run - m_new) * c);
    float rs = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(fmaf(s[v], c, -ms));
      s[v] = p;
      rs += p;
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DP / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

    bf16x8 pf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int i0 = 2 * tt;
      pf[tt] = cat(cvt4(s[4 * i0 + 0], s[4 * i0 + 1], s[4 * i0 + 2], s[4 * i0 + 3]),
                   cvt4(s[4 * i0 + 4], s[4 * i0 + 5], s[4 * i0 + 6], s[4 * i0 + 7]));
    }
#pragma unroll
    for (int db = 0; db < DP / 32; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int k0 = wave * 32 + 16 * tt + 4 * half + tr_key;
        const int k1 = k0 + 8;
        const int cc = 4 * db + tr_c;
        const bf16x4 v0 = ds_read_tr16(sV + k0 * DP + dswz<DP>(k0, cc) * 8 + tr_e);
        const bf16x4 v1 = ds_read_tr16(sV + k1 * DP + dswz<DP>(k1, cc) * 8 + tr_e);
        o[db] = mfma32(cat(v0, v1), pf[tt], o[db]);
      }
    }

    // unconditional (a past-the-end tile stores finite filler that is never
    // read unmasked), so the compiler sees fixed load counts in the loop
    if (NBUF == 1) lds_barrier();  // single buffer: everyone done reading
    store_tile(SetNext{}, NBUF == 2 ? (par ^ 1) : 0);
    lds_barrier();
    // page ids two tiles ahead, then refill the drained register set
    fetch_pages(t + 2 + NSET, SlotFetch{});
    load_tile(t + 1 + NSET, SetNext{}, SlotLoad{});
  };
  // Steps run in pairs; with an odd tile count the last step covers keys
  // >= k_end only, all masked, and leaves (m, l, O) unchanged.
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the four waves' partial states through LDS
  const float l_wave = pair_sum(l_run);
  const int any_bad = __syncthreads_or(bad_page ? 1 : 0);
  float* sO = reinterpret_cast<float*>(smem);          // [wave][d][32]
  float* sM = sO + 4 * DP * 32;                         // [wave][32]
  float* sL = sM + 4 * 32;                              // [wave][32]
#pragma unroll
  for (int db = 0; db < DP / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int d = db * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      sO[(wave * DP + d) * 32 + c32] = o[db][v];
    }
  if (half == 0) {
    sM[wave * 32 + c32] = m_run;
    sL[wave * 32 + c32] = l_wave;
  }
  __syncthreads();

  // thread -> (query column, slice of head_dim)
  const int qcol = tid & 31;
  const int dpart = tid >> 5;  // 0..7
  constexpr int DPT = D / 8;
  const DecRow mrow = dec_row(a, t0, n, sk, hk, rb, qcol);
  if (mrow.valid) {
    float mw[4], m = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = sM[w * 32 + qcol];
      m = fmaxf(m, mw[w]);
    }
    float wgt[4], l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = (m == kNegInf) ? 0.0f : fast_exp2((mw[w] - m) * c);
      l += wgt[w] * sL[w * 32 + qcol];
    }
    const float inv = l > 0.0f ? vds / l : 0.0f;
    const float nan = __builtin_nanf("");
    const int64_t prow = mrow.prow;
    float* op = a.o_part + (prow * a.num_splits + split) * D + dpart * DPT;
#pragma unroll
    for (int j = 0; j < DPT; j += 4) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = dpart * DPT + j;
        acc.x += wgt[w] * sO[(w * DP + d + 0) * 32 + qcol];
        acc.y += wgt[w] * sO[(w * DP + d + 1) * 32 + qcol];
        acc.z += wgt[w] * sO[(w * DP + d + 2) * 32 + qcol];
        acc.w += wgt[w] * sO[(w * DP + d + 3) * 32 + qcol];
      }
      *reinterpret_cast<float4*>(op + j) =
          any_bad ? make_float4(nan, nan, nan, nan)
                  : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (dpart == 0) {
      const float lse = l > 0.0f ? m * sc_eff + __logf(l) : kNegInf;
      a.lse_part[prow * a.num_splits + split] = any_bad ? nan : lse;
    }
  }
}

// ---- combine: one 64-lane workgroup per output row. The first 16 splits'
// partial rows are requested together with the split LSEs, so a step with
// at most 16 splits waits for memory once; larger split counts stream in
// chunks of 16 with the next chunk requested before the current one is
// summed. Split weights go through LDS (zero past the last split, so the
// clamped loads of a ragged last chunk add nothing).
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const CombineArgs a) {
  // head_dim elements per lane: D / 64, or D / 48 for D = 96 and 192 (whole
  // 8- or 16-byte vectors; the first 48 lanes carry the row, the others
  // re-read lane 47's and store nothing)
  constexpr int EPL = (D == 96 || D == 192) ? D / 48 : D / 64;
  constexpr int LANES = D / EPL;
  static_assert(LANES * EPL == D && (EPL == 1 || EPL == 2 || EPL == 4), "row split over lanes");
  constexpr int CH = 16;       // splits per chunk
  typedef float vecE __attribute__((ext_vector_type(EPL)));
  __shared__ float sw[256 + CH];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int S = a.num_splits;
  const float* lp = a.lse_part + (int64_t)row * S;
  const float* op = a.o_part + (int64_t)row * S * D + min(lane, LANES - 1) * EPL;
  auto load_chunk = [&](int s0, vecE (&x)[CH]) {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      x[i] = *reinterpret_cast<const vecE*>(op + (int64_t)min(s0 + i, S - 1) * D);
  };

  // straight-line code up to the sum, so that the compiler issues every
  // load before the first wait
  float xl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sj = lane + 64 * j;
    const float v = lp[min(sj, S - 1)];
    xl[j] = sj < S ? v : kNegInf;
  }
  vecE x[CH];
  load_chunk(0, x);

  float m = kNegInf;
  int has_nan = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = fmaxf(m, xl[j]);
    has_nan |= (xl[j] != xl[j]);
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) m = fmaxf(m, __shfl_xor(m, w, 64));
  has_nan = __any(has_nan);
  const float mm = m == kNegInf ? 0.0f : m;
  float tot = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float w = __expf(xl[j] - mm);  // -inf (empty or absent split) -> 0
    sw[lane + 64 * j] = w;
    tot += w;
  }
  if (lane < CH) sw[256 + lane] = 0.0f;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) tot += __shfl_xor(tot, w, 64);
  __syncthreads();
  vecE acc = {};
  for (int s0 = 0; s0 < S; s0 += CH) {
    vecE y[CH];
    const bool more = s0 + CH < S;
    if (more) load_chunk(s0 + CH, y);
#pragma unroll
    for (int i = 0; i < CH; ++i) acc += sw[s0 + i] * x[i];
    if (more) {
#pragma unroll
      for (int i = 0; i < CH; ++i) x[i] = y[i];
    }
  }
  // every split empty: zero output and lse -inf; a NaN partial (bad page
  // id) must reach the output
  float lse = tot > 0.0f ? mm + __logf(tot) : kNegInf;
  float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  if (a.sink != nullptr) {
    float w;
    lse = merge_sink(lse, (float)a.sink[row % a.hq], &w);
    inv *= w;
  }
  acc = acc * inv;
  if (has_nan) {
    lse = __builtin_nanf("");
    acc = lse;
  }
  __bf16* dst = static_cast<__bf16*>(a.out) + (int64_t)row * a.out_row_stride + lane * EPL;
  if (lane < LANES) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = (__bf16)acc[e];
  }
  if (lane == 0 && a.lse != nullptr) a.lse[row] = lse;
}

template <int D>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (decode_streams(D, a.page_size))
    return a.kv_fp8 ? launch_decode_stream_fp8<D>(a, s) : launch_decode_stream<D>(a, s);
  const int64_t grid = (int64_t)a.batch * a.hkv * a.row_blocks * a.num_splits;
  if (grid <= 0) return hipSuccess;
  if (a.kv_fp8 == 2)
    hipLaunchKernelGGL((decode_split_kernel<D, 2>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else if (a.kv_fp8 == 1)
    hipLaunchKernelGGL((decode_split_kernel<D, 1>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, 0>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)a.rows), dim3(64), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_decode<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<96>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<128>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<192>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<256>(const DecodeArgs&, hipStream_t);
template hipError_t launch_combine<64>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<96>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<128>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<192>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<256>(const CombineArgs&, hipStream_t);

}  // namespace mi_attn
