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
  // Paged K/V (page_table non-NULL): k/v point at the caches, k_bs/v_bs are
  // the page strides, cu_k is NULL, sequence b has seqused_k[b] keys (or
  // max_pages * page_size), page_size is a multiple of the 64-key tile.
  const int32_t* page_table;
  const int32_t* seqused_k;
  int32_t page_size, num_pages, max_pages;
  const __bf16* sink;  // learnable-sink logits [hq], or NULL
  // Logit soft-capping (softcap > 0): raw scores s become
  // softcap_raw(s, sc_k1x, sc_k2), i.e. scale * s -> cap * tanh(scale * s / cap)
  float softcap;
  float sc_k1x, sc_k2;
};

// Query blocks (of BM packed rows) a prefill launch covers per KV head.
// Dense batches: every sequence has num_m_blocks of them. Packed varlen
// batches: the sum over sequences of ceil(rows_b / BM) is at most
// total_rows / BM + batch, so the grid holds about as many workgroups as
// there are real blocks (not num_m_blocks per sequence).
inline int64_t fwd_blocks_per_head(const FwdArgs& a, int bm) {
  const int64_t dense = (int64_t)a.num_m_blocks * a.batch;
  if (a.cu_q == nullptr) return dense;
  const int64_t packed = ((int64_t)a.total_q * a.group + bm - 1) / bm + a.batch;
  return packed < dense ? packed : dense;
}

// Sequence bounds a packed varlen launch reads for its work item: query
// tokens [q0, q1) and, with cu_k, key tokens [k0, k1); `used` is seqused_k[b]
// (paged caches). Fields whose array is NULL are left 0.
struct FwdSeq {
  int q0, q1, k0, k1, used;
};

// Inclusive prefix sum over the 64 lanes of a wave (DPP: shifts within each
// 16-lane row, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Work item (KV head hk, sequence b, query block mb) of prefill workgroup
// blockIdx.x. Dense batches: heavy (late) query blocks first, (KV head,
// sequence) fastest. Packed varlen batches: KV head fastest, then block g of
// the concatenation of every sequence's blocks, each sequence's last
// (heaviest) block first. The search takes 64 sequences per step, one per
// lane: each lane loads its sequence's bounds (cu_q, and cu_k / seqused_k
// when given; all loads of a step issued together, one memory latency), the
// block counts are prefix-summed across the wave, and the first lane whose
// running total passes g holds the sequence; its bounds come back in `seq`.
// Returns false for a workgroup past the last block.
template <int BM>
__device__ __forceinline__ bool fwd_work_item(const FwdArgs& a, int& hk, int& b, int& mb,
                                              FwdSeq& seq) {
  // every quantity here is the same in all lanes: keep it in scalar registers
  const auto scalar = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int lin = (int)blockIdx.x;
  seq = FwdSeq{0, 0, 0, 0, 0};
  if (a.cu_q == nullptr) {
    const int nhb = a.hkv * a.batch;
    const int hb = scalar(lin % nhb);
    mb = scalar(a.num_m_blocks - 1 - lin / nhb);
    hk = scalar(hb % a.hkv);
    b = scalar(hb / a.hkv);
    return true;
  }
  hk = scalar(lin % a.hkv);
  int g = scalar(lin / a.hkv);
  const int lane = (int)(threadIdx.x & 63);
  for (int j0 = 0; j0 < a.batch; j0 += 64) {
    const int j = j0 + lane;
    const int ja = min(j, a.batch), jb = min(j + 1, a.batch);
    const int q0 = a.cu_q[ja], q1 = a.cu_q[jb];
    const int k0 = a.cu_k != nullptr ? a.cu_k[ja] : 0;
    const int k1 = a.cu_k != nullptr ? a.cu_k[jb] : 0;
    const int used = a.seqused_k != nullptr ? a.seqused_k[min(j, a.batch - 1)] : 0;
    const int len = q1 - q0;  // 0 past the last sequence
    const int nb = len > 0 ? (int)(((int64_t)len * a.group + BM - 1) / BM) : 0;
    const int incl = wave_incl_sum(nb);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > g);
    if (hit != 0) {
      const int l = scalar(__builtin_ctzll(hit));
      b = scalar(j0 + l);
      mb = scalar(__builtin_amdgcn_readlane(incl, l) - 1 - g);
      seq.q0 = scalar(__builtin_amdgcn_readlane(q0, l));
      seq.q1 = scalar(__builtin_amdgcn_readlane(q1, l));
      seq.k0 = scalar(__builtin_amdgcn_readlane(k0, l));
      seq.k1 = scalar(__builtin_amdgcn_readlane(k1, l));
      seq.used = scalar(__builtin_amdgcn_readlane(used, l));
      return true;
    }
    g -= scalar(__builtin_amdgcn_readlane(incl, 63));
  }
  return false;
}

// Keys of sequence b and the element offset of its K/V rows from a.k / a.v
// for a prefill launch: packed (cu_k), paged (rows are located per tile, so
// the base is 0) or dense. A paged sequence's key count is clamped to the
// capacity of its page-table row, so no page lookup leaves that row.
// PAGED is a compile-time copy of (a.page_table != nullptr): the dense
// kernels carry no paging code.
template <bool PAGED>
__device__ __forceinline__ void fwd_kv_extent(const FwdArgs& a, int b, const FwdSeq& seq, int& sk,
                                              int64_t& k_base, int64_t& v_base) {
  if constexpr (PAGED) {
    const int cap = a.max_pages * a.page_size;
    const int used = a.seqused_k == nullptr ? cap : a.cu_q != nullptr ? seq.used : a.seqused_k[b];
    sk = min(max(used, 0), cap);
    k_base = 0;
    v_base = 0;
  } else if (a.cu_k != nullptr) {
    sk = seq.k1 - seq.k0;
    k_base = (int64_t)seq.k0 * a.k_rs;
    v_base = (int64_t)seq.k0 * a.v_rs;
  } else {
    sk = a.seqlen_k;
    k_base = (int64_t)b * a.k_bs;
    v_base = (int64_t)b * a.v_bs;
  }
}

// Row offsets (elements from the sequence's K/V base) of the key tile that
// starts at key n0: contiguous rows, or for a paged cache the page that holds
// key n0 (page_table row b, entry n0 / page_size; a tile never straddles a
// page) plus the slot within it.
template <bool PAGED>
__device__ __forceinline__ void fwd_tile_rows(const FwdArgs& a, int b, int n0, int64_t& k_off,
                                              int64_t& v_off) {
  if constexpr (PAGED) {
    const int pi = n0 / a.page_size;
    const int pid = __builtin_amdgcn_readfirstlane(a.page_table[(int64_t)b * a.max_pages + pi]);
    const int slot = n0 - pi * a.page_size;
    k_off = (int64_t)pid * a.k_bs + (int64_t)slot * a.k_rs;
    v_off = (int64_t)pid * a.v_bs + (int64_t)slot * a.v_rs;
  } else {
    k_off = (int64_t)n0 * a.k_rs;
    v_off = (int64_t)n0 * a.v_rs;
  }
}

// For a paged cache: true when any page id covering keys [k_lo, k_hi) of
// sequence b lies outside [0, num_pages). Each lane checks every 64th page;
// the answer is the same in every wave of the workgroup.
template <bool PAGED>
__device__ __forceinline__ bool fwd_bad_pages(const FwdArgs& a, int b, int k_lo, int k_hi,
                                              int lane) {
  if constexpr (!PAGED) return false;
  if (k_hi <= k_lo) return false;
  const int p_lo = k_lo / a.page_size, p_hi = (k_hi - 1) / a.page_size;
  bool bad = false;
  for (int pi = p_lo + lane; pi <= p_hi; pi += 64) {
    const int pid = a.page_table[(int64_t)b * a.max_pages + pi];
    bad = bad || (unsigned)pid >= (unsigned)a.num_pages;
  }
  return __builtin_amdgcn_ballot_w64(bad) != 0;
}

// Paged split-KV decode arguments.
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* page_table;
  const int32_t* seqused_k;  // may be NULL
  float* o_part;             // [rows][splits][d], rows = query tokens * hq
  float* lse_part;           // [rows][splits]
  int64_t q_bs, q_hs;        // q_bs: between sequences, or between tokens with cu_q
  int32_t batch, hq, hkv, group;
  int32_t page_size, num_pages, max_pages;
  int32_t num_splits;
  int32_t row_blocks;        // ceil(max query tokens * group / 32)
  float scale;
  float scale_log2;
  int32_t wl, wr;            // < 0 unbounded (causal folded into wr = 0)
  // Packed query tokens (cu_q non-NULL): sequence b owns tokens
  // [cu_q[b], cu_q[b+1]) of q, aligned bottom-right to its keys; NULL: one
  // query token per sequence.
  const int32_t* cu_q;
  // fp8 cache (1 = OCP e4m3, 2 = OCP e5m2; 0 = bf16): one byte per element,
  // real value = descale[b][kv head] * decoded byte; descales NULL = 1
  int32_t kv_fp8;
  const float* k_descale;    // [batch][hkv] or NULL
  const float* v_descale;
  float softcap;  // > 0: logit soft-capping of scale * s (per-head descale included)
};

// The decode row of one lane: query column `col` (0..31) of row block rb of
// (sequence b, KV head hk). Rows fold the query tokens of the sequence and
// the group query heads of the KV head (row = token * group + head offset,
// as the prefill packs GQA rows). The row's query sits at key position
// sk - n + t (t its token within the sequence, n the sequence's tokens:
// bottom-right alignment) and sees keys [lo, hi]; hi < lo means none.
struct DecRow {
  bool valid;     // a real (token, head) row
  int hq;         // query head
  int64_t token;  // query token (sequence index b when one token per sequence)
  int64_t prow;   // partial / output row: token * hq_total + hq
  int lo, hi;     // visible keys
};

// Query tokens of sequence b ([t0, t0 + n)): packed by cu_q, or one token b.
__device__ __forceinline__ void dec_tokens(const DecodeArgs& a, int b, int& t0, int& n) {
  if (a.cu_q != nullptr) {
    t0 = __builtin_amdgcn_readfirstlane(a.cu_q[b]);
    n = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]) - t0;
  } else {
    t0 = b;
    n = 1;
  }
}

__device__ __forceinline__ DecRow dec_row(const DecodeArgs& a, int t0, int n, int sk, int hk,
                                          int rb, int col) {
  DecRow r;
  const int rows = n * a.group;
  const int rho0 = rb * 32 + col;
  r.valid = rho0 < rows;
  const int rho = r.valid ? rho0 : max(rows - 1, 0);  // invalid lanes: the last row's values
  const int t = rho / a.group;
  r.hq = hk * a.group + (rho - t * a.group);
  r.token = (int64_t)t0 + t;
  r.prow = r.token * a.hq + r.hq;
  const int p = sk - n + t;
  r.lo = a.wl >= 0 ? max(0, p - a.wl) : 0;
  r.hi = a.wr >= 0 ? min(p + a.wr, sk - 1) : sk - 1;
  return r;
}

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  void* out;
  int64_t out_row_stride;
  float* lse;
  int32_t rows, num_splits;
  const __bf16* sink;  // learnable-sink logits [hq] (row = b * hq + h), or NULL
  int32_t hq;
};

constexpr int kFwdBlockM = 128;   // packed query rows per workgroup (4 waves x 32), D = 256
constexpr int kFwdPPBlockM = 256; // ping-pong kernel, D = 64/128 (8 waves x 32)
constexpr int kFwdBlockN = 64;    // keys per K/V tile
constexpr int kDecBlockN = 128;   // keys per decode tile (4 waves x 32)

// The per-wave streaming decode kernel serves every head dim when each
// aligned 32-key slice lies in one page (page_size a multiple of 32); the
// tile kernel serves the other page sizes.
constexpr bool decode_streams(int head_dim, int page_size) {
  (void)head_dim;
  return page_size % 32 == 0;
}

template <int D> hipError_t launch_fwd_pp(const FwdArgs& a, hipStream_t s);
template <int D, int QB> hipError_t launch_fwd_sp(const FwdArgs& a, hipStream_t s);

// Prefill forward (launch_fwd): fused exact attention, dispatch by head dim.
//
// Method (mslk flash_attn interface.py page, `_flash_attn_fwd`; the online
// softmax in the exp2 domain with scale*log2(e) folded into one FMA, as the
// flash_bwd_sm100.py page's P = exp2(S*scale_log2 - LSE*log2e) recompute):
//   for each K/V tile of keys in the workgroup's visible range:
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
// MI355X mapping shared by both kernels:
//   * rows fold the r = Hq/Hkv query heads of one KV head into the row index
//     (row = pos*r + head offset), so each K/V tile serves all of them
//     (interface page `pack_gqa`; sm_120 PR page's qhead-into-seqlen fold);
//   * both GEMMs transposed (attn_common.hpp): one lane owns one query;
//   * K and V tiles row-major in LDS with XOR-swizzled 16-byte chunks, filled
//     by direct-to-LDS buffer loads whose descriptor ends at seqlen_k (rows
//     past it read as zero);
//   * with a paged K/V cache (interface page, page_table branch) a 64-key tile
//     lies in one page (page_size is a multiple of 64), so the tile's
//     descriptor is based at page_table[b][n0 / page_size] * page stride +
//     (n0 % page_size) rows; a workgroup first checks every page id it will
//     read and writes NaN instead when one is outside [0, num_pages). Paging
//     is a template parameter: the dense kernels carry none of it;
//   * tiles wholly outside the causal/window band are never visited;
//   * grid order: heaviest (latest) query blocks first, KV head fastest, so
//     round-robin placement keeps each KV head's K/V in a fixed subset of the
//     8 XCD L2s.
//
// head_dim 64/128: eight-wave ping-pong kernel (fwd_pp_kernel.hip), two waves
// per SIMD, one running its softmax while the other issues MFMAs.
// head_dim 256: the O accumulators alone take 128 registers per lane, so one
// wave per SIMD, software-pipelined inside the wave (fwd_sp_kernel.hip).
template <int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if constexpr (D <= 128)
    return launch_fwd_pp<D>(a, s);
  else
    return launch_fwd_sp<D, 1>(a, s);
}

template <int D> hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
template <int D> hipError_t launch_decode_stream(const DecodeArgs& a, hipStream_t s);
template <int D> hipError_t launch_decode_stream_fp8(const DecodeArgs& a, hipStream_t s);
template <int D> hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace mi_attn
