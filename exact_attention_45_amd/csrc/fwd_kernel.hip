// Prefill forward: fused exact attention, dispatch by head dim.
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
#include "kernels.hpp"

namespace mi_attn {

template <int D>
hipError_t launch_fwd(const FwdArgs& args, hipStream_t s) {
  if constexpr (D <= 128) {
    return launch_fwd_pp<D>(args, s);
  } else {
    return launch_fwd_sp<D, 1>(args, s);
  }
}

template hipError_t launch_fwd<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<96>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<128>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<192>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<256>(const FwdArgs&, hipStream_t);

}  // namespace mi_attn
