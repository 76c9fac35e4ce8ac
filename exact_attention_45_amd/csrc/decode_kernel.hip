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
#include <climits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace mi_attn {

template <int D>
struct DecTile {
  static constexpr int BN = kDecBlockN;   // 128 keys per tile
  static constexpr int KS = D + 8;
  static constexpr int VS = BN + 4;
  static constexpr int CPR = D / 8;
  static constexpr int NCH = BN * CPR / 256;
  static constexpr int LDS_TILE = BN * KS + D * VS;      // elements (bf16)
  static constexpr int LDS_MERGE = 4 * D * 32 + 4 * 64;  // floats: O^T per wave + m, l
  static constexpr int LDS_BYTES =
      (LDS_TILE * 2 > LDS_MERGE * 4) ? LDS_TILE * 2 : LDS_MERGE * 4;
};

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a) {
  using T = DecTile<D>;
  constexpr int BN = T::BN, KS = T::KS, VS = T::VS, NCH = T::NCH;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS_BYTES];
  __bf16* sK = reinterpret_cast<__bf16*>(smem);
  __bf16* sV = sK + BN * KS;

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
  sk = min(max(sk, 0), cap);
  // the query sits at position sk - 1; a left window keeps the last wl+1 keys
  const int kv_lo = a.wl >= 0 ? max(0, sk - 1 - a.wl) : 0;
  const int span = max(0, sk - kv_lo);
  int chunk = (span + a.num_splits - 1) / a.num_splits;
  chunk = (chunk + BN - 1) / BN * BN;
  const int k_begin = min(sk, kv_lo + split * chunk);
  const int k_end = min(sk, k_begin + chunk);

  // ---- this lane's query head
  const int col = rb * 32 + c32;
  const bool valid = col < a.group;
  const int hq = hk * a.group + (valid ? col : 0);
  const __bf16* qp = static_cast<const __bf16*>(a.q) + (int64_t)b * a.q_bs + (int64_t)hq * a.q_hs;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = valid ? as_bf16x8(ld16(qp + 16 * c + 8 * half)) : zero_bf16x8();

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero_f32x16();
  float m_run = kNegInf;
  float l_run = 0.0f;

  const __bf16* kc = static_cast<const __bf16*>(a.k_cache);
  const __bf16* vc = static_cast<const __bf16*>(a.v_cache);
  const int64_t tok_stride = (int64_t)a.hkv * D;
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  uint4 kreg[NCH], vreg[NCH];

  // each wave instruction moves 32 key rows x 2 chunks; 4 row groups of 32
  auto chunk_row = [&](int u) { return ((u * 4 + wave) & 3) * 32 + c32; };
  auto chunk_col = [&](int u) { return (((u * 4 + wave) >> 2) * 2 + half) * 8; };

  auto load_tile = [&](int n0) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int key = n0 + chunk_row(u);
      const int cc = chunk_col(u);
      kreg[u] = make_uint4(0, 0, 0, 0);
      vreg[u] = make_uint4(0, 0, 0, 0);
      if (key < k_end) {
        const int page = ptab[key / a.page_size];
        if (page >= 0 && page < a.num_pages) {
          const int64_t off =
              ((int64_t)page * a.page_size + key % a.page_size) * tok_stride + (int64_t)hk * D + cc;
          kreg[u] = ld16(kc + off);
          vreg[u] = ld16(vc + off);
        } else {
          bad_page = true;
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int row = chunk_row(u);
      const int cc = chunk_col(u);
      *reinterpret_cast<uint4*>(&sK[row * KS + cc]) = kreg[u];
      const bf16x8 vv = as_bf16x8(vreg[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sV[(cc + e) * VS + row] = vv[e];
    }
  };

  const float c = a.scale_log2;
  if (k_begin < k_end) load_tile(k_begin);
  for (int n0 = k_begin; n0 < k_end; n0 += BN) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (n0 + BN < k_end) load_tile(n0 + BN);

    // this wave's 32 keys: S^T = K Q^T
    f32x16 s = zero_f32x16();
    const __bf16* krow = &sK[(wave * 32 + c32) * KS + 8 * half];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc)
      s = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * cc), qf[cc], s);

    if (n0 + BN > k_end) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = n0 + wave * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (key >= k_end) s[v] = kNegInf;
      }
    }

    float mt = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[v]);
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(m_run, mt);
    const float ms = (m_new == kNegInf) ? 0.0f : m_new * c;
    // exactly 1 when the max did not move (m_run - m_new == 0), exactly 0
    // when nothing was visible before (m_run = -inf)
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
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

    bf16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i0 = 2 * t;
      pf[t] = cat(cvt4(s[4 * i0 + 0], s[4 * i0 + 1], s[4 * i0 + 2], s[4 * i0 + 3]),
                  cvt4(s[4 * i0 + 4], s[4 * i0 + 5], s[4 * i0 + 6], s[4 * i0 + 7]));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const __bf16* vrow = &sV[(db * 32 + c32) * VS + wave * 32 + 4 * half];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + 16 * t);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + 16 * t + 8);
        o[db] = mfma32(cat(v0, v1), pf[t], o[db]);
      }
    }
  }

  // ---- merge the four waves' partial states through LDS
  const float l_wave = l_run + xor32(l_run);
  const int any_bad = __syncthreads_or(bad_page ? 1 : 0);
  float* sO = reinterpret_cast<float*>(smem);          // [wave][d][32]
  float* sM = sO + 4 * D * 32;                          // [wave][32]
  float* sL = sM + 4 * 32;                              // [wave][32]
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int d = db * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      sO[(wave * D + d) * 32 + c32] = o[db][v];
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
  const int hcol = rb * 32 + qcol;
  if (hcol < a.group) {
    const int hq2 = hk * a.group + hcol;
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
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float nan = __builtin_nanf("");
    const int64_t prow = (int64_t)b * a.hq + hq2;
    float* op = a.o_part + (prow * a.num_splits + split) * D;
#pragma unroll 4
    for (int j = 0; j < DPT; ++j) {
      const int d = dpart * DPT + j;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += wgt[w] * sO[(w * D + d) * 32 + qcol];
      op[d] = any_bad ? nan : acc * inv;
    }
    if (dpart == 0) {
      const float lse = l > 0.0f ? m * a.scale + __logf(l) : kNegInf;
      a.lse_part[prow * a.num_splits + split] = any_bad ? nan : lse;
    }
  }
}

// ---- combine: one wave per output row, head_dim / 64 elements per lane
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int S = a.num_splits;
  const float* lp = a.lse_part + (int64_t)row * S;
  const float* op = a.o_part + (int64_t)row * S * D;

  float m = kNegInf;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lp[s]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) m = fmaxf(m, __shfl_xor(m, w, 64));
  // a NaN partial (bad page id) must reach the output
  int has_nan = 0;
  for (int s = lane; s < S; s += 64) has_nan |= (lp[s] != lp[s]);
  has_nan = __any(has_nan);

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  float lse = kNegInf;
  if (m != kNegInf && !has_nan) {
    float tot = 0.0f;
    for (int s = 0; s < S; ++s) tot += __expf(lp[s] - m);
    lse = m + __logf(tot);
    for (int s = 0; s < S; ++s) {
      const float w = __expf(lp[s] - lse);
      const float* src = op + (int64_t)s * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += w * src[e];
    }
  } else if (has_nan) {
    lse = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = lse;
  }
  __bf16* dst = static_cast<__bf16*>(a.out) + (int64_t)row * a.out_row_stride + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = (__bf16)acc[e];
  if (lane == 0 && a.lse != nullptr) a.lse[row] = lse;
}

template <int D>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.batch * a.hkv * a.row_blocks * a.num_splits;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_decode<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<128>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<256>(const DecodeArgs&, hipStream_t);
template hipError_t launch_combine<64>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<128>(const CombineArgs&, hipStream_t);
template hipError_t launch_combine<256>(const CombineArgs&, hipStream_t);

}  // namespace mi_attn
