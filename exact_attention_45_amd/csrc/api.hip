// C ABI entry points: argument validation, mask normalisation, launch
// configuration. Every check here runs before any HIP call, so invalid
// requests return an error without touching the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "bwd.hpp"
#include "kernels.hpp"
#include "mi_attn.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MI_ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s) { return s >= 0 && (s % 8) == 0; }
// Head dims of the forward, the decode and the combine (96 and 192 run in the
// LDS layouts of 128 and 256).
bool dim_supported(int d) { return d == 64 || d == 96 || d == 128 || d == 192 || d == 256; }

// Mask normalisation (interface page, `_flash_attn_fwd`): causal forces a
// right window of 0; negative sizes are unbounded.
void normalise_window(int causal, int wl_in, int wr_in, int* wl, int* wr) {
  *wl = wl_in < 0 ? -1 : wl_in;
  *wr = wr_in < 0 ? -1 : wr_in;
  if (causal) *wr = 0;
}

// softmax_scale * log2(e), the factor the kernels apply to raw scores inside
// exp2. A zero scale (every score 0: uniform weights over the visible keys)
// is raised to a tiny positive value: masked scores are -inf, and -inf * 0
// would be NaN where -inf * 1e-30 is -inf (weight 0); visible raw scores
// times 1e-30 round to exactly 0 against the running max, so the weights
// stay exactly uniform. The LSE uses softmax_scale itself.
constexpr float kMinExp2Scale = 1e-30f;
float exp2_scale(float scale) {
  const float c = scale * 1.4426950408889634f;
  return c > kMinExp2Scale ? c : kMinExp2Scale;
}

constexpr size_t kAlign = 256;
constexpr int64_t kFwdRowsPerTile = mi_attn::kFwdBlockN;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Split count when the caller passes 0. Same shape as the interface page's
// `num_splits_heuristic` (no split for <= 4 key blocks; otherwise enough
// splits to give every compute unit work, capped at 128 and at the number
// of key blocks). The streaming kernel runs one wave per (sequence, KV head,
// row block, split) and aims at one wave per SIMD (four per compute unit);
// the tile kernel runs one workgroup per (sequence, KV head, row block,
// split) and aims at two workgroups per compute unit.
// The compute-unit count is that of the gfx950 parts this library is built
// for (MI350X / MI355X: 256), a constant rather than a device query, so the
// split count and the workspace size are pure functions of the parameters
// and sizing makes no HIP call. A partitioned device with fewer units only
// gets more splits than it needs, never a wrong result.
constexpr int kComputeUnits = 256;
// Query tokens per sequence (the maximum), query rows of the launch, and
// 32-row blocks per (sequence, KV head): one token per sequence unless
// cu_seqlens_q packs several.
int decode_max_q(const mi_attn_decode_params* p) {
  return p->cu_seqlens_q != nullptr ? p->max_seqlen_q : 1;
}
size_t decode_rows(const mi_attn_decode_params* p) {
  return (p->cu_seqlens_q != nullptr ? (size_t)p->total_q : (size_t)p->batch) * p->num_heads_q;
}
int decode_row_blocks(const mi_attn_decode_params* p) {
  const int64_t group = p->num_heads_q / p->num_heads_kv;
  return (int)(((int64_t)decode_max_q(p) * group + 31) / 32);
}

int split_heuristic(const mi_attn_decode_params* p) {
  const int cap = p->max_pages_per_seq * p->page_size;
  const int n_blocks = (cap + mi_attn::kDecBlockN - 1) / mi_attn::kDecBlockN;
  if (n_blocks <= 4) return 1;
  const int cus = kComputeUnits;
  const long work = (long)p->batch * p->num_heads_kv * decode_row_blocks(p);
  const long per_cu = mi_attn::decode_streams(p->head_dim, p->page_size) ? 4L : 2L;
  const long want = std::max(1L, (per_cu * cus) / std::max(1L, work));
  return (int)std::max(1L, std::min<long>({want, 128L, (long)n_blocks}));
}

// Shape and scalar checks (enough to size the workspace).
int check_decode(const mi_attn_decode_params* p) {
  if (p == nullptr) return fail(MI_ATTN_EINVAL, "params is NULL");
  if (p->batch < 0 || p->num_heads_q <= 0 || p->num_heads_kv <= 0)
    return fail(MI_ATTN_EINVAL, "batch must be >= 0 and head counts > 0");
  if (p->num_heads_q % p->num_heads_kv != 0)
    return fail(MI_ATTN_EINVAL, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)",
                p->num_heads_q, p->num_heads_kv);
  if (!dim_supported(p->head_dim))
    return fail(MI_ATTN_EUNSUPPORTED, "head_dim %d not supported (64, 96, 128, 192, 256)",
                p->head_dim);
  if (p->page_size <= 0 || p->num_pages <= 0 || p->max_pages_per_seq <= 0)
    return fail(MI_ATTN_EINVAL, "page_size, num_pages and max_pages_per_seq must be > 0");
  if ((int64_t)p->max_pages_per_seq * p->page_size > INT32_MAX)
    return fail(MI_ATTN_EBOUNDS, "max_pages_per_seq * page_size overflows int32");
  if ((int64_t)p->num_pages * p->page_size * p->num_heads_kv * p->head_dim > INT64_MAX / 4)
    return fail(MI_ATTN_EINVAL, "cache too large");
  if (p->num_splits < 0 || p->num_splits > 256)
    return fail(MI_ATTN_EINVAL, "num_splits must be in 0..256 (got %d)", p->num_splits);
  if (!isfinite(p->softmax_scale) || p->softmax_scale < 0.0f)
    return fail(MI_ATTN_EUNSUPPORTED, "softmax_scale must be finite and >= 0");
  if (p->kv_dtype != MI_ATTN_KV_BF16 && p->kv_dtype != MI_ATTN_KV_FP8_E4M3 &&
      p->kv_dtype != MI_ATTN_KV_FP8_E5M2)
    return fail(MI_ATTN_EUNSUPPORTED, "kv_dtype %d not supported (bf16, fp8 e4m3, fp8 e5m2)",
                p->kv_dtype);
  if (!isfinite(p->softcap) || p->softcap < 0.0f)
    return fail(MI_ATTN_EUNSUPPORTED, "softcap must be finite and >= 0 (0: none)");
  if (p->cu_seqlens_q != nullptr) {
    if (p->max_seqlen_q < 0 || p->total_q < 0)
      return fail(MI_ATTN_EINVAL, "max_seqlen_q and total_q must be >= 0 with cu_seqlens_q");
    if ((int64_t)p->max_seqlen_q * (p->num_heads_q / p->num_heads_kv) > INT32_MAX - 32 ||
        (int64_t)p->total_q * p->num_heads_q > INT32_MAX)
      return fail(MI_ATTN_EINVAL, "query tokens * heads overflow int32");
  }
  return MI_ATTN_OK;
}

// Pointer, alignment and stride checks, needed only to launch.
int check_decode_pointers(const mi_attn_decode_params* p) {
  if (decode_rows(p) == 0) return MI_ATTN_OK;
  if (!p->q || !p->k_cache || !p->v_cache || !p->page_table || !p->out)
    return fail(MI_ATTN_EINVAL, "q, k_cache, v_cache, page_table and out must be non-NULL");
  if (!aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->v_cache) || !aligned16(p->out))
    return fail(MI_ATTN_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!stride_ok(p->q_batch_stride) || !stride_ok(p->q_head_stride) ||
      !stride_ok(p->o_batch_stride) || !stride_ok(p->o_head_stride))
    return fail(MI_ATTN_EINVAL, "q/out strides must be non-negative multiples of 8 elements");
  return MI_ATTN_OK;
}

int resolved_splits(const mi_attn_decode_params* p) {
  return p->num_splits > 0 ? p->num_splits : split_heuristic(p);
}

size_t workspace_for(const mi_attn_decode_params* p, int splits) {
  const size_t rows = decode_rows(p);
  return round_up(rows * splits * p->head_dim * sizeof(float)) +
         round_up(rows * splits * sizeof(float));
}

template <class F>
hipError_t by_dim(int d, F&& f) {
  switch (d) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 96: return f(std::integral_constant<int, 96>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 192: return f(std::integral_constant<int, 192>{});
    default: return f(std::integral_constant<int, 256>{});
  }
}


}  // namespace

extern "C" {

const char* mi_attn_last_error(void) { return g_err; }

const char* mi_attn_version(void) { return "mi_attn 0.1.0 gfx950"; }

int mi_attn_fwd(const mi_attn_fwd_params* p, void* stream) {
  if (p == nullptr) return fail(MI_ATTN_EINVAL, "params is NULL");
  const bool paged = p->page_table != nullptr;
  if (paged) {
    // interface page: the page_table branch rejects cu_seqlens_k
    if (p->cu_seqlens_k != nullptr)
      return fail(MI_ATTN_EINVAL, "page_table is not supported with cu_seqlens_k");
    if (p->page_size <= 0 || p->num_pages <= 0 || p->max_pages_per_seq <= 0)
      return fail(MI_ATTN_EINVAL, "page_size, num_pages and max_pages_per_seq must be > 0");
    if (p->page_size % mi_attn::kFwdBlockN != 0)
      return fail(MI_ATTN_EUNSUPPORTED, "page_size %d must be a multiple of %d for the prefill "
                  "forward", p->page_size, mi_attn::kFwdBlockN);
    if ((int64_t)p->page_size * p->max_pages_per_seq > INT32_MAX ||
        (int64_t)p->batch * p->max_pages_per_seq > INT32_MAX)
      return fail(MI_ATTN_EINVAL, "page table too large for 32-bit indexing");
  }
  const bool varlen = p->cu_seqlens_q != nullptr || (!paged && p->cu_seqlens_k != nullptr);
  if (varlen && !paged && (p->cu_seqlens_q == nullptr || p->cu_seqlens_k == nullptr))
    return fail(MI_ATTN_EINVAL, "cu_seqlens_q and cu_seqlens_k must both be given");
  if (p->batch < 0 || p->num_heads_q <= 0 || p->num_heads_kv <= 0)
    return fail(MI_ATTN_EINVAL, "batch must be >= 0 and head counts > 0");
  if (p->num_heads_q % p->num_heads_kv != 0)
    return fail(MI_ATTN_EINVAL, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)",
                p->num_heads_q, p->num_heads_kv);
  if (!dim_supported(p->head_dim))
    return fail(MI_ATTN_EUNSUPPORTED, "head_dim %d not supported (64, 96, 128, 192, 256)",
                p->head_dim);
  if (!isfinite(p->softmax_scale) || p->softmax_scale < 0.0f)
    return fail(MI_ATTN_EUNSUPPORTED, "softmax_scale must be finite and >= 0");
  if (!isfinite(p->softcap) || p->softcap < 0.0f)
    return fail(MI_ATTN_EUNSUPPORTED, "softcap must be finite and >= 0 (0: none)");
  int max_q, max_k;
  if (varlen) {
    if (p->max_seqlen_q < 0 || (!paged && p->max_seqlen_k < 0) || p->total_q < 0)
      return fail(MI_ATTN_EINVAL, "max_seqlen_q/k and total_q must be >= 0 for varlen");
    max_q = p->max_seqlen_q;
    max_k = p->max_seqlen_k;
  } else {
    if (p->seqlen_q < 0 || (!paged && p->seqlen_k < 0))
      return fail(MI_ATTN_EINVAL, "seqlen_q and seqlen_k must be >= 0");
    max_q = p->seqlen_q;
    max_k = p->seqlen_k;
  }
  const int group = p->num_heads_q / p->num_heads_kv;
  if ((int64_t)max_q * group > INT32_MAX - mi_attn::kFwdPPBlockM)
    return fail(MI_ATTN_EINVAL, "seqlen_q * (num_heads_q / num_heads_kv) overflows int32");
  if (p->batch == 0 || max_q == 0) return ok();
  if (!p->q || !p->k || !p->v || !p->out)
    return fail(MI_ATTN_EINVAL, "q, k, v and out must be non-NULL");
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->out))
    return fail(MI_ATTN_EINVAL, "q, k, v and out must be 16-byte aligned");
  const int64_t strides[] = {p->q_row_stride, p->q_head_stride, p->k_row_stride, p->k_head_stride,
                             p->v_row_stride, p->v_head_stride, p->o_row_stride, p->o_head_stride};
  for (int64_t s : strides)
    if (!stride_ok(s))
      return fail(MI_ATTN_EINVAL, "row/head strides must be non-negative multiples of 8");
  if (p->q_row_stride < p->head_dim || p->k_row_stride < p->head_dim ||
      p->v_row_stride < p->head_dim || p->o_row_stride < p->head_dim)
    return fail(MI_ATTN_EINVAL, "row strides must be >= head_dim (rows may not overlap)");
  if ((int64_t)kFwdRowsPerTile * (p->k_row_stride + p->v_row_stride) * 2 > INT32_MAX)
    return fail(MI_ATTN_EINVAL, "K/V row stride too large for 32-bit tile offsets");
  if (!varlen) {
    const int64_t bstr[] = {p->q_batch_stride, p->o_batch_stride};
    for (int64_t s : bstr)
      if (!stride_ok(s))
        return fail(MI_ATTN_EINVAL, "batch strides must be non-negative multiples of 8");
  }
  if (!varlen || paged) {
    // dense: batch strides; paged: page strides
    if (!stride_ok(p->k_batch_stride) || !stride_ok(p->v_batch_stride))
      return fail(MI_ATTN_EINVAL, "K/V batch (or page) strides must be non-negative multiples of 8");
  }
  (void)max_k;

  mi_attn::FwdArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.out = p->out;
  a.lse = p->lse;
  a.q_bs = p->q_batch_stride;
  a.q_rs = p->q_row_stride;
  a.q_hs = p->q_head_stride;
  a.k_bs = p->k_batch_stride;
  a.k_rs = p->k_row_stride;
  a.k_hs = p->k_head_stride;
  a.v_bs = p->v_batch_stride;
  a.v_rs = p->v_row_stride;
  a.v_hs = p->v_head_stride;
  a.o_bs = p->o_batch_stride;
  a.o_rs = p->o_row_stride;
  a.o_hs = p->o_head_stride;
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = paged ? nullptr : p->cu_seqlens_k;
  a.batch = p->batch;
  a.seqlen_q = varlen ? 0 : p->seqlen_q;
  a.seqlen_k = (varlen || paged) ? 0 : p->seqlen_k;
  a.page_table = p->page_table;
  a.seqused_k = paged ? p->seqused_k : nullptr;
  a.page_size = paged ? p->page_size : 0;
  a.num_pages = paged ? p->num_pages : 0;
  a.max_pages = paged ? p->max_pages_per_seq : 0;
  a.sink = static_cast<const __bf16*>(p->learnable_sink);
  // soft-capping; with a zero scale every score is 0 and stays 0
  a.softcap = p->softmax_scale > 0.0f ? p->softcap : 0.0f;
  if (a.softcap > 0.0f) {
    a.sc_k1x = 2.0f * 1.4426950408889634f * p->softmax_scale / a.softcap;
    a.sc_k2 = a.softcap / p->softmax_scale;
  }
  a.hq = p->num_heads_q;
  a.hkv = p->num_heads_kv;
  a.group = group;
  a.total_q = p->total_q;
  a.max_rows = max_q * group;
  a.scale = p->softmax_scale;
  a.scale_log2 = exp2_scale(p->softmax_scale);
  normalise_window(p->causal, p->window_left, p->window_right, &a.wl, &a.wr);
  if (((int64_t)a.max_rows + mi_attn::kFwdBlockM - 1) / mi_attn::kFwdBlockM * a.hkv * a.batch >
      INT32_MAX)
    return fail(MI_ATTN_EINVAL, "launch grid too large");

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = by_dim(p->head_dim, [&](auto dc) {
    return mi_attn::launch_fwd<decltype(dc)::value>(a, s);
  });
  if (e != hipSuccess) return fail(MI_ATTN_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int mi_attn_decode_num_splits(const mi_attn_decode_params* p) {
  int rc = check_decode(p);
  if (rc != MI_ATTN_OK) return rc;
  return resolved_splits(p);
}

size_t mi_attn_decode_workspace_bytes(const mi_attn_decode_params* p) {
  if (check_decode(p) != MI_ATTN_OK) return 0;
  ok();
  return workspace_for(p, resolved_splits(p));
}

}  // extern "C"

// Scratch for mi_attn_decode_splitkv_noalloc: the decode partials live in
// this file-scope device array (one copy per GPU, held until the process
// ends) instead of a caller workspace. Host code never passes `scratch`
// itself (its host-side name is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device
// (scratch_address below).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The decode after validation: partials in `ws` (device memory of at least
// workspace_for(p, splits) bytes, 256-byte aligned), then the combine.
int decode_launch(const mi_attn_decode_params* p, int splits, void* ws, void* stream) {
  const int group = p->num_heads_q / p->num_heads_kv;
  const size_t rows = decode_rows(p);
  mi_attn::DecodeArgs a{};
  a.q = p->q;
  a.k_cache = p->k_cache;
  a.v_cache = p->v_cache;
  a.page_table = p->page_table;
  a.seqused_k = p->seqused_k;
  a.o_part = static_cast<float*>(ws);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        round_up(rows * splits * p->head_dim * sizeof(float)));
  a.q_bs = p->q_batch_stride;
  a.q_hs = p->q_head_stride;
  a.batch = p->batch;
  a.hq = p->num_heads_q;
  a.hkv = p->num_heads_kv;
  a.group = group;
  a.page_size = p->page_size;
  a.num_pages = p->num_pages;
  a.max_pages = p->max_pages_per_seq;
  a.num_splits = splits;
  a.row_blocks = decode_row_blocks(p);
  a.cu_q = p->cu_seqlens_q;
  a.scale = p->softmax_scale;
  a.scale_log2 = exp2_scale(p->softmax_scale);
  int wl, wr;
  normalise_window(p->causal, p->window_left, p->window_right, &wl, &wr);
  a.wl = wl;
  a.wr = wr;
  a.kv_fp8 = p->kv_dtype == MI_ATTN_KV_FP8_E4M3 ? 1 : p->kv_dtype == MI_ATTN_KV_FP8_E5M2 ? 2 : 0;
  a.k_descale = a.kv_fp8 ? p->k_descale : nullptr;
  a.v_descale = a.kv_fp8 ? p->v_descale : nullptr;
  a.softcap = p->softmax_scale > 0.0f ? p->softcap : 0.0f;
  if ((int64_t)a.batch * a.hkv * a.row_blocks * splits > INT32_MAX)
    return fail(MI_ATTN_EINVAL, "launch grid too large");

  mi_attn::CombineArgs cb{};
  cb.o_part = a.o_part;
  cb.lse_part = a.lse_part;
  cb.out = p->out;
  cb.lse = p->lse;
  cb.rows = (int)rows;
  cb.num_splits = splits;
  cb.sink = static_cast<const __bf16*>(p->learnable_sink);
  cb.hq = p->num_heads_q;
  // out rows are (batch, head): require the (b, h) -> row map to be affine
  if (p->o_batch_stride != (int64_t)p->num_heads_q * p->o_head_stride)
    return fail(MI_ATTN_EINVAL, "out must have o_batch_stride == num_heads_q * o_head_stride");
  cb.out_row_stride = p->o_head_stride;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = by_dim(p->head_dim, [&](auto dc) {
    hipError_t r = mi_attn::launch_decode<decltype(dc)::value>(a, s);
    if (r != hipSuccess) return r;
    return mi_attn::launch_combine<decltype(dc)::value>(cb, s);
  });
  if (e != hipSuccess) return fail(MI_ATTN_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up on the first call on each
// device, with that device current), or NULL with the error set.
void* scratch_address(int* rc) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = fail(MI_ATTN_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *rc = fail(MI_ATTN_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *rc = fail(MI_ATTN_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int mi_attn_decode_splitkv(const mi_attn_decode_params* p, void* stream) {
  int rc = check_decode(p);
  if (rc == MI_ATTN_OK) rc = check_decode_pointers(p);
  if (rc != MI_ATTN_OK) return rc;
  if (decode_rows(p) == 0 || decode_max_q(p) == 0) return ok();
  const int splits = resolved_splits(p);
  const size_t need = workspace_for(p, splits);
  if (p->workspace == nullptr || p->workspace_bytes < need)
    return fail(MI_ATTN_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                p->workspace == nullptr ? (size_t)0 : p->workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(p->workspace) & (kAlign - 1)) != 0)
    return fail(MI_ATTN_EWORKSPACE, "workspace must be 256-byte aligned");
  return decode_launch(p, splits, p->workspace, stream);
}

int mi_attn_decode_splitkv_noalloc(const mi_attn_decode_params* p, void* stream) {
  int rc = check_decode(p);
  if (rc == MI_ATTN_OK) rc = check_decode_pointers(p);
  if (rc != MI_ATTN_OK) return rc;
  if (decode_rows(p) == 0 || decode_max_q(p) == 0) return ok();
  const int splits = resolved_splits(p);
  const size_t need = workspace_for(p, splits);
  if (need > kScratchBytes)
    return fail(MI_ATTN_EWORKSPACE, "partials need %zu bytes, beyond the %zu-byte static "
                "scratch of the no-allocation decode (use mi_attn_decode_splitkv with a "
                "workspace, or fewer splits)", need, kScratchBytes);
  void* ws = scratch_address(&rc);
  if (ws == nullptr) return rc;
  return decode_launch(p, splits, ws, stream);
}

int mi_attn_combine(const float* o_partial, const float* lse_partial, void* out,
                    int64_t out_row_stride, float* lse, int32_t rows, int32_t num_splits,
                    int32_t head_dim, void* stream) {
  if (rows < 0) return fail(MI_ATTN_EINVAL, "rows must be >= 0");
  if (num_splits < 1 || num_splits > 256)
    return fail(MI_ATTN_EINVAL, "num_splits must be in 1..256 (got %d)", num_splits);
  if (!dim_supported(head_dim))
    return fail(MI_ATTN_EUNSUPPORTED, "head_dim %d not supported (64, 96, 128, 192, 256)",
                head_dim);
  if (rows == 0) return ok();
  if (!o_partial || !lse_partial || !out)
    return fail(MI_ATTN_EINVAL, "o_partial, lse_partial and out must be non-NULL");
  if (out_row_stride < head_dim || (out_row_stride % 8) != 0 || !aligned16(out))
    return fail(MI_ATTN_EINVAL, "out must be 16-byte aligned with a row stride >= head_dim, "
                                "multiple of 8");
  mi_attn::CombineArgs cb{};
  cb.o_part = o_partial;
  cb.lse_part = lse_partial;
  cb.out = out;
  cb.out_row_stride = out_row_stride;
  cb.lse = lse;
  cb.rows = rows;
  cb.num_splits = num_splits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = by_dim(head_dim, [&](auto dc) {
    return mi_attn::launch_combine<decltype(dc)::value>(cb, s);
  });
  if (e != hipSuccess) return fail(MI_ATTN_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Backward: shape, scalar and stride checks, then BwdArgs (enough to size
// the workspace; pointers are checked only to launch).
int check_bwd(const mi_attn_bwd_params* p, mi_attn::BwdArgs* a) {
  if (p == nullptr) return fail(MI_ATTN_EINVAL, "params is NULL");
  const bool varlen = p->cu_seqlens_q != nullptr || p->cu_seqlens_k != nullptr;
  if (varlen && (p->cu_seqlens_q == nullptr || p->cu_seqlens_k == nullptr))
    return fail(MI_ATTN_EINVAL, "cu_seqlens_q and cu_seqlens_k must both be given");
  if (p->batch < 0 || p->num_heads_q <= 0 || p->num_heads_kv <= 0)
    return fail(MI_ATTN_EINVAL, "batch must be >= 0 and head counts > 0");
  if (p->num_heads_q % p->num_heads_kv != 0)
    return fail(MI_ATTN_EINVAL, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)",
                p->num_heads_q, p->num_heads_kv);
  if (!dim_supported(p->head_dim))
    return fail(MI_ATTN_EUNSUPPORTED, "backward head_dim %d not supported (64, 96, 128, 192, 256)",
                p->head_dim);
  if (!isfinite(p->softmax_scale) || p->softmax_scale < 0.0f)
    return fail(MI_ATTN_EUNSUPPORTED, "softmax_scale must be finite and >= 0");
  int max_q, max_k;
  if (varlen) {
    if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0 || p->total_q < 0)
      return fail(MI_ATTN_EINVAL, "max_seqlen_q/k and total_q must be >= 0 for varlen");
    max_q = p->max_seqlen_q;
    max_k = p->max_seqlen_k;
  } else {
    if (p->seqlen_q < 0 || p->seqlen_k < 0)
      return fail(MI_ATTN_EINVAL, "seqlen_q and seqlen_k must be >= 0");
    max_q = p->seqlen_q;
    max_k = p->seqlen_k;
  }
  const int group = p->num_heads_q / p->num_heads_kv;
  if ((int64_t)max_q * group > INT32_MAX - mi_attn::kBwdBlockM ||
      (int64_t)max_k > INT32_MAX - mi_attn::kBwdBlockN)
    return fail(MI_ATTN_EINVAL, "sequence lengths overflow int32");
  if (p->batch > 65535 || p->num_heads_kv > 65535)
    return fail(MI_ATTN_EINVAL, "batch and num_heads_kv must be <= 65535");
  const int64_t rs[] = {p->q_row_stride, p->k_row_stride, p->v_row_stride, p->o_row_stride,
                        p->do_row_stride, p->dq_row_stride, p->dk_row_stride, p->dv_row_stride};
  const int64_t hs[] = {p->q_head_stride, p->k_head_stride, p->v_head_stride,
                        p->o_head_stride, p->do_head_stride, p->dq_head_stride,
                        p->dk_head_stride, p->dv_head_stride};
  for (int i = 0; i < 8; ++i) {
    if (!stride_ok(rs[i]) || !stride_ok(hs[i]))
      return fail(MI_ATTN_EINVAL, "row/head strides must be non-negative multiples of 8");
    if (rs[i] < p->head_dim)
      return fail(MI_ATTN_EINVAL, "row strides must be >= head_dim (rows may not overlap)");
    if ((int64_t)mi_attn::kBwdTileM * rs[i] * 2 > INT32_MAX)
      return fail(MI_ATTN_EINVAL, "row stride too large for 32-bit tile offsets");
  }
  if (!varlen) {
    const int64_t bs[] = {p->q_batch_stride, p->k_batch_stride, p->v_batch_stride,
                          p->o_batch_stride, p->do_batch_stride, p->dq_batch_stride,
                          p->dk_batch_stride, p->dv_batch_stride};
    for (int64_t s : bs)
      if (!stride_ok(s))
        return fail(MI_ATTN_EINVAL, "batch strides must be non-negative multiples of 8");
  }
  *a = mi_attn::BwdArgs{};
  a->q = p->q;
  a->k = p->k;
  a->v = p->v;
  a->o = p->out;
  a->dout = p->dout;
  a->lse = p->lse;
  a->dq = p->dq;
  a->dk = p->dk;
  a->dv = p->dv;
  a->q_bs = p->q_batch_stride;
  a->q_rs = p->q_row_stride;
  a->q_hs = p->q_head_stride;
  a->k_bs = p->k_batch_stride;
  a->k_rs = p->k_row_stride;
  a->k_hs = p->k_head_stride;
  a->v_bs = p->v_batch_stride;
  a->v_rs = p->v_row_stride;
  a->v_hs = p->v_head_stride;
  a->o_bs = p->o_batch_stride;
  a->o_rs = p->o_row_stride;
  a->o_hs = p->o_head_stride;
  a->do_bs = p->do_batch_stride;
  a->do_rs = p->do_row_stride;
  a->do_hs = p->do_head_stride;
  a->dq_bs = p->dq_batch_stride;
  a->dq_rs = p->dq_row_stride;
  a->dq_hs = p->dq_head_stride;
  a->dk_bs = p->dk_batch_stride;
  a->dk_rs = p->dk_row_stride;
  a->dk_hs = p->dk_head_stride;
  a->dv_bs = p->dv_batch_stride;
  a->dv_rs = p->dv_row_stride;
  a->dv_hs = p->dv_head_stride;
  a->cu_q = varlen ? p->cu_seqlens_q : nullptr;
  a->cu_k = varlen ? p->cu_seqlens_k : nullptr;
  a->batch = p->batch;
  a->seqlen_q = max_q;
  a->seqlen_k = max_k;
  a->hq = p->num_heads_q;
  a->hkv = p->num_heads_kv;
  a->group = group;
  a->total_q = varlen ? p->total_q : 0;
  a->scale = p->softmax_scale;
  a->scale_log2 = exp2_scale(p->softmax_scale);
  normalise_window(p->causal, p->window_left, p->window_right, &a->wl, &a->wr);
  return MI_ATTN_OK;
}

// Workspace: dPsum, then LSE log2 e (float32 per query row and head each),
// then the dK/dV split partials when the walk is split.
size_t bwd_workspace_for(const mi_attn::BwdArgs& a, int head_dim) {
  const int64_t n = mi_attn::bwd_dpsum_elems(a);
  if (n <= 0) return 0;
  const int64_t parts = mi_attn::bwd_part_elems(a, mi_attn::bwd_splits(a, head_dim), head_dim);
  return 2 * round_up((size_t)n * sizeof(float)) + round_up((size_t)parts * sizeof(float));
}

}  // namespace

extern "C" {

size_t mi_attn_bwd_workspace_bytes(const mi_attn_bwd_params* p) {
  mi_attn::BwdArgs a;
  if (check_bwd(p, &a) != MI_ATTN_OK) return 0;
  ok();
  return bwd_workspace_for(a, p->head_dim);
}

int mi_attn_bwd(const mi_attn_bwd_params* p, void* stream) {
  mi_attn::BwdArgs a;
  const int st = check_bwd(p, &a);
  if (st != MI_ATTN_OK) return st;
  if (p->batch == 0) return ok();
  // no query rows: no workspace, and dk, dv are written as zeros
  const size_t need = bwd_workspace_for(a, p->head_dim);
  if (!p->q || !p->k || !p->v || !p->out || !p->dout || !p->dq || !p->dk || !p->dv ||
      (need > 0 && !p->lse))
    return fail(MI_ATTN_EINVAL, "q, k, v, out, dout, lse, dq, dk and dv must be non-NULL");
  const void* ptrs[] = {p->q, p->k, p->v, p->out, p->dout, p->dq, p->dk, p->dv};
  for (const void* q : ptrs)
    if (!aligned16(q)) return fail(MI_ATTN_EINVAL, "tensors must be 16-byte aligned");
  if (need > 0 && (p->workspace == nullptr || p->workspace_bytes < need))
    return fail(MI_ATTN_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                p->workspace == nullptr ? (size_t)0 : p->workspace_bytes);
  if (need > 0 && !aligned16(p->workspace))
    return fail(MI_ATTN_EINVAL, "workspace must be 16-byte aligned");
  const size_t rows_b = round_up((size_t)mi_attn::bwd_dpsum_elems(a) * sizeof(float));
  a.dpsum = need > 0 ? static_cast<float*>(p->workspace) : nullptr;
  a.lse_log2 =
      need > 0 ? reinterpret_cast<float*>(static_cast<char*>(p->workspace) + rows_b) : nullptr;
  a.splits = need > 0 ? mi_attn::bwd_splits(a, p->head_dim) : 1;
  a.dkv_part = a.splits > 1
                   ? reinterpret_cast<float*>(static_cast<char*>(p->workspace) + 2 * rows_b)
                   : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = by_dim(p->head_dim, [&](auto dc) {
    return mi_attn::launch_bwd<decltype(dc)::value>(a, s);
  });
  if (e != hipSuccess) return fail(MI_ATTN_EHIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
