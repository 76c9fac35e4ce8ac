/*
 * mi_attn.h - C ABI of the MI355X (gfx950) exact-attention library.
 *
 * Two operations, both exact scaled-dot-product attention with a natural-log
 * log-sum-exp (LSE) output:
 *
 *   mi_attn_fwd             prefill / training-style forward over dense or
 *                           packed variable-length (cu_seqlens) batches.
 *   mi_attn_decode_splitkv  one query token per sequence against a paged K/V
 *                           cache, split along the key axis into partials
 *                           that an LSE-weighted combine then merges.
 *
 * What is computed (the forward of the mslk flash_attn interface.py page,
 * `_flash_attn_fwd` / `flash_attn_varlen_func`; LSE is the natural-log
 * log-sum-exp that the flash_bwd_sm100.py page's probability recompute
 * P = exp2(S * scale * log2e - LSE * log2e) assumes):
 *
 *   for batch b, query head h, query row i:
 *     g     = h / (Hq / Hkv)                      (consecutive GQA groups)
 *     s_ij  = softmax_scale * dot(q[b,i,h,:], k[b,j,g,:])   for visible j
 *     LSE_i = log(sum_j exp(s_ij))
 *     O_i   = sum_j exp(s_ij - LSE_i) * v[b,j,g,:]        (rounded to bf16)
 *   A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Visible keys (interface page, mask normalisation; bottom-right alignment
 * as in the backward page's causal/window block bounds): with
 * off = seqlen_k - seqlen_q of that sequence, key j is visible to row i iff
 *   j < seqlen_k,
 *   window_left  < 0  or  j >= i + off - window_left,
 *   window_right < 0  or  j <= i + off + window_right,
 * and causal != 0 forces window_right = 0. A negative window size means
 * "unbounded" (the interface page's None).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or synchronises; work is enqueued on
 *     `stream` (a hipStream_t; NULL means the null stream) and runs
 *     asynchronously.
 *   - Element types: q, k, v, out are bfloat16 (passed as void*); lse and the
 *     split partials are float32; index arrays are int32.
 *   - Strides are in elements. The last (head_dim) dimension must be
 *     contiguous; base pointers and strides must keep 16-byte alignment of
 *     each row (head_dim % 8 == 0, strides % 8 == 0, pointers 16-byte
 *     aligned).
 *   - Supported head_dim: 64, 96, 128, 192, 256 for every entry point (the
 *     interface page allows <= 256 in multiples of 8; other sizes return
 *     MI_ATTN_EUNSUPPORTED).
 *   - Return value: MI_ATTN_OK, or a negative mi_attn_status; on error
 *     nothing is enqueued and mi_attn_last_error() describes the problem.
 *   - The contents of device index arrays (cu_seqlens, seqused_k,
 *     page_table) are trusted: the host cannot read them without a
 *     synchronisation. Callers that cannot guarantee them should check on
 *     the host first (the Python binding does, on request). The decode
 *     kernel still refuses to dereference a page id outside [0, num_pages):
 *     the affected split is written as NaN instead of faulting.
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MI_ATTN_OK = 0,
  MI_ATTN_EINVAL = -1,        /* bad pointer, shape, stride or alignment      */
  MI_ATTN_EUNSUPPORTED = -2,  /* valid request the library does not implement */
  MI_ATTN_EBOUNDS = -3,       /* host-visible lengths exceed a table capacity */
  MI_ATTN_EWORKSPACE = -4,    /* workspace missing or too small               */
  MI_ATTN_EHIP = -5           /* the HIP runtime reported an error at launch  */
} mi_attn_status;

/* ------------------------------------------------------------------------
 * Prefill forward.
 *
 * Dense batch (cu_seqlens_q == cu_seqlens_k == NULL):
 *   q   [batch, seqlen_q, num_heads_q,  head_dim]  strides q_batch_stride,
 *                                                   q_row_stride, q_head_stride
 *   k,v [batch, seqlen_k, num_heads_kv, head_dim]  (k_*, v_* strides)
 *   out [batch, seqlen_q, num_heads_q,  head_dim]  (o_* strides)
 *   lse [batch, num_heads_q, seqlen_q] float32, contiguous, or NULL.
 *
 * Packed variable-length batch (both cu_seqlens non-NULL; interface page,
 * `flash_attn_varlen_func`): sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); batch strides are ignored.
 *   q   [total_q, num_heads_q, head_dim]
 *   k,v [total_k, num_heads_kv, head_dim]
 *   lse [num_heads_q, total_q] float32, contiguous, or NULL.
 *   total_q must equal cu_seqlens_q[batch]; max_seqlen_q / max_seqlen_k
 *   must bound every sequence's length (together they size the launch
 *   grid); seqlen_q / seqlen_k are ignored.
 *
 * Paged K/V (page_table non-NULL; interface page, the page_table branch of
 * `_flash_attn_fwd`: a KV cache in pages, e.g. prefill of new tokens after a
 * cached prefix): cu_seqlens_k must be NULL; queries are dense or packed by
 * cu_seqlens_q as above.
 *   k,v [num_pages, page_size, num_heads_kv, head_dim]: k_batch_stride /
 *       v_batch_stride are the strides between pages, row and head strides
 *       as above
 *   page_table [batch, max_pages_per_seq] int32, row-contiguous: key t of
 *       sequence b lives in page page_table[b * max_pages_per_seq +
 *       t / page_size], slot t % page_size
 *   seqused_k [batch] int32 keys of each sequence, or NULL for
 *       max_pages_per_seq * page_size; each must be in
 *       [0, max_pages_per_seq * page_size]
 *   seqlen_k and max_seqlen_k are ignored; queries are aligned bottom-right
 *   to each sequence's seqused_k keys.
 * page_size must be a positive multiple of 64 (a 64-key tile never straddles
 * pages; other sizes return MI_ATTN_EUNSUPPORTED) and num_pages,
 * max_pages_per_seq positive. The kernel checks every page id a workgroup
 * will read against [0, num_pages) before touching the cache; a workgroup
 * that finds one outside writes NaN to its rows of out and lse instead.
 * For dense K/V, page_table must be NULL and the four paging fields are
 * ignored.
 *
 * num_heads_q must be a multiple of num_heads_kv. Query heads sharing a KV
 * head are processed together (GQA packing), so one K/V tile load serves all
 * of them. softmax_scale must be finite; the Python binding passes
 * 1/sqrt(head_dim) when the caller gives none (interface page default).
 *
 * learnable_sink (interface page, `learnable_sink`: bf16, one per query head),
 * or NULL: head h's logit s_h joins every row's softmax denominator without a
 * value, so LSE = log(exp(s_h) + sum_j exp(scale * q.k_j)) and
 * O = sum_j exp(scale * q.k_j - LSE) v_j; a row with no visible key gets
 * O = 0 and LSE = s_h; s_h = -inf is no sink.
 *
 * softcap (interface page, `softcap` of `_flash_attn_fwd`; 0 means none):
 * every scaled score x = scale * q.k_j is replaced by softcap * tanh(x /
 * softcap) before the softmax (and before any sink is merged), so scores
 * stay inside (-softcap, softcap); the LSE is over the capped scores. Must
 * be finite and >= 0 (otherwise MI_ATTN_EUNSUPPORTED).
 * --------------------------------------------------------------------- */
typedef struct {
  const void *q, *k, *v;
  void *out;
  float *lse;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  int32_t batch, seqlen_q, seqlen_k;
  int32_t num_heads_q, num_heads_kv, head_dim;
  const int32_t *cu_seqlens_q, *cu_seqlens_k; /* device, [batch+1], or NULL  */
  int32_t total_q;                            /* varlen: cu_seqlens_q[batch],
                                                 the rows of q and lse; it
                                                 also sizes the launch grid */
  int32_t max_seqlen_q, max_seqlen_k;         /* varlen: host upper bounds   */
  const int32_t *page_table;                  /* device, paged K/V, or NULL  */
  float softmax_scale;
  int32_t causal, window_left, window_right;
  const int32_t *seqused_k;                   /* device [batch], paged only  */
  int32_t page_size, num_pages, max_pages_per_seq; /* paged only           */
  const void *learnable_sink;                 /* device bf16 [num_heads_q], or NULL */
  float softcap;                              /* 0: none; > 0: logit soft-capping */
} mi_attn_fwd_params;

int mi_attn_fwd(const mi_attn_fwd_params *p, void *stream);

/* ------------------------------------------------------------------------
 * Split-KV decode over a paged cache (split-K decoding page,
 * triton_splitk.py `FwOp.apply`; interface page, the page_table and
 * num_splits paths of `_flash_attn_fwd` and `flash_attn_combine`).
 *
 *   q        [batch, num_heads_q, head_dim] bf16, strides q_batch_stride,
 *            q_head_stride (one query token per sequence)
 *   k_cache,
 *   v_cache  [num_pages, page_size, num_heads_kv, head_dim] bf16, contiguous
 *   page_table [batch, max_pages_per_seq] int32, row-contiguous: token t of
 *            sequence b lives in page page_table[b][t / page_size], slot
 *            t % page_size
 *   seqused_k [batch] int32 keys per sequence, or NULL for
 *            max_pages_per_seq * page_size; each must be in
 *            [0, max_pages_per_seq * page_size]
 *   out      [batch, num_heads_q, head_dim] bf16, strides o_batch_stride,
 *            o_head_stride
 *   lse      [batch, num_heads_q] float32 contiguous, or NULL
 *
 * The query sits at position seqused_k[b] - 1 (bottom-right alignment), so
 * causal and window_right change nothing; window_left >= 0 restricts keys to
 * the last window_left + 1.
 *
 * Several query tokens per sequence (cu_seqlens_q non-NULL; interface page,
 * `flash_attn_varlen_func` with a page table and splits, e.g. a speculative
 * decoding step): sequence b owns query tokens [cu_seqlens_q[b],
 * cu_seqlens_q[b+1]) of
 *   q    [total_q, num_heads_q, head_dim]  (q_batch_stride is the stride
 *        between tokens, q_head_stride between heads)
 *   out  [total_q, num_heads_q, head_dim]  (o_batch_stride between tokens)
 *   lse  [total_q, num_heads_q] float32, or NULL
 * with cu_seqlens_q a device int32 [batch + 1] array, total_q =
 * cu_seqlens_q[batch] and max_seqlen_q >= every sequence's token count (host
 * ints; max_seqlen_q sizes the launch, total_q the workspace). The n tokens
 * of sequence b sit bottom-right at key positions seqused_k[b] - n ..
 * seqused_k[b] - 1, so causal / window_right now matter: with causal, token
 * i sees keys <= seqused_k[b] - n + i. With cu_seqlens_q NULL (one token per
 * sequence) the three fields are ignored.
 *
 * Keys are split into num_splits contiguous ranges (num_splits == 0 picks a
 * count from the occupancy heuristic; 1..256 are taken as given). Each split
 * writes float32 partials (O_s, LSE_s) into the workspace; the combine step
 * (the same kernel as mi_attn_combine) then forms
 *   LSE = log(sum_s exp(LSE_s)),  O = sum_s exp(LSE_s - LSE) * O_s,
 * where an empty split has LSE_s = -inf and contributes nothing.
 *
 * workspace: caller-allocated device memory of at least
 * mi_attn_decode_workspace_bytes(p) bytes, 256-byte aligned. Two launches
 * on `stream`; concurrent calls must use distinct workspaces.
 *
 * fp8 cache (kv_dtype == MI_ATTN_KV_FP8_E4M3 or MI_ATTN_KV_FP8_E5M2; sm_120
 * PR page, fp8 KV-cache decode, e4m3/e5m2): k_cache and v_cache hold one OCP
 * e4m3 (or e5m2) byte per element, same
 * [num_pages, page_size, num_heads_kv, head_dim] layout; the cached value is
 * k_descale[b * num_heads_kv + g] * fp8(byte) (likewise V), with
 * k_descale / v_descale device float32 [batch, num_heads_kv], or NULL for 1.
 * The query stays bf16 and the arithmetic is the bf16 path's (each byte is
 * widened to bf16 exactly). Every head_dim and page_size of the bf16 cache
 * is supported. With kv_dtype == MI_ATTN_KV_BF16 the descale pointers are
 * ignored.
 * --------------------------------------------------------------------- */
enum { MI_ATTN_KV_BF16 = 0, MI_ATTN_KV_FP8_E4M3 = 1, MI_ATTN_KV_FP8_E5M2 = 2 };

typedef struct {
  const void *q;
  const void *k_cache, *v_cache;
  const int32_t *page_table;
  const int32_t *seqused_k;
  void *out;
  float *lse;
  int64_t q_batch_stride, q_head_stride;
  int64_t o_batch_stride, o_head_stride;
  int32_t batch, num_heads_q, num_heads_kv, head_dim;
  int32_t page_size, num_pages, max_pages_per_seq;
  float softmax_scale;
  int32_t causal, window_left, window_right;
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
  int32_t kv_dtype;                     /* MI_ATTN_KV_BF16, _FP8_E4M3 or _FP8_E5M2 */
  const float *k_descale, *v_descale;   /* fp8 only: [batch, num_heads_kv] or NULL */
  const void *learnable_sink;           /* device bf16 [num_heads_q], or NULL; as for
                                           mi_attn_fwd, merged in the combine step */
  float softcap;                        /* 0: none; > 0: logit soft-capping, as for
                                           mi_attn_fwd (on the descaled scores) */
  const int32_t *cu_seqlens_q;          /* device [batch+1] packed query tokens, or NULL
                                           for one token per sequence */
  int32_t max_seqlen_q, total_q;        /* with cu_seqlens_q: host bounds (see above) */
} mi_attn_decode_params;

/* The split count mi_attn_decode_splitkv will use for *p (resolves
 * num_splits == 0), or a negative mi_attn_status if *p is invalid. */
int mi_attn_decode_num_splits(const mi_attn_decode_params *p);

/* Workspace bytes mi_attn_decode_splitkv needs for *p; 0 if *p is invalid
 * (mi_attn_last_error() then says why; with no query row at all a valid
 * request also needs 0 bytes, and the error string is then empty). Layout:
 * float32 O partials [rows][splits][head_dim], then float32 LSE partials
 * [rows][splits], each 256-byte aligned, rows = batch * num_heads_q (one
 * token per sequence) or total_q * num_heads_q. */
size_t mi_attn_decode_workspace_bytes(const mi_attn_decode_params *p);

int mi_attn_decode_splitkv(const mi_attn_decode_params *p, void *stream);

/* The same decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * identical arguments, kernels and results as mi_attn_decode_splitkv, except
 * that p->workspace and p->workspace_bytes are ignored. The float32 partials
 * go to a static scratch array of 64 MiB inside the library, one per GPU,
 * created when the library's code is loaded on that GPU and held until the
 * process ends; nothing is allocated or freed by this call. A request whose
 * partials (mi_attn_decode_workspace_bytes(p)) exceed 64 MiB returns
 * MI_ATTN_EWORKSPACE. The first call on each device looks the array's device
 * address up (hipGetSymbolAddress) with that device current; a failed
 * lookup returns MI_ATTN_EHIP.
 * Every call on one GPU uses that GPU's one array and leaves the last call's
 * partials in it: calls that can overlap on one GPU (different streams, or
 * different host threads without ordering) race and must be serialised by
 * the caller; calls in order on one stream are safe. */
int mi_attn_decode_splitkv_noalloc(const mi_attn_decode_params *p, void *stream);

/* ------------------------------------------------------------------------
 * LSE-weighted combine of split partials (interface page,
 * `flash_attn_combine` / `_flash_attn_fwd_combine`; split-K page,
 * `merge_attentions`).
 *
 *   o_partial   [rows, num_splits, head_dim] float32, contiguous
 *   lse_partial [rows, num_splits] float32, contiguous
 *   out         bf16, row r at out + r * out_row_stride (head_dim contiguous)
 *   lse         [rows] float32, or NULL
 * num_splits in 1..256, head_dim in {64, 96, 128, 192, 256}. A row whose partial LSEs
 * are all -inf gets O = 0 and LSE = -inf. This is the merge the decode path
 * runs; exported so a caller holding partials from elsewhere (for example
 * key shards on other devices) can merge them.
 * --------------------------------------------------------------------- */
int mi_attn_combine(const float *o_partial, const float *lse_partial, void *out,
                    int64_t out_row_stride, float *lse, int32_t rows, int32_t num_splits,
                    int32_t head_dim, void *stream);

/* ------------------------------------------------------------------------
 * Backward pass of the prefill forward (Blackwell backward page
 * flash_bwd_sm100.py and the interface page's `_flash_attn_bwd`): given the
 * forward's inputs q, k, v, its output out and LSE, and the output gradient
 * dout, writes dq, dk, dv for
 *   P = exp(scale * q.k^T - LSE) over the visible keys,
 *   dv = P^T dout,  dS = P * (dout v^T - rowsum(out * dout)),
 *   dq = scale * dS k,  dk = scale * dS^T q,
 * with dk / dv of a KV head summed over the query heads that read it (GQA).
 *
 * Layouts as mi_attn_fwd: q, out, dout, dq share the query layout (dense
 * [batch, seqlen_q, heads, head_dim] or packed [total_q, heads, head_dim]
 * with cu_seqlens_q), k, v, dk, dv the key layout, each with its own
 * batch/row/head strides (elements; row and head strides non-negative
 * multiples of 8, head_dim contiguous); every tensor bf16, 16-byte aligned.
 * lse is the forward's float32 LSE in its layout ([batch, num_heads_q,
 * seqlen_q] dense, [num_heads_q, total_q] packed); a row with LSE = -inf
 * (no visible key) gets dq = 0 and contributes nothing to dk, dv. Masks
 * (causal, window_left, window_right, bottom-right alignment) and
 * softmax_scale mean what they mean for mi_attn_fwd; cu_seqlens_q and
 * cu_seqlens_k are given together or not at all. Paged K/V and the
 * learnable sink are not part of the backward.
 *
 * head_dim 64, 96, 128, 192 or 256 (others return MI_ATTN_EUNSUPPORTED). The result
 * is deterministic: nothing is accumulated with atomics. The caller owns
 * every buffer, including the workspace (size from
 * mi_attn_bwd_workspace_bytes; a smaller one returns MI_ATTN_EWORKSPACE):
 * float32 row sums of out * dout and the LSE in base 2 (LSE * log2 e), one
 * each per query row and head, then, when few key blocks would leave the
 * device idle, float32 dk / dv partials of up to four parts of each key
 * block's walk over the queries, summed in a fixed order. Work is enqueued on `stream`; nothing is
 * allocated and the stream is not synchronised.
 * --------------------------------------------------------------------- */
typedef struct {
  const void *q, *k, *v, *out, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  int64_t do_batch_stride, do_row_stride, do_head_stride;
  int64_t dq_batch_stride, dq_row_stride, dq_head_stride;
  int64_t dk_batch_stride, dk_row_stride, dk_head_stride;
  int64_t dv_batch_stride, dv_row_stride, dv_head_stride;
  int32_t batch, seqlen_q, seqlen_k;
  int32_t num_heads_q, num_heads_kv, head_dim;
  const int32_t *cu_seqlens_q, *cu_seqlens_k; /* device, [batch+1], or NULL */
  int32_t total_q;                            /* varlen: cu_seqlens_q[batch] */
  int32_t max_seqlen_q, max_seqlen_k;         /* varlen: host upper bounds   */
  float softmax_scale;
  int32_t causal, window_left, window_right;
  void *workspace;
  size_t workspace_bytes;
} mi_attn_bwd_params;

/* Workspace bytes mi_attn_bwd needs for *p; 0 if *p is invalid
 * (mi_attn_last_error() then says why) or needs none. */
size_t mi_attn_bwd_workspace_bytes(const mi_attn_bwd_params *p);

int mi_attn_bwd(const mi_attn_bwd_params *p, void *stream);

/* Message for the last non-OK status returned on the calling thread. */
const char *mi_attn_last_error(void);

/* Library version string. */
const char *mi_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI_ATTN_H */
