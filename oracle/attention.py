"""Full-score-matrix float64 attention oracle (test infrastructure only).

Definition followed (the forward the attention front end computes; see the
mslk flash_attn interface.py page, `_flash_attn_fwd` docstring and argument
checks, and the Blackwell backward page flash_bwd_sm100.py, where the
probabilities are recomputed as exp2(S*scale*log2e - LSE*log2e), which fixes
LSE as the natural-log log-sum-exp of the scaled scores):

  for each batch b, query head h, query i:
    g      = h // (Hq / Hkv)                  consecutive GQA grouping
    s_ij   = scale * <q[b,i,h,:], k[b,j,g,:]>  for visible keys j
    LSE_i  = log sum_j exp(s_ij)              natural log
    O_i    = sum_j exp(s_ij - LSE_i) v[b,j,g,:]
  a query with no visible key has O = 0 and LSE = -inf (the split-K page's
  empty-input short-circuit; the sm_120 PR page's all-masked-row guard).

Visible keys (interface page, mask normalization in `_flash_attn_fwd`; the
backward page's causal/window block bounds, which offset by seqlen_k-seqlen_q):
  off = Sk - Sq  (bottom-right alignment)
  j visible iff 0 <= j < Sk
             and (window_left  is None or j >= i + off - window_left)
             and (window_right is None or j <= i + off + window_right)
  causal forces window_right = 0; both window bounds are inclusive.

Inputs are float64 arrays converted exactly from the same bf16 bit patterns the
GPU reads. All arithmetic is float64.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------- masks ----

def normalize_window(causal: bool, window_left: Optional[int], window_right: Optional[int]):
    """Returns (window_left, window_right) with None meaning unbounded.

    Negative sizes are read as unbounded (the C ABI's encoding of None).
    Causal forces window_right = 0 (interface page, `_flash_attn_fwd`).
    """
    wl = None if (window_left is None or window_left < 0) else int(window_left)
    wr = None if (window_right is None or window_right < 0) else int(window_right)
    if causal:
        wr = 0
    return wl, wr


def visible_mask(seqlen_q: int, seqlen_k: int, causal: bool = False,
                 window_left: Optional[int] = None,
                 window_right: Optional[int] = None, rows=None) -> np.ndarray:
    """Boolean (Sq, Sk) matrix of visible (query, key) pairs, bottom-right aligned.

    `rows` restricts the result to the given query positions (n, Sk).
    """
    wl, wr = normalize_window(causal, window_left, window_right)
    i = np.arange(seqlen_q, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    i = i[:, None]
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    diag = i + (seqlen_k - seqlen_q)
    vis = np.ones((i.shape[0], seqlen_k), dtype=bool)
    if wl is not None:
        vis &= j >= diag - wl
    if wr is not None:
        vis &= j <= diag + wr
    return vis


# ------------------------------------------------------------- one head ----

def softmax_lse_rows(s: np.ndarray, vis: np.ndarray, sink: Optional[float] = None):
    """Row-wise log-sum-exp and probabilities of masked scores.

    s, vis: (n, Sk). Returns (P (n, Sk), LSE (n,)). Empty rows: P = 0, LSE = -inf.
    sink: a learnable-sink logit (interface page, `learnable_sink`, one per
    query head), read as one more term of every row's softmax denominator that
    carries no value: LSE = log(exp(sink) + sum_j exp(s_j)), P_j = exp(s_j - LSE).
    A row with no visible key then has P = 0 and LSE = sink.
    """
    s = np.where(vis, s, NEG_INF)
    nonempty = vis.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=NEG_INF), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    lsum = e.sum(axis=1)
    lse = np.full(s.shape[0], NEG_INF)
    lse[nonempty] = m[nonempty] + np.log(lsum[nonempty])
    if sink is not None and sink != NEG_INF:
        hi = np.maximum(lse, sink)
        lse = hi + np.log(np.exp(lse - hi) + np.exp(sink - hi))
    p = np.zeros_like(e)
    p[nonempty] = np.where(vis[nonempty], np.exp(s[nonempty] - lse[nonempty, None]), 0.0)
    return p, lse


def softcap_scores(s: np.ndarray, softcap: Optional[float]) -> np.ndarray:
    """Logit soft-capping of the scaled scores (interface page, `softcap`
    argument of `_flash_attn_fwd`, turned into a score modifier whose body the
    pages do not show; 0 or None means none). Reading: cap * tanh(s / cap),
    which keeps every score in (-cap, cap) and equals s to first order."""
    if softcap is None or softcap == 0.0:
        return s
    return softcap * np.tanh(s / softcap)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   vis: np.ndarray, sink: Optional[float] = None,
                   softcap: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Single head. q (Sq, D), k (Sk, D), v (Sk, Dv), vis (Sq, Sk) -> O (Sq, Dv), LSE (Sq,).
    sink: this head's learnable-sink logit or None (softmax_lse_rows); softcap:
    the soft-capping constant or None (softcap_scores)."""
    s = softcap_scores(scale * (q @ k.T), softcap)
    p, lse = softmax_lse_rows(s, vis, sink)
    return p @ v, lse


def _sink_of(sink, h):
    return None if sink is None else float(sink[h])


# ------------------------------------------------------- dense / varlen ----

def attention_dense(q, k, v, scale, causal=False, window_left=None, window_right=None,
                    sink=None, softcap=None):
    """q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D) float64 -> O (B, Sq, Hq, Dv), LSE (B, Hq, Sq).
    sink: per-query-head learnable-sink logits (Hq,) or None."""
    B, Sq, Hq, _ = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    r = Hq // Hkv
    vis = visible_mask(Sq, Sk, causal, window_left, window_right)
    out = np.zeros((B, Sq, Hq, v.shape[-1]))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // r
            out[b, :, h], lse[b, h] = attention_head(q[b, :, h], k[b, :, g], v[b, :, g], scale, vis,
                                                     _sink_of(sink, h), softcap)
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                     window_left=None, window_right=None, sink=None, softcap=None):
    """Packed sequences. q (Tq, Hq, D), k/v (Tk, Hkv, D) -> O (Tq, Hq, Dv), LSE (Hq, Tq).

    The LSE layout (num_heads, total_q) is the interface page's varlen layout.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    r = Hq // Hkv
    out = np.zeros((q.shape[0], Hq, v.shape[-1]))
    lse = np.full((Hq, q.shape[0]), NEG_INF)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        if q1 == q0:
            continue
        vis = visible_mask(q1 - q0, k1 - k0, causal, window_left, window_right)
        for h in range(Hq):
            g = h // r
            out[q0:q1, h], lse[h, q0:q1] = attention_head(q[q0:q1, h], k[k0:k1, g],
                                                          v[k0:k1, g], scale, vis,
                                                          _sink_of(sink, h), softcap)
    return out, lse


# -------------------------------------------------------------- backward ----

def attention_head_backward(q, k, v, dout, scale, vis):
    """Gradients of one head's attention output (backward page flash_bwd_sm100.py:
    recompute P from S and LSE, dV = P^T dO, dP = dO V^T, dS = P * (dP - dPsum),
    dQ = scale dS K, dK = scale dS^T Q; the interface page's backward
    preprocess defines dPsum as the row sum of O * dO).

    q (Sq, D), k (Sk, D), v (Sk, Dv), dout (Sq, Dv), vis (Sq, Sk) ->
    dq (Sq, D), dk (Sk, D), dv (Sk, Dv). A query with no visible key has
    P = 0 and so contributes nothing."""
    s = scale * (q @ k.T)
    p, _ = softmax_lse_rows(s, vis)
    o = p @ v
    dv = p.T @ dout
    dp = dout @ v.T
    dpsum = np.sum(o * dout, axis=1)
    ds = p * (dp - dpsum[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_dense_backward(q, k, v, dout, scale, causal=False, window_left=None,
                             window_right=None):
    """q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D), dout (B, Sq, Hq, Dv) float64 ->
    dq, dk, dv shaped like q, k, v. With GQA, a KV head's dK and dV sum the
    contributions of every query head that reads it (the interface page's
    backward reduces them over the qhead_per_kvhead heads)."""
    B, Sq, Hq, _ = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    r = Hq // Hkv
    vis = visible_mask(Sq, Sk, causal, window_left, window_right)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // r
            gq, gk, gv = attention_head_backward(q[b, :, h], k[b, :, g], v[b, :, g],
                                                 dout[b, :, h], scale, vis)
            dq[b, :, h] = gq
            dk[b, :, g] += gk
            dv[b, :, g] += gv
    return dq, dk, dv


def attention_varlen_backward(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                              window_left=None, window_right=None):
    """Packed sequences: q (Tq, Hq, D), k/v (Tk, Hkv, D), dout (Tq, Hq, Dv) ->
    dq, dk, dv shaped like q, k, v; each sequence as attention_dense_backward."""
    Hq, Hkv = q.shape[1], k.shape[1]
    r = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        vis = visible_mask(q1 - q0, k1 - k0, causal, window_left, window_right)
        for h in range(Hq):
            g = h // r
            gq, gk, gv = attention_head_backward(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g],
                                                 dout[q0:q1, h], scale, vis)
            dq[q0:q1, h] = gq
            dk[k0:k1, g] += gk
            dv[k0:k1, g] += gv
    return dq, dk, dv


def attention_rows(q_rows: np.ndarray, row_index: np.ndarray, k: np.ndarray, v: np.ndarray,
                   scale: float, seqlen_q: int, causal=False, window_left=None,
                   window_right=None, softcap=None):
    """Selected query rows of one (sequence, head) problem, for sampling huge inputs.

    q_rows (n, D) are the queries at positions row_index (n,) of a length-seqlen_q
    query sequence; k (Sk, D), v (Sk, Dv) are that head's keys and values.
    Returns O (n, Dv), LSE (n,), computed from the same definition row by row.
    """
    vis = visible_mask(seqlen_q, k.shape[0], causal, window_left, window_right, rows=row_index)
    return attention_head(q_rows, k, v, scale, vis, softcap=softcap)


# ------------------------------------------------------------- split-KV ----

def split_bounds(seqlen_k: int, num_splits: int) -> List[Tuple[int, int]]:
    """Contiguous key ranges [s*c, min(Sk, (s+1)*c)) with c = ceil(Sk / num_splits).

    The split-K page (triton_splitk.py, `FwOp.apply`) sizes splits as
    ceil(Mk / split_k). Trailing ranges may be empty.
    """
    c = -(-seqlen_k // num_splits) if seqlen_k > 0 else 0
    return [(min(seqlen_k, s * c), min(seqlen_k, (s + 1) * c)) for s in range(num_splits)]


def attention_partials(q, k, v, scale, vis, bounds: Sequence[Tuple[int, int]], softcap=None):
    """Per-split (O_s, LSE_s) for one head: attention restricted to each key range.

    q (n, D), k/v (Sk, D), vis (n, Sk). Returns O (S, n, Dv), LSE (S, n). An
    empty range (or one with no visible key for a row) gives O = 0, LSE = -inf.
    """
    n = q.shape[0]
    o_parts = np.zeros((len(bounds), n, v.shape[-1]))
    lse_parts = np.full((len(bounds), n), NEG_INF)
    for s, (a, b) in enumerate(bounds):
        if b <= a:
            continue
        o_parts[s], lse_parts[s] = attention_head(q, k[a:b], v[a:b], scale, vis[:, a:b],
                                                  softcap=softcap)
    return o_parts, lse_parts


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """LSE-weighted merge of split partials (interface page, `flash_attn_combine`;
    split-K page, `merge_attentions`).

    o_parts (S, ..., Dv), lse_parts (S, ...):
      LSE = max_s LSE_s + log sum_s exp(LSE_s - max_s LSE_s)
      O   = sum_s exp(LSE_s - LSE) O_s
    A split with LSE_s = -inf contributes nothing; if all are -inf, O = 0 and
    LSE = -inf.
    """
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    total = w.sum(axis=0)
    lse = np.full(m.shape, NEG_INF)
    lse[finite] = m_safe[finite] + np.log(total[finite])
    lse_safe = np.where(finite, lse, 0.0)
    wn = np.where(np.isfinite(lse_parts), np.exp(lse_parts - lse_safe), 0.0)
    out = (wn[..., None] * o_parts).sum(axis=0)
    out[~finite] = 0.0
    return out, lse


# --------------------------------------------------------------- paged -----

def paged_gather(cache: np.ndarray, page_table_row: np.ndarray, seqlen: int) -> np.ndarray:
    """Contiguous (seqlen, Hkv, D) view of one sequence stored in a paged cache.

    cache (num_pages, page_size, Hkv, D); token t of the sequence lives in page
    page_table_row[t // page_size], slot t % page_size (interface page, the
    page_table branch of `_flash_attn_fwd`).
    """
    page_size = cache.shape[1]
    n_pages = -(-seqlen // page_size)
    pages = [cache[int(page_table_row[p])] for p in range(n_pages)]
    if not pages:
        return np.zeros((0,) + cache.shape[2:])
    return np.concatenate(pages, axis=0)[:seqlen]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of OCP 8-bit floating point E4M3 codes (the fp8 e4m3 format the
    sm_120 PR page's fp8 KV-cache decode stores), as float64.

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    mantissa m: e > 0 gives (1 + m/8) * 2**(e - 7), e = 0 the subnormal
    (m/8) * 2**-6; the two codes with e = 15 and m = 7 are NaN, and there are
    no infinities (largest finite magnitude 448).
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """Values of OCP 8-bit floating point E5M2 codes (the other fp8 KV-cache
    format the sm_120 PR page's decode accepts), as float64.

    Bit 7 is the sign, bits 6..2 the exponent field e (bias 15), bits 1..0 the
    mantissa m: 0 < e < 31 gives (1 + m/4) * 2**(e - 15), e = 0 the subnormal
    (m/4) * 2**-14; e = 31 is infinity when m = 0 and NaN otherwise (largest
    finite magnitude 57344).
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def with_sink(out, lse, sink):
    """Adds learnable-sink logits to a finished (O, LSE): LSE' = log(exp(LSE)
    + exp(sink)), O' = O * exp(LSE - LSE'). out[..., :] rows line up with lse
    (out has lse's shape plus the value axis); sink broadcasts against lse.
    Equal to putting the sink into the softmax (softmax_lse_rows); used where
    the keys were split."""
    sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), lse.shape)
    hi = np.maximum(lse, sink)
    new = hi + np.log(np.exp(lse - hi) + np.exp(sink - hi))
    w = np.where(np.isfinite(lse), np.exp(lse - new), 0.0)
    return out * w[..., None], new


def paged_decode(q, k_cache, v_cache, page_table, seqused_k, scale, num_splits=1,
                 causal=False, window_left=None, window_right=None, heads=None,
                 k_descale=None, v_descale=None, sink=None, softcap=None):
    """One query per sequence over a paged cache.

    q (B, Hq, D) float64. Returns O (B, Hq, Dv), LSE (B, Hq), and the split
    partials (S, B, Hq, Dv), (S, B, Hq) of the contiguous-range partition used
    by split_bounds, combined with `combine` to form O and LSE. `heads` limits
    the work to a subset of query heads (others are left at zero / -inf).
    k_descale / v_descale (B, Hkv), for a quantized cache (sm_120 PR page, fp8
    KV-cache decode with per-(batch, kv_head) descales): sequence b's keys of
    KV head g are k_descale[b, g] times the cached values (likewise V); the
    caches are then the decoded values (e4m3_decode or e5m2_decode of the
    stored codes).
    sink: per-query-head learnable-sink logits (Hq,), merged after the split
    combine (with_sink). softcap: as attention_head.
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    r = Hq // Hkv
    heads = range(Hq) if heads is None else heads
    o_parts = np.zeros((num_splits, B, Hq, v_cache.shape[-1]))
    lse_parts = np.full((num_splits, B, Hq), NEG_INF)
    for b in range(B):
        sk = int(seqused_k[b])
        kb = paged_gather(k_cache, page_table[b], sk)
        vb = paged_gather(v_cache, page_table[b], sk)
        if k_descale is not None:
            kb = kb * np.asarray(k_descale, dtype=np.float64)[b][None, :, None]
        if v_descale is not None:
            vb = vb * np.asarray(v_descale, dtype=np.float64)[b][None, :, None]
        vis = visible_mask(1, sk, causal, window_left, window_right)
        bounds = split_bounds(sk, num_splits)
        for h in heads:
            g = h // r
            o, l = attention_partials(q[b, h][None, :], kb[:, g], vb[:, g], scale, vis, bounds,
                                      softcap)
            o_parts[:, b, h] = o[:, 0]
            lse_parts[:, b, h] = l[:, 0]
    out, lse = combine(o_parts, lse_parts)
    if sink is not None:
        out, lse = with_sink(out, lse, np.asarray(sink, dtype=np.float64)[None, :])
    return out, lse, o_parts, lse_parts


def paged_prefill(q, k_cache, v_cache, page_table, seqused_k, scale, causal=False,
                  window_left=None, window_right=None, cu_seqlens_q=None, sink=None,
                  softcap=None):
    """Queries against a paged K/V cache (interface page, the page_table branch
    of `_flash_attn_fwd`: caches (num_pages, page_size, Hkv, D), a
    (B, max_pages) page table, per-sequence key counts seqused_k).

    q is dense (B, Sq, Hq, D), or packed (Tq, Hq, D) with cu_seqlens_q. The keys
    of sequence b are its seqused_k[b] cached tokens (None: the capacity of its
    page-table row, max_pages * page_size) gathered through the page table;
    the definition then applies with the queries aligned bottom-right to those
    keys. Returns O shaped like q and LSE (B, Hq, Sq) dense or (Hq, Tq) packed.
    """
    B = page_table.shape[0]
    cap = page_table.shape[1] * k_cache.shape[1]
    Hq, Hkv = q.shape[-2], k_cache.shape[2]
    r = Hq // Hkv
    packed = cu_seqlens_q is not None
    out = np.zeros(q.shape[:-1] + (v_cache.shape[-1],))
    lse = np.full((Hq, q.shape[0]) if packed else (B, Hq, q.shape[1]), NEG_INF)
    for b in range(B):
        sk = cap if seqused_k is None else int(seqused_k[b])
        kb = paged_gather(k_cache, page_table[b], sk)
        vb = paged_gather(v_cache, page_table[b], sk)
        if packed:
            q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            qb = q[q0:q1]
        else:
            qb = q[b]
        if qb.shape[0] == 0:
            continue
        vis = visible_mask(qb.shape[0], sk, causal, window_left, window_right)
        for h in range(Hq):
            g = h // r
            o, l = attention_head(qb[:, h], kb[:, g], vb[:, g], scale, vis, _sink_of(sink, h),
                                  softcap)
            if packed:
                out[q0:q1, h], lse[h, q0:q1] = o, l
            else:
                out[b, :, h], lse[b, h] = o, l
    return out, lse


# ------------------------------------------------------- accounting --------

def visible_pairs(seqlen_q: int, seqlen_k: int, causal=False, window_left=None,
                  window_right=None) -> int:
    """Number of visible (query, key) pairs of one head (for FLOP accounting)."""
    return int(visible_mask(seqlen_q, seqlen_k, causal, window_left, window_right).sum())


def bf16_round_nearest_even(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits: with x = m * 2**e, 0.5 <= |m| < 1, the grid
    spacing is 2**(e - 8). Scaling by a power of two is exact, so np.round
    (half to even) on the scaled value rounds exactly. Used by tests to state
    expected outputs at the output precision.
    """
    f = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(f)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def flops_causal_adjusted(head_dim: int, num_heads_q: int, pairs_per_head: int) -> float:
    """4 * D * visible pairs * heads: two matmuls, two flops per multiply-add."""
    return 4.0 * head_dim * num_heads_q * pairs_per_head

