"""Plants plausible mistakes in the oracle (CPU only) and checks a pin catches each.

Each mutant rewrites one line of one oracle function from its source text,
installs it in the oracle module for the duration of the test, runs every
pin, and requires at least one pin to fail.
"""
import inspect
import textwrap

import pytest

import oracle.attention as A
from tests import oracle_pins as P

MUTANTS = [
    # (function, original text, mistaken text, what the mistake is)
    ("visible_mask", "vis &= j >= diag - wl", "vis &= j > diag - wl", "left window off by one"),
    ("visible_mask", "vis &= j <= diag + wr", "vis &= j < diag + wr", "right window exclusive"),
    ("visible_mask", "diag = i + (seqlen_k - seqlen_q)", "diag = i", "top-left causal alignment"),
    ("visible_mask", "diag = i + (seqlen_k - seqlen_q)", "diag = i + (seqlen_q - seqlen_k)",
     "offset sign flipped"),
    ("normalize_window", "wr = 0", "wl = 0", "causal sets the wrong side"),
    ("softmax_lse_rows", "lse[nonempty] = m[nonempty] + np.log(lsum[nonempty])",
     "lse[nonempty] = np.log(lsum[nonempty])", "LSE drops the max term"),
    ("softmax_lse_rows", "lse[nonempty] = m[nonempty] + np.log(lsum[nonempty])",
     "lse[nonempty] = m[nonempty] + np.log2(lsum[nonempty])", "LSE in base 2"),
    ("attention_head", "softcap_scores(scale * (q @ k.T), softcap)",
     "softcap_scores((q @ k.T), softcap)", "scale dropped"),
    ("attention_head", "return p @ v, lse", "return p @ v[::-1], lse", "values reversed"),
    ("attention_dense", "g = h // r", "g = h % Hkv", "interleaved GQA grouping"),
    ("attention_varlen", "g = h // r", "g = h % Hkv", "interleaved GQA grouping (varlen)"),
    ("attention_varlen", "k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])",
     "k0, k1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])", "key offsets from query cu"),
    ("combine", "wn = np.where(np.isfinite(lse_parts), np.exp(lse_parts - lse_safe), 0.0)",
     "wn = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)",
     "combine weights not normalised"),
    ("combine", "lse[finite] = m_safe[finite] + np.log(total[finite])",
     "lse[finite] = m_safe[finite]", "combined LSE keeps only the max"),
    ("split_bounds", "return [(min(seqlen_k, s * c), min(seqlen_k, (s + 1) * c)) for s in range(num_splits)]",
     "return [(min(seqlen_k, s * c), min(seqlen_k, (s + 1) * c - 1)) for s in range(num_splits)]",
     "split ranges drop their last key"),
    ("paged_gather", "pages = [cache[int(page_table_row[p])] for p in range(n_pages)]",
     "pages = [cache[p] for p in range(n_pages)]", "page table ignored"),
    ("paged_decode", "g = h // r", "g = h % Hkv", "interleaved GQA grouping (paged)"),
    ("paged_prefill", "g = h // r", "g = h % Hkv", "interleaved GQA grouping (paged prefill)"),
    ("e4m3_decode", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)", "e4m3 exponent bias 8 (the FNUZ bias)"),
    ("softmax_lse_rows", "lse = hi + np.log(np.exp(lse - hi) + np.exp(sink - hi))",
     "lse = hi + np.log(np.exp(lse - hi) + np.exp(-sink - hi))", "sink sign flipped"),
    ("softmax_lse_rows", "lse = hi + np.log(np.exp(lse - hi) + np.exp(sink - hi))",
     "lse = hi", "sink replaces the log-sum instead of adding to it"),
    ("with_sink", "w = np.where(np.isfinite(lse), np.exp(lse - new), 0.0)",
     "w = np.where(np.isfinite(lse), 1.0, 0.0)", "sink merge leaves O unscaled"),
    ("e4m3_decode", "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7", "e4m3 subnormal scale"),
    ("e5m2_decode", "np.exp2(e - 15.0)", "np.exp2(e - 16.0)", "e5m2 exponent bias 16 (the FNUZ bias)"),
    ("e5m2_decode", "(m / 4.0) * 2.0 ** -14", "(m / 4.0) * 2.0 ** -15", "e5m2 subnormal scale"),
    ("e5m2_decode", "e = (c >> 2) & 0x1F", "e = (c >> 3) & 0x1F", "e5m2 read with e4m3's field split"),
    ("paged_decode", "kb = kb * np.asarray(k_descale, dtype=np.float64)[b][None, :, None]",
     "kb = kb * np.asarray(v_descale, dtype=np.float64)[b][None, :, None]", "K scaled by the V descale"),
    ("paged_decode", "vb = vb * np.asarray(v_descale, dtype=np.float64)[b][None, :, None]",
     "vb = vb * np.asarray(v_descale, dtype=np.float64)[0][None, :, None]", "V descale of sequence 0 for all"),
    ("softcap_scores", "return softcap * np.tanh(s / softcap)", "return softcap * np.tanh(s)",
     "soft cap without the 1/cap inside"),
    ("softcap_scores", "return softcap * np.tanh(s / softcap)", "return np.tanh(s / softcap)",
     "soft cap without the outer cap"),
    ("softcap_scores", "return softcap * np.tanh(s / softcap)", "return np.clip(s, -softcap, softcap)",
     "hard clip instead of tanh"),
    ("attention_head_backward", "ds = p * (dp - dpsum[:, None])", "ds = p * dp",
     "backward drops the dPsum term"),
    ("attention_head_backward", "dq = scale * (ds @ k)", "dq = ds @ k", "dQ without the scale"),
    ("attention_head_backward", "dk = scale * (ds.T @ q)", "dk = scale * (p.T @ q)",
     "dK from P instead of dS"),
    ("attention_head_backward", "dv = p.T @ dout", "dv = p.T @ dout[::-1]", "dO rows reversed"),
    ("attention_dense_backward", "dk[b, :, g] += gk", "dk[b, :, g] = gk",
     "GQA dK keeps only the last query head"),
    ("attention_dense_backward", "vis = visible_mask(Sq, Sk, causal, window_left, window_right)",
     "vis = visible_mask(Sq, Sk, False, None, None)", "backward ignores the mask"),
    ("attention_varlen_backward", "k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])",
     "k0, k1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])",
     "backward key offsets from query cu"),
    ("paged_prefill", "sk = cap if seqused_k is None else int(seqused_k[b])", "sk = cap",
     "seqused_k ignored (paged prefill)"),
    ("paged_prefill", "vis = visible_mask(qb.shape[0], sk, causal, window_left, window_right)",
     "vis = visible_mask(qb.shape[0], qb.shape[0], causal, window_left, window_right)",
     "queries aligned to their own length, not the cached keys"),
    ("paged_prefill", "kb = paged_gather(k_cache, page_table[b], sk)",
     "kb = paged_gather(k_cache, page_table[0], sk)", "every sequence reads row 0 of the table"),
]


@pytest.mark.parametrize("fn,orig,bad,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, fn, orig, bad, what):
    src = textwrap.dedent(inspect.getsource(getattr(A, fn)))
    assert orig in src, f"mutation anchor not found in {fn}"
    ns = dict(vars(A))
    exec(compile(src.replace(orig, bad), f"<mutant {fn}>", "exec"), ns)
    monkeypatch.setattr(A, fn, ns[fn])
    results = P.run_all()
    failed = [k for k, (ok, _) in results.items() if not ok]
    assert failed, f"no pin caught mutant '{what}'"
