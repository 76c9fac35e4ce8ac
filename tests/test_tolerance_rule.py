"""CPU checks of the parity tolerance rule (tests/gpu_util.check).

A model of the kernels' rounding (P rounded to bf16 before P V, O rounded to
bf16, everything else exact) on a packed batch of 150 short causal sequences
has an element whose error against the float64 oracle passes 1e-2 (a row
with two visible keys and large |v|). The rule admits it through the bf16-P
bound and nothing else; a planted error just past that bound, or on an
element the bound does not cover, is rejected.
"""
import numpy as np
import pytest

import oracle.attention as OA
import workloads as W
from tests.gpu_util import MAX_ABS, check, f64


def _rne_bf16(x):
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


@pytest.fixture(scope="module")
def case():
    lens = [(i * 37) % 97 if i % 11 else 0 for i in range(149)] + [390]
    w = W.varlen_case(len("over_64_sequences"), lens, lens, 8, 2, 128, causal=True)
    q, k, v = f64(w.q), f64(w.k), f64(w.v)
    o_ref, l_ref = OA.attention_varlen(q, k, v, w.cu_seqlens_q, w.cu_seqlens_k, w.softmax_scale,
                                       True, None, None)
    absv = OA.attention_varlen(q, k, np.abs(v), w.cu_seqlens_q, w.cu_seqlens_k,
                               w.softmax_scale, True, None, None)[0]
    # the rounding model, per sequence and head, from the score definition
    o_mod = np.zeros_like(o_ref)
    cu = w.cu_seqlens_q
    for b in range(len(lens)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        for h in range(8):
            g = h // 4
            s = w.softmax_scale * q[s0:s1, h] @ k[s0:s1, g].T
            s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o_mod[s0:s1, h] = _rne_bf16((_rne_bf16(p) @ v[s0:s1, g]) / p.sum(axis=1, keepdims=True))
    return o_mod, o_ref, l_ref, absv


def test_bf16_p_model_passes_only_through_the_bound(case):
    o_mod, o_ref, l_ref, absv = case
    err = np.abs(o_mod - o_ref)
    assert (err > MAX_ABS).sum() >= 1  # the effect the rule is for does occur
    with pytest.raises(AssertionError):
        check(o_mod, o_ref, l_ref, l_ref, what="model without |V| output")
    stats = check(o_mod, o_ref, l_ref, l_ref, what="model", absv=lambda: absv)
    assert stats["bf16_p_bound_elements"] == int((err > MAX_ABS).sum())


def test_planted_errors_are_rejected(case):
    o_mod, o_ref, l_ref, absv = case
    i = np.unravel_index(np.argmax(np.abs(o_mod - o_ref)), o_ref.shape)
    e = 2.0 ** -9 * absv[i]
    bound = e + 0.5 * 2.0 ** (np.frexp(abs(o_ref[i]) + e)[1] - 8) + 1e-5
    bad = o_mod.copy()
    bad[i] = o_ref[i] + np.sign(o_mod[i] - o_ref[i]) * (bound * 1.01)
    with pytest.raises(AssertionError):
        check(bad, o_ref, l_ref, l_ref, what="past the bound", absv=lambda: absv)
    # a 0.02 error on an element of a long row (tiny bf16-P bound) is rejected
    j = np.unravel_index(np.argmin(absv + (np.abs(o_ref) > 1)), o_ref.shape)
    bad = o_mod.copy()
    bad[j] = o_ref[j] + 0.02
    with pytest.raises(AssertionError):
        check(bad, o_ref, l_ref, l_ref, what="long row", absv=lambda: absv)
