"""GPU parity of the prefill forward over a paged K/V cache (mi_attn_fwd with
a page table, through the C ABI) against the float64 oracle: dense and packed
queries, ragged key counts, every head dim and several page sizes; the paged
and contiguous layouts give bit-identical results; a page id outside the cache
poisons only its own sequence."""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def run_paged(mi, w, page_table=None, **kw):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    pt = dev_i32(w.page_table if page_table is None else page_table)
    extra = {}
    if w.cu_seqlens_q is not None:
        extra.update(cu_seqlens_q=dev_i32(w.cu_seqlens_q), max_seqlen_q=w.max_seqlen_q)
    su = None if w.seqused_k is None else dev_i32(w.seqused_k)
    out, lse = mi.mi_attn_fwd(q, k, v, page_table=pt, seqused_k=su,
                              softmax_scale=w.softmax_scale, causal=w.causal,
                              window_left=w.window_left, window_right=w.window_right,
                              **extra, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_paged(w, page_table=None):
    return OA.paged_prefill(f64(w.q), f64(w.k), f64(w.v),
                            w.page_table if page_table is None else page_table, w.seqused_k,
                            w.softmax_scale, w.causal, w.window_left, w.window_right,
                            cu_seqlens_q=w.cu_seqlens_q)


CASES = [
    # (name, B, Hq, Hkv, D, page_size, pages_per_seq, seqused_k, seqlen_q | seqlens_q, causal, wl, wr)
    ("d128_page64_causal_ragged", 3, 8, 2, 128, 64, 6, [300, 384, 77], 64, True, None, None),
    ("d128_page256_window", 2, 8, 4, 128, 256, 3, [700, 513], 200, True, 150, None),
    ("d64_page64_noncausal", 2, 4, 4, 64, 64, 4, [250, 129], 40, False, None, None),
    ("d256_page128_causal", 2, 4, 2, 256, 128, 4, [450, 300], 120, True, None, None),
    ("d256_page64_window_both", 1, 4, 1, 256, 64, 5, [320], 90, False, 40, 12),
    ("d128_full_rows_no_seqused", 2, 8, 2, 128, 128, 2, None, 100, True, None, None),
    ("d128_packed_q", 4, 8, 2, 128, 64, 5, [300, 0, 190, 64], [100, 7, 0, 64], True, None, None),
    ("d256_packed_q_window", 3, 4, 2, 256, 128, 3, [380, 128, 250], [90, 128, 1], True, 60, None),
    # more sequences than a wave has lanes: the work-item search reads
    # cu_seqlens_q and seqused_k 64 sequences at a time
    ("d128_packed_q_over_64_seqs", 70, 4, 2, 128, 64, 2, [(i * 29) % 128 for i in range(70)],
     [min((i * 13) % 21 if i % 9 else 0, (i * 29) % 128) for i in range(70)], True, None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_prefill_elementwise(gpu_lib, case):
    name, B, Hq, Hkv, D, ps, pps, used, sq, causal, wl, wr = case
    print(f"[case] {name}", flush=True)
    kw = dict(seqlens_q=sq) if isinstance(sq, list) else dict(seqlen_q=sq)
    w = W.paged_prefill_case(zlib.crc32(name.encode()) % 10000, B, Hq, Hkv, D, ps, pps, used,
                             num_pages=B * pps + 3, causal=causal, window_left=wl,
                             window_right=wr, name=name, **kw)
    out, lse = run_paged(gpu_lib, w)
    o_ref, l_ref = oracle_paged(w)
    st = check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name)
    print(name, st)


def test_chunked_prefill_size(gpu_lib):
    """512 new tokens per sequence after a 1536-token cached prefix, 256-token
    pages in a permuted table, GQA 16/2, D128."""
    w = W.paged_prefill_case(31, 2, 16, 2, 128, 256, 8, [2048, 1900], seqlen_q=512,
                             causal=True, name="chunked_prefill")
    out, lse = run_paged(gpu_lib, w)
    o_ref, l_ref = oracle_paged(w)
    print(check(host_f64(out), o_ref, host_f64(lse), l_ref, what=w.name))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_paged_equals_contiguous_bitwise(gpu_lib, d):
    """The same keys read through a permuted page table or from a contiguous
    (B, Sk, Hkv, D) layout give bit-identical outputs (same tiles, same order)."""
    B, Hq, Hkv, ps, pps, Sq = 2, 4, 2, 64, 5, 150
    w = W.paged_prefill_case(40 + d, B, Hq, Hkv, d, ps, pps, None, seqlen_q=Sq, causal=True)
    o1, l1 = run_paged(gpu_lib, w)
    k = np.stack([w.k[w.page_table[b]].reshape(pps * ps, Hkv, d) for b in range(B)])
    v = np.stack([w.v[w.page_table[b]].reshape(pps * ps, Hkv, d) for b in range(B)])
    o2, l2 = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(k), dev_bf16(v),
                                 softmax_scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_bad_page_id_poisons_only_its_sequence(gpu_lib):
    """A page id outside [0, num_pages) is never dereferenced: the kernel's
    page check turns that sequence's rows into NaN; the others are exact."""
    w = W.paged_prefill_case(50, 3, 4, 2, 128, 64, 4, [200, 256, 100], seqlen_q=80,
                             causal=True, num_pages=12)
    bad = w.page_table.copy()
    bad[1, 2] = 12          # == num_pages: out of range
    out, lse = run_paged(gpu_lib, w, page_table=bad)
    o, l = host_f64(out), host_f64(lse)
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(l[1]))
    o_ref, l_ref = oracle_paged(w)
    for b in (0, 2):
        check(o[b], o_ref[b], l[b], l_ref[b], what=f"seq {b}")
    with pytest.raises(gpu_lib.MiAttnError):
        run_paged(gpu_lib, w, page_table=bad, check_bounds=True)
