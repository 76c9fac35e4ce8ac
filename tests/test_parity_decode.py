"""GPU parity of the paged split-KV decode and of the combine kernel (through
the C ABI) against the float64 oracle."""
import numpy as np
import pytest
import torch

import exact_attention_45_amd as mi_mod
import oracle.attention as OA
import workloads as W
from tests.gpu_util import bf16_ulp, check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def run_decode(mi, w, num_splits=None, window_left=None, check_bounds=False):
    q, kc, vc = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    pt = dev_i32(w.page_table)
    su = dev_i32(w.seqused_k)
    ns = w.num_splits if num_splits is None else num_splits
    out, lse = mi.mi_attn_decode_splitkv(q, kc, vc, pt, seqused_k=su,
                                         softmax_scale=w.softmax_scale, num_splits=ns,
                                         window_left=window_left, check_bounds=check_bounds)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(w, window_left=None, heads=None):
    o, l, _, _ = OA.paged_decode(f64(w.q), f64(w.k), f64(w.v), w.page_table, w.seqused_k,
                                 w.softmax_scale, num_splits=1, window_left=window_left,
                                 heads=heads)
    return o, l


CASES = [
    # (name, B, Hq, Hkv, D, page_size, pages_per_seq, extra_pages, seqused, splits, wl)
    ("gqa8_page256_ragged", 3, 16, 2, 128, 256, 5, 3, [1, 700, 1280], 4, None),
    ("mha_page16_many_splits", 2, 4, 4, 64, 16, 20, 0, [320, 33], 16, None),
    ("gqa32_page64_heuristic", 2, 32, 1, 128, 64, 12, 5, [768, 500], 0, None),
    ("gqa80_rowblocks_page128", 2, 80, 1, 64, 128, 4, 0, [512, 130], 3, None),
    ("d256_page32", 2, 8, 2, 256, 32, 9, 1, [288, 100], 5, None),
    ("empty_and_tiny", 4, 8, 2, 128, 64, 3, 0, [0, 1, 64, 65], 8, None),
    ("more_splits_than_tiles", 1, 8, 1, 128, 64, 2, 0, [100], 64, None),
    ("window_left", 2, 16, 4, 128, 128, 6, 2, [700, 90], 4, 200),
    ("gqa3_nonpow2", 2, 6, 2, 128, 256, 2, 0, [400, 512], 2, None),
    # head dims 96 and 192 (in the layouts of 128 and 256: the streaming
    # kernel when the page size is a multiple of 32, else the tile kernel)
    ("d96_page16_gqa4", 2, 8, 2, 96, 16, 30, 2, [480, 37], 6, None),
    ("d96_page256_mha", 1, 4, 4, 96, 256, 3, 0, [700], 4, None),
    ("d192_page64_window", 2, 8, 1, 192, 64, 6, 1, [380, 64], 3, 150),
    ("d192_page32_ragged", 3, 16, 2, 192, 32, 10, 0, [1, 320, 129], 5, None),
    # the tile kernel at head dims 192 and 256 (page sizes not multiples of 32)
    ("d192_page16_tile", 2, 16, 2, 192, 16, 25, 0, [390, 17], 4, None),
    ("d256_page48_tile", 2, 8, 2, 256, 48, 8, 1, [380, 47], 3, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_elementwise(gpu_lib, case):
    name, B, Hq, Hkv, D, ps, pps, extra, used, splits, wl = case
    print(f"[case] decode {name}", flush=True)
    w = W.paged_decode_case(len(name) * 7 + B, B, Hq, Hkv, D, ps, pps,
                            num_pages=B * pps + extra, seqused_k=used, num_splits=splits)
    out, lse = run_decode(gpu_lib, w, window_left=wl, check_bounds=True)
    o_ref, l_ref = oracle_decode(w, window_left=wl)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))


def test_full_size_decode(gpu_lib):
    """The paged decode workload (B16, GQA 32/4, D128, Sk 32768, 256-token
    pages, 16 splits), every output element."""
    print("[case] full-size paged decode", flush=True)
    w = W.standard_config(5)
    out, lse = run_decode(gpu_lib, w)
    o_ref, l_ref = oracle_decode(w)
    print(w.name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=w.name))


def test_split_count_does_not_change_result(gpu_lib):
    w = W.paged_decode_case(77, 2, 16, 2, 128, 256, 8, seqused_k=[2048, 1500])
    outs = [run_decode(gpu_lib, w, num_splits=s) for s in (1, 3, 16)]
    o_ref, l_ref = oracle_decode(w)
    for o, l in outs:
        check(host_f64(o), o_ref, host_f64(l), l_ref, what="splits")
    # different partitions agree with each other far inside the tolerance
    d = (outs[0][0].float() - outs[2][0].float()).abs().max().item()
    assert d <= 8e-3


def test_decode_deterministic(gpu_lib):
    w = W.paged_decode_case(78, 2, 16, 2, 128, 64, 8, seqused_k=[512, 300], num_splits=4)
    o1, l1 = run_decode(gpu_lib, w)
    o2, l2 = run_decode(gpu_lib, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_bad_page_id_gives_nan_not_a_fault(gpu_lib):
    """A page id outside the cache is never dereferenced: the affected
    sequence's outputs become NaN, the others stay correct."""
    w = W.paged_decode_case(79, 2, 8, 2, 128, 64, 4, seqused_k=[256, 256], num_splits=2)
    w.page_table = w.page_table.copy()
    w.page_table[0, 3] = 10_000_000
    out, lse = run_decode(gpu_lib, w)
    o = host_f64(out)
    assert np.isnan(o[0]).all() and np.isnan(host_f64(lse)[0]).all()
    good = W.paged_decode_case(79, 2, 8, 2, 128, 64, 4, seqused_k=[256, 256], num_splits=2)
    o_ref, l_ref = oracle_decode(good)
    check(o[1], o_ref[1], host_f64(lse)[1], l_ref[1], what="untouched sequence")


def test_host_bounds_check_rejects_bad_table(gpu_lib):
    w = W.paged_decode_case(80, 1, 8, 2, 128, 64, 2, seqused_k=[128])
    w.page_table = w.page_table.copy()
    w.page_table[0, 1] = -1
    with pytest.raises(mi_mod.MiAttnError) as e:
        run_decode(gpu_lib, w, check_bounds=True)
    assert e.value.code == mi_mod.MI_ATTN_EBOUNDS


@pytest.mark.parametrize("rows,splits,d", [(37, 1, 64), (100, 16, 128), (9, 256, 256),
                                           (64, 5, 128), (20, 7, 96), (33, 17, 192)])
def test_combine_kernel(gpu_lib, rows, splits, d):
    rng = np.random.default_rng(rows * splits + d)
    o_part = rng.standard_normal((rows, splits, d)).astype(np.float32)
    lse_part = (rng.standard_normal((rows, splits)) * 3).astype(np.float32)
    lse_part[rng.random((rows, splits)) < 0.2] = -np.inf   # empty splits
    lse_part[0, :] = -np.inf                               # a row with nothing
    out, lse = gpu_lib.mi_attn_combine(torch.from_numpy(o_part).cuda(),
                                       torch.from_numpy(lse_part).cuda())
    torch.cuda.synchronize()
    # oracle combine expects splits first
    o_ref, l_ref = OA.combine(np.moveaxis(o_part.astype(np.float64), 1, 0),
                              np.moveaxis(lse_part.astype(np.float64), 1, 0))
    # unit-scale synthetic partials: bf16 output rounding alone is ~1e-3 on
    # average, so bound each element by one bf16 ulp of the exact value
    o = host_f64(out)
    assert np.all(np.isfinite(o))
    assert np.all(np.abs(o - o_ref) <= bf16_ulp(o_ref) + 1e-30)
    l = host_f64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(l), ~fin)
    assert np.abs(l[fin] - l_ref[fin]).max() <= 1e-5
    assert np.all(o[0] == 0) and np.isneginf(l[0])


def test_decode_zero_scale(gpu_lib):
    """softmax_scale = 0: uniform weights over each sequence's keys; ragged
    lengths leave masked key slots in the last slice, which must get weight
    0 (not NaN), and an empty sequence gets O = 0, LSE = -inf."""
    print("[case] decode zero scale", flush=True)
    w = W.paged_decode_case(91, 3, 16, 2, 128, 64, 5, seqused_k=[1, 250, 0], num_splits=3,
                            softmax_scale=0.0)
    out, lse = run_decode(gpu_lib, w)
    o_ref, l_ref = oracle_decode(w)
    print("decode scale0", check(host_f64(out), o_ref, host_f64(lse), l_ref, what="scale0"))


def test_decode_rejects_bad_out_and_lse(gpu_lib):
    """Caller-supplied out must be (B, Hq, D) bf16 and lse a contiguous
    float32 (B, Hq) tensor on the same device; the binding refuses anything
    the combine would write past."""
    w = W.paged_decode_case(92, 2, 8, 2, 128, 64, 2, num_splits=2)
    q, kc, vc = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    pt = dev_i32(w.page_table)
    bad = [
        dict(out=torch.empty(2, 4, 128, dtype=torch.bfloat16, device="cuda")),
        dict(out=torch.empty(2, 8, 128, dtype=torch.float16, device="cuda")),
        dict(lse=torch.empty(2, 8, dtype=torch.bfloat16, device="cuda")),
        dict(lse=torch.empty(2, 4, dtype=torch.float32, device="cuda")),
        dict(lse=torch.empty(8, 2, dtype=torch.float32, device="cuda").t()),
        dict(lse=torch.empty(2, 8, dtype=torch.float32)),
    ]
    for kw in bad:
        with pytest.raises(gpu_lib.MiAttnError) as e:
            gpu_lib.mi_attn_decode_splitkv(q, kc, vc, pt, num_splits=2, **kw)
        assert e.value.code == gpu_lib.MI_ATTN_EINVAL, kw


# Several query tokens per sequence (packed by cu_seqlens_q) against the paged
# cache, split along the keys and combined: the queries sit bottom-right at
# the end of each sequence's keys. Reference: the oracle's paged prefill
# (the same definition, no split).
VARLEN_CASES = [
    # (name, B, Hq, Hkv, D, page_size, pages_per_seq, seqused, q_lens, splits, causal, wl)
    ("spec4_causal_gqa8_page256", 3, 16, 2, 128, 256, 5, [700, 1280, 5], [4, 1, 3], 4, True, None),
    ("mixed_noncausal_d64_page16", 4, 8, 2, 64, 16, 20, [320, 33, 0, 100], [2, 8, 0, 5], 0,
     False, None),
    ("window_causal_mha", 2, 4, 4, 128, 64, 6, [384, 200], [8, 6], 3, True, 50),
    ("gqa32_rows_span_blocks", 2, 32, 1, 128, 64, 4, [256, 77], [8, 3], 2, True, None),
    ("more_tokens_than_keys", 1, 8, 2, 128, 64, 2, [3], [6], 2, True, None),
    ("d256_stream_path", 2, 8, 2, 256, 32, 9, [288, 100], [3, 2], 5, True, None),
    ("d256_page48_tile_path", 2, 8, 2, 256, 48, 8, [380, 47], [4, 2], 3, True, None),
    ("page48_tile_path", 2, 8, 2, 128, 48, 8, [380, 47], [5, 1], 3, True, 100),
    ("d96_spec_causal", 2, 8, 2, 96, 64, 5, [300, 17], [4, 2], 3, True, None),
    ("d192_spec_window", 2, 8, 2, 192, 32, 9, [288, 100], [3, 5], 4, True, 60),
]


def run_varlen_decode(mi, w, q_lens, splits, causal, wl, noalloc=False):
    q, kc, vc = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    fn = mi.mi_attn_decode_splitkv_noalloc if noalloc else mi.mi_attn_decode_splitkv
    out, lse = fn(q, kc, vc, dev_i32(w.page_table), seqused_k=dev_i32(w.seqused_k),
                  cu_seqlens_q=dev_i32(w.cu_seqlens_q), max_seqlen_q=max(q_lens),
                  softmax_scale=w.softmax_scale, num_splits=splits, causal=causal,
                  window_left=wl, check_bounds=True)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_decode_elementwise(gpu_lib, case):
    name, B, Hq, Hkv, D, ps, pps, used, q_lens, splits, causal, wl = case
    print(f"[case] varlen decode {name}", flush=True)
    w = W.paged_prefill_case(len(name) * 13 + B, B, Hq, Hkv, D, ps, pps, used, seqlens_q=q_lens)
    out, lse = run_varlen_decode(gpu_lib, w, q_lens, splits, causal, wl)
    o_ref, l_ref = OA.paged_prefill(f64(w.q), f64(w.k), f64(w.v), w.page_table, w.seqused_k,
                                    w.softmax_scale, causal=causal, window_left=wl,
                                    cu_seqlens_q=w.cu_seqlens_q)
    print(name, check(host_f64(out), o_ref, host_f64(lse).T, l_ref, what=name))


def test_varlen_decode_one_token_equals_decode(gpu_lib):
    """cu_seqlens_q with one token per sequence is the plain decode, bit for bit."""
    print("[case] varlen decode with one token per sequence", flush=True)
    w = W.paged_decode_case(95, 3, 16, 2, 128, 64, 6, seqused_k=[384, 200, 1], num_splits=4)
    q, kc, vc = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    pt, su = dev_i32(w.page_table), dev_i32(w.seqused_k)
    o1, l1 = gpu_lib.mi_attn_decode_splitkv(q, kc, vc, pt, seqused_k=su, num_splits=4)
    cu = dev_i32(np.arange(4, dtype=np.int32))
    o2, l2 = gpu_lib.mi_attn_decode_splitkv(q, kc, vc, pt, seqused_k=su, num_splits=4,
                                            cu_seqlens_q=cu, max_seqlen_q=1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_varlen_decode_full_size_speculative(gpu_lib):
    """The paged decode workload's cache (B16, GQA 32/4, D128, Sk 32768,
    permuted 256-token pages) with 4 causal query tokens per sequence (a
    speculative decoding step), split heuristic: sampled heads, every token."""
    print("[case] varlen decode full size, 4 tokens per sequence", flush=True)
    w = W.paged_prefill_case(1005, 16, 32, 4, 128, 256, 128, [32768] * 16, seqlens_q=[4] * 16)
    out, lse = run_varlen_decode(gpu_lib, w, [4] * 16, 0, True, None)
    o_gpu, l_gpu = host_f64(out), host_f64(lse)
    heads = [0, 7, 8, 31]
    r = 8
    for b in (0, 5, 15):
        kb = OA.paged_gather(f64(w.k), w.page_table[b], 32768)
        vb = OA.paged_gather(f64(w.v), w.page_table[b], 32768)
        t0 = int(w.cu_seqlens_q[b])
        vis = OA.visible_mask(4, 32768, True)
        for h in heads:
            o, l = OA.attention_head(f64(w.q[t0:t0 + 4, h]), kb[:, h // r], vb[:, h // r],
                                     w.softmax_scale, vis)
            check(o_gpu[t0:t0 + 4, h], o, l_gpu[t0:t0 + 4, h], l, what=f"seq {b} head {h}")


def test_varlen_decode_noalloc_matches(gpu_lib):
    print("[case] varlen decode through the no-allocation entry point", flush=True)
    case = VARLEN_CASES[0]
    name, B, Hq, Hkv, D, ps, pps, used, q_lens, splits, causal, wl = case
    w = W.paged_prefill_case(len(name) * 13 + B, B, Hq, Hkv, D, ps, pps, used, seqlens_q=q_lens)
    o1, l1 = run_varlen_decode(gpu_lib, w, q_lens, splits, causal, wl)
    o2, l2 = run_varlen_decode(gpu_lib, w, q_lens, splits, causal, wl, noalloc=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.isneginf(), l2.isneginf()) and torch.equal(l1[~l1.isneginf()],
                                                                   l2[~l2.isneginf()])
