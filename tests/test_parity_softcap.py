"""GPU parity of logit soft-capping (softcap > 0 in mi_attn_fwd and
mi_attn_decode_splitkv through the C ABI) against the float64 oracle, whose
reading caps every scaled score x to cap * tanh(x / cap) (oracle
softcap_scores). Caps of 1 and 5 against scaled scores of about N(0, 1)
make the capping strong and mild. Same tolerance as the uncapped forward
(tests/gpu_util.py): tanh is evaluated in fp32 through exp2 and a
reciprocal, an error of a few 1e-7 of the cap per score."""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu

DENSE = [
    # (name, B, Sq, Sk, Hq, Hkv, D, causal, wl, cap)
    ("d128_causal_gqa4_cap1", 1, 300, 300, 8, 2, 128, True, None, 1.0),
    ("d128_noncausal_cap5", 2, 200, 260, 4, 4, 128, False, None, 5.0),
    ("d64_window_cap2", 1, 333, 333, 4, 1, 64, True, 40, 2.0),
    ("d256_causal_cap1", 1, 257, 257, 4, 2, 256, True, None, 1.0),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_softcap_prefill_dense(gpu_lib, case):
    name, B, Sq, Sk, Hq, Hkv, D, causal, wl, cap = case
    print(f"[case] softcap {name}", flush=True)
    w = W.dense_case(zlib.crc32(name.encode()) % 10000, B, Sq, Sk, Hq, Hkv, D, causal=causal,
                     window_left=wl)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   softmax_scale=w.softmax_scale, causal=causal, window_left=wl,
                                   softcap=cap)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_dense(f64(w.q), f64(w.k), f64(w.v), w.softmax_scale, causal=causal,
                                      window_left=wl, softcap=cap)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))
    # the capping changes the result (the inputs are not in its linear range)
    o_plain, _ = OA.attention_dense(f64(w.q), f64(w.k), f64(w.v), w.softmax_scale, causal=causal,
                                    window_left=wl)
    assert np.abs(o_plain - o_ref).max() > 0.05


def test_softcap_prefill_varlen_and_paged(gpu_lib):
    print("[case] softcap varlen + paged", flush=True)
    lens = [1, 190, 77, 0, 130]
    w = W.varlen_case(515, lens, lens, 8, 2, 128, causal=True)
    kw = dict(cu_seqlens_q=dev_i32(w.cu_seqlens_q), cu_seqlens_k=dev_i32(w.cu_seqlens_k),
              max_seqlen_q=max(lens), max_seqlen_k=max(lens), softmax_scale=w.softmax_scale,
              causal=True, softcap=1.5)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_varlen(f64(w.q), f64(w.k), f64(w.v), w.cu_seqlens_q, w.cu_seqlens_k,
                                       w.softmax_scale, causal=True, softcap=1.5)
    print("varlen", check(host_f64(out), o_ref, host_f64(lse), l_ref, what="varlen softcap"))
    wp = W.paged_prefill_case(616, 2, 8, 2, 128, 64, 5, [300, 129], seqlen_q=100, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(wp.q), dev_bf16(wp.k), dev_bf16(wp.v),
                                   page_table=dev_i32(wp.page_table),
                                   seqused_k=dev_i32(wp.seqused_k),
                                   softmax_scale=wp.softmax_scale, causal=True, softcap=1.5)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.paged_prefill(f64(wp.q), f64(wp.k), f64(wp.v), wp.page_table, wp.seqused_k,
                                    wp.softmax_scale, causal=True, softcap=1.5)
    print("paged", check(host_f64(out), o_ref, host_f64(lse), l_ref, what="paged softcap"))


DECODE = [
    # (name, D, page_size, kv) -- the streaming kernel (page sizes that are multiples
    # of 32) and the tile kernel (other page sizes)
    ("stream_bf16_d128", 128, 64, "bf16"),
    ("stream_fp8_d128", 128, 256, "fp8_e4m3"),
    ("stream_d256", 256, 64, "bf16"),
    ("stream_fp8_d256", 256, 64, "fp8_e4m3"),
    ("stream_d96", 96, 32, "bf16"),
    ("stream_fp8_d192", 192, 64, "fp8_e4m3"),
    ("tile_page48_d128", 128, 48, "bf16"),
    ("tile_page48_d256", 256, 48, "bf16"),
    ("tile_fp8_page16_d192", 192, 16, "fp8_e4m3"),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_softcap_decode(gpu_lib, case):
    name, D, ps, kv = case
    print(f"[case] softcap decode {name}", flush=True)
    seed = zlib.crc32(name.encode()) % 10000
    B, Hq, Hkv, pps = 3, 16, 2, 6
    used = [1, min(200, ps * pps - 5), ps * pps]  # ragged, within the pages' capacity
    if kv == "bf16":
        w = W.paged_decode_case(seed, B, Hq, Hkv, D, ps, pps, seqused_k=used, num_splits=3)
        kc, vc = dev_bf16(w.k), dev_bf16(w.v)
        kd = vd = None
        k64, v64 = f64(w.k), f64(w.v)
    else:
        w = W.paged_decode_fp8_case(seed, B, Hq, Hkv, D, ps, pps, seqused_k=used, num_splits=3)
        kc = torch.from_numpy(w.k).cuda().view(torch.float8_e4m3fn)
        vc = torch.from_numpy(w.v).cuda().view(torch.float8_e4m3fn)
        kd, vd = torch.from_numpy(w.k_descale).cuda(), torch.from_numpy(w.v_descale).cuda()
        k64, v64 = OA.e4m3_decode(w.k), OA.e4m3_decode(w.v)
    out, lse = gpu_lib.mi_attn_decode_splitkv(dev_bf16(w.q), kc, vc, dev_i32(w.page_table),
                                              seqused_k=dev_i32(w.seqused_k),
                                              softmax_scale=w.softmax_scale, num_splits=3,
                                              k_descale=kd, v_descale=vd, softcap=1.0)
    torch.cuda.synchronize()
    o_ref, l_ref, _, _ = OA.paged_decode(f64(w.q), k64, v64, w.page_table, w.seqused_k,
                                         w.softmax_scale, num_splits=1, k_descale=w.k_descale,
                                         v_descale=w.v_descale, softcap=1.0)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))


def test_softcap_zero_is_off_and_huge_cap_is_identity(gpu_lib):
    """softcap = 0 gives the uncapped kernel's exact bits; a cap of 1e4 is
    within the tolerance of the uncapped result."""
    w = W.dense_case(88, 1, 200, 200, 4, 2, 128, causal=True)
    args = (dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v))
    o0, l0 = gpu_lib.mi_attn_fwd(*args, causal=True)
    o1, l1 = gpu_lib.mi_attn_fwd(*args, causal=True, softcap=0.0)
    o2, l2 = gpu_lib.mi_attn_fwd(*args, causal=True, softcap=1e4)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    check(host_f64(o2), host_f64(o0), host_f64(l2), host_f64(l0), what="cap 1e4")


def test_softcap_full_size_sampled(gpu_lib):
    """The causal GQA S4096 D128 workload with softcap 30 (the bench's soft-capped line):
    sampled query rows of heads 0, 13, 31 against the oracle row by row."""
    print("[case] softcap full size", flush=True)
    w = W.standard_config(2)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   softmax_scale=w.softmax_scale, causal=True, softcap=30.0)
    torch.cuda.synchronize()
    S = w.seqlen_q
    pos = np.array([0, 1, 63, 64, 255, 1000, 2047, 2048, 3333, S - 1])
    q, k, v = f64(w.q[0]), f64(w.k[0]), f64(w.v[0])
    o_gpu = host_f64(out[0][torch.as_tensor(pos)])
    l_gpu = host_f64(lse[0][:, torch.as_tensor(pos)])
    r = w.num_heads_q // w.num_heads_kv
    for h in (0, 13, 31):
        g = h // r
        o_ref, l_ref = OA.attention_rows(q[pos, h], pos, k[:, g], v[:, g], w.softmax_scale, S,
                                         True, softcap=30.0)
        check(o_gpu[:, h], o_ref, l_gpu[h], l_ref, what=f"softcap full size head {h}")
