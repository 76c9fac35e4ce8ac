"""GPU parity of the learnable sink (one bf16 logit per query head; through
the C ABI) in every path that applies it: the ping-pong prefill kernel
(D64/D128), the pipelined one (D256), packed and paged queries, and the split
decode's combine (bf16 and fp8 caches), against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def sink_bits(seed, hq):
    """bf16 sink logits in [-2, 3] (bit patterns), drawn from their own seed."""
    rng = np.random.default_rng(seed)
    return W.round_to_bf16_bits(rng.uniform(-2.0, 3.0, hq).astype(np.float32))


@pytest.mark.parametrize("name,B,Sq,Sk,Hq,Hkv,D,causal,wl", [
    ("d128_causal_gqa4", 2, 300, 300, 8, 2, 128, True, None),
    ("d64_sq_gt_sk_empty_rows", 1, 200, 90, 4, 2, 64, True, None),
    ("d256_window", 1, 260, 260, 4, 2, 256, True, 70),
])
def test_sink_dense(gpu_lib, name, B, Sq, Sk, Hq, Hkv, D, causal, wl):
    print(f"[case] sink {name}", flush=True)
    w = W.dense_case(61 + D, B, Sq, Sk, Hq, Hkv, D, causal=causal, window_left=wl)
    sk = sink_bits(7 + D, Hq)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   softmax_scale=w.softmax_scale, causal=causal, window_left=wl,
                                   learnable_sink=dev_bf16(sk))
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_dense(f64(w.q), f64(w.k), f64(w.v), w.softmax_scale, causal, wl,
                                      None, sink=f64(sk))
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))
    if Sq > Sk:  # rows with no visible key: O = 0, LSE = the sink
        rows = Sq - Sk
        assert np.all(host_f64(out)[:, :rows] == 0)
        assert np.allclose(host_f64(lse)[:, :, :rows], f64(sk)[None, :, None], atol=1e-6, rtol=0)


def test_sink_varlen_and_paged(gpu_lib):
    w = W.varlen_case(71, [120, 0, 333], [120, 0, 333], 8, 2, 128, causal=True)
    sk = sink_bits(72, 8)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   cu_seqlens_q=dev_i32(w.cu_seqlens_q),
                                   cu_seqlens_k=dev_i32(w.cu_seqlens_k),
                                   max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k,
                                   softmax_scale=w.softmax_scale, causal=True,
                                   learnable_sink=dev_bf16(sk))
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_varlen(f64(w.q), f64(w.k), f64(w.v), w.cu_seqlens_q,
                                       w.cu_seqlens_k, w.softmax_scale, True, sink=f64(sk))
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="varlen")
    wp = W.paged_prefill_case(73, 2, 8, 2, 128, 64, 4, [200, 256], seqlen_q=70, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(wp.q), dev_bf16(wp.k), dev_bf16(wp.v),
                                   page_table=dev_i32(wp.page_table),
                                   seqused_k=dev_i32(wp.seqused_k),
                                   softmax_scale=wp.softmax_scale, causal=True,
                                   learnable_sink=dev_bf16(sk))
    torch.cuda.synchronize()
    o_ref, l_ref = OA.paged_prefill(f64(wp.q), f64(wp.k), f64(wp.v), wp.page_table, wp.seqused_k,
                                    wp.softmax_scale, True, sink=f64(sk))
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="paged")


@pytest.mark.parametrize("D,ps,pps", [(128, 256, 4), (96, 64, 16), (192, 32, 32), (256, 48, 21)],
                         ids=["stream_d128", "stream_d96", "stream_d192", "tile_d256_page48"])
@pytest.mark.parametrize("fp8", [False, True])
def test_sink_decode(gpu_lib, fp8, D, ps, pps):
    B, Hq, Hkv = 3, 16, 2
    sk = sink_bits(80, Hq)
    if fp8:
        w = W.paged_decode_fp8_case(81, B, Hq, Hkv, D, ps, pps, seqused_k=[1000, 1, 513],
                                    num_splits=4)
        kc = torch.from_numpy(w.k).cuda().view(torch.float8_e4m3fn)
        vc = torch.from_numpy(w.v).cuda().view(torch.float8_e4m3fn)
        extra = dict(k_descale=torch.from_numpy(w.k_descale).cuda(),
                     v_descale=torch.from_numpy(w.v_descale).cuda())
        kd, vd = OA.e4m3_decode(w.k), OA.e4m3_decode(w.v)
    else:
        w = W.paged_decode_case(81, B, Hq, Hkv, D, ps, pps, seqused_k=[1000, 1, 513], num_splits=4)
        kc, vc, extra = dev_bf16(w.k), dev_bf16(w.v), {}
        kd, vd = f64(w.k), f64(w.v)
    out, lse = gpu_lib.mi_attn_decode_splitkv(dev_bf16(w.q), kc, vc, dev_i32(w.page_table),
                                              seqused_k=dev_i32(w.seqused_k),
                                              softmax_scale=w.softmax_scale, num_splits=4,
                                              learnable_sink=dev_bf16(sk), **extra)
    torch.cuda.synchronize()
    o_ref, l_ref, _, _ = OA.paged_decode(f64(w.q), kd, vd, w.page_table, w.seqused_k,
                                         w.softmax_scale, num_splits=1, k_descale=w.k_descale,
                                         v_descale=w.v_descale, sink=f64(sk))
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"decode fp8={fp8}")


def test_sink_minus_inf_is_no_sink(gpu_lib):
    w = W.dense_case(90, 1, 150, 150, 4, 2, 128, causal=True)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    o1, l1 = gpu_lib.mi_attn_fwd(q, k, v, causal=True)
    ninf = torch.full((4,), float("-inf"), dtype=torch.bfloat16, device="cuda")
    o2, l2 = gpu_lib.mi_attn_fwd(q, k, v, causal=True, learnable_sink=ninf)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
