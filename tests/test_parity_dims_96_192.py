"""GPU parity of the prefill forward at head dims 96 and 192 (mi_attn_fwd
through the C ABI; the head-dim-128 and -256 kernels in their LDS layouts,
reading only the real columns) against the float64 oracle: dense causal and
non-causal, GQA, ragged tails, packed sequences, a paged cache, softcap and
a learnable sink. Tolerance as for every forward (tests/gpu_util.py)."""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu

DENSE = [
    # (name, B, Sq, Sk, Hq, Hkv, D, causal, wl)
    ("d96_causal_gqa4", 1, 333, 333, 8, 2, 96, True, None),
    ("d96_noncausal_sq_lt_sk", 2, 100, 257, 4, 4, 96, False, None),
    ("d96_window", 1, 300, 300, 4, 1, 96, True, 50),
    ("d192_causal_gqa2", 1, 300, 300, 4, 2, 192, True, None),
    ("d192_noncausal_ragged", 2, 130, 190, 2, 1, 192, False, None),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_dims_dense(gpu_lib, case):
    name, B, Sq, Sk, Hq, Hkv, D, causal, wl = case
    print(f"[case] dims {name}", flush=True)
    w = W.dense_case(zlib.crc32(name.encode()) % 10000, B, Sq, Sk, Hq, Hkv, D, causal=causal,
                     window_left=wl)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), causal=causal,
                                   window_left=wl)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_dense(f64(w.q), f64(w.k), f64(w.v), w.softmax_scale, causal=causal,
                                      window_left=wl)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))


@pytest.mark.parametrize("d", [96, 192])
def test_dims_varlen_paged_softcap_sink(gpu_lib, d):
    print(f"[case] dims {d} varlen / paged / softcap / sink", flush=True)
    lens = [1, 150, 0, 77]
    w = W.varlen_case(700 + d, lens, lens, 4, 2, d, causal=True)
    sink = W.round_to_bf16_bits(np.array([0.5, -1.0, 2.0, 0.0], dtype=np.float32))
    kw = dict(cu_seqlens_q=dev_i32(w.cu_seqlens_q), cu_seqlens_k=dev_i32(w.cu_seqlens_k),
              max_seqlen_q=max(lens), max_seqlen_k=max(lens), causal=True, softcap=2.0,
              learnable_sink=dev_bf16(sink))
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_varlen(f64(w.q), f64(w.k), f64(w.v), w.cu_seqlens_q,
                                       w.cu_seqlens_k, w.softmax_scale, causal=True,
                                       softcap=2.0, sink=f64(sink))
    print("varlen", check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"varlen d{d}"))
    wp = W.paged_prefill_case(800 + d, 2, 4, 2, d, 64, 4, [250, 65], seqlen_q=70, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(wp.q), dev_bf16(wp.k), dev_bf16(wp.v),
                                   page_table=dev_i32(wp.page_table),
                                   seqused_k=dev_i32(wp.seqused_k), causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.paged_prefill(f64(wp.q), f64(wp.k), f64(wp.v), wp.page_table, wp.seqused_k,
                                    wp.softmax_scale, causal=True)
    print("paged", check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"paged d{d}"))


@pytest.mark.parametrize("d,hq,hkv,s", [(96, 32, 4, 4096), (192, 16, 2, 8192)])
def test_dims_full_size_sampled(gpu_lib, d, hq, hkv, s):
    """The bench's D96 (GQA 32/4, S4096) and D192 (GQA 16/2, S8192) causal prefills:
    sampled query rows of three heads against the oracle row by row."""
    print(f"[case] dims {d} full size", flush=True)
    w = W.dense_case(1006 if d == 96 else 1007, 1, s, s, hq, hkv, d, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), causal=True)
    torch.cuda.synchronize()
    pos = np.array([0, 1, 63, 64, 127, 128, 1000, s // 2, s - 2, s - 1])
    q, k, v = f64(w.q[0]), f64(w.k[0]), f64(w.v[0])
    o_gpu = host_f64(out[0][torch.as_tensor(pos)])
    l_gpu = host_f64(lse[0][:, torch.as_tensor(pos)])
    r = hq // hkv
    for h in (0, hq // 2 + 1, hq - 1):
        g = h // r
        o_ref, l_ref = OA.attention_rows(q[pos, h], pos, k[:, g], v[:, g], w.softmax_scale, s, True)
        check(o_gpu[:, h], o_ref, l_gpu[h], l_ref, what=f"d{d} full size head {h}")
