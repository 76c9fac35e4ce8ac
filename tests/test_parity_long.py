"""GPU parity at long context lengths, where offsets and row indices pass
the ranges the benchmark shapes reach: a causal prefill of 65,536 tokens and
a split-KV decode over a 1,048,576-key paged cache, each checked against the
float64 oracle on sampled rows (every row's full score vector)."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def test_causal_prefill_s65536_sampled_rows(gpu_lib):
    """B1, GQA 8/1, S 65,536, D128, causal: rows at tile and half boundaries and
    the last row, three heads."""
    print("[case] long causal prefill S65536", flush=True)
    S, Hq, Hkv, D = 65536, 8, 1, 128
    w = W.dense_case(65536, 1, S, S, Hq, Hkv, D, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                   softmax_scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    o, l = host_f64(out), host_f64(lse)
    q, k, v = f64(w.q), f64(w.k), f64(w.v)
    rows = [0, 1, 63, 64, 12345, 32767, 32768, 65472, 65535]
    got_o, got_l, want_o, want_l, want_a = [], [], [], [], []
    for h in (0, 3, 7):
        for i in rows:
            s = w.softmax_scale * (k[0, :i + 1, 0] @ q[0, i, h])
            m = s.max()
            p = np.exp(s - m)
            want_o.append((p @ v[0, :i + 1, 0]) / p.sum())
            want_l.append(m + np.log(p.sum()))
            want_a.append((p @ np.abs(v[0, :i + 1, 0])) / p.sum())
            got_o.append(o[0, i, h])
            got_l.append(l[0, h, i])
    # the mean bound applies to the sampled rows together (a row with one or
    # two visible keys carries O(1) outputs and their plain bf16 rounding)
    print(check(np.array(got_o), np.array(want_o), np.array(got_l), np.array(want_l),
                what="sampled rows", absv=lambda: np.array(want_a)))


def test_decode_one_million_keys(gpu_lib):
    """One sequence of 1,048,576 keys (2,048 pages of 512 tokens in a
    permuted table) and one of 777,777, GQA 4/1, D64, the split heuristic."""
    print("[case] long decode 1M keys", flush=True)
    B, Hq, Hkv, D, ps, pps = 2, 4, 1, 64, 512, 2048
    w = W.paged_decode_case(1 << 20, B, Hq, Hkv, D, ps, pps, seqused_k=[1 << 20, 777777],
                            num_splits=0)
    out, lse = gpu_lib.mi_attn_decode_splitkv(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                              dev_i32(w.page_table),
                                              seqused_k=dev_i32(w.seqused_k),
                                              softmax_scale=w.softmax_scale, num_splits=0,
                                              check_bounds=True)
    torch.cuda.synchronize()
    o_ref, l_ref, _, _ = OA.paged_decode(f64(w.q), f64(w.k), f64(w.v), w.page_table,
                                         w.seqused_k, w.softmax_scale, num_splits=1)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="decode 1M keys")
