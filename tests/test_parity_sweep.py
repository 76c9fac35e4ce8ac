"""Seeded random-shape sweep (GPU, through the C ABI) against the float64
oracle: shapes, head dims, GQA ratios, masks, ragged lengths and page sizes
drawn from a fixed generator, so every run checks the same cases. It covers
combinations the hand-written cases do not name: each case is small (at most
a few hundred rows) and compared element by element under the stated
tolerance (tests/gpu_util.py for outputs, tests/test_parity_bwd.py for
gradients)."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64
from tests.test_parity_bwd import check_grad

pytestmark = pytest.mark.gpu

DIMS = [64, 96, 128, 192, 256]


def _heads(rng):
    hkv = int(rng.choice([1, 2, 4]))
    r = int(rng.choice([1, 2, 3, 4, 8]))
    return hkv * r, hkv


def _mask(rng):
    kind = int(rng.integers(0, 4))
    if kind == 0:
        return False, None, None
    if kind == 1:
        return True, None, None
    if kind == 2:
        return True, int(rng.integers(0, 200)), None
    return False, int(rng.integers(0, 150)), int(rng.integers(0, 60))


@pytest.mark.parametrize("i", range(24))
def test_sweep_dense_and_varlen(gpu_lib, i):
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice(DIMS))
    hq, hkv = _heads(rng)
    causal, wl, wr = _mask(rng)
    if i % 2 == 0:
        B = int(rng.integers(1, 4))
        sq, sk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        print(f"[case] sweep dense {i}: B{B} Sq{sq} Sk{sk} H{hq}/{hkv} D{d} causal={causal} "
              f"wl={wl} wr={wr}", flush=True)
        w = W.dense_case(8000 + i, B, sq, sk, hq, hkv, d, causal=causal, window_left=wl,
                         window_right=wr)
        out, lse = gpu_lib.mi_attn_fwd(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                       softmax_scale=w.softmax_scale, causal=causal,
                                       window_left=wl, window_right=wr)
        torch.cuda.synchronize()
        fn = lambda v: OA.attention_dense(f64(w.q), f64(w.k), v, w.softmax_scale, causal, wl, wr)
    else:
        n = int(rng.integers(1, 7))
        lq = [int(x) for x in rng.integers(0, 200, n)]
        lk = [int(x) for x in rng.integers(0, 250, n)]
        print(f"[case] sweep varlen {i}: q{lq} k{lk} H{hq}/{hkv} D{d} causal={causal} "
              f"wl={wl} wr={wr}", flush=True)
        w = W.varlen_case(8000 + i, lq, lk, hq, hkv, d, causal=causal, window_left=wl,
                          window_right=wr)
        out, lse = gpu_lib.mi_attn_fwd(
            dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), cu_seqlens_q=dev_i32(w.cu_seqlens_q),
            cu_seqlens_k=dev_i32(w.cu_seqlens_k), max_seqlen_q=max(lq), max_seqlen_k=max(lk),
            softmax_scale=w.softmax_scale, causal=causal, window_left=wl, window_right=wr)
        torch.cuda.synchronize()
        fn = lambda v: OA.attention_varlen(f64(w.q), f64(w.k), v, w.cu_seqlens_q,
                                           w.cu_seqlens_k, w.softmax_scale, causal, wl, wr)
    o_ref, l_ref = fn(f64(w.v))
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"sweep {i}",
          absv=lambda: fn(np.abs(f64(w.v)))[0])


@pytest.mark.parametrize("i", range(12))
def test_sweep_paged_prefill(gpu_lib, i):
    rng = np.random.default_rng(7100 + i)
    d = int(rng.choice(DIMS))
    hq, hkv = _heads(rng)
    causal, wl, wr = _mask(rng)
    ps = int(rng.choice([64, 128, 256]))
    B = int(rng.integers(1, 4))
    pps = int(rng.integers(1, 5))
    used = [int(x) for x in rng.integers(0, ps * pps + 1, B)]
    lq = [int(x) for x in rng.integers(0, 150, B)]
    print(f"[case] sweep paged {i}: page{ps} x{pps} used{used} q{lq} H{hq}/{hkv} D{d} "
          f"causal={causal} wl={wl} wr={wr}", flush=True)
    w = W.paged_prefill_case(8100 + i, B, hq, hkv, d, ps, pps, used, seqlens_q=lq,
                             num_pages=B * pps + 2, causal=causal, window_left=wl,
                             window_right=wr)
    out, lse = gpu_lib.mi_attn_fwd(
        dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), page_table=dev_i32(w.page_table),
        seqused_k=dev_i32(w.seqused_k), cu_seqlens_q=dev_i32(w.cu_seqlens_q),
        max_seqlen_q=max(lq), softmax_scale=w.softmax_scale, causal=causal, window_left=wl,
        window_right=wr)
    torch.cuda.synchronize()
    fn = lambda v: OA.paged_prefill(f64(w.q), f64(w.k), v, w.page_table, w.seqused_k,
                                    w.softmax_scale, causal, wl, wr, cu_seqlens_q=w.cu_seqlens_q)
    o_ref, l_ref = fn(f64(w.v))
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"sweep paged {i}",
          absv=lambda: fn(np.abs(f64(w.v)))[0])


@pytest.mark.parametrize("i", range(12))
def test_sweep_decode(gpu_lib, i):
    rng = np.random.default_rng(7200 + i)
    d = int(rng.choice(DIMS))
    hq, hkv = _heads(rng)
    ps = int(rng.choice([16, 32, 48, 64, 128, 256]))
    B = int(rng.integers(1, 5))
    pps = int(rng.integers(1, 8))
    used = [int(x) for x in rng.integers(0, ps * pps + 1, B)]
    splits = int(rng.integers(0, 9))
    fp8 = i % 3 == 2
    print(f"[case] sweep decode {i}: page{ps} x{pps} used{used} H{hq}/{hkv} D{d} "
          f"splits{splits} fp8={fp8}", flush=True)
    if fp8:
        w = W.paged_decode_fp8_case(8200 + i, B, hq, hkv, d, ps, pps, num_pages=B * pps + 1,
                                    seqused_k=used, num_splits=splits)
        kc = torch.from_numpy(w.k).cuda().view(torch.float8_e4m3fn)
        vc = torch.from_numpy(w.v).cuda().view(torch.float8_e4m3fn)
        kd, vd = torch.from_numpy(w.k_descale).cuda(), torch.from_numpy(w.v_descale).cuda()
        k64, v64 = OA.e4m3_decode(w.k), OA.e4m3_decode(w.v)
    else:
        w = W.paged_decode_case(8200 + i, B, hq, hkv, d, ps, pps, num_pages=B * pps + 1,
                                seqused_k=used, num_splits=splits)
        kc, vc, kd, vd = dev_bf16(w.k), dev_bf16(w.v), None, None
        k64, v64 = f64(w.k), f64(w.v)
    out, lse = gpu_lib.mi_attn_decode_splitkv(dev_bf16(w.q), kc, vc, dev_i32(w.page_table),
                                              seqused_k=dev_i32(w.seqused_k),
                                              softmax_scale=w.softmax_scale, num_splits=splits,
                                              k_descale=kd, v_descale=vd, check_bounds=True)
    torch.cuda.synchronize()
    fn = lambda v: OA.paged_decode(f64(w.q), k64, v, w.page_table, w.seqused_k,
                                   w.softmax_scale, num_splits=1, k_descale=w.k_descale,
                                   v_descale=w.v_descale)[:2]
    o_ref, l_ref = fn(v64)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"sweep decode {i}",
          absv=lambda: fn(np.abs(v64))[0])


@pytest.mark.parametrize("i", range(10))
def test_sweep_backward(gpu_lib, i):
    rng = np.random.default_rng(7300 + i)
    d = int(rng.choice(DIMS))
    hq, hkv = _heads(rng)
    causal, wl, wr = _mask(rng)
    B = int(rng.integers(1, 3))
    sq, sk = int(rng.integers(1, 260)), int(rng.integers(1, 260))
    print(f"[case] sweep backward {i}: B{B} Sq{sq} Sk{sk} H{hq}/{hkv} D{d} causal={causal} "
          f"wl={wl} wr={wr}", flush=True)
    w = W.dense_case(8300 + i, B, sq, sk, hq, hkv, d, causal=causal, window_left=wl,
                     window_right=wr)
    g = W.grad_output(8300 + i, (B, sq, hq, d))
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    kw = dict(softmax_scale=w.softmax_scale, causal=causal, window_left=wl, window_right=wr)
    out, lse = gpu_lib.mi_attn_fwd(q, k, v, **kw)
    dq, dk, dv = gpu_lib.mi_attn_bwd(q, k, v, out, dev_bf16(g), lse, **kw)
    torch.cuda.synchronize()
    ref = OA.attention_dense_backward(f64(w.q), f64(w.k), f64(w.v), f64(g), w.softmax_scale,
                                      causal=causal, window_left=wl, window_right=wr)
    for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(host_f64(got), r, f"sweep backward {i} {nm}")
