"""The no-allocation decode entry point (mi_attn_decode_splitkv_noalloc,
through the C ABI) against the workspace entry point it shares its kernels
with, and against the float64 oracle: two calls in a row, the second on a
smaller input, then a request too large for the static scratch."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def _inputs(w):
    return (dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.page_table),
            dev_i32(w.seqused_k))


def _compare(mi, w, num_splits, window_left=None):
    q, kc, vc, pt, su = _inputs(w)
    B, hq, d = q.shape
    out_ws, lse_ws = mi.mi_attn_decode_splitkv(q, kc, vc, pt, seqused_k=su,
                                               softmax_scale=w.softmax_scale,
                                               num_splits=num_splits, window_left=window_left)
    out = torch.full((B, hq, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, hq), 7.0, dtype=torch.float32, device="cuda")
    mi.mi_attn_decode_splitkv_noalloc(q, kc, vc, pt, seqused_k=su, out=out, lse=lse,
                                      softmax_scale=w.softmax_scale, num_splits=num_splits,
                                      window_left=window_left)
    torch.cuda.synchronize()
    # same kernels, same split count: the same bits
    assert torch.equal(out.view(torch.int16), out_ws.view(torch.int16))
    assert torch.equal(lse.isneginf(), lse_ws.isneginf())
    assert torch.equal(lse[~lse.isneginf()], lse_ws[~lse_ws.isneginf()])
    o_ref, l_ref, _, _ = OA.paged_decode(f64(w.q), f64(w.k), f64(w.v), w.page_table,
                                         w.seqused_k, w.softmax_scale, num_splits=1,
                                         window_left=window_left)
    return check(host_f64(out), o_ref, host_f64(lse), l_ref, what="noalloc")


def test_noalloc_decode_matches_workspace_decode(gpu_lib):
    print("[case] no-alloc decode: large then smaller input", flush=True)
    # first call: GQA 8, D128, 256-token pages, ragged lengths incl. an empty one
    w1 = W.paged_decode_case(501, 6, 32, 4, 128, 256, 12, num_pages=80,
                             seqused_k=[3072, 1, 0, 2900, 1500, 777], num_splits=0)
    print("first", _compare(gpu_lib, w1, 0))
    # second call, smaller: D64, 16-token pages, explicit split count, a window;
    # the scratch still holds the first call's partials
    w2 = W.paged_decode_case(502, 2, 4, 2, 64, 16, 9, seqused_k=[140, 33], num_splits=5)
    print("second", _compare(gpu_lib, w2, 5, window_left=40))


def test_noalloc_decode_rejects_partials_beyond_scratch(gpu_lib):
    print("[case] no-alloc decode: too large for the scratch", flush=True)
    B, hq, hkv, d = 512, 64, 8, 256
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, 256, hkv, d, dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
    # 512 * 64 rows x 16 splits x (256 + 1) floats: about 539 MB of partials
    with pytest.raises(gpu_lib.MiAttnError) as e:
        gpu_lib.mi_attn_decode_splitkv_noalloc(q, kc, kc, pt, out=out, num_splits=16)
    assert e.value.code == gpu_lib.MI_ATTN_EWORKSPACE
    assert "scratch" in str(e.value)
