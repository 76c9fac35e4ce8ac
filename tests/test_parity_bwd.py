"""GPU parity of the attention backward (mi_attn_bwd through the C ABI)
against the float64 oracle's gradients on the same bf16 inputs.

The forward runs first on the GPU (mi_attn_fwd), and its bf16 output and
float32 LSE feed the backward, as in training. The oracle differentiates the
exact function of the bf16 inputs q, k, v and dO.

Tolerance, per gradient tensor G with reference G_ref:
  max |G - G_ref| <= 2e-2 * max(1, max |G_ref|)
  mean |G - G_ref| <= 5e-3 * max(1, mean |G_ref|)
Derivation: the kernels round P and dS to bf16 before their products
(relative error up to 2**-9 per term), take rowsum(O dO) from the bf16
forward output, and round each gradient to bf16 (half an ulp, up to 2**-9
relative, 2**-10 on average). A gradient element is a sum over keys (dQ) or
over the group's queries (dK, dV); when a few terms dominate it (an early
key under a causal mask, whose probability is about 1/i for query i) the
term errors do not average out and the sum keeps up to 2**-9 of its
magnitude: 2**-9 + 2**-10 = 2.9e-3 of the mean magnitude in all, which the
mean bound covers with a margin of 1.7; single elements stay well inside
2e-2 of the largest one.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 5e-3


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    mx = float(err.max(initial=0.0))
    mean = float(err.mean()) if err.size else 0.0
    scale_max = max(1.0, float(np.abs(ref).max(initial=0.0)))
    scale_mean = max(1.0, float(np.abs(ref).mean()) if ref.size else 0.0)
    assert mx <= MAX_REL * scale_max, f"{what}: max abs {mx:.3e} (ref max {scale_max:.3e})"
    assert mean <= MEAN_REL * scale_mean, f"{what}: mean abs {mean:.3e}"
    return {"max_abs": mx, "mean_abs": mean, "ref_max": scale_max}


def run_dense(mi, w, g):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    kw = dict(softmax_scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
              window_right=w.window_right)
    out, lse = mi.mi_attn_fwd(q, k, v, **kw)
    dq, dk, dv = mi.mi_attn_bwd(q, k, v, out, dev_bf16(g), lse, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


DENSE = [
    # (name, B, Sq, Sk, Hq, Hkv, D, causal, wl, wr)
    ("mha_d64_s200", 2, 200, 200, 4, 4, 64, False, None, None),
    ("gqa4_d128_causal_s333", 1, 333, 333, 8, 2, 128, True, None, None),
    ("causal_sq_lt_sk", 1, 100, 300, 4, 1, 128, True, None, None),
    ("causal_sq_gt_sk_empty_rows", 1, 300, 100, 4, 2, 64, True, None, None),
    ("window_50_10", 2, 257, 257, 4, 2, 128, False, 50, 10),
    ("mqa8_d128_causal", 1, 190, 190, 8, 1, 128, True, None, None),
    ("local_window_causal_d64", 1, 400, 400, 2, 1, 64, True, 64, None),
    ("tiny_one_key", 1, 5, 1, 2, 1, 128, False, None, None),
    # 8 key blocks x 16 KV heads x 4 sequences = 512 workgroups: one split
    # (dK, dV written directly); the cases above take the split path
    ("no_split_mha16_b4_s1024_d64", 4, 1024, 1024, 16, 16, 64, True, None, None),
    # head_dim 256 (paired dK/dV waves, 64-key workgroups): split path,
    # bottom-right window with Sq != Sk, MQA, and 16 key blocks x 16 KV
    # heads x 2 sequences = 512 workgroups (one split)
    ("gqa2_d256_causal_s300", 1, 300, 300, 4, 2, 256, True, None, None),
    ("window_40_7_d256_sq_gt_sk", 2, 257, 200, 2, 1, 256, False, 40, 7),
    ("mqa4_d256_causal_s129", 1, 129, 129, 4, 1, 256, True, None, None),
    ("no_split_mha16_b2_s1024_d256", 2, 1024, 1024, 16, 16, 256, True, None, None),
    # one KV head, four splits: 16 key blocks over 64 workgroups, so two XCDs
    # share each walk with interleaved key blocks
    ("interleaved_xcd_mqa4_d256_s1024", 1, 1024, 1024, 4, 1, 256, True, None, None),
    ("interleaved_xcd_mqa4_d128_s2048", 1, 2048, 2048, 4, 1, 128, True, None, None),
    # head dims 96 and 192 (the layouts of 128 and 256, products over the real columns)
    ("gqa4_d96_causal_s300", 1, 300, 300, 8, 2, 96, True, None, None),
    ("window_30_5_d96_sq_lt_sk", 2, 150, 260, 4, 2, 96, False, 30, 5),
    ("gqa2_d192_causal_s333", 1, 333, 333, 4, 2, 192, True, None, None),
    ("mha_d192_s200_split", 2, 200, 200, 2, 2, 192, False, None, None),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_bwd_dense_elementwise(gpu_lib, case):
    name, B, Sq, Sk, Hq, Hkv, D, causal, wl, wr = case
    print(f"[case] bwd {name}", flush=True)
    seed = zlib.crc32(name.encode()) % 10000
    w = W.dense_case(seed, B, Sq, Sk, Hq, Hkv, D, causal=causal, window_left=wl, window_right=wr)
    g = W.grad_output(seed, (B, Sq, Hq, D))
    dq, dk, dv = run_dense(gpu_lib, w, g)
    ref = OA.attention_dense_backward(f64(w.q), f64(w.k), f64(w.v), f64(g), w.softmax_scale,
                                      causal=causal, window_left=wl, window_right=wr)
    for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        print(name, nm, check_grad(host_f64(got), r, f"{name} {nm}"))


@pytest.mark.parametrize("D", [96, 128, 192, 256])
def test_bwd_varlen_elementwise(gpu_lib, D):
    """Packed sequences with an empty query sequence, a one-token one and
    ragged tails; GQA 4:1, causal (bottom-right per sequence)."""
    print(f"[case] bwd varlen D{D}", flush=True)
    lq, lk = [1, 130, 0, 77, 200], [1, 150, 40, 77, 129]
    w = W.varlen_case(4242 + D, lq, lk, 8, 2, D, causal=True)
    g = W.grad_output(4242 + D, (sum(lq), 8, D))
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    cq, ck = dev_i32(w.cu_seqlens_q), dev_i32(w.cu_seqlens_k)
    kw = dict(cu_seqlens_q=cq, cu_seqlens_k=ck, max_seqlen_q=max(lq), max_seqlen_k=max(lk),
              softmax_scale=w.softmax_scale, causal=True)
    out, lse = gpu_lib.mi_attn_fwd(q, k, v, **kw)
    dq, dk, dv = gpu_lib.mi_attn_bwd(q, k, v, out, dev_bf16(g), lse, **kw)
    torch.cuda.synchronize()
    ref = OA.attention_varlen_backward(f64(w.q), f64(w.k), f64(w.v), f64(g), w.cu_seqlens_q,
                                       w.cu_seqlens_k, w.softmax_scale, causal=True)
    for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        print("varlen", D, nm, check_grad(host_f64(got), r, f"varlen D{D} {nm}"))
    # keys of the sequence with no queries get exactly zero gradients
    k0, k1 = int(w.cu_seqlens_k[2]), int(w.cu_seqlens_k[3])
    assert not host_f64(dk)[k0:k1].any() and not host_f64(dv)[k0:k1].any()


def test_bwd_deterministic_and_strided(gpu_lib):
    """Two calls give identical bits; q/dq as views into a larger buffer
    (non-contiguous head and row strides) give the same result as
    contiguous tensors."""
    print("[case] bwd determinism / strides", flush=True)
    w = W.dense_case(77, 2, 190, 190, 4, 2, 128, causal=True)
    g = W.grad_output(77, (2, 190, 4, 128))
    a = run_dense(gpu_lib, w, g)
    b = run_dense(gpu_lib, w, g)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    out, lse = gpu_lib.mi_attn_fwd(q, k, v, softmax_scale=w.softmax_scale, causal=True)
    big = torch.zeros(2, 190, 6, 128, dtype=torch.bfloat16, device="cuda")
    big[:, :, 1:5] = q
    qv = big[:, :, 1:5]
    dq_big = torch.full((2, 190, 4, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    dqv = dq_big[..., :128]
    dq, dk, dv = gpu_lib.mi_attn_bwd(qv, k, v, out, dev_bf16(g), lse,
                                     softmax_scale=w.softmax_scale, causal=True, dq=dqv)
    torch.cuda.synchronize()
    assert torch.equal(dqv.contiguous().view(torch.int16), a[0].view(torch.int16))
    assert torch.isnan(dq_big[..., 128:].float()).all()  # untouched


def test_bwd_full_size_sampled(gpu_lib):
    """The causal GQA prefill workload's shape (B1, Hq32, Hkv4, S4096, D128):
    dQ rows, and dK / dV rows of sampled keys, against the oracle restricted
    to the query rows (dQ) or key rows (dK, dV) it needs."""
    print("[case] bwd full size", flush=True)
    w = W.standard_config(2)
    B, Sq, Hq, D = w.q.shape
    Hkv = w.k.shape[2]
    g = W.grad_output(w.seed, w.q.shape)
    dq, dk, dv = run_dense(gpu_lib, w, g)
    dq, dk, dv = host_f64(dq), host_f64(dk), host_f64(dv)
    q, k, v, go = f64(w.q), f64(w.k), f64(w.v), f64(g)
    r = Hq // Hkv
    scale = w.softmax_scale
    # dQ of sampled query rows of sampled heads: P and dP of those rows only
    for h in (0, 13, 31):
        gk = h // r
        for i in (0, 1, 777, 2048, 4095):
            s = scale * (k[0, :i + 1, gk] @ q[0, i, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ v[0, :i + 1, gk]
            dp = v[0, :i + 1, gk] @ go[0, i, h]
            ds = p * (dp - o @ go[0, i, h])
            want = scale * (ds @ k[0, :i + 1, gk])
            check_grad(dq[0, i, h], want, f"dq row {i} head {h}")
    # dK / dV of sampled keys of KV head 1: every query head of the group,
    # every query that sees the key (causal: i >= j)
    gk = 1
    keys = (0, 5, 2047, 4095)
    dk_w = np.zeros((len(keys), D))
    dv_w = np.zeros((len(keys), D))
    causal = np.tril(np.ones((Sq, Sq), dtype=bool))
    for h in range(gk * r, gk * r + r):
        s = scale * (q[0, :, h] @ k[0, :, gk].T)
        s[~causal] = -np.inf
        pr = np.exp(s - s.max(axis=1, keepdims=True))
        pr /= pr.sum(axis=1, keepdims=True)
        dpsum = np.sum((pr @ v[0, :, gk]) * go[0, :, h], axis=1)
        for n, j in enumerate(keys):
            ds_j = pr[:, j] * (go[0, :, h] @ v[0, j, gk] - dpsum)
            dv_w[n] += pr[:, j] @ go[0, :, h]
            dk_w[n] += scale * (ds_j @ q[0, :, h])
        del s, pr
    for n, j in enumerate(keys):
        check_grad(dk[0, j, gk], dk_w[n], f"dk key {j}")
        check_grad(dv[0, j, gk], dv_w[n], f"dv key {j}")


def test_bwd_full_size_sampled_d256(gpu_lib):
    """The long causal GQA prefill workload's shape (B1, Hq16, Hkv2, S16384,
    D256): dQ rows of sampled heads, and dK / dV rows of keys in the last 512
    positions (every query that sees them is among the last 512 rows, whose
    probabilities need the whole row of keys)."""
    print("[case] bwd full size d256", flush=True)
    w = W.standard_config(3)
    B, Sq, Hq, D = w.q.shape
    Hkv = w.k.shape[2]
    g = W.grad_output(w.seed, w.q.shape)
    dq, dk, dv = run_dense(gpu_lib, w, g)
    dq, dk, dv = host_f64(dq), host_f64(dk), host_f64(dv)
    q, k, v, go = f64(w.q), f64(w.k), f64(w.v), f64(g)
    r = Hq // Hkv
    scale = w.softmax_scale
    for h in (0, 9, 15):
        gk = h // r
        for i in (0, 63, 64, 9001, 16383):
            s = scale * (k[0, :i + 1, gk] @ q[0, i, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ v[0, :i + 1, gk]
            dp = v[0, :i + 1, gk] @ go[0, i, h]
            ds = p * (dp - o @ go[0, i, h])
            want = scale * (ds @ k[0, :i + 1, gk])
            check_grad(dq[0, i, h], want, f"dq row {i} head {h}")
    gk = 1
    keys = (Sq - 512, Sq - 64, Sq - 1)  # a 64-key block start, the last block
    i0 = keys[0]
    dk_w = np.zeros((len(keys), D))
    dv_w = np.zeros((len(keys), D))
    rows = np.arange(i0, Sq)
    for h in range(gk * r, gk * r + r):
        s = scale * (q[0, i0:, h] @ k[0, :, gk].T)
        s[np.arange(Sq)[None, :] > rows[:, None]] = -np.inf
        pr = np.exp(s - s.max(axis=1, keepdims=True))
        pr /= pr.sum(axis=1, keepdims=True)
        dpsum = np.sum((pr @ v[0, :, gk]) * go[0, i0:, h], axis=1)
        for n, j in enumerate(keys):
            ds_j = pr[:, j] * (go[0, i0:, h] @ v[0, j, gk] - dpsum)
            dv_w[n] += pr[:, j] @ go[0, i0:, h]
            dk_w[n] += scale * (ds_j @ q[0, i0:, h])
        del s, pr
    for n, j in enumerate(keys):
        check_grad(dk[0, j, gk], dk_w[n], f"dk key {j}")
        check_grad(dv[0, j, gk], dv_w[n], f"dv key {j}")


def test_bwd_zero_scale(gpu_lib):
    """softmax_scale = 0: P is uniform over each row's visible keys, dQ = dK =
    0, dV = P^T dO; masked keys (causal, rows with no key) must not give NaN."""
    print("[case] bwd zero scale", flush=True)
    for B, Sq, Sk, D in ((1, 130, 130, 128), (1, 90, 40, 64), (1, 100, 100, 256), (1, 70, 70, 96),
                         (1, 66, 66, 192)):
        w = W.dense_case(93 + Sq, B, Sq, Sk, 4, 2, D, causal=True, softmax_scale=0.0)
        g = W.grad_output(93 + Sq, (B, Sq, 4, D))
        dq, dk, dv = run_dense(gpu_lib, w, g)
        ref = OA.attention_dense_backward(f64(w.q), f64(w.k), f64(w.v), f64(g), 0.0,
                                          causal=True)
        for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            print("scale0", nm, check_grad(host_f64(got), r, f"scale0 {nm}"))


def test_bwd_rejects_head_dim_80(gpu_lib):
    """A head dim outside 64/96/128/192/256 is refused before any launch."""
    w = W.dense_case(3, 1, 64, 64, 2, 1, 80)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    lse = torch.zeros(1, 2, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.MiAttnError) as e:
        gpu_lib.mi_attn_bwd(q, k, v, q, q, lse)
    assert e.value.code == gpu_lib.MI_ATTN_EUNSUPPORTED
