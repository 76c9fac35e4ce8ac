"""GPU parity of the prefill forward (mi_attn_fwd through the C ABI) against
the float64 oracle, element by element on mid-size cases and on sampled rows
at the full benchmark sizes."""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64, run_parallel

pytestmark = pytest.mark.gpu


def run_dense(mi, w, **kw):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    out, lse = mi.mi_attn_fwd(q, k, v, softmax_scale=w.softmax_scale, causal=w.causal,
                              window_left=w.window_left, window_right=w.window_right, **kw)
    torch.cuda.synchronize()
    return out, lse


def run_varlen(mi, w):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    out, lse = mi.mi_attn_fwd(q, k, v, cu_seqlens_q=dev_i32(w.cu_seqlens_q),
                              cu_seqlens_k=dev_i32(w.cu_seqlens_k), max_seqlen_q=w.max_seqlen_q,
                              max_seqlen_k=w.max_seqlen_k, softmax_scale=w.softmax_scale,
                              causal=w.causal, window_left=w.window_left,
                              window_right=w.window_right)
    torch.cuda.synchronize()
    return out, lse


DENSE_CASES = [
    # (name, B, Sq, Sk, Hq, Hkv, D, causal, wl, wr)
    ("mha_d64_noncausal_ragged", 2, 200, 333, 2, 2, 64, False, None, None),
    ("gqa4_d128_causal_ragged", 2, 333, 333, 8, 2, 128, True, None, None),
    ("gqa4_d64_causal_sq_lt_sk", 1, 200, 517, 4, 1, 64, True, None, None),
    ("mha_d64_causal_sq_gt_sk", 1, 300, 150, 2, 2, 64, True, None, None),
    ("gqa2_d128_window_both", 2, 400, 400, 6, 3, 128, False, 37, 11),
    ("gqa3_d128_window_left_only", 1, 290, 290, 6, 2, 128, False, 50, None),
    ("gqa2_d128_window_right_only", 1, 190, 260, 4, 2, 128, False, None, 5),
    ("gqa2_d256_causal", 1, 257, 257, 4, 2, 256, True, None, None),
    ("mqa_d256_noncausal_ragged", 1, 130, 190, 2, 1, 256, False, None, None),
    ("mqa16_d128_causal", 1, 129, 129, 16, 1, 128, True, None, None),
    ("gqa8_d128_causal_window", 1, 700, 700, 16, 2, 128, True, 100, None),
    ("one_key", 1, 1, 1, 2, 1, 128, False, None, None),
    ("one_query_many_keys", 3, 1, 1000, 8, 2, 128, True, None, None),
]


def oracle_dense(w):
    return OA.attention_dense(f64(w.q), f64(w.k), f64(w.v), w.softmax_scale, w.causal,
                              w.window_left, w.window_right)


@pytest.mark.parametrize("case", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_elementwise(gpu_lib, case):
    name, B, Sq, Sk, Hq, Hkv, D, causal, wl, wr = case
    print(f"[case] {name}", flush=True)
    w = W.dense_case(zlib.crc32(name.encode()) % 10000, B, Sq, Sk, Hq, Hkv, D, causal=causal, window_left=wl,
                     window_right=wr)
    out, lse = run_dense(gpu_lib, w)
    o_ref, l_ref = oracle_dense(w)
    st = check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name)
    print(name, st)


def test_config1_tiny_mha(gpu_lib):
    w = W.standard_config(1)
    out, lse = run_dense(gpu_lib, w)
    o_ref, l_ref = oracle_dense(w)
    print("tiny", check(host_f64(out), o_ref, host_f64(lse), l_ref, what="config1"))


VARLEN_CASES = [
    ("causal_ragged", [0, 1, 127, 128, 129, 300, 64], None, True, None, None, 8, 2, 128),
    ("window", [513, 77, 1030, 5], None, True, 64, 0, 8, 4, 128),
    ("cross_lengths_noncausal", [10, 200, 0, 33], [50, 20, 7, 0], False, None, None, 4, 1, 64),
    ("d256_causal", [100, 260], None, True, None, None, 4, 2, 256),
    # more than eight sequences, empty ones among them
    ("many_sequences", [33, 0, 257, 5, 128, 1, 0, 96, 300, 64, 0, 17, 200, 2, 129, 40, 0, 90, 11],
     None, True, None, None, 8, 2, 128),
    ("many_sequences_d256", [65, 0, 3, 140, 1, 0, 77, 129, 12, 200, 0], None, True, None, None,
     4, 2, 256),
    # more sequences than a wave has lanes (the block search takes 64 per
    # step), many short with empty ones and the longest last (a row with two
    # visible keys here is where bf16 P rounding passes 1e-2: tests/gpu_util.py)
    ("over_64_sequences", [(i * 37) % 97 if i % 11 else 0 for i in range(149)] + [390],
     None, True, None, None, 8, 2, 128),
    ("over_64_sequences_window_d256", [(i * 53) % 131 if i % 7 else 0 for i in range(70)] + [300],
     None, True, 100, 0, 4, 2, 256),
    # exactly one wave of sequences, and one more (the second search step
    # holds a single sequence)
    ("exactly_64_sequences", [(i * 41) % 90 + 1 for i in range(64)], None, True, None, None, 8, 2,
     128),
    ("65_sequences_last_alone", [(i * 29) % 70 for i in range(64)] + [257], None, True, None, None,
     4, 4, 128),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_elementwise(gpu_lib, case):
    name, lq, lk, causal, wl, wr, hq, hkv, d = case
    print(f"[case] varlen {name}", flush=True)
    lk = lq if lk is None else lk
    w = W.varlen_case(len(name), lq, lk, hq, hkv, d, causal=causal, window_left=wl,
                      window_right=wr)
    out, lse = run_varlen(gpu_lib, w)
    o_ref, l_ref = OA.attention_varlen(f64(w.q), f64(w.k), f64(w.v), w.cu_seqlens_q,
                                       w.cu_seqlens_k, w.softmax_scale, causal, wl, wr)
    absv = lambda: OA.attention_varlen(f64(w.q), f64(w.k), np.abs(f64(w.v)), w.cu_seqlens_q,
                                       w.cu_seqlens_k, w.softmax_scale, causal, wl, wr)[0]
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name, absv=absv))


def _sample_rows(rng, n_rows, count, must=()):
    idx = set(int(x) for x in must if 0 <= x < n_rows)
    idx |= set(int(x) for x in rng.choice(n_rows, size=min(count, n_rows), replace=False))
    return np.array(sorted(idx))


def test_full_size_causal_gqa_s4096_d128_every_element(gpu_lib):
    """The causal GQA S4096 D128 workload: every output element and every LSE
    against the oracle (32 full fp64 score matrices)."""
    print("[case] full-size causal GQA S4096 D128, all outputs", flush=True)
    w = W.standard_config(2)
    out, lse = run_dense(gpu_lib, w)
    o_gpu, l_gpu = host_f64(out[0]), host_f64(lse[0])
    S, r = w.seqlen_q, w.num_heads_q // w.num_heads_kv
    vis = OA.visible_mask(S, S, w.causal, w.window_left, w.window_right)
    q, k, v = f64(w.q[0]), f64(w.k[0]), f64(w.v[0])

    def head(h):
        return lambda: OA.attention_head(q[:, h], k[:, h // r], v[:, h // r], w.softmax_scale, vis)
    res = run_parallel([head(h) for h in range(w.num_heads_q)])
    o_ref = np.stack([o for o, _ in res], axis=1)  # (S, Hq, D)
    l_ref = np.stack([l for _, l in res], axis=0)  # (Hq, S)
    print(w.name, check(o_gpu, o_ref, l_gpu, l_ref, what=w.name))


def test_full_size_long_causal_gqa_s16384_d256_all_heads(gpu_lib):
    """The long causal GQA S16384 D256 workload: all 16 query heads on every
    row next to a 64-key tile boundary (positions 64t - 1 and 64t), the last
    64 rows and 64 random rows (about 640 rows per head)."""
    print("[case] full-size long causal GQA S16384 D256, all heads", flush=True)
    w = W.standard_config(3)
    out, lse = run_dense(gpu_lib, w)
    S, r = w.seqlen_q, w.num_heads_q // w.num_heads_kv
    rng = np.random.default_rng(3)
    edges = [p for t in range(S // 64) for p in (64 * t - 1, 64 * t)]
    pos = _sample_rows(rng, S, 64, must=edges + list(range(S - 64, S)))
    o_gpu = host_f64(out[0][torch.as_tensor(pos)])    # (n, Hq, D)
    l_gpu = host_f64(lse[0][:, torch.as_tensor(pos)])  # (Hq, n)
    k_all, v_all = f64(w.k[0]), f64(w.v[0])

    def head(h):
        q = f64(w.q[0, pos, h])
        return lambda: OA.attention_rows(q, pos, k_all[:, h // r], v_all[:, h // r],
                                         w.softmax_scale, S, w.causal, w.window_left,
                                         w.window_right)
    res = run_parallel([head(h) for h in range(w.num_heads_q)], workers=4)
    o_ref = np.stack([o for o, _ in res], axis=1)
    l_ref = np.stack([l for _, l in res], axis=0)
    print(w.name, len(pos), "rows per head", check(o_gpu, o_ref, l_gpu, l_ref, what=w.name))


def test_full_size_varlen_window_every_element(gpu_lib):
    """The varlen sliding-window workload (8 packed sequences, window 1024):
    every output element and every LSE against the oracle."""
    print("[case] full-size varlen window workload, all outputs", flush=True)
    w = W.standard_config(4)
    out, lse = run_varlen(gpu_lib, w)
    o_gpu, l_gpu = host_f64(out), host_f64(lse)
    cu = w.cu_seqlens_q
    r = w.num_heads_q // w.num_heads_kv
    q, k, v = f64(w.q), f64(w.k), f64(w.v)
    jobs, keys = [], []
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        vis = OA.visible_mask(t1 - t0, t1 - t0, w.causal, w.window_left, w.window_right)
        for h in range(w.num_heads_q):
            jobs.append(lambda t0=t0, t1=t1, h=h, vis=vis: OA.attention_head(
                q[t0:t1, h], k[t0:t1, h // r], v[t0:t1, h // r], w.softmax_scale, vis))
            keys.append((t0, t1, h))
    o_ref = np.zeros_like(o_gpu)
    l_ref = np.zeros_like(l_gpu)
    for (t0, t1, h), (o, l) in zip(keys, run_parallel(jobs)):
        o_ref[t0:t1, h] = o
        l_ref[h, t0:t1] = l
    print(w.name, check(o_gpu, o_ref, l_gpu, l_ref, what=w.name))


def test_deterministic(gpu_lib):
    w = W.dense_case(5, 1, 777, 777, 8, 2, 128, causal=True)
    o1, l1 = run_dense(gpu_lib, w)
    o2, l2 = run_dense(gpu_lib, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_gqa_packing_equals_replicated_mha(gpu_lib):
    """Packed GQA and MHA with replicated KV heads give bit-identical rows."""
    w = W.dense_case(6, 1, 300, 300, 8, 2, 128, causal=True)
    o1, l1 = run_dense(gpu_lib, w)
    w_rep = W.dense_case(6, 1, 300, 300, 8, 2, 128, causal=True)
    w_rep.k = np.repeat(w.k, 4, axis=2)
    w_rep.v = np.repeat(w.v, 4, axis=2)
    w_rep.num_heads_kv = 8
    o2, l2 = run_dense(gpu_lib, w_rep)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_strided_inputs_and_canaries(gpu_lib):
    """q/k/v as slices of a fused qkv buffer; out inside a guarded buffer."""
    B, S, Hq, Hkv, D = 2, 150, 4, 2, 128
    w = W.dense_case(8, B, S, S, Hq, Hkv, D, causal=True)
    qkv = torch.zeros(B, S, Hq + 2 * Hkv, D, dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :Hq] = dev_bf16(w.q)
    qkv[:, :, Hq:Hq + Hkv] = dev_bf16(w.k)
    qkv[:, :, Hq + Hkv:] = dev_bf16(w.v)
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    canary = -12345.0
    big = torch.full((B * S * Hq * D + 2048,), canary, dtype=torch.bfloat16, device="cuda")
    out = big[1024:1024 + B * S * Hq * D].view(B, S, Hq, D)
    lse_big = torch.full((B * Hq * S + 512,), canary, dtype=torch.float32, device="cuda")
    lse = lse_big[256:256 + B * Hq * S].view(B, Hq, S)
    gpu_lib.mi_attn_fwd(q, k, v, out=out, lse=lse, softmax_scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    assert torch.all(big[:1024] == canary) and torch.all(big[-1024:] == canary)
    assert torch.all(lse_big[:256] == canary) and torch.all(lse_big[-256:] == canary)
    o_ref, l_ref = oracle_dense(w)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="strided")


def test_fully_masked_rows_give_zero_and_neg_inf(gpu_lib):
    # Sq > Sk with causal: the first Sq - Sk query rows see no key
    w = W.dense_case(9, 1, 100, 40, 2, 1, 64, causal=True)
    out, lse = run_dense(gpu_lib, w)
    o = host_f64(out)
    l = host_f64(lse)
    assert np.all(o[0, :60] == 0.0)
    assert np.all(np.isneginf(l[0, :, :60]))
    o_ref, l_ref = oracle_dense(w)
    check(o, o_ref, l, l_ref, what="masked rows")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_zero_scale_uniform_weights(gpu_lib, d):
    """softmax_scale = 0: every score is 0, so each row averages the values of
    its visible keys (LSE = ln |visible keys|); masked keys (causal, ragged
    tails, fully masked rows) must still get weight 0, not NaN."""
    print(f"[case] zero scale D{d}", flush=True)
    w = W.dense_case(77 + d, 2, 150, 203, 4, 2, d, causal=True, softmax_scale=0.0)
    out, lse = run_dense(gpu_lib, w)
    o_ref, l_ref = oracle_dense(w)
    print("zero scale", check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"scale0 D{d}"))
    # Sq > Sk: the first rows see no key
    w = W.dense_case(78 + d, 1, 100, 40, 2, 1, d, causal=True, softmax_scale=0.0)
    out, lse = run_dense(gpu_lib, w)
    o_ref, l_ref = oracle_dense(w)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what=f"scale0 empty rows D{d}")


def test_zero_scale_varlen_window(gpu_lib):
    print("[case] zero scale varlen window", flush=True)
    lq = [70, 1, 0, 129, 300]
    w = W.varlen_case(79, lq, lq, 8, 2, 128, causal=True, window_left=50, window_right=0,
                      softmax_scale=0.0)
    out, lse = run_varlen(gpu_lib, w)
    o_ref, l_ref = OA.attention_varlen(f64(w.q), f64(w.k), f64(w.v), w.cu_seqlens_q,
                                       w.cu_seqlens_k, 0.0, True, 50, 0)
    print("zero scale varlen", check(host_f64(out), o_ref, host_f64(lse), l_ref,
                                     what="scale0 varlen"))
