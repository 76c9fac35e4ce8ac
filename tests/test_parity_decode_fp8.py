"""GPU parity of the fp8 (OCP e4m3 and e5m2) KV-cache decode with per-(batch, KV head)
descales (mi_attn_decode_splitkv through the C ABI) against the float64
oracle run on the decoded cache values."""
import zlib

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W
from tests.gpu_util import check, dev_bf16, dev_i32, f64, host_f64

pytestmark = pytest.mark.gpu


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def dev_f32(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def run_fp8(mi, w, num_splits=None, window_left=None, as_float8=False):
    kc, vc = dev_u8(w.k), dev_u8(w.v)
    if w.kv_dtype == "fp8_e5m2":  # uint8 means e4m3 bytes: e5m2 needs its dtype
        kc, vc = kc.view(torch.float8_e5m2), vc.view(torch.float8_e5m2)
    elif as_float8:
        kc, vc = kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn)
    out, lse = mi.mi_attn_decode_splitkv(
        dev_bf16(w.q), kc, vc, dev_i32(w.page_table), seqused_k=dev_i32(w.seqused_k),
        softmax_scale=w.softmax_scale,
        num_splits=w.num_splits if num_splits is None else num_splits,
        window_left=window_left, k_descale=dev_f32(w.k_descale), v_descale=dev_f32(w.v_descale),
        check_bounds=True)
    torch.cuda.synchronize()
    return out, lse


def decode_codes(w, codes):
    return OA.e5m2_decode(codes) if w.kv_dtype == "fp8_e5m2" else OA.e4m3_decode(codes)


def oracle_fp8(w, window_left=None, heads=None):
    o, l, _, _ = OA.paged_decode(f64(w.q), decode_codes(w, w.k), decode_codes(w, w.v), w.page_table,
                                 w.seqused_k, w.softmax_scale, num_splits=1,
                                 window_left=window_left, heads=heads,
                                 k_descale=w.k_descale, v_descale=w.v_descale)
    return o, l


CASES = [
    # (name, B, Hq, Hkv, D, page_size, pages_per_seq, extra_pages, seqused, splits, wl, descale)
    ("gqa8_page256_ragged", 3, 16, 2, 128, 256, 5, 3, [1, 700, 1280], 4, None, True),
    ("gqa4_page64_d64", 2, 16, 4, 64, 64, 10, 2, [600, 65], 6, None, True),
    ("mha_page32_no_descale", 2, 4, 4, 128, 32, 12, 0, [384, 200], 5, None, False),
    ("gqa32_heuristic_splits", 2, 32, 1, 128, 128, 8, 1, [1024, 333], 0, None, True),
    ("window_left", 2, 8, 2, 128, 256, 4, 0, [900, 300], 3, 150, True),
    ("empty_and_tiny", 4, 8, 2, 64, 64, 3, 0, [0, 1, 64, 65], 8, None, True),
    # the streaming kernel at head dims 96, 192 (LDS rows of 128 and 256
    # columns, loads spread over the cache's chunks only) and 256
    ("stream_d96_page32_ragged", 3, 8, 2, 96, 32, 12, 1, [1, 370, 129], 5, None, True),
    ("stream_d256_page32", 2, 8, 2, 256, 32, 9, 1, [288, 100], 5, None, True),
    ("stream_d192_page64_gqa8", 2, 16, 2, 192, 64, 6, 1, [350, 130], 4, None, True),
    # the tile kernel: page sizes that are not multiples of 32
    ("tile_page16_d128", 2, 16, 2, 128, 16, 30, 2, [470, 33], 6, None, True),
    ("tile_d96_page48_window", 2, 8, 2, 96, 48, 8, 0, [380, 47], 3, 100, True),
    ("tile_page48_d64_empty", 3, 8, 4, 64, 48, 4, 0, [0, 150, 47], 2, None, False),
    ("tile_d256_page48", 2, 8, 2, 256, 48, 8, 0, [380, 47], 3, None, True),
    ("tile_d192_page16", 2, 16, 2, 192, 16, 25, 1, [390, 200], 4, None, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_decode_elementwise(gpu_lib, case):
    name, B, Hq, Hkv, D, ps, pps, extra, used, splits, wl, ds = case
    print(f"[case] fp8 decode {name}", flush=True)
    w = W.paged_decode_fp8_case(zlib.crc32(name.encode()) % 10000, B, Hq, Hkv, D, ps, pps,
                                num_pages=B * pps + extra, seqused_k=used, num_splits=splits,
                                descale=ds)
    out, lse = run_fp8(gpu_lib, w, window_left=wl)
    o_ref, l_ref = oracle_fp8(w, window_left=wl)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))


E5M2_CASES = [c for c in CASES if c[0] in ("gqa8_page256_ragged", "gqa4_page64_d64",
                                            "window_left", "empty_and_tiny",
                                            "stream_d256_page32", "tile_d96_page48_window")]


@pytest.mark.parametrize("case", E5M2_CASES, ids=[c[0] for c in E5M2_CASES])
def test_e5m2_decode_elementwise(gpu_lib, case):
    name, B, Hq, Hkv, D, ps, pps, extra, used, splits, wl, ds = case
    print(f"[case] e5m2 decode {name}", flush=True)
    w = W.paged_decode_fp8_case(zlib.crc32(name.encode()) % 10000 + 1, B, Hq, Hkv, D, ps, pps,
                                num_pages=B * pps + extra, seqused_k=used, num_splits=splits,
                                descale=ds, fmt="e5m2")
    out, lse = run_fp8(gpu_lib, w, window_left=wl)
    o_ref, l_ref = oracle_fp8(w, window_left=wl)
    print(name, check(host_f64(out), o_ref, host_f64(lse), l_ref, what=name))


@pytest.mark.parametrize("D,ps", [(128, 64), (256, 64), (96, 64), (96, 48), (256, 48)])  # 3 stream, 2 tile
def test_e5m2_every_finite_code_decodes_exactly(gpu_lib, D, ps):
    """As the e4m3 case below for e5m2: each of its 248 finite codes placed in
    V comes back exactly (every e5m2 value is a bf16 value)."""
    B, Hq, Hkv = 2, 4, 4
    w = W.paged_decode_fp8_case(78, B, Hq, Hkv, D, ps, 1, seqused_k=[1, 1], num_splits=1,
                                descale=False, fmt="e5m2")
    finite = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)
    codes = np.resize(finite, (B, Hkv, D))
    for b in range(B):
        w.v[w.page_table[b, 0], 0] = codes[b]
    out, lse = run_fp8(gpu_lib, w)
    got = host_f64(out).reshape(B, Hkv, Hq // Hkv, D)
    want = OA.e5m2_decode(codes)[:, :, None, :]
    assert np.array_equal(got, np.broadcast_to(want, got.shape))
    o_ref, l_ref = oracle_fp8(w)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="one key e5m2")


def test_fp8_mixed_formats_rejected(gpu_lib):
    w = W.paged_decode_fp8_case(5, 1, 4, 2, 128, 64, 2)
    kc = dev_u8(w.k).view(torch.float8_e4m3fn)
    vc = dev_u8(w.v).view(torch.float8_e5m2)
    with pytest.raises(gpu_lib.MiAttnError) as e:
        gpu_lib.mi_attn_decode_splitkv(dev_bf16(w.q), kc, vc, dev_i32(w.page_table),
                                       seqused_k=dev_i32(w.seqused_k))
    assert e.value.code == gpu_lib.MI_ATTN_EINVAL


@pytest.mark.parametrize("D,ps", [(128, 64), (256, 64), (192, 64), (192, 16)])  # 3 stream, tile
def test_fp8_every_code_decodes_exactly(gpu_lib, D, ps):
    """One key per sequence: O is that key's V row times its descale, so every
    finite e4m3 code placed in V must come back exactly (vs = 1, the value is
    a bf16 value); the float8_e4m3fn tensor dtype is accepted as well."""
    B, Hq, Hkv = 2, 4, 4
    w = W.paged_decode_fp8_case(77, B, Hq, Hkv, D, ps, 1, seqused_k=[1, 1], num_splits=1,
                                descale=False)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = np.resize(finite, (B, Hkv, D))  # cycles through all 254 finite codes
    for b in range(B):
        w.v[w.page_table[b, 0], 0] = codes[b]
    out, lse = run_fp8(gpu_lib, w, as_float8=True)
    got = host_f64(out).reshape(B, Hkv, Hq // Hkv, D)
    want = OA.e4m3_decode(codes)[:, :, None, :]
    assert np.array_equal(got, np.broadcast_to(want, got.shape))
    o_ref, l_ref = oracle_fp8(w)
    check(host_f64(out), o_ref, host_f64(lse), l_ref, what="one key")


def test_fp8_full_size_decode_sampled(gpu_lib):
    """The paged decode workload's shape with an fp8 cache (B16, GQA 32/4,
    D128, Sk 32768, 256-token pages, 16 splits); the oracle checks four
    sequences' heads 0, 13, 31."""
    w = W.paged_decode_fp8_case(1005, 16, 32, 4, 128, 256, 128, num_splits=16,
                                name="paged_fp8_b16_sk32768")
    out, lse = run_fp8(gpu_lib, w)
    o_all, l_all = host_f64(out), host_f64(lse)
    heads = [0, 13, 31]
    for b in (0, 5, 10, 15):
        # only sequence b's pages, behind an identity table (the oracle decodes
        # what it is given to float64)
        pages = w.page_table[b]
        wb = W.Workload(name="b", kind="paged", q=w.q[b:b + 1], k=w.k[pages], v=w.v[pages],
                        num_heads_q=32, num_heads_kv=4, head_dim=128,
                        softmax_scale=w.softmax_scale,
                        page_table=np.arange(len(pages), dtype=np.int32)[None],
                        seqused_k=w.seqused_k[b:b + 1],
                        k_descale=w.k_descale[b:b + 1], v_descale=w.v_descale[b:b + 1])
        o_ref, l_ref = oracle_fp8(wb, heads=heads)
        for h in heads:
            check(o_all[b, h], o_ref[0, h], l_all[b, h], l_ref[0, h], what=f"seq {b} head {h}")


@pytest.mark.parametrize("descale", [0.0, -1.0, float("nan")])
def test_fp8_tile_path_key_descale_edges(gpu_lib, descale):
    """The tile kernel (page size 48) with a key descale of 0 (every score 0:
    uniform weights over the visible keys), or negative / NaN (no meaning for
    a cache scale: that sequence's output and LSE are NaN, the others'
    unaffected)."""
    w = W.paged_decode_fp8_case(31, 2, 8, 2, 128, 48, 4, seqused_k=[150, 60], num_splits=2)
    w.k_descale[0, :] = descale
    out, lse = run_fp8(gpu_lib, w)
    o, l = host_f64(out), host_f64(lse)
    o_ref, l_ref = oracle_fp8(w)
    if descale == 0.0:
        check(o, o_ref, l, l_ref, what="zero key descale")
    else:
        assert np.isnan(o[0]).all() and np.isnan(l[0]).all()
        check(o[1:], o_ref[1:], l[1:], l_ref[1:], what="other sequence")


@pytest.mark.parametrize("D,ps", [(128, 64), (256, 32), (96, 32), (192, 64), (256, 48)])  # 4 stream, tile
def test_fp8_varlen_decode(gpu_lib, D, ps):
    """fp8 e4m3 cache with descales and three causal query tokens per
    sequence (packed by cu_seqlens_q): against the oracle's paged prefill over
    the decoded, descaled cache values."""
    print(f"[case] fp8 varlen decode D{D} page {ps}", flush=True)
    w = W.paged_decode_fp8_case(97, 3, 16, 2, D, ps, 384 // ps, num_pages=3 * (384 // ps) + 2,
                                seqused_k=[384, 130, 2], num_splits=3)
    q_lens = [3, 1, 3]
    rng = np.random.default_rng(98)
    qp = W.round_to_bf16_bits(rng.standard_normal((sum(q_lens), 16, D), dtype=np.float32))
    cu = np.zeros(4, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    out, lse = gpu_lib.mi_attn_decode_splitkv(
        dev_bf16(qp), dev_u8(w.k), dev_u8(w.v), dev_i32(w.page_table),
        seqused_k=dev_i32(w.seqused_k), cu_seqlens_q=dev_i32(cu), max_seqlen_q=3, causal=True,
        softmax_scale=w.softmax_scale, num_splits=3, k_descale=dev_f32(w.k_descale),
        v_descale=dev_f32(w.v_descale), check_bounds=True)
    torch.cuda.synchronize()
    # cached values: each page's codes times the descale of the sequence owning it
    kd = np.full((w.k.shape[0], 2), np.nan)
    vd = np.full((w.v.shape[0], 2), np.nan)
    for b in range(3):
        kd[w.page_table[b]] = w.k_descale[b]
        vd[w.page_table[b]] = w.v_descale[b]
    kval = OA.e4m3_decode(w.k) * kd[:, None, :, None]
    vval = OA.e4m3_decode(w.v) * vd[:, None, :, None]
    o_ref, l_ref = OA.paged_prefill(f64(qp), kval, vval, w.page_table, w.seqused_k,
                                    w.softmax_scale, causal=True, cu_seqlens_q=cu)
    print("fp8 varlen", check(host_f64(out), o_ref, host_f64(lse).T, l_ref, what="fp8 varlen"))
