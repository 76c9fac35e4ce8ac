"""Seeded synthetic inputs for the attention forward and the paged split-KV decode.

This module holds no attention arithmetic. It only draws random numbers, rounds
them to bfloat16, and lays them out in the shapes the attention API takes. Both
the CPU oracle (through the tests) and the HIP library (through the tests and
the benchmark) consume exactly the bit patterns produced here, so the two sides
see identical inputs.

Shapes follow the attention front end's conventions (FlashAttention CuTe-DSL
interface page, `_flash_attn_fwd` argument checks):
  dense   q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D)
  varlen  q (total_q, Hq, D), k/v (total_k, Hkv, D), cu_seqlens int32 (B+1,)
  paged   k/v cache (num_pages, page_size, Hkv, D), page_table int32 (B, max_pages)

Recipe (one generator per workload, numpy PCG64 via default_rng(seed)):
  * every value is a float32 draw from N(0, 1), rounded to bfloat16 by
    round-to-nearest-even; the bf16 bit patterns are stored as uint16;
  * Q, K, V are drawn in that order from the same generator;
  * varlen lengths are drawn first (integers, inclusive bounds);
  * the paged decode page permutation is drawn after V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "round_to_bf16_bits",
    "bf16_bits_to_f64",
    "bf16_bits_to_f32",
    "Workload",
    "dense_case",
    "varlen_case",
    "paged_decode_case",
    "standard_config",
    "STANDARD_CONFIGS",
]


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even.

    Inputs are finite normal draws, so NaN/Inf handling is not needed; the
    function asserts finiteness instead of silently mishandling them.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    chunk = 1 << 24
    for s in range(0, flat_in.size, chunk):
        u = flat_in[s:s + chunk].view(np.uint32)
        assert np.all((u & 0x7F800000) != 0x7F800000), "non-finite input"
        lsb = (u >> 16) & 1
        flat_out[s:s + chunk] = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return round_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclasses.dataclass
class Workload:
    """One synthetic attention problem.

    kind is "dense", "varlen", "paged" (decode) or "paged_prefill". Tensors hold bf16 bit patterns
    (uint16) or int32 index arrays. Mask parameters follow the front end's
    convention: causal flag plus window sizes, where None means unbounded.
    """
    name: str
    kind: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    softmax_scale: float
    causal: bool = False
    window_left: Optional[int] = None
    window_right: Optional[int] = None
    batch: int = 1
    seqlen_q: int = 0
    seqlen_k: int = 0
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None
    max_seqlen_q: int = 0
    max_seqlen_k: int = 0
    page_table: Optional[np.ndarray] = None
    seqused_k: Optional[np.ndarray] = None
    page_size: int = 0
    num_splits: int = 0
    seed: int = 0
    kv_dtype: str = "bf16"                  # "bf16", "fp8_e4m3" or "fp8_e5m2": k/v hold uint8 codes
    k_descale: Optional[np.ndarray] = None  # fp8: float32 (B, Hkv), or None for 1
    v_descale: Optional[np.ndarray] = None


def dense_case(seed: int, batch: int, seqlen_q: int, seqlen_k: int, hq: int, hkv: int,
               d: int, causal: bool = False, window_left: Optional[int] = None,
               window_right: Optional[int] = None, softmax_scale: Optional[float] = None,
               name: str = "dense") -> Workload:
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (batch, seqlen_q, hq, d))
    k = _normal_bf16(rng, (batch, seqlen_k, hkv, d))
    v = _normal_bf16(rng, (batch, seqlen_k, hkv, d))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    return Workload(name=name, kind="dense", q=q, k=k, v=v, num_heads_q=hq, num_heads_kv=hkv,
                    head_dim=d, softmax_scale=scale, causal=causal, window_left=window_left,
                    window_right=window_right, batch=batch, seqlen_q=seqlen_q,
                    seqlen_k=seqlen_k, max_seqlen_q=seqlen_q, max_seqlen_k=seqlen_k, seed=seed)


def grad_output(seed: int, shape) -> np.ndarray:
    """Output gradient dO for a backward workload: bf16 N(0, 1) bit patterns of
    the given shape (the forward output's), from its own generator seeded with
    seed + 7919 so the forward inputs of the same seed are unchanged."""
    return _normal_bf16(np.random.default_rng(seed + 7919), shape)


def _cu(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def varlen_case(seed: int, seqlens_q, seqlens_k, hq: int, hkv: int, d: int,
                causal: bool = False, window_left: Optional[int] = None,
                window_right: Optional[int] = None, softmax_scale: Optional[float] = None,
                name: str = "varlen", rng: Optional[np.random.Generator] = None) -> Workload:
    """Packed variable-length batch. Lengths are given; the generator draws Q, K, V."""
    rng = np.random.default_rng(seed) if rng is None else rng
    seqlens_q = [int(x) for x in seqlens_q]
    seqlens_k = [int(x) for x in seqlens_k]
    assert len(seqlens_q) == len(seqlens_k)
    cu_q, cu_k = _cu(seqlens_q), _cu(seqlens_k)
    q = _normal_bf16(rng, (int(cu_q[-1]), hq, d))
    k = _normal_bf16(rng, (int(cu_k[-1]), hkv, d))
    v = _normal_bf16(rng, (int(cu_k[-1]), hkv, d))
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    return Workload(name=name, kind="varlen", q=q, k=k, v=v, num_heads_q=hq, num_heads_kv=hkv,
                    head_dim=d, softmax_scale=scale, causal=causal, window_left=window_left,
                    window_right=window_right, batch=len(seqlens_q), cu_seqlens_q=cu_q,
                    cu_seqlens_k=cu_k, max_seqlen_q=max(seqlens_q, default=0),
                    max_seqlen_k=max(seqlens_k, default=0), seed=seed)


def paged_decode_case(seed: int, batch: int, hq: int, hkv: int, d: int, page_size: int,
                      pages_per_seq: int, num_pages: Optional[int] = None,
                      seqused_k=None, num_splits: int = 0,
                      softmax_scale: Optional[float] = None, name: str = "paged") -> Workload:
    """One query token per sequence against a paged K/V cache.

    The page table is a seeded random permutation of all pages (drawn after V):
    page_table[b, p] = perm[b * pages_per_seq + p]. With num_pages larger than
    batch * pages_per_seq some pages are never referenced.
    """
    rng = np.random.default_rng(seed)
    if num_pages is None:
        num_pages = batch * pages_per_seq
    assert num_pages >= batch * pages_per_seq
    q = _normal_bf16(rng, (batch, hq, d))
    k = _normal_bf16(rng, (num_pages, page_size, hkv, d))
    v = _normal_bf16(rng, (num_pages, page_size, hkv, d))
    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = np.ascontiguousarray(perm[:batch * pages_per_seq].reshape(batch, pages_per_seq))
    if seqused_k is None:
        seqused = np.full(batch, pages_per_seq * page_size, dtype=np.int32)
    else:
        seqused = np.asarray(seqused_k, dtype=np.int32).reshape(batch)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    return Workload(name=name, kind="paged", q=q, k=k, v=v, num_heads_q=hq, num_heads_kv=hkv,
                    head_dim=d, softmax_scale=scale, batch=batch, seqlen_q=1,
                    seqlen_k=pages_per_seq * page_size, max_seqlen_q=1,
                    max_seqlen_k=int(seqused.max(initial=0)), page_table=page_table,
                    seqused_k=seqused, page_size=page_size, num_splits=num_splits, seed=seed)


def _fp8_codes(x: np.ndarray, fmt: str) -> np.ndarray:
    """float32 values -> OCP fp8 codes (uint8) of format fmt ("e4m3" or
    "e5m2"), round to nearest even, via torch's float8 casts. Callers keep |x|
    well below the format's largest finite value (448, 57344)."""
    import torch
    dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dt).view(
        torch.uint8).numpy()


def paged_decode_fp8_case(seed: int, batch: int, hq: int, hkv: int, d: int, page_size: int,
                          pages_per_seq: int, num_pages: Optional[int] = None, seqused_k=None,
                          num_splits: int = 0, descale: bool = True,
                          softmax_scale: Optional[float] = None,
                          name: str = "paged_fp8", fmt: str = "e4m3") -> Workload:
    """paged_decode_case with an fp8 K/V cache (OCP e4m3, or e5m2 with
    fmt="e5m2") and per-(batch, KV head) descales. Draw order: Q (bf16), K and V values (float32 N(0,1)), the page
    permutation, then the K and V descale factors f ~ U[0.5, 2]. Descale =
    f / 16; a page owned by sequence b stores codes of value / descale[b, g]
    (|value / descale| < 200, far from e4m3's 448); pages no sequence uses
    are stored with descale 1/16. descale=False stores every page with 1 and
    passes no descales (the kernel's default)."""
    rng = np.random.default_rng(seed)
    if num_pages is None:
        num_pages = batch * pages_per_seq
    assert num_pages >= batch * pages_per_seq
    q = _normal_bf16(rng, (batch, hq, d))
    kx = rng.standard_normal((num_pages, page_size, hkv, d), dtype=np.float32)
    vx = rng.standard_normal((num_pages, page_size, hkv, d), dtype=np.float32)
    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = np.ascontiguousarray(perm[:batch * pages_per_seq].reshape(batch, pages_per_seq))
    if descale:
        kd = (rng.uniform(0.5, 2.0, (batch, hkv)) / 16.0).astype(np.float32)
        vd = (rng.uniform(0.5, 2.0, (batch, hkv)) / 16.0).astype(np.float32)
        kpage = np.full((num_pages, hkv), 1.0 / 16.0, dtype=np.float32)
        vpage = np.full((num_pages, hkv), 1.0 / 16.0, dtype=np.float32)
        for b in range(batch):
            kpage[page_table[b]] = kd[b]
            vpage[page_table[b]] = vd[b]
        kx /= kpage[:, None, :, None]
        vx /= vpage[:, None, :, None]
    else:
        kd = vd = None
    k = _fp8_codes(kx, fmt)
    del kx
    v = _fp8_codes(vx, fmt)
    del vx
    if seqused_k is None:
        seqused = np.full(batch, pages_per_seq * page_size, dtype=np.int32)
    else:
        seqused = np.asarray(seqused_k, dtype=np.int32).reshape(batch)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    return Workload(name=name, kind="paged", q=q, k=k, v=v, num_heads_q=hq, num_heads_kv=hkv,
                    head_dim=d, softmax_scale=scale, batch=batch, seqlen_q=1,
                    seqlen_k=pages_per_seq * page_size, max_seqlen_q=1,
                    max_seqlen_k=int(seqused.max(initial=0)), page_table=page_table,
                    seqused_k=seqused, page_size=page_size, num_splits=num_splits, seed=seed,
                    kv_dtype="fp8_" + fmt, k_descale=kd, v_descale=vd)


def paged_prefill_case(seed: int, batch: int, hq: int, hkv: int, d: int, page_size: int,
                       pages_per_seq: int, seqused_k, seqlen_q: Optional[int] = None,
                       seqlens_q=None, num_pages: Optional[int] = None, causal: bool = False,
                       window_left: Optional[int] = None, window_right: Optional[int] = None,
                       softmax_scale: Optional[float] = None,
                       name: str = "paged_prefill") -> Workload:
    """New query tokens against a paged K/V cache (e.g. prefill after a cached
    prefix). Queries are dense (batch, seqlen_q, hq, d) or, with seqlens_q,
    packed (sum, hq, d) with cu_seqlens_q. Draw order: Q, K cache, V cache,
    then the page permutation (page_table[b, p] = perm[b * pages_per_seq + p]).
    seqused_k (keys per sequence) may be None for full page-table rows.
    """
    rng = np.random.default_rng(seed)
    if num_pages is None:
        num_pages = batch * pages_per_seq
    assert num_pages >= batch * pages_per_seq
    if seqlens_q is not None:
        seqlens_q = [int(x) for x in seqlens_q]
        assert len(seqlens_q) == batch
        cu_q = _cu(seqlens_q)
        q = _normal_bf16(rng, (int(cu_q[-1]), hq, d))
        max_q = max(seqlens_q, default=0)
    else:
        cu_q = None
        q = _normal_bf16(rng, (batch, seqlen_q, hq, d))
        max_q = seqlen_q
    k = _normal_bf16(rng, (num_pages, page_size, hkv, d))
    v = _normal_bf16(rng, (num_pages, page_size, hkv, d))
    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = np.ascontiguousarray(perm[:batch * pages_per_seq].reshape(batch, pages_per_seq))
    seqused = None if seqused_k is None else np.asarray(seqused_k, dtype=np.int32).reshape(batch)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    cap = pages_per_seq * page_size
    return Workload(name=name, kind="paged_prefill", q=q, k=k, v=v, num_heads_q=hq,
                    num_heads_kv=hkv, head_dim=d, softmax_scale=scale, causal=causal,
                    window_left=window_left, window_right=window_right, batch=batch,
                    seqlen_q=0 if seqlens_q is not None else seqlen_q, seqlen_k=cap,
                    cu_seqlens_q=cu_q, max_seqlen_q=max_q,
                    max_seqlen_k=cap if seqused is None else int(seqused.max(initial=0)),
                    page_table=page_table, seqused_k=seqused, page_size=page_size, seed=seed)


STANDARD_CONFIGS = {
    1: "tiny non-causal MHA: B1 Hq=Hkv=2 S256 D64",
    2: "causal GQA prefill: B1 Hq32 Hkv4 S4096 D128",
    3: "long causal GQA prefill: B1 Hq16 Hkv2 S16384 D256",
    4: "varlen causal sliding window: 8 seqs U[512,8192] Hq32 Hkv8 D128 wl1024 wr0",
    5: "paged split-KV decode: B16 Hq32 Hkv4 D128 Sk32768 page256 16 splits",
}


def standard_config(i: int) -> Workload:
    """The five benchmark workloads; workload i uses seed 1000 + i."""
    seed = 1000 + i
    if i == 1:
        return dense_case(seed, 1, 256, 256, 2, 2, 64, causal=False, name="tiny_mha_s256_d64")
    if i == 2:
        return dense_case(seed, 1, 4096, 4096, 32, 4, 128, causal=True,
                          name="causal_gqa32x4_s4096_d128")
    if i == 3:
        return dense_case(seed, 1, 16384, 16384, 16, 2, 256, causal=True,
                          name="causal_gqa16x2_s16384_d256")
    if i == 4:
        rng = np.random.default_rng(seed)
        lengths = rng.integers(512, 8193, size=8)
        return varlen_case(seed, lengths, lengths, 32, 8, 128, causal=True, window_left=1024,
                           window_right=0, name="varlen8_window1024_gqa32x8_d128", rng=rng)
    if i == 5:
        return paged_decode_case(seed, 16, 32, 4, 128, page_size=256, pages_per_seq=128,
                                 num_splits=16, name="paged_decode_b16_gqa32x4_sk32768_d128")
    raise ValueError(f"unknown standard workload {i}")
