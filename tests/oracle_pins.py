"""Checks that pin the float64 oracle to facts outside itself.

Each pin returns (ok: bool, detail: str) instead of asserting, so the same
pins can be run against deliberately broken copies of the oracle (see
test_oracle_mutants.py) to show that a plausible mistake fails at least one.

What each pin rests on:
  brute_*        an independent scalar-loop reading of the definition
  one_key        softmax over one element: O = v0, LSE = s00 exactly
  equal_keys     two equal scores: O = (v0+v1)/2, LSE = s + ln 2
  zero_query     Q = 0 makes every visible score 0, so LSE = ln |J(i)| and
                 O = mean of visible V rows; |J(i)| comes from a closed-form
                 interval length, not from the oracle's mask
  prob_sum       sum_j exp(s_ij - LSE_i) = 1
  const_v        convexity: V rows all equal c => O = c
  causal_row0    causal, Sq = Sk: query 0 sees key 0 only
  gqa_as_mha     GQA equals MHA with each KV head repeated Hq/Hkv times
  split_combine  combining split partials equals the unsplit result,
                 including empty splits
  paged          paged gather equals the contiguous layout
  e4m3           all 256 fp8 codes decode as torch's float8_e4m3fn does, and
                 closed-form values (1, 448, 2**-6, 2**-9, -0, NaN codes)
  e5m2           all 256 fp8 codes decode as torch's float8_e5m2 does, and
                 closed-form values (1, 57344, 2**-14, 2**-16, +-inf, NaN codes)
  descale        per-(batch, KV head) descales equal decoding a cache whose
                 pages were scaled beforehand, page by page
  sink_as_key    a learnable sink equals one more key whose score is the sink
                 (an extra head-dim coordinate makes it exact for every query)
                 and whose value is zero, run through the no-sink path
  sink_merge     the sink put into the softmax equals merging it into a
                 finished (O, LSE) in the log domain; sink = -inf changes
                 nothing; a row with no visible key gets O = 0, LSE = sink
  paged_prefill  queries (dense and packed) against a paged cache equal the
                 scalar loops run on contiguous copies built token by token,
                 with ragged seqused_k, Sq < Sk, empty sequences and masks
  softcap_limits a large soft cap leaves the scores unchanged (to 1/cap**2),
                 small scores pass through to first order, and every
                 probability ratio in a row stays within exp(2 cap)
  bwd_fd         backward gradients equal central finite differences of the
                 scalar-loop forward (loss sum(O * G)), GQA, Sq != Sk, masks,
                 rows with no visible key
  bwd_varlen     packed-sequence gradients equal finite differences of the
                 varlen forward, with different query and key lengths
  bwd_closed     one key: dV = sum of dO over the group's heads and queries,
                 dQ = dK = 0; sum over keys of dK is 0 (rows of dS sum to 0)
  bwd_torch      torch float64 autograd through an explicit masked softmax
  torch_sdpa     torch's float64 scaled_dot_product_attention on CPU, with
                 an explicit boolean mask built from the closed-form interval
"""
from __future__ import annotations

import math

import numpy as np

import oracle.attention as A
import oracle.brute as BR

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False, f"shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    diff = np.where(np.isnan(diff), np.inf, diff)
    m = float(diff.max(initial=0.0))
    return m <= tol, f"max diff {m:.3e}"


def interval_count(i, sq, sk, causal, wl, wr):
    """|J(i)| from the closed-form interval [max(0, c - wl), min(sk - 1, c + wr)], c = i + sk - sq."""
    c = i + sk - sq
    right = 0 if causal else (None if wr is None or wr < 0 else wr)
    left = None if wl is None or wl < 0 else wl
    lo = 0 if left is None else max(0, c - left)
    hi = sk - 1 if right is None else min(sk - 1, c + right)
    return max(0, hi - lo + 1), lo, hi


MASKS = [
    dict(causal=False, window_left=None, window_right=None),
    dict(causal=True, window_left=None, window_right=None),
    dict(causal=False, window_left=2, window_right=1),
    dict(causal=True, window_left=3, window_right=None),
    dict(causal=False, window_left=0, window_right=0),
    dict(causal=False, window_left=None, window_right=2),
    dict(causal=False, window_left=1, window_right=None),
]

SHAPES = [  # (B, Sq, Sk, Hq, Hkv, D)
    (1, 5, 5, 2, 1, 4),
    (2, 3, 7, 2, 2, 3),
    (1, 7, 4, 3, 1, 5),   # Sq > Sk: early causal rows see nothing
    (1, 1, 6, 4, 2, 8),   # one query (decode-like)
]


def pin_brute_dense():
    worst = 0.0
    for si, (B, Sq, Sk, Hq, Hkv, D) in enumerate(SHAPES):
        rng = _rng(100 + si)
        q = rng.standard_normal((B, Sq, Hq, D))
        k = rng.standard_normal((B, Sk, Hkv, D))
        v = rng.standard_normal((B, Sk, Hkv, D + 1))
        scale = 0.7
        for mk in MASKS:
            o, l = A.attention_dense(q, k, v, scale, **mk)
            ob, lb = BR.attention_loops(q.tolist(), k.tolist(), v.tolist(), scale, **mk)
            ok1, d1 = _close(o, np.array(ob))
            ok2, d2 = _close(l, np.array(lb))
            if not (ok1 and ok2):
                return False, f"shape {SHAPES[si]} mask {mk}: O {d1}, LSE {d2}"
            worst = max(worst, float(np.nanmax(np.abs(o - np.array(ob)))))
    return True, f"worst {worst:.2e}"


def pin_brute_varlen():
    rng = _rng(7)
    lq, lk = [3, 0, 5, 2], [4, 2, 5, 6]
    Hq, Hkv, D = 4, 2, 3
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((cu_q[-1], Hq, D))
    k = rng.standard_normal((cu_k[-1], Hkv, D))
    v = rng.standard_normal((cu_k[-1], Hkv, D))
    for mk in MASKS:
        o, l = A.attention_varlen(q, k, v, cu_q, cu_k, 0.5, **mk)
        for b in range(len(lq)):
            if lq[b] == 0:
                continue
            qs = q[cu_q[b]:cu_q[b + 1]][None]
            ks = k[cu_k[b]:cu_k[b + 1]][None]
            vs = v[cu_k[b]:cu_k[b + 1]][None]
            ob, lb = BR.attention_loops(qs.tolist(), ks.tolist(), vs.tolist(), 0.5, **mk)
            ok1, d1 = _close(o[cu_q[b]:cu_q[b + 1]], np.array(ob)[0])
            ok2, d2 = _close(l[:, cu_q[b]:cu_q[b + 1]], np.array(lb)[0])
            if not (ok1 and ok2):
                return False, f"seq {b} mask {mk}: O {d1}, LSE {d2}"
    return True, "ok"


def pin_one_key():
    rng = _rng(11)
    q = rng.standard_normal((1, 1, 1, 6))
    k = rng.standard_normal((1, 1, 1, 6))
    v = rng.standard_normal((1, 1, 1, 6))
    scale = 0.3
    o, l = A.attention_dense(q, k, v, scale)
    s00 = scale * float(np.dot(q[0, 0, 0], k[0, 0, 0]))
    ok1, d1 = _close(o[0, 0, 0], v[0, 0, 0], 0.0)
    ok2, d2 = _close(l[0, 0, 0], s00, 1e-15)
    return ok1 and ok2, f"O {d1}, LSE {d2}"


def pin_equal_keys():
    rng = _rng(12)
    q = rng.standard_normal((1, 1, 1, 5))
    k1 = rng.standard_normal(5)
    k = np.stack([k1, k1])[None, :, None, :]
    v = rng.standard_normal((1, 2, 1, 5))
    scale = 0.9
    o, l = A.attention_dense(q, k, v, scale)
    s = scale * float(np.dot(q[0, 0, 0], k1))
    ok1, d1 = _close(o[0, 0, 0], (v[0, 0, 0] + v[0, 1, 0]) / 2)
    ok2, d2 = _close(l[0, 0, 0], s + math.log(2.0))
    return ok1 and ok2, f"O {d1}, LSE {d2}"


def pin_zero_query():
    for (Sq, Sk) in [(6, 6), (4, 9), (9, 4), (1, 5)]:
        rng = _rng(Sq * 31 + Sk)
        q = np.zeros((1, Sq, 2, 3))
        k = rng.standard_normal((1, Sk, 1, 3))
        v = rng.standard_normal((1, Sk, 1, 3))
        for mk in MASKS:
            o, l = A.attention_dense(q, k, v, 1.0, **mk)
            for i in range(Sq):
                n, lo, hi = interval_count(i, Sq, Sk, mk["causal"], mk["window_left"],
                                           mk["window_right"])
                exp_lse = math.log(n) if n > 0 else -math.inf
                exp_o = v[0, lo:hi + 1, 0].mean(axis=0) if n > 0 else np.zeros(3)
                for h in range(2):
                    ok1, d1 = _close(l[0, h, i], exp_lse)
                    ok2, d2 = _close(o[0, i, h], exp_o)
                    if not (ok1 and ok2):
                        return False, f"Sq{Sq} Sk{Sk} {mk} row {i}: LSE {d1}, O {d2}"
    # the varlen sliding-window workload's rule: query i of a length-L sequence
    # sees min(i + 1, window_left + 1) keys
    L, wl = 40, 9
    q = np.zeros((1, L, 1, 2))
    k = _rng(5).standard_normal((1, L, 1, 2))
    _, l = A.attention_dense(q, k, k, 1.0, causal=True, window_left=wl, window_right=0)
    want = np.log(np.minimum(np.arange(L) + 1, wl + 1))
    ok, d = _close(l[0, 0], want)
    return ok, f"window count rule {d}"


def pin_prob_sum():
    rng = _rng(13)
    q = rng.standard_normal((1, 8, 2, 4)) * 3
    k = rng.standard_normal((1, 8, 2, 4)) * 3
    for mk in MASKS:
        vis = A.visible_mask(8, 8, **mk)
        _, l = A.attention_dense(q, k, k, 0.8, **mk)
        for h in range(2):
            s = 0.8 * q[0, :, h] @ k[0, :, h].T
            for i in range(8):
                if not vis[i].any():
                    continue
                tot = float(np.exp(s[i][vis[i]] - l[0, h, i]).sum())
                if abs(tot - 1.0) > TOL:
                    return False, f"{mk} row {i}: sum {tot}"
    return True, "ok"


def pin_const_v():
    rng = _rng(14)
    q = rng.standard_normal((2, 5, 4, 3))
    k = rng.standard_normal((2, 7, 2, 3))
    c = rng.standard_normal(6)
    v = np.broadcast_to(c, (2, 7, 2, 6)).copy()
    for mk in MASKS:
        o, l = A.attention_dense(q, k, v, 1.1, **mk)
        for b in range(2):
            for i in range(5):
                for h in range(4):
                    want = c if np.isfinite(l[b, h, i]) else np.zeros(6)
                    ok, d = _close(o[b, i, h], want)
                    if not ok:
                        return False, f"{mk} ({b},{i},{h}) {d}"
    return True, "ok"


def pin_causal_row0():
    rng = _rng(15)
    q = rng.standard_normal((1, 6, 2, 4))
    k = rng.standard_normal((1, 6, 1, 4))
    v = rng.standard_normal((1, 6, 1, 4))
    o, l = A.attention_dense(q, k, v, 0.5, causal=True)
    for h in range(2):
        ok1, d1 = _close(o[0, 0, h], v[0, 0, 0], 0.0)
        ok2, d2 = _close(l[0, h, 0], 0.5 * float(np.dot(q[0, 0, h], k[0, 0, 0])), 1e-15)
        if not (ok1 and ok2):
            return False, f"head {h}: O {d1} LSE {d2}"
    return True, "ok"


def pin_gqa_as_mha():
    rng = _rng(16)
    B, S, Hq, Hkv, D = 2, 6, 6, 2, 4
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    r = Hq // Hkv
    k_rep = np.repeat(k, r, axis=2)  # head h uses KV head h // r
    v_rep = np.repeat(v, r, axis=2)
    for mk in MASKS:
        o1, l1 = A.attention_dense(q, k, v, 0.6, **mk)
        o2, l2 = A.attention_dense(q, k_rep, v_rep, 0.6, **mk)
        ok1, d1 = _close(o1, o2, 0.0)
        ok2, d2 = _close(l1, l2, 0.0)
        if not (ok1 and ok2):
            return False, f"{mk}: O {d1} LSE {d2}"
    return True, "ok"


def pin_split_combine():
    rng = _rng(17)
    n, Sk, D = 3, 23, 5
    q = rng.standard_normal((n, D))
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    for mk in MASKS:
        vis = A.visible_mask(n, Sk, **mk)
        o_ref, l_ref = A.attention_head(q, k, v, 0.4, vis)
        for ns in [1, 2, 5, 23, 40]:  # 40 splits of 23 keys leaves empty splits
            op, lp = A.attention_partials(q, k, v, 0.4, vis, A.split_bounds(Sk, ns))
            o, l = A.combine(op, lp)
            ok1, d1 = _close(o, o_ref)
            ok2, d2 = _close(l, l_ref)
            if not (ok1 and ok2):
                return False, f"{mk} splits {ns}: O {d1} LSE {d2}"
        # an irregular hand-made partition, including an empty range
        bounds = [(0, 4), (4, 4), (4, 17), (17, 23)]
        op, lp = A.attention_partials(q, k, v, 0.4, vis, bounds)
        o, l = A.combine(op, lp)
        ok1, d1 = _close(o, o_ref)
        ok2, d2 = _close(l, l_ref)
        if not (ok1 and ok2):
            return False, f"{mk} irregular: O {d1} LSE {d2}"
    return True, "ok"


def pin_paged():
    rng = _rng(18)
    B, Hq, Hkv, D, ps, pps = 3, 4, 2, 5, 4, 3
    num_pages = B * pps + 2
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((num_pages, ps, Hkv, D))
    vc = rng.standard_normal((num_pages, ps, Hkv, D))
    table = rng.permutation(num_pages)[:B * pps].reshape(B, pps)
    used = np.array([12, 5, 9])
    o, l, _, _ = A.paged_decode(q, kc, vc, table, used, 0.7, num_splits=3)
    for b in range(B):
        # contiguous copy built with explicit per-token indexing
        kb = np.stack([kc[table[b, t // ps], t % ps] for t in range(used[b])])
        vb = np.stack([vc[table[b, t // ps], t % ps] for t in range(used[b])])
        o2, l2 = A.attention_dense(q[b][None, None], kb[None], vb[None], 0.7)
        ok1, d1 = _close(o[b], o2[0, 0])
        ok2, d2 = _close(l[b], l2[0, :, 0])
        if not (ok1 and ok2):
            return False, f"seq {b}: O {d1} LSE {d2}"
    return True, "ok"


def pin_paged_prefill():
    rng = _rng(21)
    B, Hq, Hkv, D, ps, pps = 3, 4, 2, 3, 4, 3
    num_pages = B * pps + 1
    kc = rng.standard_normal((num_pages, ps, Hkv, D))
    vc = rng.standard_normal((num_pages, ps, Hkv, D))
    table = rng.permutation(num_pages)[:B * pps].reshape(B, pps)
    used = np.array([10, 0, 12])
    masks = [dict(causal=True), dict(window_left=2, window_right=1), dict()]

    def contiguous(cache, b):
        return np.stack([cache[table[b, t // ps], t % ps] for t in range(used[b])]) \
            if used[b] else np.zeros((0, Hkv, D))

    # dense queries: Sq = 5 new tokens after a cached prefix (Sq < Sk), one
    # sequence with no keys
    Sq = 5
    q = rng.standard_normal((B, Sq, Hq, D))
    for mk in masks:
        o, l = A.paged_prefill(q, kc, vc, table, used, 0.6, **mk)
        for b in range(B):
            kb, vb = contiguous(kc, b), contiguous(vc, b)
            if used[b] == 0:
                if not (np.all(o[b] == 0) and np.all(l[b] == -np.inf)):
                    return False, f"{mk} seq {b}: no keys must give O = 0, LSE = -inf"
                continue
            ob, lb = BR.attention_loops(q[b][None], kb[None], vb[None], 0.6, **mk)
            ok1, d1 = _close(o[b], np.array(ob[0]))
            ok2, d2 = _close(l[b], np.array(lb[0]))
            if not (ok1 and ok2):
                return False, f"dense {mk} seq {b}: O {d1} LSE {d2}"
    # packed queries of lengths 2, 0, 6 (one longer than its keys: leading
    # rows see nothing under causal)
    lens = [2, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    qp = rng.standard_normal((int(cu[-1]), Hq, D))
    used_p = np.array([7, 3, 4])
    for mk in masks:
        o, l = A.paged_prefill(qp, kc, vc, table, used_p, 0.6, cu_seqlens_q=cu, **mk)
        for b in range(B):
            q0, q1 = int(cu[b]), int(cu[b + 1])
            if q1 == q0:
                continue
            kb = np.stack([kc[table[b, t // ps], t % ps] for t in range(used_p[b])])
            vb = np.stack([vc[table[b, t // ps], t % ps] for t in range(used_p[b])])
            ob, lb = BR.attention_loops(qp[q0:q1][None], kb[None], vb[None], 0.6, **mk)
            ok1, d1 = _close(o[q0:q1], np.array(ob[0]))
            ok2, d2 = _close(l[:, q0:q1], np.array(lb[0]))
            if not (ok1 and ok2):
                return False, f"packed {mk} seq {b}: O {d1} LSE {d2}"
    # seqused_k = None means the whole page-table row
    o, l = A.paged_prefill(q, kc, vc, table, None, 0.6, causal=True)
    kb = np.stack([kc[table[0, t // ps], t % ps] for t in range(pps * ps)])
    vb = np.stack([vc[table[0, t // ps], t % ps] for t in range(pps * ps)])
    ob, lb = BR.attention_loops(q[0][None], kb[None], vb[None], 0.6, causal=True)
    ok1, d1 = _close(o[0], np.array(ob[0]))
    ok2, d2 = _close(l[0], np.array(lb[0]))
    if not (ok1 and ok2):
        return False, f"seqused None: O {d1} LSE {d2}"
    return True, "ok"


def pin_e4m3():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = A.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    if not same.all():
        bad = np.flatnonzero(~same)[:4]
        return False, f"codes {bad.tolist()}: {mine[bad].tolist()} vs torch {ref[bad].tolist()}"
    closed = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0xB8: -1.0, 0x3C: 1.5}
    for c, v in closed.items():
        if A.e4m3_decode(np.array([c]))[0] != v:
            return False, f"code {c:#x} != {v}"
    if not (np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.signbit(mine[0x80])):
        return False, "NaN codes / negative zero"
    return True, "ok"


def pin_e5m2():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = A.e5m2_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    if not same.all():
        bad = np.flatnonzero(~same)[:4]
        return False, f"codes {bad.tolist()}: {mine[bad].tolist()} vs torch {ref[bad].tolist()}"
    closed = {0x3C: 1.0, 0x7B: 57344.0, 0x04: 2.0 ** -14, 0x01: 2.0 ** -16, 0xBC: -1.0,
              0x3E: 1.5, 0x7C: math.inf, 0xFC: -math.inf}
    for c, v in closed.items():
        if A.e5m2_decode(np.array([c]))[0] != v:
            return False, f"code {c:#x} != {v}"
    if not (np.isnan(mine[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]).all() and np.signbit(mine[0x80])):
        return False, "NaN codes / negative zero"
    return True, "ok"


def pin_descale():
    rng = _rng(23)
    B, Hq, Hkv, D, ps, pps = 2, 4, 2, 3, 4, 2
    num_pages = B * pps
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((num_pages, ps, Hkv, D))
    vc = rng.standard_normal((num_pages, ps, Hkv, D))
    table = rng.permutation(num_pages).reshape(B, pps)
    used = np.array([7, 8])
    ks = rng.uniform(0.5, 2.0, (B, Hkv))
    vs = rng.uniform(0.5, 2.0, (B, Hkv))
    o, l, _, _ = A.paged_decode(q, kc, vc, table, used, 0.4, num_splits=2,
                                k_descale=ks, v_descale=vs)
    # every page belongs to one sequence: scale that page's heads by its owner's descales
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        for p_ in table[b]:
            for g in range(Hkv):
                kc2[p_, :, g] *= ks[b, g]
                vc2[p_, :, g] *= vs[b, g]
    o2, l2, _, _ = A.paged_decode(q, kc2, vc2, table, used, 0.4, num_splits=1)
    ok1, d1 = _close(o, o2)
    ok2, d2 = _close(l, l2)
    return (ok1 and ok2), f"O {d1} LSE {d2}"


def pin_sink_as_key():
    rng = _rng(25)
    B, S, Hq, Hkv, D = 2, 7, 4, 2, 3
    scale = 0.5
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    sink = rng.uniform(-2.0, 3.0, Hq)
    o, l = A.attention_dense(q, k, v, scale, sink=sink)
    # per query head h: q' = [q, 1], real keys [k, 0], the sink key
    # [0, sink_h / scale] (score exactly sink_h), value 0, visible to all
    r = Hq // Hkv
    for h in range(Hq):
        g = h // r
        for b in range(B):
            q2 = np.concatenate([q[b, :, h], np.ones((S, 1))], axis=1)
            k2 = np.concatenate([np.concatenate([k[b, :, g], np.zeros((S, 1))], axis=1),
                                 np.concatenate([np.zeros((1, D)), [[sink[h] / scale]]], axis=1)])
            v2 = np.concatenate([v[b, :, g], np.zeros((1, D))])
            o2, l2 = A.attention_head(q2, k2, v2, scale, np.ones((S, S + 1), dtype=bool))
            ok1, d1 = _close(o[b, :, h], o2)
            ok2, d2 = _close(l[b, h], l2)
            if not (ok1 and ok2):
                return False, f"b {b} h {h}: O {d1} LSE {d2}"
    return True, "ok"


def pin_sink_merge():
    rng = _rng(26)
    Sq, Sk, Hq, D = 6, 9, 2, 4
    q = rng.standard_normal((1, Sq, Hq, D))
    k = rng.standard_normal((1, Sk, 1, D))
    v = rng.standard_normal((1, Sk, 1, D))
    sink = np.array([0.7, -1.3])
    for mk in [dict(causal=True), dict(window_left=2, window_right=0), dict()]:
        o, l = A.attention_dense(q, k, v, 0.6, sink=sink, **mk)
        o0, l0 = A.attention_dense(q, k, v, 0.6, **mk)
        # with_sink wants O's leading axes in LSE's order: (B, Hq, Sq, D)
        om, lm = A.with_sink(o0.transpose(0, 2, 1, 3), l0, sink[None, :, None])
        om = om.transpose(0, 2, 1, 3)
        ok1, d1 = _close(o, om)
        ok2, d2 = _close(l, lm)
        if not (ok1 and ok2):
            return False, f"{mk}: O {d1} LSE {d2}"
        on, ln_ = A.attention_dense(q, k, v, 0.6, sink=np.full(Hq, -np.inf), **mk)
        if not (np.array_equal(on, o0) and np.array_equal(ln_, l0)):
            return False, f"{mk}: sink -inf changed the result"
    # Sq > Sk causal: the first rows see no key
    o, l = A.attention_dense(q, k[:, :3], v[:, :3], 0.6, causal=True, sink=sink)
    if not (np.all(o[0, :3] == 0) and np.allclose(l[0, :, :3], sink[:, None], rtol=0, atol=0)):
        return False, "row with no key: O must be 0 and LSE the sink"
    return True, "ok"


def pin_torch_sdpa():
    import torch
    import torch.nn.functional as F
    rng = _rng(19)
    for (Sq, Sk) in [(7, 7), (5, 9)]:
        B, Hq, Hkv, D = 2, 4, 2, 6
        q = rng.standard_normal((B, Sq, Hq, D))
        k = rng.standard_normal((B, Sk, Hkv, D))
        v = rng.standard_normal((B, Sk, Hkv, D))
        for mk in MASKS:
            o, l = A.attention_dense(q, k, v, 0.45, **mk)
            mask = np.zeros((Sq, Sk), dtype=bool)
            for i in range(Sq):
                n, lo, hi = interval_count(i, Sq, Sk, mk["causal"], mk["window_left"],
                                           mk["window_right"])
                if n > 0:
                    mask[i, lo:hi + 1] = True
            rows = mask.any(axis=1)
            tq = torch.from_numpy(q).permute(0, 2, 1, 3)
            tk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
            tv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
            tm = torch.from_numpy(mask)
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=0.45)
            ref = ref.permute(0, 2, 1, 3).numpy()
            s = torch.matmul(tq, tk.transpose(-1, -2)) * 0.45
            s = s.masked_fill(~tm, float("-inf"))
            lse_ref = torch.logsumexp(s, dim=-1).numpy()
            ok1, d1 = _close(o[:, rows], ref[:, rows])
            ok2, d2 = _close(l, lse_ref)
            if not (ok1 and ok2):
                return False, f"Sq{Sq} Sk{Sk} {mk}: O {d1} LSE {d2}"
    return True, "ok"


def pin_softcap_limits():
    rng = _rng(41)
    B, Sq, Sk, Hq, Hkv, D = 2, 6, 9, 4, 2, 5
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    for mk in (MASKS[0], MASKS[1], MASKS[2]):
        o0, l0 = A.attention_dense(q, k, v, 0.5, **mk)
        # cap 1e4: |s - cap tanh(s / cap)| <= |s|**3 / (3 cap**2) ~ 1e-7
        o1, l1 = A.attention_dense(q, k, v, 0.5, softcap=1e4, **mk)
        ok1, d1 = _close(o1, o0, 1e-6)
        ok2, d2 = _close(l1, l0, 1e-6)
        if not (ok1 and ok2):
            return False, f"large cap {mk}: O {d1} LSE {d2}"
        # tiny scores (scale 1e-4, |s| < 1e-3) against cap 0.5: the cubic
        # term |s|**3 / (3 cap**2) stays under 2e-9
        o2, l2 = A.attention_dense(q, k, v, 1e-4, **mk)
        o3, l3 = A.attention_dense(q, k, v, 1e-4, softcap=0.5, **mk)
        ok1, d1 = _close(o3, o2, 1e-8)
        ok2, d2 = _close(l3, l2, 1e-8)
        if not (ok1 and ok2):
            return False, f"small scores {mk}: O {d1} LSE {d2}"
    # saturation: huge scores, cap 1 -> probabilities within a factor e**2
    qs, ks = q[:1, :, :1] * 50.0, k[:1, :, :1] * 50.0
    s_full = np.ones((Sq, Sk), dtype=bool)
    o, lse = A.attention_head(qs[0, :, 0], ks[0, :, 0], v[0, :, 0], 1.0, s_full, softcap=1.0)
    for i in range(Sq):
        # P_ij = exp(t_ij - LSE_i) with t in (-1, 1): LSE_i - ln Sk in (-1, 1)
        if not (-1.0 < lse[i] - math.log(Sk) < 1.0):
            return False, f"row {i}: LSE {lse[i]} not within 1 of ln {Sk}"
    # the capping is strictly increasing: keys with distinct scores keep
    # distinct, equally ordered capped scores (a one-key row's LSE is its
    # capped score), also past the cap (|s| / cap up to ~8)
    q3, k3 = q[0, :, 0], k[0, :, 0]
    s = q3 @ k3.T
    one = np.ones((1, 1), dtype=bool)
    for i in range(Sq):
        t = np.array([A.attention_head(q3[i:i + 1], k3[j:j + 1], v[0, j:j + 1, 0], 1.0, one,
                                       softcap=1.0)[1][0] for j in range(Sk)])
        order = np.argsort(s[i], kind="stable")
        if not np.all(np.diff(t[order]) > 0):
            return False, f"row {i}: capped scores not strictly increasing with the scores"
        if not np.all(np.abs(t) < 1.0):
            return False, f"row {i}: a capped score reaches the cap"
    return True, "ok"


def _fd_grads(loss, arrays, h=1e-6):
    """Central differences of loss(*arrays) with respect to every element."""
    out = []
    for n, x in enumerate(arrays):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = [a.copy() for a in arrays]
            args[n][idx] += h
            lp = loss(*args)
            args[n][idx] -= 2 * h
            lm = loss(*args)
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


def pin_bwd_fd():
    rng = _rng(31)
    cases = [((1, 4, 6, 4, 2, 3), MASKS[1]), ((1, 5, 5, 2, 1, 3), MASKS[2]),
             ((2, 3, 4, 2, 2, 2), MASKS[0]), ((1, 6, 3, 2, 1, 2), MASKS[1]),
             ((1, 5, 7, 4, 2, 2), MASKS[3])]
    # (B, Sq, Sk, Hq, Hkv, D); Sq 6 > Sk 3 causal leaves rows with no key
    for (B, Sq, Sk, Hq, Hkv, D), mk in cases:
        q = rng.standard_normal((B, Sq, Hq, D))
        k = rng.standard_normal((B, Sk, Hkv, D))
        v = rng.standard_normal((B, Sk, Hkv, D))
        g = rng.standard_normal((B, Sq, Hq, D))

        def loss(q, k, v):
            o, _ = BR.attention_loops(q, k, v, 0.6, **mk)
            return float((np.array(o) * g).sum())
        want = _fd_grads(loss, [q, k, v])
        got = A.attention_dense_backward(q, k, v, g, 0.6, **mk)
        for name, a, b in zip("qkv", got, want):
            ok, d = _close(a, b, 1e-6)
            if not ok:
                return False, f"{(B, Sq, Sk, Hq, Hkv, D)} {mk} d{name}: {d}"
    return True, "ok"


def pin_bwd_varlen():
    rng = _rng(32)
    cu_q = np.array([0, 3, 3, 7])
    cu_k = np.array([0, 2, 5, 11])
    Hq, Hkv, D = 2, 1, 2
    q = rng.standard_normal((7, Hq, D))
    k = rng.standard_normal((11, Hkv, D))
    v = rng.standard_normal((11, Hkv, D))
    g = rng.standard_normal((7, Hq, D))
    for mk in (MASKS[1], MASKS[2]):
        def loss(q, k, v):
            o, _ = A.attention_varlen(q, k, v, cu_q, cu_k, 0.8, **mk)
            return float((o * g).sum())
        want = _fd_grads(loss, [q, k, v])
        got = A.attention_varlen_backward(q, k, v, g, cu_q, cu_k, 0.8, **mk)
        for name, a, b in zip("qkv", got, want):
            ok, d = _close(a, b, 1e-6)
            if not ok:
                return False, f"varlen {mk} d{name}: {d}"
    return True, "ok"


def pin_bwd_closed():
    rng = _rng(33)
    B, Sq, Hq, Hkv, D = 2, 5, 4, 2, 3
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, 1, Hkv, D))
    v = rng.standard_normal((B, 1, Hkv, D))
    g = rng.standard_normal((B, Sq, Hq, D))
    dq, dk, dv = A.attention_dense_backward(q, k, v, g, 0.9)
    want_dv = g.reshape(B, Sq, Hkv, Hq // Hkv, D).sum(axis=(1, 3))[:, None]
    for name, a, b in (("dv", dv, want_dv), ("dq", dq, np.zeros_like(dq)),
                       ("dk", dk, np.zeros_like(dk))):
        ok, d = _close(a, b, 1e-12)
        if not ok:
            return False, f"one key {name}: {d}"
    Sk = 6
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    for mk in (MASKS[0], MASKS[1]):
        _, dk, _ = A.attention_dense_backward(q, k, v, g, 0.9, **mk)
        ok, d = _close(dk.sum(axis=1), np.zeros((B, Hkv, D)), 1e-12)
        if not ok:
            return False, f"sum of dK over keys {mk}: {d}"
    return True, "ok"


def pin_bwd_torch():
    import torch
    rng = _rng(34)
    B, Sq, Sk, Hq, Hkv, D = 2, 6, 9, 4, 2, 5
    r = Hq // Hkv
    for mk in (MASKS[0], MASKS[1], MASKS[2]):
        q = rng.standard_normal((B, Sq, Hq, D))
        k = rng.standard_normal((B, Sk, Hkv, D))
        v = rng.standard_normal((B, Sk, Hkv, D))
        g = rng.standard_normal((B, Sq, Hq, D))
        mask = np.zeros((Sq, Sk), dtype=bool)
        for i in range(Sq):
            n, lo, hi = interval_count(i, Sq, Sk, mk["causal"], mk["window_left"],
                                       mk["window_right"])
            if n > 0:
                mask[i, lo:hi + 1] = True
        tq = torch.from_numpy(q.copy()).requires_grad_()
        tk = torch.from_numpy(k.copy()).requires_grad_()
        tv = torch.from_numpy(v.copy()).requires_grad_()
        qh = tq.permute(0, 2, 1, 3)
        kh = tk.repeat_interleave(r, dim=2).permute(0, 2, 1, 3)
        vh = tv.repeat_interleave(r, dim=2).permute(0, 2, 1, 3)
        s = torch.matmul(qh, kh.transpose(-1, -2)) * 0.5
        s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vh).permute(0, 2, 1, 3)
        (o * torch.from_numpy(g)).sum().backward()
        got = A.attention_dense_backward(q, k, v, g, 0.5, **mk)
        for name, a, t in zip("qkv", got, (tq, tk, tv)):
            ok, d = _close(a, t.grad.numpy(), 1e-10)
            if not ok:
                return False, f"{mk} d{name}: {d}"
    return True, "ok"


def pin_rows_match_full():
    rng = _rng(20)
    Sq, Sk, D = 9, 13, 4
    q = rng.standard_normal((Sq, D))
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    for mk in MASKS:
        o, l = A.attention_head(q, k, v, 0.3, A.visible_mask(Sq, Sk, **mk))
        idx = np.array([0, 4, 8])
        o2, l2 = A.attention_rows(q[idx], idx, k, v, 0.3, Sq, **mk)
        ok1, d1 = _close(o2, o[idx], 0.0)
        ok2, d2 = _close(l2, l[idx], 0.0)
        if not (ok1 and ok2):
            return False, f"{mk}: O {d1} LSE {d2}"
    return True, "ok"


ALL_PINS = {
    "brute_dense": pin_brute_dense,
    "brute_varlen": pin_brute_varlen,
    "one_key": pin_one_key,
    "equal_keys": pin_equal_keys,
    "zero_query": pin_zero_query,
    "prob_sum": pin_prob_sum,
    "const_v": pin_const_v,
    "causal_row0": pin_causal_row0,
    "gqa_as_mha": pin_gqa_as_mha,
    "split_combine": pin_split_combine,
    "paged": pin_paged,
    "paged_prefill": pin_paged_prefill,
    "e4m3": pin_e4m3,
    "e5m2": pin_e5m2,
    "sink_as_key": pin_sink_as_key,
    "sink_merge": pin_sink_merge,
    "descale": pin_descale,
    "softcap_limits": pin_softcap_limits,
    "bwd_fd": pin_bwd_fd,
    "bwd_varlen": pin_bwd_varlen,
    "bwd_closed": pin_bwd_closed,
    "bwd_torch": pin_bwd_torch,
    "torch_sdpa": pin_torch_sdpa,
    "rows_match_full": pin_rows_match_full,
}


def run_all():
    """Runs every pin; returns {name: (ok, detail)}. Exceptions count as failures."""
    res = {}
    for name, fn in ALL_PINS.items():
        try:
            res[name] = fn()
        except Exception as e:  # a mutant may crash a pin: that is a detection
            res[name] = (False, f"raised {type(e).__name__}: {e}")
    return res
