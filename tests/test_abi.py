"""CPU tests of the C ABI: the library loads, exports every declared symbol,
the ctypes mirrors match the C struct layout, and invalid arguments return
their documented status before anything touches a device."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import exact_attention_45_amd as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_attn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mi_attn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mi.lib_path()):
        pytest.fail("libmiattn.so is not built (python -m exact_attention_45_amd.build)")
    return mi.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"mi_attn_fwd", "mi_attn_decode_splitkv", "mi_attn_combine",
            "mi_attn_decode_workspace_bytes", "mi_attn_last_error"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", mi.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mi_attn_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        assert hasattr(lib, n)


def test_struct_layout_matches_header():
    """Compiles a C program against the header and compares offsets with ctypes."""
    structs = {"mi_attn_fwd_params": mi.FwdParams, "mi_attn_decode_params": mi.DecodeParams,
               "mi_attn_bwd_params": mi.BwdParams}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = {}
    for ln in out.splitlines():
        s, f, v = ln.split()
        got[(s, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
    # every C field is mirrored
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for cname, py in structs.items():
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + cname, src).group(1)
        decl_names = []
        for stmt in body.split(";"):
            stmt = re.sub(r"//.*", "", stmt).strip()
            if stmt:
                decl_names += [re.findall(r"(\w+)\s*$", piece)[0] for piece in stmt.split(",")]
        assert set(decl_names) == {f for f, _ in py._fields_}, cname


FAKE = 0x10000  # 16-byte aligned fake device address; never dereferenced


def _fwd(**kw):
    p = mi.FwdParams()
    p.q = p.k = p.v = p.out = FAKE
    p.batch, p.seqlen_q, p.seqlen_k = 1, 16, 16
    p.num_heads_q, p.num_heads_kv, p.head_dim = 4, 2, 128
    p.q_row_stride = p.k_row_stride = p.v_row_stride = p.o_row_stride = 512
    p.q_head_stride = p.k_head_stride = p.v_head_stride = p.o_head_stride = 128
    p.q_batch_stride = p.k_batch_stride = p.v_batch_stride = p.o_batch_stride = 8192
    p.softmax_scale = 0.125
    p.window_left = p.window_right = -1
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _call_fwd(lib, p):
    return lib.mi_attn_fwd(ctypes.byref(p), None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=80), mi.MI_ATTN_EUNSUPPORTED),
    (dict(head_dim=160), mi.MI_ATTN_EUNSUPPORTED),
    (dict(head_dim=512), mi.MI_ATTN_EUNSUPPORTED),
    (dict(num_heads_q=5), mi.MI_ATTN_EINVAL),
    (dict(num_heads_kv=0), mi.MI_ATTN_EINVAL),
    (dict(q=0), mi.MI_ATTN_EINVAL),
    (dict(out=FAKE + 2), mi.MI_ATTN_EINVAL),
    (dict(q_row_stride=100), mi.MI_ATTN_EINVAL),
    (dict(k_batch_stride=-8), mi.MI_ATTN_EINVAL),
    (dict(page_table=FAKE), mi.MI_ATTN_EINVAL),  # paging sizes missing
    (dict(page_table=FAKE, page_size=32, num_pages=8, max_pages_per_seq=2),
     mi.MI_ATTN_EUNSUPPORTED),  # page_size not a multiple of the 64-key tile
    (dict(page_table=FAKE, page_size=64, num_pages=8, max_pages_per_seq=2,
          cu_seqlens_k=FAKE), mi.MI_ATTN_EINVAL),  # interface page: no cu_seqlens_k with pages
    (dict(page_table=FAKE, page_size=64, num_pages=8, max_pages_per_seq=2,
          k_batch_stride=-8), mi.MI_ATTN_EINVAL),  # page stride
    (dict(page_table=FAKE, page_size=64, num_pages=8, max_pages_per_seq=1 << 30),
     mi.MI_ATTN_EINVAL),  # table capacity overflows int32
    (dict(cu_seqlens_q=FAKE), mi.MI_ATTN_EINVAL),
    (dict(softmax_scale=float("nan")), mi.MI_ATTN_EUNSUPPORTED),
    (dict(softmax_scale=-1.0), mi.MI_ATTN_EUNSUPPORTED),
    (dict(seqlen_q=-1), mi.MI_ATTN_EINVAL),
    (dict(softcap=-1.0), mi.MI_ATTN_EUNSUPPORTED),
    (dict(softcap=float("inf")), mi.MI_ATTN_EUNSUPPORTED),
])
def test_fwd_invalid_arguments(lib, kw, code):
    rc = _call_fwd(lib, _fwd(**kw))
    assert rc == code, (rc, mi.mi_attn_last_error())
    assert mi.mi_attn_last_error()


def test_fwd_null_params(lib):
    assert lib.mi_attn_fwd(None, None) == mi.MI_ATTN_EINVAL


def test_fwd_empty_problems_are_noops(lib):
    # nothing to compute: returns OK without launching
    assert _call_fwd(lib, _fwd(batch=0)) == mi.MI_ATTN_OK
    assert _call_fwd(lib, _fwd(seqlen_q=0)) == mi.MI_ATTN_OK


def _dec(**kw):
    p = mi.DecodeParams()
    p.q = p.k_cache = p.v_cache = p.page_table = p.out = FAKE
    p.q_batch_stride, p.q_head_stride = 32 * 128, 128
    p.o_batch_stride, p.o_head_stride = 32 * 128, 128
    p.batch, p.num_heads_q, p.num_heads_kv, p.head_dim = 16, 32, 4, 128
    p.page_size, p.num_pages, p.max_pages_per_seq = 256, 2048, 128
    p.softmax_scale = 0.088
    p.window_left = p.window_right = -1
    p.num_splits = 16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_decode_workspace_size(lib):
    p = _dec()
    n = lib.mi_attn_decode_workspace_bytes(ctypes.byref(p))
    rows, splits, d = 16 * 32, 16, 128
    want = -(-rows * splits * d * 4 // 256) * 256 + -(-rows * splits * 4 // 256) * 256
    assert n == want
    assert lib.mi_attn_decode_num_splits(ctypes.byref(p)) == 16


@pytest.mark.parametrize("kw,code", [
    (dict(num_splits=300), mi.MI_ATTN_EINVAL),
    (dict(num_splits=-1), mi.MI_ATTN_EINVAL),
    (dict(head_dim=80), mi.MI_ATTN_EUNSUPPORTED),
    (dict(num_heads_q=30), mi.MI_ATTN_EINVAL),
    (dict(page_size=0), mi.MI_ATTN_EINVAL),
    (dict(page_table=0), mi.MI_ATTN_EINVAL),
    (dict(k_cache=FAKE + 4), mi.MI_ATTN_EINVAL),
    (dict(max_pages_per_seq=1 << 24, page_size=1 << 10), mi.MI_ATTN_EBOUNDS),
    (dict(kv_dtype=3), mi.MI_ATTN_EUNSUPPORTED),                      # no such cache type
    (dict(softcap=float("nan")), mi.MI_ATTN_EUNSUPPORTED),
])
def test_decode_invalid_arguments(lib, kw, code):
    p = _dec(**kw)
    assert lib.mi_attn_decode_splitkv(ctypes.byref(p), None) == code, mi.mi_attn_last_error()
    # sizing the workspace needs shapes only: pointer problems do not block it
    pointer_only = set(kw) <= {"page_table", "k_cache", "q", "v_cache", "out"}
    n = lib.mi_attn_decode_workspace_bytes(ctypes.byref(p))
    assert (n > 0) if pointer_only else (n == 0)


@pytest.mark.parametrize("kv", [mi.MI_ATTN_KV_FP8_E4M3, mi.MI_ATTN_KV_FP8_E5M2])
def test_decode_fp8_params_accepted_by_validation(lib, kv):
    # fp8 (either format) with head_dim 128 and 256-token pages sizes like the bf16 cache
    p = _dec(kv_dtype=kv)
    assert lib.mi_attn_decode_num_splits(ctypes.byref(p)) == 16
    assert lib.mi_attn_decode_workspace_bytes(ctypes.byref(p)) == \
        lib.mi_attn_decode_workspace_bytes(ctypes.byref(_dec()))


def test_decode_workspace_checks(lib):
    p = _dec()
    need = lib.mi_attn_decode_workspace_bytes(ctypes.byref(p))
    p.workspace, p.workspace_bytes = 0, need
    assert lib.mi_attn_decode_splitkv(ctypes.byref(p), None) == mi.MI_ATTN_EWORKSPACE
    p.workspace, p.workspace_bytes = 0x100000, need - 1
    assert lib.mi_attn_decode_splitkv(ctypes.byref(p), None) == mi.MI_ATTN_EWORKSPACE
    p.workspace, p.workspace_bytes = 0x100010, need  # not 256-byte aligned
    assert lib.mi_attn_decode_splitkv(ctypes.byref(p), None) == mi.MI_ATTN_EWORKSPACE
    assert "256" in mi.mi_attn_last_error()


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, 128, 0, 4, 0, 128), mi.MI_ATTN_EINVAL),      # zero splits
    ((FAKE, FAKE, FAKE, 128, 0, 4, 257, 128), mi.MI_ATTN_EINVAL),    # too many
    ((FAKE, FAKE, FAKE, 128, 0, 4, 4, 100), mi.MI_ATTN_EUNSUPPORTED),
    ((FAKE, FAKE, FAKE, 64, 0, 4, 4, 128), mi.MI_ATTN_EINVAL),       # row stride < D
    ((0, FAKE, FAKE, 128, 0, 4, 4, 128), mi.MI_ATTN_EINVAL),
])
def test_combine_invalid_arguments(lib, args, code):
    assert lib.mi_attn_combine(*args, None) == code


def test_version(lib):
    assert "gfx950" in mi.mi_attn_version()


def _bwd(**kw):
    p = mi.BwdParams()
    p.q = p.k = p.v = p.out = p.dout = p.lse = p.dq = p.dk = p.dv = FAKE
    B, S, Hq, Hkv, D = 2, 1000, 8, 2, 128
    for t, h in (("q", Hq), ("o", Hq), ("do", Hq), ("dq", Hq), ("k", Hkv), ("v", Hkv),
                 ("dk", Hkv), ("dv", Hkv)):
        setattr(p, f"{t}_batch_stride", S * h * D)
        setattr(p, f"{t}_row_stride", h * D)
        setattr(p, f"{t}_head_stride", D)
    p.batch, p.seqlen_q, p.seqlen_k = B, S, S
    p.num_heads_q, p.num_heads_kv, p.head_dim = Hq, Hkv, D
    p.softmax_scale = 0.088
    p.window_left = p.window_right = -1
    p.workspace, p.workspace_bytes = FAKE, 1 << 30
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _bwd_ws(batch, hq, hkv, d, rows_q, max_k):
    """One float32 row sum and one base-2 LSE per (query row, head), then float32 dK and dV
    partials of each split of the dK/dV walk (splits: about 512 workgroups of
    128 keys, 64 at head_dim 192 and 256, at most 4), each part 256-byte rounded."""
    rnd = lambda x: -(-x // 256) * 256
    bn = 64 if d > 128 else 128
    wg = -(-max_k // bn) * hkv * batch
    splits = max(1, min(4, -(-512 // wg)))
    parts = splits * batch * max_k * hkv * 2 * d if splits > 1 else 0
    return 2 * rnd(rows_q * hq * 4) + rnd(parts * 4)


def test_bwd_workspace_size(lib):
    assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(_bwd())) == _bwd_ws(2, 8, 2, 128, 2000, 1000)
    p = _bwd(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, total_q=777, max_seqlen_q=500, max_seqlen_k=500)
    assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(p)) == _bwd_ws(2, 8, 2, 128, 777, 500)
    # enough key blocks: one split, no partials
    p = _bwd(batch=64, seqlen_q=1024, seqlen_k=1024)
    assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(p)) == _bwd_ws(64, 8, 2, 128, 64 * 1024, 1024)
    assert _bwd_ws(64, 8, 2, 128, 64 * 1024, 1024) == 2 * 64 * 1024 * 8 * 4
    for kw in (dict(), dict(seqlen_q=4096, seqlen_k=4096)):  # split, then one split
        p = _bwd(head_dim=256, **kw)
        S = kw.get("seqlen_q", 1000)
        assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(p)) == _bwd_ws(2, 8, 2, 256, 2 * S, S)
    assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(_bwd(head_dim=96))) == _bwd_ws(
        2, 8, 2, 96, 2000, 1000)
    assert lib.mi_attn_bwd_workspace_bytes(ctypes.byref(_bwd(head_dim=80))) == 0
    assert "head_dim" in mi.mi_attn_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=80), mi.MI_ATTN_EUNSUPPORTED),
    (dict(head_dim=160), mi.MI_ATTN_EUNSUPPORTED),
    (dict(num_heads_q=7), mi.MI_ATTN_EINVAL),
    (dict(dout=0), mi.MI_ATTN_EINVAL),
    (dict(dk=FAKE + 4), mi.MI_ATTN_EINVAL),
    (dict(do_row_stride=100), mi.MI_ATTN_EINVAL),
    (dict(dq_head_stride=-8), mi.MI_ATTN_EINVAL),
    (dict(dv_row_stride=64), mi.MI_ATTN_EINVAL),           # rows would overlap (< head_dim)
    (dict(cu_seqlens_k=FAKE), mi.MI_ATTN_EINVAL),          # cu_seqlens go together
    (dict(softmax_scale=float("inf")), mi.MI_ATTN_EUNSUPPORTED),
    (dict(seqlen_k=-1), mi.MI_ATTN_EINVAL),
    (dict(workspace=0), mi.MI_ATTN_EWORKSPACE),
    (dict(workspace_bytes=100), mi.MI_ATTN_EWORKSPACE),
    (dict(batch=70000), mi.MI_ATTN_EINVAL),
])
def test_bwd_invalid_arguments(lib, kw, code):
    rc = lib.mi_attn_bwd(ctypes.byref(_bwd(**kw)), None)
    assert rc == code, (rc, mi.mi_attn_last_error())
    assert mi.mi_attn_last_error()


def test_bwd_null_and_empty(lib):
    assert lib.mi_attn_bwd(None, None) == mi.MI_ATTN_EINVAL
    assert lib.mi_attn_bwd(ctypes.byref(_bwd(batch=0)), None) == mi.MI_ATTN_OK
