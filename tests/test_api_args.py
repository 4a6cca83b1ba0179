"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import decode_attention_paged_attn_amd as pda
from decode_attention_paged_attn_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pda.library_path()):
        build_lib.build()
    return pda.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_api():
    names = set(declared_functions())
    assert {"paged_decode_attn", "paged_decode_attn_partial", "merge_partials",
            "pda_workspace_size", "pda_workspace_layout", "pda_last_error",
            "pda_version", "paged_decode_attn_fp8", "paged_decode_attn_partial_fp8",
            "paged_kv_append", "pda_multi_query_workspace_size", "paged_multi_query_attn",
            "paged_multi_query_attn_partial", "paged_multi_query_attn_fp8",
            "paged_multi_query_attn_partial_fp8"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_empty_error(lib):
    assert b"gfx950" in lib.pda_version()


def _ws(B=2, Hq=8, Hkv=2, D=128, bs=16, mb=32, P=0):
    n = ctypes.c_size_t(0)
    rc = pda.load_library().pda_workspace_size(B, Hq, Hkv, D, bs, mb, P, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), 1),        # Hq % Hkv != 0
    (dict(Hq=48, Hkv=4), 2),       # G = 12 not built
    (dict(D=64), 2),
    (dict(bs=32), 2),
    (dict(P=24), 1),               # not a multiple of the block size
    (dict(P=-16), 1),
    (dict(P=1 << 21), 2),          # above the largest unit
    (dict(Hq=12, Hkv=4), 2),       # G = 3 not built (1, 2, 4, 6, 8 are)
    (dict(Hq=128, Hkv=128), 2),    # more than 64 KV heads
    (dict(B=-1), 1),
    (dict(mb=-1), 1),
    (dict(Hkv=0), 1),
])
def test_workspace_size_rejects(lib, kw, code):
    rc, _ = _ws(**kw)
    assert rc == code
    assert lib.pda_last_error()


def test_decode_workspace_size_covers_every_kv_head_count(lib):
    """paged_decode_attn_workspace_size (no Hkv argument) is the largest
    pda_workspace_size over the supported KV-head counts of Hq."""
    for B, Hq, mb, P in ((3, 32, 100, 256), (16, 32, 12800, 512), (1, 8, 1, 0)):
        n = ctypes.c_size_t(0)
        assert lib.paged_decode_attn_workspace_size(B, Hq, 128, 16, mb, P, ctypes.byref(n)) == 0
        per = []
        for Hkv in range(1, Hq + 1):
            if Hq % Hkv == 0:
                rc, m = _ws(B=B, Hq=Hq, Hkv=Hkv, mb=mb, P=P)
                if rc == 0:
                    per.append(m)
        assert per and n.value == max(per)
        assert pda.decode_workspace_size(B, Hq, mb, P) == n.value
    n = ctypes.c_size_t(0)
    assert lib.paged_decode_attn_workspace_size(2, 8, 64, 16, 4, 0, ctypes.byref(n)) == 2   # D
    assert lib.paged_decode_attn_workspace_size(-1, 8, 128, 16, 4, 0, ctypes.byref(n)) == 1
    assert lib.paged_decode_attn_workspace_size(2, 8, 128, 16, 4, 24, ctypes.byref(n)) == 1
    assert lib.paged_decode_attn_workspace_size(2, 0, 128, 16, 4, 0, ctypes.byref(n)) == 1
    assert lib.paged_decode_attn_workspace_size(2, 8, 128, 16, 4, 0, None) == 1


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (48, 8), (64, 8), (32, 32), (40, 40), (48, 48),
                                   (12, 3), (10, 5), (6, 6), (56, 7), (30, 5)])
def test_workspace_size_accepts_the_head_shapes(lib, Hq, Hkv):
    """The pages' GQA (Q32:KV8, Q48:KV8, Q64:KV8) and MHA (Q32:KV32, Q40:KV40,
    Q48:KV48) shapes, and odd KV-head counts, are built."""
    rc, n = _ws(B=4, Hq=Hq, Hkv=Hkv, mb=64)
    assert rc == 0 and n > 0
    c = ctypes.c_size_t(0)
    assert lib.pda_multi_query_workspace_size(4, 20, Hq, Hkv, 128, 16, 64, 0,
                                              ctypes.byref(c)) == 0 and c.value > 0


def test_workspace_size_formula(lib):
    # header int32[4 + B], lse fp32[n_slots, Hq], o fp32[n_slots, Hq, D], each 256-aligned
    B, Hq, Hkv, mb, P = 3, 32, 8, 100, 256
    rc, n = _ws(B=B, Hq=Hq, Hkv=Hkv, mb=mb, P=P)
    assert rc == 0
    lay = pda.workspace_layout(B, Hq, Hkv, mb, P)
    align = lambda x: (x + 255) // 256 * 256   # noqa: E731
    slots = lay["n_runs"] + B
    assert lay["n_slots"] == slots and lay["unit_tokens"] == P
    assert lay["header_offset"] == 0
    assert lay["lse_offset"] == align(4 * (4 + B))
    assert lay["o_offset"] == lay["lse_offset"] + align(4 * slots * Hq)
    assert lay["total_bytes"] == lay["o_offset"] + align(4 * slots * Hq * 128)
    # the size covers both KV formats (their run counts may differ)
    assert n == max(lay["total_bytes"], pda.workspace_layout(B, Hq, Hkv, mb, P, kv_fp8=True)["total_bytes"])
    assert pda.workspace_layout(B, Hq, Hkv, mb, 0)["unit_tokens"] == 16
    assert pda.workspace_size(0, Hq, Hkv, mb, P) == 0


def _call_attn(lib, **over):
    a = dict(out=1, q=1, k=1, v=1, bt=1, bt_stride=4, ctx=1, B=2, Hq=8, Hkv=2, D=128, bs=16,
             nblocks=10, mb=4, scale=0.1, P=0, lse=None, ws=256, ws_bytes=1 << 30, stream=None)
    a.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)   # noqa: E731
    return lib.paged_decode_attn(vp(a["out"]), vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]),
                                 a["bt_stride"], vp(a["ctx"]), a["B"], a["Hq"], a["Hkv"], a["D"],
                                 a["bs"], a["nblocks"], a["mb"], a["scale"], a["P"], vp(a["lse"]),
                                 vp(a["ws"]), a["ws_bytes"], vp(a["stream"]))


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(ctx=None), 1),
    (dict(Hq=6, Hkv=4), 1),
    (dict(D=96), 2),
    (dict(bs=8), 2),
    (dict(P=40), 1),
    (dict(bt_stride=3), 1),        # narrower than max_blocks_per_seq
    (dict(nblocks=0), 1),
    (dict(scale=float("inf")), 1),
    (dict(ws=None), 1),
    (dict(ws_bytes=16), 1),        # too small
    (dict(ws=257), 1),             # misaligned
])
def test_paged_decode_attn_rejects_before_launch(lib, over, code):
    assert _call_attn(lib, **over) == code
    assert lib.pda_last_error()


def test_empty_batch_is_a_no_op(lib):
    assert _call_attn(lib, B=0, out=None, q=None, ws=None) == 0


def test_merge_partials_rejects(lib):
    vp = ctypes.c_void_p
    assert lib.merge_partials(vp(1), None, vp(1), vp(1), 0, 2, 8, 128, None) == 1
    assert lib.merge_partials(vp(1), None, vp(1), vp(1), 2, 2, 8, 64, None) == 2
    assert lib.merge_partials(None, None, vp(1), vp(1), 2, 2, 8, 128, None) == 1
    assert lib.merge_partials(vp(1), None, vp(1), vp(1), 2, 0, 8, 128, None) == 0


def test_partial_requires_lse(lib):
    vp = ctypes.c_void_p
    rc = lib.paged_decode_attn_partial(vp(1), None, vp(1), vp(1), vp(1), vp(1), 4, vp(1), 2, 8,
                                       2, 128, 16, 10, 4, 0.1, 0, vp(256), 1 << 30, None)
    assert rc == 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from decode_attention_paged_attn_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setenv("PDA_LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load_library()


def test_kv_append_rejects(lib):
    vp = ctypes.c_void_p
    args = [vp(1), vp(1), vp(1), vp(1), vp(1), 4, vp(1), 2, 8, 128, 16, 10, 4, None]
    bad_d = list(args)
    bad_d[9] = 64
    assert lib.paged_kv_append(*bad_d) == 2
    bad_ptr = list(args)
    bad_ptr[0] = None
    assert lib.paged_kv_append(*bad_ptr) == 1
    bad_stride = list(args)
    bad_stride[5] = 3
    assert lib.paged_kv_append(*bad_stride) == 1
    empty = list(args)
    empty[7] = 0
    assert lib.paged_kv_append(*empty) == 0


# --- multi-query ------------------------------------------------------------------

def _mq_ws(S=3, T=9, Hq=8, Hkv=2, D=128, bs=16, mb=32, P=0):
    n = ctypes.c_size_t(0)
    rc = pda.load_library().pda_multi_query_workspace_size(S, T, Hq, Hkv, D, bs, mb, P,
                                                           ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(S=4001), 2),             # more sequences than the plan kernel holds
    (dict(S=-1), 1),
    (dict(T=-1), 1),
    (dict(Hq=12, Hkv=4), 2),       # G = 3 not built
    (dict(Hq=7, Hkv=2), 1),        # Hq % Hkv != 0
    (dict(Hq=128, Hkv=128), 2),    # more than 64 KV heads
    (dict(Hq=0), 1),
    (dict(D=64), 2),
    (dict(bs=32), 2),
    (dict(P=24), 1),
    (dict(P=-16), 1),
    (dict(P=1 << 21), 2),
    (dict(mb=-1), 1),
])
def test_multi_query_workspace_size_rejects(lib, kw, code):
    rc, _ = _mq_ws(**kw)
    assert rc == code
    assert lib.pda_last_error()


def test_multi_query_workspace_size_empty_and_limit(lib):
    assert _mq_ws(S=0) == (0, 0)
    assert _mq_ws(T=0) == (0, 0)
    rc, n = _mq_ws(S=4000, T=12000)
    assert rc == 0 and n > 0 and n % 256 == 0
    assert pda.multi_query_workspace_size(4000, 12000, 8, 2, 32) == n


def _call_mq(lib, fp8=False, **over):
    a = dict(out=1, lse=None, q=1, qs=1, T=9, k=1, v=1, bt=1, bt_stride=4, ctx=1, S=3, Hq=8,
             Hkv=2, D=128, bs=16, nblocks=10, mb=4, scale=0.1, k_scale=0.5, v_scale=0.5,
             causal=1, P=0, ws=256, ws_bytes=1 << 30, stream=None)
    a.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)   # noqa: E731
    head = (vp(a["out"]), vp(a["lse"]), vp(a["q"]), vp(a["qs"]), a["T"], vp(a["k"]), vp(a["v"]),
            vp(a["bt"]), a["bt_stride"], vp(a["ctx"]), a["S"], a["Hq"], a["Hkv"], a["D"], a["bs"],
            a["nblocks"], a["mb"], a["scale"])
    tail = (a["causal"], a["P"], vp(a["ws"]), a["ws_bytes"], vp(a["stream"]))
    if fp8:
        return lib.paged_multi_query_attn_fp8(*head, a["k_scale"], a["v_scale"], *tail)
    return lib.paged_multi_query_attn(*head, *tail)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(qs=None), 1),
    (dict(k=None), 1),
    (dict(bt=None), 1),
    (dict(ctx=None), 1),
    (dict(S=4001), 2),
    (dict(Hq=12, Hkv=4), 2),
    (dict(D=96), 2),
    (dict(P=40), 1),
    (dict(bt_stride=3), 1),        # narrower than max_blocks_per_seq
    (dict(nblocks=0), 1),
    (dict(scale=float("nan")), 1),
    (dict(ws=None), 1),
    (dict(ws_bytes=16), 1),        # too small
    (dict(ws=257), 1),             # misaligned
])
def test_multi_query_rejects_before_launch(lib, fp8, over, code):
    assert _call_mq(lib, fp8=fp8, **over) == code
    assert lib.pda_last_error()


@pytest.mark.parametrize("over", [dict(k_scale=float("inf")), dict(v_scale=float("nan"))])
def test_multi_query_fp8_rejects_bad_scales(lib, over):
    assert _call_mq(lib, fp8=True, **over) == 1


def test_multi_query_empty_is_a_no_op(lib):
    assert _call_mq(lib, S=0, out=None, q=None, ws=None) == 0
    assert _call_mq(lib, T=0, out=None, q=None, ws=None) == 0
    assert _call_mq(lib, fp8=True, S=0, out=None, q=None, ws=None) == 0


def test_fused_append_rejects(lib):
    vp = ctypes.c_void_p

    def call(**over):
        a = dict(out=1, q=1, kn=1, vn=1, B=2, ws=256)
        a.update(over)
        f = lambda x: None if x is None else vp(x)   # noqa: E731
        return lib.paged_decode_attn_append(f(a["out"]), f(a["q"]), f(a["kn"]), f(a["vn"]), vp(1),
                                            vp(1), vp(1), 4, vp(1), a["B"], 8, 2, 128, 16, 10, 4,
                                            0.1, 0, None, f(a["ws"]), 1 << 30, None)
    assert call(kn=None) == 1
    assert call(vn=None) == 1
    assert call(out=None) == 1
    assert call(ws=257) == 1
    assert call(B=0, out=None, q=None, kn=None, vn=None, ws=None) == 0


def test_fp8_append_rejects(lib):
    vp = ctypes.c_void_p

    def call(ks=0.5, vs=0.5, ptr=1, B=2):
        p = None if ptr is None else vp(ptr)
        return lib.paged_kv_append_fp8(p, vp(1), vp(1), vp(1), vp(1), 4, vp(1), B, 2, 128, 16, 10,
                                       4, ks, vs, None)
    assert call(ks=float("inf")) == 1
    assert call(vs=float("nan")) == 1
    assert call(ks=0.0) == 1
    assert call(ptr=None) == 1
    assert call(B=0, ptr=None) == 0


def test_fp8_fused_append_rejects(lib):
    vp = ctypes.c_void_p

    def call(ks=0.5, vs=0.5, kn=1):
        return lib.paged_decode_attn_append_fp8(vp(1), vp(1), None if kn is None else vp(kn),
                                                vp(1), vp(1), vp(1), vp(1), 4, vp(1), 2, 8, 2,
                                                128, 16, 10, 4, 0.1, ks, vs, 0, None, vp(256),
                                                1 << 30, None)
    assert call(kn=None) == 1
    assert call(ks=0.0) == 1
    assert call(vs=float("inf")) == 1


def test_stream_read_rejects(lib):
    vp = ctypes.c_void_p
    assert lib.pda_stream_read(None, 64, vp(256), 1, None) == 1
    assert lib.pda_stream_read(vp(256), 64, None, 1, None) == 1
    assert lib.pda_stream_read(vp(257), 64, vp(256), 1, None) == 1     # misaligned source
    assert lib.pda_stream_read(vp(256), 60, vp(256), 0, None) == 1     # size not a multiple of 16
    assert b"16" in lib.pda_last_error()
    assert lib.pda_stream_read(None, 0, None, 1, None) == 0           # nothing to read


def test_lds_probe_rejects(lib):
    vp = ctypes.c_void_p
    assert lib.pda_lds_probe(4, vp(256), 1, 1, None) == 1              # no such form
    assert lib.pda_lds_probe(-1, vp(256), 1, 1, None) == 1
    assert lib.pda_lds_probe(0, vp(256), -1, 1, None) == 1             # negative sizes
    assert lib.pda_lds_probe(0, vp(256), 1, -1, None) == 1
    assert lib.pda_lds_probe(0, None, 1, 1, None) == 1                 # null out
    assert b"null" in lib.pda_last_error()
    assert lib.pda_lds_probe(3, None, 0, 1, None) == 0                 # nothing to launch
