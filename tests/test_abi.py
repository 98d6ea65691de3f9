"""The C ABI: library loads, exports what include/attn.h declares, and rejects
bad arguments on the host before anything is enqueued.

These tests never launch a kernel: every call carries an argument the library
must refuse.  They only run where no GPU is visible, so that even a
validation bug cannot send the fake pointers below to a device.
"""

import ctypes
import os
import re

import pytest
import torch

import transformer_causal_head_amd as tch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="host-validation tests use fake pointers; CPU only")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(tch.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = tch.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_strerror_covers_all_codes():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert tch.attn_strerror(code) and "unknown" not in tch.attn_strerror(code)
    assert "unknown" in tch.attn_strerror(-99)


def test_workspace_query():
    n = tch.attn_decode_workspace_bytes(64, 32, 8, 128, 32768, tch.ATTN_BF16)
    # one (m, l, o[128]) fp32 record per (sequence, query head, key chunk),
    # and for the even split the first and last range of each (sequence, K/V
    # head) as two int32
    rec = 64 * 32 * (128 + 2) * 4
    seg = 64 * 8 * 2 * 4
    assert n > seg and (n - seg) % rec == 0 and 1 <= (n - seg) // rec <= 32768 // 32
    assert tch.attn_decode_workspace_bytes(64, 32, 8, 128, 32768, tch.ATTN_F32) == 0
    assert tch.attn_decode_workspace_bytes(64, 30, 8, 128, 32768, tch.ATTN_BF16) == 0
    assert tch.attn_decode_workspace_bytes(0, 32, 8, 128, 32768, tch.ATTN_BF16) == 0
    # a window shorter than the cache: shorter chunks, and only the chunks a
    # window can touch get a slot
    assert tch.attn_decode_window_workspace_bytes(64, 32, 8, 128, 32768, 0, tch.ATTN_BF16) == n
    nw = tch.attn_decode_window_workspace_bytes(64, 32, 8, 128, 32768, 1024, tch.ATTN_BF16)
    assert nw > seg and (nw - seg) % rec == 0 and (nw - seg) // rec <= 32
    assert tch.attn_decode_window_workspace_bytes(64, 32, 8, 128, 32768, 40000,
                                                  tch.ATTN_BF16) == n


FAKE = ctypes.c_void_p(0x1000)


def _prefill(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, LSE=None, B=1, Nq=4, Nkv=2, S=16, Dh=128,
             causal=1, window=0, scale=0.125, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    return tch.lib().attn_prefill(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Nq"],
                                  a["Nkv"], a["S"], a["Dh"], a["causal"], a["window"],
                                  a["scale"], a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), tch.ATTN_EINVAL),
    (dict(K=None), tch.ATTN_EINVAL),
    (dict(V=None), tch.ATTN_EINVAL),
    (dict(O=None), tch.ATTN_EINVAL),
    (dict(B=0), tch.ATTN_EINVAL),
    (dict(Nq=0), tch.ATTN_EINVAL),
    (dict(Nkv=-2), tch.ATTN_EINVAL),
    (dict(S=0), tch.ATTN_EINVAL),
    (dict(Dh=0), tch.ATTN_EINVAL),
    (dict(Nq=6, Nkv=4), tch.ATTN_EGQA),
    (dict(Dh=257), tch.ATTN_EUNSUPPORTED),
    (dict(dtype=7), tch.ATTN_EUNSUPPORTED),
    (dict(causal=0, window=4), tch.ATTN_EINVAL),
    (dict(causal=2), tch.ATTN_EINVAL),
    (dict(scale=0.0), tch.ATTN_EINVAL),
    (dict(scale=-1.0), tch.ATTN_EINVAL),
    (dict(scale=float("inf")), tch.ATTN_EINVAL),
    (dict(scale=float("nan")), tch.ATTN_EINVAL),
    # one head of the MFMA kernel must fit a 31-bit byte range
    (dict(S=8388608), tch.ATTN_EUNSUPPORTED),
    (dict(S=16777216, Dh=64), tch.ATTN_EUNSUPPORTED),
    (dict(S=4194304, Dh=256), tch.ATTN_EUNSUPPORTED),
])
def test_prefill_rejects(kw, code):
    assert _prefill(**kw) == code


def _decode(**kw):
    a = dict(q=FAKE, K=FAKE, V=FAKE, lens=FAKE, O=FAKE, B=2, Nq=8, Nkv=2, Dh=128, Tcap=64,
             LSE=None, ws=FAKE, ws_bytes=1 << 30, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    return tch.lib().attn_decode(a["q"], a["K"], a["V"], a["lens"], a["O"], a["B"], a["Nq"],
                                 a["Nkv"], a["Dh"], a["Tcap"], a["LSE"], a["ws"],
                                 a["ws_bytes"], a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), tch.ATTN_EINVAL),
    (dict(K=None), tch.ATTN_EINVAL),
    (dict(V=None), tch.ATTN_EINVAL),
    (dict(lens=None), tch.ATTN_EINVAL),
    (dict(O=None), tch.ATTN_EINVAL),
    (dict(B=0), tch.ATTN_EINVAL),
    (dict(Tcap=0), tch.ATTN_EINVAL),
    (dict(Nq=8, Nkv=3), tch.ATTN_EGQA),
    (dict(Dh=300), tch.ATTN_EUNSUPPORTED),
    (dict(dtype=5), tch.ATTN_EUNSUPPORTED),
    (dict(ws=None), tch.ATTN_EWORKSPACE),
    (dict(ws_bytes=16), tch.ATTN_EWORKSPACE),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def test_python_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tch.attn_prefill(q, q, q, q.clone(), None)


def _decode_tensors(dtype=torch.bfloat16, k=None, v=None, o=None, kn=None, vn=None):
    B, Nq, Nkv, Dh, T = 2, 4, 2, 64, 8
    q = torch.zeros(B, Nq, Dh, dtype=dtype)
    return dict(q=q, Kcache=torch.zeros(B, Nkv, T, Dh, dtype=k or dtype),
                Vcache=torch.zeros(B, Nkv, T, Dh, dtype=v or dtype),
                lens=torch.ones(B, dtype=torch.int32), O=torch.zeros(B, Nq, Dh, dtype=o or dtype),
                knew=torch.zeros(B, Nkv, Dh, dtype=kn or dtype),
                vnew=torch.zeros(B, Nkv, Dh, dtype=vn or dtype))


@pytest.mark.parametrize("mix", [dict(k=torch.float32), dict(v=torch.float32),
                                 dict(o=torch.float32), dict(kn=torch.float32),
                                 dict(vn=torch.float32)])
@pytest.mark.parametrize("entry", ["attn_decode", "attn_decode_window", "attn_decode_padded",
                                   "attn_decode_append"])
def test_decode_binding_refuses_mixed_dtypes(entry, mix):
    # the C ABI takes q's element type for every buffer: a bf16 query with an
    # fp32 cache (or output, or new row) must be refused before the library
    # is called.  The tensors are on the CPU, so a call would raise too; the
    # message shows which check fired.
    if entry != "attn_decode_append" and ("kn" in mix or "vn" in mix):
        pytest.skip("no new rows in this entry point")
    t = _decode_tensors(**mix)
    args = {"attn_decode": (t["q"], t["Kcache"], t["Vcache"], t["lens"], t["O"]),
            "attn_decode_window": (t["q"], t["Kcache"], t["Vcache"], t["lens"], t["O"]),
            "attn_decode_padded": (t["q"], t["Kcache"], t["Vcache"], t["lens"], None, t["O"]),
            "attn_decode_append": (t["q"], t["knew"], t["vnew"], t["Kcache"], t["Vcache"],
                                   t["lens"], t["lens"], t["O"])}[entry]
    with pytest.raises(ValueError, match="share one dtype"):
        getattr(tch, entry)(*args)


@pytest.mark.parametrize("entry", ["attn_prefill", "attn_decode", "attn_prefill_cache"])
def test_binding_requires_float32_lse(entry):
    # LSE is fp32 in the C ABI: a 4-byte integer tensor must be refused
    if entry == "attn_decode":
        t = _decode_tensors()
        lse = torch.zeros(2, 4, dtype=torch.int32)
        call = lambda: tch.attn_decode(t["q"], t["Kcache"], t["Vcache"], t["lens"], t["O"], lse)
    else:
        q = torch.zeros(1, 2, 4, 8, dtype=torch.bfloat16)
        lse = torch.zeros(1, 2, 4, dtype=torch.int32)
        if entry == "attn_prefill":
            call = lambda: tch.attn_prefill(q, q, q, q.clone(), lse)
        else:
            call = lambda: tch.attn_prefill_cache(q, q, q, torch.full((1,), 4, dtype=torch.int32),
                                                  q.clone(), lse)
    with pytest.raises(ValueError, match="LSE must be float32"):
        call()


def _prefill_cache(**kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, lens=FAKE, O=FAKE, LSE=None, B=2, Nq=8, Nkv=2, Sq=16,
             Dh=128, Tcap=64, window=0, scale=0.125, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    return tch.lib().attn_prefill_cache(a["Q"], a["K"], a["V"], a["lens"], a["O"], a["LSE"],
                                        a["B"], a["Nq"], a["Nkv"], a["Sq"], a["Dh"], a["Tcap"],
                                        a["window"], a["scale"], a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), tch.ATTN_EINVAL),
    (dict(lens=None), tch.ATTN_EINVAL),
    (dict(O=None), tch.ATTN_EINVAL),
    (dict(B=0), tch.ATTN_EINVAL),
    (dict(Sq=0), tch.ATTN_EINVAL),
    (dict(Tcap=0), tch.ATTN_EINVAL),
    (dict(Sq=65), tch.ATTN_EINVAL),
    (dict(Nq=6, Nkv=4), tch.ATTN_EGQA),
    (dict(Dh=257), tch.ATTN_EUNSUPPORTED),
    (dict(dtype=3), tch.ATTN_EUNSUPPORTED),
    (dict(scale=0.0), tch.ATTN_EINVAL),
    (dict(scale=float("nan")), tch.ATTN_EINVAL),
    (dict(Tcap=8388608), tch.ATTN_EUNSUPPORTED),
])
def test_prefill_cache_rejects(kw, code):
    assert _prefill_cache(**kw) == code


def _decode_window(**kw):
    a = dict(q=FAKE, K=FAKE, V=FAKE, lens=FAKE, O=FAKE, B=2, Nq=8, Nkv=2, Dh=128, Tcap=64,
             window=16, scale=0.1, LSE=None, ws=FAKE, ws_bytes=1 << 30, dtype=tch.ATTN_BF16,
             stream=None)
    a.update(kw)
    return tch.lib().attn_decode_window(a["q"], a["K"], a["V"], a["lens"], a["O"], a["B"],
                                        a["Nq"], a["Nkv"], a["Dh"], a["Tcap"], a["window"],
                                        a["scale"], a["LSE"], a["ws"], a["ws_bytes"],
                                        a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), tch.ATTN_EINVAL),
    (dict(lens=None), tch.ATTN_EINVAL),
    (dict(Tcap=0), tch.ATTN_EINVAL),
    (dict(scale=-1.0), tch.ATTN_EINVAL),
    (dict(scale=float("inf")), tch.ATTN_EINVAL),
    (dict(Nq=8, Nkv=3), tch.ATTN_EGQA),
    (dict(Dh=300), tch.ATTN_EUNSUPPORTED),
    (dict(ws=None), tch.ATTN_EWORKSPACE),
    (dict(ws_bytes=16), tch.ATTN_EWORKSPACE),
])
def test_decode_window_rejects(kw, code):
    assert _decode_window(**kw) == code


def _append(**kw):
    a = dict(Kn=FAKE, Vn=FAKE, K=FAKE, V=FAKE, pos=FAKE, B=2, Nkv=2, Snew=4, Dh=128, Tcap=64,
             rolling=0, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    return tch.lib().attn_kv_append(a["Kn"], a["Vn"], a["K"], a["V"], a["pos"], a["B"],
                                    a["Nkv"], a["Snew"], a["Dh"], a["Tcap"], a["rolling"],
                                    a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(Kn=None), tch.ATTN_EINVAL),
    (dict(V=None), tch.ATTN_EINVAL),
    (dict(pos=None), tch.ATTN_EINVAL),
    (dict(B=0), tch.ATTN_EINVAL),
    (dict(Snew=0), tch.ATTN_EINVAL),
    (dict(Tcap=-1), tch.ATTN_EINVAL),
    (dict(rolling=2), tch.ATTN_EINVAL),
    (dict(Snew=65), tch.ATTN_EINVAL),
    (dict(dtype=9), tch.ATTN_EUNSUPPORTED),
    (dict(Dh=257), tch.ATTN_EUNSUPPORTED),
])
def test_kv_append_rejects(kw, code):
    assert _append(**kw) == code


def _backward(padded=False, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, LSE=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE, B=1,
             Nq=4, Nkv=2, S=16, Dh=128, causal=1, window=0, scale=0.125, ws=FAKE,
             ws_bytes=1 << 20, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    if padded:  # the padded form rejects exactly what the plain one does
        return tch.lib().attn_backward_padded(
            a["Q"], a["K"], a["V"], FAKE, a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
            a["B"], a["Nq"], a["Nkv"], a["S"], a["Dh"], a["causal"], a["window"], a["scale"],
            a["ws"], a["ws_bytes"], a["dtype"], a["stream"])
    return tch.lib().attn_backward(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"],
                                   a["dK"], a["dV"], a["B"], a["Nq"], a["Nkv"], a["S"], a["Dh"],
                                   a["causal"], a["window"], a["scale"], a["ws"], a["ws_bytes"],
                                   a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), tch.ATTN_EINVAL),
    (dict(LSE=None), tch.ATTN_EINVAL),
    (dict(dV=None), tch.ATTN_EINVAL),
    (dict(S=0), tch.ATTN_EINVAL),
    (dict(causal=0, window=3), tch.ATTN_EINVAL),
    (dict(scale=0.0), tch.ATTN_EINVAL),
    (dict(Nq=6, Nkv=4), tch.ATTN_EGQA),
    (dict(Dh=512), tch.ATTN_EUNSUPPORTED),
    (dict(ws=None), tch.ATTN_EWORKSPACE),
    (dict(ws_bytes=4), tch.ATTN_EWORKSPACE),
    (dict(S=8388608), tch.ATTN_EUNSUPPORTED),
])
@pytest.mark.parametrize("padded", [False, True])
def test_backward_rejects(kw, code, padded):
    assert _backward(padded=padded, **kw) == code


def test_backward_workspace_query():
    assert tch.attn_backward_workspace_bytes(2, 8, 2, 100, 128, tch.ATTN_BF16) == 2 * 2 * 8 * 100 * 4
    assert tch.attn_backward_workspace_bytes(2, 8, 3, 100, 128, tch.ATTN_BF16) == 0


@no_gpu
@pytest.mark.parametrize("args,code", [
    ((None, 2, 100, FAKE, None), tch.ATTN_EINVAL),
    ((FAKE, 0, 100, FAKE, None), tch.ATTN_EINVAL),
    ((FAKE, 2, 0, FAKE, None), tch.ATTN_EINVAL),
    ((FAKE, 2, 100, None, None), tch.ATTN_EINVAL),
])
def test_pack_key_mask_rejects(args, code):
    assert tch.lib().attn_pack_key_mask(*args) == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(Nkv=3), tch.ATTN_EGQA),
    (dict(causal=0, window=4), tch.ATTN_EINVAL),
    (dict(Dh=300), tch.ATTN_EUNSUPPORTED),
    (dict(Q=None), tch.ATTN_EINVAL),
    (dict(scale=0.0), tch.ATTN_EINVAL),
])
def test_padded_entry_points_reject(kw, code):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, B=1, Nq=4, Nkv=2, S=16, Dh=128, causal=1, window=0,
             scale=0.125)
    a.update(kw)
    L = tch.lib()
    assert L.attn_prefill_padded(a["Q"], a["K"], a["V"], FAKE, a["O"], None, a["B"], a["Nq"],
                                 a["Nkv"], a["S"], a["Dh"], a["causal"], a["window"], a["scale"],
                                 tch.ATTN_BF16, None) == code
    if "causal" in kw:
        return  # the cache forms are causal by construction
    assert L.attn_prefill_cache_padded(a["Q"], a["K"], a["V"], FAKE, FAKE, a["O"], None, a["B"],
                                       a["Nq"], a["Nkv"], 4, a["Dh"], a["S"], 0, a["scale"],
                                       tch.ATTN_BF16, None) == code
    assert L.attn_decode_padded(a["Q"], a["K"], a["V"], FAKE, FAKE, a["O"], a["B"], a["Nq"],
                                a["Nkv"], a["Dh"], a["S"], 0, a["scale"], None, FAKE, 1 << 30,
                                tch.ATTN_BF16, None) == code


@no_gpu
def test_padded_cache_forms_check_chunk_and_workspace():
    L = tch.lib()
    # a chunk longer than the cache
    assert L.attn_prefill_cache_padded(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 32, 128,
                                       16, 0, 0.125, tch.ATTN_BF16, None) == tch.ATTN_EINVAL
    # the split-K decode needs its workspace
    assert L.attn_decode_padded(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 8, 128, 4096, 0, 0.1,
                                None, None, 0, tch.ATTN_BF16, None) == tch.ATTN_EWORKSPACE


@no_gpu
@pytest.mark.parametrize("args,code", [
    ((None, 16, 64, 10000.0, None), tch.ATTN_EINVAL),
    ((FAKE, 0, 64, 10000.0, None), tch.ATTN_EINVAL),
    ((FAKE, 16, 63, 10000.0, None), tch.ATTN_EINVAL),
    ((FAKE, 16, 64, 1.0, None), tch.ATTN_EINVAL),
    ((FAKE, 16, 64, float("inf"), None), tch.ATTN_EINVAL),
])
def test_rope_table_rejects(args, code):
    assert tch.lib().attn_rope_cos_sin(*args) == code


def _rope(**kw):
    a = dict(X=FAKE, Y=FAKE, positions=None, start=None, table=FAKE, P=64, B=1, H=4, S=16, Dh=128,
             style=0, dtype=tch.ATTN_BF16)
    a.update(kw)
    return tch.lib().attn_rope(a["X"], a["Y"], a["positions"], a["start"], a["table"], a["P"],
                               a["B"], a["H"], a["S"], a["Dh"], a["style"], a["dtype"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(X=None), tch.ATTN_EINVAL),
    (dict(table=None), tch.ATTN_EINVAL),
    (dict(Dh=127), tch.ATTN_EINVAL),
    (dict(style=2), tch.ATTN_EINVAL),
    (dict(P=0), tch.ATTN_EINVAL),
    (dict(S=0), tch.ATTN_EINVAL),
    (dict(dtype=7), tch.ATTN_EUNSUPPORTED),
])
def test_rope_rejects(kw, code):
    assert _rope(**kw) == code


def _append_rope(**kw):
    a = dict(Kn=FAKE, Vn=FAKE, Kc=FAKE, Vc=FAKE, pos=FAKE, positions=None, table=FAKE, P=64, B=2,
             Nkv=2, Snew=3, Dh=128, Tcap=16, rolling=0, style=0, dtype=tch.ATTN_BF16)
    a.update(kw)
    return tch.lib().attn_kv_append_rope(a["Kn"], a["Vn"], a["Kc"], a["Vc"], a["pos"],
                                         a["positions"], a["table"], a["P"], a["B"], a["Nkv"],
                                         a["Snew"], a["Dh"], a["Tcap"], a["rolling"], a["style"],
                                         a["dtype"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(pos=None), tch.ATTN_EINVAL),
    (dict(table=None), tch.ATTN_EINVAL),
    (dict(Snew=20), tch.ATTN_EINVAL),
    (dict(Dh=7), tch.ATTN_EINVAL),
    (dict(style=-1), tch.ATTN_EINVAL),
    (dict(rolling=2), tch.ATTN_EINVAL),
    (dict(dtype=3), tch.ATTN_EUNSUPPORTED),
])
def test_kv_append_rope_rejects(kw, code):
    assert _append_rope(**kw) == code


def _decode_append(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, Kc=FAKE, Vc=FAKE, lens=FAKE, slot=FAKE, O=FAKE, B=4, Nq=32,
             Nkv=8, Dh=128, Tcap=4096, window=0, scale=0.1, LSE=None, ws=None, wsb=0,
             dtype=tch.ATTN_BF16)
    a.update(kw)
    return tch.lib().attn_decode_append(a["q"], a["kn"], a["vn"], a["Kc"], a["Vc"], a["lens"],
                                        a["slot"], a["O"], a["B"], a["Nq"], a["Nkv"], a["Dh"],
                                        a["Tcap"], a["window"], a["scale"], a["LSE"], a["ws"],
                                        a["wsb"], a["dtype"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(slot=None), tch.ATTN_EINVAL),
    (dict(kn=None), tch.ATTN_EINVAL),
    (dict(Nkv=5), tch.ATTN_EGQA),
    (dict(Tcap=0), tch.ATTN_EINVAL),
    (dict(scale=-1.0), tch.ATTN_EINVAL),
    (dict(Dh=512), tch.ATTN_EUNSUPPORTED),
    (dict(), tch.ATTN_EWORKSPACE),           # the split-K decode needs its workspace
])
def test_decode_append_rejects(kw, code):
    assert _decode_append(**kw) == code


def _decode_noalloc(**kw):
    a = dict(q=FAKE, K=FAKE, V=FAKE, lens=FAKE, O=FAKE, B=2, Nq=8, Nkv=2, Dh=128, Tcap=64,
             LSE=None, dtype=tch.ATTN_BF16, stream=None)
    a.update(kw)
    return tch.lib().attn_decode_noalloc(a["q"], a["K"], a["V"], a["lens"], a["O"], a["B"],
                                         a["Nq"], a["Nkv"], a["Dh"], a["Tcap"], a["LSE"],
                                         a["dtype"], a["stream"])


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), tch.ATTN_EINVAL),
    (dict(lens=None), tch.ATTN_EINVAL),
    (dict(O=None), tch.ATTN_EINVAL),
    (dict(B=0), tch.ATTN_EINVAL),
    (dict(Tcap=0), tch.ATTN_EINVAL),
    (dict(Nq=8, Nkv=3), tch.ATTN_EGQA),
    (dict(Dh=300), tch.ATTN_EUNSUPPORTED),
    (dict(dtype=5), tch.ATTN_EUNSUPPORTED),
    # twice the decode workload's batch needs 40 MB of partials: more than the fixed scratch
    (dict(B=128, Nq=32, Nkv=8, Tcap=32768), tch.ATTN_ESCRATCH),
    (dict(B=1, Nq=32, Nkv=8, Tcap=1 << 22), tch.ATTN_ESCRATCH),
])
def test_decode_noalloc_rejects(kw, code):
    assert _decode_noalloc(**kw) == code


def test_decode_noalloc_limit_covers_the_decode_workload():
    # the 64-sequence, 32/8-head, 32768-slot decode at head size 128 fits the fixed
    # scratch; twice its batch does not
    need = tch.attn_decode_workspace_bytes(64, 32, 8, 128, 32768, tch.ATTN_BF16)
    assert 0 < need <= tch.ATTN_NOALLOC_SCRATCH_BYTES
    assert tch.attn_decode_workspace_bytes(128, 32, 8, 128, 32768,
                                           tch.ATTN_BF16) > tch.ATTN_NOALLOC_SCRATCH_BYTES
    header = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in header
    assert tch.ATTN_NOALLOC_SCRATCH_BYTES == 32 << 20


@no_gpu
@pytest.mark.parametrize("entry", ["attn_prefill_rope", "attn_prefill_cache_rope", "attn_decode_rope"])
@pytest.mark.parametrize("kw,code", [
    (dict(table=None), tch.ATTN_EINVAL),
    (dict(P=0), tch.ATTN_EINVAL),
    (dict(style=2), tch.ATTN_EINVAL),
    (dict(Dh=65), tch.ATTN_EINVAL),      # rotation pairs need an even head size
    (dict(Nq=6, Nkv=4), tch.ATTN_EGQA),  # then the checks of the unrotated form
    (dict(Q=None), tch.ATTN_EINVAL),
])
def test_rope_entry_points_reject(entry, kw, code):
    a = dict(Q=FAKE, table=FAKE, P=100, style=0, Dh=128, Nq=8, Nkv=2)
    a.update(kw)
    L = tch.lib()
    if entry == "attn_prefill_rope":
        st = L.attn_prefill_rope(a["Q"], FAKE, FAKE, None, FAKE, None, 1, a["Nq"], a["Nkv"], 16,
                                 a["Dh"], 1, 0, 0.125, a["table"], a["P"], None, None, a["style"],
                                 tch.ATTN_BF16, None)
    elif entry == "attn_prefill_cache_rope":
        st = L.attn_prefill_cache_rope(a["Q"], FAKE, FAKE, FAKE, None, FAKE, None, 2, a["Nq"],
                                       a["Nkv"], 16, a["Dh"], 64, 0, 0.125, a["table"], a["P"],
                                       None, None, a["style"], tch.ATTN_BF16, None)
    else:
        st = L.attn_decode_rope(a["Q"], FAKE, FAKE, FAKE, None, FAKE, 2, a["Nq"], a["Nkv"], a["Dh"],
                                64, 0, 0.125, a["table"], a["P"], None, a["style"], None, FAKE,
                                1 << 30, tch.ATTN_BF16, None)
    assert st == code
