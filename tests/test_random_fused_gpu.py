"""Seeded random shapes for the fused calls: each against the two calls it replaces.

attn_prefill_rope, attn_prefill_cache_rope, attn_decode_rope, attn_decode_append and
attn_kv_append_rope on shapes drawn
from a fixed seed (head sizes 64-256, groups to 32, batches to 64, windows,
key-padding masks, every position mode, both rotation layouts), each compared
with attn_rope followed by the unrotated call (for the rotating append: attn_rope
on the new keys, then attn_kv_append), or with attn_kv_append followed
by attn_decode_window.  Both sides compute the same rows in the same order, so
the bits must match (the caches too, for the append).  One exception: at head
size 256 an unrotated or non-appending decode large enough for the even split
takes it while the fused decode keeps chunk mode, so there the two agree up to
accumulation order.  The fused calls are checked against the oracle by
test_rope_fused_gpu.py and test_cache_gpu.py.
"""

import numpy as np
import pytest
import torch

import transformer_causal_head_amd as tch
from helpers import device, say, takes_even_split

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261204)


def _pick(xs):
    return xs[int(_rng.integers(0, len(xs)))]


def _bits_equal(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _agree(O1, L1, O2, L2, same_form):
    if same_form:
        return _bits_equal(O1, O2) and torch.equal(L1, L2)
    live = torch.isfinite(L1)
    if not torch.equal(live, torch.isfinite(L2)):
        return False
    return ((O1.float() - O2.float()).abs().max().item() <= 2e-2
            and (not live.any() or (L1[live] - L2[live]).abs().max().item() <= 2e-3))


def _key_bits(B, T, g):
    dev = device()
    m = torch.ones(B, T, dtype=torch.bool)
    for b in range(B):
        m[b, :int(g.integers(0, T // 2 + 1))] = False  # left padding
        if T > 10:
            s = int(g.integers(0, T - 5))
            m[b, s:s + int(g.integers(1, 6))] = False  # a hole
    bits = torch.empty(B, (T + 63) // 64, dtype=torch.int64, device=dev)
    tch.attn_pack_key_mask(m.to(dev), bits)
    return bits


def _prefill_cases(n):
    out = []
    for i in range(n):
        Nkv, G, Dh = _pick([1, 2, 4, 8]), _pick([1, 2, 4]), _pick([64, 128, 128, 256])
        B = int(_rng.integers(1, 4))
        S = int(_rng.integers(1, 4097))
        while B * Nkv * G * S * Dh > 16 * 2 ** 20:
            S //= 2
        S = max(S, 1)
        causal = bool(_rng.random() < 0.8)
        window = int(_rng.integers(1, S + 65)) if (causal and _rng.random() < 0.3) else 0
        out.append((i, B, Nkv * G, Nkv, S, Dh, causal, window, _pick(["implicit", "start", "explicit"]),
                    _pick(["pairs", "half"]), bool(_rng.random() < 0.3)))
    return out


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,causal,window,mode,style,pad", _prefill_cases(30))
def test_prefill_rope_random(i, B, Nq, Nkv, S, Dh, causal, window, mode, style, pad):
    dev = device()
    g = np.random.default_rng(100 + i)
    torch.manual_seed(100 + i)
    q = torch.randn(B, Nq, S, Dh, device=dev).to(torch.bfloat16)
    k = torch.randn(B, Nkv, S, Dh, device=dev).to(torch.bfloat16)
    v = torch.randn(B, Nkv, S, Dh, device=dev).to(torch.bfloat16)
    P = S + 3000
    table = tch.rope_table(P, Dh, device=dev)
    pos = start = None
    if mode == "start":
        start = torch.from_numpy(g.integers(0, P - S + 1, B).astype(np.int32)).to(dev)
    elif mode == "explicit":
        pos = torch.from_numpy(g.integers(0, P, (B, S)).astype(np.int32)).to(dev)
    bits = _key_bits(B, S, g) if pad else None
    say(f"random fused prefill {(i, B, Nq, Nkv, S, Dh, causal, window, mode, style, pad)}")
    O1, L1 = torch.empty_like(q), torch.empty(B, Nq, S, device=dev)
    tch.attn_prefill_rope(q, k, v, O1, L1, table, key_bits=bits, positions=pos, start=start,
                          style=style, causal=int(causal), window=window)
    qr = tch.rope(q, table, positions=pos, start=start, style=style)
    O2, L2 = torch.empty_like(q), torch.empty(B, Nq, S, device=dev)
    if pad:
        tch.attn_prefill_padded(qr, k, v, bits, O2, L2, causal=int(causal), window=window)
    else:
        tch.attn_prefill(qr, k, v, O2, L2, causal=int(causal), window=window)
    torch.cuda.synchronize()
    assert _agree(O1, L1, O2, L2, True)


def _decode_cases(n):
    out = []
    for i in range(n):
        Nkv, G, Dh = _pick([1, 2, 4, 8]), _pick([1, 2, 4, 8, 16, 32]), _pick([64, 128, 128, 256])
        if Dh == 256 and G > 16:
            G = 16
        B = int(_rng.integers(1, 65))
        Tcap = int(_rng.integers(16, 8193))
        while B * Nkv * Tcap * Dh > 32 * 2 ** 20:
            Tcap //= 2
        Tcap = max(Tcap, 16)
        window = int(_rng.integers(1, Tcap)) if _rng.random() < 0.3 else 0
        out.append((i, B, Nkv * G, Nkv, Dh, Tcap, window, bool(_rng.random() < 0.5),
                    _pick(["pairs", "half"]), bool(_rng.random() < 0.3)))
    return out


def _decode_inputs(seed, B, Nq, Nkv, Dh, Tcap):
    dev = device()
    g = np.random.default_rng(seed)
    torch.manual_seed(seed)
    q = torch.randn(B, Nq, Dh, device=dev).to(torch.bfloat16)
    kc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(torch.bfloat16)
    vc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(torch.bfloat16)
    lens = torch.from_numpy(g.integers(1, Tcap + 1, B).astype(np.int32)).to(dev)
    return g, q, kc, vc, lens


@pytest.mark.parametrize("i,B,Nq,Nkv,Dh,Tcap,window,explicit,style,pad", _decode_cases(30))
def test_decode_rope_random(i, B, Nq, Nkv, Dh, Tcap, window, explicit, style, pad):
    dev = device()
    g, q, kc, vc, lens = _decode_inputs(500 + i, B, Nq, Nkv, Dh, Tcap)
    P = Tcap + 2000
    table = tch.rope_table(P, Dh, device=dev)
    pos = torch.from_numpy(g.integers(0, P, B).astype(np.int32)).to(dev) if explicit else None
    bits = _key_bits(B, Tcap, g) if pad else None
    ws = torch.empty(tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, tch.ATTN_BF16),
                     dtype=torch.uint8, device=dev)
    say(f"random fused decode {(i, B, Nq, Nkv, Dh, Tcap, window, explicit, style, pad)}")
    O1, L1 = torch.empty_like(q), torch.empty(B, Nq, device=dev)
    tch.attn_decode_rope(q, kc, vc, lens, O1, L1, table, workspace=ws, key_bits=bits, positions=pos,
                         style=style, window=window)
    at = (pos if explicit else lens - 1).view(B, 1).contiguous()
    qr = tch.rope(q.view(B, Nq, 1, Dh), table, positions=at, style=style).view(B, Nq, Dh)
    O2, L2 = torch.empty_like(q), torch.empty(B, Nq, device=dev)
    if pad:
        tch.attn_decode_padded(qr, kc, vc, lens, bits, O2, L2, workspace=ws, window=window)
    else:
        tch.attn_decode_window(qr, kc, vc, lens, O2, L2, workspace=ws, window=window)
    torch.cuda.synchronize()
    same_form = not (Dh == 256 and not pad and takes_even_split(B, Nq, Nkv, Dh, Tcap, window))
    assert _agree(O1, L1, O2, L2, same_form)


@pytest.mark.parametrize("i,B,Nq,Nkv,Dh,Tcap,window,explicit,style,pad", _decode_cases(30))
def test_decode_append_random(i, B, Nq, Nkv, Dh, Tcap, window, explicit, style, pad):
    # explicit, style and pad are drawn for the shared generator and unused here
    dev = device()
    g, q, kc, vc, lens = _decode_inputs(1500 + i, B, Nq, Nkv, Dh, Tcap)
    knew = torch.randn(B, Nkv, Dh, device=dev).to(torch.bfloat16)
    vnew = torch.randn(B, Nkv, Dh, device=dev).to(torch.bfloat16)
    slot = (lens - 1).contiguous()
    ws = torch.empty(tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, tch.ATTN_BF16),
                     dtype=torch.uint8, device=dev)
    say(f"random decode with append {(i, B, Nq, Nkv, Dh, Tcap, window)}")
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    O1, L1 = torch.empty_like(q), torch.empty(B, Nq, device=dev)
    tch.attn_decode_append(q, knew, vnew, k1, v1, lens, slot, O1, L1, workspace=ws, window=window)
    tch.attn_kv_append(knew[:, :, None].contiguous(), vnew[:, :, None].contiguous(), k2, v2, slot)
    O2, L2 = torch.empty_like(q), torch.empty(B, Nq, device=dev)
    tch.attn_decode_window(q, k2, v2, lens, O2, L2, workspace=ws, window=window)
    torch.cuda.synchronize()
    assert _bits_equal(k1, k2) and _bits_equal(v1, v2), "cache rows"
    same_form = not (Dh == 256 and takes_even_split(B, Nq, Nkv, Dh, Tcap, window))
    assert _agree(O1, L1, O2, L2, same_form)


def _chunk_cases(n):
    out = []
    for i in range(n):
        Nkv, G, Dh = _pick([1, 2, 4, 8]), _pick([1, 2, 4, 8]), _pick([64, 128, 128, 256])
        B = int(_rng.integers(1, 5))
        Tcap = int(_rng.integers(16, 8193))
        while B * Nkv * Tcap * Dh > 16 * 2 ** 20:
            Tcap //= 2
        Tcap = max(Tcap, 16)
        Sq = int(_rng.integers(1, min(Tcap, 2048) + 1))
        window = int(_rng.integers(1, Tcap + 65)) if _rng.random() < 0.3 else 0
        out.append((i, B, Nkv * G, Nkv, Sq, Dh, Tcap, window, _pick(["implicit", "start", "explicit"]),
                    _pick(["pairs", "half"]), bool(_rng.random() < 0.3)))
    return out


@pytest.mark.parametrize("i,B,Nq,Nkv,Sq,Dh,Tcap,window,mode,style,pad", _chunk_cases(30))
def test_prefill_cache_rope_random(i, B, Nq, Nkv, Sq, Dh, Tcap, window, mode, style, pad):
    # a chunk of Sq queries at the end of lens[b] cached keys; the two-pass form
    # rotates the chunk at the positions the fused call uses (lens[b] - Sq + i
    # when none are given)
    dev = device()
    g = np.random.default_rng(2500 + i)
    torch.manual_seed(2500 + i)
    q = torch.randn(B, Nq, Sq, Dh, device=dev).to(torch.bfloat16)
    kc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(torch.bfloat16)
    vc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(torch.bfloat16)
    lens_np = g.integers(Sq, Tcap + 1, B).astype(np.int32)
    lens = torch.from_numpy(lens_np).to(dev)
    P = Tcap + 3000
    table = tch.rope_table(P, Dh, device=dev)
    pos = start = None
    if mode == "start":
        start_np = g.integers(0, P - Sq + 1, B).astype(np.int32)
        start = torch.from_numpy(start_np).to(dev)
        at = start_np[:, None] + np.arange(Sq, dtype=np.int32)[None, :]
    elif mode == "explicit":
        at = g.integers(0, P, (B, Sq)).astype(np.int32)
        pos = torch.from_numpy(at).to(dev)
    else:
        at = (lens_np - Sq)[:, None] + np.arange(Sq, dtype=np.int32)[None, :]
    bits = _key_bits(B, Tcap, g) if pad else None
    say(f"random fused chunk {(i, B, Nq, Nkv, Sq, Dh, Tcap, window, mode, style, pad)}")
    O1, L1 = torch.empty_like(q), torch.empty(B, Nq, Sq, device=dev)
    tch.attn_prefill_cache_rope(q, kc, vc, lens, O1, L1, table, key_bits=bits, positions=pos,
                                start=start, style=style, window=window)
    qr = tch.rope(q, table, positions=torch.from_numpy(np.ascontiguousarray(at)).to(dev), style=style)
    O2, L2 = torch.empty_like(q), torch.empty(B, Nq, Sq, device=dev)
    tch.attn_prefill_cache(qr, kc, vc, lens, O2, L2, window=window, key_bits=bits)
    torch.cuda.synchronize()
    assert _agree(O1, L1, O2, L2, True)


def _append_cases(n):
    out = []
    for i in range(n):
        B, Nkv, Dh = int(_rng.integers(1, 9)), _pick([1, 2, 4, 8]), _pick([40, 64, 80, 128, 256])
        Tcap = int(_rng.integers(16, 4097))
        rolling = bool(_rng.random() < 0.4)
        Snew = int(_rng.integers(1, 301)) if rolling else int(_rng.integers(1, min(300, Tcap) + 1))
        out.append((i, B, Nkv, Snew, Dh, Tcap, rolling, bool(_rng.random() < 0.5),
                    _pick(["pairs", "half"]), _pick(["bf16", "f32"])))
    return out


@pytest.mark.parametrize("i,B,Nkv,Snew,Dh,Tcap,rolling,explicit,style,dtype", _append_cases(30))
def test_kv_append_rope_random(i, B, Nkv, Snew, Dh, Tcap, rolling, explicit, style, dtype):
    dev = device()
    g = np.random.default_rng(3500 + i)
    torch.manual_seed(3500 + i)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    knew = torch.randn(B, Nkv, Snew, Dh, device=dev).to(dt)
    vnew = torch.randn(B, Nkv, Snew, Dh, device=dev).to(dt)
    kc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(dt)
    vc = torch.randn(B, Nkv, Tcap, Dh, device=dev).to(dt)
    hi = 3 * Tcap if rolling else Tcap - Snew
    pos_np = g.integers(0, hi + 1, B).astype(np.int32)
    P = int(pos_np.max()) + Snew + 500
    table = tch.rope_table(P, Dh, device=dev)
    at = g.integers(0, P, (B, Snew)).astype(np.int32) if explicit else \
        pos_np[:, None] + np.arange(Snew, dtype=np.int32)[None, :]
    pos = torch.from_numpy(pos_np).to(dev)
    say(f"random rotating append {(i, B, Nkv, Snew, Dh, Tcap, rolling, explicit, style, dtype)}")
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    tch.attn_kv_append_rope(knew, vnew, k1, v1, pos, table,
                            positions=torch.from_numpy(at).to(dev) if explicit else None,
                            rolling=int(rolling), style=style)
    kr = tch.rope(knew, table, positions=torch.from_numpy(np.ascontiguousarray(at)).to(dev), style=style)
    tch.attn_kv_append(kr, vnew, k2, v2, pos, rolling=int(rolling))
    torch.cuda.synchronize()
    assert _bits_equal(k1, k2) and _bits_equal(v1, v2)
