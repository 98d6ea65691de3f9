"""RoPE fused into the attention calls: attn_prefill_rope, attn_prefill_cache_rope
and attn_decode_rope rotate the queries as they load them.

Each fused call must give the same bits as the two passes it replaces (attn_rope
on q, then the unrotated call on the rotated q), since the kernels compute the
rotation with the same fp32 arithmetic and the same single rounding, where both
take the same launch form (at head size 256 an unrotated decode large enough
for the even split takes it, while the rotating decode keeps chunk mode, whose
accumulation order differs; no case here is of that kind); and it
must match the oracle (oracle.rope_ref on q and k, rounded to the stored type,
then the attention oracle) at the stated tolerance.  Keys are rotated before
the call, by attn_rope or by the rotating cache append, as the page's layer
cache stores them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say, takes_even_split

pytestmark = pytest.mark.gpu


def _round(x, dtype):
    # float64 -> the stored element type -> float64 (nearest even)
    if dtype == "bf16":
        return workloads.to_f64(workloads.f32_to_bf16_bits(x.astype(np.float32)), "bf16")
    return x.astype(np.float32).astype(np.float64)


def _positions(mode, B, S, P, base_fn, seed):
    """(positions [B, S] numpy or None, start [B] numpy or None, the positions used)."""
    rng = np.random.default_rng(seed)
    if mode == "explicit":
        pos = rng.integers(0, P, (B, S)).astype(np.int32)
        return pos, None, pos
    if mode == "start":
        start = rng.integers(0, P - S, B).astype(np.int32)
        return None, start, start[:, None] + np.arange(S)[None, :]
    return None, None, base_fn()


def _t(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("dtype,B,Nq,Nkv,S,Dh,causal,window,style,mode", [
    ("bf16", 2, 16, 4, 700, 128, True, 0, "pairs", "implicit"),
    ("bf16", 2, 16, 4, 700, 128, True, 0, "half", "explicit"),
    ("bf16", 1, 8, 8, 333, 128, True, 100, "half", "start"),
    ("bf16", 1, 8, 2, 300, 128, False, 0, "pairs", "start"),
    ("bf16", 1, 16, 16, 4096, 128, True, 0, "half", "implicit"),   # key-split form
    ("bf16", 1, 32, 32, 8192, 128, True, 0, "pairs", "explicit"),  # four rounds, drawn tail
    ("bf16", 2, 32, 8, 4096, 128, True, 1000, "half", "start"),    # GQA window, four rounds
    ("bf16", 2, 8, 8, 257, 64, True, 0, "pairs", "explicit"),
    ("bf16", 1, 8, 4, 300, 256, True, 0, "half", "implicit"),
    ("bf16", 1, 4, 2, 130, 80, True, 0, "half", "explicit"),       # general kernel
    ("f32", 1, 4, 2, 150, 64, True, 0, "pairs", "implicit"),
    ("f32", 1, 4, 4, 90, 48, True, 20, "half", "start"),
])
def test_prefill_rope(dtype, B, Nq, Nkv, S, Dh, causal, window, style, mode):
    dev = device()
    P = S + 500
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=S + Dh)
    tq, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (q, k, v))
    table = tch.rope_table(P, Dh, device=dev)
    pos, start, used = _positions(mode, B, S, P, lambda: np.tile(np.arange(S), (B, 1)), seed=Dh)
    tpos, tstart = _t(pos, dev), _t(start, dev)
    tkr = torch.empty_like(tk)
    tch.attn_rope(tk, tkr, table, positions=tpos, start=tstart, style=style)
    O1 = torch.empty_like(tq)
    L1 = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
    tch.attn_prefill_rope(tq, tkr, tv, O1, L1, table, positions=tpos, start=tstart, style=style,
                          causal=int(causal), window=window)
    # the two passes it replaces
    tqr = torch.empty_like(tq)
    tch.attn_rope(tq, tqr, table, positions=tpos, start=tstart, style=style)
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    tch.attn_prefill(tqr, tkr, tv, O2, L2, causal=int(causal), window=window)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(O1.view(bits), O2.view(bits)) and torch.equal(L1, L2)
    qf, kf, vf = (workloads.to_f64(a, dtype) for a in (q, k, v))
    qr = _round(oracle.rope_ref(qf, used, style=style), dtype)
    kr = _round(oracle.rope_ref(kf, used, style=style), dtype)
    if S > 1024:   # sampled rows of the long case
        rows = workloads.sample_rows(B, Nq, S, 64, seed=3, forced_rows=(0, S // 2, S - 1))
        Or, Lr = oracle.attention_rows_ref(qr, kr, vf, rows, causal=causal, window=window)
        Og = workloads.to_f64(workloads.from_torch(O1, dtype), dtype)
        Lg = L1.cpu().numpy().astype(np.float64)
        got = (np.stack([Og[b, h, i] for b, h, i in rows]), np.array([Lg[b, h, i] for b, h, i in rows]))
    else:
        Or, Lr = oracle.attention_ref(qr, kr, vf, causal=causal, window=window)
        got = (workloads.to_f64(workloads.from_torch(O1, dtype), dtype),
               L1.cpu().numpy().astype(np.float64))
    say(f"prefill_rope {dtype} Dh={Dh} {style} {mode}: "
        f"{check(*got, Or, Lr, dtype, (Dh, style, mode), storage_allowance=True)}")


@pytest.mark.parametrize("dtype,B,Nq,Nkv,Sq,Dh,Tcap,lens,window,style,mode", [
    ("bf16", 3, 16, 4, 100, 128, 900, [900, 300, 100], 0, "half", "implicit"),
    ("bf16", 2, 8, 8, 64, 128, 700, [700, 64], 128, "pairs", "explicit"),
    ("bf16", 2, 8, 2, 40, 64, 500, [500, 41], 0, "pairs", "start"),
    ("f32", 2, 4, 2, 20, 64, 200, [200, 20], 0, "half", "implicit"),
])
def test_prefill_cache_rope(dtype, B, Nq, Nkv, Sq, Dh, Tcap, lens, window, style, mode):
    dev = device()
    P = Tcap + 300
    lens_a, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, Dh, Tcap, lens, dtype, seed=Sq)
    tQ, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (Q, kc, vc))
    table = tch.rope_table(P, Dh, device=dev)
    # the cached keys are rotated at their cache positions 0 .. lens-1
    tkr = torch.empty_like(tk)
    tch.attn_rope(tk, tkr, table, style=style)
    pos, start, used = _positions(mode, B, Sq, P,
                                  lambda: lens_a[:, None] - Sq + np.arange(Sq)[None, :], seed=Sq)
    tpos, tstart = _t(pos, dev), _t(start, dev)
    tl = _t(lens_a, dev)
    O1 = torch.empty_like(tQ)
    L1 = torch.empty((B, Nq, Sq), dtype=torch.float32, device=dev)
    tch.attn_prefill_cache_rope(tQ, tkr, tv, tl, O1, L1, table, positions=tpos, start=tstart,
                                style=style, window=window)
    tQr = torch.empty_like(tQ)   # the two passes: the chunk rows at the positions used
    tch.attn_rope(tQ, tQr, table, positions=_t(used.astype(np.int32), dev), style=style)
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    tch.attn_prefill_cache(tQr, tkr, tv, tl, O2, L2, window=window)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(O1.view(bits), O2.view(bits)) and torch.equal(L1, L2)
    Qf, kf, vf = (workloads.to_f64(a, dtype) for a in (Q, kc, vc))
    Qr = _round(oracle.rope_ref(Qf, used, style=style), dtype)
    kr = _round(oracle.rope_ref(np.nan_to_num(kf), np.arange(Tcap), style=style), dtype)
    Or, Lr = oracle.chunk_ref(Qr, kr, vf, lens_a, window=window)
    say(f"prefill_cache_rope {dtype} Dh={Dh} {style} {mode}: "
        f"{check(workloads.to_f64(workloads.from_torch(O1, dtype), dtype), L1.cpu().numpy().astype(np.float64), Or, Lr, dtype, (Dh, style, mode), storage_allowance=True)}")


@pytest.mark.parametrize("dtype,B,Nq,Nkv,Dh,Tcap,lens,window,style,explicit,padded", [
    ("bf16", 4, 32, 8, 128, 3000, [3000, 1, 1500, 2001], 0, "half", False, False),
    ("bf16", 3, 32, 1, 128, 2100, [2100, 640, 1025], 0, "pairs", True, False),   # MQA
    ("bf16", 2, 16, 2, 64, 1500, [1500, 700], 300, "pairs", False, False),
    ("bf16", 2, 8, 2, 256, 1200, [1200, 333], 0, "half", True, False),
    ("bf16", 3, 16, 4, 128, 2000, [2000, 1000, 37], 0, "half", False, True),     # key mask
    ("bf16", 64, 32, 8, 128, 2048, None, 0, "pairs", True, True),   # key mask, even split
    ("bf16", 64, 32, 8, 128, 2048, None, 0, "half", False, False),  # even split
    ("bf16", 32, 32, 1, 128, 4096, None, 0, "pairs", True, False),  # MQA, even split
    ("f32", 2, 8, 2, 64, 400, [400, 17], 0, "half", True, False),                 # general
])
def test_decode_rope(dtype, B, Nq, Nkv, Dh, Tcap, lens, window, style, explicit, padded):
    dev = device()
    P = Tcap + 100
    if B >= 32:
        assert takes_even_split(B, Nq, Nkv, Dh, Tcap, window)
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, dtype, seed=Dh + B,
                                                lens=lens)
    tq, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (q, kc, vc))
    table = tch.rope_table(P, Dh, device=dev)
    tkr = torch.empty_like(tk)
    tch.attn_rope(tk, tkr, table, style=style)   # cached key at row j sits at position j
    rng = np.random.default_rng(Dh)
    qpos = rng.integers(0, P, B).astype(np.int32) if explicit else lens_a - 1
    tpos = _t(qpos.astype(np.int32), dev) if explicit else None
    tl = _t(lens_a, dev)
    mask = workloads.key_mask(B, Tcap, hole_frac=0.1, seed=5) if padded else None
    bits_t = tch.pack_key_mask(_t(mask, dev)) if padded else None
    ws = torch.empty(max(1, tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window,
                                                                   tch._dtype_code(tq))),
                     dtype=torch.uint8, device=dev)
    O1 = torch.empty_like(tq)
    L1 = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    tch.attn_decode_rope(tq, tkr, tv, tl, O1, L1, table, workspace=ws, key_bits=bits_t,
                         positions=tpos, style=style, window=window)
    tqr = torch.empty_like(tq)
    tch.attn_rope(tq[:, :, None].contiguous(), tqr[:, :, None], table,
                  positions=_t(qpos[:, None].astype(np.int32), dev), style=style)
    O2, L2 = torch.empty_like(O1), torch.empty_like(L1)
    if padded:
        tch.attn_decode_padded(tqr, tkr, tv, tl, bits_t, O2, L2, ws, window=window)
    else:
        tch.attn_decode_window(tqr, tkr, tv, tl, O2, L2, ws, window=window)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(O1.view(bits), O2.view(bits)) and torch.equal(L1, L2)
    qf, kf, vf = (workloads.to_f64(a, dtype) for a in (q, kc, vc))
    qr = _round(oracle.rope_ref(qf[:, :, None], qpos[:, None], style=style), dtype)[:, :, 0]
    kr = _round(oracle.rope_ref(np.nan_to_num(kf), np.arange(Tcap), style=style), dtype)
    if padded:
        Or, Lr = oracle.decode_ref(qr, kr, vf, lens_a, window=window, key_mask=mask)
    else:
        Or, Lr = oracle.decode_ref(qr, kr, vf, lens_a, window=window)
    say(f"decode_rope {dtype} Dh={Dh} {style} explicit={explicit} padded={padded}: "
        f"{check(workloads.to_f64(workloads.from_torch(O1, dtype), dtype), L1.cpu().numpy().astype(np.float64), Or, Lr, dtype, (Dh, style), storage_allowance=True)}")


@pytest.mark.parametrize("style", ["pairs", "half"])
def test_left_padded_generation_fused(style):
    # three prompts of 50, 120 and 200 tokens left-padded to 200, then 16 tokens
    # generated one at a time; positions count from each prompt's first token.
    # The queries are rotated inside the attention calls only.  Every row of a
    # real token must match the oracle run on that sequence alone.
    dev = device()
    Nq, Nkv, Dh, P0, steps = 32, 8, 128, 200, 16
    real = [50, 120, 200]
    B, T = len(real), P0 + steps
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, T, Dh, "bf16", seed=97)
    mask = np.zeros((B, T), bool)
    for b, n in enumerate(real):
        mask[b, P0 - n:] = True
    pos = workloads.token_positions(mask)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    tpos = torch.from_numpy(pos).to(dev)
    bits = tch.pack_key_mask(torch.from_numpy(mask).to(dev))
    table = tch.rope_table(T, Dh, device=dev)
    Kc = torch.zeros((B, Nkv, T, Dh), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    tch.attn_kv_append_rope(tk[:, :, :P0].contiguous(), tv[:, :, :P0].contiguous(), Kc, Vc, zero,
                            table, positions=tpos[:, :P0].contiguous(), style=style)
    Op = torch.empty((B, Nq, P0, Dh), dtype=torch.bfloat16, device=dev)
    Lp = torch.empty((B, Nq, P0), dtype=torch.float32, device=dev)
    tch.attn_prefill_cache_rope(tq[:, :, :P0].contiguous(), Kc, Vc,
                                torch.full((B,), P0, dtype=torch.int32, device=dev), Op, Lp, table,
                                key_bits=bits, positions=tpos[:, :P0].contiguous(), style=style)
    outs, lses = [Op], [Lp]
    ws = torch.empty(tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, T, tch.ATTN_BF16),
                     dtype=torch.uint8, device=dev)
    for t in range(P0, T):
        at = torch.full((B,), t, dtype=torch.int32, device=dev)
        tch.attn_kv_append_rope(tk[:, :, t:t + 1].contiguous(), tv[:, :, t:t + 1].contiguous(), Kc,
                                Vc, at, table, positions=tpos[:, t:t + 1].contiguous(), style=style)
        O = torch.empty((B, Nq, Dh), dtype=torch.bfloat16, device=dev)
        L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
        tch.attn_decode_rope(tq[:, :, t].contiguous(), Kc, Vc, at + 1, O, L, table, workspace=ws,
                             key_bits=bits, positions=tpos[:, t].contiguous(), style=style)
        outs.append(O[:, :, None])
        lses.append(L[:, :, None])
    torch.cuda.synchronize()
    Og = workloads.to_f64(workloads.from_torch(torch.cat(outs, dim=2), "bf16"), "bf16")
    Lg = torch.cat(lses, dim=2).cpu().numpy().astype(np.float64)
    qf, kf, vf = (workloads.to_f64(a, "bf16") for a in (q, k, v))
    for b, n in enumerate(real):
        r = P0 - n
        own = np.arange(T - r)[None, :]
        qb = _round(oracle.rope_ref(qf[b:b + 1, :, r:], own, style=style), "bf16")
        kb = _round(oracle.rope_ref(kf[b:b + 1, :, r:], own, style=style), "bf16")
        Or, Lr = oracle.attention_ref(qb, kb, vf[b:b + 1, :, r:])
        errs = check(Og[b:b + 1, :, r:], Lg[b:b + 1, :, r:], Or, Lr, "bf16", (style, b),
                     storage_allowance=True)
        assert np.all(Og[b, :, :r] == 0) and np.all(np.isneginf(Lg[b, :, :r]))
        say(f"fused padded generation {style} prompt {n}: {errs}")
