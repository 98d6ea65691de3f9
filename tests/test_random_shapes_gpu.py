"""GPU parity on seeded random shapes.

The hand-picked edge cases elsewhere pin the boundaries one at a time; these
cases draw the shape parameters together (batch, query and K/V heads, length,
head size, window, causal or not, bf16 or fp32; for chunked prefill the chunk
and the cached lengths; for decode the lengths, the capacity and the window)
from a fixed seed, so that combinations nobody listed are checked against the
float64 oracle on every element.  Head sizes 64 / 128 / 256 in bf16 run the
MFMA kernels; other head sizes and fp32 run the general row kernels.  The
backward cases use the backward tests' bound, and the key-padding cases the
padding tests' (rows that see no key must be exactly O = 0, LSE = -inf).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, run_prefill, say, stored_o_backward
from test_backward_gpu import _check as _check_grads, _grads, _inputs as _grad_inputs
from test_rope_padding_gpu import _split_dead

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)


def _pick(xs):
    return xs[int(_rng.integers(0, len(xs)))]


def _prefill_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4])
        G = _pick([1, 2, 3, 4, 8])
        B = int(_rng.integers(1, 3))
        S = int(_rng.integers(1, 700))
        dtype = "bf16" if _rng.random() < 0.75 else "f32"
        Dh = _pick([64, 128, 128, 256]) if (dtype == "bf16" and _rng.random() < 0.8) else \
            _pick([8, 40, 72, 96, 128, 136])
        causal = bool(_rng.random() < 0.8)
        window = int(_rng.integers(1, S + 65)) if (causal and _rng.random() < 0.4) else 0
        cases.append((i, B, Nkv * G, Nkv, S, Dh, dtype, causal, window))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,dtype,causal,window", _prefill_cases(60))
def test_random_prefill(i, B, Nq, Nkv, S, Dh, dtype, causal, window):
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=100 + i)
    scale = 1.0 / math.sqrt(Dh)
    O, L = run_prefill(q, k, v, dtype, causal, window, scale)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, dtype) for x in (q, k, v)),
                                  causal=causal, window=window, scale=scale)
    say(f"random prefill {i} {(B, Nq, Nkv, S, Dh, dtype, causal, window)}: "
        f"{check(O, L, Or, Lr, dtype, (i, B, Nq, Nkv, S, Dh, causal, window), storage_allowance=True)}")


def _chunk_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4])
        G = _pick([1, 2, 4, 8])
        B = int(_rng.integers(1, 4))
        Sq = int(_rng.integers(1, 300))
        Tcap = int(_rng.integers(Sq, Sq + 900))
        lens = [int(x) for x in _rng.integers(Sq, Tcap + 1, B)]
        Dh = _pick([64, 128, 256])
        window = int(_rng.integers(1, 400)) if _rng.random() < 0.4 else 0
        cases.append((i, B, Nkv * G, Nkv, Sq, Tcap, lens, Dh, window))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,Sq,Tcap,lens,Dh,window", _chunk_cases(32))
def test_random_chunked_prefill(i, B, Nq, Nkv, Sq, Tcap, lens, Dh, window):
    lens_a, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, Dh, Tcap, lens, "bf16", seed=300 + i)
    dev = device()
    tQ, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (Q, kc, vc))
    tl = torch.from_numpy(lens_a).to(dev)
    O, L = tch.prefill_cache(tQ, tk, tv, tl, window=window)
    torch.cuda.synchronize()
    O = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
    Or, Lr = oracle.chunk_ref(workloads.to_f64(Q, "bf16"), workloads.to_f64(kc, "bf16"),
                              workloads.to_f64(vc, "bf16"), lens_a, window=window)
    say(f"random chunk {i} {(B, Nq, Nkv, Sq, Tcap, lens, Dh, window)}: "
        f"{check(O, L.cpu().numpy().astype(np.float64), Or, Lr, 'bf16', (i, lens, window), storage_allowance=True)}")


def _decode_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4, 8])
        G = _pick([1, 2, 4, 8, 16, 32])
        B = int(_rng.integers(1, 9))
        Tcap = int(_rng.integers(1, 5000))
        lens = [int(x) for x in _rng.integers(1, Tcap + 1, B)]
        dtype = "bf16" if _rng.random() < 0.8 else "f32"
        Dh = _pick([64, 128, 256]) if dtype == "bf16" else _pick([32, 64, 128])
        window = int(_rng.integers(1, Tcap + 100)) if _rng.random() < 0.35 else 0
        cases.append((i, B, Nkv * G, Nkv, Tcap, lens, Dh, dtype, window))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,Tcap,lens,Dh,dtype,window", _decode_cases(40))
def test_random_decode(i, B, Nq, Nkv, Tcap, lens, Dh, dtype, window):
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, dtype, seed=500 + i,
                                                lens=lens)
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, dtype, dev) for x in (q, kc, vc))
    tl = torch.from_numpy(lens_a).to(dev)
    O, L = tch.decode(tq, tk, tv, tl, window=window)
    torch.cuda.synchronize()
    O = workloads.to_f64(workloads.from_torch(O, dtype), dtype)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, dtype), workloads.to_f64(kc, dtype),
                               workloads.to_f64(vc, dtype), lens_a, window=window)
    say(f"random decode {i} {(B, Nq, Nkv, Tcap, Dh, dtype, window)}: "
        f"{check(O, L.cpu().numpy().astype(np.float64), Or, Lr, dtype, (i, lens, window), storage_allowance=True)}")


def _backward_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4])
        G = _pick([1, 2, 4])
        B = int(_rng.integers(1, 3))
        S = int(_rng.integers(1, 400))
        dtype = "bf16" if _rng.random() < 0.75 else "f32"
        Dh = _pick([64, 128]) if (dtype == "bf16" and _rng.random() < 0.8) else _pick([16, 48, 80, 128])
        causal = bool(_rng.random() < 0.8)
        window = int(_rng.integers(1, S + 65)) if (causal and _rng.random() < 0.4) else 0
        cases.append((i, B, Nkv * G, Nkv, S, Dh, dtype, causal, window))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,dtype,causal,window", _backward_cases(16))
def test_random_backward(i, B, Nq, Nkv, S, Dh, dtype, causal, window):
    q, k, v, dO = _grad_inputs(B, Nq, Nkv, S, Dh, dtype, seed=700 + i)
    if dtype == "bf16":
        # the backward is given the oracle's O (stored in bf16) and LSE, and
        # held to the oracle's gradients for that stored O
        O_st, LSE, *ref = stored_o_backward(*(workloads.to_f64(x, dtype) for x in (q, k, v, dO)),
                                            causal=causal, window=window)
        got = _grads(q, k, v, dO, dtype, causal, window, given=(O_st, LSE))
    else:
        got = _grads(q, k, v, dO, dtype, causal, window)
        ref = oracle.backward_ref(*(workloads.to_f64(x, dtype) for x in (q, k, v, dO)),
                                  causal=causal, window=window)
    _check_grads(got, ref, dtype, (i, B, Nq, Nkv, S, Dh, causal, window))


def _padded_cases(n, decode):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4])
        G = _pick([1, 2, 4, 8])
        B = int(_rng.integers(1, 4))
        T = int(_rng.integers(2, 3000 if decode else 600))
        Dh = _pick([64, 128, 256])
        pads = [int(x) for x in _rng.integers(0, T, B)] if _rng.random() < 0.6 else None
        holes = float(_pick([0.0, 0.1, 0.5]))
        window = int(_rng.integers(1, T + 50)) if _rng.random() < 0.3 else 0
        lens = [int(x) for x in _rng.integers(1, T + 1, B)] if decode else None
        cases.append((i, B, Nkv * G, Nkv, T, Dh, pads, holes, window, lens))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,pads,holes,window,lens", _padded_cases(14, False))
def test_random_prefill_padded(i, B, Nq, Nkv, S, Dh, pads, holes, window, lens):
    dev = device()
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=900 + i)
    m = workloads.key_mask(B, S, pads=pads, hole_frac=holes, seed=900 + i)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    O, L = tch.prefill(tq, tk, tv, window=window, key_mask=torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
    Lg = L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(a, "bf16") for a in (q, k, v)),
                                  window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "prefill")
    errs = "no row sees a key" if not live.any() else check(
        Og[live], Lg[live], Or[live], Lr[live], "bf16", (i, S, Dh, pads, holes, window),
        storage_allowance=True)
    say(f"random padded prefill {i} S={S} Dh={Dh} dead rows {n_dead}: {errs}")


@pytest.mark.parametrize("i,B,Nq,Nkv,Tcap,Dh,pads,holes,window,lens", _padded_cases(14, True))
def test_random_decode_padded(i, B, Nq, Nkv, Tcap, Dh, pads, holes, window, lens):
    dev = device()
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, "bf16",
                                                seed=1100 + i, lens=lens)
    m = workloads.key_mask(B, Tcap, pads=pads, hole_frac=holes, seed=1100 + i)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    O, L = tch.decode(tq, tk, tv, torch.from_numpy(lens_a).to(dev), window=window,
                      key_mask=torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
    Lg = L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), workloads.to_f64(kc, "bf16"),
                               workloads.to_f64(vc, "bf16"), lens_a, window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "decode")
    errs = "no row sees a key" if not live.any() else check(
        Og[live], Lg[live], Or[live], Lr[live], "bf16", (i, Tcap, pads, holes, window),
        storage_allowance=True)
    say(f"random padded decode {i} Tcap={Tcap} Dh={Dh} dead rows {n_dead}: {errs}")
