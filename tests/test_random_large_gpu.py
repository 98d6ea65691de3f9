"""GPU parity on seeded random shapes large enough for the multi-round paths.

test_random_shapes_gpu.py draws small shapes, whose grids fit the chip once.
These cases draw shapes whose prefill grids run several rounds (the 8-wave
forms, the run-time drawn tail, ragged last tiles, key-padding masks) and
decode batches large enough for the even split (with masks and windows), from a
fixed seed, and backward passes of 1000-9000 tokens (several key blocks and
query tiles per head, windows, key padding).  The prefill is checked on seeded
sampled rows (plus forced rows at the ends and at tile boundaries) against the
oracle's single-row attention, the decode on every row (rows that see no key
must be exactly O = 0, LSE = -inf), the backward on sampled gradient rows.
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, grad_rows_ratio, say, set_oracle_rows
from test_backward_gpu import BF16_REL
from test_rope_padding_gpu import _split_dead

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)


def _pick(xs):
    return xs[int(_rng.integers(0, len(xs)))]


class _Lazy:
    def __init__(self, arr):
        self.arr, self.shape = arr, arr.shape

    def __getitem__(self, idx):
        return workloads.to_f64(self.arr[idx], "bf16")


def _prefill_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4, 8])
        G = _pick([1, 2, 4, 8])
        Dh = _pick([64, 128, 128, 256])
        B = int(_rng.integers(1, 5))
        S = int(_rng.integers(700, 8001))
        while B * Nkv * G * S * Dh > 48 * 2 ** 20:
            S //= 2
        S = max(S, 65)
        causal = bool(_rng.random() < 0.8)
        window = int(_rng.integers(1, S + 65)) if (causal and _rng.random() < 0.35) else 0
        pad = causal and bool(_rng.random() < 0.25)
        cases.append((i, B, Nkv * G, Nkv, S, Dh, causal, window, pad))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,causal,window,pad", _prefill_cases(24))
def test_large_prefill(i, B, Nq, Nkv, S, Dh, causal, window, pad):
    dev = device()
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=900 + i)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    rows = workloads.sample_rows(B, Nq, S, 48, seed=i,
                                 forced_rows=(0, S - 1, S // 2, min(S - 1, 64), min(S - 1, 255)))
    m = None
    if pad:
        pads = [int(x) for x in np.random.default_rng(i).integers(0, S, B)]
        m = workloads.key_mask(B, S, pads=pads, hole_frac=0.1, seed=i)
        O, L = tch.prefill(tq, tk, tv, causal=causal, window=window,
                           key_mask=torch.from_numpy(m).to(dev))
    else:
        O, L = tch.prefill(tq, tk, tv, causal=causal, window=window)
    torch.cuda.synchronize()
    idx = tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    Og = workloads.to_f64(workloads.from_torch(O[idx], "bf16"), "bf16")
    Lg = L[idx].cpu().numpy().astype(np.float64)
    del tq, tk, tv, O, L
    what = (i, B, Nq, Nkv, S, Dh, causal, window, pad)
    if pad:
        # a padded prefill is a chunk of S queries against its own S keys
        Or, Lr = oracle.chunk_ref(_Lazy(q), _Lazy(k), _Lazy(v), [S] * B, rows=rows, key_mask=m,
                                  window=window)
        live, n_dead = _split_dead(Og, Lg, Or, Lr, "large padded prefill")
        errs = check(Og[live], Lg[live], Or[live], Lr[live], "bf16", what, storage_allowance=True)
        say(f"large padded prefill {what}: {errs}, {n_dead} rows without keys")
    else:
        Or, Lr = oracle.attention_rows_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)), rows,
                                           causal=causal, window=window)
        say(f"large prefill {what}: {check(Og, Lg, Or, Lr, 'bf16', what, storage_allowance=True)}")


def _decode_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4, 8])
        G = _pick([1, 2, 4, 8, 16, 32])
        Dh = _pick([64, 128, 128, 256])
        if Dh == 256 and G > 16:
            G = 16
        B = int(_rng.integers(4, 65))
        Tcap = int(_rng.integers(1000, 12001))
        while B * Nkv * Tcap * Dh > 64 * 2 ** 20:
            Tcap //= 2
        window = int(_rng.integers(1, Tcap)) if _rng.random() < 0.3 else 0
        pad = bool(_rng.random() < 0.3)
        cases.append((i, B, Nkv * G, Nkv, Dh, Tcap, window, pad))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,Dh,Tcap,window,pad", _decode_cases(16))
def test_large_decode(i, B, Nq, Nkv, Dh, Tcap, window, pad):
    dev = device()
    lens, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, "bf16", seed=1300 + i)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    m = None
    if pad:
        pads = [int(x) for x in np.random.default_rng(i).integers(0, Tcap // 2, B)]
        m = workloads.key_mask(B, Tcap, pads=pads, hole_frac=0.2, seed=i)
    O, L = tch.decode(tq, tk, tv, torch.from_numpy(lens).to(dev), window=window,
                      key_mask=torch.from_numpy(m).to(dev) if pad else None)
    torch.cuda.synchronize()
    Og = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
    Lg = L.cpu().numpy().astype(np.float64)
    del tq, tk, tv, O, L
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), _Lazy(kc), _Lazy(vc), lens,
                               window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "large decode")
    what = (i, B, Nq, Nkv, Dh, Tcap, window, pad)
    errs = check(Og[live], Lg[live], Or[live], Lr[live], "bf16", what, storage_allowance=True)
    say(f"large decode {what}: {errs}, {n_dead} rows without keys")


def _backward_cases(n):
    cases = []
    for i in range(n):
        Nkv = _pick([1, 2, 4, 8])
        G = _pick([1, 2, 4])
        Dh = _pick([64, 128, 128, 256])
        B = int(_rng.integers(1, 3))
        S = int(_rng.integers(1000, 9000))
        while B * Nkv * G * S * Dh > 40 * 2 ** 20:
            S //= 2
        causal = bool(_rng.random() < 0.85)
        window = int(_rng.integers(1, S + 65)) if (causal and _rng.random() < 0.3) else 0
        pad = bool(_rng.random() < 0.25)
        cases.append((i, B, Nkv * G, Nkv, S, Dh, causal, window, pad))
    return cases


@pytest.mark.parametrize("i,B,Nq,Nkv,S,Dh,causal,window,pad", _backward_cases(12))
def test_large_backward(i, B, Nq, Nkv, S, Dh, causal, window, pad):
    # sampled dQ rows (plus rows 0, S/2 and S-1) and the dK / dV rows of keys
    # near the end (each seen by few queries) or, without a plain causal mask,
    # anywhere; each row held to the backward's bound against its own scale,
    # as the full-size backward test does.  The sampled query rows take the
    # oracle's O and LSE before the backward, so their dQ is fixed by oracle
    # values (with O as stored in bf16).
    dev = device()
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=3000 + i)
    dO = workloads.draw((B, Nq, S, Dh), "bf16", 3000 + i, 3)
    tq, tk, tv, tdo = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v, dO))
    m, km = None, None
    if pad:
        pads = [int(x) for x in np.random.default_rng(i).integers(0, S // 2, B)]
        m = workloads.key_mask(B, S, pads=pads, hole_frac=0.1, seed=i)
        km = torch.from_numpy(m).to(dev)
    O, L = tch.prefill(tq, tk, tv, causal=causal, window=window, key_mask=km)
    qr = workloads.sample_rows(B, Nq, S, 12, seed=i, forced_rows=(0, S - 1, S // 2))
    shift = set_oracle_rows(O, L, _Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr, causal=causal,
                            window=window, key_mask=m)
    dQ, dK, dV = tch.backward(tq, tk, tv, O, L, tdo, causal=causal, window=window, key_mask=km)
    torch.cuda.synchronize()
    rng = np.random.default_rng(i + 7)
    kr = [(int(rng.integers(0, B)), int(rng.integers(0, Nkv)), j) for j in (S - 1, S - 33, S - 100, S - 129)]
    if not causal or window:
        kr.append((0, 0, int(rng.integers(0, S))))
    idx = lambda rows: tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    got = [workloads.to_f64(workloads.from_torch(t[idx(r)], "bf16"), "bf16")
           for t, r in ((dQ, qr), (dK, kr), (dV, kr))]
    del tq, tk, tv, tdo, O, L, dQ, dK, dV
    ref = oracle.backward_rows_ref(_Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr, kr, causal=causal,
                                   window=window, key_mask=m)
    ref = (ref[0] + shift, ref[1], ref[2])
    what = (i, B, Nq, Nkv, S, Dh, causal, window, pad)
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        ratio = grad_rows_ratio(g, r)
        assert np.all(ratio <= BF16_REL), f"{what} {name}: worst row-relative error {ratio.max():.3g}"
        out.append(f"{name} {ratio.max():.2e}")
    say(f"large backward {what}, row-relative: " + " ".join(out))
