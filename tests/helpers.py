"""Shared helpers of the GPU parity tests: run the library on seeded inputs
and compare with the float64 oracle on the same stored values."""

import math

import numpy as np
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads

# tolerances: fp32 max abs 1e-5 on O and LSE; bf16 max abs 1e-2 and mean abs
# 1e-3 on O, max abs 1e-3 on LSE
F32_TOL = 1e-5
BF16_MAX, BF16_MEAN, BF16_LSE = 1e-2, 1e-3, 1e-3


def half_ulp_bf16(x):
    """Half a bf16 unit in the last place at |x| (the storage rounding of O)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(int) - 8)


def check(O_gpu, LSE_gpu, O_ref, LSE_ref, dtype, what, storage_allowance=False):
    """Element-wise comparison at the stated tolerance; returns the errors.

    storage_allowance: small edge-case shapes can produce |O| >= 4 in rows
    with few keys, where rounding the exact value to bf16 alone may exceed
    1e-2; such tests allow 1e-2 plus that half ulp per element.
    """
    err = np.abs(O_gpu - O_ref)
    lerr = np.abs(LSE_gpu - LSE_ref) if LSE_gpu is not None else np.zeros(1)
    assert np.all(np.isfinite(O_gpu)), f"{what}: non-finite output"
    if dtype == "f32":
        assert err.max() <= F32_TOL, f"{what}: O max err {err.max():.3g}"
        assert lerr.max() <= F32_TOL, f"{what}: LSE max err {lerr.max():.3g}"
    else:
        bound = BF16_MAX + (half_ulp_bf16(O_ref) if storage_allowance else 0.0)
        worst = np.argmax(err - bound)
        assert np.all(err <= bound), (
            f"{what}: O err {err.flat[worst]:.4g} at {np.unravel_index(worst, err.shape)}")
        assert err.mean() <= BF16_MEAN, f"{what}: O mean err {err.mean():.3g}"
        assert lerr.max() <= BF16_LSE, f"{what}: LSE max err {lerr.max():.3g}"
    return float(err.max()), float(err.mean()), float(lerr.max())


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def run_prefill(q, k, v, dtype, causal, window, scale):
    """Stored inputs -> (O as float64 numpy, LSE numpy) from the library."""
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, dtype, dev) for x in (q, k, v))
    O = torch.empty_like(tq)
    LSE = torch.empty(tq.shape[:3], dtype=torch.float32, device=dev)
    tch.attn_prefill(tq, tk, tv, O, LSE, causal=int(causal), window=window,
                     scale=scale if scale is not None else 1.0 / math.sqrt(q.shape[-1]))
    torch.cuda.synchronize()
    return workloads.to_f64(workloads.from_torch(O, dtype), dtype), LSE.cpu().numpy().astype(np.float64)


def run_decode(q, kc, vc, lens, dtype):
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, dtype, dev) for x in (q, kc, vc))
    tl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev)
    O, LSE = tch.decode(tq, tk, tv, tl)
    torch.cuda.synchronize()
    return workloads.to_f64(workloads.from_torch(O, dtype), dtype), LSE.cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)


def takes_even_split(B, Nq, Nkv, Dh, Tcap, window):
    # Whether a bf16 decode of this shape takes the even split.  Its workspace
    # ends in two int32 per (sequence, K/V head) after the fp32 partials of
    # G (Dh + 2) floats per slot; the chunked form has the partials only.  With
    # a key mask the library also needs every wavefront's range to fit the 1024
    # flag words it stages (at most B*Nkv*(L/32+1)*64/C(W) + 3 steps), which is
    # checked here for every shape.
    G = Nq // Nkv
    ws = tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, tch.ATTN_BF16)
    per_slot = G * (Dh + 2) * 4
    ev = (ws - B * Nkv * 8) % per_slot == 0 and ws % per_slot != 0
    L = window if 0 < window < Tcap else Tcap
    W = 512 if G >= 16 else 1024
    cw = 64 * ((W + 1) // 2) + 55 * (W // 2)
    return ev and B * Nkv * ((L + 31) // 32 + 1) * 64 // cw + 3 <= 1022


def set_oracle_rows(O, LSE, Q, K, V, dO, q_rows, causal=True, window=0, key_mask=None):
    """Give the sampled query rows the oracle's forward output before a backward.

    A row's dQ depends on its own O and LSE (and on K, V): the backward forms
    P_i from LSE_i and Delta_i = rowsum(dO_i * O_i) from O_i as stored.  This
    writes the oracle's O_i (rounded to bf16 from fp32, as the forward stores
    it) and LSE_i into the device tensors O, LSE, so that those rows' gradient
    is fixed by oracle values alone.  It returns, per row, what that rounding
    of O does to the oracle's dQ_i: Delta_i moves by
    dDelta_i = dO_i . (bf16(O_i) - O_i), every dS_ij = P_ij (dP_ij - Delta_i)
    by -P_ij dDelta_i, so dQ_i = scale * sum_j dS_ij K_j moves by
    -scale * dDelta_i * sum_j P_ij K_j.  In a row whose weight sits mostly on
    one key the gradient is small while Delta is not; at head size 256 that
    shift reaches 3 % of such a row's largest element.  Q, K, V, dO may be
    lazily widened arrays.  Returns [len(q_rows), Dh], to add to the oracle's
    dQ rows.
    """
    Nq, Dh = Q.shape[1], Q.shape[3]
    Nkv = K.shape[1]
    scale = 1.0 / math.sqrt(Dh)
    heads = {}
    shift = np.empty((len(q_rows), Dh))
    o_rows = np.empty((len(q_rows), Dh), dtype=np.float32)
    lse_rows = np.empty(len(q_rows), dtype=np.float32)
    for t, (b, h, i) in enumerate(q_rows):
        g = oracle.kv_head_of(h, Nq, Nkv)
        if (b, g) not in heads:
            heads[(b, g)] = (np.asarray(K[b, g], dtype=np.float64), np.asarray(V[b, g], dtype=np.float64))
        Kb, Vb = heads[(b, g)]
        o, lse, P = oracle.head_attention(np.asarray(Q[b, h, i], dtype=np.float64)[None, :], [i], Kb, Vb,
                                          causal, window, scale, return_probs=True,
                                          key_ok=None if key_mask is None else key_mask[b])
        o_rows[t], lse_rows[t] = o[0], lse[0]
        o_stored = workloads.to_f64(workloads.f32_to_bf16_bits(o_rows[t]), "bf16")
        d_delta = np.dot(np.asarray(dO[b, h, i], dtype=np.float64), o_stored - o[0])
        shift[t] = -scale * d_delta * (P[0] @ Kb)
    idx = tuple(torch.tensor(c, device=O.device) for c in zip(*q_rows))
    O[idx] = torch.from_numpy(o_rows).to(O.device).to(O.dtype)
    LSE[idx] = torch.from_numpy(lse_rows).to(LSE.device)
    return shift


def grad_rows_ratio(g, r):
    """Row-relative error of sampled gradient rows: |g - r| over the row's
    largest |r|, floored at 1 % of the largest sampled element (and 1 for rows
    whose exact gradient is 0)."""
    scale_row = np.maximum(np.abs(r).max(axis=1, keepdims=True), 1e-2 * np.abs(r).max())
    scale_row = np.where(scale_row > 0, scale_row, 1.0)
    return np.abs(g - r) / scale_row


def stored_o_backward(Q, K, V, dO, causal=True, window=0, scale=None):
    """The oracle's forward and backward with O as the forward stores it.

    The backward takes O and LSE as inputs and forms Delta = rowsum(dO * O)
    from the O it is given.  Returns O rounded to bf16 (from fp32, as the
    forward rounds it), the exact LSE, and the oracle's dQ, dK, dV shifted to
    that stored O: with dDelta_i = dO_i . (bf16(O_i) - O_i), every
    dS_ij = P_ij (dP_ij - Delta_i) moves by -P_ij dDelta_i, so dQ_i moves by
    -scale * dDelta_i * sum_j P_ij K_j and dK_j by -scale * sum_i P_ij dDelta_i Q_i
    (over the group's query heads); dV does not depend on Delta.  Giving the
    backward these O and LSE makes its expected gradients a function of
    oracle values alone; in rows whose weight sits on a few keys the rounding
    of O moves Delta by far more than the rest of the backward's roundings.
    """
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    dQ, dK, dV = oracle.backward_ref(Q, K, V, dO, causal=causal, window=window, scale=scale)
    O_st = np.empty((B, Nq, S, Dh))
    LSE = np.empty((B, Nq, S))
    for b in range(B):
        for h in range(Nq):
            g = oracle.kv_head_of(h, Nq, Nkv)
            o, lse, P = oracle.head_attention(Q[b, h], np.arange(S), K[b, g], V[b, g], causal, window,
                                              scale, return_probs=True)
            O_st[b, h] = workloads.to_f64(workloads.f32_to_bf16_bits(o.astype(np.float32)), "bf16")
            LSE[b, h] = lse
            d_delta = np.sum(dO[b, h] * (O_st[b, h] - o), axis=1)
            dQ[b, h] -= scale * d_delta[:, None] * (P @ K[b, g])
            dK[b, g] -= scale * (P * d_delta[:, None]).T @ Q[b, h]
    return O_st, LSE, dQ, dK, dV
