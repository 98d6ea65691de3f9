"""GPU parity of attn_backward against the float64 oracle's gradients.

The GPU forward produces O and LSE, as in training; the backward then takes
dO.  The oracle computes the exact gradients of the same definition from the
stored inputs.  Tolerance, from the arithmetic (see the backward section of
the design notes): the gradients are stored in bf16 and Delta = dO . O uses
the bf16-stored O, so a correct kernel differs from the exact values by up to
~0.9 % of (1 + |ref|) and ~5e-4 on average on these inputs (an emulation of
those roundings against the oracle); the bound is twice that.
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import device, grad_rows_ratio, say, set_oracle_rows

pytestmark = pytest.mark.gpu

BF16_REL = 1.6e-2   # per element: |err| <= BF16_REL * (1 + |ref|)
# on average: mean |err| <= BF16_MEAN_REL * mean |ref| + BF16_MEAN_FLOOR.  The
# bf16 roundings the backward's arithmetic requires (stored O, the P and dS
# operands, the stored gradients) give a mean error of 2.3-2.8e-3 of mean |ref|
# on every emulated shape, short or long (test_backward_tolerance.py), so the
# bound scales with the gradients' size: twice 2^-8 of it, plus a floor
BF16_MEAN_REL = 2.0 ** -7
BF16_MEAN_FLOOR = 1e-4
F32_REL = 1e-4


def _grads(q, k, v, dO, dtype, causal, window, scale=None, given=None):
    # given: (O, LSE) as float64 arrays to pass to the backward instead of the
    # library's own forward output
    dev = device()
    tq, tk, tv, tdo = (workloads.to_torch(x, dtype, dev) for x in (q, k, v, dO))
    if given is None:
        O, L = tch.prefill(tq, tk, tv, causal=causal, window=window, scale=scale)
    else:
        O = torch.from_numpy(given[0].astype(np.float32)).to(dev).to(tq.dtype)
        L = torch.from_numpy(given[1].astype(np.float32)).to(dev)
    dQ, dK, dV = tch.backward(tq, tk, tv, O, L, tdo, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return [workloads.to_f64(workloads.from_torch(t, dtype), dtype) for t in (dQ, dK, dV)]


def _check(got, ref, dtype, what):
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(g - r)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        rel = BF16_REL if dtype == "bf16" else F32_REL
        worst = np.argmax(err - rel * (1 + np.abs(r)))
        assert np.all(err <= rel * (1 + np.abs(r))), (
            f"{what} {name}: err {err.flat[worst]:.3g} at {np.unravel_index(worst, err.shape)} "
            f"ref {r.flat[worst]:.3g}")
        if dtype == "bf16":
            bound = BF16_MEAN_REL * np.abs(r).mean() + BF16_MEAN_FLOOR
            assert err.mean() <= bound, f"{what} {name}: mean err {err.mean():.3g} > {bound:.3g}"
        out.append(f"{name} {err.max():.2e}/{err.mean():.2e}")
    say(f"backward {what}: " + " ".join(out))


def _inputs(B, Nq, Nkv, S, Dh, dtype, seed):
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=seed)
    dO = workloads.draw((B, Nq, S, Dh), dtype, seed, 3)
    return q, k, v, dO


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,causal,window", [
    (1, 2, 2, 1, 128, True, 0),
    (2, 4, 4, 63, 128, True, 0),
    (1, 4, 2, 65, 128, True, 0),
    (1, 8, 2, 300, 128, True, 0),       # GQA 4, ragged
    (1, 4, 1, 257, 128, True, 0),       # MQA
    (1, 4, 4, 700, 128, True, 100),     # window
    (1, 4, 2, 130, 128, False, 0),      # non-causal
    (2, 4, 1, 257, 64, True, 0),
    (1, 2, 2, 200, 256, True, 30),      # head size 256 (MFMA): window
    (2, 2, 2, 65, 256, True, 0),
    (1, 4, 4, 300, 256, True, 0),       # ragged, several key blocks
    (1, 8, 2, 257, 256, True, 0),       # GQA 4
    (1, 4, 1, 129, 256, False, 0),      # MQA, non-causal
    (2, 8, 4, 4, 128, False, 0),        # 4 tokens: gradients of order 1, mean error scales with them
    (2, 8, 2, 16, 64, False, 0),
])
def test_backward_bf16(B, Nq, Nkv, S, Dh, causal, window):
    q, k, v, dO = _inputs(B, Nq, Nkv, S, Dh, "bf16", seed=S + Dh)
    got = _grads(q, k, v, dO, "bf16", causal, window)
    ref = oracle.backward_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v, dO)),
                              causal=causal, window=window)
    _check(got, ref, "bf16", (B, Nq, Nkv, S, Dh, causal, window))


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window,scale", [
    (1, 2, 2, 5, 4, 0, 0.5),            # the tiny fp32 workload's shape
    (1, 4, 2, 100, 64, 7, 0.1),
    (2, 2, 1, 33, 80, 0, None),
])
def test_backward_f32(B, Nq, Nkv, S, Dh, window, scale):
    q, k, v, dO = _inputs(B, Nq, Nkv, S, Dh, "f32", seed=Dh)
    got = _grads(q, k, v, dO, "f32", True, window, scale)
    ref = oracle.backward_ref(*(workloads.to_f64(x, "f32") for x in (q, k, v, dO)),
                              causal=True, window=window, scale=scale)
    _check(got, ref, "f32", (B, Nq, Nkv, S, Dh, window))


def test_backward_deterministic():
    q, k, v, dO = _inputs(1, 8, 2, 400, 128, "bf16", seed=5)
    a = _grads(q, k, v, dO, "bf16", True, 0)
    b = _grads(q, k, v, dO, "bf16", True, 0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("Nkv,Dh", [(32, 128), (8, 128), (32, 64), (8, 256)])
def test_backward_repeat_bitwise_long(Nkv, Dh):
    # dK / dV at head size 128 pass the weights from one wavefront to another
    # through LDS; three calls on an 8192-token causal input give the same bits
    B, Nq, S = 1, 32, 8192
    dev = device()
    g = torch.Generator(device=dev).manual_seed(Nkv + Dh)
    tq = torch.randn(B, Nq, S, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    tk = torch.randn(B, Nkv, S, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    tv = torch.randn(B, Nkv, S, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    tdo = torch.randn(B, Nq, S, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    O, L = tch.prefill(tq, tk, tv)
    runs = []
    for _ in range(3):
        grads = tch.backward(tq, tk, tv, O, L, tdo)
        torch.cuda.synchronize()
        runs.append([x.view(torch.int16).clone() for x in grads])
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert torch.equal(a, b)


def test_backward_workspace_checked():
    dev = device()
    t = torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16, device=dev)
    L = torch.zeros(1, 2, 16, dtype=torch.float32, device=dev)
    small = torch.empty(8, dtype=torch.uint8, device=dev)
    with pytest.raises(tch.AttnError) as e:
        tch.attn_backward(t, t, t, t, t, L, t.clone(), t.clone(), t.clone(), workspace=small)
    assert e.value.status == tch.ATTN_EWORKSPACE


class _Lazy:
    """Widens slices of stored bf16 values to float64 on access."""

    def __init__(self, arr):
        self.arr, self.shape = arr, arr.shape

    def __getitem__(self, idx):
        return workloads.to_f64(self.arr[idx], "bf16")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("Nkv", [32, 8])
def test_backward_full_size_sampled_rows(Nkv):
    # the bench's backward shape (32768-token causal attention, 32 query heads,
    # head size 128, MHA and GQA 32/8): seeded dQ rows anywhere plus rows 0 and
    # S-1, and dK / dV rows of keys in the last tile (each seen by <= 64 queries
    # per head), against the oracle's row form
    B, Nq, S, Dh = 1, 32, 32768, 128
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=0)
    dO = workloads.draw((B, Nq, S, Dh), "bf16", 0, 3)
    dev = device()
    tq, tk, tv, tdo = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v, dO))
    O, L = tch.prefill(tq, tk, tv)
    qr = workloads.sample_rows(B, Nq, S, 10, seed=5, forced_rows=(0, S - 1))
    shift = set_oracle_rows(O, L, _Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr)
    dQ, dK, dV = tch.backward(tq, tk, tv, O, L, tdo)
    torch.cuda.synchronize()
    kr = [(0, 0, S - 1), (0, Nkv // 2, S - 33), (0, Nkv - 1, S - 64)]
    idx = lambda rows: tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    got = [workloads.to_f64(workloads.from_torch(t[idx(r)], "bf16"), "bf16")
           for t, r in ((dQ, qr), (dK, kr), (dV, kr))]
    del tq, tk, tv, tdo, O, L, dQ, dK, dV
    ref = oracle.backward_rows_ref(_Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr, kr)
    ref = (ref[0] + shift, ref[1], ref[2])
    # At this length the weights are ~1/S and the gradient rows are small
    # (a last-tile key's dV is ~1e-5), so (1 + |ref|) would say little: each
    # sampled row is held to the same relative bound against its own scale,
    # floored at 1 % of the largest sampled row (query 0 sees only key 0, and
    # its exact dQ is 0).  The sampled query rows take the oracle's O and LSE
    # before the backward, so their dQ is fixed by oracle values (with O as
    # stored in bf16).
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        ratio = grad_rows_ratio(g, r)
        assert np.all(np.isfinite(g)), name
        assert np.all(ratio <= BF16_REL), f"{name}: worst row-relative error {ratio.max():.3g}"
        out.append(f"{name} {ratio.max():.2e}")
    say(f"backward full size Nkv={Nkv}, row-relative: " + " ".join(out))


@pytest.mark.timeout(300)
def test_backward_head256_sampled_rows():
    # head size 256 on the MFMA kernels at a long shape (16384-token causal
    # GQA 32/8, the head-size-256 prefill shape of the benchmark): seeded dQ
    # rows plus rows 0 and S-1, and dK / dV rows of keys in the last tile,
    # against the oracle's row form, held as in the 32768-token test above
    B, Nq, Nkv, S, Dh = 1, 32, 8, 16384, 256
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=2)
    dO = workloads.draw((B, Nq, S, Dh), "bf16", 2, 3)
    dev = device()
    tq, tk, tv, tdo = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v, dO))
    O, L = tch.prefill(tq, tk, tv)
    qr = workloads.sample_rows(B, Nq, S, 10, seed=7, forced_rows=(0, S - 1))
    shift = set_oracle_rows(O, L, _Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr)
    dQ, dK, dV = tch.backward(tq, tk, tv, O, L, tdo)
    torch.cuda.synchronize()
    kr = [(0, 0, S - 1), (0, Nkv // 2, S - 33), (0, Nkv - 1, S - 64)]
    idx = lambda rows: tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    got = [workloads.to_f64(workloads.from_torch(t[idx(r)], "bf16"), "bf16")
           for t, r in ((dQ, qr), (dK, kr), (dV, kr))]
    del tq, tk, tv, tdo, O, L, dQ, dK, dV
    ref = oracle.backward_rows_ref(_Lazy(q), _Lazy(k), _Lazy(v), _Lazy(dO), qr, kr)
    ref = (ref[0] + shift, ref[1], ref[2])
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        ratio = grad_rows_ratio(g, r)
        assert np.all(np.isfinite(g)), name
        assert np.all(ratio <= BF16_REL), f"{name}: worst row-relative error {ratio.max():.3g}"
        out.append(f"{name} {ratio.max():.2e}")
    say("backward head size 256, row-relative: " + " ".join(out))


def _key_mask(B, S, pattern, seed):
    m = np.ones((B, S), dtype=bool)
    if pattern == "left":       # left padding: the first queries of a row see no key
        for b in range(B):
            m[b, :min(S - 1, 3 + 17 * b)] = False
    elif pattern == "mid":      # a run of padding inside the sequence
        m[:, S // 3:S // 3 + 40] = False
    elif pattern == "random":   # about 10 % of the keys hidden anywhere
        m = np.random.default_rng(seed).random((B, S)) > 0.1
    return m


def _grads_padded(q, k, v, dO, dtype, mask, window):
    dev = device()
    tq, tk, tv, tdo = (workloads.to_torch(x, dtype, dev) for x in (q, k, v, dO))
    tm = torch.from_numpy(mask).to(dev)
    O, L = tch.prefill(tq, tk, tv, causal=True, window=window, key_mask=tm)
    dQ, dK, dV = tch.backward(tq, tk, tv, O, L, tdo, causal=True, window=window, key_mask=tm)
    torch.cuda.synchronize()
    return [workloads.to_f64(workloads.from_torch(t, dtype), dtype) for t in (dQ, dK, dV)]


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window,pattern,dtype", [
    (2, 4, 2, 300, 128, 0, "left", "bf16"),     # queries that see no key: dQ = 0
    (2, 4, 4, 257, 128, 0, "mid", "bf16"),      # whole 64-key tiles of padding
    (1, 8, 2, 400, 128, 100, "random", "bf16"),
    (2, 4, 1, 200, 64, 0, "random", "bf16"),
    (1, 4, 4, 300, 256, 0, "left", "bf16"),
    (1, 8, 2, 160, 256, 30, "mid", "bf16"),
    (2, 4, 2, 90, 80, 0, "left", "bf16"),       # head size 80: row kernels
    (1, 2, 1, 70, 64, 7, "random", "f32"),      # fp32: row kernels
])
def test_backward_padded(B, Nq, Nkv, S, Dh, window, pattern, dtype):
    mask = _key_mask(B, S, pattern, seed=S)
    q, k, v, dO = _inputs(B, Nq, Nkv, S, Dh, dtype, seed=S + Dh + 1)
    got = _grads_padded(q, k, v, dO, dtype, mask, window)
    ref = oracle.backward_ref(*(workloads.to_f64(x, dtype) for x in (q, k, v, dO)),
                              causal=True, window=window, key_mask=mask)
    _check(got, ref, dtype, ("padded", pattern, B, Nq, Nkv, S, Dh, window))
    # exact zeros where the definition gives them: padding keys receive no
    # gradient, queries that saw no key pass none
    dQ, dK, dV = got
    for b in range(B):
        hidden = ~mask[b]
        assert np.all(dK[b][:, hidden] == 0) and np.all(dV[b][:, hidden] == 0)
        blind = np.flatnonzero(np.cumsum(mask[b]) == 0)  # causal: no real key at or before i
        assert np.all(dQ[b][:, blind] == 0)


@pytest.mark.parametrize("Dh", [64, 128, 256])
def test_backward_all_true_mask_is_the_unpadded_backward(Dh):
    # an all-true mask takes the same kernels and paths: identical bits
    B, Nq, Nkv, S = 2, 8, 2, 333
    q, k, v, dO = _inputs(B, Nq, Nkv, S, Dh, "bf16", seed=Dh + 9)
    a = _grads(q, k, v, dO, "bf16", True, 0)
    b = _grads_padded(q, k, v, dO, "bf16", np.ones((B, S), dtype=bool), 0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
