"""Pins of the oracle's backward pass (softmax_vjp, backward_ref).

Tied to what the pages print (the softmax Jacobian's largest entries for two
score rows), to central finite differences of the forward oracle, to torch's
float64 autograd through scaled_dot_product_attention (an independent
library routine), and to structural facts (GQA sums over the repeated heads;
masked pairs pass no gradient).  CPU only.
"""

import numpy as np
import pytest
import torch

from oracle import attention_ref, backward_ref, softmax_rows, softmax_vjp


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _jacobian(z):
    P, _, _ = softmax_rows(np.asarray(z, dtype=np.float64)[None, :])
    n = len(z)
    # row i of the Jacobian is the gradient of p_i: a VJP with the unit vector e_i
    return np.stack([softmax_vjp(P, np.eye(n)[i][None, :])[0] for i in range(n)])


def test_softmax_jacobian_printed_extremes():
    # textbook, "Почему делить на корень из d_h": the largest Jacobian entry is
    # 0.22 for scores (0, 1, 2) and 1.2e-5 for (0, 11.3, 22.6), 18 000 times less
    j1 = np.abs(_jacobian([0.0, 1.0, 2.0])).max()
    j2 = np.abs(_jacobian([0.0, 11.3, 22.6])).max()
    assert round(j1, 2) == 0.22
    assert abs(j2 - 1.2e-5) < 0.05e-5
    assert round(j1 / j2, -3) == 18000


def test_softmax_jacobian_rows_sum_to_zero_and_symmetric():
    # the weights sum to 1 whatever z is, so every column of dp/dz sums to 0;
    # p_i (delta_ij - p_j) is symmetric in i and j
    J = _jacobian([0.3, -1.2, 2.5, 0.0])
    np.testing.assert_allclose(J.sum(axis=0), 0.0, atol=1e-15)
    np.testing.assert_allclose(J, J.T, atol=1e-15)


def test_masked_entry_gets_no_gradient():
    P, _, _ = softmax_rows(np.array([[3.0, 1.0, -np.inf]]))
    dz = softmax_vjp(P, np.array([[0.7, -0.2, 5.0]]))
    assert dz[0, 2] == 0.0


def _loss(Q, K, V, dO, causal, window, scale):
    O, _ = attention_ref(Q, K, V, causal=causal, window=window, scale=scale)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("Nq,Nkv,S,Dh,causal,window", [
    (2, 1, 5, 3, True, 0),
    (4, 2, 6, 2, True, 3),
    (2, 2, 4, 3, False, 0),
])
def test_backward_matches_finite_differences(Nq, Nkv, S, Dh, causal, window):
    Q, K, V = _rand((1, Nq, S, Dh), 1), _rand((1, Nkv, S, Dh), 2), _rand((1, Nkv, S, Dh), 3)
    dO = _rand((1, Nq, S, Dh), 4)
    scale = 0.6
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=causal, window=window, scale=scale)
    h = 1e-6
    for X, dX in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            keep = X[idx]
            X[idx] = keep + h
            lp = _loss(Q, K, V, dO, causal, window, scale)
            X[idx] = keep - h
            lm = _loss(Q, K, V, dO, causal, window, scale)
            X[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(dX, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window", [
    (2, 4, 4, 9, 8, 0),
    (1, 8, 2, 12, 16, 0),
    (1, 4, 1, 10, 8, 4),
])
def test_backward_matches_torch_autograd(B, Nq, Nkv, S, Dh, window):
    import torch.nn.functional as F
    Q, K, V = _rand((B, Nq, S, Dh), 5), _rand((B, Nkv, S, Dh), 6), _rand((B, Nkv, S, Dh), 7)
    dO = _rand((B, Nq, S, Dh), 8)
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=True, window=window)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    ok = j <= i
    if window:
        ok = ok & (i - j < window)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, enable_gqa=(Nq != Nkv))
    out.backward(torch.tensor(dO))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-10)


def test_gqa_gradient_is_sum_over_repeats():
    # textbook, "Как K/V-головы доходят до голов Q": a shared K/V head is
    # repeated for its query heads, so its gradient is the sum over the repeats
    B, Nq, Nkv, S, Dh = 1, 8, 2, 7, 4
    Q, K, V = _rand((B, Nq, S, Dh), 9), _rand((B, Nkv, S, Dh), 10), _rand((B, Nkv, S, Dh), 11)
    dO = _rand((B, Nq, S, Dh), 12)
    dQ, dK, dV = backward_ref(Q, K, V, dO)
    G = Nq // Nkv
    dQm, dKm, dVm = backward_ref(Q, np.repeat(K, G, axis=1), np.repeat(V, G, axis=1), dO)
    np.testing.assert_allclose(dQ, dQm, atol=1e-13)
    np.testing.assert_allclose(dK, dKm.reshape(B, Nkv, G, S, Dh).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dV, dVm.reshape(B, Nkv, G, S, Dh).sum(axis=2), atol=1e-13)


def test_causal_and_window_gradients_are_local():
    B, Nq, S, Dh, W = 1, 2, 10, 4, 3
    Q, K, V = _rand((B, Nq, S, Dh), 13), _rand((B, Nq, S, Dh), 14), _rand((B, Nq, S, Dh), 15)
    dO = _rand((B, Nq, S, Dh), 16)
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=True, window=W)
    # a change of dO at query i reaches only keys i-W+1 .. i
    dO2 = dO.copy()
    dO2[:, :, 7] += 1.0
    _, dK2, dV2 = backward_ref(Q, K, V, dO2, causal=True, window=W)
    changed = np.any(np.abs(dV2 - dV) > 0, axis=(0, 1, 3))
    assert np.flatnonzero(changed).tolist() == [5, 6, 7]
    changed = np.any(np.abs(dK2 - dK) > 0, axis=(0, 1, 3))
    assert set(np.flatnonzero(changed).tolist()) <= {5, 6, 7}
    # the last key is seen only by the last query
    P_last = 1.0 / np.sum(np.exp(np.asarray(
        [Q[0, 0, S - 1] @ K[0, 0, j] for j in range(S - W, S)]) / 2.0
        - Q[0, 0, S - 1] @ K[0, 0, S - 1] / 2.0))
    np.testing.assert_allclose(dV[0, 0, S - 1], P_last * dO[0, 0, S - 1], atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3), (False, 0)])
def test_backward_rows_equal_full_backward(causal, window):
    # the row form used at long sequence lengths gives the full form's rows
    from oracle import backward_rows_ref
    B, Nq, Nkv, S, Dh = 2, 4, 2, 9, 5
    Q, K, V = _rand((B, Nq, S, Dh), 21), _rand((B, Nkv, S, Dh), 22), _rand((B, Nkv, S, Dh), 23)
    dO = _rand((B, Nq, S, Dh), 24)
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=causal, window=window, scale=0.4)
    qr = [(0, 0, 0), (1, 3, 8), (0, 2, 4), (1, 1, 5)]
    kr = [(0, 0, 0), (1, 1, 8), (0, 1, 3), (1, 0, 6)]
    rq, rk, rv = backward_rows_ref(Q, K, V, dO, qr, kr, causal=causal, window=window, scale=0.4)
    np.testing.assert_allclose(rq, [dQ[t] for t in qr], atol=1e-13)
    np.testing.assert_allclose(rk, [dK[t] for t in kr], atol=1e-13)
    np.testing.assert_allclose(rv, [dV[t] for t in kr], atol=1e-13)


def _loss_masked(Q, K, V, dO, key_mask, window, scale):
    O, _ = attention_ref(Q, K, V, causal=True, window=window, scale=scale, key_mask=key_mask)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window", [
    (2, 2, 1, 6, 3, 0),
    (2, 4, 2, 5, 2, 3),
])
def test_backward_with_key_mask_matches_finite_differences(B, Nq, Nkv, S, Dh, window):
    # textbook, "Паддинг": the padding mask joins the causal mask and the window.
    # Row 0 is left-padded by two tokens, so its first two queries see no key at
    # all (O = 0 there, and no gradient flows through them); row 1 has a padding
    # key in the middle.
    key_mask = np.ones((B, S), dtype=bool)
    key_mask[0, :2] = False
    key_mask[1, 2] = False
    Q, K, V = _rand((B, Nq, S, Dh), 31), _rand((B, Nkv, S, Dh), 32), _rand((B, Nkv, S, Dh), 33)
    dO = _rand((B, Nq, S, Dh), 34)
    scale = 0.7
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=True, window=window, scale=scale,
                              key_mask=key_mask)
    h = 1e-6
    for X, dX in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            keep = X[idx]
            X[idx] = keep + h
            lp = _loss_masked(Q, K, V, dO, key_mask, window, scale)
            X[idx] = keep - h
            lm = _loss_masked(Q, K, V, dO, key_mask, window, scale)
            X[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(dX, num, rtol=1e-6, atol=1e-8)
    # padding keys receive nothing; queries that see no key pass nothing
    assert np.all(dK[0, :, :2] == 0) and np.all(dV[0, :, :2] == 0)
    assert np.all(dK[1, :, 2] == 0) and np.all(dV[1, :, 2] == 0)
    assert np.all(dQ[0, :, :2] == 0)


def test_backward_with_key_mask_matches_torch_autograd():
    # an independent library routine: torch's float64 autograd through
    # scaled_dot_product_attention with the causal and padding masks combined
    # (every query sees at least one key, where the library's result is defined)
    import torch.nn.functional as F
    B, Nq, Nkv, S, Dh = 2, 4, 2, 9, 8
    key_mask = np.ones((B, S), dtype=bool)
    key_mask[0, 3:5] = False
    key_mask[1, 7] = False
    Q, K, V = _rand((B, Nq, S, Dh), 41), _rand((B, Nkv, S, Dh), 42), _rand((B, Nkv, S, Dh), 43)
    dO = _rand((B, Nq, S, Dh), 44)
    dQ, dK, dV = backward_ref(Q, K, V, dO, causal=True, key_mask=key_mask)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    ok = (j <= i)[None, None] & torch.tensor(key_mask)[:, None, None, :]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, enable_gqa=True)
    out.backward(torch.tensor(dO))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-10)


def test_backward_all_true_key_mask_is_no_mask_and_rows_agree():
    from oracle import backward_rows_ref
    B, Nq, Nkv, S, Dh = 2, 4, 2, 9, 5
    Q, K, V = _rand((B, Nq, S, Dh), 51), _rand((B, Nkv, S, Dh), 52), _rand((B, Nkv, S, Dh), 53)
    dO = _rand((B, Nq, S, Dh), 54)
    ones = np.ones((B, S), dtype=bool)
    a = backward_ref(Q, K, V, dO, window=4)
    b = backward_ref(Q, K, V, dO, window=4, key_mask=ones)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    key_mask = ones.copy()
    key_mask[0, :3] = False
    key_mask[1, 5] = False
    dQ, dK, dV = backward_ref(Q, K, V, dO, window=4, key_mask=key_mask)
    qr = [(0, 0, 0), (0, 1, 2), (0, 3, 7), (1, 2, 5), (1, 0, 8)]
    kr = [(0, 0, 1), (0, 1, 3), (1, 1, 5), (1, 0, 8)]
    rq, rk, rv = backward_rows_ref(Q, K, V, dO, qr, kr, window=4, key_mask=key_mask)
    np.testing.assert_allclose(rq, [dQ[t] for t in qr], atol=1e-13)
    np.testing.assert_allclose(rk, [dK[t] for t in kr], atol=1e-13)
    np.testing.assert_allclose(rv, [dV[t] for t in kr], atol=1e-13)
