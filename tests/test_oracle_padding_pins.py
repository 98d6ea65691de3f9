"""Pins of the oracle's key-padding mask (the ``key_mask`` argument of
attention_ref, chunk_ref and decode_ref).

Tied to a hand computation, to facts that follow from the definition (padding
keys pass nothing: changing them changes no output; a left-padded batch row,
with positions counted from its first real token, reproduces the unpadded
sequence exactly -- with RoPE too; a padded decode equals a decode over the
cache with the padding slots removed), to the chosen reading for a row that
sees no key (O = 0, LSE = -inf), and to torch's scaled_dot_product_attention
with a boolean mask (an independent library routine).  CPU only.
"""

import numpy as np
import pytest
import torch

from oracle import attention_ref, chunk_ref, decode_ref, rope_ref


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_computed_row():
    # one query, keys 0 (pad), 1, 2 with scores 5 (ignored), 1, 3 -> weights e/(e+e^3), e^3/(e+e^3)
    Q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    K = np.array([[5.0, 0], [1.0, 0], [3.0, 0]]).reshape(1, 1, 3, 2)
    V = np.array([[100.0, 0], [1.0, 0], [0.0, 1]]).reshape(1, 1, 3, 2)
    Qf = np.repeat(Q, 3, axis=2)
    O, L = attention_ref(Qf, K, V, causal=False, scale=1.0, key_mask=np.array([[False, True, True]]))
    w1 = 1.0 / (1.0 + np.exp(2.0))  # e^1 / (e^1 + e^3)
    np.testing.assert_allclose(O[0, 0, 2], [w1, 1 - w1], atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 2], 3.0 + np.log(1.0 + np.exp(-2.0)), atol=1e-15)


def test_all_true_mask_is_no_mask():
    Q, K, V = _rand((2, 4, 9, 8), 1), _rand((2, 2, 9, 8), 2), _rand((2, 2, 9, 8), 3)
    ones = np.ones((2, 9), bool)
    a = attention_ref(Q, K, V, window=4)
    b = attention_ref(Q, K, V, window=4, key_mask=ones)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_padding_keys_pass_nothing():
    Q, K, V = _rand((2, 4, 12, 8), 4), _rand((2, 2, 12, 8), 5), _rand((2, 2, 12, 8), 6)
    mask = np.ones((2, 12), bool)
    mask[0, [0, 1, 5]] = False
    mask[1, 11] = False
    O, L = attention_ref(Q, K, V, key_mask=mask)
    K2, V2 = K.copy(), V.copy()
    for b in range(2):
        K2[b, :, ~mask[b]] += 50.0
        V2[b, :, ~mask[b]] = 1e30  # finite: a zero weight times NaN would still be NaN
    O2, L2 = attention_ref(Q, K2, V2, key_mask=mask)
    # rows that see at least one key are unchanged; (0, .., 0) and (0, .., 1) see only pads
    np.testing.assert_array_equal(O2[:, :, 2:], O[:, :, 2:])
    np.testing.assert_array_equal(L2, L)


def test_row_without_visible_key():
    Q, K, V = _rand((1, 2, 5, 4), 7), _rand((1, 2, 5, 4), 8), _rand((1, 2, 5, 4), 9)
    mask = np.array([[False, False, True, True, True]])
    O, L = attention_ref(Q, K, V, key_mask=mask)
    assert np.all(O[:, :, :2] == 0) and np.all(L[:, :, :2] == -np.inf)
    assert np.all(np.isfinite(O[:, :, 2:])) and np.all(np.isfinite(L[:, :, 2:]))


@pytest.mark.parametrize("window,style", [(0, None), (3, None), (0, "pairs"), (4, "half")])
def test_left_padding_reproduces_the_unpadded_sequence(window, style):
    # batch row b holds pad[b] padding tokens then the real sequence; keys of
    # the pads are masked, positions count from the first real token
    Nq, Nkv, S, Dh = 4, 2, 11, 8
    pad = [0, 3, 6]
    B = len(pad)
    real_q = [_rand((1, Nq, S - p, Dh), 10 + p) for p in pad]
    real_k = [_rand((1, Nkv, S - p, Dh), 20 + p) for p in pad]
    real_v = [_rand((1, Nkv, S - p, Dh), 30 + p) for p in pad]
    Q = np.zeros((B, Nq, S, Dh))
    K = np.zeros((B, Nkv, S, Dh))
    V = np.zeros((B, Nkv, S, Dh))
    mask = np.zeros((B, S), bool)
    pos = np.zeros((B, S), int)
    for b, p in enumerate(pad):
        Q[b, :, p:], K[b, :, p:], V[b, :, p:] = real_q[b][0], real_k[b][0], real_v[b][0]
        Q[b, :, :p] = K[b, :, :p] = V[b, :, :p] = 9.0
        mask[b, p:] = True
        pos[b, p:] = np.arange(S - p)
    if style:
        Q, K = rope_ref(Q, pos, style=style), rope_ref(K, pos, style=style)
    O, L = attention_ref(Q, K, V, window=window, key_mask=mask)
    for b, p in enumerate(pad):
        q, k = real_q[b], real_k[b]
        if style:
            q = rope_ref(q, [np.arange(S - p)], style=style)
            k = rope_ref(k, [np.arange(S - p)], style=style)
        Ou, Lu = attention_ref(q, k, real_v[b], window=window)
        np.testing.assert_allclose(O[b, :, p:], Ou[0], atol=1e-12)
        np.testing.assert_allclose(L[b, :, p:], Lu[0], atol=1e-12)
        assert np.all(O[b, :, :p] == 0)


def test_matches_torch_sdpa_with_boolean_mask():
    import torch.nn.functional as F
    B, Nq, Nkv, S, Dh = 2, 4, 2, 10, 8
    Q, K, V = _rand((B, Nq, S, Dh), 11), _rand((B, Nkv, S, Dh), 12), _rand((B, Nkv, S, Dh), 13)
    mask = np.random.default_rng(14).random((B, S)) > 0.3
    mask[:, 0] = True  # every row sees key 0, so torch's softmax has no empty row
    O, L = attention_ref(Q, K, V, window=6, key_mask=mask)
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    ok = (j <= i) & (i - j < 6)
    full = torch.tensor(ok[None, None] & mask[:, None, None, :])
    out = F.scaled_dot_product_attention(torch.tensor(Q), torch.tensor(K), torch.tensor(V),
                                         attn_mask=full, enable_gqa=True)
    np.testing.assert_allclose(O, out.numpy(), atol=1e-12)


def test_decode_equals_cache_without_padding_slots():
    B, Nq, Nkv, T, Dh = 3, 8, 2, 20, 8
    q = _rand((B, Nq, Dh), 15)
    Kc, Vc = _rand((B, Nkv, T, Dh), 16), _rand((B, Nkv, T, Dh), 17)
    lens = np.array([20, 13, 7])
    mask = np.random.default_rng(18).random((B, T)) > 0.4
    for b in range(B):
        mask[b, lens[b] - 1] = True
    O, L = decode_ref(q, Kc, Vc, lens, key_mask=mask)
    for b in range(B):
        keep = np.flatnonzero(mask[b, :lens[b]])
        Ob, Lb = decode_ref(q[b:b + 1], Kc[b:b + 1][:, :, keep], Vc[b:b + 1][:, :, keep], [len(keep)])
        np.testing.assert_allclose(O[b], Ob[0], atol=1e-13)
        np.testing.assert_allclose(L[b], Lb[0], atol=1e-13)


def test_chunk_rows_equal_full_prefill_rows():
    B, Nq, Nkv, S, Sq, Dh = 2, 4, 1, 16, 5, 8
    Q, K, V = _rand((B, Nq, S, Dh), 19), _rand((B, Nkv, S, Dh), 20), _rand((B, Nkv, S, Dh), 21)
    mask = np.ones((B, S), bool)
    mask[0, :4] = False
    mask[1, [2, 9, 14]] = False
    lens = [S, 12]
    for b, n in enumerate(lens):
        Of, Lf = attention_ref(Q[b:b + 1, :, :n], K[b:b + 1, :, :n], V[b:b + 1, :, :n], window=5,
                               key_mask=mask[b:b + 1, :n])
        Oc, Lc = chunk_ref(Q[b:b + 1, :, n - Sq:n], K[b:b + 1], V[b:b + 1], [n], window=5,
                           key_mask=mask[b:b + 1])
        np.testing.assert_allclose(Oc[0], Of[0, :, n - Sq:], atol=1e-13)
        np.testing.assert_allclose(Lc[0], Lf[0, :, n - Sq:], atol=1e-13)
