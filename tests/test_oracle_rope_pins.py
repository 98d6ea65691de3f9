"""Pins of the oracle's rotary position embedding (rope_ref, rope_table_ref,
append_rope_ref).

Tied to the property the textbook states (after the rotation q_i . k_j
depends only on i - j; V and position 0 untouched), to closed forms written
out as numbers (a 2-D rotation by 1 radian, the slowest pair's frequency
10000^(-1/2) at head size 4), to RoFormer's complex-number form of the same
rotation, and to an independent library routine (the LLaMA rotary code in
``transformers``, float64 inputs).  CPU only.
"""

import numpy as np
import pytest
import torch

from oracle import append_ref, append_rope_ref, rope_angles, rope_ref, rope_table_ref

COS1, SIN1 = 0.5403023058681398, 0.8414709848078965  # cos(1 rad), sin(1 rad)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_two_dims_is_a_rotation_by_the_position():
    # head size 2: one pair, theta_0 = base^0 = 1, so position p turns (x, y) by p radians
    X = np.array([1.0, 0.0, 0.0, 1.0, 2.0, -3.0]).reshape(1, 3, 1, 2)
    Y = rope_ref(X, [[1]], style="pairs")
    np.testing.assert_allclose(Y[0, 0, 0], [COS1, SIN1], atol=1e-15)
    np.testing.assert_allclose(Y[0, 1, 0], [-SIN1, COS1], atol=1e-15)
    np.testing.assert_allclose(Y[0, 2, 0], [2 * COS1 + 3 * SIN1, 2 * SIN1 - 3 * COS1], atol=1e-14)


def test_slowest_pair_frequency():
    # head size 4, base 10000: pair 1 turns by p * 10000^(-2/4) = p / 100
    X = np.zeros((1, 1, 1, 4))
    X[..., 2] = 1.0
    Y = rope_ref(X, [[100]], style="pairs")
    np.testing.assert_allclose(Y[0, 0, 0], [0, 0, COS1, SIN1], atol=1e-14)
    Yh = rope_ref(X, [[100]], style="half")   # half layout: dims 0, 2 form pair 0
    np.testing.assert_allclose(Yh[0, 0, 0], [-np.sin(100.0), 0, np.cos(100.0), 0], atol=1e-14)


@pytest.mark.parametrize("style", ["pairs", "half"])
def test_scores_depend_only_on_the_offset(style):
    Dh = 64
    q = _rand((1, 1, 1, Dh), 1)
    k = _rand((1, 1, 1, Dh), 2)

    def score(i, j):
        return float(rope_ref(q, [[i]], style=style)[0, 0, 0] @ rope_ref(k, [[j]], style=style)[0, 0, 0])

    for i, j in ((5, 2), (0, 0), (300, 17), (4000, 4000)):
        for t in (1, 37, 2048):
            assert abs(score(i, j) - score(i + t, j + t)) < 1e-9 * (1 + abs(score(i, j)))
    assert abs(score(123, 123) - float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-11


@pytest.mark.parametrize("style", ["pairs", "half"])
def test_norms_kept_and_position_zero_is_identity(style):
    X = _rand((2, 3, 5, 16), 3)
    pos = np.arange(10).reshape(2, 5) * 91
    Y = rope_ref(X, pos, style=style)
    np.testing.assert_allclose(np.linalg.norm(Y, axis=-1), np.linalg.norm(X, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(rope_ref(X, np.zeros((2, 5), int), style=style), X)


def test_complex_form_of_roformer():
    # RoFormer writes the 2-D case as multiplication by e^{i p theta}: pairs
    # (x[2m], x[2m+1]) as complex numbers, times exp(i * p * theta_m)
    Dh, base = 32, 500.0
    X = _rand((1, 2, 6, Dh), 4)
    pos = np.array([[0, 1, 2, 77, 1000, 65535]])
    z = X[..., 0::2] + 1j * X[..., 1::2]
    m = np.arange(Dh // 2)
    rot = np.exp(1j * pos[:, None, :, None] * base ** (-2.0 * m / Dh))
    w = z * rot
    Y = rope_ref(X, pos, base=base, style="pairs")
    np.testing.assert_allclose(Y[..., 0::2], w.real, atol=1e-12)
    np.testing.assert_allclose(Y[..., 1::2], w.imag, atol=1e-12)


def test_half_layout_is_a_permutation_of_pairs():
    Dh = 8
    X = _rand((1, 1, 4, Dh), 5)
    pos = [[3, 9, 1000, 5]]
    perm = np.ravel(np.stack([np.arange(Dh // 2), np.arange(Dh // 2) + Dh // 2], axis=1))
    np.testing.assert_allclose(rope_ref(X, pos, style="half")[..., perm],
                               rope_ref(X[..., perm], pos, style="pairs"), atol=1e-15)


def test_half_layout_matches_llama_rotary_code():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    B, H, S, Dh, base = 2, 3, 7, 32, 10000.0
    q, k = _rand((B, H, S, Dh), 6), _rand((B, H, S, Dh), 7)
    pos = np.array([[0, 1, 2, 3, 4, 5, 6], [9, 10, 11, 500, 501, 4095, 2]])
    # the library's frequencies (float32) against theta_m = base^(-2m/Dh)
    cfg = LlamaConfig(hidden_size=H * Dh, num_attention_heads=H, head_dim=Dh, rope_theta=base)
    inv = LlamaRotaryEmbedding(cfg).inv_freq.double().numpy()
    np.testing.assert_allclose(rope_angles(1, Dh, base), inv, rtol=2e-7)
    # its rotation (rotate_half form) fed with exact float64 angles
    ang = rope_angles(pos, Dh, base)
    cos = torch.tensor(np.concatenate([np.cos(ang)] * 2, axis=-1))
    sin = torch.tensor(np.concatenate([np.sin(ang)] * 2, axis=-1))
    tq, tk = apply_rotary_pos_emb(torch.tensor(q), torch.tensor(k), cos, sin)
    np.testing.assert_allclose(rope_ref(q, pos, base, "half"), tq.numpy(), atol=1e-13)
    np.testing.assert_allclose(rope_ref(k, pos, base, "half"), tk.numpy(), atol=1e-13)


def test_table_columns():
    T = rope_table_ref(50, 8)
    np.testing.assert_array_equal(T[0], [1, 1, 1, 1, 0, 0, 0, 0])
    assert abs(T[1, 0] - COS1) < 1e-15 and abs(T[1, 4] - SIN1) < 1e-15
    np.testing.assert_allclose(T[:, :4] ** 2 + T[:, 4:] ** 2, 1.0, atol=1e-15)
    with pytest.raises(ValueError):
        rope_angles([1], 5)


def test_append_rotates_keys_not_values():
    B, Nkv, T, Snew, Dh = 2, 2, 12, 3, 8
    Kc, Vc = _rand((B, Nkv, T, Dh), 8), _rand((B, Nkv, T, Dh), 9)
    Kn, Vn = _rand((B, Nkv, Snew, Dh), 10), _rand((B, Nkv, Snew, Dh), 11)
    pos = [4, 10]
    K2, V2 = append_rope_ref(Kc, Vc, Kn, Vn, pos, rolling=True)
    _, Vplain = append_ref(Kc, Vc, Kn, Vn, pos, rolling=True)
    np.testing.assert_array_equal(V2, Vplain)
    for b in range(B):
        for i in range(Snew):
            slot = (pos[b] + i) % T
            # key written at slot is the new key turned by its absolute position
            np.testing.assert_allclose(K2[b, :, slot],
                                       rope_ref(Kn[b:b + 1, :, i:i + 1], [[pos[b] + i]])[0, :, 0],
                                       atol=1e-15)
    # explicit positions (padding) override the absolute ones
    K3, _ = append_rope_ref(Kc, Vc, Kn, Vn, pos, positions=np.zeros((B, Snew), int), rolling=True)
    np.testing.assert_array_equal(K3, append_ref(Kc, Vc, Kn, Vn, pos, rolling=True)[0])
