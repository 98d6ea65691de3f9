"""Pins of the oracle's cache-side functions: chunked prefill against a cache,
windowed decode, and the cache append (linear and rolling buffer).

Each is tied to something other than itself: the full prefill oracle (pinned
in test_oracle_pins.py), a pure-Python brute force with explicit positions,
and the textbook's generation walk-through (prefill a prompt, then decode
token by token over a window-bounded cache, and get the full pass back).
CPU only.
"""

import math

import numpy as np
import pytest

from oracle import append_ref, attention_ref, chunk_ref, decode_ref


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("window", [0, 5, 16])
def test_chunked_prefill_pieces_equal_full(window):
    # textbook, "Prefill и decode": a prompt filled chunk by chunk, with the
    # causal mask inside each chunk, gives the rows of the one-pass prefill
    B, Nq, Nkv, S, Dh = 2, 4, 2, 37, 8
    Q, K, V = _rand((B, Nq, S, Dh), 1), _rand((B, Nkv, S, Dh), 2), _rand((B, Nkv, S, Dh), 3)
    O, L = attention_ref(Q, K, V, causal=True, window=window)
    cuts = [0, 1, 10, 11, 30, 37]
    for s0, s1 in zip(cuts[:-1], cuts[1:]):
        Oc, Lc = chunk_ref(Q[:, :, s0:s1], K, V, [s1, s1], window=window)
        np.testing.assert_allclose(Oc, O[:, :, s0:s1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lc, L[:, :, s0:s1], rtol=0, atol=1e-12)


def test_chunk_rows_equal_full_chunk():
    B, Nq, Nkv, Sq, T, Dh = 2, 4, 1, 6, 20, 5
    Q, K, V = _rand((B, Nq, Sq, Dh), 4), _rand((B, Nkv, T, Dh), 5), _rand((B, Nkv, T, Dh), 6)
    lens = [9, 20]
    O, L = chunk_ref(Q, K, V, lens, window=4)
    rows = [(0, 0, 0), (1, 3, 5), (0, 2, 3), (1, 1, 0)]
    Or, Lr = chunk_ref(Q, K, V, lens, window=4, rows=rows)
    for t, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(Or[t], O[b, h, i], rtol=0, atol=1e-13)
        assert abs(Lr[t] - L[b, h, i]) < 1e-13


def _brute_chunk(Q, K, V, lens, window, scale):
    # pure-Python loops: query i of sequence b at position lens[b] - Sq + i
    B, Nq, Sq, Dh = Q.shape
    Nkv = K.shape[1]
    O = np.zeros((B, Nq, Sq, Dh))
    L = np.zeros((B, Nq, Sq))
    for b in range(B):
        n = lens[b]
        for h in range(Nq):
            g = h // (Nq // Nkv)
            for i in range(Sq):
                pos = n - Sq + i
                vis = [j for j in range(n) if j <= pos and (window <= 0 or pos - j < window)]
                s = {j: scale * sum(float(Q[b, h, i, d]) * float(K[b, g, j, d]) for d in range(Dh))
                     for j in vis}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in vis}
                tot = sum(w.values())
                for d in range(Dh):
                    O[b, h, i, d] = sum(w[j] * float(V[b, g, j, d]) for j in vis) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


@pytest.mark.parametrize("window,seed", [(0, 7), (3, 8), (1, 9)])
def test_chunk_brute_force(window, seed):
    B, Nq, Nkv, Sq, T, Dh = 2, 4, 2, 3, 8, 3
    Q, K, V = _rand((B, Nq, Sq, Dh), seed), _rand((B, Nkv, T, Dh), seed + 1), \
        _rand((B, Nkv, T, Dh), seed + 2)
    lens = [3, 8]
    O, L = chunk_ref(Q, K, V, lens, window=window, scale=0.7)
    Ob, Lb = _brute_chunk(Q, K, V, lens, window, 0.7)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_chunk_rejects_short_cache():
    Q = np.zeros((1, 1, 4, 2))
    K = np.zeros((1, 1, 8, 2))
    with pytest.raises(ValueError):
        chunk_ref(Q, K, K, [3])
    with pytest.raises(ValueError):
        chunk_ref(Q, K, K, [9])


@pytest.mark.parametrize("window", [1, 4, 50])
def test_windowed_decode_equals_prefill_row(window):
    # a decode step of token t-1 is row t-1 of the prefill, window included
    B, Nq, Nkv, S, Dh = 2, 4, 2, 30, 6
    Q, K, V = _rand((B, Nq, S, Dh), 10), _rand((B, Nkv, S, Dh), 11), _rand((B, Nkv, S, Dh), 12)
    O, L = attention_ref(Q, K, V, causal=True, window=window)
    for t in (1, 2, 9, 30):
        Od, Ld = decode_ref(Q[:, :, t - 1], K, V, [t, t], window=window)
        np.testing.assert_allclose(Od, O[:, :, t - 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Ld, L[:, :, t - 1], rtol=0, atol=1e-12)


def test_textbook_generation_with_window_cache():
    # textbook, "Prefill и decode" walk-through: 10 tokens, 8 query heads over
    # 2 K/V heads, head size 32, window_size 4; prefill 7 tokens, then decode
    # 3 tokens one at a time with a cache that keeps only the last window
    # positions, and the outputs equal the one-pass result.  The page's window
    # admits i - j <= 4 (5 keys); in the i - j < window convention that is
    # window 5, and a rolling buffer of 5 slots that receives each new token
    # before it attends ("Скользящее окно": Mistral's rolling buffer cache).
    Nq, Nkv, T, Dh, W = 8, 2, 10, 32, 5
    Q, K, V = _rand((1, Nq, T, Dh), 20), _rand((1, Nkv, T, Dh), 21), _rand((1, Nkv, T, Dh), 22)
    full, full_lse = attention_ref(Q, K, V, causal=True, window=W)

    # prefill of the 7-token prompt: a chunk against a cache holding those 7
    pre, _ = chunk_ref(Q[:, :, :7], K[:, :, :7], V[:, :, :7], [7], window=W)
    np.testing.assert_allclose(pre, full[:, :, :7], rtol=0, atol=1e-12)

    # the rolling buffer after the prompt keeps positions 2..6
    Kb = np.full((1, Nkv, W, Dh), np.nan)
    Vb = np.full((1, Nkv, W, Dh), np.nan)
    Kb, Vb = append_ref(Kb, Vb, K[:, :, :7], V[:, :, :7], [0], rolling=True)
    for t in range(7, T):
        Kb, Vb = append_ref(Kb, Vb, K[:, :, t:t + 1], V[:, :, t:t + 1], [t], rolling=True)
        # the buffer now holds exactly positions t-4..t: attend to all of it
        o, lse = decode_ref(Q[:, :, t], Kb, Vb, [min(t + 1, W)])
        np.testing.assert_allclose(o, full[:, :, t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, full_lse[:, :, t], rtol=0, atol=1e-12)


def test_append_linear_positions():
    B, Nkv, T, Dh = 2, 3, 10, 4
    Kc = _rand((B, Nkv, T, Dh), 30)
    Vc = _rand((B, Nkv, T, Dh), 31)
    Kn = _rand((B, Nkv, 3, Dh), 32)
    Vn = _rand((B, Nkv, 3, Dh), 33)
    K2, V2 = append_ref(Kc, Vc, Kn, Vn, [0, 7])
    np.testing.assert_array_equal(K2[0, :, 0:3], Kn[0])
    np.testing.assert_array_equal(V2[1, :, 7:10], Vn[1])
    np.testing.assert_array_equal(K2[0, :, 3:], Kc[0, :, 3:])
    np.testing.assert_array_equal(K2[1, :, :7], Kc[1, :, :7])
    np.testing.assert_array_equal(Kc, _rand((B, Nkv, T, Dh), 30))  # input untouched
    with pytest.raises(ValueError):
        append_ref(Kc, Vc, Kn, Vn, [0, 8])


def test_rolling_buffer_keeps_last_window():
    # token p's key is the constant p, so the buffer's content names positions
    W, Dh = 4, 2
    Kb = np.full((1, 1, W, Dh), -1.0)
    Vb = Kb.copy()
    for p in range(11):
        row = np.full((1, 1, 1, Dh), float(p))
        Kb, Vb = append_ref(Kb, Vb, row, row, [p], rolling=True)
        held = sorted(set(Kb[0, 0, :, 0].tolist()) - {-1.0})
        assert held == list(range(max(0, p - W + 1), p + 1))
        assert Kb[0, 0, p % W, 0] == p
    # a rolling append longer than the buffer keeps its last W rows
    rows = np.arange(10, dtype=np.float64).reshape(1, 1, 10, 1).repeat(Dh, axis=3)
    K3, _ = append_ref(np.zeros((1, 1, W, Dh)), np.zeros((1, 1, W, Dh)), rows, rows, [3],
                       rolling=True)
    assert sorted(K3[0, 0, :, 0].tolist()) == [6.0, 7.0, 8.0, 9.0]
    assert K3[0, 0, (3 + 9) % W, 0] == 9.0
