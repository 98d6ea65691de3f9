"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test names its source.  Together they are chosen so that a plausible slip
in the oracle (a dropped scale, a transposed mask, softmax over the wrong axis,
PV with the operands swapped, the GQA map taken modulo instead of divided, an
off-by-one window, a wrong LSE) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (allowed_mask, attention_ref, attention_rows_ref, decode_ref,
                    head_attention, kv_head_of, softmax_rows)
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- worked example (textbook, "Численный пример") ------------------------

def _worked():
    g = _golden("worked_example.json")
    Q = np.array(g["Q"], float)[None, None]
    K = np.array(g["K"], float)[None, None]
    V = np.array(g["V"], float)[None, None]
    return g, Q, K, V


def test_worked_example_probabilities_match_printed():
    g, Q, K, V = _worked()
    _, _, P = head_attention(Q[0, 0], np.arange(3), K[0, 0], V[0, 0],
                             causal=True, window=0, scale=1 / math.sqrt(2),
                             return_probs=True)
    np.testing.assert_allclose(P, np.array(g["P_printed"]), atol=1e-4)
    # the masked (future) weights are exactly zero
    assert P[0, 1] == 0.0 and P[0, 2] == 0.0 and P[1, 2] == 0.0


def test_worked_example_output_matches_printed():
    g, Q, K, V = _worked()
    O, _ = attention_ref(Q, K, V, causal=True, scale=1 / math.sqrt(2))
    # the PyTorch printout carries correctly rounded digits
    np.testing.assert_allclose(O[0, 0], np.array(g["O_torch_printed"]), atol=6e-5)
    # the hand computation rounds its weights first: within 2e-4
    np.testing.assert_allclose(O[0, 0], np.array(g["O_hand_printed"]), atol=2e-4)


def test_worked_example_default_scale_is_head_size():
    # default scale must be 1/sqrt(d_h) = 1/sqrt(2) here (not 1, not 1/d_h)
    g, Q, K, V = _worked()
    O_default, _ = attention_ref(Q, K, V, causal=True)
    np.testing.assert_allclose(O_default[0, 0], np.array(g["O_torch_printed"]), atol=6e-5)


def test_worked_example_lse_from_printed_row_sums():
    # LSE_i = m_i + ln l_i = ln(sum_j exp(S_ij)) over visible keys.  Row 0 has
    # one visible key with score 0.7071; rows 1, 2 have the printed sums of
    # exponentials 3.0281 and 8.1695.
    g, Q, K, V = _worked()
    _, LSE = attention_ref(Q, K, V, causal=True, scale=1 / math.sqrt(2))
    sums = g["exp_row_sums_printed"]
    expected = [g["scores_printed"][0][0], math.log(sums[1]), math.log(sums[2])]
    np.testing.assert_allclose(LSE[0, 0], expected, atol=1e-4)


def test_exercise_one_output():
    g, Q, K, _ = _worked()
    V2 = np.array(g["exercise1_V"], float)[None, None]
    O, _ = attention_ref(Q, K, V2, causal=True, scale=1 / math.sqrt(2))
    np.testing.assert_allclose(O[0, 0, 2], g["exercise1_o2_printed"], atol=2e-4)


# --- softmax values (textbook tables, Chinese post) ------------------------

def test_softmax_tables():
    t = _golden("softmax_tables.json")
    for case in t["saturation"]["cases"]:
        P, _, _ = softmax_rows(np.array(case["z"], float)[None])
        if "tol" in case:
            np.testing.assert_allclose(P[0], case["p"], atol=case["tol"])
        else:
            np.testing.assert_allclose(P[0], case["p"], rtol=case["rel_tol"])
    sd = t["soft_dictionary"]
    P, _, _ = softmax_rows(np.array(sd["z"], float)[None])
    np.testing.assert_allclose(P[0], sd["p"], atol=sd["tol"])


def test_softmax_masked_entry_exactly_zero():
    z = np.array([[3.0, 1.0, -np.inf]])
    P, m, l = softmax_rows(z)
    assert P[0, 2] == 0.0
    assert abs(P[0].sum() - 1.0) < 1e-15
    assert m[0] == 3.0


def test_softmax_shift_invariance():
    # textbook exercise 5: adding one constant to a row leaves softmax unchanged
    rng = np.random.default_rng(5)
    A = rng.standard_normal((7, 11))
    P1, _, _ = softmax_rows(A)
    P2, _, _ = softmax_rows(A + rng.standard_normal((7, 1)) * 50)
    np.testing.assert_allclose(P1, P2, atol=1e-13)


def test_softmax_normalises_last_axis():
    # softmax over keys (last axis), not over queries
    A = np.array([[0.0, 1.0], [5.0, -3.0], [2.0, 2.0]])
    P, _, _ = softmax_rows(A)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-15)
    assert not np.allclose(P.sum(axis=0), 1.0)


# --- properties of the full oracle ------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_probability_rows_sum_to_one_and_future_is_zero():
    S, Dh = 37, 16
    q, k, v = _rand((S, Dh), 1), _rand((S, Dh), 2), _rand((S, Dh), 3)
    for window in (0, 5):
        _, _, P = head_attention(q, np.arange(S), k, v, True, window, 0.25,
                                 return_probs=True)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
        i, j = np.indices(P.shape)
        assert np.all(P[j > i] == 0.0)
        if window:
            assert np.all(P[(i - j) >= window] == 0.0)
            assert np.all(P[(j <= i) & ((i - j) < window)] > 0.0)


def test_output_is_explicit_weighted_sum():
    # o_i = sum_j P_ij v_j (textbook formula; Chinese post's PV section)
    S, Dh = 9, 5
    q, k, v = _rand((S, Dh), 4), _rand((S, Dh), 5), _rand((S, Dh), 6)
    O, _, P = head_attention(q, np.arange(S), k, v, True, 0, 0.7, return_probs=True)
    for i in range(S):
        acc = np.zeros(Dh)
        for j in range(S):
            acc += P[i, j] * v[j]
        np.testing.assert_allclose(O[i], acc, atol=1e-13)
    # and the Chinese post's example weights
    w = np.array(_golden("softmax_tables.json")["weighted_sum"]["p"])
    vv = _rand((4, 3), 7)
    np.testing.assert_allclose(w @ vv, 0.1 * vv[0] + 0.2 * vv[1] + 0.6 * vv[2] + 0.1 * vv[3],
                               atol=1e-15)


def test_lse_normalises_scores():
    # sum_j exp(A_ij - LSE_i) = 1 over visible keys
    S, Dh = 13, 8
    q, k, v = _rand((S, Dh), 8), _rand((S, Dh), 9), _rand((S, Dh), 10)
    _, LSE = head_attention(q, np.arange(S), k, v, True, 4, 0.3)
    for i in range(S):
        tot = 0.0
        for j in range(S):
            if j <= i and i - j < 4:
                tot += math.exp(0.3 * float(q[i] @ k[j]) - LSE[i])
        assert abs(tot - 1.0) < 1e-12


def test_causality_last_token_perturbation():
    # Swedish/English note: change the last token, earlier rows are unchanged
    B, H, S, Dh = 1, 3, 10, 8
    Q, K, V = _rand((B, H, S, Dh), 11), _rand((B, H, S, Dh), 12), _rand((B, H, S, Dh), 13)
    O1, L1 = attention_ref(Q, K, V, causal=True)
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[:, :, -1] += 1.0
    K2[:, :, -1] -= 2.0
    V2[:, :, -1] += 3.0
    O2, L2 = attention_ref(Q2, K2, V2, causal=True)
    assert np.array_equal(O1[:, :, :-1], O2[:, :, :-1])
    assert np.array_equal(L1[:, :, :-1], L2[:, :, :-1])
    assert not np.allclose(O1[:, :, -1], O2[:, :, -1])


def test_non_causal_sees_future():
    B, H, S, Dh = 1, 1, 6, 4
    Q, K, V = _rand((B, H, S, Dh), 14), _rand((B, H, S, Dh), 15), _rand((B, H, S, Dh), 16)
    O1, _ = attention_ref(Q, K, V, causal=False)
    V2 = V.copy()
    V2[:, :, -1] += 1.0
    O2, _ = attention_ref(Q, K, V2, causal=False)
    assert not np.allclose(O1[:, :, 0], O2[:, :, 0])


# --- GQA / MQA mapping (textbook, "Виды по числу голов K/V") -------------

def test_gqa_mapping_printed_example():
    t = _golden("softmax_tables.json")["gqa_mapping"]
    assert [kv_head_of(h, t["H"], t["G"]) for h in range(t["H"])] == t["kv_head"]
    with pytest.raises(ValueError):
        kv_head_of(0, 6, 4)


def test_gqa_equals_mha_on_repeat_interleaved_kv():
    # the repository's _repeat_kv_heads order == repeat_interleave(H/G, dim=1)
    B, H, G, S, Dh = 2, 8, 2, 7, 4
    Q, K, V = _rand((B, H, S, Dh), 17), _rand((B, G, S, Dh), 18), _rand((B, G, S, Dh), 19)
    O, L = attention_ref(Q, K, V, causal=True, window=3)
    Kr, Vr = np.repeat(K, H // G, axis=1), np.repeat(V, H // G, axis=1)
    Om, Lm = attention_ref(Q, Kr, Vr, causal=True, window=3)
    assert np.array_equal(O, Om) and np.array_equal(L, Lm)
    # the other plausible order (h mod G) gives a different answer
    Kt, Vt = np.tile(K, (1, H // G, 1, 1)), np.tile(V, (1, H // G, 1, 1))
    Ot, _ = attention_ref(Q, Kt, Vt, causal=True, window=3)
    assert not np.allclose(O, Ot)


def test_mqa_is_broadcast():
    B, H, S, Dh = 1, 4, 6, 4
    Q, K, V = _rand((B, H, S, Dh), 20), _rand((B, 1, S, Dh), 21), _rand((B, 1, S, Dh), 22)
    O, _ = attention_ref(Q, K, V, causal=True)
    for h in range(H):
        Oh, _ = attention_ref(Q[:, h:h + 1], K, V, causal=True)
        assert np.array_equal(O[:, h:h + 1], Oh)


# --- sliding window --------------------------------------------------------

def test_window_visible_key_counts():
    # window w: query i sees keys max(0, i-w+1) .. i, i.e. min(i+1, w) keys
    ok = allowed_mask(np.arange(12), 12, causal=True, window=4)
    assert list(ok.sum(axis=1)) == [min(i + 1, 4) for i in range(12)]
    assert ok[9, 6] and not ok[9, 5] and not ok[9, 10]


def test_window_covering_sequence_is_causal():
    B, H, S, Dh = 1, 2, 9, 4
    Q, K, V = _rand((B, H, S, Dh), 23), _rand((B, H, S, Dh), 24), _rand((B, H, S, Dh), 25)
    Oc, Lc = attention_ref(Q, K, V, causal=True)
    for w in (S, S + 5):
        Ow, Lw = attention_ref(Q, K, V, causal=True, window=w)
        assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)
    Ow, _ = attention_ref(Q, K, V, causal=True, window=S - 1)
    assert not np.allclose(Oc[:, :, -1], Ow[:, :, -1])
    assert np.array_equal(Oc[:, :, :-1], Ow[:, :, :-1])


def test_window_without_causal_rejected():
    with pytest.raises(ValueError):
        allowed_mask(np.arange(3), 3, causal=False, window=2)


# --- brute force on tiny inputs (pure Python scalars) ----------------------

def _brute(Q, K, V, causal, window, scale):
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    O = [[[[0.0] * Dh for _ in range(S)] for _ in range(Nq)] for _ in range(B)]
    LSE = [[[0.0] * S for _ in range(Nq)] for _ in range(B)]
    for b in range(B):
        for h in range(Nq):
            g = (h * Nkv) // Nq          # == h // (Nq / Nkv) when Nkv divides Nq
            for i in range(S):
                vis = [j for j in range(S)
                       if (not causal or j <= i) and (window <= 0 or i - j < window)]
                s = {j: scale * sum(float(Q[b, h, i, d]) * float(K[b, g, j, d])
                                    for d in range(Dh)) for j in vis}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in vis}
                tot = sum(w.values())
                for d in range(Dh):
                    O[b][h][i][d] = sum(w[j] * float(V[b, g, j, d]) for j in vis) / tot
                LSE[b][h][i] = mx + math.log(tot)
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,causal,window,seed", [
    (1, 2, 2, 5, 4, True, 0, 0),
    (2, 4, 2, 8, 3, True, 3, 1),
    (1, 6, 1, 7, 5, True, 2, 2),
    (1, 3, 3, 6, 8, False, 0, 3),
    (2, 8, 4, 8, 2, True, 1, 4),
])
def test_brute_force_agrees(B, Nq, Nkv, S, Dh, causal, window, seed):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, Nq, S, Dh))
    K = rng.standard_normal((B, Nkv, S, Dh))
    V = rng.standard_normal((B, Nkv, S, Dh))
    scale = 1.0 / math.sqrt(Dh) * (1.7 if seed % 2 else 1.0)
    O, L = attention_ref(Q, K, V, causal=causal, window=window, scale=scale)
    Ob, Lb = _brute(Q, K, V, causal, window, scale)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(L, Lb, atol=1e-12)


# --- independent library routine: torch CPU float64 SDPA ---------------------

@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window", [
    (1, 4, 4, 6, 8, 0),       # the textbook's SDPA check shape [1, 4, 6, 8]
    (2, 8, 2, 33, 16, 0),
    (1, 8, 2, 40, 16, 7),
    (1, 4, 1, 17, 32, 0),
])
def test_torch_sdpa_cross_check(B, Nq, Nkv, S, Dh, window):
    rng = np.random.default_rng(100 + S)
    Q = rng.standard_normal((B, Nq, S, Dh))
    K = rng.standard_normal((B, Nkv, S, Dh))
    V = rng.standard_normal((B, Nkv, S, Dh))
    O, L = attention_ref(Q, K, V, causal=True, window=window)
    tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    mask = j <= i
    if window:
        mask &= (i - j) < window
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, enable_gqa=(Nkv != Nq))
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    # LSE against torch.logsumexp of the masked, scaled scores
    Kr = torch.repeat_interleave(tk, Nq // Nkv, dim=1)
    sc = (tq @ Kr.transpose(-1, -2)) / math.sqrt(Dh)
    sc = sc.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(sc, dim=-1).numpy(), atol=1e-12)


# --- sampled rows and decode -------------------------------------------------

def test_sampled_rows_equal_full():
    B, Nq, Nkv, S, Dh = 2, 4, 2, 21, 8
    rng = np.random.default_rng(30)
    Q = rng.standard_normal((B, Nq, S, Dh))
    K = rng.standard_normal((B, Nkv, S, Dh))
    V = rng.standard_normal((B, Nkv, S, Dh))
    O, L = attention_ref(Q, K, V, causal=True, window=6)
    tr = workloads.sample_rows(B, Nq, S, 20, seed=1, forced_rows=(0, S - 1))
    Os, Ls = attention_rows_ref(Q, K, V, tr, causal=True, window=6)
    for t, (b, h, i) in enumerate(tr):
        np.testing.assert_allclose(Os[t], O[b, h, i], atol=1e-13)
        np.testing.assert_allclose(Ls[t], L[b, h, i], atol=1e-13)


def test_decode_equals_prefill_last_row():
    # textbook, "Prefill и decode": prefill then one-token decode steps give
    # the rows of the full pass
    B, Nq, Nkv, S, Dh = 2, 8, 2, 10, 16
    rng = np.random.default_rng(31)
    Q = rng.standard_normal((B, Nq, S, Dh))
    K = rng.standard_normal((B, Nkv, S, Dh))
    V = rng.standard_normal((B, Nkv, S, Dh))
    O, L = attention_ref(Q, K, V, causal=True)
    Tcap = 12
    Kc = np.full((B, Nkv, Tcap, Dh), np.nan)
    Vc = np.full((B, Nkv, Tcap, Dh), np.nan)
    Kc[:, :, :S], Vc[:, :, :S] = K, V
    for t in range(7, S + 1):
        lens = np.array([t, t])
        Od, Ld = decode_ref(Q[:, :, t - 1], Kc, Vc, lens)
        np.testing.assert_allclose(Od, O[:, :, t - 1], atol=1e-13)
        np.testing.assert_allclose(Ld, L[:, :, t - 1], atol=1e-13)
    # ragged lengths, each row against its own prefix
    lens = np.array([3, 9])
    Od, _ = decode_ref(Q[:, :, 0], Kc, Vc, lens)
    for b in range(B):
        Ob, _ = attention_ref(Q[b:b + 1, :, :1].repeat(lens[b], axis=2)[:, :, :lens[b]],
                              K[b:b + 1, :, :lens[b]], V[b:b + 1, :, :lens[b]], causal=False)
        np.testing.assert_allclose(Od[b], Ob[0, :, 0], atol=1e-13)
    with pytest.raises(ValueError):
        decode_ref(Q[:, :, 0], Kc, Vc, np.array([0, 3]))
