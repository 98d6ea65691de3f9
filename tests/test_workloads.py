"""Seeded input generation and closed-form work counts (CPU only)."""

import json
import os

import numpy as np
import torch

import workloads
from oracle import allowed_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, np.inf, -np.inf, 1e-40,
                  1.00390625, 1.01171875], dtype=np.float32),   # two exact ties
    ]).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.isnan(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(
        np.array([np.nan], np.float32))))[0]


def test_torch_roundtrip():
    q, _, _ = workloads.prefill_inputs(1, 2, 2, 5, 4, "bf16")
    t = workloads.to_torch(q, "bf16")
    assert t.dtype == torch.bfloat16 and tuple(t.shape) == (1, 2, 5, 4)
    assert np.array_equal(workloads.from_torch(t, "bf16"), q)
    np.testing.assert_array_equal(t.double().numpy(), workloads.to_f64(q, "bf16"))


def test_prefill_inputs_deterministic():
    a = workloads.prefill_inputs(1, 2, 2, 5, 4, "f32", seed=0)
    b = workloads.prefill_inputs(1, 2, 2, 5, 4, "f32", seed=0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert a[0].dtype == np.float32 and a[0].shape == (1, 2, 5, 4)
    # N(0,1): sample moments of a larger draw
    q, _, _ = workloads.prefill_inputs(1, 4, 4, 256, 64, "bf16")
    f = workloads.to_f64(q, "bf16")
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01


def test_decode_lens_recipe_and_poison():
    cfg = workloads.WORKLOADS["decode_bf16_b64_h32kv8_t32768_d128"]
    lens = np.random.default_rng(0).integers(cfg["len_lo"], cfg["len_hi"], cfg["B"],
                                             endpoint=True)
    assert lens.sum() == 1101299 and lens.min() == 1110 and lens.max() == 32680
    # a small version of the same recipe: poison beyond the lengths
    lens_s, q, kc, vc = workloads.decode_inputs(3, 4, 2, 8, 16, 4, 16, seed=0)
    f = workloads.to_f64(kc, "bf16")
    for b in range(3):
        assert np.isfinite(f[b, :, :lens_s[b]]).all()
        assert np.isnan(f[b, :, lens_s[b]:]).all()


def test_visible_pairs_closed_form_matches_mask_count():
    for S in (1, 2, 7, 64, 100):
        for window in (0, 1, 3, 16, 99, 100, 150):
            ok = allowed_mask(np.arange(S), S, causal=True, window=window)
            assert workloads.visible_pairs_per_head(S, True, window) == int(ok.sum())
    assert workloads.visible_pairs_per_head(9, False, 0) == 81


def test_op_counts_match_german_page():
    # the page prints attention costs 1.4e11 (s = d = 4096) and 8.8e12
    # (s = 32768); the causal count over visible pairs at 32 heads x 128
    # reproduces both to the printed two digits
    with open(os.path.join(GOLDEN, "softmax_tables.json")) as f:
        cases = json.load(f)["op_counts"]["cases"]
    for c in cases:
        flops, _ = workloads.prefill_work(1, c["heads"], c["heads"], c["S"], c["Dh"],
                                          True, 0, 2)
        assert abs(flops - c["printed"]) <= 0.05 * 10 ** np.floor(np.log10(c["printed"]))


def test_sample_rows_forced_and_in_range():
    tr = workloads.sample_rows(4, 32, 8192, 1024, seed=1, forced_rows=(0, 4095, 4096, 8191))
    assert len(tr) == 1024 + 8
    assert all(0 <= b < 4 and 0 <= h < 32 and 0 <= i < 8192 for b, h, i in tr)
    assert (0, 0, 4096) in tr and (3, 31, 8191) in tr
