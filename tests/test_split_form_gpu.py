"""The key-split form of the prefill (one-round causal grids with at least
4096 keys per head) against the oracle and against the unsplit form.

In that form each 8-wave workgroup holds 128 query rows; waves 0-3 stream the
first half of its key tiles and waves 4-7 the second half, and the two
partial results are merged by the online-softmax rescaling rule.  The same
sequence inside a batch large enough for several rounds runs unsplit, so the
two results differ only in summation order: they are held to each other at
the bf16 tolerance, and the split run is held to the float64 oracle on
sampled rows, including the first and last rows and rows at the halves'
boundaries.  The cases cover a ragged last tile, a window, grouped-query
heads, and groups of two query heads per K/V head, where the first query
tiles have a single key tile and the second half of their workgroup none.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import BF16_LSE, BF16_MAX, check, device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Nq,Nkv,S,window,copies", [
    (16, 16, 4096, 0, 4),     # MHA
    (8, 8, 8192, 0, 4),       # longer heads
    (8, 8, 5000, 0, 4),       # ragged last tile
    (16, 16, 4096, 1000, 4),  # window: an odd number of tiles in some workgroups
    (16, 8, 4096, 0, 4),      # two query heads per K/V head: single-tile workgroups
])
def test_split_form(Nq, Nkv, S, window, copies):
    dev = device()
    q, k, v = workloads.prefill_inputs(1, Nq, Nkv, S, 128, "bf16", seed=S + Nq + Nkv + window)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    say(f"split form Nq={Nq} Nkv={Nkv} S={S} window={window}")
    O1, L1 = tch.prefill(tq, tk, tv, causal=True, window=window)
    Ob, Lb = tch.prefill(tq.expand(copies, -1, -1, -1).contiguous(),
                         tk.expand(copies, -1, -1, -1).contiguous(),
                         tv.expand(copies, -1, -1, -1).contiguous(), causal=True, window=window)
    torch.cuda.synchronize()
    d = (O1[0].float() - Ob[copies - 1].float()).abs()
    dl = (L1[0] - Lb[copies - 1]).abs()
    assert d.max().item() <= BF16_MAX and dl.max().item() <= BF16_LSE, (d.max().item(), dl.max().item())
    say(f"  split vs unsplit: max |dO| {d.max().item():.2e}, max |dLSE| {dl.max().item():.2e}")
    # sampled rows against the oracle
    forced = [0, 1, 63, 64, 127, 128, 255, 256, S // 2 - 1, S // 2, S - 129, S - 128, S - 2, S - 1]
    rows = workloads.sample_rows(1, Nq, S, 96, seed=7, forced_rows=forced)
    Qf, Kf, Vf = (workloads.to_f64(a, "bf16") for a in (q, k, v))
    Or, Lr = oracle.attention_rows_ref(Qf, Kf, Vf, rows, causal=True, window=window,
                                       scale=1.0 / math.sqrt(128))
    Og = workloads.to_f64(workloads.from_torch(O1, "bf16"), "bf16")
    Lg = L1.cpu().numpy().astype(np.float64)
    got = np.stack([Og[b, h, i] for b, h, i in rows])
    lg = np.array([Lg[b, h, i] for b, h, i in rows])
    say(f"  vs oracle on {len(rows)} rows: {check(got, lg, Or, Lr, 'bf16', (Nq, S, window))}")
