"""A sequence's prefill result does not depend on the launch form it runs in.

The host picks the workgroup shape from the grid size: a grid that would
fill the chip at most once runs as 4-wave workgroups, two per CU, at head
size 128, and with strided query blocks at head sizes 64 and 256.  Larger
grids run 8-wave (head size 256: 4-wave) workgroups with consecutive blocks.
Every wave computes its own rows in the same order in all of these, so a
sequence run alone (small grid) and the same sequence inside a large batch
(several rounds) must give the same bits, and the alone run must match the
float64 oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Nq,Nkv,S,Dh,causal,window,copies", [
    (32, 32, 1024, 128, True, 0, 8),     # 4-wave form alone, 8-wave in the batch
    (32, 8, 2048, 128, True, 0, 8),      # GQA
    (16, 16, 777, 128, True, 0, 24),     # ragged last tile
    (32, 32, 1024, 128, False, 0, 8),    # non-causal
    (32, 32, 2000, 128, True, 300, 8),   # window
    (32, 32, 1024, 64, True, 0, 8),      # strided blocks alone
    (16, 16, 1024, 256, True, 0, 40),    # strided blocks alone, 4-wave form at 256
])
def test_prefill_same_bits_in_any_launch_form(Nq, Nkv, S, Dh, causal, window, copies):
    dev = device()
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    q, k, v = workloads.prefill_inputs(1, Nq, Nkv, S, Dh, "bf16", seed=S + Dh + Nkv)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    O1, L1 = tch.prefill(tq, tk, tv, causal=causal, window=window)
    # the batch: the same sequence in every slot, so that the grid spans several rounds
    Ob, Lb = tch.prefill(tq.expand(copies, -1, -1, -1).contiguous(),
                         tk.expand(copies, -1, -1, -1).contiguous(),
                         tv.expand(copies, -1, -1, -1).contiguous(), causal=causal, window=window)
    torch.cuda.synchronize()
    say(f"launch forms Nq={Nq} Nkv={Nkv} S={S} Dh={Dh} causal={causal} window={window}: "
        f"alone and in a batch of {copies} on {n_cu} CUs")
    for c in range(copies):
        assert torch.equal(O1[0].view(torch.int16), Ob[c].view(torch.int16)), c
        assert torch.equal(L1[0], Lb[c]), c
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(a, "bf16") for a in (q, k, v)),
                                  causal=causal, window=window, scale=1.0 / math.sqrt(Dh))
    Og = workloads.to_f64(workloads.from_torch(O1, "bf16"), "bf16")
    say(f"  vs oracle: {check(Og, L1.cpu().numpy().astype(np.float64), Or, Lr, 'bf16', (Nq, S, Dh), storage_allowance=True)}")
