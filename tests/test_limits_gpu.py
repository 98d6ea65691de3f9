"""GPU parity at the largest head the bf16 MFMA prefill addresses.

The kernel reads one head of K and V through a buffer descriptor whose byte
range is 31 bits wide, so a head may hold at most (2^31 - 1) // (2 * Dh)
rows: 8388607 tokens at head size 128.  One causal prefill of exactly that
length (one head, window 4096 so that it runs in milliseconds) is checked on
sampled rows, including the last, against the float64 oracle.  That one row
more is rejected on the host is checked without a GPU, with placeholder
pointers (tests/test_abi.py).

Inputs are drawn on the device from a seeded generator (8.6 GB would take too
long to draw on the host); each sampled row's reference is the oracle's
single-query attention over that row's window of keys, copied back.
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say

pytestmark = pytest.mark.gpu

DH = 128
S_MAX = (2 ** 31 - 1) // (2 * DH)  # 8388607
WINDOW = 4096


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.timeout(300)
def test_prefill_at_the_largest_head():
    dev = device()
    g = torch.Generator(device=dev).manual_seed(31)
    q, k, v = (torch.randn(1, 1, S_MAX, DH, device=dev, dtype=torch.bfloat16, generator=g)
               for _ in range(3))
    say(f"limits: prefill S={S_MAX} Dh={DH} window={WINDOW}")
    O, L = tch.prefill(q, k, v, window=WINDOW)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = sorted({0, 1, 63, 64, WINDOW - 1, WINDOW, WINDOW + 1, 1 << 20, (1 << 22) + 17,
                   S_MAX - 65, S_MAX - 2, S_MAX - 1, *[int(x) for x in rng.integers(0, S_MAX, 8)]})
    Og, Lg, Or, Lr = [], [], [], []
    for i in rows:
        lo = max(0, i - WINDOW + 1)
        # row i sees keys lo .. i: a single query against i - lo + 1 cached keys
        o, l = oracle.decode_ref(_f64(q[0, :, i])[None], _f64(k[:, :, lo:i + 1]),
                                 _f64(v[:, :, lo:i + 1]), np.array([i - lo + 1]))
        Or.append(o[0, 0]); Lr.append(l[0, 0])
        Og.append(_f64(O[0, 0, i])); Lg.append(float(L[0, 0, i]))
    say(f"  {len(rows)} rows: {check(np.array(Og), np.array(Lg), np.array(Or), np.array(Lr), 'bf16', 'largest head')}")
