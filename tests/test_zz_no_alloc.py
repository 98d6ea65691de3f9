"""The allocation-free decode entry point (attn_decode_noalloc) against
attn_decode, through the C ABI.

attn_decode_noalloc runs the same kernels as attn_decode with the partials in
the library's fixed device scratch instead of a caller's workspace, so the two
must give the same bits; both are also held to the oracle at the stated bf16
tolerance.  Two calls in a row, the second with a smaller input, show that a
call does not depend on what the previous one left in the scratch.
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say

pytestmark = pytest.mark.gpu


def _run(B, Nq, Nkv, Dh, Tcap, lens, seed):
    dev = device()
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, "bf16",
                                                seed=seed, lens=lens)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    tl = torch.from_numpy(np.asarray(lens_a, np.int32)).to(dev)
    O1, L1 = torch.empty_like(tq), torch.empty((B, Nq), dtype=torch.float32, device=dev)
    tch.attn_decode_noalloc(tq, tk, tv, tl, O1, L1)
    torch.cuda.synchronize()
    ws = torch.empty(max(1, tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, tch.ATTN_BF16)),
                     dtype=torch.uint8, device=dev)
    O2, L2 = torch.empty_like(tq), torch.empty_like(L1)
    tch.attn_decode(tq, tk, tv, tl, O2, L2, ws)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)), "O differs from attn_decode"
    assert torch.equal(L1, L2), "LSE differs from attn_decode"
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), workloads.to_f64(kc, "bf16"),
                               workloads.to_f64(vc, "bf16"), lens_a)
    got = workloads.to_f64(workloads.from_torch(O1, "bf16"), "bf16")
    return check(got, L1.cpu().numpy().astype(np.float64), Or, Lr, "bf16", (B, Nq, Nkv, Dh, Tcap))


def test_noalloc_twice_second_smaller():
    # first call: 16 sequences, 32/8 heads, up to 8000 cached keys (many partial
    # slots); second: 3 sequences, MQA 16/1, short caches, fewer and different slots
    say("noalloc: B=16 Nq=32 Nkv=8 Dh=128 Tcap=8000")
    say(f"  {_run(16, 32, 8, 128, 8000, None, seed=5)}")
    say("noalloc: B=3 Nq=16 Nkv=1 Dh=128 Tcap=900 lens=[1, 640, 900]")
    say(f"  {_run(3, 16, 1, 128, 900, [1, 640, 900], seed=6)}")


def test_noalloc_head_sizes_and_general_kernel():
    say("noalloc: Dh 64 and 256")
    say(f"  {_run(4, 8, 2, 64, 3000, [3000, 1, 1500, 2999], seed=7)}")
    say(f"  {_run(2, 32, 4, 256, 2500, [2500, 700], seed=8)}")
    # head size 80 takes the general kernel, which needs no scratch at all
    say(f"  {_run(2, 4, 2, 80, 300, [300, 5], seed=9)}")
