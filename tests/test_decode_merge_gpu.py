"""GPU parity of the decode merge on rows with many chunk partials.

The merge gives a (sequence, query head) row up to 16 wavefronts when it has
many partial slots, each folding a contiguous run of slots under its own running
max; the runs are then folded together in LDS.  These cases reach every
wavefront count (1, 2, 4, 8, 16), rows whose slot count is below the wavefront
count (some wavefronts fold nothing), windows, and key-padding masks that make
whole runs of chunks, or a whole row, see no key.  Each is checked on every
element against the float64 oracle's decode (the merge identity there is the
plain softmax over all visible keys at once).
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say
from test_rope_padding_gpu import _split_dead

pytestmark = pytest.mark.gpu


def _chunk(B, Nkv, L, G):
    # the host's chunk rule (restated in the chunk-size tests)
    floor = 224 if G >= 16 else 640
    for ch in (1792, 1152, 896, 640, 384, 224, 160, 96):
        if ch <= floor or B * Nkv * -(-L // ch) >= (1024 if G >= 16 else 2048):
            return ch
    return floor


def _waves(B, Nkv, Tcap, G, window):
    # wavefronts per row the host gives the merge: the fewest of 1..16 that
    # leave each at most 16 slots (one round of requests)
    L = window if 0 < window < Tcap else Tcap
    ch = _chunk(B, Nkv, L, G)
    slots = -(-Tcap // ch)
    if L < Tcap:
        slots = min(slots, -(-L // ch) + 1)
    mw = 1
    while mw < 16 and -(-slots // mw) > 16:
        mw *= 2
    return mw


@pytest.mark.parametrize("Dh,B,Nq,Nkv,Tcap,lens,window,pads,block,mw", [
    (128, 2, 32, 1, 32768, [32768, 5], 0, None, None, 16),     # 147 slots; the second row has 1
    (128, 1, 8, 1, 65000, [65000], 0, None, None, 8),          # 102 slots of 640 keys
    (128, 2, 32, 1, 32768, [32768, 20500], 20000, None, None, 8),  # windowed: 91 slots
    (128, 4, 32, 8, 12000, [12000, 9000, 640, 641], 0, None, None, 2),
    (128, 8, 32, 8, 32768, [32768, 1, 30000, 12345, 640, 7000, 32767, 2048], 0, None, None, 4),
    (128, 64, 32, 8, 20000, None, 0, None, None, 1),
    (64, 1, 32, 1, 32768, [32768], 0, None, None, 16),
    (256, 1, 32, 1, 32768, [31000], 0, None, None, 16),
    # key padding: chunks 5..110 see padding only, and the second row no key at all
    (128, 2, 32, 1, 32768, [32768, 30000], 0, [0, 30000], (1000, 25000), 16),
    (128, 1, 8, 1, 65000, [65000], 0, [40000], None, 8),       # the first 62 slots dead
    # 586 chunks of 224 keys: with a mask (chunk mode) each merge wavefront
    # folds 36-37 slots in three rounds of requests; without one the even
    # split's 512 pieces leave 32 per wavefront, two rounds
    (128, 1, 32, 1, 131072, [131072], 0, [5], None, 16),
    (128, 1, 32, 1, 131072, [131072], 0, None, None, 16),
])
def test_decode_merge_waves(Dh, B, Nq, Nkv, Tcap, lens, window, pads, block, mw):
    assert _waves(B, Nkv, Tcap, Nq // Nkv, window) == mw
    say(f"merge case Dh={Dh} B={B} {Nq}/{Nkv} Tcap={Tcap} window={window} waves={mw}")
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, "bf16",
                                                seed=Tcap + B + Dh, lens=lens)
    m = None
    if pads is not None or block is not None:
        m = workloads.key_mask(B, Tcap, pads=pads, seed=Tcap, block=block)
    dev = device()
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    O, L = tch.decode(tq, tk, tv, torch.from_numpy(lens_a).to(dev), window=window,
                      key_mask=None if m is None else torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
    Lg = L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), workloads.to_f64(kc, "bf16"),
                               workloads.to_f64(vc, "bf16"), lens_a, window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "decode")
    errs = check(Og[live], Lg[live], Or[live], Lr[live], "bf16", (Dh, B, Tcap, window, pads),
                 storage_allowance=True)
    say(f"  dead rows {n_dead}: {errs}")
