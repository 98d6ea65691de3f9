"""The tail of a long prefill grid is handed out at run time; the bits do not change.

A causal bf16 prefill without a window or cache whose grid covers the chip
four or more times draws its last quarter of work items from per-XCD counters
at run time, so that an XCD that runs ahead takes over the last items of a
slower one.  Which workgroup computes
an item does not change how the item is computed, so the drawn order must give
exactly the bits of the fixed order.  A launch into a stream being captured
into a graph takes the fixed order, which is what these tests compare against.
Each stream has its own set of counters, which every launch leaves cleared
for the next; the other tests here run launches on two streams at once and
many launches back to back on one stream.
"""

import pytest
import torch

import transformer_causal_head_amd as tch
import workloads
from helpers import device, say

pytestmark = pytest.mark.gpu

# each of these grids covers a 256-CU chip at least four times
SHAPES = [
    # B, Nq, Nkv, S, Dh, window
    (1, 32, 32, 8192, 128, 0),     # 1024 workgroups: 32 heads x 32 query tiles
    (2, 32, 8, 4096, 128, 0),      # GQA
    (2, 32, 8, 4096, 128, 1024),   # with a window: always the fixed order
    (1, 32, 32, 8192, 64, 0),
    (1, 16, 16, 8192, 256, 0),
    (3, 16, 16, 6000, 128, 0),     # ragged last query tile
]


def _inputs(B, Nq, Nkv, S, Dh, seed):
    dev = device()
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=seed)
    return tuple(workloads.to_torch(a, "bf16", dev) for a in (q, k, v))


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,Nq,Nkv,S,Dh,window", SHAPES)
def test_graph_replay_gives_the_eager_bits(B, Nq, Nkv, S, Dh, window):
    say(f"drawn tail vs graph replay B={B} Nq={Nq} Nkv={Nkv} S={S} Dh={Dh} window={window}")
    tq, tk, tv = _inputs(B, Nq, Nkv, S, Dh, seed=S + Dh)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq, S), dtype=torch.float32, device=tq.device)
    tch.attn_prefill(tq, tk, tv, O, L, causal=1, window=window)
    torch.cuda.synchronize()
    Oe, Le = O.clone(), L.clone()

    Og = torch.full_like(tq, float("nan"))
    Lg = torch.full((B, Nq, S), float("nan"), dtype=torch.float32, device=tq.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            tch.attn_prefill(tq, tk, tv, Og, Lg, causal=1, window=window)
    torch.cuda.synchronize()
    for r in range(3):
        Og.fill_(float("nan"))
        Lg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(Og, Oe), f"replay {r}: O differs from the eager launch"
        assert torch.equal(Lg, Le), f"replay {r}: LSE differs from the eager launch"
        # eager work between the replays: the same call outside the graph
        tch.attn_prefill(tq, tk, tv, O, L, causal=1, window=window)
        torch.cuda.synchronize()
        assert _same(O, Oe) and torch.equal(L, Le), f"eager launch after replay {r}"


def test_two_streams_at_once():
    B, Nq, Nkv, S, Dh = 1, 32, 32, 8192, 128
    say("drawn tail: two streams at once, 4 launches each")
    A = _inputs(B, Nq, Nkv, S, Dh, seed=11)
    Bq = _inputs(B, Nq, Nkv, S, Dh, seed=12)
    refs = []
    for x in (A, Bq):
        O = torch.empty_like(x[0])
        L = torch.empty((B, Nq, S), dtype=torch.float32, device=x[0].device)
        tch.attn_prefill(*x, O, L, causal=1)
        torch.cuda.synchronize()
        refs.append((O, L))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {0: [], 1: []}
    for i in range(4):
        for j, (x, s) in enumerate(((A, s1), (Bq, s2))):
            O = torch.full_like(x[0], float("nan"))
            L = torch.full((B, Nq, S), float("nan"), dtype=torch.float32, device=x[0].device)
            outs[j].append((O, L))
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                tch.attn_prefill(*x, O, L, causal=1)
    torch.cuda.synchronize()
    for j in (0, 1):
        for i, (O, L) in enumerate(outs[j]):
            assert _same(O, refs[j][0]) and torch.equal(L, refs[j][1]), (j, i)


def test_back_to_back_launches_on_one_stream():
    # 80 launches queued at once: each must find its stream's counters cleared
    # by the launch before it
    B, Nq, Nkv, S, Dh = 1, 32, 32, 8192, 128
    n = 80
    say(f"drawn tail: {n} launches in flight on one stream")
    x = _inputs(B, Nq, Nkv, S, Dh, seed=13)
    O0 = torch.empty_like(x[0])
    L0 = torch.empty((B, Nq, S), dtype=torch.float32, device=x[0].device)
    tch.attn_prefill(*x, O0, L0, causal=1)
    torch.cuda.synchronize()
    outs = [(torch.full_like(x[0], float("nan")),
             torch.full((B, Nq, S), float("nan"), dtype=torch.float32, device=x[0].device))
            for _ in range(n)]
    torch.cuda.synchronize()
    for O, L in outs:
        tch.attn_prefill(*x, O, L, causal=1)
    torch.cuda.synchronize()
    for i, (O, L) in enumerate(outs):
        assert _same(O, O0) and torch.equal(L, L0), i


def test_key_padded_graph_replay_gives_the_eager_bits():
    # the key-padded kernel draws its tail the same way
    B, Nq, Nkv, S, Dh = 2, 32, 32, 8192, 128
    say("drawn tail, key-padded: eager vs graph replay")
    tq, tk, tv = _inputs(B, Nq, Nkv, S, Dh, seed=21)
    mask = torch.ones(B, S, dtype=torch.bool, device=tq.device)
    mask[0, :700] = False          # left padding
    mask[1, 3000:3100] = False     # a hole
    bits = torch.empty(B, (S + 63) // 64, dtype=torch.int64, device=tq.device)
    tch.attn_pack_key_mask(mask, bits)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq, S), dtype=torch.float32, device=tq.device)
    tch.attn_prefill_padded(tq, tk, tv, bits, O, L, causal=1)
    torch.cuda.synchronize()
    Og = torch.full_like(tq, float("nan"))
    Lg = torch.full((B, Nq, S), float("nan"), dtype=torch.float32, device=tq.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            tch.attn_prefill_padded(tq, tk, tv, bits, Og, Lg, causal=1)
    torch.cuda.synchronize()
    for r in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert _same(Og, O), f"replay {r}: O differs"
        # rows that see no key carry LSE = -inf on both sides
        assert torch.equal(Lg, L), f"replay {r}: LSE differs"


def test_three_streams_interleaved_shapes():
    # three streams, each with its own counter set, take turns launching
    # grids of different sizes (all long enough to draw their tails); every
    # result must match the same call made alone
    dev = device()
    shapes = [(1, 32, 32, 8192, 128), (2, 16, 16, 8192, 128), (1, 32, 8, 12288, 128)]
    inputs = [_inputs(B, Nq, Nkv, S, Dh, seed=30 + k) for k, (B, Nq, Nkv, S, Dh) in enumerate(shapes)]
    say("drawn tail: three streams, interleaved shapes")
    refs = []
    for (B, Nq, Nkv, S, Dh), x in zip(shapes, inputs):
        O = torch.empty_like(x[0])
        L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
        tch.attn_prefill(*x, O, L, causal=1)
        torch.cuda.synchronize()
        refs.append((O, L))
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for r in range(6):
        for k, s in enumerate(streams):
            j = (k + r) % len(shapes)
            B, Nq, Nkv, S, Dh = shapes[j]
            O = torch.empty_like(inputs[j][0])
            L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
            with torch.cuda.stream(s):
                O.fill_(float("nan"))
                tch.attn_prefill(*inputs[j], O, L, causal=1)
            outs.append((j, O, L))
    torch.cuda.synchronize()
    for n, (j, O, L) in enumerate(outs):
        assert _same(O, refs[j][0]) and torch.equal(L, refs[j][1]), (n, j)
