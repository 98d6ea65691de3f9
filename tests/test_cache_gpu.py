"""GPU parity of the cache-side entry points against the float64 oracle:
chunked prefill against a cache (attn_prefill_cache), windowed decode
(attn_decode_window), the cache append (attn_kv_append, linear and rolling),
and generation end to end (chunked prefill, then appends and decode steps over
a window-bounded rolling cache, against the one-pass oracle)."""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say, takes_even_split

pytestmark = pytest.mark.gpu


class _Lazy:
    """Widens cache slices to float64 on access (the caches can be large)."""

    def __init__(self, arr, dtype):
        self.arr, self.dtype, self.shape = arr, dtype, arr.shape

    def __getitem__(self, idx):
        return workloads.to_f64(self.arr[idx], self.dtype)


def _run_chunk(Q, kc, vc, lens, dtype, window, scale=None):
    dev = device()
    tQ, tk, tv = (workloads.to_torch(x, dtype, dev) for x in (Q, kc, vc))
    tl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev)
    O, L = tch.prefill_cache(tQ, tk, tv, tl, window=window, scale=scale)
    torch.cuda.synchronize()
    return workloads.to_f64(workloads.from_torch(O, dtype), dtype), L.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,Nq,Nkv,Sq,Tcap,lens,window", [
    (2, 8, 2, 64, 300, [64, 300], 0),          # chunk of exactly one tile, ragged caches
    (2, 8, 2, 100, 700, [100, 613], 0),
    (3, 4, 4, 1, 257, [1, 2, 257], 0),         # one-row chunks
    (2, 8, 2, 130, 1000, [130, 999], 64),      # window
    (1, 32, 8, 257, 2048, [2048], 300),        # GQA 4, window, chunk past a query tile
    (2, 4, 1, 300, 600, [300, 600], 0),        # MQA; sequence 0 is a plain prefill
    (1, 8, 8, 40, 5000, [4321], 1),            # window 1: only the diagonal
])
def test_prefill_cache_bf16(B, Nq, Nkv, Sq, Tcap, lens, window):
    lens_a, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, 128, Tcap, lens, "bf16", seed=Sq)
    O, L = _run_chunk(Q, kc, vc, lens_a, "bf16", window)
    Or, Lr = oracle.chunk_ref(workloads.to_f64(Q, "bf16"), _Lazy(kc, "bf16"), _Lazy(vc, "bf16"),
                              lens_a, window=window)
    say(f"prefill_cache {B, Nq, Nkv, Sq, Tcap, lens, window}: "
        f"{check(O, L, Or, Lr, 'bf16', (Sq, lens, window), storage_allowance=True)}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("window", [0, 4096])
def test_prefill_cache_full_size_sampled_rows(window):
    # the chunk `bench.py --cache-paths` times: the last 2048 tokens of a
    # 32768-token context, 32 query / 8 K/V heads, on seeded sampled rows plus
    # the chunk's first and last rows, against the oracle's chunk attention
    B, Nq, Nkv, Sq, Dh, Tcap = 1, 32, 8, 2048, 128, 32768
    lens_a, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, Dh, Tcap, [Tcap], "bf16", seed=5)
    O, L = _run_chunk(Q, kc, vc, lens_a, "bf16", window)
    rows = workloads.sample_rows(B, Nq, Sq, 64, seed=11, forced_rows=(0, 1, Sq // 2, Sq - 1))
    Or, Lr = oracle.chunk_ref(_Lazy(Q, "bf16"), _Lazy(kc, "bf16"), _Lazy(vc, "bf16"), lens_a,
                              window=window, rows=rows)
    Og = np.stack([O[b, h, i] for b, h, i in rows])
    Lg = np.array([L[b, h, i] for b, h, i in rows])
    say(f"prefill_cache full size window={window}: "
        f"{check(Og, Lg, Or, Lr, 'bf16', ('chunk 2048 of 32768', window), storage_allowance=True)}")


@pytest.mark.parametrize("Dh,dtype,window", [(64, "f32", 0), (80, "bf16", 9), (128, "f32", 20),
                                              (64, "bf16", 0), (256, "bf16", 30)])
def test_prefill_cache_other_head_sizes(Dh, dtype, window):
    lens_a, Q, kc, vc = workloads.chunk_inputs(2, 4, 2, 33, Dh, 200, [33, 180], dtype, seed=Dh)
    O, L = _run_chunk(Q, kc, vc, lens_a, dtype, window, scale=0.3)
    Or, Lr = oracle.chunk_ref(workloads.to_f64(Q, dtype), workloads.to_f64(kc, dtype),
                              workloads.to_f64(vc, dtype), lens_a, window=window, scale=0.3)
    check(O, L, Or, Lr, dtype, (Dh, dtype, window), storage_allowance=True)


@pytest.mark.parametrize("window", [0, 200])
def test_chunked_prefill_pieces(window):
    # a 1000-token prompt filled in four chunks equals the one-pass prefill
    B, Nq, Nkv, S = 2, 8, 2, 1000
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, 128, "bf16", seed=77)
    dev = device()
    tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (k, v))
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)),
                                  causal=True, window=window)
    cuts = [0, 300, 301, 700, 1000]
    for s0, s1 in zip(cuts[:-1], cuts[1:]):
        tq = workloads.to_torch(np.ascontiguousarray(q[:, :, s0:s1]), "bf16", dev)
        tl = torch.full((B,), s1, dtype=torch.int32, device=dev)
        O, L = tch.prefill_cache(tq, tk, tv, tl, window=window)
        torch.cuda.synchronize()
        Og = workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16")
        check(Og, L.cpu().numpy().astype(np.float64), Or[:, :, s0:s1], Lr[:, :, s0:s1], "bf16",
              (s0, s1, window), storage_allowance=True)


def _run_decode(q, kc, vc, lens, dtype, window, scale=None):
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, dtype, dev) for x in (q, kc, vc))
    tl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev)
    O, L = tch.decode(tq, tk, tv, tl, window=window, scale=scale)
    torch.cuda.synchronize()
    return workloads.to_f64(workloads.from_torch(O, dtype), dtype), L.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,Nq,Nkv,Tcap,lens,window", [
    (6, 32, 8, 3000, [1, 31, 32, 33, 2000, 3000], 1),
    (6, 32, 8, 3000, [1, 31, 32, 33, 2000, 3000], 32),
    (6, 32, 8, 3000, [1, 31, 32, 33, 2000, 3000], 100),
    (4, 16, 2, 5000, [4097, 5000, 97, 1000], 4096),
    (3, 8, 8, 2100, [1024, 1025, 2048], 5000),          # window past every length
    (16, 32, 8, 16384, None, 1000),                     # 384-key chunks, windows across them
])
def test_decode_window_bf16(B, Nq, Nkv, Tcap, lens, window):
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, 128, Tcap, 1, Tcap, seed=window,
                                                lens=lens)
    O, L = _run_decode(q, kc, vc, lens_a, "bf16", window)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), _Lazy(kc, "bf16"), _Lazy(vc, "bf16"),
                               lens_a, window=window)
    say(f"decode window {window}: {check(O, L, Or, Lr, 'bf16', window, storage_allowance=True)}")


@pytest.mark.parametrize("Dh,dtype,Nq,Nkv", [(64, "f32", 4, 2), (128, "bf16", 6, 2),
                                             (64, "bf16", 4, 2), (256, "bf16", 32, 1)])
def test_decode_window_other_shapes(Dh, dtype, Nq, Nkv):
    lens_a, q, kc, vc = workloads.decode_inputs(3, Nq, Nkv, Dh, 400, 1, 400, dtype, seed=Dh,
                                                lens=[400, 17, 250])
    O, L = _run_decode(q, kc, vc, lens_a, dtype, 40, scale=0.2)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, dtype), workloads.to_f64(kc, dtype),
                               workloads.to_f64(vc, dtype), lens_a, window=40, scale=0.2)
    check(O, L, Or, Lr, dtype, (Dh, dtype), storage_allowance=True)


@pytest.mark.parametrize("dtype,Dh,Snew,Tcap,pos,rolling", [
    ("bf16", 128, 3, 50, [0, 47], 0),
    ("bf16", 128, 7, 20, [15, 0], 1),
    ("bf16", 128, 45, 20, [3, 40], 1),       # longer than the buffer: last 20 rows win
    ("f32", 64, 5, 16, [11, 2], 0),
    ("bf16", 3, 4, 9, [2, 8], 1),            # odd row length: 2-byte copies
])
def test_kv_append(dtype, Dh, Snew, Tcap, pos, rolling):
    B, Nkv = 2, 3
    dev = device()
    kc = workloads.draw((B, Nkv, Tcap, Dh), dtype, 5, 1)
    vc = workloads.draw((B, Nkv, Tcap, Dh), dtype, 5, 2)
    kn = workloads.draw((B, Nkv, Snew, Dh), dtype, 5, 3)
    vn = workloads.draw((B, Nkv, Snew, Dh), dtype, 5, 4)
    tk, tv, tkn, tvn = (workloads.to_torch(x, dtype, dev) for x in (kc, vc, kn, vn))
    tpos = torch.tensor(pos, dtype=torch.int32, device=dev)
    tch.attn_kv_append(tkn, tvn, tk, tv, tpos, rolling=rolling)
    torch.cuda.synchronize()
    Kr, Vr = oracle.append_ref(kc, vc, kn, vn, pos, rolling=bool(rolling))
    assert np.array_equal(workloads.from_torch(tk, dtype), Kr)  # bit-exact copy
    assert np.array_equal(workloads.from_torch(tv, dtype), Vr)


@pytest.mark.parametrize("mode", ["rolling", "linear", "fused"])
def test_generation_over_window_cache(mode):
    # the textbook's walk-through at attention-kernel scale: a 200-token prompt
    # by chunked prefill, then 40 tokens one at a time, window 64; each output
    # row must match the one-pass oracle.  "fused" appends each token inside
    # the decode call (attn_decode_append) on a linear cache that holds NaN in
    # every row not yet written
    Nq, Nkv, Dh, T, P, W = 32, 8, 128, 240, 200, 64
    q, k, v = workloads.prefill_inputs(1, Nq, Nkv, T, Dh, "bf16", seed=91)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)),
                                  causal=True, window=W)
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
    # prompt: its K/V form a linear cache, the chunk is the whole prompt
    O, L = tch.prefill_cache(tq[:, :, :P].contiguous(), tk[:, :, :P].contiguous(),
                             tv[:, :, :P].contiguous(),
                             torch.tensor([P], dtype=torch.int32, device=dev), window=W)
    torch.cuda.synchronize()
    check(workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16"),
          L.cpu().numpy().astype(np.float64), Or[:, :, :P], Lr[:, :, :P], "bf16", "prompt",
          storage_allowance=True)
    cap = W if mode == "rolling" else T
    Kc = torch.full((1, Nkv, cap, Dh), float("nan"), dtype=torch.bfloat16, device=dev)
    Vc = torch.full((1, Nkv, cap, Dh), float("nan"), dtype=torch.bfloat16, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    tch.attn_kv_append(tk[:, :, :P].contiguous(), tv[:, :, :P].contiguous(), Kc, Vc, zero,
                       rolling=int(mode == "rolling"))
    for t in range(P, T):
        pos = torch.tensor([t], dtype=torch.int32, device=dev)
        qt = tq[:, :, t].contiguous()
        if mode == "fused":
            O = torch.empty_like(qt)
            L = torch.empty((1, Nq), dtype=torch.float32, device=dev)
            ws = torch.empty(tch.attn_decode_window_workspace_bytes(1, Nq, Nkv, Dh, cap, W,
                                                                    tch.ATTN_BF16),
                             dtype=torch.uint8, device=dev)
            tch.attn_decode_append(qt, tk[:, :, t].contiguous(), tv[:, :, t].contiguous(), Kc, Vc,
                                   pos + 1, pos, O, L, ws, window=W)
            torch.cuda.synchronize()
            check(workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16"),
                  L.cpu().numpy().astype(np.float64), Or[:, :, t], Lr[:, :, t], "bf16", (mode, t),
                  storage_allowance=True)
            continue
        tch.attn_kv_append(tk[:, :, t:t + 1].contiguous(), tv[:, :, t:t + 1].contiguous(), Kc, Vc,
                           pos, rolling=int(mode == "rolling"))
        if mode == "rolling":   # the buffer holds exactly the window: attend to all of it
            O, L = tch.decode(qt, Kc, Vc, torch.tensor([min(t + 1, W)], dtype=torch.int32,
                                                       device=dev))
        else:
            O, L = tch.decode(qt, Kc, Vc, pos + 1, window=W)
        torch.cuda.synchronize()
        check(workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16"),
              L.cpu().numpy().astype(np.float64), Or[:, :, t], Lr[:, :, t], "bf16", (mode, t),
              storage_allowance=True)


@pytest.mark.parametrize("dtype,B,Nq,Nkv,Dh,Tcap,lens,window,rolling,unaligned", [
    ("bf16", 6, 32, 8, 128, 3000, [1, 31, 32, 33, 1792, 3000], 0, False, False),
    ("bf16", 4, 16, 2, 64, 5000, [4097, 5000, 97, 1000], 100, False, False),
    ("bf16", 3, 32, 1, 256, 2100, [1024, 1025, 2048], 0, False, False),     # MQA, Dh 256
    ("bf16", 5, 32, 8, 128, 700, [700, 700, 350, 1, 699], 0, True, False),  # rolling buffer
    ("bf16", 3, 8, 2, 128, 600, [600, 17, 250], 40, False, True),           # unaligned new rows
    ("f32", 3, 4, 2, 64, 400, [400, 17, 250], 40, False, False),            # general kernels
    # batches that take the even split (asserted through the workspace layout)
    ("bf16", 64, 32, 8, 128, 4096, None, 0, False, False),
    ("bf16", 64, 16, 8, 64, 8192, None, 2000, False, False),                # window
    ("bf16", 64, 32, 8, 128, 2048, None, 0, True, False),                   # rolling buffer
    ("bf16", 32, 32, 1, 128, 6000, None, 0, False, True),                   # MQA, unaligned rows
])
def test_decode_append(dtype, B, Nq, Nkv, Dh, Tcap, lens, window, rolling, unaligned):
    # one decode step whose new K/V rows are appended in the same call: the
    # cache must equal the oracle's append, and O / LSE must be bit-identical
    # to attn_kv_append followed by the decode, and match the oracle
    dev = device()
    if B >= 32:
        assert takes_even_split(B, Nq, Nkv, Dh, Tcap, window)
    if rolling:   # a full buffer: every slot holds a key
        lens = [Tcap] * B
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, dtype, seed=Dh,
                                                lens=lens)
    kn = workloads.draw((B, Nkv, 1, Dh), dtype, Dh, 21)
    vn = workloads.draw((B, Nkv, 1, Dh), dtype, Dh, 22)
    if rolling:   # token positions past the capacity: slot = position mod Tcap
        slot = np.array([Tcap + 37 * b + 5 for b in range(B)]) % Tcap
    else:
        slot = lens_a - 1
    tq, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (q, kc, vc))
    # the new token's row has never been written (an empty cache slot): NaN
    # before the call, so nothing may read its old bytes
    for b in range(B):
        tk[b, :, int(slot[b])] = float("nan")
        tv[b, :, int(slot[b])] = float("nan")
    tk2, tv2 = tk.clone(), tv.clone()
    tkn, tvn = (workloads.to_torch(a, dtype, dev) for a in (kn, vn))
    if unaligned:  # the same values 2 bytes into a buffer: the two-launch path
        buf = torch.zeros(2 * tkn.numel() + 8, dtype=tkn.dtype, device=dev)
        buf[1:1 + tkn.numel()].copy_(tkn.reshape(-1))
        buf[tkn.numel() + 3:2 * tkn.numel() + 3].copy_(tvn.reshape(-1))
        tkn_u = buf[1:1 + tkn.numel()].view(B, Nkv, Dh)
        tvn_u = buf[tkn.numel() + 3:2 * tkn.numel() + 3].view(B, Nkv, Dh)
    else:
        tkn_u, tvn_u = tkn[:, :, 0], tvn[:, :, 0]
    tl = torch.from_numpy(np.asarray(lens_a, np.int32)).to(dev)
    ts = torch.from_numpy(np.asarray(slot, np.int32)).to(dev)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    nb = tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, tch._dtype_code(tq))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    tch.attn_decode_append(tq, tkn_u, tvn_u, tk, tv, tl, ts, O, L, ws, window=window)
    # the two-launch reference on the other copy
    tch.attn_kv_append(tkn, tvn, tk2, tv2, ts, rolling=0)
    O2, L2 = torch.empty_like(O), torch.empty_like(L)
    tch.attn_decode_window(tq, tk2, tv2, tl, O2, L2, ws, window=window)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
    # bit patterns: the caches hold NaN past each length
    assert torch.equal(bits(tk), bits(tk2)) and torch.equal(bits(tv), bits(tv2))
    assert torch.equal(O, O2) and torch.equal(L, L2)
    Kr, Vr = oracle.append_ref(kc, vc, kn, vn, slot)  # bit-exact copy of the new rows
    as_bits = lambda a: a.view(np.uint16) if dtype == "bf16" else a.astype(np.float32).view(np.uint32)
    assert np.array_equal(as_bits(workloads.from_torch(tk, dtype)), as_bits(Kr))
    assert np.array_equal(as_bits(workloads.from_torch(tv, dtype)), as_bits(Vr))
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, dtype), _Lazy(Kr, dtype), _Lazy(Vr, dtype),
                               lens_a, window=window)
    got = workloads.to_f64(workloads.from_torch(O, dtype), dtype)
    say(f"decode_append {dtype} Dh={Dh} rolling={rolling} unaligned={unaligned}: "
        f"{check(got, L.cpu().numpy().astype(np.float64), Or, Lr, dtype, lens, storage_allowance=True)}")
