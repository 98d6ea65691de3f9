"""GPU parity of rotary position embedding and key-padding masks against the
float64 oracle: the cos/sin table, attn_rope (both layouts, explicit / start /
implicit positions, vector and element paths, in place), the rotating cache
append, mask packing (bit-exact), the padded prefill, chunked prefill and
decode (MFMA and general kernels, rows that see no key), and a left-padded
batch generated end to end (RoPE on q and k, padded prompt, rotating appends,
padded decode steps) against the oracle run on each unpadded sequence.

Tolerances: the table is within one fp32 ulp of the cos / sin of the
double-precision angle (plus that angle's own rounding); a rotated
bf16 element within one bf16 rounding (2^-8 relative) plus 1e-5, an fp32 one
within 2e-6 (1 + |x|); attention outputs as in the other parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, say, takes_even_split

pytestmark = pytest.mark.gpu


def _f64(t, dtype):
    return workloads.to_f64(workloads.from_torch(t, dtype), dtype)


def _check_rope(got, ref, dtype, what):
    err = np.abs(got - ref)
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    else:
        bound = 2e-6 * (1 + np.abs(ref))
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (f"{what}: err {err.flat[worst]:.3g} ref {ref.flat[worst]:.3g} "
                                  f"at {np.unravel_index(worst, err.shape)}")
    return float(err.max())


@pytest.mark.parametrize("P,Dh,base", [(4097, 128, 10000.0), (70000, 64, 500000.0), (33, 2, 10.0)])
def test_rope_table(P, Dh, base):
    got = tch.rope_table(P, Dh, base, device()).cpu().numpy().astype(np.float64)
    ref = oracle.rope_table_ref(P, Dh, base)
    # one fp32 ulp of the value, plus the double-precision rounding of the
    # angle p * theta_m itself (a few 2^-53 of it), which both sides carry
    ang = oracle.rope_angles(np.arange(P), Dh, base)
    bound = 2.0 ** -23 * np.abs(ref) + 4 * 2.0 ** -53 * (1 + np.concatenate([ang, ang], axis=-1))
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err {err.max():.3g}, worst excess {(err - bound).max():.3g}"


@pytest.mark.parametrize("dtype,Dh,style,mode", [
    ("bf16", 128, "pairs", "positions"),
    ("bf16", 128, "half", "start"),
    ("bf16", 64, "half", "none"),
    ("f32", 128, "pairs", "start"),
    ("f32", 80, "half", "positions"),
    ("bf16", 40, "pairs", "positions"),   # head size not a multiple of 16: element path
    ("bf16", 6, "half", "none"),
])
def test_rope(dtype, Dh, style, mode):
    dev = device()
    B, H, S, P = 2, 3, 37, 70000
    x = workloads.draw((B, H, S, Dh), dtype, Dh, 5)
    rng = np.random.default_rng(Dh)
    positions = start = None
    if mode == "positions":
        pos = rng.integers(0, P, (B, S)).astype(np.int32)
        pos[0, 0], pos[1, 1] = P - 1, 0
        positions = torch.from_numpy(pos).to(dev)
    elif mode == "start":
        st = np.array([0, P - S], np.int32)
        pos = st[:, None] + np.arange(S)
        start = torch.from_numpy(st).to(dev)
    else:
        pos = np.broadcast_to(np.arange(S), (B, S))
    table = tch.rope_table(P, Dh, device=dev)
    tx = workloads.to_torch(x, dtype, dev)
    y = tch.rope(tx, table, positions=positions, start=start, style=style)
    torch.cuda.synchronize()
    got = _f64(y, dtype)
    ref = oracle.rope_ref(workloads.to_f64(x, dtype), pos, style=style)
    e = _check_rope(got, ref, dtype, (dtype, Dh, style, mode))
    # in place gives the same bits
    tch.rope(tx, table, positions=positions, start=start, style=style, out=tx)
    torch.cuda.synchronize()
    assert torch.equal(tx, y)
    say(f"rope {dtype} Dh={Dh} {style} {mode}: max err {e:.3g}")


def test_rope_unaligned_buffers_take_the_element_path():
    # a view 2 bytes into a buffer: the 16-byte vector path is not allowed,
    # the element path must give the same bits
    dev = device()
    B, H, S, Dh, P = 2, 4, 50, 128, 1000
    x = workloads.to_torch(workloads.draw((B, H, S, Dh), "bf16", 3, 5), "bf16", dev)
    table = tch.rope_table(P, Dh, device=dev)
    aligned = tch.rope(x, table, style="half")
    n = x.numel()
    buf = torch.zeros(2 * n + 16, dtype=torch.bfloat16, device=dev)
    xin = buf[1:1 + n].view(B, H, S, Dh)
    yout = buf[n + 3:2 * n + 3].view(B, H, S, Dh)
    xin.copy_(x)
    tch.rope(xin, table, style="half", out=yout)
    torch.cuda.synchronize()
    assert torch.equal(yout, aligned)


@pytest.mark.parametrize("dtype,Dh,Snew,Tcap,pos,rolling,explicit,style", [
    ("bf16", 128, 3, 50, [0, 47], 0, False, "pairs"),
    ("bf16", 128, 45, 20, [3, 40], 1, False, "half"),   # longer than the buffer
    ("f32", 64, 5, 16, [11, 2], 1, True, "pairs"),
    ("bf16", 40, 4, 9, [2, 5], 0, True, "half"),        # element path
])
def test_kv_append_rope(dtype, Dh, Snew, Tcap, pos, rolling, explicit, style):
    dev = device()
    B, Nkv, P = 2, 3, 4096
    kc = workloads.draw((B, Nkv, Tcap, Dh), dtype, 6, 1)
    vc = workloads.draw((B, Nkv, Tcap, Dh), dtype, 6, 2)
    kn = workloads.draw((B, Nkv, Snew, Dh), dtype, 6, 3)
    vn = workloads.draw((B, Nkv, Snew, Dh), dtype, 6, 4)
    positions = (np.random.default_rng(Dh).integers(0, P, (B, Snew)).astype(np.int32)
                 if explicit else None)
    tk, tv, tkn, tvn = (workloads.to_torch(a, dtype, dev) for a in (kc, vc, kn, vn))
    table = tch.rope_table(P, Dh, device=dev)
    tch.attn_kv_append_rope(tkn, tvn, tk, tv, torch.tensor(pos, dtype=torch.int32, device=dev),
                            table, positions=None if positions is None else
                            torch.from_numpy(positions).to(dev), rolling=rolling, style=style)
    torch.cuda.synchronize()
    Kr, _ = oracle.append_rope_ref(workloads.to_f64(kc, dtype), workloads.to_f64(vc, dtype),
                                   workloads.to_f64(kn, dtype), workloads.to_f64(vn, dtype), pos,
                                   positions=positions, rolling=bool(rolling), style=style)
    _check_rope(_f64(tk, dtype), Kr, dtype, "K cache")
    # V rows are copied bit for bit, and so are the untouched K rows
    _, Vbits = oracle.append_ref(kc, vc, kn, vn, pos, rolling=bool(rolling))
    assert np.array_equal(workloads.from_torch(tv, dtype), Vbits)
    marker, _ = oracle.append_ref(np.zeros((B, Nkv, Tcap, 1)), np.zeros((B, Nkv, Tcap, 1)),
                                  np.ones((B, Nkv, Snew, 1)), np.ones((B, Nkv, Snew, 1)), pos,
                                  rolling=bool(rolling))
    kept = marker[..., 0] == 0
    assert np.array_equal(workloads.from_torch(tk, dtype)[kept], kc[kept])


@pytest.mark.parametrize("B,T", [(3, 1), (2, 64), (4, 65), (2, 1000)])
def test_pack_key_mask(B, T):
    dev = device()
    m = workloads.key_mask(B, T, hole_frac=0.5, seed=T)
    expect = np.zeros((B, (T + 63) // 64), np.uint64)
    for b in range(B):
        for j in np.flatnonzero(m[b]):
            expect[b, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    got = tch.pack_key_mask(torch.from_numpy(m).to(dev)).cpu().numpy().view(np.uint64)
    assert np.array_equal(got, expect)
    # uint8 flags: any nonzero byte is a real token
    u8 = (m.astype(np.uint8) * np.uint8(37))
    got8 = tch.pack_key_mask(torch.from_numpy(u8).to(dev)).cpu().numpy().view(np.uint64)
    assert np.array_equal(got8, expect)


def _split_dead(O, L, Or, Lr, what):
    """Rows that see no key must be exactly O = 0, LSE = -inf; returns the others."""
    dead = np.isneginf(Lr)
    assert np.all(O[dead] == 0), f"{what}: row without keys is not zero"
    assert np.all(np.isneginf(L[dead])), f"{what}: row without keys has a finite LSE"
    return ~dead, int(dead.sum())


@pytest.mark.parametrize("dtype,B,Nq,Nkv,S,Dh,causal,window,pads,holes,block", [
    ("bf16", 3, 8, 2, 300, 128, True, 0, [0, 70, 150], 0.1, None),   # left padding, dead rows
    ("bf16", 2, 4, 4, 257, 128, True, 100, [5, 0], 0.3, None),
    ("bf16", 2, 4, 1, 200, 64, True, 0, None, 0.0, (64, 128)),      # a whole tile of padding
    ("bf16", 1, 2, 2, 130, 256, False, 0, None, 0.5, None),
    ("bf16", 2, 2, 1, 90, 80, True, 0, [10, 0], 0.2, None),         # general kernel
    ("f32", 2, 4, 2, 100, 64, True, 7, [0, 30], 0.2, None),
])
def test_prefill_padded(dtype, B, Nq, Nkv, S, Dh, causal, window, pads, holes, block):
    dev = device()
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=S)
    m = workloads.key_mask(B, S, pads=pads, hole_frac=holes, seed=S, block=block)
    tq, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (q, k, v))
    O, L = tch.prefill(tq, tk, tv, causal=causal, window=window,
                       key_mask=torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og, Lg = _f64(O, dtype), L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(a, dtype) for a in (q, k, v)), causal=causal,
                                  window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "prefill")
    errs = check(Og[live], Lg[live], Or[live], Lr[live], dtype, (dtype, S, Dh, pads),
                 storage_allowance=True)
    say(f"prefill padded {dtype} S={S} Dh={Dh} dead rows {n_dead}: {errs}")


@pytest.mark.parametrize("B,Nq,Nkv,Sq,Tcap,lens,window,pads,holes", [
    (2, 8, 2, 100, 700, [100, 613], 0, [0, 200], 0.1),
    (1, 32, 8, 257, 2048, [2048], 300, None, 0.3),
    (2, 4, 1, 40, 300, [40, 290], 0, [60, 0], 0.0),   # sequence 0: every row sees padding only
])
def test_prefill_cache_padded(B, Nq, Nkv, Sq, Tcap, lens, window, pads, holes):
    dev = device()
    lens_a, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, 128, Tcap, lens, "bf16", seed=Sq)
    m = workloads.key_mask(B, Tcap, pads=pads, hole_frac=holes, seed=Sq)
    tQ, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (Q, kc, vc))
    O, L = tch.prefill_cache(tQ, tk, tv, torch.from_numpy(lens_a).to(dev), window=window,
                             key_mask=torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og, Lg = _f64(O, "bf16"), L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.chunk_ref(workloads.to_f64(Q, "bf16"), workloads.to_f64(kc, "bf16"),
                              workloads.to_f64(vc, "bf16"), lens_a, window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "chunk")
    errs = check(Og[live], Lg[live], Or[live], Lr[live], "bf16", (Sq, lens, pads),
                 storage_allowance=True)
    say(f"prefill_cache padded Sq={Sq} dead rows {n_dead}: {errs}")


class _Lazy:
    def __init__(self, arr, dtype):
        self.arr, self.dtype, self.shape = arr, dtype, arr.shape

    def __getitem__(self, idx):
        return workloads.to_f64(self.arr[idx], self.dtype)


@pytest.mark.parametrize("dtype,B,Nq,Nkv,Dh,Tcap,lens,window,pads,holes,block", [
    ("bf16", 6, 32, 8, 128, 3000, [1, 31, 33, 2000, 3000, 100], 0, [0, 0, 40, 500, 2999, 0], 0.2,
     None),                                              # sequence 2 sees padding only
    ("bf16", 16, 32, 8, 128, 16384, None, 1000, None, 0.5, (64, 2048)),
    ("bf16", 4, 16, 2, 64, 5000, [4097, 5000, 97, 1000], 0, [100, 0, 0, 999], 0.1, None),
    ("bf16", 3, 32, 1, 128, 2100, [1024, 1025, 2048], 0, [0, 1000, 0], 0.3, None),  # MQA
    ("bf16", 3, 4, 2, 256, 700, [700, 17, 250], 40, [0, 20, 220], 0.2, None),
    ("f32", 3, 4, 2, 64, 400, [400, 17, 250], 40, [0, 20, 100], 0.2, None),         # general
    # grids large enough for the even split (ranges of steps over all sequences,
    # the mask's flag words staged per piece); one sequence sees padding only
    ("bf16", 64, 32, 8, 128, 4096, None, 0, [(37 * i) % 900 for i in range(63)] + [4096], 0.1,
     None),
    ("bf16", 32, 32, 1, 128, 8192, None, 0, [(101 * i) % 2500 for i in range(32)], 0.2, None),
    ("bf16", 48, 16, 4, 64, 6000, None, 0, [(53 * i) % 1200 for i in range(48)], 0.1, None),
    ("bf16", 64, 8, 8, 128, 8192, None, 3000, [(71 * i) % 4000 for i in range(64)], 0.3, None),
])
def test_decode_padded(dtype, B, Nq, Nkv, Dh, Tcap, lens, window, pads, holes, block):
    dev = device()
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, dtype, seed=Tcap,
                                                lens=lens)
    m = workloads.key_mask(B, Tcap, pads=pads, hole_frac=holes, seed=Tcap, block=block)
    tq, tk, tv = (workloads.to_torch(a, dtype, dev) for a in (q, kc, vc))
    if B >= 32:
        assert takes_even_split(B, Nq, Nkv, Dh, Tcap, window)
    O, L = tch.decode(tq, tk, tv, torch.from_numpy(lens_a).to(dev), window=window,
                      key_mask=torch.from_numpy(m).to(dev))
    torch.cuda.synchronize()
    Og, Lg = _f64(O, dtype), L.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, dtype), _Lazy(kc, dtype), _Lazy(vc, dtype),
                               lens_a, window=window, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "decode")
    errs = check(Og[live], Lg[live], Or[live], Lr[live], dtype, (dtype, Tcap, pads),
                 storage_allowance=True)
    say(f"decode padded {dtype} Dh={Dh} Tcap={Tcap} dead rows {n_dead}: {errs}")


def _bf16_round(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x.astype(np.float32))).astype(
        np.float64)


@pytest.mark.parametrize("style", ["half", "pairs"])
def test_left_padded_generation_with_rope(style):
    # three prompts of 50, 120 and 200 tokens left-padded to 200, then 24
    # tokens generated one at a time; positions count from each prompt's first
    # token.  Every output row of a real token must match the oracle run on
    # that sequence alone (RoPE'd q and k rounded to bf16 as they are stored);
    # rows of padding tokens see no key and are zero.
    dev = device()
    Nq, Nkv, Dh, P0, steps = 32, 8, 128, 200, 24
    real = [50, 120, 200]
    B, T = len(real), P0 + steps
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, T, Dh, "bf16", seed=93)
    mask = np.zeros((B, T), bool)
    for b, n in enumerate(real):
        mask[b, P0 - n:] = True
    pos = workloads.token_positions(mask)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    tpos = torch.from_numpy(pos).to(dev)
    tmask = torch.from_numpy(mask).to(dev)
    table = tch.rope_table(T, Dh, device=dev)
    Kc = torch.zeros((B, Nkv, T, Dh), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    # prompt: rotated keys into the cache, rotated queries against it
    tch.attn_kv_append_rope(tk[:, :, :P0].contiguous(), tv[:, :, :P0].contiguous(), Kc, Vc, zero,
                            table, positions=tpos[:, :P0].contiguous(), style=style)
    qp = tch.rope(tq[:, :, :P0].contiguous(), table, positions=tpos[:, :P0].contiguous(),
                  style=style)
    Op, Lp = tch.prefill_cache(qp, Kc, Vc, torch.full((B,), P0, dtype=torch.int32, device=dev),
                               key_mask=tmask)
    outs, lses = [Op], [Lp]
    for t in range(P0, T):
        at = torch.full((B,), t, dtype=torch.int32, device=dev)
        tch.attn_kv_append_rope(tk[:, :, t:t + 1].contiguous(), tv[:, :, t:t + 1].contiguous(), Kc,
                                Vc, at, table, positions=tpos[:, t:t + 1].contiguous(), style=style)
        qt = tch.rope(tq[:, :, t:t + 1].contiguous(), table, positions=tpos[:, t:t + 1].contiguous(),
                      style=style)
        O, L = tch.decode(qt[:, :, 0].contiguous(), Kc, Vc, at + 1, key_mask=tmask)
        outs.append(O[:, :, None])
        lses.append(L[:, :, None])
    torch.cuda.synchronize()
    Og = _f64(torch.cat(outs, dim=2), "bf16")
    Lg = torch.cat(lses, dim=2).cpu().numpy().astype(np.float64)
    qf, kf, vf = (workloads.to_f64(a, "bf16") for a in (q, k, v))
    for b, n in enumerate(real):
        r = P0 - n
        own = np.arange(T - r)[None, :]
        qb = _bf16_round(oracle.rope_ref(qf[b:b + 1, :, r:], own, style=style))
        kb = _bf16_round(oracle.rope_ref(kf[b:b + 1, :, r:], own, style=style))
        Or, Lr = oracle.attention_ref(qb, kb, vf[b:b + 1, :, r:])
        errs = check(Og[b:b + 1, :, r:], Lg[b:b + 1, :, r:], Or, Lr, "bf16", (style, b),
                     storage_allowance=True)
        assert np.all(Og[b, :, :r] == 0) and np.all(np.isneginf(Lg[b, :, :r]))
        say(f"padded generation {style} prompt {n}: {errs}")


def test_bench_shapes_sampled_rows():
    # the shapes bench.py --rope-padding times, on seeded sampled rows:
    # RoPE in place on 32 x 32768 x 128 queries (half layout), and the padded
    # prefill of 4 x 8192 tokens, 32/8 heads, left padding 0/1024/2048/4096
    dev = device()
    B, H, S, Dh = 1, 32, 32768, 128
    x = workloads.draw((B, H, S, Dh), "bf16", 0, 0)
    tx = workloads.to_torch(x, "bf16", dev)
    tch.attn_rope(tx, tx, tch.rope_table(S, Dh, device=dev), style="half")
    rows = workloads.sample_rows(B, H, S, 64, seed=7, forced_rows=(0, S - 1))
    idx = tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    got = workloads.to_f64(workloads.from_torch(tx[idx], "bf16"), "bf16")
    sel = np.stack([workloads.to_f64(x[b, h, i], "bf16") for b, h, i in rows])
    ref = oracle.rope_ref(sel[None, None], np.array([[i for _, _, i in rows]]), style="half")[0, 0]
    _check_rope(got, ref, "bf16", "rope, bench shape")
    del tx

    B, Nq, Nkv, S = 4, 32, 8, 8192
    pads = [0, 1024, 2048, 4096]
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=0)
    m = workloads.key_mask(B, S, pads=pads)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    O, L = tch.prefill(tq, tk, tv, key_mask=torch.from_numpy(m).to(dev))
    rows = workloads.sample_rows(B, Nq, S, 256, seed=8,
                                 forced_rows=(0, 1023, 1024, 2047, 2048, 4095, 4096, 8191))
    idx = tuple(torch.tensor(c, device=dev) for c in zip(*rows))
    Og = workloads.to_f64(workloads.from_torch(O[idx], "bf16"), "bf16")
    Lg = L[idx].cpu().numpy().astype(np.float64)
    del tq, tk, tv, O, L

    class Lazy:
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __getitem__(self, i):
            return workloads.to_f64(self.a[i], "bf16")

    Or, Lr = oracle.chunk_ref(Lazy(q), Lazy(k), Lazy(v), [S] * B, rows=rows, key_mask=m)
    live, n_dead = _split_dead(Og, Lg, Or, Lr, "padded prefill, bench shape")
    errs = check(Og[live], Lg[live], Or[live], Lr[live], "bf16", "padded prefill, bench shape")
    say(f"bench shapes: padded prefill {len(rows)} rows ({n_dead} without keys): {errs}")
