"""GPU parity: the HIP library against the float64 oracle on seeded inputs.

The named workloads run at their full sizes in the launch configuration the
benchmark times; long ones are checked on seeded sampled rows (plus forced
rows at the boundaries), the others on every output element.  Edge cases
cover ragged lengths, every grouped-query layout the kernels specialise, the
window boundary, non-causal attention and the general kernel.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_causal_head_amd as tch
import workloads
from helpers import check, device, run_decode, run_prefill, say

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _prefill_case(cfg, seed=0):
    q, k, v = workloads.prefill_inputs(cfg["B"], cfg["Nq"], cfg["Nkv"], cfg["S"], cfg["Dh"],
                                       cfg["dtype"], seed=seed)
    return q, k, v


# --- the named workloads ----------------------------------------------------

def test_tiny_fp32_full():
    cfg = W["tiny_fp32_b1_h2_s5_d4"]
    q, k, v = _prefill_case(cfg)
    O, L = run_prefill(q, k, v, "f32", True, 0, cfg["scale"])
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "f32") for x in (q, k, v)),
                                  causal=True, scale=cfg["scale"])
    say(f"tiny fp32 errors {check(O, L, Or, Lr, 'f32', 'tiny')}")


def test_mha_s1024_full():
    cfg = W["mha_bf16_b2_h32_s1024_d128"]
    q, k, v = _prefill_case(cfg)
    O, L = run_prefill(q, k, v, "bf16", True, 0, None)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)), causal=True)
    say(f"mha s1024 errors {check(O, L, Or, Lr, 'bf16', 'mha_s1024')}")


def _sampled(cfg):
    q, k, v = _prefill_case(cfg)
    say(f"inputs ready {cfg['S']}")
    O, L = run_prefill(q, k, v, "bf16", True, cfg["window"], None)
    tr = workloads.sample_rows(cfg["B"], cfg["Nq"], cfg["S"], cfg["sample"], seed=1,
                               forced_rows=cfg["forced_rows"])
    Qf, Kf, Vf = (workloads.to_f64(x, "bf16") for x in (q, k, v))
    Or, Lr = oracle.attention_rows_ref(Qf, Kf, Vf, tr, causal=True, window=cfg["window"])
    idx = tuple(np.array(tr).T)
    return check(O[idx], L[idx], Or, Lr, "bf16", cfg)


def test_mha_s32768_sampled_rows():
    say(f"mha s32768 errors {_sampled(W['mha_bf16_b1_h32_s32768_d128'])}")


def test_gqa_window_s8192_sampled_rows():
    say(f"gqa window errors {_sampled(W['gqa_bf16_b4_h32kv8_s8192_w4096_d128'])}")


def test_decode_b64_full():
    cfg = W["decode_bf16_b64_h32kv8_t32768_d128"]
    lens, q, kc, vc = workloads.decode_inputs(cfg["B"], cfg["Nq"], cfg["Nkv"], cfg["Dh"],
                                              cfg["Tcap"], cfg["len_lo"], cfg["len_hi"])
    say(f"decode inputs ready, sum(lens)={int(lens.sum())}")
    O, L = run_decode(q, kc, vc, lens, "bf16")
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), _LazyF64(kc), _LazyF64(vc), lens)
    say(f"decode errors {check(O, L, Or, Lr, 'bf16', 'decode')}")


class _LazyF64:
    """Widens bf16 cache slices on access, so the full cache is never copied."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape
        self._last = (None, None)

    def __getitem__(self, idx):
        key = repr(idx)
        if self._last[0] != key:  # consecutive query heads share a K/V slice
            self._last = (key, workloads.to_f64(self.bits[idx], "bf16"))
        return self._last[1]


# --- prefill edge cases -------------------------------------------------------

@pytest.mark.parametrize("B,Nq,Nkv,S,causal,window", [
    (1, 1, 1, 1, True, 0),        # one token
    (1, 4, 4, 2, True, 0),
    (2, 2, 2, 63, True, 0),       # below one key tile
    (1, 2, 2, 65, True, 0),       # one key past a tile
    (1, 4, 1, 200, True, 0),      # MQA, ragged
    (2, 8, 2, 257, True, 0),      # GQA 4, ragged past a query tile
    (1, 6, 3, 300, True, 0),      # GQA 2
    (1, 8, 1, 129, True, 0),      # GQA 8 (two head subgroups)
    (1, 3, 1, 100, True, 0),      # GQA 3 (odd group)
    (1, 4, 4, 700, True, 1),      # window 1: only the diagonal
    (1, 4, 2, 700, True, 64),     # window equal to a tile
    (2, 8, 2, 600, True, 100),    # window not aligned to tiles
    (1, 2, 2, 513, True, 600),    # window longer than the sequence
    (1, 4, 4, 130, False, 0),     # non-causal
    (1, 4, 2, 77, False, 0),      # non-causal GQA ragged
])
def test_prefill_edge_cases_bf16(B, Nq, Nkv, S, causal, window):
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, 128, "bf16", seed=S + 7 * Nq)
    O, L = run_prefill(q, k, v, "bf16", causal, window, None)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)),
                                  causal=causal, window=window)
    check(O, L, Or, Lr, "bf16", (B, Nq, Nkv, S, causal, window), storage_allowance=True)


@pytest.mark.parametrize("Dh", [64, 256])
@pytest.mark.parametrize("B,Nq,Nkv,S,causal,window", [
    (1, 2, 2, 1, True, 0),
    (2, 4, 4, 65, True, 0),       # one key past a tile
    (1, 8, 2, 300, True, 0),      # GQA 4, ragged
    (1, 6, 3, 257, True, 0),      # GQA 2, past a query tile
    (1, 4, 1, 200, True, 0),      # MQA
    (2, 8, 2, 600, True, 100),    # window not aligned to tiles
    (1, 4, 4, 700, True, 1),      # window 1
    (1, 4, 2, 130, False, 0),     # non-causal
])
def test_prefill_mfma_head_sizes(Dh, B, Nq, Nkv, S, causal, window):
    # the MFMA kernel at head sizes 64 and 256 (same cases as at 128)
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=S + Dh)
    O, L = run_prefill(q, k, v, "bf16", causal, window, None)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)),
                                  causal=causal, window=window)
    check(O, L, Or, Lr, "bf16", (Dh, B, Nq, Nkv, S, causal, window), storage_allowance=True)


@pytest.mark.parametrize("Dh,S,Nq,Nkv,window,dtype", [
    (4, 5, 2, 2, 0, "f32"),
    (64, 100, 4, 2, 0, "f32"),
    (128, 70, 4, 1, 20, "f32"),
    (256, 33, 2, 2, 0, "f32"),
    (1, 9, 2, 1, 3, "f32"),
    (64, 90, 4, 2, 0, "bf16"),
    (80, 50, 2, 2, 7, "bf16"),
    (256, 40, 4, 4, 0, "bf16"),
])
def test_prefill_general_kernel(Dh, S, Nq, Nkv, window, dtype):
    q, k, v = workloads.prefill_inputs(1, Nq, Nkv, S, Dh, dtype, seed=Dh + S)
    scale = 0.5 / math.sqrt(Dh)
    O, L = run_prefill(q, k, v, dtype, True, window, scale)
    Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, dtype) for x in (q, k, v)),
                                  causal=True, window=window, scale=scale)
    check(O, L, Or, Lr, dtype, (Dh, S, dtype), storage_allowance=True)


def test_prefill_scale_is_respected():
    q, k, v = workloads.prefill_inputs(1, 4, 2, 150, 128, "bf16", seed=3)
    for scale in (0.02, 0.3):
        O, L = run_prefill(q, k, v, "bf16", True, 0, scale)
        Or, Lr = oracle.attention_ref(*(workloads.to_f64(x, "bf16") for x in (q, k, v)),
                                      causal=True, scale=scale)
        check(O, L, Or, Lr, "bf16", scale, storage_allowance=True)


# --- properties on the GPU ----------------------------------------------------

def test_causality_bitwise_on_gpu():
    # perturbing the last token leaves every earlier output row bit-identical
    q, k, v = workloads.prefill_inputs(1, 8, 2, 333, 128, "bf16", seed=11)
    O1, L1 = run_prefill(q, k, v, "bf16", True, 0, None)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x, other in ((q2, 12), (k2, 13), (v2, 14)):
        x[:, :, -1] = workloads.draw(x[:, :, -1].shape, "bf16", 99, other)
    O2, L2 = run_prefill(q2, k2, v2, "bf16", True, 0, None)
    assert np.array_equal(O1[:, :, :-1], O2[:, :, :-1])
    assert np.array_equal(L1[:, :, :-1], L2[:, :, :-1])
    assert not np.array_equal(O1[:, :, -1], O2[:, :, -1])


def test_prefill_deterministic():
    q, k, v = workloads.prefill_inputs(2, 8, 2, 1000, 128, "bf16", seed=5)
    O1, L1 = run_prefill(q, k, v, "bf16", True, 300, None)
    O2, L2 = run_prefill(q, k, v, "bf16", True, 300, None)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_gqa_matches_mha_on_repeated_kv():
    q, k, v = workloads.prefill_inputs(1, 8, 2, 400, 128, "bf16", seed=21)
    O, L = run_prefill(q, k, v, "bf16", True, 0, None)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    Om, Lm = run_prefill(q, kr, vr, "bf16", True, 0, None)
    np.testing.assert_allclose(O, Om, atol=1e-6)
    np.testing.assert_allclose(L, Lm, atol=1e-6)


def test_window_covering_sequence_equals_causal():
    q, k, v = workloads.prefill_inputs(1, 4, 4, 300, 128, "bf16", seed=8)
    Oc, Lc = run_prefill(q, k, v, "bf16", True, 0, None)
    Ow, Lw = run_prefill(q, k, v, "bf16", True, 300, None)
    np.testing.assert_allclose(Oc, Ow, atol=1e-6)
    np.testing.assert_allclose(Lc, Lw, atol=1e-6)


def test_lse_may_be_null():
    dev = device()
    q, k, v = workloads.prefill_inputs(1, 4, 4, 100, 128, "bf16", seed=2)
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
    O = torch.empty_like(tq)
    tch.attn_prefill(tq, tk, tv, O, None)
    torch.cuda.synchronize()
    O_ref, _ = run_prefill(q, k, v, "bf16", True, 0, None)
    assert np.array_equal(workloads.to_f64(workloads.from_torch(O, "bf16"), "bf16"), O_ref)


def test_bad_flags_rejected_with_real_tensors():
    dev = device()
    t = torch.zeros(1, 4, 16, 128, dtype=torch.bfloat16, device=dev)
    O = torch.empty_like(t)
    with pytest.raises(tch.AttnError) as e:
        tch.attn_prefill(t, t, t, O, None, causal=0, window=4)
    assert e.value.status == tch.ATTN_EINVAL
    k3 = torch.zeros(1, 3, 16, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tch.AttnError) as e:
        tch.attn_prefill(t, k3, k3, O, None)
    assert e.value.status == tch.ATTN_EGQA


# --- decode edge cases --------------------------------------------------------

@pytest.mark.parametrize("B,Nq,Nkv,Tcap,lens", [
    (4, 32, 8, 3000, [1, 2, 1023, 3000]),           # length 1, chunk edges, full cache
    (3, 8, 8, 2100, [1024, 1025, 2048]),            # MHA (G = 1)
    (2, 16, 8, 700, [700, 63]),                      # G = 2
    (2, 16, 2, 5000, [4097, 5000]),                 # G = 8
    (2, 4, 1, 333, [333, 17]),                       # MQA G = 4
    (2, 6, 2, 300, [300, 5]),                        # G = 3: general kernel
    (1, 4, 4, 65, [65]),
])
def test_decode_edge_cases(B, Nq, Nkv, Tcap, lens):
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, 128, Tcap, 1, Tcap, seed=Tcap,
                                                lens=lens)
    O, L = run_decode(q, kc, vc, lens_a, "bf16")
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), workloads.to_f64(kc, "bf16"),
                               workloads.to_f64(vc, "bf16"), lens_a)
    check(O, L, Or, Lr, "bf16", (B, Nq, Nkv, Tcap, lens), storage_allowance=True)


# wavefronts of the even split's partial grid, at most (its workspace slots
# are B * Nkv + EVEN_WAVES; 16 or more query heads per K/V head use half as
# many wavefronts); it serves up to 64 sequences (at head size 256 only
# with at most 16 query heads per K/V head) when the chunk mode's grid would
# have at least EVEN_WAVES / 2 items
EVEN_WAVES = 1024


def _decode_chunk(B, Nkv, Tcap, G):
    # the host's choice of keys per chunk, restated: the longest candidate that
    # gives at least 2048 (sequence, K/V head, chunk) items at full length,
    # 1024 with 16 or more query heads per K/V head, but not shorter than 640
    # keys (224 with 16 or more query heads per K/V head)
    floor = 224 if G >= 16 else 640
    for ch in (1792, 1152, 896, 640, 384, 224, 160, 96):
        if ch <= floor or B * Nkv * -(-Tcap // ch) >= (1024 if G >= 16 else 2048):
            return ch
    return floor


@pytest.mark.parametrize("B,Nq,Nkv,Tcap,ch", [
    (16, 32, 8, 3000, 640),     # the item count alone would ask for 160
    (9, 8, 1, 32768, 640),      # few long sequences: 96 by the item count
    (16, 32, 8, 12000, 640),
    (16, 32, 8, 16384, 896),
    (24, 32, 8, 16384, 1152),
    (16, 32, 2, 16384, 384),    # 16 query heads per K/V head: 1024 items
    (9, 32, 1, 3000, 224),      # MQA, the floor for wide groups
    (64, 32, 1, 32768, 1792),   # MQA with 32 query heads
    (80, 32, 8, 3000, 896),     # more than 64 sequences: chunk mode without a mask
])
@pytest.mark.parametrize("masked", [False, True])
def test_decode_chunk_sizes(B, Nq, Nkv, Tcap, ch, masked):
    # every chunk length the host can pick, with lengths on and around chunk
    # edges; the workspace size shows which chunk length was taken.  Without a
    # key-padding mask the larger grids of up to 64 sequences run the even
    # split (the workspace also holds its slots); an all-true mask keeps the
    # same case in chunk mode.
    assert _decode_chunk(B, Nkv, Tcap, Nq // Nkv) == ch
    ws = tch.attn_decode_workspace_bytes(B, Nq, Nkv, 128, Tcap, tch.ATTN_BF16)
    slots = B * Nkv * -(-Tcap // ch)
    seg = 0
    if B <= 64 and slots >= EVEN_WAVES // 2:
        slots = max(slots, B * Nkv + EVEN_WAVES)
        seg = B * Nkv * 2 * 4  # the first and last range of each (sequence, K/V head)
    assert ws == slots * (Nq // Nkv) * (128 + 2) * 4 + seg
    rng = np.random.default_rng(Tcap + B)
    lens = rng.integers(1, Tcap, B, endpoint=True)
    lens[:8] = [1, 31, 32, 33, ch - 1, ch, ch + 1, Tcap]
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, 128, Tcap, 1, Tcap, seed=ch,
                                                lens=lens)
    if masked:
        dev = device()
        tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
        tl = torch.from_numpy(np.asarray(lens_a, dtype=np.int32)).to(dev)
        Ot, Lt = tch.decode(tq, tk, tv, tl, key_mask=torch.ones(B, Tcap, dtype=torch.bool, device=dev))
        torch.cuda.synchronize()
        O = workloads.to_f64(workloads.from_torch(Ot, "bf16"), "bf16")
        L = Lt.cpu().numpy().astype(np.float64)
        del tq, tk, tv
    else:
        O, L = run_decode(q, kc, vc, lens_a, "bf16")
    rows = [(b, h) for b in range(8) for h in (0, Nq - 1)]
    rows += [(int(b), int(h)) for b, h in zip(rng.integers(8, B, 32), rng.integers(0, Nq, 32))]
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), _LazyF64(kc), _LazyF64(vc), lens_a,
                               rows=rows)
    Os = np.stack([O[b, h] for b, h in rows])
    Ls = np.array([L[b, h] for b, h in rows])
    say(f"chunk {ch}: errors {check(Os, Ls, Or, Lr, 'bf16', (B, Nkv, Tcap, ch), storage_allowance=True)}")


def _even_lens(kind, B, Tcap, rng):
    if kind == "short":          # many whole segments inside one wavefront's range
        return rng.integers(1, 100, B, endpoint=True)
    if kind == "one_long":       # one segment split over many more than 64 ranges
        lens = np.ones(B, dtype=np.int64)
        lens[B // 2] = Tcap
        return lens
    return rng.integers(1, Tcap, B, endpoint=True)


@pytest.mark.parametrize("Dh,B,Nq,Nkv,Tcap,kind,window", [
    (128, 64, 32, 8, 100, "short", 0),        # 50 of the 1024 wavefronts in use
    (128, 64, 32, 8, 3000, "ragged", 0),
    (128, 64, 32, 8, 5000, "ragged", 100),    # window: segments start mid-step
    (128, 37, 32, 1, 4000, "ragged", 0),      # 32 query heads per K/V head (two blocks)
    (128, 16, 4, 1, 60000, "one_long", 0),    # a row's pieces run past one merge round
    (128, 16, 32, 1, 60000, "one_long", 0),
    (64, 45, 16, 4, 2500, "ragged", 0),
    (64, 64, 32, 2, 3000, "ragged", 777),
    (256, 64, 32, 8, 3000, "ragged", 0),      # head size 256: one block of query heads
    (256, 16, 16, 1, 20000, "one_long", 300),
])
def test_decode_even_split(Dh, B, Nq, Nkv, Tcap, kind, window):
    # up to 64 sequences without a key-padding mask: the visible steps of all
    # (sequence, K/V head) pairs are cut into wavefront ranges (64 : 55 for
    # wavefronts on even and odd XCDs); ranges
    # that hold several segments, segments split over many ranges, windows,
    # and totals too small to fill the grid
    rng = np.random.default_rng(Tcap + B + Dh)
    lens = _even_lens(kind, B, Tcap, rng)
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, seed=B + Dh,
                                                lens=lens)
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
    tl = torch.from_numpy(np.asarray(lens_a, dtype=np.int32)).to(dev)
    Ot, Lt = tch.decode(tq, tk, tv, tl, window=window)
    torch.cuda.synchronize()
    O = workloads.to_f64(workloads.from_torch(Ot, "bf16"), "bf16")
    L = Lt.cpu().numpy().astype(np.float64)
    rows = [(b, h) for b in range(B) for h in (0, Nq - 1)]
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), _LazyF64(kc), _LazyF64(vc), lens_a,
                               window=window, rows=rows)
    Os = np.stack([O[b, h] for b, h in rows])
    Ls = np.array([L[b, h] for b, h in rows])
    say(f"even split {kind}: errors {check(Os, Ls, Or, Lr, 'bf16', (Dh, B, Nq, Nkv, Tcap, window), storage_allowance=True)}")


@pytest.mark.parametrize("Dh,B,Nq,Nkv,Tcap,lens", [
    (64, 4, 16, 4, 3000, [1, 33, 2999, 3000]),
    (256, 4, 16, 4, 3000, [1, 33, 2999, 3000]),
    (128, 3, 32, 1, 2500, [2500, 97, 1]),        # MQA with 32 query heads: two head blocks
    (128, 2, 24, 1, 700, [700, 300]),            # 24 heads: second block partly empty
    (64, 2, 32, 1, 900, [900, 450]),
    (256, 2, 64, 2, 900, [1, 900]),              # G = 32 at head size 256
])
def test_decode_mfma_head_sizes_and_groups(Dh, B, Nq, Nkv, Tcap, lens):
    lens_a, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, seed=Dh + Nq,
                                                lens=lens)
    O, L = run_decode(q, kc, vc, lens_a, "bf16")
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "bf16"), workloads.to_f64(kc, "bf16"),
                               workloads.to_f64(vc, "bf16"), lens_a)
    check(O, L, Or, Lr, "bf16", (Dh, B, Nq, Nkv, Tcap, lens), storage_allowance=True)
    assert tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, tch.ATTN_BF16) > 0


@pytest.mark.parametrize("Dh", [4, 64, 128])
def test_decode_fp32(Dh):
    lens_a, q, kc, vc = workloads.decode_inputs(3, 4, 2, Dh, 50, 1, 50, dtype="f32", seed=Dh,
                                                lens=[50, 1, 20])
    O, L = run_decode(q, kc, vc, lens_a, "f32")
    Or, Lr = oracle.decode_ref(workloads.to_f64(q, "f32"), workloads.to_f64(kc, "f32"),
                               workloads.to_f64(vc, "f32"), lens_a)
    check(O, L, Or, Lr, "f32", Dh)


def test_decode_equals_prefill_row():
    # a decode step of row t-1 against t cached keys reproduces prefill row t-1
    S = 1500
    q, k, v = workloads.prefill_inputs(2, 8, 2, S, 128, "bf16", seed=31)
    Op, Lp = run_prefill(q, k, v, "bf16", True, 0, None)
    for t in (1, 64, 1024, 1025, S):
        lens = np.array([t, t], dtype=np.int32)
        Od, Ld = run_decode(np.ascontiguousarray(q[:, :, t - 1]), k, v, lens, "bf16")
        np.testing.assert_allclose(Od, Op[:, :, t - 1], atol=2e-2)
        np.testing.assert_allclose(Ld, Lp[:, :, t - 1], atol=2e-3)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("Dh,Nkv,window,append", [
    (64, 8, 0, False), (128, 8, 0, False), (256, 8, 0, False), (128, 1, 0, False),
    (128, 8, 4096, False), (128, 8, 0, True), (64, 8, 0, True),
])
def test_decode_repeat_bitwise_full_size(Dh, Nkv, window, append):
    # The split-K decode kernel streams each chunk through two LDS stages with
    # no workgroup barrier, so a copy into a stage must wait for that stage's
    # reads; a copy that overtook them would change the rows it raced on from
    # one call to the next.  At the decode workload's size (64 sequences, 32
    # query heads, cached lengths 1024..32768) five calls give the same bits,
    # also with a window and with the append fused into the call.
    B, Nq, Tcap = 64, 32, 32768
    dev = device()
    lens = np.random.default_rng(0).integers(1024, Tcap, B, endpoint=True).astype(np.int32)
    g = torch.Generator(device=dev).manual_seed(Dh * 10 + Nkv)
    kc = torch.randn(B, Nkv, Tcap, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    vc = torch.randn(B, Nkv, Tcap, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    q = torch.randn(B, Nq, Dh, device=dev, dtype=torch.bfloat16, generator=g)
    tl = torch.from_numpy(lens).to(dev)
    O = torch.empty_like(q)
    L = torch.empty(B, Nq, device=dev)
    ws = torch.empty(tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, 0),
                     dtype=torch.uint8, device=dev)
    if append:
        kn = torch.randn(B, Nkv, Dh, device=dev, dtype=torch.bfloat16, generator=g)
        vn = torch.randn(B, Nkv, Dh, device=dev, dtype=torch.bfloat16, generator=g)
        slot = (tl - 1).to(torch.int32)
        call = lambda: tch.attn_decode_append(q, kn, vn, kc, vc, tl, slot, O, L, workspace=ws)
    else:
        call = lambda: tch.attn_decode_window(q, kc, vc, tl, O, L, workspace=ws, window=window)
    outs = []
    for _ in range(5):
        call()
        torch.cuda.synchronize()
        outs.append((O.view(torch.int16).clone(), L.view(torch.int32).clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    assert torch.isfinite(O.float()).all()
    say(f"decode repeat Dh={Dh} Nkv={Nkv} window={window} append={append}: 5 calls bit-identical")


def test_decode_deterministic_and_workspace_checked():
    lens, q, kc, vc = workloads.decode_inputs(8, 32, 8, 128, 4096, 1, 4096, seed=4)
    O1, L1 = run_decode(q, kc, vc, lens, "bf16")
    O2, L2 = run_decode(q, kc, vc, lens, "bf16")
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    dev = device()
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
    tl = torch.from_numpy(lens).to(dev)
    O = torch.empty_like(tq)
    small = torch.empty(64, dtype=torch.uint8, device=dev)
    with pytest.raises(tch.AttnError) as e:
        tch.attn_decode(tq, tk, tv, tl, O, None, small)
    assert e.value.status == tch.ATTN_EWORKSPACE
