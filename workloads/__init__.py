"""Seeded synthetic inputs for the attention workloads.

Shared by the test suite, the smoke check and the benchmark, on both sides of
every parity check (GPU library and float64 oracle).  This module holds none
of the attention arithmetic: only shapes, seeded N(0,1) draws, float32 ->
bfloat16 round-to-nearest-even, NaN poisoning of unused cache slots, row
sampling, and the closed-form work counts used to express throughput.

Recipe (all draws from ``numpy.random.default_rng``):
  * prefill: seed 0; Q, K, V drawn in that order as float32 standard normals of
    shape [B,Nq,S,Dh], [B,Nkv,S,Dh], [B,Nkv,S,Dh]; bf16 workloads round each
    float32 to the nearest bfloat16 (ties to even).  The oracle sees the same
    rounded values widened to float64.
  * decode: seed 0; first the cached lengths lens[B] uniform on [lo, hi]
    (both ends included), then q [B,Nq,Dh], then per sequence b the valid
    cache part K[b, :, :lens[b]] followed by V[b, :, :lens[b]]; cache slots at
    or past lens[b] hold NaN so that any read beyond the length shows up.
  * sampled output rows of the long workloads: seed 1, n draws of (b, h, i)
    with b, h, i drawn in that order per component, plus forced rows.
"""

import numpy as np

# Workloads, named by what they are.  The shapes are the pages': the
# Chinese post's [2, 32, 1024, 128] example, 32 heads of size 128, a 32/8
# grouped-query split with a 4096-token window, and 32768-token context.
WORKLOADS = {
    "tiny_fp32_b1_h2_s5_d4": dict(
        kind="prefill", B=1, Nq=2, Nkv=2, S=5, Dh=4, dtype="f32",
        causal=True, window=0, scale=0.5),
    "mha_bf16_b2_h32_s1024_d128": dict(
        kind="prefill", B=2, Nq=32, Nkv=32, S=1024, Dh=128, dtype="bf16",
        causal=True, window=0, scale=None),
    "mha_bf16_b1_h32_s32768_d128": dict(
        kind="prefill", B=1, Nq=32, Nkv=32, S=32768, Dh=128, dtype="bf16",
        causal=True, window=0, scale=None, sample=256, forced_rows=(0, 32767)),
    "gqa_bf16_b4_h32kv8_s8192_w4096_d128": dict(
        kind="prefill", B=4, Nq=32, Nkv=8, S=8192, Dh=128, dtype="bf16",
        causal=True, window=4096, scale=None, sample=1024,
        forced_rows=(0, 4095, 4096, 8191)),
    "decode_bf16_b64_h32kv8_t32768_d128": dict(
        kind="decode", B=64, Nq=32, Nkv=8, Dh=128, Tcap=32768, dtype="bf16",
        len_lo=1024, len_hi=32768),
}

BF16_NAN_BITS = 0x7FC0


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits):
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr, dtype):
    """Stored values (bf16 bits or float32) widened exactly to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def to_torch(arr, dtype, device=None):
    """Stored values as a torch tensor (bf16 bits are reinterpreted, not cast)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device) if device is not None else t


def from_torch(t, dtype):
    """Inverse of ``to_torch``: bf16 tensors come back as uint16 bits."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().astype(np.float32)


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=0):
    """Q, K, V for a prefill workload, stored as bf16 bits or float32."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Nq, S, Dh), dtype)
    k = _draw(rng, (B, Nkv, S, Dh), dtype)
    v = _draw(rng, (B, Nkv, S, Dh), dtype)
    return q, k, v


def decode_inputs(B, Nq, Nkv, Dh, Tcap, len_lo, len_hi, dtype="bf16", seed=0,
                  lens=None):
    """lens, q, Kcache, Vcache for one decode step; unused slots are NaN.

    ``lens`` may be given explicitly (then nothing is drawn for it).
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_lo, len_hi, B, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    if lens.shape != (B,) or lens.min() < 1 or lens.max() > Tcap:
        raise ValueError("lens must be [B] within [1, Tcap]")
    q = _draw(rng, (B, Nq, Dh), dtype)
    if dtype == "bf16":
        kc = np.full((B, Nkv, Tcap, Dh), BF16_NAN_BITS, dtype=np.uint16)
        vc = np.full((B, Nkv, Tcap, Dh), BF16_NAN_BITS, dtype=np.uint16)
    else:
        kc = np.full((B, Nkv, Tcap, Dh), np.nan, dtype=np.float32)
        vc = np.full((B, Nkv, Tcap, Dh), np.nan, dtype=np.float32)
    for b in range(B):
        n = int(lens[b])
        kc[b, :, :n] = _draw(rng, (Nkv, n, Dh), dtype)
        vc[b, :, :n] = _draw(rng, (Nkv, n, Dh), dtype)
    return lens.astype(np.int32), q, kc, vc


def sample_rows(B, Nq, S, n, seed=1, forced_rows=()):
    """Seeded (b, h, i) output rows to check on a long workload."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, B, n)
    h = rng.integers(0, Nq, n)
    i = rng.integers(0, S, n)
    triples = [(int(x), int(y), int(z)) for x, y, z in zip(b, h, i)]
    for r in forced_rows:
        triples.append((0, 0, int(r)))
        triples.append((B - 1, Nq - 1, int(r)))
    return triples


def visible_pairs_per_head(S, causal, window):
    """Closed-form count of (query, key) pairs the mask admits in one head."""
    if not causal:
        return S * S
    if window <= 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def prefill_work(B, Nq, Nkv, S, Dh, causal, window, elem_bytes):
    """Algorithmic FLOPs and compulsory HBM bytes of one prefill call.

    FLOPs count 2 per multiply-add over visible pairs only, for QK^T and PV
    (4 * Dh per pair); bytes are one read of Q, K, V, one write of O and
    of the fp32 LSE.
    """
    pairs = visible_pairs_per_head(S, causal, window)
    flops = 4 * Dh * pairs * B * Nq
    nbytes = (2 * B * Nq * S * Dh + 2 * B * Nkv * S * Dh) * elem_bytes + 4 * B * Nq * S
    return flops, nbytes


def decode_work(lens, Nq, Nkv, Dh, elem_bytes):
    """Algorithmic FLOPs and compulsory HBM bytes of one decode step.

    Bytes: every visible cached K and V row once per K/V head, plus q, O and
    lens; FLOPs: 4 * Dh per (query head, key).
    """
    total = int(np.sum(lens))
    B = len(lens)
    nbytes = 2 * total * Nkv * Dh * elem_bytes + 2 * B * Nq * Dh * elem_bytes + 4 * B
    flops = 4 * Dh * Nq * total
    return flops, nbytes
