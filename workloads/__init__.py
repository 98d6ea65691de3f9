"""Seeded synthetic inputs for the attention workloads.

Shared by the test suite, the smoke check and the benchmark, on both sides of
every parity check (GPU library and float64 oracle).  This module holds none
of the attention arithmetic: only shapes, seeded N(0,1) draws, float32 ->
bfloat16 round-to-nearest-even, NaN poisoning of unused cache slots, row
sampling, and the closed-form work counts used to express throughput.

Recipe (all draws from ``numpy.random.default_rng``):
  * a tensor is filled in row-major order by consecutive blocks of 2^20
    float32 standard normals; block i of tensor stream t under seed s comes
    from ``default_rng([s, t, i])``, so the values do not depend on how many
    threads fill the blocks; bf16 tensors round each float32 to the nearest
    bfloat16 (ties to even).  The oracle sees the same rounded values widened
    to float64.
  * prefill: seed 0; Q, K, V are streams 0, 1, 2 with shapes [B,Nq,S,Dh],
    [B,Nkv,S,Dh], [B,Nkv,S,Dh].
  * decode: seed 0; first the cached lengths lens[B] = default_rng(seed)
    .integers(lo, hi, B, endpoint=True); q is stream 10; the valid part
    K[b, :, :lens[b]] of sequence b is stream 1000 + b and V[b, :, :lens[b]]
    is stream 2000 + b (each an [Nkv, lens[b], Dh] block); cache slots at or
    past lens[b] hold NaN so that any read beyond the length shows up.
  * sampled output rows of the long workloads: seed 1, n draws of (b, h, i)
    with b, h, i drawn in that order per component, plus forced rows.
"""

import os
from concurrent.futures import ThreadPoolExecutor

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


BLOCK = 1 << 20
_THREADS = min(16, os.cpu_count() or 1)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    out = t.astype(np.uint16).reshape(x.shape)
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


def _fill_block(flat, seed, stream, i, dtype):
    lo = i * BLOCK
    n = min(BLOCK, flat.size - lo)
    x = np.random.default_rng([seed, stream, i]).standard_normal(n, dtype=np.float32)
    flat[lo:lo + n] = f32_to_bf16_bits(x) if dtype == "bf16" else x


def draw(shape, dtype, seed, stream, pool=None):
    """One seeded N(0,1) tensor (bf16 bits or float32), filled block by block."""
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(-1)
    nblocks = (flat.size + BLOCK - 1) // BLOCK
    if pool is None or nblocks == 1:
        for i in range(nblocks):
            _fill_block(flat, seed, stream, i, dtype)
    else:
        list(pool.map(lambda i: _fill_block(flat, seed, stream, i, dtype), range(nblocks)))
    return out


def prefill_inputs(B, Nq, Nkv, S, Dh, dtype, seed=0):
    """Q, K, V for a prefill workload, stored as bf16 bits or float32."""
    with ThreadPoolExecutor(_THREADS) as pool:
        q = draw((B, Nq, S, Dh), dtype, seed, 0, pool)
        k = draw((B, Nkv, S, Dh), dtype, seed, 1, pool)
        v = draw((B, Nkv, S, Dh), dtype, seed, 2, pool)
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
    q = draw((B, Nq, Dh), dtype, seed, 10)
    if dtype == "bf16":
        kc = np.empty((B, Nkv, Tcap, Dh), dtype=np.uint16)
        vc = np.empty((B, Nkv, Tcap, Dh), dtype=np.uint16)
        poison = BF16_NAN_BITS
    else:
        kc = np.empty((B, Nkv, Tcap, Dh), dtype=np.float32)
        vc = np.empty((B, Nkv, Tcap, Dh), dtype=np.float32)
        poison = np.nan

    def one(b):
        n = int(lens[b])
        for cache, stream in ((kc, 1000 + b), (vc, 2000 + b)):
            cache[b, :, :n] = draw((Nkv, n, Dh), dtype, seed, stream)
            cache[b, :, n:] = poison

    with ThreadPoolExecutor(_THREADS) as pool:
        list(pool.map(one, range(B)))
    return lens.astype(np.int32), q, kc, vc


def chunk_inputs(B, Nq, Nkv, Sq, Dh, Tcap, lens, dtype="bf16", seed=0):
    """lens, Q [B,Nq,Sq,Dh], Kcache, Vcache for a chunk of Sq queries per
    sequence whose keys are the last Sq of lens[b] cached rows (caches drawn as
    in decode_inputs, NaN past each length; Q is stream 11)."""
    lens, _, kc, vc = decode_inputs(B, Nq, Nkv, Dh, Tcap, 1, Tcap, dtype, seed, lens=lens)
    if int(np.min(lens)) < Sq:
        raise ValueError("every length must cover the chunk")
    Q = draw((B, Nq, Sq, Dh), dtype, seed, 11)
    return lens, Q, kc, vc


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


def key_mask(B, T, pads=None, hole_frac=0.0, seed=0, block=None):
    """Seeded key-padding mask, bool [B, T] (True = real token).

    pads[b] leading keys of row b are padding (left padding of a batch of
    prompts of different lengths); each other key is padding with probability
    hole_frac; ``block`` = (start, stop) makes keys start..stop-1 of every row
    padding (a whole tile of padding keys).
    """
    rng = np.random.default_rng(seed + 7919)
    m = rng.random((B, T)) >= hole_frac
    if pads is not None:
        for b, p in enumerate(pads):
            m[b, :p] = False
    if block is not None:
        m[:, block[0]:block[1]] = False
    return m


def token_positions(mask):
    """Positions counted from each row's first real token (padding tokens get 0):
    the positions a model passes to RoPE for a padded batch."""
    return np.maximum(np.cumsum(mask, axis=1) - 1, 0).astype(np.int32)
