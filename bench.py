"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole path over one batch of synthetic input:
  * causal multi-head prefill, bf16, B=1, 32 heads, S=32768, Dh=128
    (the long-context workload; 8.796e12 algorithmic FLOPs per call), then
  * one KV-cache decode step, bf16, 64 sequences, 32 query / 8 K/V heads,
    Dh=128, cached lengths uniform in [1024, 32768].
After the timed steps the two other bf16 prefill workloads are timed on their
own and reported as sub-objects: grouped-query 32/8 heads, B=4, S=8192,
window 4096 (`gqa_window`), and B=2, 32 heads, S=1024 over eight rotating
input sets (`mha_s1024`).
Inputs are seeded N(0,1) draws (see workloads/), resident in HBM before the
timed region.  W untimed steps, then K timed steps bracketed by device
synchronisation; kernel durations come from HIP events recorded on the stream
the kernels are launched on.  Prints ONE JSON line:
  value = prefill TFLOP/s (2 FLOP per multiply-add, visible pairs only),
  decode = decode throughput in GB/s of compulsory HBM traffic,
  roofline = the prefill kernel (the dominant one) against bf16 dense MFMA peak,
  cpu_baseline = the float64 oracle on a bounded sample of the same prefill.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PREFILL = "mha_bf16_b1_h32_s32768_d128"
DECODE = "decode_bf16_b64_h32kv8_t32768_d128"
# the other two bf16 prefill workloads, timed on their own after the main step
GQA_WINDOW = "gqa_bf16_b4_h32kv8_s8192_w4096_d128"
MHA_S1024 = "mha_bf16_b2_h32_s1024_d128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# HBM traffic of one launch measured with rocprofv3 --pmc FETCH_SIZE /
# WRITE_SIZE, scaled by the same counters on a copy of known size (one
# FETCH_SIZE unit = 2047.9 bytes, one WRITE_SIZE unit = 1024 bytes); valid only
# for the kernel source it was taken on (sha256[:16] of the .hip file).
TRAFFIC = {
    "prefill_bf16.hip": {"64e736153821d8b4": 3553643950},  # 3.281e+09 fetched + 2.727e+08 written
    # partial + merge kernels
    "decode_bf16.hip": {"10b5908f1eec1680": 4520626259},   # 4.517e+09 fetched + 3.792e+06 written
}


def _kernel_sha(name):
    p = os.path.join(ROOT, "transformer_causal_head_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _cpu_baseline(q, k, v, cfg, budget_s=12.0):
    """Time the float64 oracle on sampled prefill rows of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    heads = 4  # the sample is drawn from heads 0..3 of batch 0
    S, Dh = cfg["S"], cfg["Dh"]
    tr = sorted(workloads.sample_rows(1, heads, S, 65536, seed=1))
    Qh = workloads.to_f64(q[:, :heads], "bf16")
    Kh = workloads.to_f64(k[:, :heads], "bf16")
    Vh = workloads.to_f64(v[:, :heads], "bf16")
    done, flops, t0 = 0, 0, time.perf_counter()
    while done < len(tr) and time.perf_counter() - t0 < budget_s:
        part = tr[done:done + 256]
        oracle.attention_rows_ref(Qh, Kh, Vh, part, causal=True, window=cfg["window"])
        # causal row i without a window sees i + 1 keys: 4 * Dh FLOPs each
        flops += sum(4 * Dh * (i + 1) for _, _, i in part)
        done += len(part)
    dt = time.perf_counter() - t0
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} seeded (head, row) pairs of heads 0-3, {dt:.1f} s, "
                      f"float64 NumPy full score rows"}


PROBE_LIB = os.path.join(ROOT, "_build", "libhbm_probe.so")
ISSUE_LIB = os.path.join(ROOT, "_build", "libissue_probe.so")


def _build_probe():
    """Compile the probes beside this file (benchmark tooling, not the library) into _build/."""
    from transformer_causal_head_amd import build as lib_build
    os.makedirs(os.path.dirname(PROBE_LIB), exist_ok=True)
    for src, lib in (("hbm_probe.hip", PROBE_LIB), ("issue_probe.hip", ISSUE_LIB)):
        obj = lib_build._compile(src, ROOT, os.path.dirname(lib))
        lib_build._link([obj], lib)
        print("built", lib)


def _issue_probe(torch, dev, iters=4000):
    """Matrix-core / VALU / LDS issue probe (issue_probe.hip): one line per mix.

    ns_per_mfma: elapsed time per MFMA slot of one SIMD's MFMA waves, i.e.
    elapsed / (iters * 32 * MFMA waves per SIMD); a 32x32x16 bf16 MFMA is 32
    cycles of the matrix core, so 32 / ns_per_mfma is the clock in GHz when the
    matrix core is never idle.  ns_per_slot: elapsed / (iters * 32)."""
    import ctypes
    if not os.path.exists(ISSUE_LIB):
        raise RuntimeError(f"{ISSUE_LIB} is missing: run `python bench.py --build-probe` first")
    L = ctypes.CDLL(ISSUE_LIB)
    L.issue_probe.restype = ctypes.c_int
    L.issue_probe.argtypes = [ctypes.c_int] * 8 + [ctypes.c_void_p, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(n_cu * 2 * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # (kind, waves, lds, reuse, exp, nv): kind 0 MFMA, 1 VALU, 2 both in one wave, 3 split
    mixes = [(0, 4, 0, 1, 0, 0), (0, 8, 0, 1, 0, 0), (0, 4, 1, 1, 0, 0), (0, 8, 1, 1, 0, 0),
             (0, 4, 1, 2, 0, 0), (0, 8, 1, 2, 0, 0),
             (1, 4, 0, 1, 1, 2), (1, 4, 0, 1, 1, 4), (1, 4, 0, 1, 1, 8), (1, 4, 0, 1, 0, 4),
             (1, 4, 0, 1, 0, 8),
             (2, 4, 0, 1, 1, 2), (2, 4, 0, 1, 1, 4), (2, 4, 0, 1, 1, 8), (2, 4, 0, 1, 0, 4),
             (2, 4, 0, 1, 0, 8), (2, 8, 0, 1, 1, 4), (2, 8, 0, 1, 0, 4),
             (2, 4, 1, 1, 1, 4), (2, 4, 1, 1, 0, 4), (2, 8, 1, 1, 1, 4), (2, 8, 1, 1, 0, 4),
             (3, 8, 0, 1, 1, 4), (3, 8, 0, 1, 1, 8), (3, 8, 0, 1, 0, 4), (3, 8, 0, 1, 0, 8),
             (3, 8, 1, 1, 1, 4)]
    for kind, waves, lds, reuse, exp, nv in mixes:
        def launch():
            rc = L.issue_probe(kind, waves, n_cu, iters, lds, reuse, exp, nv, out.data_ptr(),
                               ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"issue_probe returned {rc}")
        ms = _time(torch, launch, 5, 2)
        mfma_waves = 0 if kind == 1 else (waves // 4 if kind != 3 else waves // 8)
        row = {"kind": ["mfma", "valu", "mixed", "split"][kind], "waves_per_cu": waves,
               "lds_operand": bool(lds), "reuse": reuse, "valu_per_slot": nv, "exp": bool(exp),
               "us": round(ms * 1e3, 1), "ns_per_slot": round(ms * 1e6 / (iters * 32), 2)}
        if mfma_waves:
            row["ns_per_mfma"] = round(ms * 1e6 / (iters * 32 * mfma_waves), 2)
        print(json.dumps(row), flush=True)
    # LDS read bandwidth per CU: 16-byte row reads, transposing 8-byte read pairs, and the
    # pairs feeding one MFMA each (every kind moves 1 KB per wave per slot)
    L.lds_probe.restype = ctypes.c_int
    L.lds_probe.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    for kind, waves in ((4, 4), (4, 8), (5, 4), (5, 8), (6, 4), (6, 8)):
        def launch():
            rc = L.lds_probe(kind, waves, n_cu, iters, out.data_ptr(),
                             ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"lds_probe returned {rc}")
        ms = _time(torch, launch, 5, 2)
        nbytes = n_cu * waves * iters * 32 * 1024
        row = {"kind": {4: "lds_b128", 5: "lds_tr_b64_pairs", 6: "lds_tr_b64_pairs+mfma"}[kind],
               "waves_per_cu": waves, "us": round(ms * 1e3, 1),
               "lds_GBs_per_cu": round(nbytes / n_cu / (ms * 1e-3) / 1e9, 1),
               "ns_per_slot_per_simd": round(ms * 1e6 / (iters * 32 * waves / 4), 2)}
        print(json.dumps(row), flush=True)


def _read_ceiling(torch, dev, gib=4.5, reps=5):
    """Streaming-read rate of the device (hbm_probe.hip) for a few launch shapes."""
    import ctypes
    path = PROBE_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python bench.py --build-probe` first")
    L = ctypes.CDLL(path)
    L.hbm_read_probe.restype = ctypes.c_int
    L.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = int(gib * (1 << 30)) // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rows = []
    shapes = ((1024, 4), (4096, 4), (16384, 4), (32768, 4), (8192, 8), (16384, 8))
    for nt, (blocks, unroll) in [(nt, sh) for nt in (0, 1) for sh in shapes]:
        def launch():
            rc = L.hbm_read_probe(buf.data_ptr(), nbytes, blocks, unroll, nt, sink.data_ptr(),
                                  ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"hbm_read_probe returned {rc}")
        launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            launch()
        b.record(stream)
        b.synchronize()
        gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        rows.append({"blocks": blocks, "threads": 256, "loads_in_flight": unroll,
                     "non_temporal": bool(nt), "GB/s": round(gbs, 1)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"read_bytes": nbytes, "reps": reps, "sweep": rows,
                      "best_GBs": max(r["GB/s"] for r in rows)}), flush=True)


def _time(torch, fn, steps, warmup):
    """Mean ms per call, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / steps


def _prefill_line(torch, dev, tch, name, steps, warmup, sets):
    """Time one named bf16 prefill workload on its own (HIP events on the launch stream):
    `sets` input sets drawn with seeds 0.. are used in rotation, so that a workload small
    enough for the 256 MB last-level cache still reads its inputs from HBM."""
    cfg = workloads.WORKLOADS[name]
    B, Nq, Nkv, S, Dh = cfg["B"], cfg["Nq"], cfg["Nkv"], cfg["S"], cfg["Dh"]
    inputs = []
    for i in range(sets):
        q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=i)
        inputs.append(tuple(workloads.to_torch(x, "bf16", dev) for x in (q, k, v)))
        del q, k, v
    O = torch.empty_like(inputs[0][0])
    L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(Dh)
    state = {"i": 0}

    def call():
        tq, tk, tv = inputs[state["i"] % sets]
        state["i"] += 1
        tch.attn_prefill(tq, tk, tv, O, L, causal=int(cfg["causal"]), window=cfg["window"],
                         scale=scale)
    ms = _time(torch, call, steps, max(warmup, sets))
    flop, nbytes = workloads.prefill_work(B, Nq, Nkv, S, Dh, cfg["causal"], cfg["window"], 2)
    tf = flop / (ms * 1e-3) / 1e12
    del inputs, O, L
    return {"workload": name, "ms": round(ms, 5), "tflops": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "calls": steps,
            "input_sets": sets, "algorithmic_flop": flop, "compulsory_bytes": nbytes}


def _cache_paths(torch, dev, tch, steps, warmup):
    """One JSON line per cache-side entry point, on the shapes of the main workloads."""
    # chunked prefill: the last 2048 tokens of a 32768-token context, GQA 32/8
    B, Nq, Nkv, Sq, T, Dh = 1, 32, 8, 2048, 32768, 128
    lens, Q, kc, vc = workloads.chunk_inputs(B, Nq, Nkv, Sq, Dh, T, [T], "bf16", seed=0)
    tQ, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (Q, kc, vc))
    tl = torch.from_numpy(lens).to(dev)
    O = torch.empty_like(tQ)
    L = torch.empty((B, Nq, Sq), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda: tch.attn_prefill_cache(tQ, tk, tv, tl, O, L), steps, warmup)
    flop = 4 * Dh * Nq * B * sum(T - Sq + i + 1 for i in range(Sq))
    tf = flop / (ms * 1e-3) / 1e12
    print(json.dumps({"path": "attn_prefill_cache", "workload": f"B={B} Nq={Nq} Nkv={Nkv} "
                      f"Sq={Sq} lens={T} Dh={Dh} bf16 causal", "ms": round(ms, 4),
                      "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "algorithmic_flop": flop}), flush=True)
    del tQ, tk, tv, O, L

    # decode workload with a 4096-key window: linear cache, then a rolling buffer
    dc = workloads.WORKLOADS[DECODE]
    B, Nq, Nkv, Dh, T, W = dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"], dc["Tcap"], 4096
    lens, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, T, dc["len_lo"], dc["len_hi"])
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
    tl = torch.from_numpy(lens).to(dev)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, tch.attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, T, W,
                                                                   tch.ATTN_BF16)),
                     dtype=torch.uint8, device=dev)
    vis = np.minimum(lens, W).astype(np.int64)
    nbytes = int(2 * vis.sum() * Nkv * Dh * 2 + 2 * B * Nq * Dh * 2 + 4 * B)
    ms = _time(torch, lambda: tch.attn_decode_window(tq, tk, tv, tl, O, L, ws, window=W),
               steps, warmup)
    print(json.dumps({"path": "attn_decode_window", "workload": f"{DECODE} window={W}",
                      "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                      "frac_of_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": nbytes}), flush=True)
    # rolling buffer of W slots holding each sequence's last min(len, W) keys
    rk = tk[:, :, :W].contiguous()
    rv = tv[:, :, :W].contiguous()
    rl = torch.from_numpy(vis.astype(np.int32)).to(dev)
    wsr = torch.empty(max(1, tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, W, tch.ATTN_BF16)),
                      dtype=torch.uint8, device=dev)
    ms = _time(torch, lambda: tch.attn_decode(tq, rk, rv, rl, O, L, wsr), steps, warmup)
    print(json.dumps({"path": "attn_decode (rolling buffer)", "workload":
                      f"B={B} Nq={Nq} Nkv={Nkv} Dh={Dh} buffer={W} slots, lens=min(len, {W})",
                      "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                      "frac_of_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": nbytes}), flush=True)
    # one decode step with its append: fused (attn_decode_append) and as two launches
    kn = torch.randn(B, Nkv, Dh, device=dev, dtype=torch.bfloat16)
    vn = torch.randn_like(kn)
    slot = (tl - 1).contiguous()
    wsf = torch.empty(tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, T, tch.ATTN_BF16),
                      dtype=torch.uint8, device=dev)
    ms_fused = _time(torch, lambda: tch.attn_decode_append(tq, kn, vn, tk, tv, tl, slot, O, L, wsf),
                     steps, warmup)
    kn4, vn4 = kn[:, :, None].contiguous(), vn[:, :, None].contiguous()

    def two_launches():
        tch.attn_kv_append(kn4, vn4, tk, tv, slot)
        tch.attn_decode_window(tq, tk, tv, tl, O, L, wsf)

    ms_two = _time(torch, two_launches, steps, warmup)
    _, dbytes = workloads.decode_work(lens, Nq, Nkv, Dh, 2)
    print(json.dumps({"path": "attn_decode_append", "workload": f"{DECODE}, new K/V row appended "
                      "in the same call", "ms": round(ms_fused, 4),
                      "GB/s": round(dbytes / ms_fused / 1e6, 1),
                      "two_launches_ms": round(ms_two, 4), "algorithmic_bytes": dbytes}), flush=True)

    # append of one token per sequence into the rolling buffer
    kn = torch.randn(B, Nkv, 1, Dh, device=dev, dtype=torch.bfloat16)
    vn = torch.randn_like(kn)
    ms = _time(torch, lambda: tch.attn_kv_append(kn, vn, rk, rv, tl, rolling=1), steps, warmup)
    abytes = 2 * 2 * B * Nkv * Dh * 2
    print(json.dumps({"path": "attn_kv_append", "workload": f"B={B} Nkv={Nkv} Snew=1 Dh={Dh} "
                      f"rolling buffer of {W}", "ms": round(ms, 4),
                      "GB/s": round(abytes / ms / 1e6, 1), "algorithmic_bytes": abytes}),
          flush=True)


def _workloads(torch, dev, tch, steps, warmup):
    """One JSON line per named workload, each in the launch configuration the parity tests
    check at full size: the three bf16 prefill workloads against the bf16 MFMA peak and the
    decode workload against HBM bandwidth.  The 1024-token workload is short (tens of us) and
    its inputs would stay in the 256 MB last-level cache, so its calls rotate over eight input
    sets (about 400 MB) and are timed back to back."""
    for name, cfg in workloads.WORKLOADS.items():
        if cfg["kind"] != "prefill" or cfg["dtype"] != "bf16":
            continue
        B, Nq, Nkv, S, Dh = cfg["B"], cfg["Nq"], cfg["Nkv"], cfg["S"], cfg["Dh"]
        sets = 8 if S <= 4096 else 1
        inputs = []
        for i in range(sets):
            q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=i)
            inputs.append(tuple(workloads.to_torch(x, "bf16", dev) for x in (q, k, v)))
            del q, k, v
        O = torch.empty_like(inputs[0][0])
        L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(Dh)
        state = {"i": 0}

        def call():
            tq, tk, tv = inputs[state["i"] % sets]
            state["i"] += 1
            tch.attn_prefill(tq, tk, tv, O, L, causal=int(cfg["causal"]), window=cfg["window"],
                             scale=scale)
        n = steps * (20 if sets > 1 else 1)
        ms = _time(torch, call, n, max(warmup, sets))
        flop, nbytes = workloads.prefill_work(B, Nq, Nkv, S, Dh, cfg["causal"], cfg["window"], 2)
        tf = flop / (ms * 1e-3) / 1e12
        print(json.dumps({"path": "attn_prefill", "workload": name, "ms": round(ms, 4),
                          "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "algorithmic_flop": flop, "compulsory_bytes": nbytes,
                          "input_sets": sets}), flush=True)
        del inputs, O, L
    dc = workloads.WORKLOADS[DECODE]
    B, Nq, Nkv, Dh, T = dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"], dc["Tcap"]
    lens, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, T, dc["len_lo"], dc["len_hi"])
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
    del kc, vc
    tl = torch.from_numpy(lens).to(dev)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, T, tch.ATTN_BF16)),
                     dtype=torch.uint8, device=dev)
    ms = _time(torch, lambda: tch.attn_decode(tq, tk, tv, tl, O, L, ws), steps, warmup)
    _, nbytes = workloads.decode_work(lens, Nq, Nkv, Dh, 2)
    gbs = nbytes / ms / 1e6
    print(json.dumps({"path": "attn_decode", "workload": DECODE, "ms": round(ms, 4),
                      "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": nbytes}), flush=True)


def _decode_batches(torch, dev, tch, steps, warmup):
    """One JSON line per decode batch shape: few sequences at long context (every
    sequence at full length), where the chunk length, not the batch, has to supply
    the parallelism, and the decode workload's 64 sequences for reference."""
    for B, T, Nkv, Nq in ((1, 32768, 8, 32), (1, 131072, 8, 32), (4, 32768, 8, 32),
                          (8, 32768, 8, 32), (1, 32768, 1, 32), (2, 65536, 8, 64)):
        lens = np.full(B, T, dtype=np.int32)
        q = workloads.draw((B, Nq, 128), "bf16", 0, 10)
        tq = workloads.to_torch(q, "bf16", dev)
        g = torch.Generator(device=dev).manual_seed(B * 1000 + Nkv)
        # cache contents do not change the time; drawn on the device to keep set-up short
        tk = torch.randn(B, Nkv, T, 128, device=dev, dtype=torch.bfloat16, generator=g)
        tv = torch.randn(B, Nkv, T, 128, device=dev, dtype=torch.bfloat16, generator=g)
        tl = torch.from_numpy(lens).to(dev)
        O = torch.empty_like(tq)
        L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tch.attn_decode_workspace_bytes(B, Nq, Nkv, 128, T, tch.ATTN_BF16)),
                         dtype=torch.uint8, device=dev)
        ms = _time(torch, lambda: tch.attn_decode(tq, tk, tv, tl, O, L, ws), steps * 2, warmup)
        _, nbytes = workloads.decode_work(lens, Nq, Nkv, 128, 2)
        gbs = nbytes / ms / 1e6
        print(json.dumps({"path": "attn_decode", "workload": f"B={B} lens={T} Nq={Nq} Nkv={Nkv} Dh=128 bf16",
                          "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                          "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes}),
              flush=True)
        del tq, tk, tv, O, L, ws


def _head_sizes(torch, dev, tch, steps, warmup):
    """One JSON line per shape: causal MHA prefill at head sizes 64 / 128 / 256 with the same
    32-head layout, and the batched decode workload at head sizes 64 / 256 and as MQA."""
    for Dh, S in ((64, 32768), (128, 32768), (256, 16384)):
        B, H = 1, 32
        q, k, v = workloads.prefill_inputs(B, H, H, S, Dh, "bf16", seed=0)
        tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
        del q, k, v
        O = torch.empty_like(tq)
        L = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        ms = _time(torch, lambda: tch.attn_prefill(tq, tk, tv, O, L, causal=1,
                                                   scale=1.0 / math.sqrt(Dh)), steps, warmup)
        flop, _ = workloads.prefill_work(B, H, H, S, Dh, True, 0, 2)
        tf = flop / (ms * 1e-3) / 1e12
        print(json.dumps({"path": "attn_prefill", "workload": f"B={B} heads={H} S={S} Dh={Dh} "
                          "bf16 causal", "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                          "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
        del tq, tk, tv, O, L
    # non-causal attention (every query sees every key), 8192 tokens
    B, H, S, Dh = 1, 32, 8192, 128
    q, k, v = workloads.prefill_inputs(B, H, H, S, Dh, "bf16", seed=0)
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
    del q, k, v
    O = torch.empty_like(tq)
    L = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda: tch.attn_prefill(tq, tk, tv, O, L, causal=0,
                                               scale=1.0 / math.sqrt(Dh)), steps, warmup)
    flop, _ = workloads.prefill_work(B, H, H, S, Dh, False, 0, 2)
    tf = flop / (ms * 1e-3) / 1e12
    print(json.dumps({"path": "attn_prefill", "workload": f"B={B} heads={H} S={S} Dh={Dh} "
                      "bf16 non-causal", "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                      "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
    del tq, tk, tv, O, L
    dc = workloads.WORKLOADS[DECODE]
    for Dh, Nq, Nkv in ((64, 32, 8), (256, 32, 8), (128, 32, 1)):
        B, T = dc["B"], dc["Tcap"]
        lens, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, T, dc["len_lo"], dc["len_hi"])
        tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, kc, vc))
        del kc, vc
        tl = torch.from_numpy(lens).to(dev)
        O = torch.empty_like(tq)
        L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, T, tch.ATTN_BF16)),
                         dtype=torch.uint8, device=dev)
        ms = _time(torch, lambda: tch.attn_decode(tq, tk, tv, tl, O, L, ws), steps, warmup)
        _, nbytes = workloads.decode_work(lens, Nq, Nkv, Dh, 2)
        gbs = nbytes / ms / 1e6
        print(json.dumps({"path": "attn_decode", "workload": f"B={B} Nq={Nq} Nkv={Nkv} Dh={Dh} "
                          f"Tcap={T} sum(lens)={int(lens.sum())} bf16", "ms": round(ms, 4),
                          "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes": nbytes}), flush=True)
        del tq, tk, tv, O, L, ws


def _backward(torch, dev, tch, steps, warmup):
    """One JSON line per shape: attn_backward (dQ, dK, dV from O, LSE and dO) on the prefill
    workload and on GQA / head-size-64 / head-size-256 variants (the last at the 16384-token
    shape of the head-size-256 prefill line).  Algorithmic FLOPs are 2.5 times the
    forward's: five products per visible pair (S = Q K^T, dP = dO V^T, dV, dK, dQ); the
    kernels recompute S and dP once more (seven products), which is not counted."""
    for B, Nq, Nkv, S, Dh in ((1, 32, 32, 32768, 128), (1, 32, 8, 32768, 128),
                              (1, 32, 32, 32768, 64), (1, 32, 32, 16384, 256)):
        q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=0)
        tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
        del q, k, v
        tdo = torch.randn_like(tq)
        O = torch.empty_like(tq)
        L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(Dh)
        tch.attn_prefill(tq, tk, tv, O, L, causal=1, scale=scale)
        dQ, dK, dV = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(tch.attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, tch.ATTN_BF16),
                         dtype=torch.uint8, device=dev)
        ms = _time(torch, lambda: tch.attn_backward(tq, tk, tv, O, tdo, L, dQ, dK, dV,
                                                    causal=1, scale=scale, workspace=ws),
                   steps, warmup)
        fwd, _ = workloads.prefill_work(B, Nq, Nkv, S, Dh, True, 0, 2)
        flop = int(2.5 * fwd)
        tf = flop / (ms * 1e-3) / 1e12
        print(json.dumps({"path": "attn_backward", "workload": f"B={B} Nq={Nq} Nkv={Nkv} "
                          f"S={S} Dh={Dh} bf16 causal", "ms": round(ms, 4),
                          "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "algorithmic_flop": flop}), flush=True)
        del tq, tk, tv, tdo, O, L, dQ, dK, dV, ws


def _rope_padding(torch, dev, tch, steps, warmup):
    """One JSON line per measurement: RoPE in place on the prefill queries, the rotating
    cache append (a 2048-token chunk and one decode token), and the padded prefill and
    decode next to their unpadded forms on the same inputs."""
    pc = workloads.WORKLOADS[PREFILL]
    B, H, S, Dh = pc["B"], pc["Nq"], pc["S"], pc["Dh"]
    x = torch.randn(B, H, S, Dh, device=dev, dtype=torch.bfloat16)
    table = tch.rope_table(S, Dh, device=dev)
    ms = _time(torch, lambda: tch.attn_rope(x, x, table, style=1), steps, warmup)
    nbytes = 2 * x.numel() * 2 + S * Dh * 4  # rows read and written, table rows read once
    print(json.dumps({"path": "attn_rope (in place)", "workload": f"B={B} H={H} S={S} Dh={Dh} "
                      "bf16, half layout", "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                      "frac_of_hbm_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": nbytes}), flush=True)
    del x, table

    # RoPE fused into the attention call against the two passes it replaces, on the
    # 32768-token prefill (keys already rotated) and on the decode workload
    q, k, v = workloads.prefill_inputs(B, H, H, S, Dh, "bf16", seed=0)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    del q, k, v
    table = tch.rope_table(S, Dh, device=dev)
    tch.attn_rope(tk, tk, table, style=1)
    O = torch.empty_like(tq)
    L = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    qr = torch.empty_like(tq)
    scale = 1.0 / math.sqrt(Dh)
    ms_fused = _time(torch, lambda: tch.attn_prefill_rope(tq, tk, tv, O, L, table, style=1,
                                                          scale=scale), steps, warmup)

    def two_passes():
        tch.attn_rope(tq, qr, table, style=1)
        tch.attn_prefill(qr, tk, tv, O, L, scale=scale)
    ms_two = _time(torch, two_passes, steps, warmup)
    flop, _ = workloads.prefill_work(B, H, H, S, Dh, True, 0, 2)
    print(json.dumps({"path": "attn_prefill_rope", "workload": f"B={B} H={H} S={S} Dh={Dh} bf16 "
                      "causal, q rotated in the kernel (half layout)", "ms": round(ms_fused, 4),
                      "TFLOP/s": round(flop / ms_fused / 1e9, 1),
                      "two_passes_ms": round(ms_two, 4),
                      "two_passes": "attn_rope on q, then attn_prefill"}), flush=True)
    del tq, tk, tv, O, L, qr, table
    dc = workloads.WORKLOADS[DECODE]
    lens, q, kc, vc = workloads.decode_inputs(dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"], dc["Tcap"],
                                              dc["len_lo"], dc["len_hi"])
    tq, tkc, tvc = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    del kc, vc
    tl = torch.from_numpy(lens).to(dev)
    table = tch.rope_table(dc["Tcap"], dc["Dh"], device=dev)
    Od = torch.empty_like(tq)
    Ld = torch.empty((dc["B"], dc["Nq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(tch.attn_decode_workspace_bytes(dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"],
                                                     dc["Tcap"], tch.ATTN_BF16),
                     dtype=torch.uint8, device=dev)
    pos = (tl - 1).reshape(-1, 1).contiguous()
    qr = torch.empty_like(tq)
    ms_fused = _time(torch, lambda: tch.attn_decode_rope(tq, tkc, tvc, tl, Od, Ld, table,
                                                         workspace=ws, style=1), steps, warmup)

    def two_passes_d():
        tch.attn_rope(tq[:, :, None], qr[:, :, None], table, positions=pos, style=1)
        tch.attn_decode(qr, tkc, tvc, tl, Od, Ld, ws)
    ms_two = _time(torch, two_passes_d, steps, warmup)
    _, dbytes = workloads.decode_work(lens, dc["Nq"], dc["Nkv"], dc["Dh"], 2)
    print(json.dumps({"path": "attn_decode_rope", "workload": f"{DECODE}, q rotated in the kernel",
                      "ms": round(ms_fused, 4), "GB/s": round(dbytes / ms_fused / 1e6, 1),
                      "two_passes_ms": round(ms_two, 4),
                      "two_passes": "attn_rope on q, then attn_decode"}), flush=True)
    del tq, tkc, tvc, Od, Ld, ws, qr, table

    # rotating append: a 2048-token chunk of 8 K/V heads into a 32768-row cache
    Nkv, T = 8, 32768
    table = tch.rope_table(T, Dh, device=dev)
    Kc = torch.zeros(1, Nkv, T, Dh, device=dev, dtype=torch.bfloat16)
    Vc = torch.zeros_like(Kc)
    for Bn, Sn in ((1, 2048), (64, 1)):
        if Bn != Kc.shape[0]:
            Kc = torch.zeros(Bn, Nkv, T, Dh, device=dev, dtype=torch.bfloat16)
            Vc = torch.zeros_like(Kc)
        kn = torch.randn(Bn, Nkv, Sn, Dh, device=dev, dtype=torch.bfloat16)
        vn = torch.randn_like(kn)
        pos = torch.full((Bn,), T - 4096, dtype=torch.int32, device=dev)
        ms = _time(torch, lambda: tch.attn_kv_append_rope(kn, vn, Kc, Vc, pos, table, style=1),
                   steps, warmup)
        nbytes = 2 * 2 * kn.numel() * 2 + Bn * Sn * Dh * 4
        print(json.dumps({"path": "attn_kv_append_rope", "workload": f"B={Bn} Nkv={Nkv} "
                          f"Snew={Sn} Dh={Dh} bf16 into Tcap={T}", "ms": round(ms, 4),
                          "GB/s": round(nbytes / ms / 1e6, 1), "algorithmic_bytes": nbytes}),
              flush=True)
        del kn, vn
    del Kc, Vc, table

    # padded prefill: the 4 x 8192 GQA workload's shape, left padding of 0, 1024, 2048 and
    # 4096 tokens (causal, no window); FLOPs over the visible pairs only
    B, Nq, Nkv, S = 4, 32, 8, 8192
    pads = [0, 1024, 2048, 4096]
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=0)
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, k, v))
    del q, k, v
    mask = torch.from_numpy(workloads.key_mask(B, S, pads=pads)).to(dev)
    bits = tch.pack_key_mask(mask)
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(Dh)
    ms_pad = _time(torch, lambda: tch.attn_prefill_padded(tq, tk, tv, bits, O, L, scale=scale),
                   steps, warmup)
    ms_full = _time(torch, lambda: tch.attn_prefill(tq, tk, tv, O, L, scale=scale), steps, warmup)
    pairs = sum((S - p) * (S - p + 1) // 2 for p in pads)
    flop = 4 * Dh * Nq * pairs
    full_flop, _ = workloads.prefill_work(B, Nq, Nkv, S, Dh, True, 0, 2)
    print(json.dumps({"path": "attn_prefill_padded", "workload": f"B={B} Nq={Nq} Nkv={Nkv} "
                      f"S={S} Dh={Dh} bf16 causal, left padding {pads}", "ms": round(ms_pad, 4),
                      "TFLOP/s": round(flop / ms_pad / 1e9, 1),
                      "unpadded_ms": round(ms_full, 4),
                      "unpadded_TFLOP/s": round(full_flop / ms_full / 1e9, 1),
                      "algorithmic_flop": flop}), flush=True)
    del tq, tk, tv, O, L, mask, bits

    # padded decode: the batched decode workload with 10% of the cached keys padding
    dc = workloads.WORKLOADS[DECODE]
    B, Nq, Nkv, T = dc["B"], dc["Nq"], dc["Nkv"], dc["Tcap"]
    lens, q, kc, vc = workloads.decode_inputs(B, Nq, Nkv, Dh, T, dc["len_lo"], dc["len_hi"])
    tq, tk, tv = (workloads.to_torch(a, "bf16", dev) for a in (q, kc, vc))
    del kc, vc
    tl = torch.from_numpy(lens).to(dev)
    bits = tch.pack_key_mask(torch.from_numpy(workloads.key_mask(B, T, hole_frac=0.1)).to(dev))
    O = torch.empty_like(tq)
    L = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(tch.attn_decode_workspace_bytes(B, Nq, Nkv, Dh, T, tch.ATTN_BF16),
                     dtype=torch.uint8, device=dev)
    ms_pad = _time(torch, lambda: tch.attn_decode_padded(tq, tk, tv, tl, bits, O, L, ws),
                   steps, warmup)
    ms_full = _time(torch, lambda: tch.attn_decode(tq, tk, tv, tl, O, L, ws), steps, warmup)
    _, nbytes = workloads.decode_work(lens, Nq, Nkv, Dh, 2)
    print(json.dumps({"path": "attn_decode_padded", "workload": f"{DECODE}, 10% of keys padding",
                      "ms": round(ms_pad, 4), "GB/s": round(nbytes / ms_pad / 1e6, 1),
                      "unpadded_ms": round(ms_full, 4),
                      "unpadded_GB/s": round(nbytes / ms_full / 1e6, 1),
                      "algorithmic_bytes": nbytes}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="run only the streaming-read probe over 4.5 GB (HBM reference point)")
    ap.add_argument("--build-probe", action="store_true",
                    help="compile the probes (hbm_probe.hip, issue_probe.hip) and exit")
    ap.add_argument("--issue-probe", action="store_true",
                    help="run only the MFMA / VALU / LDS issue probe (issue_probe.hip)")
    ap.add_argument("--head-sizes", action="store_true",
                    help="time prefill and decode at head sizes 64 / 256 and decode with 32 "
                         "query heads per K/V head instead of the main step")
    ap.add_argument("--cache-paths", action="store_true",
                    help="time the cache-side entry points (chunked prefill, windowed and "
                         "rolling-buffer decode, append) instead of the main step")
    ap.add_argument("--rope-padding", action="store_true",
                    help="time RoPE, the rotating append and the padded prefill / decode "
                         "instead of the main step")
    ap.add_argument("--decode-batches", action="store_true",
                    help="time decode at small batches and long context (1-8 sequences, "
                    "32K-128K tokens) instead of the main step")
    ap.add_argument("--workloads", action="store_true",
                    help="time each named workload (the 1024-token, 32768-token and GQA window "
                    "prefills, and the decode step) in its own JSON line instead of the main step")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV) instead of the main step")
    args = ap.parse_args()
    if args.build_probe:
        _build_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path runs without sharding or collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_causal_head_amd as tch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2}))
        return
    if args.read_ceiling:
        _read_ceiling(torch, dev)
        return
    if args.issue_probe:
        _issue_probe(torch, dev)
        return
    if args.cache_paths:
        _cache_paths(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return
    if args.head_sizes:
        _head_sizes(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return
    if args.decode_batches:
        _decode_batches(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return
    if args.workloads:
        _workloads(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return
    if args.backward:
        _backward(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return
    if args.rope_padding:
        _rope_padding(torch, dev, tch, max(args.steps, 5), max(args.warmup, 1))
        return

    pc = workloads.WORKLOADS[PREFILL]
    dc = workloads.WORKLOADS[DECODE]
    B, Nq, Nkv, S, Dh = pc["B"], pc["Nq"], pc["Nkv"], pc["S"], pc["Dh"]
    print(f"generating inputs", file=sys.stderr, flush=True)
    q, k, v = workloads.prefill_inputs(B, Nq, Nkv, S, Dh, "bf16", seed=0)
    tq, tk, tv = (workloads.to_torch(x, "bf16", dev) for x in (q, k, v))
    O = torch.empty_like(tq)
    LSE = torch.empty((B, Nq, S), dtype=torch.float32, device=dev)
    lens, dq, kc, vc = workloads.decode_inputs(dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"],
                                               dc["Tcap"], dc["len_lo"], dc["len_hi"])
    tdq, tkc, tvc = (workloads.to_torch(x, "bf16", dev) for x in (dq, kc, vc))
    del kc, vc
    tl = torch.from_numpy(lens).to(dev)
    dO = torch.empty_like(tdq)
    dL = torch.empty((dc["B"], dc["Nq"]), dtype=torch.float32, device=dev)
    ws_bytes = tch.attn_decode_workspace_bytes(dc["B"], dc["Nq"], dc["Nkv"], dc["Dh"],
                                               dc["Tcap"], tch.ATTN_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"inputs resident", file=sys.stderr, flush=True)

    scale = 1.0 / math.sqrt(Dh)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record(stream)
        tch.attn_prefill(tq, tk, tv, O, LSE, causal=1, window=0, scale=scale)
        if e: e[1].record(stream)
        if e: e[2].record(stream)
        tch.attn_decode(tdq, tkc, tvc, tl, dO, dL, ws)
        if e: e[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    pflops, pbytes = workloads.prefill_work(B, Nq, Nkv, S, Dh, True, 0, 2)
    dflops, dbytes = workloads.decode_work(lens, dc["Nq"], dc["Nkv"], dc["Dh"], 2)
    tflops = pflops / (pre_ms * 1e-3) / 1e12
    gbs = dbytes / (dec_ms * 1e-3) / 1e9

    # the GQA sliding-window and 1024-token prefills, each timed on its own (the
    # 1024-token calls rotate over eight input sets, about 400 MB, and run back to back)
    del tq, tk, tv, O, LSE, tdq, tkc, tvc, dO, dL, ws
    torch.cuda.empty_cache()
    print("timing the GQA window and 1024-token prefills", file=sys.stderr, flush=True)
    gqa = _prefill_line(torch, dev, tch, GQA_WINDOW, args.steps, args.warmup, 1)
    short = _prefill_line(torch, dev, tch, MHA_S1024, args.steps * 20, args.warmup, 8)

    sha = _kernel_sha("prefill_bf16.hip")
    traffic = TRAFFIC["prefill_bf16.hip"].get(sha)
    dsha = _kernel_sha("decode_bf16.hip")
    dtraffic = TRAFFIC["decode_bf16.hip"].get(dsha)
    cpu = None
    if not args.no_cpu_baseline:
        print("timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = _cpu_baseline(q, k, v, pc)

    line = {
        "metric": "causal attn prefill TFLOP/s (bf16, Dh=128) + KV-cache decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{PREFILL} prefill + {DECODE} decode",
                   "prefill": {"B": B, "Nq": Nq, "Nkv": Nkv, "S": S, "Dh": Dh,
                               "causal": True, "window": 0},
                   "decode": {"B": dc["B"], "Nq": dc["Nq"], "Nkv": dc["Nkv"], "Dh": dc["Dh"],
                              "Tcap": dc["Tcap"], "sum_lens": int(lens.sum())},
                   "parallelism": "single GPU"},
        "prefill": {"ms": round(pre_ms, 4), "tflops": round(tflops, 2),
                    "algorithmic_flop": pflops},
        "decode": {"ms": round(dec_ms, 4), "value": round(gbs, 1), "unit": "GB/s",
                   "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                   "algorithmic_bytes": dbytes, "traffic": dtraffic, "kernel_sha": dsha},
        "gqa_window": gqa,
        "mha_s1024": short,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_kernel", "kernel_sha": sha},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
