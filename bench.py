#!/usr/bin/env python3
"""Benchmark of the causal linear-attention hot path on one MI355X.

One step = one causal prefill of the linear-transformer layer shape
(B=8, H=8, N=4096, d_k=d_v=64, elu(x)+1, bf16 inputs, fp32 state) through
the C ABI, inputs resident in HBM.  `value` is prefill tokens/s (B*N tokens
per step, all heads).  The same JSON line carries:
  roofline      the prefill call against the HBM roofline (algorithmic bytes:
                q, k, v read once and y written once), HIP-event timed;
  decode        batched generation, 256 sequences x 16 heads, Taylor-2 map
                (D = 273), state seeded by the library's own prefill over a
                1024-token prefix, 128 steps; steps/s and its HBM roofline
                (algorithmic bytes: state read + written, q, k, v, y);
  cpu_baseline  the float64 oracle on this host, on a bounded sample: the
                (b, h) pairs split over one worker process per core (at
                most 16, one BLAS thread each), and on one core alone;
  other_configs the Taylor-2 and 64K-token prefills, an N sweep (4K to
                64K tokens) showing time linear in N, the gated
                (scalar-decay) prefill on the headline and Taylor shapes, and
                sliding-window softmax attention (prefill and generation);
  roofline.intra_chunk_mfma_probe
                the MFMA rate of the prefill's within-chunk device code on
                LDS-resident tiles, looped (liblinattn_probe.so).
Inputs are seeded synthetic Gaussians (synth.py); nothing is read from disk.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal lin-attn prefill tokens/s + decode steps/s; % MFMA / HBM peak"
PREFILL = "layer_elu1_bf16"
DECODE = "decode_taylor2_bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
C_REF = 64                     # fixed accounting chunk for the intra term
ROTATE_BYTES = 1 << 30         # rotate input sets over >= 1 GiB (> 256 MB MALL)


def feature_dim(fmap, d_k):
    if fmap == "elu1":
        return d_k
    if fmap == "taylor2sym":
        return 1 + d_k + d_k * (d_k + 1) // 2
    return 1 + d_k + d_k * d_k


def prefill_bytes(cfg):
    """q, k, v read and y written once (+ one float32 decay per token and
    head for the gated form)."""
    es = 2 if cfg["dtype"] == "bf16" else 4
    tok = cfg["B"] * cfg["H"] * cfg["N"]
    return tok * ((2 * cfg["d_k"] + 2 * cfg["d_v"]) * es + (4 if cfg.get("gated") else 0))


def prefill_flops(cfg):
    D = feature_dim(cfg["fmap"], cfg["d_k"])
    dv = cfg["d_v"]
    score = 2 * D if cfg["fmap"] == "elu1" else 2 * cfg["d_k"] + 4
    per = 4 * D * dv + 4 * D + dv + (C_REF + 1) / 2 * (score + 2 * dv + 1)
    return per * cfg["B"] * cfg["H"] * cfg["N"]


def decode_step_bytes(cfg):
    es = 2 if cfg["dtype"] == "bf16" else 4
    D = feature_dim(cfg["fmap"], cfg["d_k"])
    bh = cfg["B"] * cfg["H"]
    return bh * (2 * D * cfg["d_v"] * 4 + 2 * D * 4
                 + (2 * cfg["d_k"] + 2 * cfg["d_v"]) * es + (4 if cfg.get("gated") else 0))


# Untimed calls before each secondary section of the default run (the
# Taylor, long-sequence, sweep, gated and sliding-window figures) when
# --warmup asks for fewer: the GPU's clocks keep rising over the first ~30 ms
# of sustained work, and these figures are meant at steady clocks whatever
# --warmup the headline is timed with.  The headline keeps --warmup exactly.
SECTION_WARMUP = 600


def prepare_prefill(args, ops, synth, torch, name=PREFILL, override=None, gated=False):
    """Inputs (rotated sets resident in HBM), workspace and the call of one
    prefill configuration; returns (cfg, step, nsets, keep) where step(i)
    runs call i and keep holds the device tensors."""
    cfg = dict(synth.WORKLOADS[name])
    cfg.update(override or {})
    cfg["gated"] = gated
    dev = "cuda:0"
    q, k, v = synth.workload_inputs(name, seed=0, **(override or {}))
    base = [ops.to_device(x, dev) for x in (q, k, v)]
    set_bytes = prefill_bytes(cfg)
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    L = ops.load_library()
    B, H, N, dk, dv = cfg["B"], cfg["H"], cfg["N"], cfg["d_k"], cfg["d_v"]
    fmap = cfg["fmap"]
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    nws = ops.workspace_bytes(fmap, tdt, B, H, N, dk, dv, 0)
    stream = ops._stream(base[0])
    # gated form: a in [0.9, 1) with 0.1% resets
    gate = (torch.from_numpy(synth.draw_gate(B, H, N, seed=0, lo=0.9, reset_p=0.001)).to(dev)
            if gated else None)
    sets = []
    for i in range(nsets):
        qd, kd, vd = (t.clone() for t in base) if i else base
        y = torch.empty_like(vd)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        g = (gate.clone() if i else gate) if gated else None
        sets.append((qd, kd, vd, y, ws, g))
    dcode = 1 if cfg["dtype"] == "bf16" else 0
    if gated:
        fn = L.linattn_prefill_gated
        calls = [(ops.MAPS[fmap], dcode, B, H, N, dk, dv, ops._ptr(s[0]), ops._ptr(s[1]),
                  ops._ptr(s[2]), ops._ptr(s[5]), 1, ops._ptr(s[3]), None, None, None,
                  None, 0, ops._ptr(s[4]), nws, stream) for s in sets]
    else:
        fn = L.linattn_prefill
        calls = [(ops.MAPS[fmap], dcode, B, H, N, dk, dv, ops._ptr(s[0]), ops._ptr(s[1]),
                  ops._ptr(s[2]), ops._ptr(s[3]), None, None, None, None, 0,
                  ops._ptr(s[4]), nws, stream) for s in sets]

    def step(i):
        rc = fn(*calls[i % nsets])
        if rc:
            raise RuntimeError(f"linattn_prefill returned {rc}")

    return cfg, step, nsets, (sets, base)


def time_prefill(args, ops, synth, torch, name=PREFILL, override=None, steps=None,
                 gated=False, warmup=None, prepared=None):
    """Untimed warm-up calls, then the timed calls of one prefill
    configuration (prepared beforehand by prepare_prefill, or here)."""
    if prepared is None:
        prepared = prepare_prefill(args, ops, synth, torch, name=name, override=override,
                                   gated=gated)
    cfg, step, nsets, keep = prepared
    nsteps = args.steps if steps is None else steps
    for i in range(args.warmup if warmup is None else warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(nsteps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / nsteps
    del keep, prepared
    return cfg, ms, nsets


def prefill_record(cfg, ms):
    """tokens/s and the HBM roofline fraction of one timed prefill config."""
    gbs = prefill_bytes(cfg) / (ms * 1e-3) / 1e9
    return {"us_per_call": ms * 1e3, "tokens_per_s": cfg["B"] * cfg["N"] / (ms * 1e-3),
            "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_frac": prefill_flops(cfg) / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def time_decode(args, ops, synth, torch, fmap="taylor2", gated=False):
    cfg = dict(synth.WORKLOADS[DECODE], fmap=fmap, gated=gated)
    dev = "cuda:0"
    pq, pk, pv, sq, sk, sv = synth.workload_inputs(DECODE, seed=0)
    qd, kd, vd = (ops.to_device(x, dev) for x in (pq, pk, pv))
    _, (S, z) = ops.prefill(qd, kd, vd, fmap, return_state=True)
    del qd, kd, vd
    T = cfg["steps"]
    steps = [ops.to_device(x, dev).permute(2, 0, 1, 3).contiguous() for x in (sq, sk, sv)]
    y = torch.empty((T, cfg["B"], cfg["H"], cfg["d_v"]), dtype=torch.bfloat16, device=dev)
    L = ops.load_library()
    stream = ops._stream(S)
    if gated:
        gates = torch.from_numpy(synth.draw_gate(T, cfg["B"], cfg["H"], seed=0, lo=0.9,
                                                 reset_p=0.001)).to(dev)
        fn = L.linattn_decode_step_gated
        calls = [(ops.MAPS[fmap], 1, cfg["B"], cfg["H"], cfg["d_k"], cfg["d_v"],
                  ops._ptr(steps[0][t]), ops._ptr(steps[1][t]), ops._ptr(steps[2][t]),
                  ops._ptr(gates[t]), 1, ops._ptr(S), ops._ptr(z), ops._ptr(y[t]),
                  stream) for t in range(T)]
    else:
        fn = L.linattn_decode_step
        calls = [(ops.MAPS[fmap], 1, cfg["B"], cfg["H"], cfg["d_k"], cfg["d_v"],
                  ops._ptr(steps[0][t]), ops._ptr(steps[1][t]), ops._ptr(steps[2][t]),
                  ops._ptr(S), ops._ptr(z), ops._ptr(y[t]), stream) for t in range(T)]

    def generation():
        for c in calls:
            rc = fn(*c)
            if rc:
                raise RuntimeError(f"linattn_decode_step returned {rc}")

    generation()  # warm-up (continues the state; values stay finite)
    torch.cuda.synchronize()
    reps = max(1, args.decode_reps)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        generation()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / (reps * T)

    # the same 128 steps captured in one HIP graph (launches replayed by the
    # runtime); per-step time = graph time / 128
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = ops._stream(S)
        for c in calls:
            rc = fn(*c[:-1], cap)
            if rc:
                raise RuntimeError(f"linattn_decode_step returned {rc}")
    g.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_graph = ev0.elapsed_time(ev1) / (reps * T)
    ok = bool(torch.isfinite(y.float()).all().item())
    return cfg, ms_step, ok, ms_graph


def time_swa(args, ops, synth, torch):
    """Sliding-window softmax attention: the prefill at the headline shape
    (w = 64) and 128 generation steps after a 1024-token prefill."""
    return {"prefill": time_swa_prefill(args, ops, synth, torch,
                                        warmup=max(args.warmup, SECTION_WARMUP)),
            "decode": time_swa_decode(args, ops, synth, torch)}


def time_swa_prefill(args, ops, synth, torch, warmup=None):
    dev = "cuda:0"
    cfg = synth.WORKLOADS["swa_bf16"]
    B, H, N, d, w = cfg["B"], cfg["H"], cfg["N"], cfg["d_k"], cfg["window"]
    q, k, v = synth.workload_inputs("swa_bf16", seed=0)
    base = [ops.to_device(x, dev) for x in (q, k, v)]
    nbytes = 4 * B * H * N * d * 2
    nsets = max(2, -(-ROTATE_BYTES // nbytes))
    sets = [[t.clone() for t in base] + [torch.empty_like(base[2])] for _ in range(nsets)]
    L = ops.load_library()
    stream = ops._stream(base[0])
    calls = [(1, B, H, N, d, w, d ** -0.5, ops._ptr(s_[0]), ops._ptr(s_[1]), ops._ptr(s_[2]),
              ops._ptr(s_[3]), None, None, stream) for s_ in sets]
    for i in range(args.warmup if warmup is None else warmup):
        assert L.linattn_swa_prefill(*calls[i % nsets]) == 0
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    steps = 100
    ev0.record()
    for i in range(steps):
        L.linattn_swa_prefill(*calls[i % nsets])
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    # MFMA work as executed: 2 key blocks of 64 per 64-query tile, scores and
    # [V | 1] products
    nt = (N + 63) // 64
    mfma_flops = B * H * nt * min(nt, (w + 63) // 64 + 1) * 2 * 64 * 64 * (d + d + 16)
    rec = {
        "workload": f"sliding-window softmax prefill, w={w}, B={B} H={H} N={N} d={d}, bf16",
        "us_per_call": ms * 1e3, "tokens_per_s": B * N / (ms * 1e-3),
        "hbm_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
        "traffic": recorded_traffic("swa_prefill"),
        "mfma_frac_as_executed": mfma_flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
    }
    del sets, base
    return rec


def time_swa_decode(args, ops, synth, torch):
    dev = "cuda:0"
    L = ops.load_library()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    dcfg = synth.WORKLOADS["swa_decode_bf16"]
    B, H, N, d, w, T = (dcfg[x] for x in ("B", "H", "N", "d_k", "window", "steps"))
    pq, pk, pv, sq, sk, sv = synth.workload_inputs("swa_decode_bf16", seed=0)
    qd, kd, vd = (ops.to_device(x, dev) for x in (pq, pk, pv))
    _, (kc, vc) = ops.swa_prefill(qd, kd, vd, w, return_cache=True)
    del qd, kd, vd
    stream = ops._stream(kc)
    st = [ops.to_device(x, dev).permute(2, 0, 1, 3).contiguous() for x in (sq, sk, sv)]
    y = torch.empty((T, B, H, d), dtype=torch.bfloat16, device=dev)
    pos = torch.full((B,), N, dtype=torch.int64, device=dev)
    stepbytes = B * H * (2 * w * d * 2 + 2 * d * 2 + 2 * d * 2) + B * 8
    dcalls = [(1, B, H, d, w, d ** -0.5, ops._ptr(st[0][t]), ops._ptr(st[1][t]),
               ops._ptr(st[2][t]), ops._ptr(pos), ops._ptr(kc), ops._ptr(vc), ops._ptr(y[t]),
               stream) for t in range(T)]
    for c_ in dcalls:
        assert L.linattn_swa_decode_step(*c_) == 0
    torch.cuda.synchronize()
    reps = max(1, args.decode_reps)
    ev0.record()
    for _ in range(reps):
        for c_ in dcalls:
            L.linattn_swa_decode_step(*c_)
    ev1.record()
    torch.cuda.synchronize()
    dms = ev0.elapsed_time(ev1) / (reps * T)
    return {
        "workload": (f"sliding-window generation step, w={w}, {B} sequences x {H} heads, "
                     f"d={d}, bf16, cache from a {N}-token prefill"),
        "ms_per_step": dms, "steps_per_s": 1e3 / dms, "algorithmic_bytes": stepbytes,
        "hbm_frac": stepbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "traffic": recorded_traffic("swa_decode"),
        "finite": bool(torch.isfinite(y.float()).all().item()),
    }


def intra_mfma_probe(torch, iters=2000):
    """MFMA rate of the prefill's within-chunk device code on LDS-resident
    bf16 tiles, looped (liblinattn_probe.so): executed MFMA flops / time."""
    import ctypes

    path = os.path.join(ROOT, "causal_linear_attention_linattn_amd", "liblinattn_probe.so")
    if not os.path.exists(path):
        return None
    P = ctypes.CDLL(path)
    P.linattn_probe_intra_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
    P.linattn_probe_intra_mfma_per_iter.argtypes = [ctypes.c_int]
    out = {}
    for name, m in (("elu1_d64", 0), ("taylor2_d16_dv64", 1)):
        per_iter = P.linattn_probe_intra_mfma_per_iter(m)
        for per_cu in (1, 2, 3):
            wgs = 256 * per_cu
            sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            args = (m, iters, wgs, ctypes.c_void_p(sink.data_ptr()), st)
            if P.linattn_probe_intra_mfma(*args):
                raise RuntimeError("intra-chunk probe launch failed")
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            P.linattn_probe_intra_mfma(*args)
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1)
            flops = wgs * 4 * iters * per_iter * 2 * 16 * 16 * 32
            tf = flops / (ms * 1e-3) / 1e12
            out[f"{name}_{per_cu}wg_per_cu"] = {"tflops": tf,
                                                "frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS}
    return out


# Sources that define the kernels behind each recorded traffic figure: the
# host launch code, the shared device code and the kernels' own files.
DIGEST_FILES = {
    "prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp", "chunk_walk.inc",
                "prefill_elu1_bf16.hip"),
    "decode": ("api.hip", "device.hpp", "shapes.hpp", "decode.hip"),
    "taylor2_prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp",
                        "chunk_walk.inc", "prefill_taylor2_bf16.hip"),
    "gated_prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp",
                      "chunk_walk.inc", "prefill_elu1_bf16_gated.hip"),
    "swa_prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp", "swa.hip"),
    "swa_decode": ("api.hip", "device.hpp", "shapes.hpp", "swa.hip"),
    "long_prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp", "chunk_walk.inc",
                     "prefill_elu1_bf16.hip"),
    "gated_taylor2_prefill": ("api.hip", "device.hpp", "shapes.hpp", "prefill_impl.hpp",
                              "chunk_walk.inc", "prefill_taylor2_bf16_gated.hip"),
}


_CODE_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|\s+', re.S)


def code_text(src):
    """C++ source with comments removed and whitespace runs collapsed, so
    that only edits which can change the compiled code change its hash."""
    def sub(m):
        t = m.group(0)
        if t.startswith("//") or t.startswith("/*") or t.isspace():
            return " "
        return t
    return re.sub(r" +", " ", _CODE_TOKENS.sub(sub, src)).strip()


def csrc_digest(kind="prefill"):
    """Hash of the code (comments and layout excluded) of the HIP sources of
    one kernel family; a traffic figure is valid only for this hash."""
    import hashlib

    d = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_linear_attention_linattn_amd", "csrc")
    for name in DIGEST_FILES[kind]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            d.update(name.encode() + b"\0" + code_text(f.read()).encode())
    return d.hexdigest()[:16]


def recorded_traffic(kind):
    """HBM bytes per call recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (profiles/traffic.txt), scaled by the plain-copy calibration.
    None when the file is missing or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    digest = csrc_digest(kind)
    for line in open(path):
        parts = line.split()
        if len(parts) == 3 and parts[0] == kind and parts[1] == digest:
            return float(parts[2])
    return None


def achievable_peaks(torch):
    """What this device reaches, beside the published peaks: three plain
    1 GiB streams of 16-byte vectors, contiguous ranges per workgroup, best
    of twelve launch shapes each (4, 8 or 16 vectors in flight per thread;
    1024 to 8192 workgroups) (a copy into a second buffer, a read-only pass,
    and an in-place read-and-write pass; bytes moved / time), and a loop of
    independent bf16 16x16x32 MFMAs on registers, at one and two waves per
    SIMD (all in liblinattn_probe.so)."""
    import ctypes

    out = {}
    path = os.path.join(ROOT, "causal_linear_attention_linattn_amd", "liblinattn_probe.so")
    if not os.path.exists(path):
        return None
    P = ctypes.CDLL(path)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    P.linattn_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for mode, name, moved in ((0, "copy", 2 * n), (1, "read", n), (2, "read_write_in_place", 2 * n)):
        best, shape = 0.0, None
        for depth in (4, 8, 16):
            for wgs in (1024, 2048, 4096, 8192):
                args = (mode, depth, ctypes.c_void_p(src.data_ptr()),
                        ctypes.c_void_p(dst.data_ptr()), n, wgs, st)
                for _ in range(2):
                    if P.linattn_probe_stream(*args):
                        raise RuntimeError("stream probe launch failed")
                reps = 8
                ev0.record()
                for _ in range(reps):
                    P.linattn_probe_stream(*args)
                ev1.record()
                torch.cuda.synchronize()
                rate = moved * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
                if rate > best:
                    best, shape = rate, f"{depth} vectors in flight per thread, {wgs} workgroups"
        out[f"hbm_{name}_GBs"] = best
        out[f"hbm_{name}_best_shape"] = shape
    out["hbm_best_frac_of_published"] = max(
        v for k, v in out.items() if k.endswith("_GBs")) / HBM_PEAK_GBS
    del src, dst
    P.linattn_probe_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    iters = 20000
    for per_simd in (1, 2):
        wgs = 256 * per_simd
        sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = (iters, wgs, ctypes.c_void_p(sink.data_ptr()), st)
        if P.linattn_probe_peak_mfma(*args):
            raise RuntimeError("MFMA loop launch failed")
        ev0.record()
        P.linattn_probe_peak_mfma(*args)
        ev1.record()
        torch.cuda.synchronize()
        flops = wgs * 4 * iters * 8 * 2 * 16 * 16 * 32
        tf = flops / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
        out[f"mfma_bf16_loop_TFLOPs_{per_simd}wave_per_simd"] = tf
    best = max(v for k, v in out.items() if k.startswith("mfma_bf16_loop"))
    out["mfma_bf16_loop_frac_of_published"] = best / MFMA_BF16_PEAK_TFLOPS
    return out


def copy_calibration(torch):
    """A plain device copy of known size (256 MiB read + 256 MiB written),
    run under rocprofv3 --pmc to scale FETCH_SIZE / WRITE_SIZE to bytes."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 3}))


def host_identity():
    """CPU model string and the cores this process may run on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


# Worker processes of the CPU baselines: at most this many, one BLAS thread
# each (a one-GPU machine grants its job a share of 16 host cores).
CPU_WORKERS_MAX = 16


def _oracle_worker(kind, w, nworkers, budget_s, barrier, results):
    """One worker of the multi-core oracle baseline (a spawned process).
    Prefill: the float64 recurrence over the (b, h) pairs p = w, w + W, ...
    of the headline workload, at most one batch element's worth of heads
    per oracle call, repeated until the budget is spent.  Decode: the
    128-step generation of the sequences b = w, w + W, ... (all heads) from
    an unseeded state.  Inputs are drawn before the barrier; only the
    oracle's own work is timed."""
    from threadpoolctl import threadpool_limits
    import numpy as np

    import oracle
    from causal_linear_attention_linattn_amd import synth

    with threadpool_limits(limits=1):
        if kind == "prefill":
            cfg = synth.WORKLOADS[PREFILL]
            q, k, v = (x.f64().reshape(cfg["B"] * cfg["H"], cfg["N"], -1)
                       for x in synth.workload_inputs(PREFILL, seed=0))
            pairs = list(range(w, cfg["B"] * cfg["H"], nworkers))
            q, k, v = q[pairs], k[pairs], v[pairs]
            unit = len(pairs) * cfg["N"]            # token-heads per pass
        else:
            cfg = synth.WORKLOADS[DECODE]
            seqs = list(range(w, cfg["B"], nworkers))
            # the step tokens of the generation workload (its stream 1); the
            # state starts unseeded, S = 0 and z = 1 (the oracle's step costs
            # the same for any state values)
            sq, sk, sv = synth.draw_qkv(cfg["B"], cfg["H"], cfg["steps"], cfg["d_k"],
                                        cfg["d_v"], 0, stream=1, dtype=cfg["dtype"],
                                        qk_scale=cfg["qk_scale"])
            q, k, v = (x.f64()[seqs] for x in (sq, sk, sv))
            D = feature_dim("taylor2", cfg["d_k"])
            S0 = np.zeros((len(seqs), cfg["H"], D, cfg["d_v"]))
            z0 = np.ones((len(seqs), cfg["H"], D))
            unit = len(seqs)                        # sequence-steps per step
        barrier.wait()
        t0 = time.perf_counter()
        done = 0
        while True:
            if kind == "prefill":
                for g0 in range(0, len(pairs), cfg["H"]):
                    sl = slice(g0, g0 + cfg["H"])
                    y, _, _ = oracle.attention_recurrent(q[sl], k[sl], v[sl], cfg["fmap"])
                done += unit
            else:
                S, z = S0, z0
                for t in range(cfg["steps"]):
                    y, S, z = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S, z,
                                                 "taylor2")
                done += unit * cfg["steps"]
            assert np.all(np.isfinite(y))
            if time.perf_counter() - t0 >= budget_s:
                break
        t1 = time.perf_counter()
    results.put((w, done, t0, t1))


def _oracle_parallel(kind, nworkers, budget_s):
    """Run the oracle in nworkers spawned processes at once; returns
    (units done, wall seconds from the first start to the last end)."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(nworkers)
    results = ctx.Queue()
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        procs = [ctx.Process(target=_oracle_worker,
                             args=(kind, w, nworkers, budget_s, barrier, results))
                 for w in range(nworkers)]
        for p_ in procs:
            p_.start()
        out = [results.get(timeout=budget_s * 4 + 300) for _ in procs]
        for p_ in procs:
            p_.join()
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    done = sum(o[1] for o in out)
    wall = max(o[3] for o in out) - min(o[2] for o in out)
    return done, wall


def cpu_baseline(synth, budget_s=10.0):
    """The float64 oracle (recurrent form) on the headline prefill workload,
    timed on this host: (b, h) pairs split over one worker process per core
    (one BLAS thread each), and on one core alone."""
    model, host_cores = host_identity()
    cfg = synth.WORKLOADS[PREFILL]
    nw = max(1, min(host_cores, CPU_WORKERS_MAX, cfg["B"] * cfg["H"]))
    done_p, wall_p = _oracle_parallel("prefill", nw, budget_s)
    done_1, wall_1 = _oracle_parallel("prefill", 1, budget_s)
    H = cfg["H"]
    return {"value": done_p / H / wall_p, "unit": "tokens/s", "cores": nw,
            "kind": "oracle",
            "sample": (f"float64 numpy recurrence over the headline workload's "
                       f"{cfg['B'] * cfg['H']} (b,h) pairs (N={cfg['N']}) split over {nw} "
                       f"worker processes, one BLAS thread each, passes repeated for "
                       f"{wall_p:.1f} s: {done_p // cfg['N']} pair-sequences; tokens count "
                       f"all {H} heads"),
            "one_core_value": done_1 / H / wall_1,
            "one_core_sample": f"{done_1 // cfg['N']} pair-sequences on one core, {wall_1:.1f} s",
            "cpu_model": model, "host_cores": host_cores,
            "label": "float64 CPU oracle vs bf16 GPU kernels: context, not like-for-like"}


def cpu_baseline_decode(synth, budget_s=8.0):
    """Oracle decode steps of the generation workload on this host: the
    256 sequences split over worker processes (one BLAS thread each), each
    running the 128 steps of its sequences from an unseeded state (S = 0,
    z = 1); and the same on one core for 1 of every 16 sequences, scaled to
    all 256."""
    model, host_cores = host_identity()
    cfg = synth.WORKLOADS[DECODE]
    nw = max(1, min(host_cores, CPU_WORKERS_MAX, cfg["B"]))
    done_p, wall_p = _oracle_parallel("decode", nw, budget_s)
    # one core: the worker for sequences 0, 16, 32, ... of a 16-way split
    done_1, wall_1 = _oracle_parallel_one("decode", budget_s)
    return {"value": done_p / cfg["B"] / wall_p, "unit": "steps/s", "cores": nw,
            "kind": "oracle",
            "sample": (f"float64 numpy decode steps, {cfg['B']} sequences x {cfg['H']} "
                       f"heads (D=273, d_v={cfg['d_v']}) split over {nw} worker processes, "
                       f"{cfg['steps']} steps per run, {wall_p:.1f} s"),
            "state": "unseeded (S = 0, z = 1); the step's cost does not depend on it",
            "one_core_value": done_1 / cfg["B"] / wall_1,
            "one_core_sample": (f"sequences 0, 16, ..., 240 on one core, {wall_1:.1f} s, "
                                f"scaled to {cfg['B']} sequences"),
            "cpu_model": model, "host_cores": host_cores}


def _oracle_parallel_one(kind, budget_s):
    """One worker process doing 1/16 of the decode sequences alone."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(1)
    results = ctx.Queue()
    p_ = ctx.Process(target=_oracle_worker,
                     args=(kind, 0, CPU_WORKERS_MAX, budget_s, barrier, results))
    p_.start()
    w, done, t0, t1 = results.get(timeout=budget_s * 4 + 300)
    p_.join()
    return done, t1 - t0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The GPU's clocks keep rising for the first ~30 ms of sustained work
    # (48 -> 43.5 us for the same prefill call); 1000 untimed calls put the
    # timed steps at the steady state.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--decode-reps", type=int, default=3,
                    help="128-step generations timed for the decode figure")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the Taylor / long-sequence prefills and the N sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain copy used to scale HBM counters")
    ap.add_argument("--only", choices=("taylor2_prefill", "gated_prefill", "swa_prefill",
                                       "swa_decode", "long_prefill", "gated_taylor2_prefill"),
                    help="time one secondary section alone and print its record "
                         "(for per-kernel profiles of that section)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (sequences and heads shard across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from causal_linear_attention_linattn_amd import synth

    # The CPU baselines run first, in spawned worker processes, before this
    # process touches the GPU.
    cpu_prefill = cpu_decode = None
    if not args.no_cpu_baseline and not args.copy_calibration and not args.only:
        cpu_prefill = cpu_baseline(synth)
        if not args.no_decode:
            cpu_decode = cpu_baseline_decode(synth)

    import torch

    from causal_linear_attention_linattn_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(ops.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ops.load_library()
    torch.cuda.init()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.only:
        if args.only == "taylor2_prefill":
            c, m_, _ = time_prefill(args, ops, synth, torch, name="based_taylor2_bf16")
            rec = prefill_record(c, m_)
        elif args.only == "gated_prefill":
            c, m_, _ = time_prefill(args, ops, synth, torch, gated=True)
            rec = prefill_record(c, m_)
        elif args.only == "long_prefill":
            c, m_, _ = time_prefill(args, ops, synth, torch, name="long_elu1_bf16")
            rec = prefill_record(c, m_)
        elif args.only == "gated_taylor2_prefill":
            c, m_, _ = time_prefill(args, ops, synth, torch, name="based_taylor2_bf16",
                                    gated=True)
            rec = prefill_record(c, m_)
        elif args.only == "swa_prefill":
            rec = time_swa_prefill(args, ops, synth, torch)
        else:
            rec = time_swa_decode(args, ops, synth, torch)
        rec["traffic"] = recorded_traffic(args.only)
        print(json.dumps({"section": args.only, **rec}), flush=True)
        return

    # The headline prefill is timed last: the sections before it keep the
    # GPU busy for a few seconds, so its warm-up calls start from steady
    # clocks (the clocks ramp over the first ~30 ms of sustained work).  Its
    # inputs are drawn and copied to the GPU first, so that no host-side
    # preparation leaves the GPU idle between the last section and its calls.
    headline = prepare_prefill(args, ops, synth, torch)
    others = {}
    if not args.no_other_configs:
        # the other prefill configurations (not the headline line)
        for name in ("based_taylor2_bf16", "long_elu1_bf16"):
            c2, ms2, _ = time_prefill(args, ops, synth, torch, name=name, steps=50,
                                      warmup=max(args.warmup, SECTION_WARMUP))
            others[name] = dict(prefill_record(c2, ms2),
                                workload=(f"prefill {c2['fmap']} B={c2['B']} H={c2['H']} "
                                          f"N={c2['N']} d_k={c2['d_k']} d_v={c2['d_v']} "
                                          f"{c2['dtype']}"))
        others["based_taylor2_bf16"]["traffic"] = recorded_traffic("taylor2_prefill")
        others["long_elu1_bf16"]["traffic"] = recorded_traffic("long_prefill")
        # linear in N: ELU1 bf16, B=1 H=8 d=64, N from 4K to 64K
        sweep = []
        for n in (4096, 8192, 16384, 32768, 65536):
            c3, ms3, _ = time_prefill(args, ops, synth, torch, name="long_elu1_bf16",
                                      override={"N": n}, steps=50,
                                      warmup=max(args.warmup, SECTION_WARMUP))
            sweep.append(dict(N=n, **prefill_record(c3, ms3)))
        others["n_sweep_elu1_b1h8_d64_bf16"] = sweep
        others["sliding_window"] = time_swa(args, ops, synth, torch)
        # the gated (scalar-decay) form on the headline and Taylor shapes
        for name in (PREFILL, "based_taylor2_bf16"):
            c4, ms4, _ = time_prefill(args, ops, synth, torch, name=name, steps=100,
                                      gated=True, warmup=max(args.warmup, SECTION_WARMUP))
            others["gated_" + name] = dict(
                prefill_record(c4, ms4),
                workload=(f"gated prefill (a in [0.9, 1), 0.1% resets) {c4['fmap']} "
                          f"B={c4['B']} H={c4['H']} N={c4['N']} d_k={c4['d_k']} "
                          f"d_v={c4['d_v']} {c4['dtype']}"))
        others["gated_" + PREFILL]["traffic"] = recorded_traffic("gated_prefill")
        others["gated_based_taylor2_bf16"]["traffic"] = recorded_traffic("gated_taylor2_prefill")
    decode_rec = None
    if not args.no_decode:
        dcfg, dms, finite, dms_graph = time_decode(args, ops, synth, torch)
        dbytes = decode_step_bytes(dcfg)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        decode_rec = {
            "value": 1e3 / dms, "unit": "steps/s", "ms_per_step": dms,
            "tokens_per_s": dcfg["B"] * 1e3 / dms, "finite": finite,
            "workload": (f"decode step, Taylor-2 d'={dcfg['d_k']} (D=273), "
                         f"{dcfg['B']} sequences x {dcfg['H']} heads, d_v={dcfg['d_v']}, "
                         f"state seeded by a {dcfg['N']}-token prefill, "
                         f"{dcfg['steps']} steps x {args.decode_reps}"),
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("decode"),
                         "algorithmic_bytes": dbytes},
            "graph": {"ms_per_step": dms_graph, "steps_per_s": 1e3 / dms_graph,
                      "hbm_frac": dbytes / (dms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "note": "the 128 steps captured in one HIP graph and replayed"},
        }
        if not args.no_other_configs:
            scfg, sms, sfinite, sms_graph = time_decode(args, ops, synth, torch,
                                                        "taylor2sym")
            sbytes = decode_step_bytes(scfg)
            decode_rec["unordered_pairs"] = {
                "workload": (f"the same decode with the unordered-pair Taylor map "
                             f"(D={feature_dim('taylor2sym', scfg['d_k'])})"),
                "ms_per_step": sms, "steps_per_s": 1e3 / sms, "finite": sfinite,
                "algorithmic_bytes": sbytes,
                "hbm_frac": sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "graph_ms_per_step": sms_graph,
                "graph_hbm_frac": sbytes / (sms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS,
            }
            gcfg, gms, gfinite, gms_graph = time_decode(args, ops, synth, torch,
                                                        "taylor2", gated=True)
            gbytes = decode_step_bytes(gcfg)
            decode_rec["gated"] = {
                "workload": "the same decode, gated (a in [0.9, 1), 0.1% resets)",
                "ms_per_step": gms, "steps_per_s": 1e3 / gms, "finite": gfinite,
                "algorithmic_bytes": gbytes,
                "hbm_frac": gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "graph_ms_per_step": gms_graph,
            }
    probe = intra_mfma_probe(torch) if not args.no_other_configs else None
    peaks = achievable_peaks(torch) if not args.no_other_configs else None

    cfg, ms, nsets = time_prefill(args, ops, synth, torch, prepared=headline)
    del headline
    tokens = cfg["B"] * cfg["N"]
    nbytes = prefill_bytes(cfg)
    flops = prefill_flops(cfg)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"causal prefill, elu(x)+1, B={cfg['B']} H={cfg['H']} "
                         f"N={cfg['N']} d_k=d_v={cfg['d_k']}, bf16 in/out, fp32 state"),
            "global_batch": cfg["B"], "seq_len": cfg["N"], "heads": cfg["H"],
            "d_k": cfg["d_k"], "d_v": cfg["d_v"], "feature_map": cfg["fmap"],
            "parallelism": "single-gpu", "input_sets_rotated": nsets,
            "seed": 0,
        },
        "roofline": {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic("prefill"),
            "kernel": ("linattn_prefill call: segment-sum pass + chunk-output "
                       "pass (one kernel when a head is one segment)"),
            "csrc_digest": csrc_digest(),
            "algorithmic_bytes": nbytes,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        },
    }
    if others:
        out["other_configs"] = others
    if probe:
        out["roofline"]["intra_chunk_mfma_probe"] = probe
    if peaks:
        peaks["headline_frac_of_read_rate"] = gbs / peaks["hbm_read_GBs"]
        out["roofline"]["achievable_on_device"] = peaks
    if decode_rec is not None:
        out["decode"] = decode_rec
    if cpu_prefill is not None:
        out["cpu_baseline"] = cpu_prefill
        cpu_prefill["gpu_over_cpu"] = out["value"] / cpu_prefill["value"]
        if cpu_decode is not None and "decode" in out:
            cpu_decode["gpu_over_cpu"] = out["decode"]["value"] / cpu_decode["value"]
            out["decode"]["cpu_baseline"] = cpu_decode
        out["cpu_baseline"]["claim_on_pages"] = (
            "the 'Transformers are RNNs' abstract claims linear transformers "
            "are up to 4000 times faster than softmax transformers at "
            "autoregressive prediction of very long sequences; the pages name "
            "no hardware for that figure")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
