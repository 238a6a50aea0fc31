"""Seeded synthetic inputs for causal linear attention.

This module holds none of the method's arithmetic.  It draws i.i.d. Gaussian
q, k, v from a counter-free PCG64 stream and rounds them to their storage type
(float32, or bfloat16 by round-to-nearest-even of the float32 value).  The HIP
library and the float64 oracle both consume exactly these stored values.

Recipe (fixed, so a seed names one input set):
  * generator: numpy.random.Generator(PCG64([seed, stream]))
  * draw order: q, then k, then v, each standard normal float64 in C order
    [B, H, N, d]
  * q and k are multiplied by `qk_scale` (1 unless the workload says
    otherwise: the Taylor prefill shape scales them by d'^(-1/4))
  * cast to float32; for bf16 storage, then rounded to nearest-even bf16.

The workloads below are the shapes the benchmark and the parity tests use:
the 4096-token prefill and the batched 1024-token generation of
"Simple linear attention language models balance the recall-throughput
tradeoff" (Knowl 5, Knowl 9) with d' = 16, d = 64 as in Knowl 5.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# name -> shape and storage; every workload is synthetic (seeded Gaussian).
WORKLOADS = {
    "tiny_elu1_f32": dict(fmap="elu1", dtype="f32", B=1, H=2, N=256,
                          d_k=16, d_v=16, qk_scale=1.0),
    "layer_elu1_bf16": dict(fmap="elu1", dtype="bf16", B=8, H=8, N=4096,
                            d_k=64, d_v=64, qk_scale=1.0),
    "based_taylor2_bf16": dict(fmap="taylor2", dtype="bf16", B=8, H=16,
                               N=2048, d_k=16, d_v=64,
                               qk_scale=16.0 ** -0.25),
    "long_elu1_bf16": dict(fmap="elu1", dtype="bf16", B=1, H=8, N=65536,
                           d_k=64, d_v=64, qk_scale=1.0),
    # generation: a 1024-token prefix seeds the state, then 128 single-token
    # steps; q, k, v plain N(0, 1).
    "decode_taylor2_bf16": dict(fmap="taylor2", dtype="bf16", B=256, H=16,
                                N=1024, steps=128, d_k=16, d_v=64,
                                qk_scale=1.0),
    # sliding-window softmax attention (w = 64, d = 64): a prefill of the
    # headline shape, and generation continuing a 1024-token prefill
    "swa_bf16": dict(fmap="swa", dtype="bf16", B=8, H=8, N=4096, d_k=64,
                     d_v=64, window=64, qk_scale=1.0),
    "swa_decode_bf16": dict(fmap="swa", dtype="bf16", B=256, H=16, N=1024,
                            steps=128, d_k=64, d_v=64, window=64,
                            qk_scale=1.0),
}


def bf16_bits_rne(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Stored:
    """One tensor as the device receives it: float32 values or bf16 bits."""

    data: np.ndarray        # float32, or uint16 bf16 bit patterns
    dtype: str              # "f32" or "bf16"

    def f64(self) -> np.ndarray:
        """The exact stored values, widened to float64 (what the oracle uses)."""
        if self.dtype == "f32":
            return self.data.astype(np.float64)
        return bf16_bits_to_f32(self.data).astype(np.float64)

    @property
    def shape(self):
        return self.data.shape


def _store(x64: np.ndarray, dtype: str) -> Stored:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return Stored(x32, "f32")
    if dtype == "bf16":
        return Stored(bf16_bits_rne(x32), "bf16")
    raise ValueError(f"unknown storage dtype {dtype!r}")


def draw_qkv(B, H, N, d_k, d_v, seed, *, dtype="bf16", qk_scale=1.0,
             stream=0):
    """Draw q, k ([B,H,N,d_k]) and v ([B,H,N,d_v]); returns (q, k, v) Stored."""
    rng = np.random.Generator(np.random.PCG64([int(seed), int(stream)]))
    q = rng.standard_normal((B, H, N, d_k))
    k = rng.standard_normal((B, H, N, d_k))
    v = rng.standard_normal((B, H, N, d_v))
    if qk_scale != 1.0:
        q *= qk_scale
        k *= qk_scale
    return _store(q, dtype), _store(k, dtype), _store(v, dtype)


def draw_gate(B, H, N, seed, *, lo=0.8, hi=1.0, reset_p=0.0, stream=2):
    """Decay coefficients a [B, H, N] (float32): uniform on [lo, hi), and
    exactly 0 with probability reset_p.  The pages give no distribution for
    them; this spans mild decay, strong decay and resets."""
    rng = np.random.Generator(np.random.PCG64([int(seed), int(stream)]))
    a = rng.uniform(lo, hi, size=(B, H, N))
    if reset_p > 0.0:
        a = np.where(rng.uniform(size=(B, H, N)) < reset_p, 0.0, a)
    return a.astype(np.float32)


def workload_inputs(name, seed=0, **override):
    """Inputs of a named workload (shape overrides allowed for small cases).

    Prefill workloads return (q, k, v).  The generation workload returns
    (prefix_q, prefix_k, prefix_v, step_q, step_k, step_v): the prefix is
    [B,H,N,d] from stream 0, the step tokens [B,H,steps,d] from stream 1.
    """
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    args = (cfg["B"], cfg["H"], cfg["N"], cfg["d_k"], cfg["d_v"], seed)
    kw = dict(dtype=cfg["dtype"], qk_scale=cfg["qk_scale"])
    if "steps" not in cfg:
        return draw_qkv(*args, **kw)
    prefix = draw_qkv(*args, stream=0, **kw)
    steps = draw_qkv(cfg["B"], cfg["H"], cfg["steps"], cfg["d_k"],
                     cfg["d_v"], seed, stream=1, **kw)
    return prefix + steps
