"""Parity of the HIP library with the float64 oracle (needs an MI355X).

Every case draws seeded inputs from `synth`, runs them through the C ABI
(via the ctypes binding) and compares element by element with the oracle
on the same stored values.  Tolerances, written per test:
  * float32 inputs: max over rows (b, h, t) of ||y - y_ref|| / ||y_ref||
    <= 1e-4; states: max over (b, h) of ||S - S_ref||_F / ||S_ref||_F
    <= 1e-4.
  * bf16 inputs: the same row norm <= 2e-2 (bf16 MFMA operands, fp32
    accumulation, bf16 output rounding).  Decode states, which are fp32
    throughout, <= 1e-4 when the step starts from an oracle state.
Full-size workloads are checked on sampled rows (the definition evaluated
one row at a time), on the final state of sampled heads, and through the
convex-hull property that every output row satisfies at any size.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_linattn_amd import ops, synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()  # raises if the HIP library is not built
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def row_err(y, ref):
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def state_err(S, ref):
    axes = tuple(range(2, S.ndim))
    num = np.sqrt(np.sum((S - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    return float(np.max(num / np.maximum(den, 1e-300)))


def gpu_prefill(q, k, v, fmap, **kw):
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    out = ops.prefill(qd, kd, vd, fmap, **kw)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------ feature map --
@pytest.mark.parametrize("fmap,d_k", [("elu1", 16), ("elu1", 32), ("elu1", 64),
                                      ("taylor2", 16), ("taylor2sym", 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_feature_map(fmap, d_k, dtype):
    _log(f"feature_map {fmap} d_k={d_k} {dtype}")
    x = synth.draw_qkv(3, 1, 333, d_k, 16, seed=11, dtype=dtype)[0]
    got = ops.to_numpy64(ops.feature_map(ops.to_device(x, DEV), fmap))
    want = oracle.feature_map(x.f64(), fmap)
    assert got.shape == want.shape
    assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)) < 2e-6


# ------------------------------------------------------- tiny fp32 config --
def test_tiny_fp32_prefill_and_decode_match_definition():
    """B=1, H=2, N=256, d=16, fp32, ELU1: prefill and 256 decode steps,
    both against the quadratic masked form (the definition)."""
    _log("tiny_elu1_f32 prefill + 256 decode steps")
    q, k, v = synth.workload_inputs("tiny_elu1_f32", seed=0)
    ref = oracle.attention_quadratic(q.f64(), k.f64(), v.f64(), "elu1")
    S_ref, z_ref = oracle.final_state(k.f64(), v.f64(), "elu1")
    y, (S, z) = gpu_prefill(q, k, v, "elu1", return_state=True)
    assert row_err(ops.to_numpy64(y), ref) <= TOL["f32"]
    assert state_err(ops.to_numpy64(S), S_ref) <= 1e-4
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= 1e-4

    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    Sd = torch.zeros((1, 2, 16, 16), dtype=torch.float32, device=DEV)
    zd = torch.zeros((1, 2, 16), dtype=torch.float32, device=DEV)
    ys = []
    for t in range(256):
        ys.append(ops.decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                  vd[:, :, t].contiguous(), Sd, zd, "elu1"))
    yd = ops.to_numpy64(torch.stack(ys, dim=2))
    assert row_err(yd, ref) <= TOL["f32"]
    assert state_err(ops.to_numpy64(Sd), S_ref) <= 1e-4
    # prefill and decode agree with each other as closely as with the oracle
    assert row_err(yd, ops.to_numpy64(y)) <= 2 * TOL["f32"]


# ----------------------------------------------- small shapes, every kernel --
SHAPES = [("elu1", 16, 16), ("elu1", 32, 32), ("elu1", 64, 64),
          ("taylor2", 16, 16), ("taylor2", 16, 32), ("taylor2", 16, 64),
          ("taylor2sym", 16, 16), ("taylor2sym", 16, 32), ("taylor2sym", 16, 64)]


def _qk_scale(fmap):
    """Taylor maps take q, k scaled by d'^(-1/4), as a model applies them."""
    return 16.0 ** -0.25 if fmap.startswith("taylor2") else 1.0


@pytest.mark.parametrize("fmap,d_k,d_v", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,seg_len", [(1, 0), (63, 0), (65, 64), (200, 64),
                                       (517, 128), (700, 0), (1000, 320), (1100, 512),
                                       (3000, 512)])
def test_prefill_small(fmap, d_k, d_v, dtype, N, seg_len):
    """Every kernel shape against the oracle, including 1- and 5-chunk
    segments.  The last two cases split the Taylor segment-sum pass in two
    (8-chunk segments): with 3 segments the output workgroups add the 4
    preceding part sums themselves, with 6 segments (10 parts) the scan
    kernel forms the prefixes."""
    _log(f"prefill {fmap} {d_k}x{d_v} {dtype} N={N} seg_len={seg_len}")
    scale = _qk_scale(fmap)
    q, k, v = synth.draw_qkv(2, 3, N, d_k, d_v, seed=N, dtype=dtype, qk_scale=scale)
    y_ref, S_ref, z_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), fmap)
    y, (S, z) = gpu_prefill(q, k, v, fmap, return_state=True, seg_len=seg_len)
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64),
                                         ("taylor2sym", 16, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_continues_from_state(fmap, d_k, d_v, dtype):
    """prefill(N1) -> state -> prefill(N2, state) == oracle over N1 + N2;
    also in place (S_out is S_in)."""
    _log(f"prefill continuation {fmap} {dtype}")
    scale = _qk_scale(fmap)
    q, k, v = synth.draw_qkv(1, 4, 448, d_k, d_v, seed=5, dtype=dtype, qk_scale=scale)
    y_ref, S_ref, z_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), fmap)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    n1 = 193
    y1, st = ops.prefill(qd[:, :, :n1].contiguous(), kd[:, :, :n1].contiguous(),
                         vd[:, :, :n1].contiguous(), fmap, return_state=True)
    for seg_len in (0, 64):
        y2, (S2, z2) = ops.prefill(qd[:, :, n1:].contiguous(), kd[:, :, n1:].contiguous(),
                                   vd[:, :, n1:].contiguous(), fmap, state=st,
                                   return_state=True, seg_len=seg_len)
        torch.cuda.synchronize()
        y = np.concatenate([ops.to_numpy64(y1), ops.to_numpy64(y2)], axis=2)
        assert row_err(y, y_ref) <= TOL[dtype]
        assert state_err(ops.to_numpy64(S2), S_ref) <= TOL[dtype]
    # in place: S_out and z_out are the input state tensors
    S_io, z_io = st[0].clone(), st[1].clone()
    L = ops.load_library()
    q2 = qd[:, :, n1:].contiguous()
    k2 = kd[:, :, n1:].contiguous()
    v2 = vd[:, :, n1:].contiguous()
    y2 = torch.empty_like(v2)
    rc = L.linattn_prefill(ops.MAPS[fmap], 0 if dtype == "f32" else 1, 1, 4, 448 - n1,
                           d_k, d_v, ops._ptr(q2), ops._ptr(k2), ops._ptr(v2),
                           ops._ptr(y2), ops._ptr(S_io), ops._ptr(z_io),
                           ops._ptr(S_io), ops._ptr(z_io), 0, None, 0,
                           ops._stream(qd))
    torch.cuda.synchronize()
    assert rc == 0
    assert state_err(ops.to_numpy64(S_io), S_ref) <= TOL[dtype]


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64),
                                         ("taylor2sym", 16, 32)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seg_len", [0, 64])
def test_prefill_from_arbitrary_state(fmap, d_k, d_v, dtype, seg_len):
    """An initial state that no prefill produced: S_in drawn at random (so
    the two rows of a Taylor pair need not agree) and z_in a real running
    sum (so every denominator stays positive).  Outputs and the returned
    state follow the recurrence from exactly that state, through one
    segment or several."""
    _log(f"prefill from an arbitrary state {fmap} {dtype} seg_len={seg_len}")
    scale = _qk_scale(fmap)
    q0, k0, v0 = synth.draw_qkv(1, 3, 100, d_k, d_v, seed=11, dtype="f32", qk_scale=scale)
    z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), fmap)[2]
    D = oracle.feature_dim(fmap, d_k)
    S_in = np.random.default_rng(12).standard_normal((1, 3, D, d_v)) * 4.0
    S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
    q, k, v = synth.draw_qkv(1, 3, 300, d_k, d_v, seed=13, dtype=dtype, qk_scale=scale)
    y_ref, S_ref, z_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), fmap,
                                                     S0=S32.astype(np.float64),
                                                     z0=z32.astype(np.float64))
    st = (torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV))
    y, (S, z) = gpu_prefill(q, k, v, fmap, state=st, return_state=True, seg_len=seg_len)
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seg_len", [0, 64])
def test_prefill_gated_from_arbitrary_state(fmap, d_k, d_v, dtype, seg_len):
    """The gated prefill from a random initial state (as above), with decays
    in [0.99, 1) so that the state still weighs at the end: the initial
    state, its rows that do not agree included, decays with the sequence."""
    _log(f"gated prefill from an arbitrary state {fmap} {dtype} seg_len={seg_len}")
    scale = _qk_scale(fmap)
    q0, k0, v0 = synth.draw_qkv(1, 3, 100, d_k, d_v, seed=21, dtype="f32", qk_scale=scale)
    z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), fmap)[2]
    D = oracle.feature_dim(fmap, d_k)
    S_in = np.random.default_rng(22).standard_normal((1, 3, D, d_v)) * 4.0
    S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
    q, k, v = synth.draw_qkv(1, 3, 300, d_k, d_v, seed=23, dtype=dtype, qk_scale=scale)
    a = synth.draw_gate(1, 3, 300, seed=23, lo=0.99)
    y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(
        q.f64(), k.f64(), v.f64(), a.astype(np.float64), fmap,
        S0=S32.astype(np.float64), z0=z32.astype(np.float64))
    st = (torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV))
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y, (S, z) = ops.prefill_gated(qd, kd, vd, _gate_dev(a), fmap, state=st, return_state=True,
                                  seg_len=seg_len)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("taylor2", 16, 64), ("taylor2sym", 16, 32)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("N", [1024, 1400])
@pytest.mark.parametrize("B,H", [(1, 3), (2, 8)])
def test_prefill_two_segments_pre_pass(fmap, d_k, d_v, dtype, gated, with_state, N, B, H):
    """Two default segments per head (16 and 22 chunks) take the Taylor
    plan without a segment-sum pass: the workgroup of segment 1 walks
    segment 0 first without outputs.  Outputs and the exported state follow
    the recurrence, from zero or from an arbitrary state, plain or gated,
    with a ragged last chunk at N = 1400.  At 16 heads (a multiple of 8)
    the two workgroups of a head are placed on one XCD."""
    _log(f"two-segment pre-pass plan {fmap} {dtype} gated={gated} state={with_state} N={N} B={B} H={H}")
    scale = _qk_scale(fmap)
    q, k, v = synth.draw_qkv(B, H, N, d_k, d_v, seed=N + 7, dtype=dtype, qk_scale=scale)
    S0 = z0 = st = None
    if with_state:
        q0, k0, v0 = synth.draw_qkv(B, H, 100, d_k, d_v, seed=31, dtype="f32", qk_scale=scale)
        z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), fmap)[2]
        D = oracle.feature_dim(fmap, d_k)
        S_in = np.random.default_rng(32).standard_normal((B, H, D, d_v)) * 4.0
        S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
        S0, z0 = S32.astype(np.float64), z32.astype(np.float64)
        st = (torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV))
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    if gated:
        a = synth.draw_gate(B, H, N, seed=N, lo=0.995)
        y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(
            q.f64(), k.f64(), v.f64(), a.astype(np.float64), fmap, S0=S0, z0=z0)
        y, (S, z) = ops.prefill_gated(qd, kd, vd, _gate_dev(a), fmap, state=st,
                                      return_state=True)
    else:
        y_ref, S_ref, z_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), fmap,
                                                         S0=S0, z0=z0)
        y, (S, z) = ops.prefill(qd, kd, vd, fmap, state=st, return_state=True)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


# (B, H, N, d): ELU1 default plans.  At two segments per head (128 to 255
# heads) one launch, in which segment 1's workgroup walks segment 0 first
# (both workgroups of a head on one XCD when the heads fill groups of 8);
# at 3 to 7 segments the segment-sum pass and direct prefixes.
ELU1_PLAN_CASES = [(16, 8, 1100, 64),   # 2 segments, heads in groups of 8
                   (3, 45, 1500, 32),   # 2 segments, 135 heads
                   (9, 16, 1030, 16),   # 2 segments, ragged
                   (5, 17, 1536, 32),   # 3 segments
                   (4, 16, 2000, 64),   # 4 segments, ragged
                   (2, 25, 2560, 16),   # 5 segments
                   (6, 6, 3544, 32)]    # 7 segments, ragged


@pytest.mark.parametrize("B,H,N,d", ELU1_PLAN_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("state", ["zero", "given", "in_place"])
def test_prefill_elu1_default_plans(B, H, N, d, dtype, state):
    """The ELU1 default plans of 2 to 7 segments per head: every output row
    and the exported state follow the recurrence, from zero, from an
    arbitrary state, and in place (S_out = S_in, where the two-segment plan
    takes the segment-sum pass and the scan instead), for both input
    types."""
    _log(f"elu1 default plan B={B} H={H} N={N} d={d} {dtype} state={state}")
    q, k, v = synth.draw_qkv(B, H, N, d, d, seed=N + d, dtype=dtype)
    S0 = z0 = None
    Sd = zd = None
    if state != "zero":
        q0, k0, v0 = synth.draw_qkv(B, H, 90, d, d, seed=33, dtype="f32")
        _, S_in, z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), "elu1")
        S_in = S_in + np.random.default_rng(34).standard_normal(S_in.shape)
        S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
        S0, z0 = S32.astype(np.float64), z32.astype(np.float64)
        Sd, zd = torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV)
    y_ref, S_ref, z_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), "elu1",
                                                     S0=S0, z0=z0)
    L = ops.load_library()
    dt = 0 if dtype == "f32" else 1
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    nws = ops.workspace_bytes("elu1", tdt, B, H, N, d, d, 0)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y = torch.empty_like(vd)
    if state == "in_place":
        S, z = Sd, zd
    else:
        S = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
        z = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    rc = L.linattn_prefill(0, dt, B, H, N, d, d, ops._ptr(qd), ops._ptr(kd), ops._ptr(vd),
                           ops._ptr(y), ops._ptr(Sd), ops._ptr(zd), ops._ptr(S), ops._ptr(z),
                           0, ops._ptr(ws), nws, ops._stream(qd))
    assert rc == 0
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("B,H,N,d", [(16, 8, 1100, 64), (4, 32, 1500, 32), (8, 16, 1030, 16),
                                     (3, 45, 1500, 32)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [False, True])
def test_prefill_gated_elu1_two_segments(B, H, N, d, dtype, with_state):
    """Gated ELU1 at two default segments per head: at 128 heads the
    one-launch pre-pass plan (segment 1's workgroup decays and advances the
    state over segment 0 without outputs), past 128 heads the segment-sum
    plan.  Outputs and the exported state follow the gated recurrence, from
    zero or from an arbitrary state, with resets in the coefficients."""
    _log(f"gated elu1 two segments B={B} H={H} N={N} d={d} {dtype} state={with_state}")
    q, k, v = synth.draw_qkv(B, H, N, d, d, seed=N + 3 * d, dtype=dtype)
    a = synth.draw_gate(B, H, N, seed=N + 1, lo=0.97, reset_p=0.002)
    S0 = z0 = st = None
    if with_state:
        q0, k0, v0 = synth.draw_qkv(B, H, 90, d, d, seed=35, dtype="f32")
        _, S_in, z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), "elu1")
        S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
        S0, z0 = S32.astype(np.float64), z32.astype(np.float64)
        st = (torch.from_numpy(S32).to(DEV), torch.from_numpy(z32).to(DEV))
    y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(
        q.f64(), k.f64(), v.f64(), a.astype(np.float64), "elu1", S0=S0, z0=z0)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y, (S, z) = ops.prefill_gated(qd, kd, vd, _gate_dev(a), "elu1", state=st, return_state=True)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64)])
def test_prefill_deterministic_and_segment_invariant(fmap, d_k, d_v):
    _log(f"determinism / segment invariance {fmap}")
    scale = _qk_scale(fmap)
    q, k, v = synth.draw_qkv(2, 2, 1000, d_k, d_v, seed=3, dtype="bf16", qk_scale=scale)
    y_ref = oracle.attention_recurrent(q.f64(), k.f64(), v.f64(), fmap)[0]
    outs = {}
    for seg_len in (0, 64, 192, 1024):
        a = ops.to_numpy64(gpu_prefill(q, k, v, fmap, seg_len=seg_len))
        b = ops.to_numpy64(gpu_prefill(q, k, v, fmap, seg_len=seg_len))
        assert np.array_equal(a, b), "run-to-run results differ"
        assert row_err(a, y_ref) <= TOL["bf16"]
        outs[seg_len] = a
    for s, a in outs.items():
        assert row_err(a, outs[1024]) <= TOL["bf16"]


@pytest.mark.parametrize("seg_len", [0, 64])
def test_unordered_pair_state_is_the_folded_ordered_state(seg_len):
    """Same inputs through both Taylor maps: the unordered-pair final state
    equals the ordered one folded, (S[a,b] + S[b,a]) / sqrt 2 off the
    diagonal and S[a,a] on it; the outputs agree, since the kernels do."""
    _log(f"taylor2sym vs folded taylor2 state, seg_len={seg_len}")
    q, k, v = synth.draw_qkv(2, 3, 300, 16, 32, seed=8, dtype="f32",
                             qk_scale=_qk_scale("taylor2"))
    y_o, (S_o, z_o) = gpu_prefill(q, k, v, "taylor2", return_state=True, seg_len=seg_len)
    y_s, (S_s, z_s) = gpu_prefill(q, k, v, "taylor2sym", return_state=True, seg_len=seg_len)
    S_o, z_o = ops.to_numpy64(S_o), ops.to_numpy64(z_o)
    S_s, z_s = ops.to_numpy64(S_s), ops.to_numpy64(z_s)
    d = 16
    sq = S_o[:, :, 1 + d:].reshape(2, 3, d, d, 32)
    zq = z_o[:, :, 1 + d:].reshape(2, 3, d, d)
    fold_S = [S_o[:, :, :1 + d]]
    fold_z = [z_o[:, :, :1 + d]]
    for a, b in oracle.sym_pairs(d):
        if a == b:
            fold_S.append(sq[:, :, a, a][:, :, None])
            fold_z.append(zq[:, :, a, a][:, :, None])
        else:
            fold_S.append(((sq[:, :, a, b] + sq[:, :, b, a]) / np.sqrt(2))[:, :, None])
            fold_z.append(((zq[:, :, a, b] + zq[:, :, b, a]) / np.sqrt(2))[:, :, None])
    assert state_err(S_s, np.concatenate(fold_S, axis=2)) <= 1e-5
    assert state_err(z_s[..., None], np.concatenate(fold_z, axis=2)[..., None]) <= 1e-5
    assert row_err(ops.to_numpy64(y_s), ops.to_numpy64(y_o)) <= 1e-5


# ----------------------------------------------------------------- decode --
@pytest.mark.parametrize("fmap,d_k,d_v", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_from_oracle_state(fmap, d_k, d_v, dtype):
    """The state after a random prefix (oracle, float64 -> fp32) feeds both
    sides; 8 decode steps must match the oracle's recurrence."""
    _log(f"decode {fmap} {d_k}x{d_v} {dtype}")
    B, H, P, T = 3, 5, 96, 8
    q, k, v = synth.draw_qkv(B, H, P, d_k, d_v, seed=21, dtype=dtype)
    qs, ks, vs = synth.draw_qkv(B, H, T, d_k, d_v, seed=21, dtype=dtype, stream=1)
    S0, z0 = oracle.final_state(k.f64(), v.f64(), fmap)
    S0 = S0.astype(np.float32)
    z0 = z0.astype(np.float32)
    y_ref, S_ref, z_ref = oracle.attention_recurrent(qs.f64(), ks.f64(), vs.f64(), fmap,
                                                     S0.astype(np.float64),
                                                     z0.astype(np.float64))
    Sd = torch.from_numpy(S0).to(DEV)
    zd = torch.from_numpy(z0).to(DEV)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (qs, ks, vs))
    ys = []
    for t in range(T):
        ys.append(ops.decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                  vd[:, :, t].contiguous(), Sd, zd, fmap))
    torch.cuda.synchronize()
    y = ops.to_numpy64(torch.stack(ys, dim=2))
    assert row_err(y, y_ref) <= TOL[dtype]
    assert state_err(ops.to_numpy64(Sd), S_ref) <= 1e-4
    assert state_err(ops.to_numpy64(zd)[..., None], z_ref[..., None]) <= 1e-4


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64)])
def test_decode_graph_replays_match_eager(fmap, d_k, d_v):
    """Eight decode steps captured in one HIP graph: every replay (state
    reset between replays by an eager copy, other eager work in between)
    gives bit-identical outputs and state to the same steps run eagerly."""
    _log(f"decode graph replays {fmap}")
    B, H, P, T = 3, 4, 64, 8
    q, k, v = synth.draw_qkv(B, H, P, d_k, d_v, seed=31, dtype="bf16")
    qs, ks, vs = synth.draw_qkv(B, H, T, d_k, d_v, seed=31, dtype="bf16", stream=1)
    S0, z0 = oracle.final_state(k.f64(), v.f64(), fmap)
    S0d = torch.from_numpy(S0.astype(np.float32)).to(DEV)
    z0d = torch.from_numpy(z0.astype(np.float32)).to(DEV)
    step = [ops.to_device(x, DEV).permute(2, 0, 1, 3).contiguous() for x in (qs, ks, vs)]

    S_e, z_e = S0d.clone(), z0d.clone()
    y_e = [ops.decode_step(step[0][t], step[1][t], step[2][t], S_e, z_e, fmap)
           for t in range(T)]
    torch.cuda.synchronize()

    S_g, z_g = S0d.clone(), z0d.clone()
    y_g = torch.empty((T, B, H, d_v), dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(T):
            ops.decode_step(step[0][t], step[1][t], step[2][t], S_g, z_g, fmap, out=y_g[t])
    for r in range(3):
        S_g.copy_(S0d)
        z_g.copy_(z0d)
        junk = (S0d * 2.0).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for t in range(T):
            assert torch.equal(y_g[t], y_e[t]), (r, t)
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e), r


@pytest.mark.parametrize("case", ["one_segment", "part_sums", "scan", "taylor_state",
                                  "taylor_pre_pass", "gated_taylor_pre_pass", "gated",
                                  "elu1_pre_pass", "sliding_window"])
def test_prefill_graph_replays_match_eager(case):
    """Prefill calls captured in one HIP graph: every replay (other eager work
    in between) gives bit-identical outputs and final states to the same
    calls run eagerly.  The cases cover one segment per head, output
    workgroups adding their predecessors' part sums, the scan kernel, the
    Taylor state export, the Taylor two-segment plan without a segment-sum
    pass (plain and gated), the same plan for ELU1, the gated form, and the
    sliding-window prefill
    with a generation step (its caches restored by an eager copy before
    each replay)."""
    _log(f"prefill graph replays {case}")
    fmap, d_k, d_v, N, seg = {"one_segment": ("elu1", 64, 64, 300, 0),
                              "part_sums": ("elu1", 64, 64, 1000, 192),
                              "scan": ("elu1", 64, 64, 1000, 64),
                              "taylor_state": ("taylor2", 16, 64, 700, 64),
                              "taylor_pre_pass": ("taylor2", 16, 64, 1024, 0),
                              "gated_taylor_pre_pass": ("taylor2", 16, 64, 1024, 0),
                              "gated": ("elu1", 64, 64, 1000, 64),
                              "elu1_pre_pass": ("elu1", 64, 64, 1100, 0),
                              "sliding_window": ("elu1", 64, 64, 700, 0)}[case]
    q, k, v = synth.draw_qkv(2, 3, N, d_k, d_v, seed=41, dtype="bf16", qk_scale=_qk_scale(fmap))
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    ad = _gate_dev(synth.draw_gate(2, 3, N, seed=41, reset_p=0.01))
    w = 64
    qs, ks, vs = (ops.to_device(x, DEV)[:, :, 0].contiguous()
                  for x in synth.draw_qkv(2, 3, 1, d_k, d_v, seed=41, dtype="bf16", stream=1))
    pos = torch.full((2,), N, dtype=torch.int64, device=DEV)

    def run(caches=None):
        if case == "sliding_window":
            y, (kc, vc) = ops.swa_prefill(qd, kd, vd, w, return_cache=True)
            kc2, vc2 = caches if caches is not None else (kc, vc)
            yd = ops.swa_decode_step(qs, ks, vs, pos, kc2, vc2, w)
            return [y, yd, kc2, vc2]
        if case.startswith("gated"):
            y, (S, z) = ops.prefill_gated(qd, kd, vd, ad, fmap, return_state=True, seg_len=seg)
            return [y, S, z]
        y, (S, z) = ops.prefill(qd, kd, vd, fmap, return_state=True, seg_len=seg)
        return [y, S, z]

    if case == "sliding_window":
        _, (kc0, vc0) = ops.swa_prefill(qd, kd, vd, w, return_cache=True)
        kc_g, vc_g = kc0.clone(), vc0.clone()
        eager = run((kc0.clone(), vc0.clone()))
    else:
        eager = run()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = run((kc_g, vc_g)) if case == "sliding_window" else run()
    for r in range(3):
        if case == "sliding_window":
            kc_g.copy_(kc0)
            vc_g.copy_(vc0)
        junk = (vd.float() * 2.0).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (a, b) in enumerate(zip(captured, eager)):
            assert torch.equal(a, b), (r, i)


# ------------------------------------------- in place, many segments ------
def _segment_ends(t0, n, seg_len):
    """First and last row (global index) of every segment of one call."""
    rows = set()
    for s in range(0, n, seg_len):
        rows.add(t0 + s)
        rows.add(t0 + min(s + seg_len, n) - 1)
    return rows


@pytest.mark.parametrize("fmap,d_k,d_v,B,H", [("elu1", 64, 64, 32, 8),
                                              ("taylor2", 16, 64, 8, 8),
                                              ("taylor2sym", 16, 32, 8, 8)])
@pytest.mark.parametrize("gated", [False, True])
def test_prefill_in_place_many_segments(fmap, d_k, d_v, B, H, gated):
    """Continuation in place (S_out is S_in, z_out is z_in) through calls
    of 1, 4, 3 and 9 segments per head (seg_len 64, 128, 64) with many heads,
    so that the segments of one head run on different XCDs in no fixed
    order.  The first and last row of every segment of every call and the
    final state of every head follow the oracle's recurrence over the whole
    concatenated sequence."""
    if gated:
        B //= 2   # the gated row oracle forms running decay products per row
    _log(f"prefill in place, many segments {fmap} gated={gated} B={B} H={H}")
    parts = [(100, 0), (256, 64), (384, 128), (576, 64)]   # (tokens, seg_len)
    N = sum(n for n, _ in parts)
    q, k, v = synth.draw_qkv(B, H, N, d_k, d_v, seed=21, dtype="bf16",
                             qk_scale=_qk_scale(fmap))
    a = synth.draw_gate(B, H, N, seed=21, lo=0.9, reset_p=0.002) if gated else None
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    ad = _gate_dev(a) if gated else None
    D = oracle.feature_dim(fmap, d_k)
    S = torch.zeros((B, H, D, d_v), dtype=torch.float32, device=DEV)
    z = torch.zeros((B, H, D), dtype=torch.float32, device=DEV)
    L = ops.load_library()
    m = ops.MAPS[fmap]
    y = torch.empty_like(vd)
    rows = set()
    t0 = 0
    for n, seg_len in parts:
        sl = lambda x: x[:, :, t0:t0 + n].contiguous()
        qs, ks, vs = sl(qd), sl(kd), sl(vd)
        ys = torch.empty_like(vs)
        nws = ops.workspace_bytes(fmap, torch.bfloat16, B, H, n, d_k, d_v, seg_len)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
        if gated:
            gs = ad[:, :, t0:t0 + n].contiguous()
            rc = L.linattn_prefill_gated(m, 1, B, H, n, d_k, d_v, ops._ptr(qs), ops._ptr(ks),
                                         ops._ptr(vs), ops._ptr(gs), 1, ops._ptr(ys),
                                         ops._ptr(S), ops._ptr(z), ops._ptr(S), ops._ptr(z),
                                         seg_len, ops._ptr(ws), nws, ops._stream(qd))
        else:
            rc = L.linattn_prefill(m, 1, B, H, n, d_k, d_v, ops._ptr(qs), ops._ptr(ks),
                                   ops._ptr(vs), ops._ptr(ys), ops._ptr(S), ops._ptr(z),
                                   ops._ptr(S), ops._ptr(z), seg_len, ops._ptr(ws), nws,
                                   ops._stream(qd))
        assert rc == 0
        y[:, :, t0:t0 + n] = ys
        rows |= _segment_ends(t0, n, seg_len or n)
        t0 += n
    torch.cuda.synchronize()
    y = ops.to_numpy64(y)
    S = ops.to_numpy64(S)
    z = ops.to_numpy64(z)
    q64, k64, v64 = q.f64(), k.f64(), v.f64()
    rng = np.random.default_rng(22)
    rows = sorted(rows | set(rng.integers(0, N, 8).tolist()))
    for b in range(B):
        for h in range(H):
            if gated:
                ref = oracle.attention_gated_rows(q64[b, h], k64[b, h], v64[b, h],
                                                  a[b, h].astype(np.float64), fmap, rows)
            else:
                ref = oracle.attention_rows(q64[b, h], k64[b, h], v64[b, h], fmap, rows)
            assert row_err(y[b, h, rows], ref) <= TOL["bf16"], (b, h)
    if gated:
        S_ref, z_ref = oracle.gated_final_state(k64, v64, a.astype(np.float64), fmap)
    else:
        S_ref, z_ref = oracle.final_state(k64, v64, fmap)
    assert state_err(S, S_ref) <= TOL["bf16"]
    assert state_err(z[..., None], z_ref[..., None]) <= TOL["bf16"]


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("seg_len", [0, 64])
def test_prefill_in_place_from_arbitrary_ordered_state(gated, seg_len):
    """In place (S_out is S_in) from a random ordered Taylor state whose rows
    (a, b) and (b, a) differ: the kernels walk only the symmetric part of the
    pair block, and the export adds the antisymmetric part back (decayed, in
    the gated form) from the same S_in it overwrites.  One segment and five
    (the scanned path that aliasing takes), 32 heads; all outputs and the
    final state against the oracle's recurrence from that state."""
    fmap, d_k, d_v, B, H, N = "taylor2", 16, 64, 4, 8, 300
    _log(f"prefill in place from an arbitrary ordered state gated={gated} seg_len={seg_len}")
    scale = _qk_scale(fmap)
    q0, k0, v0 = synth.draw_qkv(B, H, 100, d_k, d_v, seed=31, dtype="f32", qk_scale=scale)
    z_in = oracle.attention_recurrent(q0.f64(), k0.f64(), v0.f64(), fmap)[2]
    D = oracle.feature_dim(fmap, d_k)
    S_in = np.random.default_rng(32).standard_normal((B, H, D, d_v)) * 4.0
    S32, z32 = S_in.astype(np.float32), z_in.astype(np.float32)
    q, k, v = synth.draw_qkv(B, H, N, d_k, d_v, seed=33, dtype="bf16", qk_scale=scale)
    a = synth.draw_gate(B, H, N, seed=33, lo=0.99) if gated else None
    if gated:
        y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(
            q.f64(), k.f64(), v.f64(), a.astype(np.float64), fmap,
            S0=S32.astype(np.float64), z0=z32.astype(np.float64))
    else:
        y_ref, S_ref, z_ref = oracle.attention_recurrent(
            q.f64(), k.f64(), v.f64(), fmap, S0=S32.astype(np.float64),
            z0=z32.astype(np.float64))
    S = torch.from_numpy(S32).to(DEV)
    z = torch.from_numpy(z32).to(DEV)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y = torch.empty_like(vd)
    nws = ops.workspace_bytes(fmap, torch.bfloat16, B, H, N, d_k, d_v, seg_len)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    L = ops.load_library()
    m = ops.MAPS[fmap]
    if gated:
        ad = _gate_dev(a)
        rc = L.linattn_prefill_gated(m, 1, B, H, N, d_k, d_v, ops._ptr(qd), ops._ptr(kd),
                                     ops._ptr(vd), ops._ptr(ad), 1, ops._ptr(y),
                                     ops._ptr(S), ops._ptr(z), ops._ptr(S), ops._ptr(z),
                                     seg_len, ops._ptr(ws), nws, ops._stream(qd))
    else:
        rc = L.linattn_prefill(m, 1, B, H, N, d_k, d_v, ops._ptr(qd), ops._ptr(kd),
                               ops._ptr(vd), ops._ptr(y), ops._ptr(S), ops._ptr(z),
                               ops._ptr(S), ops._ptr(z), seg_len, ops._ptr(ws), nws,
                               ops._stream(qd))
    assert rc == 0
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


# ------------------------------------------------------- gated form ------
def _gate_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("fmap,d_k,d_v", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,seg_len", [(1, 0), (63, 0), (65, 64), (200, 64),
                                       (517, 128), (700, 0), (1100, 512), (3000, 512)])
def test_prefill_gated_small(fmap, d_k, d_v, dtype, N, seg_len):
    """Gated prefill (a in [0.8, 1) with 2% resets) against the oracle's
    gated recurrence, outputs and final state, ragged tails and segments."""
    _log(f"prefill_gated {fmap} {d_k}x{d_v} {dtype} N={N} seg_len={seg_len}")
    q, k, v = synth.draw_qkv(2, 3, N, d_k, d_v, seed=N, dtype=dtype,
                             qk_scale=_qk_scale(fmap))
    a = synth.draw_gate(2, 3, N, seed=N, reset_p=0.02)
    y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(q.f64(), k.f64(), v.f64(),
                                                           a.astype(np.float64), fmap)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y, (S, z) = ops.prefill_gated(qd, kd, vd, _gate_dev(a), fmap, return_state=True,
                                  seg_len=seg_len)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert row_err(ops.to_numpy64(y), y_ref) <= tol
    assert state_err(ops.to_numpy64(S), S_ref) <= tol
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64),
                                         ("taylor2sym", 16, 32)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate_kind", ["strong", "resets", "ones", "unnormalized"])
def test_prefill_gated_regimes(fmap, d_k, d_v, dtype, gate_kind):
    """Strong decay (a in [0, 0.5)), frequent resets, a = 1 (must equal the
    plain prefill) and the unnormalised read, over many segments (the
    scanned prefix) and a continuation from a state."""
    _log(f"prefill_gated regime {gate_kind} {fmap} {dtype}")
    B, H, N = 1, 4, 1000
    q, k, v = synth.draw_qkv(B, H, N, d_k, d_v, seed=41, dtype=dtype,
                             qk_scale=_qk_scale(fmap))
    if gate_kind == "strong":
        a = synth.draw_gate(B, H, N, seed=41, lo=0.0, hi=0.5)
    elif gate_kind == "resets":
        a = synth.draw_gate(B, H, N, seed=41, lo=0.9, hi=1.0, reset_p=0.1)
    elif gate_kind == "ones":
        a = np.ones((B, H, N), dtype=np.float32)
    else:
        a = synth.draw_gate(B, H, N, seed=41, lo=0.95, hi=1.0, reset_p=0.01)
    normalize = gate_kind != "unnormalized"
    a64 = a.astype(np.float64)
    y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(q.f64(), k.f64(), v.f64(),
                                                           a64, fmap, normalize=normalize)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    ad = _gate_dev(a)
    tol = TOL[dtype]
    for seg_len in (0, 64, 192):
        y, (S, z) = ops.prefill_gated(qd, kd, vd, ad, fmap, normalize=normalize,
                                      return_state=True, seg_len=seg_len)
        torch.cuda.synchronize()
        assert row_err(ops.to_numpy64(y), y_ref) <= tol, seg_len
        assert state_err(ops.to_numpy64(S), S_ref) <= tol, seg_len
        assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= tol, seg_len
    if gate_kind == "ones":
        y_plain = ops.prefill(qd, kd, vd, fmap, seg_len=64)
        y_g = ops.prefill_gated(qd, kd, vd, ad, fmap, seg_len=64)
        torch.cuda.synchronize()
        assert row_err(ops.to_numpy64(y_g), ops.to_numpy64(y_plain)) <= 1e-5
    # continuation through a state: prefix 0..n1, then the rest
    n1 = 321
    sl = lambda x, lo, hi: x[:, :, lo:hi].contiguous()
    _, st = ops.prefill_gated(sl(qd, 0, n1), sl(kd, 0, n1), sl(vd, 0, n1),
                              ad[:, :, :n1].contiguous(), fmap, normalize=normalize,
                              return_state=True)
    y2, (S2, _) = ops.prefill_gated(sl(qd, n1, N), sl(kd, n1, N), sl(vd, n1, N),
                                    ad[:, :, n1:].contiguous(), fmap, normalize=normalize,
                                    state=st, return_state=True, seg_len=64)
    torch.cuda.synchronize()
    assert row_err(ops.to_numpy64(y2), y_ref[:, :, n1:]) <= tol
    assert state_err(ops.to_numpy64(S2), S_ref) <= tol


@pytest.mark.parametrize("fmap,d_k,d_v", [("elu1", 64, 64), ("taylor2", 16, 64),
                                         ("taylor2sym", 16, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("normalize", [True, False])
def test_decode_gated_from_oracle_state(fmap, d_k, d_v, dtype, normalize):
    """Gated steps from an oracle state (a prefix of 96 gated tokens), with
    some steps resetting, against the oracle's gated recurrence."""
    _log(f"decode_gated {fmap} {dtype} normalize={normalize}")
    B, H, P, T = 3, 5, 96, 8
    q, k, v = synth.draw_qkv(B, H, P, d_k, d_v, seed=51, dtype=dtype)
    qs, ks, vs = synth.draw_qkv(B, H, T, d_k, d_v, seed=51, dtype=dtype, stream=1)
    a0 = synth.draw_gate(B, H, P, seed=51)
    a = synth.draw_gate(B, H, T, seed=51, lo=0.5, reset_p=0.1, stream=3)
    S0, z0 = oracle.gated_final_state(k.f64(), v.f64(), a0.astype(np.float64), fmap)
    S0 = S0.astype(np.float32)
    z0 = z0.astype(np.float32)
    y_ref, S_ref, z_ref = oracle.attention_gated_recurrent(
        qs.f64(), ks.f64(), vs.f64(), a.astype(np.float64), fmap,
        S0.astype(np.float64), z0.astype(np.float64), normalize=normalize)
    Sd = torch.from_numpy(S0).to(DEV)
    zd = torch.from_numpy(z0).to(DEV)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (qs, ks, vs))
    ad = _gate_dev(a)
    ys = []
    for t in range(T):
        ys.append(ops.decode_step_gated(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                        vd[:, :, t].contiguous(), ad[:, :, t].contiguous(),
                                        Sd, zd, fmap, normalize=normalize))
    torch.cuda.synchronize()
    y = ops.to_numpy64(torch.stack(ys, dim=2))
    assert row_err(y, y_ref) <= TOL[dtype]
    assert state_err(ops.to_numpy64(Sd), S_ref) <= 1e-4
    assert state_err(ops.to_numpy64(zd)[..., None], z_ref[..., None]) <= 1e-4


def test_gated_prefill_then_decode_matches_one_recurrence():
    """Gated prefill writes the state, gated decode continues it: the same
    numbers as one gated recurrence over both parts."""
    _log("gated prefill -> gated decode")
    fmap, d_k, d_v = "taylor2sym", 16, 64
    B, H, P, T = 2, 3, 300, 6
    q, k, v = synth.draw_qkv(B, H, P + T, d_k, d_v, seed=61, dtype="bf16",
                             qk_scale=_qk_scale(fmap))
    a = synth.draw_gate(B, H, P + T, seed=61, lo=0.9, reset_p=0.01)
    y_ref, S_ref, _ = oracle.attention_gated_recurrent(q.f64(), k.f64(), v.f64(),
                                                       a.astype(np.float64), fmap)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    ad = _gate_dev(a)
    y1, (S, z) = ops.prefill_gated(qd[:, :, :P].contiguous(), kd[:, :, :P].contiguous(),
                                   vd[:, :, :P].contiguous(), ad[:, :, :P].contiguous(),
                                   fmap, return_state=True)
    ys = [ops.decode_step_gated(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                vd[:, :, t].contiguous(), ad[:, :, t].contiguous(),
                                S, z, fmap) for t in range(P, P + T)]
    torch.cuda.synchronize()
    y = np.concatenate([ops.to_numpy64(y1), ops.to_numpy64(torch.stack(ys, dim=2))], axis=2)
    assert row_err(y, y_ref) <= TOL["bf16"]
    assert state_err(ops.to_numpy64(S), S_ref) <= TOL["bf16"]


# ---------------------------------------------------- sliding window ------
def _stored_f64(x):
    return x.f64()


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,w", [(1, 1), (63, 64), (65, 16), (200, 64), (517, 100),
                                 (300, 1000), (130, 1)])
def test_swa_prefill_small(d, dtype, N, w):
    """Sliding-window prefill against the oracle's band-masked softmax, and
    the ring cache it leaves (bit-exact copies of k, v rows)."""
    _log(f"swa_prefill d={d} {dtype} N={N} w={w}")
    q, k, v = synth.draw_qkv(2, 3, N, d, d, seed=N + w, dtype=dtype)
    scale = d ** -0.5
    y_ref = oracle.swa_attention(q.f64(), k.f64(), v.f64(), w, scale)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y, (kc, vc) = ops.swa_prefill(qd, kd, vd, w, return_cache=True)
    torch.cuda.synchronize()
    assert row_err(ops.to_numpy64(y), y_ref) <= TOL[dtype]
    kc_ref, vc_ref = oracle.swa_cache_after_prefill(k.f64(), v.f64(), w)
    assert np.array_equal(ops.to_numpy64(kc), kc_ref)
    assert np.array_equal(ops.to_numpy64(vc), vc_ref)


def test_swa_default_scale_is_one_over_sqrt_d():
    """The sliding-window entry points take NaN for their default softmax
    scale 1/sqrt(d): bit-identical to passing that scale, and an explicit
    scale is honoured (checked against the oracle at scale 0.3)."""
    _log("swa default scale")
    d, w, N = 64, 48, 300
    q, k, v = synth.draw_qkv(2, 3, N, d, d, seed=77, dtype="bf16")
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y0 = ops.swa_prefill(qd, kd, vd, w)
    y1 = ops.swa_prefill(qd, kd, vd, w, scale=d ** -0.5)
    y2 = ops.swa_prefill(qd, kd, vd, w, scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert row_err(ops.to_numpy64(y2), oracle.swa_attention(q.f64(), k.f64(), v.f64(), w, 0.3)) <= TOL["bf16"]
    _, (kc, vc) = ops.swa_prefill(qd, kd, vd, w, return_cache=True)
    qs, ks, vs = (ops.to_device(x, DEV)[:, :, 0].contiguous()
                  for x in synth.draw_qkv(2, 3, 1, d, d, seed=78, dtype="bf16", stream=1))
    pos = torch.full((2,), N, dtype=torch.int64, device=DEV)
    kc2, vc2 = kc.clone(), vc.clone()
    z0 = ops.swa_decode_step(qs, ks, vs, pos, kc, vc, w)
    z1 = ops.swa_decode_step(qs, ks, vs, pos, kc2, vc2, w, scale=d ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(z0, z1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("w", [64, 100])
def test_swa_prefill_long_runs(dtype, w):
    """B=1 H=2 N=70000 (a ragged last tile), w spanning 2 and 3 key blocks
    per tile: rows at the start, around tile boundaries, at the end and a
    random sample against the oracle's single rows."""
    _log(f"swa_prefill long runs {dtype} w={w}")
    d, N = 64, 70000
    q, k, v = synth.draw_qkv(1, 2, N, d, d, seed=w, dtype=dtype)
    scale = d ** -0.5
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y = ops.to_numpy64(ops.swa_prefill(qd, kd, vd, w))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w)
    rows = sorted(set(list(range(0, 130)) + list(range(300, 340)) + list(range(635, 645))
                      + list(range(N - 70, N)) + rng.integers(0, N, 60).tolist()))
    q64, k64, v64 = q.f64(), k.f64(), v.f64()
    for h in range(2):
        ref = oracle.swa_rows(q64[0, h], k64[0, h], v64[0, h], w, scale, rows)
        assert row_err(y[0, h, rows], ref) <= TOL[dtype], h


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("w,P", [(64, 100), (16, 5), (100, 40), (128, 130), (200, 300),
                                 (1000, 50)])
def test_swa_decode_continues_prefill(d, dtype, w, P):
    """Prefill P tokens (writing the caches), then 12 decode steps: every
    step's output equals the oracle's dense form over all P + 12 tokens.
    Windows up to 128 take the preloading step kernel, larger ones the
    looping one."""
    _log(f"swa_decode d={d} {dtype} w={w} P={P}")
    B, H, T = 2, 3, 12
    q, k, v = synth.draw_qkv(B, H, P + T, d, d, seed=7 + w, dtype=dtype)
    scale = 0.7 * d ** -0.5
    y_ref = oracle.swa_attention(q.f64(), k.f64(), v.f64(), w, scale)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    sl = lambda x: x[:, :, :P].contiguous()
    _, (kc, vc) = ops.swa_prefill(sl(qd), sl(kd), sl(vd), w, scale=scale, return_cache=True)
    pos = torch.full((B,), P, dtype=torch.int64, device=DEV)
    ys = []
    for t in range(P, P + T):
        ys.append(ops.swa_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                      vd[:, :, t].contiguous(), pos, kc, vc, w, scale=scale))
        pos += 1
    torch.cuda.synchronize()
    y = ops.to_numpy64(torch.stack(ys, dim=2))
    assert row_err(y, y_ref[:, :, P:]) <= TOL[dtype]
    kc_ref, vc_ref = oracle.swa_cache_after_prefill(k.f64(), v.f64(), w)
    assert np.array_equal(ops.to_numpy64(kc), kc_ref)
    assert np.array_equal(ops.to_numpy64(vc), vc_ref)


def test_swa_decode_positions_per_sequence():
    """Sequences at different positions in one step (one from an empty cache
    at 0, one deep in the ring), and a negative position: NaN output and an
    untouched cache for that sequence only."""
    _log("swa_decode per-sequence positions")
    d, w, T = 64, 32, 40
    q, k, v = synth.draw_qkv(3, 2, 200, d, d, seed=9, dtype="f32")
    scale = d ** -0.5
    starts = [0, 150, 0]
    kc = np.zeros((3, 2, w, d), dtype=np.float32)
    vc = np.zeros((3, 2, w, d), dtype=np.float32)
    k64, v64 = k.f64(), v.f64()
    kc1, vc1 = oracle.swa_cache_after_prefill(k64[1:2, :, :150], v64[1:2, :, :150], w)
    kc[1:2], vc[1:2] = kc1, vc1
    kcd = torch.from_numpy(kc).to(DEV)
    vcd = torch.from_numpy(vc).to(DEV)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    pos = torch.tensor([0, 150, -1], dtype=torch.int64, device=DEV)
    ys = []
    for t in range(T):
        idx = torch.tensor([starts[0] + t, starts[1] + t, 0], device=DEV)
        pick = lambda x: torch.stack([x[b, :, idx[b]] for b in range(3)]).contiguous()
        ys.append(ops.swa_decode_step(pick(qd), pick(kd), pick(vd), pos, kcd, vcd, w))
        pos[:2] += 1
    torch.cuda.synchronize()
    y = ops.to_numpy64(torch.stack(ys, dim=2))       # [3, 2, T, d]
    q64 = q.f64()
    for b in range(2):
        for h in range(2):
            rows = list(range(starts[b], starts[b] + T))
            ref = oracle.swa_rows(q64[b, h], k64[b, h], v64[b, h], w, scale, rows)
            assert row_err(y[b, h], ref) <= TOL["f32"], (b, h)
    assert np.all(np.isnan(y[2]))
    assert np.array_equal(ops.to_numpy64(kcd[2]), np.zeros((2, w, d)))


# ------------------------------------------------------ full-size configs --
def _sampled_rows(n, rng, count=32):
    rows = set([0, n - 1]) | set(rng.integers(0, n, size=count).tolist())
    return sorted(rows)


def _default_segments(BH, N):
    """Segment length (tokens) of the library's default plan: enough
    segments per head for about 256 workgroups, each of at least 8 chunks
    of 64 tokens (the plan formed in csrc/api.hip)."""
    nchunks = -(-N // 64)
    nseg = max(1, min(-(-256 // BH), max(1, nchunks // 8)))
    return 64 * -(-nchunks // nseg)


@pytest.mark.parametrize("name,rows_per_head", [("layer_elu1_bf16", 8),
                                                ("based_taylor2_bf16", 8),
                                                ("long_elu1_bf16", 64)])
def test_full_size_prefill(name, rows_per_head):
    """Full-size workloads in the default launch configuration.  Every
    (b, h) is checked against the definition on t = 0, t = N - 1, the first
    and last row of every segment of the default plan (up to N = 4096: of
    every chunk) and random rows (rows_per_head in all, at least); the final
    state of every head against its closed form; every row against the
    convex hull."""
    _log(f"full-size prefill {name}")
    cfg = synth.WORKLOADS[name]
    fmap = cfg["fmap"]
    B, H, N = cfg["B"], cfg["H"], cfg["N"]
    q, k, v = synth.workload_inputs(name, seed=0)
    y, (S, z) = gpu_prefill(q, k, v, fmap, return_state=True)
    y = ops.to_numpy64(y)
    assert np.all(np.isfinite(y))
    # convex hull: every output coordinate lies within the running min/max of v
    v64 = v.f64()
    lo = np.minimum.accumulate(v64, axis=2)
    hi = np.maximum.accumulate(v64, axis=2)
    slack = 2e-2 * (hi - lo) + 1e-6
    assert np.all(y >= lo - slack) and np.all(y <= hi + slack)
    del lo, hi, slack
    seg = _default_segments(B * H, N)
    ends = {0, N - 1} | _segment_ends(0, N, seg)
    if N <= 4096:
        # both rows at every chunk boundary: whatever segment lengths the
        # plan picks (the two-segment plans split unevenly), each segment's
        # first and last rows are among them
        ends |= {t for c in range(1, -(-N // 64)) for t in (64 * c - 1, 64 * c)}
    ends = sorted(ends)
    rng = np.random.default_rng(1)
    q64, k64 = q.f64(), k.f64()
    for b in range(B):
        for h in range(H):
            extra = max(4, rows_per_head - len(ends))
            rows = sorted(set(ends) | set(rng.integers(0, N, size=extra).tolist()))
            ref = oracle.attention_rows(q64[b, h], k64[b, h], v64[b, h], fmap, rows)
            assert row_err(y[b, h, rows], ref) <= TOL["bf16"], (b, h)
    S_ref, z_ref = oracle.final_state(k64, v64, fmap)
    assert state_err(ops.to_numpy64(S), S_ref) <= TOL["bf16"]
    assert state_err(ops.to_numpy64(z)[..., None], z_ref[..., None]) <= TOL["bf16"]


def test_full_size_gated_prefill():
    """The bench workload (ELU1, B=8 H=8 N=4096 d=64, bf16) with a in
    [0.9, 1) and 0.1% resets, default launch: sampled rows and final states
    of sampled heads against the oracle's gated definition."""
    _log("full-size gated prefill layer_elu1_bf16")
    name = "layer_elu1_bf16"
    cfg = synth.WORKLOADS[name]
    fmap = cfg["fmap"]
    B, H, N = cfg["B"], cfg["H"], cfg["N"]
    q, k, v = synth.workload_inputs(name, seed=0)
    a = synth.draw_gate(B, H, N, seed=0, lo=0.9, reset_p=0.001)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    y, (S, z) = ops.prefill_gated(qd, kd, vd, _gate_dev(a), fmap, return_state=True)
    torch.cuda.synchronize()
    y = ops.to_numpy64(y)
    S = ops.to_numpy64(S)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(3)
    q64, k64, v64 = q.f64(), k.f64(), v.f64()
    a64 = a.astype(np.float64)
    for _ in range(6):
        b, h = int(rng.integers(0, B)), int(rng.integers(0, H))
        rows = _sampled_rows(N, rng)
        ref = oracle.attention_gated_rows(q64[b, h], k64[b, h], v64[b, h], a64[b, h],
                                          fmap, rows)
        assert row_err(y[b, h, rows], ref) <= TOL["bf16"], (b, h)
        S_ref, _ = oracle.gated_final_state(k64[b, h], v64[b, h], a64[b, h], fmap)
        assert state_err(S[b, h][None, None], S_ref[None, None]) <= TOL["bf16"]


def test_full_size_swa_prefill_and_decode():
    """The bench-shaped sliding window (bf16, B=8 H=8 N=4096 d=64, w=64):
    sampled rows of the prefill against the oracle, then 16 decode steps of
    all 64 sequences x heads continuing its cache."""
    _log("full-size swa prefill + decode")
    B, H, N, d, w, T = 8, 8, 4096, 64, 64, 16
    q, k, v = synth.draw_qkv(B, H, N + T, d, d, seed=0, dtype="bf16")
    scale = d ** -0.5
    qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
    sl = lambda x: x[:, :, :N].contiguous()
    y, (kc, vc) = ops.swa_prefill(sl(qd), sl(kd), sl(vd), w, return_cache=True)
    pos = torch.full((B,), N, dtype=torch.int64, device=DEV)
    ys = []
    for t in range(N, N + T):
        ys.append(ops.swa_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                      vd[:, :, t].contiguous(), pos, kc, vc, w))
        pos += 1
    torch.cuda.synchronize()
    y = ops.to_numpy64(y)
    yd = ops.to_numpy64(torch.stack(ys, dim=2))
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(yd))
    q64, k64, v64 = q.f64(), k.f64(), v.f64()
    rng = np.random.default_rng(4)
    for _ in range(8):
        b, h = int(rng.integers(0, B)), int(rng.integers(0, H))
        rows = _sampled_rows(N, rng)
        ref = oracle.swa_rows(q64[b, h], k64[b, h], v64[b, h], w, scale, rows)
        assert row_err(y[b, h, rows], ref) <= TOL["bf16"], (b, h)
        ref = oracle.swa_rows(q64[b, h], k64[b, h], v64[b, h], w, scale,
                              list(range(N, N + T)))
        assert row_err(yd[b, h], ref) <= TOL["bf16"], (b, h)


@pytest.mark.parametrize("fmap", ["taylor2", "taylor2sym"])
def test_full_size_decode_after_prefill(fmap):
    """256 sequences x 16 heads, Taylor d'=16: the state seeded by the
    library's own prefill over a 1024-token prefix, then 128 decode steps.
    Sampled heads are checked against the oracle's recurrence over all
    1024 + 128 tokens; every output row must lie in the convex hull."""
    _log(f"full-size decode {fmap} (prefill 1024 + 128 steps)")
    name = "decode_taylor2_bf16"
    cfg = synth.WORKLOADS[name]
    pq, pk, pv, sq, sk, sv = synth.workload_inputs(name, seed=0)
    qd, kd, vd = (ops.to_device(x, DEV) for x in (pq, pk, pv))
    _, (Sd, zd) = ops.prefill(qd, kd, vd, fmap, return_state=True)
    del qd, kd, vd
    sqd, skd, svd = (ops.to_device(x, DEV) for x in (sq, sk, sv))
    T = cfg["steps"]
    ys = torch.empty((T,) + tuple(svd.shape[:2]) + (cfg["d_v"],), dtype=svd.dtype,
                     device=DEV)
    step_q = sqd.permute(2, 0, 1, 3).contiguous()
    step_k = skd.permute(2, 0, 1, 3).contiguous()
    step_v = svd.permute(2, 0, 1, 3).contiguous()
    for t in range(T):
        ops.decode_step(step_q[t], step_k[t], step_v[t], Sd, zd, fmap, out=ys[t])
    torch.cuda.synchronize()
    y = ops.to_numpy64(ys)                       # [T, B, H, d_v]
    assert np.all(np.isfinite(y))
    # convex hull over every sequence and head
    pv32 = _f32(pv)
    lo, hi = pv32.min(axis=2), pv32.max(axis=2)  # [B, H, d_v]
    sv32 = _f32(sv)
    for t in range(T):
        lo = np.minimum(lo, sv32[:, :, t])
        hi = np.maximum(hi, sv32[:, :, t])
        slack = 2e-2 * (hi - lo) + 1e-6
        assert np.all(y[t] >= lo - slack) and np.all(y[t] <= hi + slack), t
    del pv32, sv32
    rng = np.random.default_rng(2)
    S = ops.to_numpy64(Sd)
    for _ in range(8):
        b, h = int(rng.integers(0, cfg["B"])), int(rng.integers(0, cfg["H"]))
        qa = np.concatenate([_f32(pq, b, h), _f32(sq, b, h)]).astype(np.float64)
        ka = np.concatenate([_f32(pk, b, h), _f32(sk, b, h)]).astype(np.float64)
        va = np.concatenate([_f32(pv, b, h), _f32(sv, b, h)]).astype(np.float64)
        rows = list(range(cfg["N"], cfg["N"] + T))
        ref = oracle.attention_rows(qa, ka, va, fmap, rows)
        assert row_err(y[:, b, h], ref) <= TOL["bf16"], (b, h)
        S_ref, _ = oracle.final_state(ka, va, fmap)
        assert state_err(S[b, h][None, None], S_ref[None, None]) <= TOL["bf16"]


def _f32(stored, *idx):
    """Stored values (or one [b, h] slice of them) as float32."""
    data = stored.data[idx] if idx else stored.data
    if stored.dtype == "f32":
        return np.asarray(data, dtype=np.float32)
    return synth.bf16_bits_to_f32(data)
