"""linattn_prefill_noalloc -- the prefill whose segment part sums live in the
library's fixed device array instead of a caller workspace -- against
linattn_prefill with a workspace, on the same inputs, through the C ABI.

Both entry points run the same kernels with the same segment plan, so their
outputs must be bit-identical; each is also held to the float64 oracle's
tolerance (2e-2 row-relative for bf16 inputs, 1e-4 for float32).  Two calls
follow each other on one stream, the second smaller than the first, so the
second runs over what the first left in the shared array."""
import numpy as np
import pytest
import torch

import oracle
from causal_linear_attention_linattn_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ops.load_library()
    torch.cuda.init()


def _row_err(y, ref):
    return float(np.max(np.linalg.norm(y - ref, axis=-1) /
                        np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)))


def _run(L, noalloc, fmap, dtype, B, H, N, d_k, d_v, qd, kd, vd, state, seg_len):
    D = oracle.feature_dim(fmap, d_k)
    y = torch.empty_like(vd)
    S = torch.empty((B, H, D, d_v), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
    Si, zi = state if state is not None else (None, None)
    m, dt = ops.MAPS[fmap], 0 if dtype == "f32" else 1
    common = (m, dt, B, H, N, d_k, d_v, ops._ptr(qd), ops._ptr(kd), ops._ptr(vd), ops._ptr(y),
              ops._ptr(Si), ops._ptr(zi), ops._ptr(S), ops._ptr(z), seg_len)
    if noalloc:
        rc = L.linattn_prefill_noalloc(*common, ops._stream(qd))
    else:
        nws = ops.workspace_bytes(fmap, qd.dtype, B, H, N, d_k, d_v, seg_len)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
        rc = L.linattn_prefill(*common, ops._ptr(ws), nws, ops._stream(qd))
    assert rc == 0, rc
    return y, S, z


@pytest.mark.parametrize("fmap,d_k,d_v,dtype", [("elu1", 64, 64, "bf16"),
                                                ("taylor2", 16, 64, "bf16"),
                                                ("taylor2sym", 16, 32, "bf16"),
                                                ("elu1", 16, 16, "f32")])
def test_noalloc_matches_the_workspace_prefill(fmap, d_k, d_v, dtype):
    L = ops.load_library()
    scale = 16.0 ** -0.25 if fmap.startswith("taylor2") else 1.0
    # (B, H, N, seg_len): 16 segments per head (the scan kernel forms the
    # prefixes), then a smaller call of 3 segments (direct prefixes) that
    # continues from the first call's final state
    calls = [(4, 4, 1000, 64), (2, 3, 333, 128)]
    state = None
    for i, (B, H, N, seg_len) in enumerate(calls):
        print(f"noalloc {fmap} {dtype} call {i}: B={B} H={H} N={N} seg_len={seg_len}",
              flush=True)
        q, k, v = synth.draw_qkv(B, H, N, d_k, d_v, seed=30 + i, dtype=dtype, qk_scale=scale)
        qd, kd, vd = (ops.to_device(x, DEV) for x in (q, k, v))
        st = None
        S0 = z0 = None
        if state is not None:
            S0 = state[0][:B, :H].contiguous()
            z0 = state[1][:B, :H].contiguous()
            st = (S0, z0)
        y_ws, S_ws, z_ws = _run(L, False, fmap, dtype, B, H, N, d_k, d_v, qd, kd, vd, st, seg_len)
        y_na, S_na, z_na = _run(L, True, fmap, dtype, B, H, N, d_k, d_v, qd, kd, vd, st, seg_len)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws)
        assert torch.equal(S_na, S_ws)
        assert torch.equal(z_na, z_ws)
        y_ref, S_ref, _ = oracle.attention_recurrent(
            q.f64(), k.f64(), v.f64(), fmap,
            S0=None if S0 is None else ops.to_numpy64(S0),
            z0=None if z0 is None else ops.to_numpy64(z0))
        assert _row_err(ops.to_numpy64(y_na), y_ref) <= TOL[dtype]
        num = np.sqrt(np.sum((ops.to_numpy64(S_na) - S_ref) ** 2, axis=(2, 3)))
        assert np.max(num / np.sqrt(np.sum(S_ref ** 2, axis=(2, 3)))) <= TOL[dtype]
        state = (S_na, z_na)
