"""Python binding of liblinattn.so: argument marshalling only.

Every step of the computation runs in the HIP library.  PyTorch supplies
device memory and the current HIP stream; nothing here computes on the
data.  If the library is missing the first call raises ImportError -- there
is no fallback path.

Entry points (same names as the C ABI in include/linattn.h):
    feature_map(x, fmap)                      -> phi(x) float32 [..., D]
    prefill(q, k, v, fmap, state=None, ...)   -> y (and the final state)
    decode_step(q, k, v, S, z, fmap)          -> y; S, z updated in place
    prefill_noalloc(q, k, v, fmap, ...)       -> as prefill; the library's
                                                 fixed scratch, no workspace
    prefill_gated(q, k, v, gate, fmap, ...)   -> y (and the final state)
    decode_step_gated(q, k, v, gate, S, z, fmap) -> y; S, z updated in place
    swa_prefill(q, k, v, window, ...)          -> y (and the ring cache)
    swa_decode_step(q, k, v, pos, kc, vc, window) -> y; caches updated
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "liblinattn.so")

MAPS = {"elu1": 0, "taylor2": 1, "taylor2sym": 2}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace",
           4: "hip error", 5: "fixed scratch too small"}

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"linattn status {status}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the library; raises ImportError if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run "
            "`python -m causal_linear_attention_linattn_amd._build`")
    L = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    fp = ctypes.c_void_p
    L.linattn_status_string.argtypes = [i32]
    L.linattn_status_string.restype = ctypes.c_char_p
    L.linattn_version.argtypes = []
    L.linattn_version.restype = i32
    L.linattn_feature_dim.argtypes = [i32, i64]
    L.linattn_feature_dim.restype = i64
    L.linattn_supported.argtypes = [i32, i32, i64, i64]
    L.linattn_supported.restype = i32
    L.linattn_feature_map.argtypes = [i32, i32, vp, i64, i64, fp, vp]
    L.linattn_feature_map.restype = i32
    L.linattn_prefill_workspace_bytes.argtypes = [i32, i32, i64, i64, i64, i64,
                                                  i64, i64]
    L.linattn_prefill_workspace_bytes.restype = sz
    L.linattn_prefill.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp,
                                  vp, fp, fp, fp, fp, i64, vp, sz, vp]
    L.linattn_prefill.restype = i32
    L.linattn_decode_step.argtypes = [i32, i32, i64, i64, i64, i64, vp, vp, vp,
                                      fp, fp, vp, vp]
    L.linattn_decode_step.restype = i32
    L.linattn_prefill_gated.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp,
                                        fp, i32, vp, fp, fp, fp, fp, i64, vp, sz, vp]
    L.linattn_prefill_gated.restype = i32
    L.linattn_prefill_noalloc.argtypes = [i32, i32, i64, i64, i64, i64, i64, vp, vp, vp,
                                          vp, fp, fp, fp, fp, i64, vp]
    L.linattn_prefill_noalloc.restype = i32
    L.linattn_decode_step_gated.argtypes = [i32, i32, i64, i64, i64, i64, vp, vp, vp,
                                            fp, i32, fp, fp, vp, vp]
    L.linattn_decode_step_gated.restype = i32
    L.linattn_swa_prefill.argtypes = [i32, i64, i64, i64, i64, i64, ctypes.c_float, vp, vp,
                                      vp, vp, vp, vp, vp]
    L.linattn_swa_prefill.restype = i32
    L.linattn_swa_decode_step.argtypes = [i32, i64, i64, i64, i64, ctypes.c_float, vp, vp,
                                          vp, vp, vp, vp, vp, vp]
    L.linattn_swa_decode_step.restype = i32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().linattn_status_string(status).decode()
        raise LinAttnError(status, msg)


def _map_id(fmap: str) -> int:
    try:
        return MAPS[fmap]
    except KeyError:
        raise ValueError(f"unknown feature map {fmap!r}; expected one of "
                         f"{sorted(MAPS)}") from None


def _dtype_id(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"dtype {t.dtype} is not supported (float32, bfloat16)") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    """Every given tensor lives on one GPU device and is contiguous."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("linattn tensors must live on a GPU device")
        if not t.is_contiguous():
            raise ValueError("linattn tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"linattn tensors must share one device ({dev} vs {t.device})")


def _expect(name, t, shape, dtype):
    """t has exactly this shape and dtype (checked before any device use, so
    a mis-sized buffer never reaches the library, which sizes every access
    from the shape arguments)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _qkv(q, k, v, ndim):
    """q, k [..., d_k] and v [..., d_v] over the same leading dims, one dtype."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError(f"expected q, k of one shape and v with the same leading dims; "
                         f"got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    _dtype_id(q)


def feature_dim(fmap: str, d_k: int) -> int:
    return int(load_library().linattn_feature_dim(_map_id(fmap), d_k))


def supported(fmap: str, dtype: torch.dtype, d_k: int, d_v: int) -> bool:
    return bool(load_library().linattn_supported(_map_id(fmap), _DTYPES[dtype],
                                                 d_k, d_v))


def workspace_bytes(fmap, dtype, B, H, N, d_k, d_v, seg_len=0) -> int:
    n = load_library().linattn_prefill_workspace_bytes(
        _map_id(fmap), _DTYPES[dtype], B, H, N, d_k, d_v, seg_len)
    if n == ctypes.c_size_t(-1).value:
        raise LinAttnError(1, "invalid or unsupported prefill shape")
    return int(n)


def feature_map(x: torch.Tensor, fmap: str) -> torch.Tensor:
    """phi(x) over the last axis, float32 [..., D] (test/inspection export)."""
    L = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise TypeError("x must be a torch.Tensor with a feature axis")
    _dtype_id(x)
    _need_cuda(x)
    d_k = x.shape[-1]
    D = feature_dim(fmap, d_k)
    rows = x.numel() // d_k if d_k else 0
    out = torch.empty(x.shape[:-1] + (D,), dtype=torch.float32, device=x.device)
    _check(L.linattn_feature_map(_map_id(fmap), _dtype_id(x), _ptr(x), rows,
                                 d_k, _ptr(out), _stream(x)))
    return out


def prefill(q, k, v, fmap: str, *, state=None, return_state=False,
            seg_len: int = 0, out=None):
    """Causal linear attention over [B, H, N, d] inputs.

    state: optional (S, z) float32 tensors [B,H,D,d_v], [B,H,D] to continue
    from.  return_state: also return the final (S, z).  seg_len: tokens per
    workgroup segment (0 = library choice, else a multiple of 64).
    """
    return _prefill(q, k, v, None, True, fmap, state, return_state, seg_len, out)


def prefill_noalloc(q, k, v, fmap: str, *, state=None, return_state=False,
                    seg_len: int = 0, out=None):
    """prefill() through linattn_prefill_noalloc: the segment part sums go to
    the library's fixed device array instead of a workspace (the library call
    allocates nothing; this wrapper allocates y and the state only when they
    are not passed in as out= / returned)."""
    return _prefill(q, k, v, None, True, fmap, state, return_state, seg_len, out,
                    noalloc=True)


def prefill_gated(q, k, v, gate, fmap: str, *, normalize=True, state=None,
                  return_state=False, seg_len: int = 0, out=None):
    """Gated (scalar-decay) prefill: gate is float32 [B, H, N] holding a_t;
    S_t = a_t S_{t-1} + phi(k_t)^T v_t (and z).  normalize=False returns the
    numerator phi(q_t) S_t.  Other arguments as prefill()."""
    return _prefill(q, k, v, gate, normalize, fmap, state, return_state, seg_len, out)


def _prefill(q, k, v, gate, normalize, fmap, state, return_state, seg_len, out,
             noalloc=False):
    L = load_library()
    _qkv(q, k, v, 4)
    B, H, N, d_k = q.shape
    d_v = v.shape[-1]
    D = feature_dim(fmap, d_k)
    if out is not None:
        _expect("out", out, v.shape, v.dtype)
    S_in = z_in = None
    if state is not None:
        S_in, z_in = state
        _expect("state S", S_in, (B, H, D, d_v), torch.float32)
        _expect("state z", z_in, (B, H, D), torch.float32)
    if gate is not None:
        _expect("gate", gate, (B, H, N), torch.float32)
    _need_cuda(q, k, v, out, S_in, z_in, gate)
    y = out if out is not None else torch.empty_like(v)
    S_out = z_out = None
    if return_state:
        S_out = torch.empty((B, H, D, d_v), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    if noalloc:
        _check(L.linattn_prefill_noalloc(_map_id(fmap), _dtype_id(q), B, H, N, d_k, d_v,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(S_in),
                                         _ptr(z_in), _ptr(S_out), _ptr(z_out), seg_len,
                                         _stream(q)))
        return (y, (S_out, z_out)) if return_state else y
    nws = workspace_bytes(fmap, q.dtype, B, H, N, d_k, d_v, seg_len)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    if gate is None:
        _check(L.linattn_prefill(_map_id(fmap), _dtype_id(q), B, H, N, d_k, d_v,
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(S_in),
                                 _ptr(z_in), _ptr(S_out), _ptr(z_out), seg_len,
                                 _ptr(ws), nws, _stream(q)))
    else:
        _check(L.linattn_prefill_gated(_map_id(fmap), _dtype_id(q), B, H, N, d_k, d_v,
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                       1 if normalize else 0, _ptr(y), _ptr(S_in),
                                       _ptr(z_in), _ptr(S_out), _ptr(z_out), seg_len,
                                       _ptr(ws), nws, _stream(q)))
    if return_state:
        return y, (S_out, z_out)
    return y


def decode_step(q, k, v, S, z, fmap: str, *, out=None):
    """One generation step; q, k [B,H,d_k], v [B,H,d_v].  S, z updated in place."""
    return _decode(q, k, v, None, True, S, z, fmap, out)


def decode_step_gated(q, k, v, gate, S, z, fmap: str, *, normalize=True, out=None):
    """One gated step: S = a S + phi(k)^T v, z = a z + phi(k)^T with gate
    float32 [B, H] holding a; then the read as in prefill_gated."""
    return _decode(q, k, v, gate, normalize, S, z, fmap, out)


def _decode(q, k, v, gate, normalize, S, z, fmap, out):
    L = load_library()
    _qkv(q, k, v, 3)
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    D = feature_dim(fmap, d_k)
    _expect("S", S, (B, H, D, d_v), torch.float32)
    _expect("z", z, (B, H, D), torch.float32)
    if out is not None:
        _expect("out", out, v.shape, v.dtype)
    if gate is not None:
        _expect("gate", gate, (B, H), torch.float32)
    _need_cuda(q, k, v, S, z, out, gate)
    y = out if out is not None else torch.empty_like(v)
    if gate is None:
        _check(L.linattn_decode_step(_map_id(fmap), _dtype_id(q), B, H, d_k, d_v,
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                                     _ptr(y), _stream(q)))
    else:
        _check(L.linattn_decode_step_gated(_map_id(fmap), _dtype_id(q), B, H, d_k, d_v,
                                           _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                           1 if normalize else 0, _ptr(S), _ptr(z),
                                           _ptr(y), _stream(q)))
    return y


def swa_prefill(q, k, v, window: int, *, scale=None, return_cache=False, out=None):
    """Sliding-window softmax attention over [B, H, N, d] inputs.

    scale defaults to 1/sqrt(d) (the library's choice, passed as NaN).  return_cache: also return the ring caches
    (k_cache, v_cache) [B, H, window, d] for swa_decode_step."""
    L = load_library()
    _qkv(q, k, v, 4)
    if v.shape != q.shape:
        raise ValueError("expected q, k, v [B,H,N,d] of one shape")
    B, H, N, d = q.shape
    sc = float("nan") if scale is None else float(scale)  # NaN: the library's 1/sqrt(d)
    if out is not None:
        _expect("out", out, v.shape, v.dtype)
    _need_cuda(q, k, v, out)
    y = out if out is not None else torch.empty_like(v)
    kc = vc = None
    if return_cache:
        kc = torch.empty((B, H, window, d), dtype=q.dtype, device=q.device)
        vc = torch.empty_like(kc)
    _check(L.linattn_swa_prefill(_dtype_id(q), B, H, N, d, window, sc, _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(y), _ptr(kc), _ptr(vc), _stream(q)))
    if return_cache:
        return y, (kc, vc)
    return y


def swa_decode_step(q, k, v, pos, k_cache, v_cache, window: int, *, scale=None, out=None):
    """One sliding-window generation step; q, k, v [B,H,d]; pos int64 [B]
    (0-based position of this token per sequence); caches updated in place."""
    L = load_library()
    _qkv(q, k, v, 3)
    if v.shape != q.shape:
        raise ValueError("expected q, k, v [B,H,d] of one shape")
    B, H, d = q.shape
    _expect("pos", pos, (B,), torch.int64)
    _expect("k_cache", k_cache, (B, H, window, d), q.dtype)
    _expect("v_cache", v_cache, (B, H, window, d), q.dtype)
    if out is not None:
        _expect("out", out, v.shape, v.dtype)
    _need_cuda(q, k, v, pos, k_cache, v_cache, out)
    sc = float("nan") if scale is None else float(scale)  # NaN: the library's 1/sqrt(d)
    y = out if out is not None else torch.empty_like(v)
    _check(L.linattn_swa_decode_step(_dtype_id(q), B, H, d, window, sc, _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(pos), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(y), _stream(q)))
    return y


# ---------------------------------------------------------------- helpers --
def to_device(stored, device) -> torch.Tensor:
    """A synth.Stored array (float32 or bf16 bits) as a device tensor."""
    if stored.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored.data)).to(device)
    bits = np.ascontiguousarray(stored.data).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).to(device)


def to_numpy64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (exact widening of its values)."""
    return t.detach().to("cpu", torch.float32).double().numpy()
