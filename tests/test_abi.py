"""The C ABI on the CPU: it builds, loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU is touched here:
every call below fails validation, which happens before the runtime is
used)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

from causal_linear_attention_linattn_amd import ops  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from causal_linear_attention_linattn_amd import _build
        _build.build()
    return ops.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(linattn_[a-z_0-9]+)\s*\(", text)))


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "linattn.h"\nint main(void){return linattn_version() > 0 ? 0 : 1;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                    "-I", os.path.join(ROOT, "include"), str(src)], check=True)


def test_c_program_links(tmp_path, lib):
    src = tmp_path / "use.c"
    src.write_text(
        '#include <stdio.h>\n#include "linattn.h"\n'
        "int main(void){\n"
        '  printf("%d %lld\\n", linattn_version(), (long long)linattn_feature_dim(LINATTN_MAP_TAYLOR2, 16));\n'
        "  return linattn_prefill(0,1,1,1,1,64,64,0,0,0,0,0,0,0,0,0,0,0,0) == LINATTN_ERR_INVALID_ARGUMENT ? 0 : 1;\n"
        "}\n")
    exe = tmp_path / "use"
    libdir = os.path.dirname(ops.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), f"-L{libdir}", "-llinattn",
                    f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True)
    assert out.stdout.split() == ["100", "273"]


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"linattn_prefill", "linattn_decode_step", "linattn_feature_map"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH],
                        capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (linattn_\w+)", nm))
    assert set(names) <= exported


def test_feature_dim_and_supported(lib):
    assert lib.linattn_feature_dim(0, 64) == 64
    assert lib.linattn_feature_dim(1, 16) == 273
    assert lib.linattn_feature_dim(1, 3) == 13
    assert lib.linattn_feature_dim(2, 16) == 153
    assert lib.linattn_feature_dim(2, 3) == 10
    assert lib.linattn_feature_dim(7, 16) == -1
    assert lib.linattn_feature_dim(0, 0) == -1
    for dt in (0, 1):
        for d in (16, 32, 64):
            assert lib.linattn_supported(0, dt, d, d) == 1
            assert lib.linattn_supported(1, dt, 16, d) == 1
            assert lib.linattn_supported(2, dt, 16, d) == 1
        assert lib.linattn_supported(0, dt, 64, 32) == 0
        assert lib.linattn_supported(0, dt, 128, 128) == 0
        assert lib.linattn_supported(1, dt, 32, 64) == 0
        assert lib.linattn_supported(2, dt, 32, 32) == 0
    assert lib.linattn_supported(0, 2, 64, 64) == 0
    for s in range(6):
        assert lib.linattn_status_string(s)


def test_workspace_bytes(lib):
    f = lib.linattn_prefill_workspace_bytes
    bad = ctypes.c_size_t(-1).value
    # one segment per head -> no workspace
    assert f(0, 1, 1, 2, 256, 16, 16, 0) == 0
    assert f(0, 1, 64, 64, 4096, 64, 64, 0) == 0
    # explicit segments: B*H*nseg slots of NRT*NCT*256 floats, then one
    # float per slot (a gated segment's log2 decay) padded to 16 bytes
    def logs(n):
        return (4 * n + 15) // 16 * 16
    slot_elu64 = 4 * 5 * 256
    assert f(0, 1, 8, 8, 4096, 64, 64, 1024) == 64 * 4 * slot_elu64 * 4 + logs(64 * 4)
    assert f(0, 1, 8, 8, 4096, 64, 64, 4096) == 0
    # With few heads the Taylor segment-sum pass splits each segment in two
    # (B*H*(nseg-1) below 512 workgroups and halves of >= 4 chunks),
    # doubling the slots; ELU1 never splits.
    slot_tay = 10 * 5 * 256
    # 512 heads x 3 summed segments fill the GPU already: no split
    assert f(1, 1, 64, 8, 2048, 16, 64, 512) == 512 * 4 * slot_tay * 4 + logs(512 * 4)
    # 6-chunk segments would leave 3-chunk halves: no split
    assert f(1, 1, 1, 2, 4096, 16, 16, 384) == 2 * 11 * (10 * 2 * 256) * 4 + logs(2 * 11)
    assert f(1, 1, 8, 16, 2048, 16, 64, 512) == 128 * 8 * slot_tay * 4 + logs(128 * 8)
    # the unordered-pair map runs on the same kernels and workspace
    assert f(2, 1, 8, 16, 2048, 16, 64, 512) == 128 * 8 * slot_tay * 4 + logs(128 * 8)
    # ragged: 65 tokens in 64-token segments -> 2 segments
    assert f(0, 0, 1, 1, 65, 16, 16, 64) == 2 * (2 * 2 * 256) * 4 + 16
    assert f(0, 1, 1, 1, 4096, 64, 64, 100) == bad     # not a multiple of 64
    assert f(0, 1, 1, 1, 0, 64, 64, 0) == bad
    assert f(0, 1, 1, 1, 64, 64, 32, 0) == bad         # unsupported
    assert f(3, 1, 1, 1, 64, 64, 64, 0) == bad


# Fake, well separated, 16-byte aligned device addresses: validation only
# compares and aligns them; it never dereferences anything.
A = {n: ctypes.c_void_p(0x10000000 * (i + 1)) for i, n in
     enumerate(["q", "k", "v", "y", "Si", "zi", "So", "zo", "ws"])}


def _prefill(lib, **kw):
    a = dict(map=0, dtype=1, B=1, H=1, N=128, dk=64, dv=64, q=A["q"], k=A["k"],
             v=A["v"], y=A["y"], Si=None, zi=None, So=None, zo=None, seg=0,
             ws=None, wsb=0)
    a.update(kw)
    return lib.linattn_prefill(a["map"], a["dtype"], a["B"], a["H"], a["N"],
                               a["dk"], a["dv"], a["q"], a["k"], a["v"], a["y"],
                               a["Si"], a["zi"], a["So"], a["zo"], a["seg"],
                               a["ws"], a["wsb"], None)


def test_prefill_validation_codes(lib):
    INV, UNS, WS = 1, 2, 3
    assert _prefill(lib, q=None) == INV
    assert _prefill(lib, y=None) == INV
    assert _prefill(lib, N=0) == INV
    assert _prefill(lib, B=-1) == INV
    assert _prefill(lib, map=5) == INV
    assert _prefill(lib, dtype=9) == INV
    assert _prefill(lib, dk=48, dv=48) == UNS
    assert _prefill(lib, q=ctypes.c_void_p(0x10000008)) == INV   # misaligned
    assert _prefill(lib, Si=A["Si"]) == INV                        # z_in missing
    assert _prefill(lib, So=A["So"]) == INV                        # z_out missing
    assert _prefill(lib, y=A["q"]) == INV                          # y aliases q
    assert _prefill(lib, seg=65) == INV
    # 2 segments need a workspace
    assert _prefill(lib, seg=64) == WS
    assert _prefill(lib, seg=64, ws=A["ws"], wsb=10) == WS
    assert _prefill(lib, seg=64, ws=ctypes.c_void_p(0x90000004), wsb=1 << 20) == WS
    # the workspace must not overlap an input
    assert _prefill(lib, seg=64, ws=A["q"], wsb=1 << 20) == INV
    # S_out may equal S_in, but must not partially overlap it
    assert _prefill(lib, Si=A["Si"], zi=A["zi"], So=ctypes.c_void_p(0x50000010),
                    zo=A["zo"]) == INV


def _prefill_gated(lib, gate=A["zi"], normalize=1, **kw):
    a = dict(map=0, dtype=1, B=1, H=1, N=128, dk=64, dv=64, q=A["q"], k=A["k"],
             v=A["v"], y=A["y"], Si=None, zi=None, So=None, zo=None, seg=0,
             ws=None, wsb=0)
    a.update(kw)
    return lib.linattn_prefill_gated(a["map"], a["dtype"], a["B"], a["H"], a["N"],
                                     a["dk"], a["dv"], a["q"], a["k"], a["v"], gate,
                                     normalize, a["y"], a["Si"], a["zi"], a["So"],
                                     a["zo"], a["seg"], a["ws"], a["wsb"], None)


def test_gated_validation_codes(lib):
    INV, UNS, WS = 1, 2, 3
    assert _prefill_gated(lib, gate=None) == INV
    assert _prefill_gated(lib, normalize=2) == INV
    assert _prefill_gated(lib, gate=ctypes.c_void_p(0x60000002)) == INV   # misaligned
    assert _prefill_gated(lib, gate=A["y"]) == INV                        # gate aliases y
    assert _prefill_gated(lib, dk=48, dv=48) == UNS
    assert _prefill_gated(lib, seg=64) == WS
    # the workspace must not overlap the gate
    assert _prefill_gated(lib, seg=64, ws=A["zi"], wsb=1 << 20) == INV
    d = lib.linattn_decode_step_gated
    args = (1, 1, 4, 16, 16, 64, A["q"], A["k"], A["v"])
    assert d(*args, None, 1, A["Si"], A["zi"], A["y"], None) == INV
    assert d(*args, A["So"], 3, A["Si"], A["zi"], A["y"], None) == INV
    assert d(*args, A["y"], 1, A["Si"], A["zi"], A["y"], None) == INV   # gate aliases y
    assert d(1, 1, 4, 16, 32, 64, A["q"], A["k"], A["v"], A["So"], 1, A["Si"], A["zi"],
             A["y"], None) == UNS


def test_decode_and_feature_map_validation(lib):
    INV, UNS = 1, 2
    f = lib.linattn_decode_step
    assert f(1, 1, 4, 16, 16, 64, A["q"], A["k"], A["v"], None, A["zi"], A["y"], None) == INV
    assert f(1, 1, 4, 16, 16, 64, A["q"], A["k"], A["v"], A["Si"], A["zi"], A["Si"], None) == INV
    assert f(1, 1, 0, 16, 16, 64, A["q"], A["k"], A["v"], A["Si"], A["zi"], A["y"], None) == INV
    assert f(1, 1, 4, 16, 32, 64, A["q"], A["k"], A["v"], A["Si"], A["zi"], A["y"], None) == UNS
    g = lib.linattn_feature_map
    assert g(0, 1, A["q"], 10, 64, None, None) == INV
    assert g(1, 1, A["q"], 10, 64, A["y"], None) == UNS
    assert g(0, 1, A["q"], -1, 64, A["y"], None) == INV
    assert g(0, 1, A["q"], 0, 64, A["y"], None) == 0   # empty: nothing to do


def test_swa_validation_codes(lib):
    """Sliding-window entry points: every invalid argument is refused on the
    host before any launch (fake device addresses are never dereferenced)."""
    INV, UNS = 1, 2
    f = lib.linattn_swa_prefill

    def pre(**kw):
        a = dict(dtype=1, B=1, H=2, N=128, d=64, w=64, scale=0.125, q=A["q"], k=A["k"],
                 v=A["v"], y=A["y"], kc=None, vc=None)
        a.update(kw)
        return f(a["dtype"], a["B"], a["H"], a["N"], a["d"], a["w"], a["scale"], a["q"],
                 a["k"], a["v"], a["y"], a["kc"], a["vc"], None)

    assert pre(q=None) == INV
    assert pre(N=0) == INV
    assert pre(w=0) == INV
    assert pre(scale=float("inf")) == INV
    # NaN selects 1/sqrt(d): it passes the scale check, so the unsupported
    # width is what the call reports (no launch either way)
    assert pre(scale=float("nan"), d=48) == UNS
    assert pre(scale=float("-inf"), d=48) == INV
    assert pre(d=48) == UNS
    assert pre(dtype=7) == INV
    assert pre(kc=A["Si"]) == INV                     # v_cache missing
    assert pre(y=A["k"]) == INV                       # output aliases an input
    assert pre(kc=A["Si"], vc=A["Si"]) == INV         # the two caches overlap
    assert pre(q=ctypes.c_void_p(0x10000004)) == INV  # misaligned
    g = lib.linattn_swa_decode_step

    def dec(**kw):
        a = dict(dtype=1, B=2, H=2, d=64, w=64, scale=0.125, q=A["q"], k=A["k"], v=A["v"],
                 pos=A["zi"], kc=A["Si"], vc=A["So"], y=A["y"])
        a.update(kw)
        return g(a["dtype"], a["B"], a["H"], a["d"], a["w"], a["scale"], a["q"], a["k"],
                 a["v"], a["pos"], a["kc"], a["vc"], a["y"], None)

    assert dec(pos=None) == INV
    assert dec(kc=None) == INV
    assert dec(w=4097) == UNS                         # beyond the generation window
    assert dec(d=16) == UNS
    assert dec(d=16, scale=float("nan")) == UNS
    assert dec(d=16, scale=float("inf")) == INV
    assert dec(pos=ctypes.c_void_p(0x60000004)) == INV  # pos not 8-byte aligned
    assert dec(y=A["Si"]) == INV                      # y aliases the key cache
    assert dec(kc=A["q"]) == INV                      # cache aliases an input


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus 2 exits with status 2 and says why
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_digest_follows_code_not_comments():
    """The digest that keys recorded traffic changes with the code of a
    kernel family and not with its comments or layout."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = 'int f(int x) { // doubles\n  return 2 * x; /* was 3 */ }\nconst char* s = "a // b";'
    b = 'int f(int x) {\n\n    return 2 * x;\n}\n// note\nconst char* s = "a // b";'
    c = 'int f(int x) { return 3 * x; }\nconst char* s = "a // b";'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert '"a // b"' in bench.code_text(a)
    for kind in bench.DIGEST_FILES:
        assert len(bench.csrc_digest(kind)) == 16


def test_binding_rejects_mis_sized_buffers_before_the_library(lib):
    """The Python binding checks the shape, dtype and device of every tensor,
    out= included, before it calls the library (which sizes every device
    access from the shape arguments).  Host tensors of valid shapes are
    refused as host tensors; mis-shaped ones are refused for their shape or
    dtype first, so these checks run here without a GPU."""
    import torch

    q = torch.zeros(1, 2, 8, 16)
    k, v = q.clone(), q.clone()
    with pytest.raises(ValueError, match="out must have shape"):
        ops.prefill(q, k, v, "elu1", out=torch.zeros(1, 2, 8, 8))
    with pytest.raises(TypeError, match="out must be"):
        ops.prefill(q, k, v, "elu1", out=torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="expected q, k"):
        ops.prefill(q, torch.zeros(1, 2, 8, 32), v, "elu1")
    with pytest.raises(TypeError, match="share one dtype"):
        ops.prefill(q, k.bfloat16(), v, "elu1")
    with pytest.raises(TypeError, match="not supported"):
        ops.prefill(q.double(), k.double(), v.double(), "elu1")
    with pytest.raises(ValueError, match="state S must have shape"):
        ops.prefill(q, k, v, "elu1", state=(torch.zeros(1, 2, 16, 8), torch.zeros(1, 2, 16)))
    with pytest.raises(ValueError, match="gate must have shape"):
        ops.prefill_gated(q, k, v, torch.zeros(1, 2, 7), "elu1")
    with pytest.raises(ValueError, match="GPU device"):
        ops.prefill(q, k, v, "elu1")

    q3 = torch.zeros(1, 2, 16)
    S, z = torch.zeros(1, 2, 16, 16), torch.zeros(1, 2, 16)
    with pytest.raises(ValueError, match="out must have shape"):
        ops.decode_step(q3, q3, q3, S, z, "elu1", out=torch.zeros(1, 2, 8))
    with pytest.raises(TypeError, match="out must be"):
        ops.decode_step(q3, q3, q3, S, z, "elu1", out=torch.zeros(1, 2, 16).bfloat16())
    with pytest.raises(ValueError, match="S must have shape"):
        ops.decode_step(q3, q3, q3, torch.zeros(1, 2, 16, 8), z, "elu1")
    with pytest.raises(TypeError, match="z must be"):
        ops.decode_step(q3, q3, q3, S, z.double(), "elu1")
    with pytest.raises(ValueError, match="gate must have shape"):
        ops.decode_step_gated(q3, q3, q3, torch.zeros(2), S, z, "elu1")

    kc = torch.zeros(1, 2, 4, 16)
    pos = torch.zeros(1, dtype=torch.int64)
    with pytest.raises(ValueError, match="k_cache must have shape"):
        ops.swa_decode_step(q3, q3, q3, pos, torch.zeros(1, 2, 5, 16), kc, 4)
    with pytest.raises(TypeError, match="v_cache must be"):
        ops.swa_decode_step(q3, q3, q3, pos, kc, kc.bfloat16(), 4)
    with pytest.raises(ValueError, match="expected q, k"):
        ops.swa_decode_step(q3, torch.zeros(1, 2, 32), q3, pos, kc, kc.clone(), 4)
    with pytest.raises(ValueError, match="one shape"):
        ops.swa_decode_step(q3, q3, torch.zeros(1, 2, 32), pos, kc, kc.clone(), 4)
    with pytest.raises(TypeError, match="pos must be"):
        ops.swa_decode_step(q3, q3, q3, pos.int(), kc, kc.clone(), 4)
    with pytest.raises(ValueError, match="out must have shape"):
        ops.swa_decode_step(q3, q3, q3, pos, kc, kc.clone(), 4, out=torch.zeros(1, 2, 8))
    with pytest.raises(ValueError, match="out must have shape"):
        ops.swa_prefill(q, k, v, 4, out=torch.zeros(1, 2, 8, 8))
    with pytest.raises(ValueError, match="GPU device"):
        ops.swa_decode_step(q3, q3, q3, pos, kc, kc.clone(), 4)


def test_noalloc_rejects_calls_beyond_its_fixed_scratch(lib):
    """linattn_prefill_noalloc refuses, before any HIP call, a plan whose part
    sums exceed its fixed array: Taylor d_v = 64 at 128 heads in 128 segments
    of one chunk needs 128 * 128 * 51200 bytes."""
    need = lib.linattn_prefill_workspace_bytes(1, 1, 8, 16, 8192, 16, 64, 64)
    assert need > 64 << 20
    rc = lib.linattn_prefill_noalloc(
        1, 1, 8, 16, 8192, 16, 64, A["q"], A["k"], A["v"], A["y"], None, None, None, None,
        64, None)
    assert rc == 5
    assert b"fixed" in lib.linattn_status_string(5)
    # argument errors still come first
    assert lib.linattn_prefill_noalloc(1, 1, 8, 16, 8192, 16, 64, None, A["k"], A["v"],
                                       A["y"], None, None, None, None, 64, None) == 1


def test_probe_library_exports_what_bench_calls():
    """liblinattn_probe.so exports every probe entry point bench.py calls,
    and its argument checks reject bad calls on the host, before any launch."""
    from causal_linear_attention_linattn_amd import _build
    if not os.path.exists(_build.PROBE_LIB):
        _build.build()
    P = ctypes.CDLL(_build.PROBE_LIB)
    used = set(re.findall(r"\bP\.(linattn_probe_[a-z_0-9]+)",
                          open(os.path.join(ROOT, "bench.py")).read()))
    assert {"linattn_probe_stream", "linattn_probe_peak_mfma",
            "linattn_probe_intra_mfma"} <= used
    for name in used:
        assert hasattr(P, name), name
    P.linattn_probe_intra_mfma_per_iter.argtypes = [ctypes.c_int]
    assert P.linattn_probe_intra_mfma_per_iter(0) > 0
    assert P.linattn_probe_intra_mfma_per_iter(1) > 0
    assert P.linattn_probe_intra_mfma_per_iter(2) == -1
    st = P.linattn_probe_stream
    st.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below is rejected
    assert st(0, 4, None, fake, 1 << 20, 16, None) == 1        # no source
    assert st(0, 4, fake, fake, (1 << 20) + 8, 16, None) == 1  # not whole 16-byte vectors
    assert st(0, 4, fake, fake, 1 << 20, 0, None) == 1         # no workgroups
    assert st(0, 4, fake, fake, 1 << 12, 2, None) == 1         # under 4 KB per workgroup
    assert st(0, 5, fake, fake, 1 << 20, 16, None) == 1        # unsupported depth
    assert st(3, 4, fake, fake, 1 << 20, 16, None) == 1        # unknown mode
    pk = P.linattn_probe_peak_mfma
    pk.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert pk(0, 256, fake, None) == 1
    assert pk(10, 256, None, None) == 1
