"""The seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

from causal_linear_attention_linattn_amd import synth


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 1e-40, 3.0e38,
                                  1.00390625, 1.01171875], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    got = synth.bf16_bits_rne(x).view(np.int16)
    assert np.array_equal(got, want)
    back = synth.bf16_bits_to_f32(synth.bf16_bits_rne(x))
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_determinism_and_streams():
    a = synth.draw_qkv(2, 3, 17, 4, 5, seed=7)
    b = synth.draw_qkv(2, 3, 17, 4, 5, seed=7)
    c = synth.draw_qkv(2, 3, 17, 4, 5, seed=8)
    d = synth.draw_qkv(2, 3, 17, 4, 5, seed=7, stream=1)
    for x, y in zip(a, b):
        assert np.array_equal(x.data, y.data)
    assert not np.array_equal(a[0].data, c[0].data)
    assert not np.array_equal(a[0].data, d[0].data)
    assert a[0].shape == (2, 3, 17, 4) and a[2].shape == (2, 3, 17, 5)
    assert a[0].data.dtype == np.uint16


def test_draw_order_and_scale():
    rng = np.random.Generator(np.random.PCG64([3, 0]))
    q = rng.standard_normal((1, 2, 9, 4))
    k = rng.standard_normal((1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 6))
    s = 16.0 ** -0.25
    got = synth.draw_qkv(1, 2, 9, 4, 6, seed=3, dtype="f32", qk_scale=s)
    assert np.array_equal(got[0].data, (q * s).astype(np.float32))
    assert np.array_equal(got[1].data, (k * s).astype(np.float32))
    assert np.array_equal(got[2].data, v.astype(np.float32))
    assert got[0].f64().dtype == np.float64


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_small_override(name):
    cfg = synth.WORKLOADS[name]
    out = synth.workload_inputs(name, seed=0, B=1, H=1, N=8,
                                **({"steps": 3} if "steps" in cfg else {}))
    assert len(out) == (6 if "steps" in cfg else 3)
    assert out[0].shape == (1, 1, 8, cfg["d_k"])
    assert out[2].shape == (1, 1, 8, cfg["d_v"])
    if "steps" in cfg:
        assert out[3].shape == (1, 1, 3, cfg["d_k"])
    assert out[0].dtype == cfg["dtype"]


def test_only_taylor_prefill_is_scaled():
    scaled = {n for n, c in synth.WORKLOADS.items() if c["qk_scale"] != 1.0}
    assert scaled == {"based_taylor2_bf16"}
