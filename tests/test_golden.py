"""Golden fixtures: the shape facts the pages print, and the oracle regression file."""

import json
import os

import numpy as np

import oracle
from workloads import WORKLOADS, generate, reduced

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_workload_shapes_follow_the_pages():
    g = _load("shapes_from_pages.json")
    assert 1152 // g["heads_sana_0_6b"]["value"] == g["head_dim"]["value"] == 2240 // g["heads_sana_1_6b"]["value"]
    for w in WORKLOADS.values():
        assert w.D == g["head_dim"]["value"]
    f = g["ae_spatial_downsample"]["value"]
    assert WORKLOADS["sana06b_1024px"].N == (1024 // f) ** 2 == g["latent_tokens_1024px"]["value"]
    assert WORKLOADS["sana06b_1024px"].H == g["heads_sana_0_6b"]["value"]
    assert WORKLOADS["sana16b_4096px"].N == (4096 // f) ** 2 == g["latent_tokens_4096px"]["value"]
    assert WORKLOADS["sana16b_4096px"].H == g["heads_sana_1_6b"]["value"]
    T, Hl, Wl = g["video_720p_latent_grid"]["value"]
    assert WORKLOADS["video720p_rope3d"].grid == (T, Hl, Wl)
    assert WORKLOADS["video720p_rope3d"].N == T * Hl * Wl
    fh, fw = g["video_480p_frame_grid"]["value"]
    wb = WORKLOADS["video480p_blockcausal"]
    assert wb.chunk == 3 * fh * fw and wb.n_chunks == 10


def _check(o, case, rtol=1e-12):
    assert list(o.shape) == case["shape"]
    got = {"sum": o.sum(), "sum_abs": np.abs(o).sum(), "sum_sq": (o * o).sum()}
    for key, value in got.items():
        assert abs(float(value) - case[key]) <= rtol * max(1.0, abs(case[key])), key


def test_oracle_regression_fixture():
    g = _load("oracle_small.json")["cases"]
    w = WORKLOADS["noncausal_f32_b1h1n256"]
    x = generate(w).f64
    o = oracle.linattn(x["q"], x["k"], x["v"], w.eps)
    _check(o, g[w.name])
    for r, row in g[w.name]["rows"].items():
        np.testing.assert_allclose(o[0, 0, int(r)], row, rtol=1e-12, atol=0)

    wr = reduced(WORKLOADS["video720p_rope3d"], H=2, N=30, grid=(2, 3, 5))
    x = generate(wr).f64
    o = oracle.linattn(x["q"], x["k"], x["v"], wr.eps, angles=oracle.rope3d_angles(*wr.grid))
    _check(o, g["rope3d_2x3x5_h2"])

    wb = reduced(WORKLOADS["video480p_blockcausal"], H=2, N=60, chunk=20)
    x = generate(wb).f64
    o, S, z = oracle.block_causal(x["q"], x["k"], x["v"], wb.chunk, wb.eps)
    _check(o, g["blockcausal_3x20_h2"])
    np.testing.assert_allclose(z[0, 0], g["blockcausal_3x20_h2"]["z"], rtol=1e-12)


def test_generator_is_deterministic_and_bf16_exact():
    w = reduced(WORKLOADS["sana16b_4096px"], H=2, N=64)
    a, b = generate(w), generate(w)
    assert a.sha256() == b.sha256()
    # bf16 values carry at most 8 significant bits: the float64 upcast survives a
    # round trip through float32 and the low 16 bits of the float32 are zero
    f32 = a.f64["q"].astype(np.float32)
    assert np.all(f32.view(np.uint32) & 0xFFFF == 0)
    # RNE: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 and rounds to the even 1.0
    from workloads import bf16_bits_from_f32
    assert bf16_bits_from_f32(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert bf16_bits_from_f32(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    assert bf16_bits_from_f32(np.array([-0.0], np.float32))[0] == 0x8000
