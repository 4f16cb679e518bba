"""GPU tests of the temporal convolution with its cache (against the oracle)
and of the block inference loop (against a float64 replica that rounds to
bf16 where the device path stores bf16)."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from block_infer_ref import RefCache, RefLayer, bf
from block_infer_ref import block_linear_diffusion as ref_loop
from gpu_util import device, to_dev, to_np, torch_mod
from linear_attention_diffusion_amd import block_infer
from metrics import check, rel_l2
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu


def _bf16_dev(x):
    return to_dev(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)), "bf16")


@pytest.mark.parametrize("dtype,B,F,S,C,with_cache", [
    ("bf16", 1, 3, 1560, 64, True), ("bf16", 2, 1, 37, 8, True), ("bf16", 1, 5, 100, 5600 // 10, False),
    ("f32", 2, 3, 41, 24, True), ("f32", 1, 2, 7, 8, False)])
def test_temporal_conv_against_oracle(dtype, B, F, S, C, with_cache):
    torch = torch_mod()
    print(f"case conv {dtype} B={B} F={F} S={S} C={C} cache={with_cache}", flush=True)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, F, S, C)).astype(np.float32) * 0.5
    prev = rng.standard_normal((B, S, C)).astype(np.float32) * 0.5
    w = (rng.standard_normal((C, 3)) * 0.3).astype(np.float32)
    b = (rng.standard_normal(C) * 0.1).astype(np.float32)
    if dtype == "bf16":
        x, prev = bf(x), bf(prev)
        xd, pd = _bf16_dev(x), _bf16_dev(prev)
    else:
        xd, pd = (torch.from_numpy(a).to(device()) for a in (x, prev))
    wd, bd = torch.from_numpy(w).to(device()), torch.from_numpy(b).to(device())
    cache = pd.clone()
    y = la.sana_linattn_temporal_conv3(xd, wd, bd, cache_in=cache if with_cache else None, cache_out=cache)
    want, last = oracle.temporal_conv3(x, w, b, prev if with_cache else None)
    check(to_np(y), want, dtype, "temporal conv")
    assert np.array_equal(to_np(cache), last)          # in-place commit of the last frame


def _setup(B=1, C=64, H=2, frames=2, grid_hw=(3, 4), M=3, T=3, layers=2, seed=3):
    torch = torch_mod()
    spatial = grid_hw[0] * grid_hw[1]
    N = frames * spatial
    dev_layers = [block_infer.SyntheticLayer(C, H, device(), seed + i) for i in range(layers)]
    ref_layers = [RefLayer(to_np(l.wqkv), to_np(l.wo), to_np(l.conv_w), to_np(l.conv_b), H) for l in dev_layers]
    rng = np.random.default_rng(seed)
    noise = bf(rng.standard_normal((M, B, N, C)).astype(np.float32))
    step_noise = bf(rng.standard_normal((M, T - 1, B, N, C)).astype(np.float32))
    timesteps = [(j + 1) / T for j in range(T)]
    return dict(B=B, C=C, H=H, frames=frames, spatial=spatial, N=N, M=M, T=T, dev_layers=dev_layers,
                ref_layers=ref_layers, noise=noise, step_noise=step_noise, timesteps=timesteps,
                grid=(M * frames, grid_hw[0], grid_hw[1]))


@pytest.mark.parametrize("rope", [False, True])
def test_block_inference_loop(rope):
    torch = torch_mod()
    s = _setup()
    print(f"case block inference rope={rope}", flush=True)
    caches = [block_infer.BlockCache(s["B"], s["H"], s["spatial"], s["C"], torch.bfloat16, device())
              for _ in s["dev_layers"]]
    r = la.rope3d_device(*s["grid"], device()) if rope else None
    out = block_infer.block_linear_diffusion(s["dev_layers"], caches, _bf16_dev(s["noise"]),
                                             _bf16_dev(s["step_noise"]), s["timesteps"], s["frames"], rope=r)
    ref_caches = [RefCache(s["B"], s["H"], s["spatial"], s["C"]) for _ in s["ref_layers"]]
    ang = oracle.rope3d_angles(*s["grid"]) if rope else None
    want = ref_loop(s["ref_layers"], ref_caches, s["noise"], s["step_noise"], s["timesteps"], s["frames"], 1e-6, ang)
    err = rel_l2(to_np(out), want)
    print(f"block inference rope={rope}: output rel-L2 {err:.3e}", flush=True)
    assert err <= 1e-2
    for c, rc in zip(caches, ref_caches):
        assert rel_l2(to_np(c.kv), rc.S) <= 1e-2 and rel_l2(to_np(c.ksum), rc.z) <= 1e-2
        assert rel_l2(to_np(c.conv), rc.conv) <= 1e-2


def test_denoising_steps_leave_the_cache_untouched():
    """Read-only calls (every denoising step) leave all three cache parts
    bit-identical; the commit pass changes them; the committed attention state
    equals state_update over the clean pass's keys and values."""
    torch = torch_mod()
    s = _setup(M=1, T=2)
    caches = [block_infer.BlockCache(s["B"], s["H"], s["spatial"], s["C"], torch.bfloat16, device())
              for _ in s["dev_layers"]]
    x = _bf16_dev(s["noise"][0])
    block_infer.run_model(s["dev_layers"], caches, x, s["frames"], commit=True)   # commit a first chunk
    snap = [(c.kv.clone(), c.ksum.clone(), c.conv.clone()) for c in caches]
    block_infer.run_model(s["dev_layers"], caches, x, s["frames"], commit=False)
    for c, (kv, z, conv) in zip(caches, snap):
        assert torch.equal(c.kv, kv) and torch.equal(c.ksum, z) and torch.equal(c.conv, conv)
    # the commit adds exactly the layer's clean-pass keys and values
    layer, cache = s["dev_layers"][0], caches[0]
    B, N, C, H = s["B"], s["N"], s["C"], s["H"]
    qkv = (x.reshape(B * N, C) @ layer.wqkv).view(B, N, 3, H, 32)
    k, v = (qkv[:, :, i].permute(0, 2, 1, 3).contiguous() for i in (1, 2))
    kv_want, z_want = snap[0][0].clone(), snap[0][1].clone()
    la.sana_linattn_state_update(k, v, kv_want, z_want)
    block_infer.run_model(s["dev_layers"][:1], caches[:1], x, s["frames"], commit=True)
    assert rel_l2(to_np(cache.kv), to_np(kv_want)) <= 1e-6
    assert rel_l2(to_np(cache.ksum), to_np(z_want)) <= 1e-6
