"""Helpers shared by the GPU tests: move seeded inputs to the device and run the
HIP path through the C ABI binding."""

import numpy as np

import linear_attention_diffusion_amd as la


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def device():
    return torch_mod().device("cuda:0")


def to_dev(raw, dtype):
    torch = torch_mod()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(device())


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def inputs_on_device(x):
    w = x.workload
    return tuple(to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v"))


def rope_for(w, dev=None):
    return la.rope3d_device(*w.grid, dev or device())


def run_forward(x, rope=None, workspace=None):
    q, k, v = inputs_on_device(x)
    o = la.sana_linattn_forward(q, k, v, eps=x.workload.eps, rope=rope, workspace=workspace)
    return to_np(o)


def split_chunks(t, chunk):
    """Contiguous per-chunk tensors [B, H, L_c, D] of a [B, H, N, D] tensor."""
    N = t.shape[2]
    return [t[:, :, s:min(N, s + chunk)].contiguous() for s in range(0, N, chunk)]


def run_block_chunks(x, chunk, rope=None, commit=True):
    """Run the block-causal chunk loop with an in-place committed state.
    Returns (O over all chunks, final kv, final ksum) as float64 numpy."""
    torch = torch_mod()
    w = x.workload
    q, k, v = inputs_on_device(x)
    qs, ks, vs = split_chunks(q, chunk), split_chunks(k, chunk), split_chunks(v, chunk)
    kv = torch.zeros(w.B, w.H, 32, 32, device=device())
    z = torch.zeros(w.B, w.H, 32, device=device())
    outs = []
    start = 0
    for qc, kc, vc in zip(qs, ks, vs):
        r = None if rope is None else rope.at(start)
        outs.append(la.sana_linattn_block_forward(qc, kc, vc, kv_in=kv, ksum_in=z,
                                                  kv_out=kv if commit else None,
                                                  ksum_out=z if commit else None, eps=w.eps, rope=r))
        start += qc.shape[2]
    return to_np(torch.cat(outs, dim=2)), to_np(kv), to_np(z)
