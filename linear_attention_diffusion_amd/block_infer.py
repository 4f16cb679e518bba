"""Block linear diffusion inference with the constant-memory cache.

"SANA-Video" paper notes, section 4 (block linear diffusion inference): the
video is generated chunk by chunk.  Every chunk starts from noise and is
denoised over T steps; each step runs the model with the cache read only, and
once the chunk is clean the model runs once more on the clean result at t = 0
to commit the chunk into the cache.  The cache has three parts per layer: the
running sum of S = phi(K)^T V, the running sum of phi(K), and the last frame of
the temporal convolution (the conv cache).  Later chunks therefore see every
earlier chunk through O(D^2) state and one frame, never through earlier tokens.

The layers here are synthetic (seeded random weights): no trained model is
available, and the point is the control flow and the cache.  Each layer is
    QKV projection + block-causal linear attention through the cache
    ->  output projection + residual  ->  temporal conv through the conv cache
and ignores the timestep.  The attention runs in the fused projection kernels
("Sana" research note, Infra: ReLU(K)^T V fused with the QKV projection):
sana_linattn_project_state adds the chunk's phi~(K)^T V and phi(K) to a copy of
the carried state (to the cache itself on the commit pass) without writing K or
V, and sana_linattn_project_apply computes O from the queries' projection
against that state without writing Q -- the same as block_forward on the
projected Q, K, V.  With fused=False the layer instead projects with one torch
GEMM and runs block_forward on strided views of its packed output.  Readings where the pages leave a step open: the
noise schedule is the flow-matching interpolation x_t = (1 - t) x0 + t eps
(SANA's flow objective), and the model output is taken as the prediction of
the clean chunk.  Every attention and convolution step runs in this library's
HIP kernels; the projections and the elementwise schedule are torch device ops.
"""

import math

from . import binding as _b


class BlockCache:
    """One layer's cache: S [B, H, 32, 32] and z [B, H, 32] (fp32), the conv
    cache [B, S, C] (the last frame of the temporal conv's input), and whether
    anything has been committed yet."""

    def __init__(self, B, H, spatial, C, dtype, device):
        torch = _b._torch()
        self.kv = torch.zeros(B, H, 32, 32, device=device)
        self.ksum = torch.zeros(B, H, 32, device=device)
        self.conv = torch.zeros(B, spatial, C, dtype=dtype, device=device)
        self.committed = False
        # a denoising pass's state: the carried state plus the chunk, not committed
        self.step_kv = torch.empty_like(self.kv)
        self.step_ksum = torch.empty_like(self.ksum)


class SyntheticLayer:
    """A DiT-style layer with seeded random weights (see the module note).

    The QKV weight is a linear layer's [3 H 32, C] matrix: rows h*32 + d of
    w_q, w_k, w_v (its three row blocks) give feature d of head h."""

    def __init__(self, C, H, device, seed, dtype=None, fused=True):
        torch = _b._torch()
        dtype = dtype or torch.bfloat16
        g = torch.Generator().manual_seed(seed)
        self.C, self.H, self.fused = C, H, fused
        w = (torch.randn(3 * H * 32, C, generator=g) / math.sqrt(C)).to(dtype).to(device)
        self.wq, self.wk, self.wv = (w[i * H * 32:(i + 1) * H * 32] for i in range(3))
        self.wqkv_t = w.t().contiguous()          # [C, 3 H 32] for the unfused projection
        self.wo = (torch.randn(H * 32, C, generator=g) / math.sqrt(H * 32)).to(dtype).to(device)
        self.conv_w = (torch.randn(C, 3, generator=g) * 0.25).to(device)
        self.conv_b = (torch.randn(C, generator=g) * 0.05).to(device)
        # when a list: every attention call appends (x, carried kv, carried ksum,
        # the state the fused apply read (kv, ksum) or None, o, commit, pos0),
        # copies taken around the call (for inspection)
        self.record = None

    def attend(self, x, cache, commit, eps, rope, pos0, o):
        """O of the chunk's tokens into o [B, N, H, 32]: the carried state plus the
        chunk's own keys and values, committed to the cache when `commit`.
        Returns the state the fused apply read (None on the unfused path)."""
        r = None if rope is None else rope.at(pos0)
        if self.fused:
            if commit:
                kv, ks = cache.kv, cache.ksum
            else:
                kv, ks = cache.step_kv, cache.step_ksum
                kv.copy_(cache.kv)
                ks.copy_(cache.ksum)
            _b.sana_linattn_project_state(x, self.wk, self.wv, kv, ks, rope=r)
            _b.sana_linattn_project_apply(x, self.wq, kv, ks, o=o.permute(0, 2, 1, 3), eps=eps, rope=r)
            return kv, ks
        B, N, C = x.shape
        qkv = (x.reshape(B * N, C) @ self.wqkv_t).view(B, N, 3, self.H, 32)
        q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
        _b.sana_linattn_block_forward(q, k, v, o=o.permute(0, 2, 1, 3), kv_in=cache.kv, ksum_in=cache.ksum,
                                      kv_out=cache.kv if commit else None, ksum_out=cache.ksum if commit else None,
                                      eps=eps, rope=r)
        return None

    def __call__(self, x, cache, frames, commit, eps=1e-6, rope=None, pos0=0):
        """x: [B, frames * spatial, C] -> same shape.  commit: update the cache."""
        torch = _b._torch()
        B, N, C = x.shape
        H = self.H
        spatial = N // frames
        o = torch.empty(B, N, H, 32, dtype=x.dtype, device=x.device)
        carried = None if self.record is None else (cache.kv.clone(), cache.ksum.clone())
        used = self.attend(x, cache, commit, eps, rope, pos0, o)
        if self.record is not None:
            used = None if used is None else (used[0].clone(), used[1].clone())
            self.record.append((x.clone(), carried[0], carried[1], used, o.clone(), commit, pos0))
        h = x + (o.view(B * N, H * 32) @ self.wo).view(B, N, C)
        y = _b.sana_linattn_temporal_conv3(h.view(B, frames, spatial, C), self.conv_w, self.conv_b,
                                           cache_in=cache.conv if cache.committed else None,
                                           cache_out=cache.conv if commit else None)
        if commit:
            cache.committed = True
        return y.view(B, N, C)


def run_model(layers, caches, x, frames, commit, eps=1e-6, rope=None, pos0=0):
    for layer, cache in zip(layers, caches):
        x = layer(x, cache, frames, commit, eps, rope, pos0)
    return x


def block_linear_diffusion(layers, caches, noise, step_noise, timesteps, frames, eps=1e-6, rope=None):
    """The block inference loop.

    noise: [M, B, F*S, C], each chunk's starting noise at t_T; step_noise:
    [M, T-1, B, F*S, C], the eps drawn at steps T .. 2; timesteps: t_1 < ... <
    t_T in (0, 1].  Returns the M clean chunks [M, B, F*S, C]; `caches` end
    holding every chunk's commit.
    """
    torch = _b._torch()
    M = noise.shape[0]
    T = len(timesteps)
    chunk_tokens = noise.shape[2]
    outputs = []
    for i in range(M):
        x = noise[i]
        pos0 = i * chunk_tokens
        for j in range(T, 0, -1):
            y0 = run_model(layers, caches, x, frames, commit=False, eps=eps, rope=rope, pos0=pos0)
            if j == 1:
                outputs.append(y0)
                run_model(layers, caches, y0, frames, commit=True, eps=eps, rope=rope, pos0=pos0)
            else:
                t = timesteps[j - 2]
                x = (1.0 - t) * y0 + t * step_noise[i, T - j]
    return torch.stack(outputs)
