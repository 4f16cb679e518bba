"""Float64 replica of the block inference loop of
linear_attention_diffusion_amd/block_infer.py, built on the oracle (attention
and temporal conv) and NumPy matmuls.  Every tensor the device path stores in
bf16 is rounded to bf16 (nearest even) at the same point, so the two sides
differ only by accumulation order inside the fp32 device arithmetic."""

import numpy as np

import oracle
from workloads import bf16_bits_from_f32, f64_from_bf16_bits


def bf(x):
    """Round to bf16 (through fp32, nearest even), back to float64."""
    return f64_from_bf16_bits(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


class RefCache:
    def __init__(self, B, H, spatial, C):
        self.S = np.zeros((B, H, 32, 32))
        self.z = np.zeros((B, H, 32))
        # sum of the magnitudes of the terms summed into S: the scale of each
        # element's rounding error (z sums non-negative terms: it is its own)
        self.S_mag = np.zeros((B, H, 32, 32))
        self.conv_mag = np.zeros((B, spatial, C))   # |x| + |o| |W_o| of the committed frame
        self.conv = np.zeros((B, spatial, C))
        self.committed = False


class RefLayer:
    """w_q, w_k, w_v: [H 32, C] (a linear layer's weight rows); Q = x w_q^T etc.,
    rounded to bf16 as the device rounds them (stored by the unfused path,
    rounded in registers by the fused one)."""

    def __init__(self, wq, wk, wv, wo, conv_w, conv_b, H):
        self.wq, self.wk, self.wv = wq, wk, wv
        self.wo, self.conv_w, self.conv_b, self.H = wo, conv_w, conv_b, H

    def __call__(self, x, cache, frames, commit, eps, angles=None, pos0=0):
        B, N, C = x.shape
        H = self.H
        xf = x.reshape(B * N, C)
        q, k, v = (np.ascontiguousarray(bf(xf @ w.T).reshape(B, N, H, 32).transpose(0, 2, 1, 3))
                   for w in (self.wq, self.wk, self.wv))
        o, S_new, z_new = oracle.block_forward(q, k, v, cache.S, cache.z, eps, angles, pos0)
        o = bf(o).transpose(0, 2, 1, 3).reshape(B * N, H * 32)
        h = bf(x + bf(o @ self.wo).reshape(B, N, C))
        spatial = N // frames
        h_mag = np.abs(x) + (np.abs(o) @ np.abs(self.wo)).reshape(B, N, C)
        y, last = oracle.temporal_conv3(h.reshape(B, frames, spatial, C), self.conv_w, self.conv_b,
                                        cache.conv if cache.committed else None)
        if commit:
            cache.S_mag = cache.S_mag + np.matmul(np.swapaxes(_key_magnitude(k, angles, pos0), -1, -2), np.abs(v))
            cache.S = bf32(S_new)
            cache.z = bf32(z_new)
            cache.conv = last
            cache.conv_mag = h_mag.reshape(B, frames, spatial, C)[:, -1]
            cache.committed = True
        return bf(y).reshape(B, N, C)


def _key_magnitude(k, angles, pos0):
    """|phi(K)| per feature, or with RoPE the magnitude bound of each rotated
    component, |x0| |cos| + |x1| |sin| (pairs (2p, 2p+1))."""
    phik = np.maximum(k, 0.0)
    if angles is None:
        return phik
    a = angles[pos0:pos0 + k.shape[-2]]
    c, s = np.abs(np.cos(a)), np.abs(np.sin(a))
    out = np.empty_like(phik)
    out[..., 0::2] = phik[..., 0::2] * c + phik[..., 1::2] * s
    out[..., 1::2] = phik[..., 0::2] * s + phik[..., 1::2] * c
    return out


def bf32(x):
    """The device keeps the state in fp32."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def run_model(layers, caches, x, frames, commit, eps, angles=None, pos0=0):
    for layer, cache in zip(layers, caches):
        x = layer(x, cache, frames, commit, eps, angles, pos0)
    return x


def block_linear_diffusion(layers, caches, noise, step_noise, timesteps, frames, eps, angles=None):
    M = noise.shape[0]
    T = len(timesteps)
    outs = []
    for i in range(M):
        x = noise[i]
        pos0 = i * noise.shape[2]
        for j in range(T, 0, -1):
            y0 = run_model(layers, caches, x, frames, False, eps, angles, pos0)
            if j == 1:
                outs.append(y0)
                run_model(layers, caches, y0, frames, True, eps, angles, pos0)
            else:
                t = np.float32(timesteps[j - 2])
                x = bf(bf(np.float32(1.0 - t) * y0) + bf(t * step_noise[i, T - j]))
    return np.stack(outs)
