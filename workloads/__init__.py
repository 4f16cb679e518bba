"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no arithmetic of the attention method: it only draws the
random Q, K, V tensors, rounds them to the storage dtype, and names the
workload shapes.  Both the HIP path's tests/benchmark and the oracle's checks
take their inputs from here; neither side's arithmetic lives here.

Shapes (all [B, H, N, D], D = 32 = 1152/36 = 2240/70, the head width of
Sana-0.6B and Sana-1.6B: "Sana: Efficient High-Resolution Image Synthesis
with Linear Diffusion Transformers" research note, "Model architecture",
parameters paragraph):
  * 1024 px image through the 32x autoencoder -> 32x32 = 1024 latent tokens
    (same note, "Model architecture" item 1, DC-AE F32C32P1);
  * 4096 px -> 128x128 = 16384 tokens;
  * 720p, 81 frames through DCAE-V f32t4c32 -> 21x22x40 = 18480 tokens
    ("SANA-Video ..." paper notes, section 3 Stage 1);
  * 480p through Wan-VAE f8t4c16 with 2x patching -> 30x52 tokens per latent
    frame, chunks of 3 latent frames = 4680 tokens, 10 chunks.

The pages give no activation statistics, so i.i.d. Gaussians stand in for the
real activations (about half of each tensor is cut by the ReLU).

Recipe: numpy.random.default_rng(seed) (PCG64); float32 standard_normal drawn
in the order Q, K, V (then dO for the backward), each [B, H, N, D] in C order; bf16 workloads multiply by
0.5 (exact) and round to bf16 by round-to-nearest-even.  The block-causal
workload is drawn whole ([B, H, chunks*chunk_len, D]) and split along N.
"""

import hashlib
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int                      # total tokens per head (all chunks together in block mode)
    D: int = 32
    dtype: str = "bf16"         # storage dtype of Q, K, V and O: "bf16" or "f32"
    scale: float = 0.5          # multiplier applied to the N(0, 1) draws
    mode: str = "noncausal"     # "noncausal", "rope", "block"
    grid: Optional[Tuple[int, int, int]] = None   # (T, Hl, Wl) latent grid for RoPE
    chunk: Optional[int] = None                   # tokens per chunk in block mode
    eps: float = 1e-6
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def token_heads(self):
        return self.B * self.H * self.N

    @property
    def n_chunks(self):
        return 1 if self.chunk is None else -(-self.N // self.chunk)

    def bytes_per_token_head(self):
        """Algorithmic HBM bytes per token-head: read Q, K, V once, write O once."""
        return 4 * self.D * (2 if self.dtype == "bf16" else 4)


WORKLOADS = {
    w.name: w for w in [
        Workload("noncausal_f32_b1h1n256", B=1, H=1, N=256, dtype="f32", scale=1.0,
                 note="16x16 latent, fp32 I/O, parity case"),
        Workload("sana06b_1024px", B=4, H=36, N=1024,
                 note="Sana-0.6B layer at 1024 px: 32x32 latent, 36 heads"),
        Workload("sana16b_4096px", B=1, H=70, N=16384,
                 note="Sana-1.6B layer at 4096 px: 128x128 latent, 70 heads"),
        Workload("video720p_rope3d", B=1, H=70, N=21 * 22 * 40, mode="rope", grid=(21, 22, 40),
                 note="SANA-Video 720p layer: 21x22x40 latent, 3D RoPE numerator-only"),
        Workload("video480p_blockcausal", B=1, H=70, N=10 * 4680, mode="block", chunk=4680,
                 note="block-causal video: 10 chunks of 3x30x52 latent tokens"),
    ]
}

# The workload order used by reports.
WORKLOAD_ORDER = list(WORKLOADS)


def bf16_bits_from_f32(x):
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def f64_from_bf16_bits(bits):
    """Exact upcast of bfloat16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    """One seeded draw.  For bf16 workloads `raw` holds uint16 bit patterns; for
    f32 workloads it holds float32 arrays.  `f64` holds the exact float64 values
    of the same numbers, which is what the oracle consumes."""
    workload: Workload
    raw: dict
    f64: dict

    def sha256(self):
        h = hashlib.sha256()
        for name in ("q", "k", "v"):
            h.update(np.ascontiguousarray(self.raw[name]).tobytes())
        return h.hexdigest()


def generate(w: Workload, seed: Optional[int] = None, with_f64: bool = True,
             names=("q", "k", "v")) -> Inputs:
    """Draw the named tensors in order from one stream.  The backward's output
    gradient is drawn as a fourth tensor, "dout", after Q, K, V, which are
    therefore the same as the forward's."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.D)
    raw, f64 = {}, {}
    for name in names:
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.scale != 1.0:
            x *= np.float32(w.scale)
        if w.dtype == "bf16":
            raw[name] = bf16_bits_from_f32(x)
            if with_f64:
                f64[name] = f64_from_bf16_bits(raw[name])
        elif w.dtype == "f32":
            raw[name] = x
            if with_f64:
                f64[name] = x.astype(np.float64)
        else:
            raise ValueError(w.dtype)
    return Inputs(w, raw, f64)


@dataclass(frozen=True)
class ProjectionWorkload:
    """Input activations x [B, N, C] and the key, value and query weights
    [H*D, C] of one layer (the row layout of a linear layer's weight: row h*D + d is output
    feature d of head h)."""
    name: str
    B: int
    N: int
    C: int
    H: int
    D: int = 32
    seed: int = 0
    note: str = field(default="", compare=False)


# Sana-1.6B: width 2240 = 70 heads x 32 ("Sana" research note, "Model
# architecture", parameters paragraph); 4096 px -> 128 x 128 latent tokens.
PROJECTIONS = {
    p.name: p for p in [
        ProjectionWorkload("sana16b_4096px_kv_proj", B=1, N=16384, C=2240, H=70,
                           note="Sana-1.6B key/value projection of a 4096 px layer"),
    ]
}


@dataclass
class ProjectionInputs:
    workload: ProjectionWorkload
    raw: dict      # uint16 bf16 bit patterns: "x" [B, N, C], "w_k", "w_v", "w_q" [H*D, C]
    f64: dict      # their exact float64 values


def generate_projection(p: ProjectionWorkload, seed: Optional[int] = None, with_f64: bool = True,
                        names=("x", "w_k", "w_v")):
    """Recipe: numpy.random.default_rng(seed) (PCG64); float32 standard_normal
    drawn in the order x [B, N, C], w_k [H*D, C], w_v [H*D, C], w_q [H*D, C]
    (drawn up to the last of `names`, kept for those in `names`); the weights
    are multiplied by float32(1 / sqrt(C)) (unit-variance projections); all
    rounded to bf16 by round-to-nearest-even."""
    order = ("x", "w_k", "w_v", "w_q")
    rng = np.random.default_rng(p.seed if seed is None else seed)
    wscale = np.float32(1.0 / np.sqrt(p.C))
    raw, f64 = {}, {}
    for name in order[:1 + max(order.index(n) for n in names)]:
        shape = (p.B, p.N, p.C) if name == "x" else (p.H * p.D, p.C)
        a = rng.standard_normal(shape, dtype=np.float32)
        if name not in names:
            continue
        if name != "x":
            a *= wscale
        raw[name] = bf16_bits_from_f32(a)
        if with_f64:
            f64[name] = f64_from_bf16_bits(raw[name])
    return ProjectionInputs(p, raw, f64)


def reduced(w: Workload, **changes) -> Workload:
    """A smaller workload with the same distribution and mode (for fast parity cases)."""
    return replace(w, **changes)
