"""ctypes binding of libsana_linattn.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/sana_linattn.h).  torch supplies device
memory and the stream handle.  There is no CPU fallback: if the library is
missing, loading raises.
"""

import ctypes
import os

import numpy as np

from . import build as _build
from .build import LIB_PATH

SANA_OK, SANA_ERR_INVALID, SANA_ERR_UNSUPPORTED, SANA_ERR_WORKSPACE, SANA_ERR_HIP = 0, -1, -2, -3, -4
SANA_DT_F32, SANA_DT_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 8 << 20  # SANA_NOALLOC_SCRATCH_BYTES in include/sana_linattn.h

EXPORTED = (
    "sana_linattn_workspace_bytes",
    "sana_linattn_forward_launches",
    "sana_linattn_forward",
    "sana_linattn_forward_strided",
    "sana_linattn_state_update",
    "sana_linattn_project_state",
    "sana_linattn_project_state_workspace_bytes",
    "sana_linattn_project_apply",
    "sana_linattn_block_forward",
    "sana_linattn_block_forward_noalloc",
    "sana_linattn_block_forward_strided",
    "sana_linattn_block_causal",
    "sana_linattn_block_causal_strided",
    "sana_linattn_block_causal_workspace_bytes",
    "sana_linattn_apply",
    "sana_linattn_backward",
    "sana_linattn_backward_strided",
    "sana_linattn_backward_saved",
    "sana_linattn_backward_workspace_bytes",
    "sana_linattn_state_update_backward",
    "sana_linattn_temporal_conv3",
    "sana_linattn_rope3d_table",
    "sana_linattn_rope3d_axes",
    "sana_linattn_status_string",
    "sana_linattn_source_hash",
)


class sana_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


class sana_rope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
                ("n_pos", ctypes.c_int64), ("pos_offset", ctypes.c_int64),
                ("grid", ctypes.c_int32 * 3), ("pairs", ctypes.c_int32 * 3)]


_LIB = None


def lib():
    """Load the library once and declare the C prototypes."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(or python -m linear_attention_diffusion_amd.build) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    rp = ctypes.POINTER(sana_rope)
    L.sana_linattn_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.sana_linattn_workspace_bytes.restype = sz
    L.sana_linattn_forward_launches.argtypes = [i32, i32, i64, i64, i32, i32, i32, i32]
    L.sana_linattn_forward_launches.restype = i32
    L.sana_linattn_forward.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, f32, rp, vp, sz, vp]
    L.sana_linattn_forward.restype = i32
    L.sana_linattn_state_update.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, rp, vp, sz, vp]
    L.sana_linattn_state_update.restype = i32
    L.sana_linattn_project_state.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, rp, vp, sz, vp]
    L.sana_linattn_project_state.restype = i32
    L.sana_linattn_project_state_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.sana_linattn_project_state_workspace_bytes.restype = sz
    L.sana_linattn_project_apply.argtypes = [vp, vp, vp, ctypes.POINTER(sana_layout), vp, vp, i32, i32, i64, i32,
                                             i32, i32, f32, rp, vp]
    L.sana_linattn_project_apply.restype = i32
    L.sana_linattn_block_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, f32,
                                             rp, vp, sz, vp]
    L.sana_linattn_block_forward.restype = i32
    L.sana_linattn_block_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, f32,
                                                     rp, vp]
    L.sana_linattn_block_forward_noalloc.restype = i32
    L.sana_linattn_block_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i32, f32,
                                            rp, vp, sz, vp]
    L.sana_linattn_block_causal.restype = i32
    L.sana_linattn_block_causal_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32, i32]
    L.sana_linattn_block_causal_workspace_bytes.restype = sz
    L.sana_linattn_apply.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, f32, rp, vp]
    L.sana_linattn_apply.restype = i32
    L.sana_linattn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i64,
                                        i32, i32, f32, rp, vp, sz, vp]
    L.sana_linattn_backward.restype = i32
    L.sana_linattn_backward_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i32, i32]
    L.sana_linattn_backward_workspace_bytes.restype = sz
    lp = ctypes.POINTER(sana_layout)
    L.sana_linattn_forward_strided.argtypes = [vp, vp, vp, vp, lp, lp, i32, i32, i64, i32, i32, f32, rp, vp, sz, vp]
    L.sana_linattn_forward_strided.restype = i32
    L.sana_linattn_block_forward_strided.argtypes = [vp, vp, vp, vp, lp, lp, vp, vp, vp, vp, i32, i32, i64, i32, i32,
                                                     f32, rp, vp, sz, vp]
    L.sana_linattn_block_forward_strided.restype = i32
    L.sana_linattn_block_causal_strided.argtypes = [vp, vp, vp, vp, lp, lp, vp, vp, vp, vp, i32, i32, i64, i64, i32,
                                                    i32, f32, rp, vp, sz, vp]
    L.sana_linattn_block_causal_strided.restype = i32
    L.sana_linattn_backward_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, lp, lp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                i64, i64, i32, i32, f32, rp, vp, sz, vp]
    L.sana_linattn_backward_strided.restype = i32
    L.sana_linattn_backward_saved.argtypes = [vp, vp, vp, vp, vp, vp, vp, lp, lp, vp, vp, vp, vp, i32, i32, i64, i64,
                                              i32, i32, f32, rp, vp, sz, vp]
    L.sana_linattn_backward_saved.restype = i32
    L.sana_linattn_state_update_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, rp, vp]
    L.sana_linattn_state_update_backward.restype = i32
    L.sana_linattn_temporal_conv3.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp]
    L.sana_linattn_temporal_conv3.restype = i32
    L.sana_linattn_rope3d_table.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.c_double, vp, vp]
    L.sana_linattn_rope3d_table.restype = i32
    L.sana_linattn_rope3d_axes.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.c_double, vp, vp]
    L.sana_linattn_rope3d_axes.restype = i32
    L.sana_linattn_status_string.argtypes = [i32]
    L.sana_linattn_status_string.restype = ctypes.c_char_p
    L.sana_linattn_source_hash.argtypes = []
    L.sana_linattn_source_hash.restype = ctypes.c_char_p
    # refuse a library older than the kernel sources next to it
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(LIB_PATH))), "csrc")
    if os.path.isdir(csrc):
        built, want = L.sana_linattn_source_hash().decode(), _build.source_hash(csrc)
        if built != want:
            raise ImportError(f"{LIB_PATH} was compiled from other kernel sources ({built}) than those in {csrc} "
                              f"({want}): run __graft_entry__.build() (or python -m "
                              "linear_attention_diffusion_amd.build) first")
    _LIB = L
    return L


class SanaError(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__(lib().sana_linattn_status_string(code).decode())


def _check(code):
    if code != SANA_OK:
        raise SanaError(code)


def sana_linattn_status_string(code):
    return lib().sana_linattn_status_string(code).decode()


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SANA_DT_BF16
    if t.dtype == torch.float32:
        return SANA_DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}: Q, K, V, O must be bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shape4(t, name, strided=False):
    """Shape of a [B, H, N, D] device tensor: contiguous, or with strided=True
    any view whose last dimension is contiguous."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, D], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if strided:
        if t.shape[3] > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} must have contiguous features (stride 1 in its last dimension)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return tuple(t.shape)


def _view(*ts):
    """The common sana_layout of tensors that share one view, or None when they
    are all contiguous."""
    strides = {tuple(t.stride()[:3]) for t in ts}
    if len(strides) != 1:
        raise ValueError("tensors passed as one group (q, k, v[, dout] or the outputs) must share their strides")
    if all(t.is_contiguous() for t in ts):
        return None
    b, h, n = strides.pop()
    return sana_layout(b, h, n)


def _lay(view):
    return None if view is None else ctypes.byref(view)


def _stream(stream, device):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Rope:
    """Device RoPE tables and the position of token 0: full tables [n_pos, D/2]
    (float32), or, with `grid` = (T, Hl, Wl) and `pairs` = (pt, ph, pw), the
    per-axis tables of a 3D RoPE back to back (1-D float32)."""

    def __init__(self, cos, sin, pos_offset=0, grid=None, pairs=None):
        torch = _torch()
        if cos.shape != sin.shape or cos.dim() != (1 if grid else 2):
            raise ValueError("cos and sin must both be [n_pos, D/2] (or 1-D per-axis tables with a grid)")
        if cos.dtype != torch.float32 or sin.dtype != torch.float32:
            raise TypeError("RoPE tables are float32")
        if not (cos.is_cuda and sin.is_cuda and cos.is_contiguous() and sin.is_contiguous()):
            raise ValueError("RoPE tables must be contiguous device tensors")
        if (grid is None) != (pairs is None):
            raise ValueError("the per-axis form needs both grid and pairs")
        self.cos, self.sin, self.pos_offset = cos, sin, int(pos_offset)
        self.grid = tuple(int(x) for x in grid) if grid else None
        self.pairs = tuple(int(x) for x in pairs) if pairs else None

    def at(self, pos_offset):
        return Rope(self.cos, self.sin, pos_offset, self.grid, self.pairs)

    @property
    def n_pos(self):
        return self.grid[0] * self.grid[1] * self.grid[2] if self.grid else self.cos.shape[0]

    def struct(self):
        r = sana_rope(self.cos.data_ptr(), self.sin.data_ptr(), self.n_pos, self.pos_offset)
        if self.grid:
            r.grid[:] = self.grid
            r.pairs[:] = self.pairs
        return r


def _rope_arg(rope):
    return None if rope is None else ctypes.byref(rope.struct())


def rope3d_table(T, Hl, Wl, D=32, split=(8, 12, 12), base=10000.0):
    """Host 3D RoPE tables (numpy float32 cos, sin of shape [T*Hl*Wl, D/2])."""
    n = T * Hl * Wl
    cos = np.empty((n, D // 2), np.float32)
    sin = np.empty((n, D // 2), np.float32)
    _check(lib().sana_linattn_rope3d_table(T, Hl, Wl, D, split[0], split[1], split[2], float(base),
                                           cos.ctypes.data_as(ctypes.c_void_p),
                                           sin.ctypes.data_as(ctypes.c_void_p)))
    return cos, sin


def rope3d_device(T, Hl, Wl, device, D=32, split=(8, 12, 12), base=10000.0):
    torch = _torch()
    cos, sin = rope3d_table(T, Hl, Wl, D, split, base)
    return Rope(torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device))


def rope3d_axes(T, Hl, Wl, D=32, split=(8, 12, 12), base=10000.0):
    """Host per-axis tables of the same 3D RoPE (numpy float32 cos, sin of
    T*dt/2 + Hl*dh/2 + Wl*dw/2 floats: the t, h and w tables back to back)."""
    n = T * split[0] // 2 + Hl * split[1] // 2 + Wl * split[2] // 2
    cos = np.empty(n, np.float32)
    sin = np.empty(n, np.float32)
    _check(lib().sana_linattn_rope3d_axes(T, Hl, Wl, D, split[0], split[1], split[2], float(base),
                                          cos.ctypes.data_as(ctypes.c_void_p),
                                          sin.ctypes.data_as(ctypes.c_void_p)))
    return cos, sin


def rope3d_axes_device(T, Hl, Wl, device, D=32, split=(8, 12, 12), base=10000.0):
    """The 3D RoPE in per-axis form (a few KB) on `device`."""
    torch = _torch()
    cos, sin = rope3d_axes(T, Hl, Wl, D, split, base)
    return Rope(torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device), grid=(T, Hl, Wl),
                pairs=(split[0] // 2, split[1] // 2, split[2] // 2))


def workspace_bytes(B, H, N, D=32, dtype=SANA_DT_BF16, has_rope=False):
    return int(lib().sana_linattn_workspace_bytes(B, H, N, D, dtype, int(bool(has_rope))))


def forward_launches(B, H, N, chunk=None, D=32, dtype=SANA_DT_BF16, rope_form=0, dense=True):
    """Kernel launches of one forward / block_forward (chunk None: one chunk)
    or block_causal call; rope_form 0 none, 1 full tables, 2 per-axis."""
    c = N if chunk is None else chunk
    return int(lib().sana_linattn_forward_launches(B, H, N, c if c > 0 else 1, D, dtype, rope_form, int(bool(dense))))


def make_workspace(B, H, N, device, D=32, dtype=SANA_DT_BF16, has_rope=False):
    torch = _torch()
    n = workspace_bytes(B, H, N, D, dtype, has_rope)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _workspace(ws, B, H, N, D, dt, has_rope, device):
    if ws is None:
        ws = make_workspace(B, H, N, device, D, dt, has_rope)
    return ws, ws.numel() * ws.element_size()


def sana_linattn_forward(q, k, v, o=None, eps=1e-6, rope=None, workspace=None, stream=None):
    """Non-causal ReLU linear attention; returns O (allocated contiguous if not
    given).  q, k, v (one shared view) and o may be strided [B, H, N, D] views,
    e.g. of a packed [B, N, 3, H, D] projection output."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q", strided=True)
    if _shape4(k, "k", strided=True) != (B, H, N, D) or _shape4(v, "v", strided=True) != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
    elif _shape4(o, "o", strided=True) != (B, H, N, D) or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    vin, vout = _view(q, k, v), _view(o)
    ws, nbytes = _workspace(workspace, B, H, N, D, dt, rope is not None, q.device)
    if vin is None and vout is None:
        _check(lib().sana_linattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, dt, float(eps),
                                          _rope_arg(rope), _ptr(ws), nbytes, _stream(stream, q.device)))
    else:
        _check(lib().sana_linattn_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _lay(vin), _lay(vout), B, H, N,
                                                  D, dt, float(eps), _rope_arg(rope), _ptr(ws), nbytes,
                                                  _stream(stream, q.device)))
    return o


def sana_linattn_state_update(k, v, kv_state, ksum_state, rope=None, workspace=None, stream=None):
    """kv_state += sum phi~(K)^T V, ksum_state += sum phi(K), in place."""
    torch = _torch()
    B, H, N, D = _shape4(k, "k")
    if _shape4(v, "v") != (B, H, N, D) or v.dtype != k.dtype:
        raise ValueError("k and v must match")
    if tuple(kv_state.shape) != (B, H, D, D) or tuple(ksum_state.shape) != (B, H, D):
        raise ValueError("kv_state must be [B, H, D, D] and ksum_state [B, H, D]")
    for t in (kv_state, ksum_state):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("states must be contiguous float32 device tensors")
    dt = _dtype_code(k)
    ws, nbytes = _workspace(workspace, B, H, N, D, dt, rope is not None, k.device)
    _check(lib().sana_linattn_state_update(_ptr(k), _ptr(v), _ptr(kv_state), _ptr(ksum_state), B, H, N, D, dt,
                                           _rope_arg(rope), _ptr(ws), nbytes, _stream(stream, k.device)))


def project_state_workspace_bytes(B, H, N, C, D=32, dtype=SANA_DT_BF16):
    return int(lib().sana_linattn_project_state_workspace_bytes(B, H, N, C, D, dtype))


def sana_linattn_project_state(x, w_k, w_v, kv_state, ksum_state, rope=None, workspace=None, stream=None):
    """kv_state += sum phi~(K)^T V, ksum_state += sum phi(K) for K = x W_k^T and
    V = x W_v^T (per head, rounded to bf16), without writing K or V.
    x: [B, N, C] bf16; w_k, w_v: [H * D, C] bf16 (a linear layer's weight
    layout); states [B, H, D, D] and [B, H, D] float32, updated in place.
    rope: a Rope (either form) rotating key n at position pos_offset + n."""
    torch = _torch()
    if x.dim() != 3 or w_k.dim() != 2 or tuple(w_v.shape) != tuple(w_k.shape):
        raise ValueError("x must be [B, N, C] and w_k, w_v [H * D, C] of one shape")
    B, N, C = x.shape
    if w_k.shape[1] != C:
        raise ValueError("weights must have C columns")
    if kv_state.dim() != 4 or tuple(ksum_state.shape) != tuple(kv_state.shape[:3]):
        raise ValueError("kv_state must be [B, H, D, D] and ksum_state [B, H, D]")
    H, D = kv_state.shape[1], kv_state.shape[3]
    if tuple(kv_state.shape) != (B, H, D, D) or w_k.shape[0] != H * D:
        raise ValueError("states must be [B, H, D, D] with H * D weight rows")
    for name, t in (("x", x), ("w_k", w_k), ("w_v", w_v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if x.dtype != torch.bfloat16 or w_k.dtype != torch.bfloat16 or w_v.dtype != torch.bfloat16:
        raise TypeError("x, w_k, w_v must be bfloat16")
    for t in (kv_state, ksum_state):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("states must be contiguous float32 device tensors")
    if workspace is None:
        n = project_state_workspace_bytes(B, H, N, C, D)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    _check(lib().sana_linattn_project_state(_ptr(x), _ptr(w_k), _ptr(w_v), _ptr(kv_state), _ptr(ksum_state), B, H,
                                            N, C, D, SANA_DT_BF16, _rope_arg(rope), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream, x.device)))


def sana_linattn_project_apply(x, w_q, kv_state, ksum_state, o=None, eps=1e-6, rope=None, stream=None):
    """O = phi~(Q).S / (phi(Q).z + eps) for Q = x W_q^T (per head, rounded to
    bf16), without writing Q.  x: [B, N, C] bf16; w_q: [H * D, C] bf16;
    states [B, H, D, D], [B, H, D] float32.  o: a [B, H, N, D] bf16 view
    (allocated contiguous if not given), e.g. of a [B, N, H, D] buffer."""
    torch = _torch()
    if x.dim() != 3 or w_q.dim() != 2:
        raise ValueError("x must be [B, N, C] and w_q [H * D, C]")
    B, N, C = x.shape
    if kv_state.dim() != 4 or tuple(ksum_state.shape) != tuple(kv_state.shape[:3]):
        raise ValueError("kv_state must be [B, H, D, D] and ksum_state [B, H, D]")
    H, D = kv_state.shape[1], kv_state.shape[3]
    if tuple(kv_state.shape) != (B, H, D, D) or tuple(w_q.shape) != (H * D, C):
        raise ValueError("states must be [B, H, D, D] with w_q [H * D, C]")
    for name, t in (("x", x), ("w_q", w_q)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    for t in (kv_state, ksum_state):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("states must be contiguous float32 device tensors")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=x.device)
    elif _shape4(o, "o", strided=True) != (B, H, N, D) or o.dtype != torch.bfloat16:
        raise ValueError("o must be a [B, H, N, D] bfloat16 view")
    vout = _view(o)
    _check(lib().sana_linattn_project_apply(_ptr(x), _ptr(w_q), _ptr(o), _lay(vout), _ptr(kv_state),
                                            _ptr(ksum_state), B, H, N, C, D, SANA_DT_BF16, float(eps),
                                            _rope_arg(rope), _stream(stream, x.device)))
    return o


def sana_linattn_block_forward(q, k, v, o=None, kv_in=None, ksum_in=None, kv_out=None, ksum_out=None,
                               eps=1e-6, rope=None, workspace=None, stream=None):
    """One block-causal chunk; returns O.  kv_in/ksum_in None = zero state;
    kv_out/ksum_out None = do not commit.  Strided views as for the forward."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q", strided=True)
    if _shape4(k, "k", strided=True) != (B, H, N, D) or _shape4(v, "v", strided=True) != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
    elif _shape4(o, "o", strided=True) != (B, H, N, D) or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    for t, shape in ((kv_in, (B, H, D, D)), (ksum_in, (B, H, D)), (kv_out, (B, H, D, D)), (ksum_out, (B, H, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [B, H, D, D] / [B, H, D]")
    dt = _dtype_code(q)
    vin, vout = _view(q, k, v), _view(o)
    ws, nbytes = _workspace(workspace, B, H, N, D, dt, rope is not None, q.device)
    if vin is None and vout is None:
        _check(lib().sana_linattn_block_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_in), _ptr(ksum_in),
                                                _ptr(kv_out), _ptr(ksum_out), B, H, N, D, dt, float(eps),
                                                _rope_arg(rope), _ptr(ws), nbytes, _stream(stream, q.device)))
    else:
        _check(lib().sana_linattn_block_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _lay(vin), _lay(vout),
                                                        _ptr(kv_in), _ptr(ksum_in), _ptr(kv_out), _ptr(ksum_out),
                                                        B, H, N, D, dt, float(eps), _rope_arg(rope), _ptr(ws),
                                                        nbytes, _stream(stream, q.device)))
    return o


def sana_linattn_block_forward_noalloc(q, k, v, o=None, kv_in=None, ksum_in=None, kv_out=None, ksum_out=None,
                                       eps=1e-6, rope=None, stream=None):
    """sana_linattn_block_forward without a workspace: the library's static
    per-GPU scratch array stands in for it (contiguous [B, H, N, D] tensors).
    Calls that overlap on one GPU race on that array."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q")
    if _shape4(k, "k") != (B, H, N, D) or _shape4(v, "v") != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
    elif _shape4(o, "o") != (B, H, N, D) or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    for t, shape in ((kv_in, (B, H, D, D)), (ksum_in, (B, H, D)), (kv_out, (B, H, D, D)), (ksum_out, (B, H, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [B, H, D, D] / [B, H, D]")
    _check(lib().sana_linattn_block_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_in), _ptr(ksum_in),
                                                    _ptr(kv_out), _ptr(ksum_out), B, H, N, D, _dtype_code(q),
                                                    float(eps), _rope_arg(rope), _stream(stream, q.device)))
    return o


def block_causal_workspace_bytes(B, H, N, chunk, D=32, dtype=SANA_DT_BF16, has_rope=False):
    return int(lib().sana_linattn_block_causal_workspace_bytes(B, H, N, chunk, D, dtype, int(bool(has_rope))))


def sana_linattn_block_causal(q, k, v, chunk, o=None, kv_in=None, ksum_in=None, kv_out=None, ksum_out=None,
                              eps=1e-6, rope=None, workspace=None, stream=None):
    """A whole sequence in block-causal chunks of `chunk` tokens; returns O.
    kv_in/ksum_in None = zero state; kv_out/ksum_out None = do not commit.
    Strided views as for the forward."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q", strided=True)
    if _shape4(k, "k", strided=True) != (B, H, N, D) or _shape4(v, "v", strided=True) != (B, H, N, D):
        raise ValueError("q, k, v must have the same shape")
    if o is None:
        o = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
    elif _shape4(o, "o", strided=True) != (B, H, N, D) or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    for t, shape in ((kv_in, (B, H, D, D)), (ksum_in, (B, H, D)), (kv_out, (B, H, D, D)), (ksum_out, (B, H, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [B, H, D, D] / [B, H, D]")
    dt = _dtype_code(q)
    if workspace is None:
        workspace = torch.empty(max(block_causal_workspace_bytes(B, H, N, chunk, D, dt, rope is not None), 256),
                                dtype=torch.uint8, device=q.device)
    vin, vout = _view(q, k, v), _view(o)
    if vin is None and vout is None:
        _check(lib().sana_linattn_block_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_in), _ptr(ksum_in),
                                               _ptr(kv_out), _ptr(ksum_out), B, H, N, int(chunk), D, dt, float(eps),
                                               _rope_arg(rope), _ptr(workspace), workspace.numel(),
                                               _stream(stream, q.device)))
    else:
        _check(lib().sana_linattn_block_causal_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _lay(vin), _lay(vout),
                                                       _ptr(kv_in), _ptr(ksum_in), _ptr(kv_out), _ptr(ksum_out), B, H,
                                                       N, int(chunk), D, dt, float(eps), _rope_arg(rope),
                                                       _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return o


def backward_workspace_bytes(B, H, N, chunk, D=32, dtype=SANA_DT_BF16, has_rope=False):
    return lib().sana_linattn_backward_workspace_bytes(B, H, N, int(chunk), D, dtype, int(bool(has_rope)))


def sana_linattn_backward(q, k, v, dout, chunk=None, dq=None, dk=None, dv=None, kv_in=None, ksum_in=None,
                          dkv_out=None, dksum_out=None, dkv_in=None, dksum_in=None, eps=1e-6, rope=None,
                          workspace=None, stream=None):
    """Gradients of sum(dout * O) (+ <dkv_out, S_last> + dksum_out . z_last) of
    block-causal attention with chunks of `chunk` tokens (None: one chunk, the
    non-causal forward).  Returns (dq, dk, dv); dkv_in/dksum_in, when given,
    receive the gradient of the carried state kv_in/ksum_in."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q", strided=True)
    for t, name in ((k, "k"), (v, "v"), (dout, "dout")):
        if _shape4(t, name, strided=True) != (B, H, N, D) or t.dtype != q.dtype:
            raise ValueError("q, k, v, dout must have the same shape and dtype")
    outs = []
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is None:
            t = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
        elif _shape4(t, name, strided=True) != (B, H, N, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
        outs.append(t)
    for t, shape in ((kv_in, (B, H, D, D)), (ksum_in, (B, H, D)), (dkv_out, (B, H, D, D)), (dksum_out, (B, H, D)),
                     (dkv_in, (B, H, D, D)), (dksum_in, (B, H, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [B, H, D, D] / [B, H, D]")
    L = N if chunk is None else int(chunk)
    L = max(L, 1)
    dt = _dtype_code(q)
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_bytes(B, H, N, L, D, dt, rope is not None), 256),
                                dtype=torch.uint8, device=q.device)
    vin, vout = _view(q, k, v, dout), _view(*outs)
    if vin is None and vout is None:
        _check(lib().sana_linattn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(outs[0]), _ptr(outs[1]),
                                           _ptr(outs[2]), _ptr(kv_in), _ptr(ksum_in), _ptr(dkv_out), _ptr(dksum_out),
                                           _ptr(dkv_in), _ptr(dksum_in), B, H, N, L, D, dt, float(eps),
                                           _rope_arg(rope), _ptr(workspace), workspace.numel(),
                                           _stream(stream, q.device)))
    else:
        _check(lib().sana_linattn_backward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(outs[0]),
                                                   _ptr(outs[1]), _ptr(outs[2]), _lay(vin), _lay(vout), _ptr(kv_in),
                                                   _ptr(ksum_in), _ptr(dkv_out), _ptr(dksum_out), _ptr(dkv_in),
                                                   _ptr(dksum_in), B, H, N, L, D, dt, float(eps), _rope_arg(rope),
                                                   _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return tuple(outs)


def sana_linattn_backward_saved(q, k, v, dout, workspace, chunk=None, dq=None, dk=None, dv=None, dkv_out=None,
                                dksum_out=None, dkv_in=None, dksum_in=None, eps=1e-6, rope=None, stream=None):
    """sana_linattn_backward reusing the chunk states that the forward call
    (forward, block_forward or block_causal with the same q, k, v, chunk, rope
    and carried state) left in `workspace`; the workspace must be unchanged
    since that call and is consumed (one backward per forward)."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q", strided=True)
    for t, name in ((k, "k"), (v, "v"), (dout, "dout")):
        if _shape4(t, name, strided=True) != (B, H, N, D) or t.dtype != q.dtype:
            raise ValueError("q, k, v, dout must have the same shape and dtype")
    outs = []
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is None:
            t = torch.empty((B, H, N, D), dtype=q.dtype, device=q.device)
        elif _shape4(t, name, strided=True) != (B, H, N, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
        outs.append(t)
    for t, shape in ((dkv_out, (B, H, D, D)), (dksum_out, (B, H, D)), (dkv_in, (B, H, D, D)), (dksum_in, (B, H, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [B, H, D, D] / [B, H, D]")
    L = max(N if chunk is None else int(chunk), 1)
    dt = _dtype_code(q)
    vin, vout = _view(q, k, v, dout), _view(*outs)
    _check(lib().sana_linattn_backward_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(outs[0]), _ptr(outs[1]),
                                             _ptr(outs[2]), _lay(vin), _lay(vout), _ptr(dkv_out), _ptr(dksum_out),
                                             _ptr(dkv_in), _ptr(dksum_in), B, H, N, L, D, dt, float(eps),
                                             _rope_arg(rope), _ptr(workspace), workspace.numel(),
                                             _stream(stream, q.device)))
    return tuple(outs)


def sana_linattn_state_update_backward(k, v, dkv, dksum, dk=None, dv=None, rope=None, stream=None):
    """dK, dV of L = <dkv, S> + dksum . z for the state S, z that k, v add;
    returns (dk, dv)."""
    torch = _torch()
    B, H, N, D = _shape4(k, "k")
    if _shape4(v, "v") != (B, H, N, D) or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    outs = []
    for t, name in ((dk, "dk"), (dv, "dv")):
        if t is None:
            t = torch.empty_like(k)
        elif _shape4(t, name) != (B, H, N, D) or t.dtype != k.dtype:
            raise ValueError(f"{name} must match k in shape and dtype")
        outs.append(t)
    for t, shape in ((dkv, (B, H, D, D)), (dksum, (B, H, D))):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("state gradients must be contiguous float32 [B, H, D, D] / [B, H, D]")
    _check(lib().sana_linattn_state_update_backward(_ptr(k), _ptr(v), _ptr(dkv), _ptr(dksum), _ptr(outs[0]),
                                                    _ptr(outs[1]), B, H, N, D, _dtype_code(k), _rope_arg(rope),
                                                    _stream(stream, k.device)))
    return tuple(outs)


def sana_linattn_temporal_conv3(x, w, bias=None, cache_in=None, cache_out=None, y=None, stream=None):
    """y = x + depthwise 3-tap temporal conv over frames (+ bias) of x [B, F, S, C],
    the previous chunk's last frame taken from cache_in [B, S, C] (None: zeros)
    and x's last frame stored to cache_out (may be cache_in; None: no commit).
    Returns y."""
    torch = _torch()
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, F, S, C] device tensor")
    B, F, S, C = x.shape
    if y is None:
        y = torch.empty_like(x)
    elif tuple(y.shape) != (B, F, S, C) or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must match x")
    if tuple(w.shape) != (C, 3) or w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError("w must be contiguous float32 [C, 3]")
    if bias is not None and (tuple(bias.shape) != (C,) or bias.dtype != torch.float32):
        raise ValueError("bias must be float32 [C]")
    for t in (cache_in, cache_out):
        if t is not None and (tuple(t.shape) != (B, S, C) or t.dtype != x.dtype or not t.is_contiguous()):
            raise ValueError("caches must be contiguous [B, S, C] of x's dtype")
    _check(lib().sana_linattn_temporal_conv3(_ptr(x), _ptr(y), _ptr(w), _ptr(bias), _ptr(cache_in), _ptr(cache_out),
                                             B, F, S, C, _dtype_code(x), _stream(stream, x.device)))
    return y


def sana_linattn_apply(q, kv_state, ksum_state, o=None, eps=1e-6, rope=None, stream=None):
    """O = phi~(Q).S / (phi(Q).z + eps) for a given state (read only); returns O."""
    torch = _torch()
    B, H, N, D = _shape4(q, "q")
    if o is None:
        o = torch.empty_like(q)
    elif _shape4(o, "o") != (B, H, N, D) or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    if tuple(kv_state.shape) != (B, H, D, D) or tuple(ksum_state.shape) != (B, H, D):
        raise ValueError("kv_state must be [B, H, D, D] and ksum_state [B, H, D]")
    for t in (kv_state, ksum_state):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("states must be contiguous float32 device tensors")
    _check(lib().sana_linattn_apply(_ptr(q), _ptr(o), _ptr(kv_state), _ptr(ksum_state), B, H, N, D, _dtype_code(q),
                                    float(eps), _rope_arg(rope), _stream(stream, q.device)))
    return o
