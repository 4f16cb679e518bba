"""CPU tests of the C ABI: the library loads and exports every declared entry
point, argument errors come back as status codes before anything is launched,
workspace sizing behaves, and the host RoPE table builder matches the oracle's
float64 angles.  No compute call reaches a GPU here."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
from linear_attention_diffusion_amd.binding import sana_rope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sana_linattn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sana_linattn_\w+)\s*\(", text)))


def test_header_declares_what_the_binding_exports():
    assert _declared() == sorted(la.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = la.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L._name], capture_output=True, text=True).stdout
    for name in _declared():
        assert re.search(rf"\bT {name}$", out, re.M), f"{name} not exported"


def test_status_strings():
    for code in (la.SANA_OK, la.SANA_ERR_INVALID, la.SANA_ERR_UNSUPPORTED, la.SANA_ERR_WORKSPACE, la.SANA_ERR_HIP):
        assert la.sana_linattn_status_string(code).startswith("SANA_")
    assert "unknown" in la.sana_linattn_status_string(42)


def test_workspace_bytes():
    wb = la.workspace_bytes
    assert wb(1, 70, 0) == 0 and wb(0, 70, 100) == 0
    assert wb(1, 70, 16384) > 0
    assert wb(1, 70, 16384) % 256 == 0
    # invalid sizes -> 0
    assert wb(1, 70, 100, D=64) == 0 and wb(-1, 70, 100) == 0 and wb(1, 70, 100, dtype=7) == 0
    # never smaller than the state it holds (33 x 32 floats per head), and
    # bounded: at most 64 partials + 1 state + 1 counter per head
    for B, H, N in [(1, 1, 1), (4, 36, 1024), (1, 70, 16384), (1, 70, 4680), (1, 70, 46800), (2, 3, 5)]:
        for rope in (False, True):
            n = wb(B, H, N, has_rope=rope)
            assert B * H * 33 * 32 * 4 <= n <= B * H * (33 * 32 * 4 * 65 + 8) + 768, (B, H, N, n)
    # the same for either dtype
    assert wb(1, 70, 18480) == wb(1, 70, 18480, dtype=la.SANA_DT_F32)
    assert wb(1, 70, 18480, has_rope=True) == wb(1, 70, 18480, dtype=la.SANA_DT_F32, has_rope=True)


# Fake, 256-byte-aligned addresses.  Every call below carries an argument error,
# so the library must return before touching them or the GPU.
A = 0x10000000
Bp = 0x20000000
C = 0x30000000
Dp = 0x40000000
WS = 0x50000000


def _fwd(q=A, k=Bp, v=C, o=Dp, B=1, H=2, N=64, D=32, dt=la.SANA_DT_BF16, eps=1e-6, rope=None,
         ws=WS, nbytes=None):
    if nbytes is None:
        nbytes = la.workspace_bytes(max(B, 0), max(H, 0), max(N, 0))
    return la.lib().sana_linattn_forward(q, k, v, o, B, H, N, D, dt, eps, rope, ws, nbytes, None)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """More heads than the static scratch array holds: SANA_ERR_WORKSPACE before
    any device call (the pointers are fake)."""
    L = la.lib()
    limit = la.binding.NOALLOC_SCRATCH_BYTES
    for B, H, N in [(1, 4000, 64), (2, 1000, 5000), (1, 2000, 16384)]:
        assert la.workspace_bytes(B, H, N) > limit
        rc = L.sana_linattn_block_forward_noalloc(A, Bp, C, Dp, None, None, None, None, B, H, N, 32,
                                                  la.SANA_DT_BF16, 1e-6, None, None)
        assert rc == la.SANA_ERR_WORKSPACE, (B, H, N, rc)
    # the workloads this build measures fit
    for B, H, N in [(1, 70, 4680), (1, 70, 16384), (1, 70, 18480), (4, 36, 1024)]:
        for rope in (False, True):
            assert la.workspace_bytes(B, H, N, has_rope=rope) <= limit


def test_forward_argument_errors():
    E = la
    assert _fwd(q=None) == E.SANA_ERR_INVALID
    assert _fwd(o=None) == E.SANA_ERR_INVALID
    assert _fwd(q=A + 8) == E.SANA_ERR_INVALID            # misaligned
    assert _fwd(B=-1) == E.SANA_ERR_INVALID
    assert _fwd(N=-5) == E.SANA_ERR_INVALID
    assert _fwd(D=0) == E.SANA_ERR_INVALID
    assert _fwd(D=64) == E.SANA_ERR_UNSUPPORTED
    assert _fwd(D=16) == E.SANA_ERR_UNSUPPORTED
    assert _fwd(dt=5) == E.SANA_ERR_INVALID
    assert _fwd(eps=-1.0) == E.SANA_ERR_INVALID
    assert _fwd(eps=float("nan")) == E.SANA_ERR_INVALID
    assert _fwd(eps=float("inf")) == E.SANA_ERR_INVALID
    assert _fwd(o=A) == E.SANA_ERR_INVALID                # o aliases q
    assert _fwd(o=Bp + 64) == E.SANA_ERR_INVALID          # o overlaps k
    assert _fwd(ws=None) == E.SANA_ERR_WORKSPACE
    assert _fwd(nbytes=16) == E.SANA_ERR_WORKSPACE
    assert _fwd(ws=WS + 16) == E.SANA_ERR_INVALID         # workspace not 256-byte aligned
    # empty problems are no-ops, whatever the pointers
    assert _fwd(q=None, k=None, v=None, o=None, N=0, ws=None) == E.SANA_OK
    assert _fwd(q=None, k=None, v=None, o=None, B=0, ws=None) == E.SANA_OK
    # RoPE tables must cover the positions read
    r = sana_rope(0x60000000, 0x70000000, 63, 0)
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    r = sana_rope(0x60000000, 0x70000000, 100, 40)
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    r = sana_rope(0x60000000, 0x70000000, 100, -1)
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    r = sana_rope(None, 0x70000000, 100, 0)
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    r = sana_rope(0x60000004, 0x70000000, 100, 0)
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID


def test_state_update_argument_errors():
    L = la.lib()
    n = la.workspace_bytes(1, 2, 64)

    def su(k=A, v=Bp, kv=C, ks=Dp, N=64, D=32, ws=WS):
        return L.sana_linattn_state_update(k, v, kv, ks, 1, 2, N, D, la.SANA_DT_BF16, None, ws, n, None)

    assert su(kv=None) == la.SANA_ERR_INVALID
    assert su(ks=None) == la.SANA_ERR_INVALID
    assert su(kv=C + 2) == la.SANA_ERR_INVALID
    assert su(ks=C + 4 * 1024) == la.SANA_ERR_INVALID     # ksum overlaps kv (2 heads x 4 KiB)
    assert su(kv=A) == la.SANA_ERR_INVALID                # state overlaps k
    assert su(D=48) == la.SANA_ERR_UNSUPPORTED
    assert su(ws=None) == la.SANA_ERR_WORKSPACE
    assert su(k=None, v=None, kv=None, ks=None, N=0, ws=None) == la.SANA_OK


def test_project_state_argument_errors_and_workspace():
    L = la.lib()
    pw = la.project_state_workspace_bytes
    assert pw(1, 70, 16384, 2240) > 0 and pw(1, 70, 16384, 2240) % 256 == 0
    # one partial per 256-token range when there are several ranges, plus the state
    assert pw(1, 70, 16384, 2240) == 70 * 64 * 4224 + 70 * 4224
    assert pw(1, 3, 256, 64) == ((3 * 4224 + 255) // 256) * 256       # one range: no partials
    # at most 128 ranges per head, whatever N
    assert pw(1, 2, 10 ** 7, 32) <= 2 * 129 * 4224 + 512
    assert pw(1, 2, 0, 64) == 0 and pw(0, 2, 64, 64) == 0
    assert pw(1, 2, 64, 48) == 0 and pw(1, 2, 64, 0) == 0 and pw(1, 2, 64, 65536 + 32) == 0
    assert pw(1, 2, 64, 64, D=64) == 0 and pw(1, 2, 64, 64, dtype=la.SANA_DT_F32) == 0
    n = pw(1, 2, 1000, 64)

    def ps(x=A, wk=Bp, wv=C, kv=Dp, ks=Dp + 8192, B=1, H=2, N=1000, Cin=64, D=32, dt=la.SANA_DT_BF16, rope=None,
           ws=WS, nbytes=n):
        return L.sana_linattn_project_state(x, wk, wv, kv, ks, B, H, N, Cin, D, dt, rope, ws, nbytes, None)

    E = la
    assert ps(x=None) == E.SANA_ERR_INVALID
    assert ps(wv=None) == E.SANA_ERR_INVALID
    assert ps(wk=Bp + 8) == E.SANA_ERR_INVALID             # misaligned weights
    assert ps(kv=None) == E.SANA_ERR_INVALID
    assert ps(ks=Dp + 2) == E.SANA_ERR_INVALID             # misaligned state
    assert ps(ks=Dp + 4096) == E.SANA_ERR_INVALID          # ksum overlaps kv (2 heads x 4 KiB)
    assert ps(kv=A + 1024) == E.SANA_ERR_INVALID           # state inside x
    assert ps(ks=Bp + 64) == E.SANA_ERR_INVALID            # ksum inside w_k
    assert ps(Cin=48) == E.SANA_ERR_INVALID                # not a multiple of 32
    assert ps(Cin=0) == E.SANA_ERR_INVALID
    assert ps(Cin=65536 + 32) == E.SANA_ERR_INVALID
    assert ps(B=-1) == E.SANA_ERR_INVALID
    assert ps(N=-1) == E.SANA_ERR_INVALID
    assert ps(dt=9) == E.SANA_ERR_INVALID
    assert ps(D=64) == E.SANA_ERR_UNSUPPORTED
    assert ps(dt=la.SANA_DT_F32) == E.SANA_ERR_UNSUPPORTED
    assert ps(ws=None) == E.SANA_ERR_WORKSPACE
    assert ps(nbytes=n - 1) == E.SANA_ERR_WORKSPACE
    assert ps(ws=WS + 64) == E.SANA_ERR_INVALID
    # RoPE tables must cover the N positions read
    r = sana_rope(0x60000000, 0x70000000, 999, 0)
    assert ps(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    r = sana_rope(0x60000000, 0x70000000, 1000, 1)
    assert ps(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    # no tokens or no heads: the states stay as they are, nothing is touched
    assert ps(x=None, wk=None, wv=None, kv=None, ks=None, N=0, ws=None) == E.SANA_OK
    assert ps(x=None, wk=None, wv=None, kv=None, ks=None, B=0, ws=None) == E.SANA_OK


def test_binding_project_state_checks():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 2, 32, 32)
    z = torch.zeros(1, 2, 32)
    with pytest.raises(ValueError):
        la.sana_linattn_project_state(x, w, w, kv, z)          # host tensors
    with pytest.raises(ValueError):
        la.sana_linattn_project_state(x[0], w, w, kv, z)       # x must be [B, N, C]
    with pytest.raises(ValueError):
        la.sana_linattn_project_state(x, w[:, :32], w[:, :32], kv, z)   # C mismatch
    with pytest.raises(ValueError):
        la.sana_linattn_project_state(x, w, w, kv[:, :1], z[:, :1])     # H * D != weight rows


def test_project_apply_argument_errors():
    L = la.lib()
    E = la
    def pa(x=A, wq=Bp, o=WS, lay=None, kv=Dp, ks=Dp + 8192, B=1, H=2, N=1000, Cin=64, D=32,
           dt=la.SANA_DT_BF16, eps=1e-6, rope=None):
        return L.sana_linattn_project_apply(x, wq, o, lay, kv, ks, B, H, N, Cin, D, dt, eps, rope, None)

    assert pa(x=None) == E.SANA_ERR_INVALID
    assert pa(wq=None) == E.SANA_ERR_INVALID
    assert pa(o=None) == E.SANA_ERR_INVALID
    assert pa(kv=None) == E.SANA_ERR_INVALID
    assert pa(ks=Dp + 2) == E.SANA_ERR_INVALID             # misaligned state
    assert pa(wq=Bp + 8) == E.SANA_ERR_INVALID             # misaligned weights
    assert pa(o=A + 4096) == E.SANA_ERR_INVALID            # output inside x
    assert pa(o=Bp + 64) == E.SANA_ERR_INVALID             # output inside w_q
    assert pa(o=Dp - 64) == E.SANA_ERR_INVALID             # output runs into kv
    assert pa(Cin=48) == E.SANA_ERR_INVALID                # not a multiple of 32
    assert pa(Cin=0) == E.SANA_ERR_INVALID
    assert pa(B=-1) == E.SANA_ERR_INVALID
    assert pa(N=-1) == E.SANA_ERR_INVALID
    assert pa(eps=-1.0) == E.SANA_ERR_INVALID
    assert pa(eps=float("nan")) == E.SANA_ERR_INVALID
    assert pa(D=64) == E.SANA_ERR_UNSUPPORTED
    assert pa(dt=la.SANA_DT_F32) == E.SANA_ERR_UNSUPPORTED
    assert pa(lay=ctypes.byref(la.sana_layout(1000 * 2 * 32, 32, 16))) == E.SANA_ERR_INVALID   # token stride < D
    r = sana_rope(0x60000000, 0x70000000, 999, 0)          # tables shorter than N
    assert pa(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID
    # no tokens or no heads: nothing is touched
    assert pa(x=None, wq=None, o=None, kv=None, ks=None, N=0) == E.SANA_OK
    assert pa(x=None, wq=None, o=None, kv=None, ks=None, B=0) == E.SANA_OK


def test_binding_project_apply_checks():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 2, 32, 32)
    z = torch.zeros(1, 2, 32)
    with pytest.raises(ValueError):
        la.sana_linattn_project_apply(x, w, kv, z)                      # host tensors
    with pytest.raises(ValueError):
        la.sana_linattn_project_apply(x[0], w, kv, z)                   # x must be [B, N, C]
    with pytest.raises(ValueError):
        la.sana_linattn_project_apply(x, w, kv[:, :1], z[:, :1])        # H * D != weight rows
    with pytest.raises(ValueError):
        la.sana_linattn_project_apply(x, w, kv, z[:, :, :16])           # ksum shape


def test_block_forward_argument_errors():
    L = la.lib()
    n = la.workspace_bytes(1, 2, 64)
    S_IN, Z_IN, S_OUT, Z_OUT = 0x80000000, 0x90000000, 0xA0000000, 0xB0000000

    def bf(q=A, o=Dp, kv_in=S_IN, ks_in=Z_IN, kv_out=S_OUT, ks_out=Z_OUT):
        return L.sana_linattn_block_forward(q, Bp, C, o, kv_in, ks_in, kv_out, ks_out, 1, 2, 64, 32,
                                            la.SANA_DT_BF16, 1e-6, None, WS, n, None)

    assert bf(kv_in=None) == la.SANA_ERR_INVALID          # kv_in without ksum_in
    assert bf(ks_out=None) == la.SANA_ERR_INVALID         # kv_out without ksum_out
    assert bf(kv_out=S_IN + 64) == la.SANA_ERR_INVALID    # partial overlap of in and out states
    assert bf(ks_out=S_IN) == la.SANA_ERR_INVALID         # ksum_out inside kv_in
    assert bf(kv_in=A) == la.SANA_ERR_INVALID             # state overlaps q
    assert bf(o=C) == la.SANA_ERR_INVALID                 # o aliases v
    assert bf(q=None) == la.SANA_ERR_INVALID


def test_rope3d_table_matches_oracle_angles():
    import oracle
    T, Hl, Wl = 4, 6, 5
    cos, sin = la.rope3d_table(T, Hl, Wl)
    ang = oracle.rope3d_angles(T, Hl, Wl)
    # float32 rounding of cos/sin only
    np.testing.assert_allclose(cos, np.cos(ang), rtol=0, atol=6e-8)
    np.testing.assert_allclose(sin, np.sin(ang), rtol=0, atol=6e-8)
    # full 720p grid: same
    cos, sin = la.rope3d_table(21, 22, 40)
    ang = oracle.rope3d_angles(21, 22, 40)
    assert np.max(np.abs(cos - np.cos(ang))) < 6e-8 and np.max(np.abs(sin - np.sin(ang))) < 6e-8


def test_rope3d_table_errors():
    L = la.lib()
    buf = np.empty(64, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.sana_linattn_rope3d_table(1, 2, 2, 32, 8, 12, 10, 1e4, p, p) == la.SANA_ERR_INVALID  # sum != D
    assert L.sana_linattn_rope3d_table(1, 2, 2, 32, 7, 13, 12, 1e4, p, p) == la.SANA_ERR_INVALID  # odd split
    assert L.sana_linattn_rope3d_table(1, 2, 2, 32, 8, 12, 12, 0.0, p, p) == la.SANA_ERR_INVALID  # bad base
    assert L.sana_linattn_rope3d_table(1, 2, 2, 32, 8, 12, 12, 1e4, None, p) == la.SANA_ERR_INVALID
    assert L.sana_linattn_rope3d_table(0, 2, 2, 32, 8, 12, 12, 1e4, None, None) == la.SANA_OK


def _axes_index(T, Hl, Wl, pairs):
    """Per-axis table offset of pair p at position n, written out plainly."""
    pt, ph, pw = pairs
    idx = np.empty((T * Hl * Wl, pt + ph + pw), np.int64)
    for t in range(T):
        for h in range(Hl):
            for w in range(Wl):
                n = (t * Hl + h) * Wl + w
                for p in range(pt + ph + pw):
                    if p < pt:
                        idx[n, p] = t * pt + p
                    elif p < pt + ph:
                        idx[n, p] = T * pt + h * ph + (p - pt)
                    else:
                        idx[n, p] = T * pt + Hl * ph + w * pw + (p - pt - ph)
    return idx


@pytest.mark.parametrize("grid,split", [((4, 6, 5), (8, 12, 12)), ((21, 22, 40), (8, 12, 12)),
                                        ((3, 2, 7), (4, 8, 20))])
def test_rope3d_axes_equal_the_full_tables(grid, split):
    """Every entry of the full table is, bit for bit, the per-axis entry of its
    position's coordinate (the form the kernels stage in LDS)."""
    cos_a, sin_a = la.rope3d_axes(*grid, split=split)
    cos_f, sin_f = la.rope3d_table(*grid, split=split)
    idx = _axes_index(*grid, tuple(x // 2 for x in split))
    assert cos_a.size == grid[0] * split[0] // 2 + grid[1] * split[1] // 2 + grid[2] * split[2] // 2
    assert np.array_equal(cos_a[idx], cos_f) and np.array_equal(sin_a[idx], sin_f)


def test_rope3d_axes_argument_errors():
    L = la.lib()
    buf = np.empty(64, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.sana_linattn_rope3d_axes(1, 2, 2, 32, 8, 12, 10, 1e4, p, p) == la.SANA_ERR_INVALID
    assert L.sana_linattn_rope3d_axes(1, 2, 2, 32, 7, 13, 12, 1e4, p, p) == la.SANA_ERR_INVALID
    assert L.sana_linattn_rope3d_axes(1, 2, 2, 32, 8, 12, 12, -1.0, p, p) == la.SANA_ERR_INVALID
    assert L.sana_linattn_rope3d_axes(1, 2, 2, 32, 8, 12, 12, 1e4, p, None) == la.SANA_ERR_INVALID
    assert L.sana_linattn_rope3d_axes(0, 0, 0, 32, 8, 12, 12, 1e4, None, None) == la.SANA_OK


def test_rope_axis_form_argument_errors():
    """The per-axis RoPE form is checked before any launch: a grid matching
    n_pos, pairs summing to 16, tables within the LDS copy, exact
    coordinates, and no pairs in the full form."""
    def axes(grid=(1, 8, 8), pairs=(4, 6, 6), n_pos=None, pos=0, cos=0x60000000):
        r = sana_rope(cos, 0x70000000, grid[0] * grid[1] * grid[2] if n_pos is None else n_pos, pos)
        r.grid[:] = grid
        r.pairs[:] = pairs
        return _fwd(rope=ctypes.byref(r))
    E = la
    assert axes(pairs=(4, 6, 5)) == E.SANA_ERR_INVALID            # pairs do not sum to D/2
    assert axes(pairs=(-1, 6, 11)) == E.SANA_ERR_INVALID
    assert axes(pairs=(3, 6, 7)) == E.SANA_ERR_INVALID             # odd pair counts
    assert axes(grid=(1, 8, 0)) == E.SANA_ERR_INVALID             # empty axis
    assert axes(grid=(1, -8, -8)) == E.SANA_ERR_INVALID
    assert axes(n_pos=65) == E.SANA_ERR_INVALID                   # n_pos is the grid's size
    assert axes(grid=(1, 8, 7)) == E.SANA_ERR_INVALID             # 56 positions < 64 tokens
    assert axes(pos=1) == E.SANA_ERR_INVALID                      # 65th position outside the grid
    assert axes(grid=(1, 4, 200), pairs=(0, 0, 16)) == E.SANA_ERR_INVALID   # 3200 floats > 1024
    assert axes(grid=(1, 1024, 1024), pairs=(16, 0, 0)) == E.SANA_ERR_INVALID  # Hl*Wl >= 2^20
    assert axes(cos=0x60000002) == E.SANA_ERR_INVALID             # tables 4-byte aligned
    r = sana_rope(0x60000000, 0x70000000, 64, 0)
    r.pairs[:] = (4, 6, 6)                                        # pairs without a grid
    assert _fwd(rope=ctypes.byref(r)) == E.SANA_ERR_INVALID


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        la.sana_linattn_forward(x, x, x)


def test_binding_rope_checks():
    torch = pytest.importorskip("torch")
    t2 = torch.zeros(8, 16)
    t1 = torch.zeros(40)
    with pytest.raises(ValueError):
        la.Rope(t2, t2)                                   # host tensors
    with pytest.raises(ValueError):
        la.Rope(t1, t1, grid=(1, 2, 4))                   # grid without pairs
    with pytest.raises(ValueError):
        la.Rope(t2, t2, grid=(1, 2, 4), pairs=(4, 6, 6))  # per-axis tables are 1-D
    with pytest.raises(TypeError):
        la.Rope(t2.double(), t2.double())


def test_apply_argument_errors():
    L = la.lib()

    def ap(q=A, o=Dp, kv=C, ks=0x50000000, N=64, D=32, eps=1e-6):
        return L.sana_linattn_apply(q, o, kv, ks, 1, 2, N, D, la.SANA_DT_BF16, eps, None, None)

    assert ap(q=None) == la.SANA_ERR_INVALID
    assert ap(kv=None) == la.SANA_ERR_INVALID
    assert ap(ks=None) == la.SANA_ERR_INVALID
    assert ap(o=A) == la.SANA_ERR_INVALID                 # o aliases q
    assert ap(o=C) == la.SANA_ERR_INVALID                 # o overlaps the state
    assert ap(eps=-1.0) == la.SANA_ERR_INVALID
    assert ap(D=64) == la.SANA_ERR_UNSUPPORTED
    assert ap(q=None, o=None, kv=None, ks=None, N=0) == la.SANA_OK


def test_block_causal_argument_errors_and_workspace():
    L = la.lib()
    n = la.block_causal_workspace_bytes(1, 2, 640, 64)
    assert n >= la.workspace_bytes(1, 2, 640)          # per-chunk states on top of one state
    assert la.block_causal_workspace_bytes(1, 2, 640, 640) == la.workspace_bytes(1, 2, 640)
    assert la.block_causal_workspace_bytes(1, 2, 640, 0) == 0
    assert la.block_causal_workspace_bytes(1, 2, 640, 7) > la.block_causal_workspace_bytes(1, 2, 640, 70)

    def bc(chunk=64, ws=WS, nbytes=n, q=A):
        return L.sana_linattn_block_causal(q, Bp, C, Dp, None, None, None, None, 1, 2, 640, chunk, 32,
                                           la.SANA_DT_BF16, 1e-6, None, ws, nbytes, None)

    assert bc(chunk=0) == la.SANA_ERR_INVALID
    assert bc(chunk=-4) == la.SANA_ERR_INVALID
    assert bc(ws=None) == la.SANA_ERR_WORKSPACE
    assert bc(nbytes=la.workspace_bytes(1, 2, 640)) == la.SANA_ERR_WORKSPACE   # too small for 10 chunks
    assert bc(q=None) == la.SANA_ERR_INVALID


def test_backward_argument_errors_and_workspace():
    L = la.lib()
    n = la.backward_workspace_bytes(1, 2, 640, 64)
    assert n == la.block_causal_workspace_bytes(1, 2, 640, 64)
    assert la.backward_workspace_bytes(1, 2, 640, 0) == 0
    span = 1 * 2 * 640 * 32 * 2                       # bytes of one bf16 [1, 2, 640, 32] tensor
    dQ, dK, dV = (0x60000000 + i * 0x01000000 for i in range(3))
    S1, Z1, S2, Z2 = 0x68000000, 0x68100000, 0x68200000, 0x68300000

    def bw(q=A, k=Bp, v=C, do=Dp, dq=dQ, dk=dK, dv=dV, kv_in=None, ks_in=None, dkv_out=None, dks_out=None,
           dkv_in=None, dks_in=None, N=640, chunk=64, eps=1e-6, ws=WS, nbytes=n):
        return L.sana_linattn_backward(q, k, v, do, dq, dk, dv, kv_in, ks_in, dkv_out, dks_out, dkv_in, dks_in,
                                       1, 2, N, chunk, 32, la.SANA_DT_BF16, eps, None, ws, nbytes, None)

    assert bw(chunk=0) == la.SANA_ERR_INVALID
    assert bw(eps=-1.0) == la.SANA_ERR_INVALID
    assert bw(do=None) == la.SANA_ERR_INVALID
    assert bw(dv=None) == la.SANA_ERR_INVALID
    assert bw(dq=dQ + 8) == la.SANA_ERR_INVALID             # misaligned
    assert bw(dq=A) == la.SANA_ERR_INVALID                  # output aliases an input
    assert bw(dk=dQ + 64) == la.SANA_ERR_INVALID            # outputs overlap
    assert bw(kv_in=S1) == la.SANA_ERR_INVALID              # state without its key sum
    assert bw(dkv_out=S1) == la.SANA_ERR_INVALID
    assert bw(dkv_in=S1) == la.SANA_ERR_INVALID
    assert bw(dkv_out=S1, dks_out=Z1, dkv_in=S1 + 64, dks_in=Z2) == la.SANA_ERR_INVALID   # partial overlap
    assert bw(dkv_in=dV, dks_in=Z1) == la.SANA_ERR_INVALID  # state gradient overlaps an output
    assert bw(kv_in=S1, ks_in=Z1, dkv_in=S1, dks_in=Z2) == la.SANA_ERR_INVALID   # only dkv_out may be shared
    assert bw(ws=None) == la.SANA_ERR_WORKSPACE
    assert bw(nbytes=la.workspace_bytes(1, 2, 640)) == la.SANA_ERR_WORKSPACE
    assert bw(q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None, N=0, ws=None) == la.SANA_OK
    assert span < 0x01000000

    # the saved-state backward checks the same arguments (it has no carried state)
    def bws(dq=dQ, dkv_out=None, dks_out=None, dkv_in=None, dks_in=None, chunk=64, ws=WS, nbytes=n):
        return L.sana_linattn_backward_saved(A, Bp, C, Dp, dq, dK, dV, None, None, dkv_out, dks_out, dkv_in, dks_in,
                                             1, 2, 640, chunk, 32, la.SANA_DT_BF16, 1e-6, None, ws, nbytes, None)
    assert bws(chunk=0) == la.SANA_ERR_INVALID
    assert bws(dq=A) == la.SANA_ERR_INVALID
    assert bws(dkv_out=S1) == la.SANA_ERR_INVALID
    assert bws(dkv_in=dV, dks_in=Z1) == la.SANA_ERR_INVALID
    assert bws(ws=None) == la.SANA_ERR_WORKSPACE
    assert bws(nbytes=16) == la.SANA_ERR_WORKSPACE


def test_workspace_may_not_overlap_the_call_buffers():
    """The part of the workspace a call writes may overlap none of its tensors,
    states or RoPE tables: SANA_ERR_INVALID before anything is launched."""
    L = la.lib()
    E = la.SANA_ERR_INVALID
    assert _fwd(ws=A) == E                      # over q
    assert _fwd(ws=A + 4096) == E               # inside q (2 heads x 64 tokens x 64 B = 8 KiB)
    assert _fwd(ws=Dp) == E                     # over o
    assert _fwd(ws=Bp + 256) == E               # inside k
    tables = sana_rope(WS + 1024, 0x70000000, 64, 0)   # cos table inside the workspace
    assert _fwd(rope=ctypes.byref(tables), nbytes=la.workspace_bytes(1, 2, 64, has_rope=True)) == E
    tables = sana_rope(0x60000000, WS, 64, 0)          # sin table at the workspace
    assert _fwd(rope=ctypes.byref(tables), nbytes=la.workspace_bytes(1, 2, 64, has_rope=True)) == E
    # a workspace right after q's last byte is fine as far as overlaps go (the
    # call then fails later only because the pointers are fake: not tested)
    n = la.workspace_bytes(1, 2, 64)
    S, Z = 0x68000000, 0x68100000
    assert L.sana_linattn_block_forward(A, Bp, C, Dp, S, Z, S, Z, 1, 2, 64, 32, la.SANA_DT_BF16, 1e-6, None, S, n,
                                        None) == E              # over the state it commits
    assert L.sana_linattn_block_forward(A, Bp, C, Dp, None, None, S, Z, 1, 2, 64, 32, la.SANA_DT_BF16, 1e-6, None,
                                        Z - 256, n, None) == E  # runs into the key sum
    assert L.sana_linattn_state_update(A, Bp, C, Dp, 1, 2, 64, 32, la.SANA_DT_BF16, None, C, n, None) == E
    assert L.sana_linattn_state_update(A, Bp, C, Dp, 1, 2, 64, 32, la.SANA_DT_BF16, None, Bp, n, None) == E
    nb = la.backward_workspace_bytes(1, 2, 640, 64)
    dQ = 0x60000000
    assert L.sana_linattn_backward(A, Bp, C, Dp, dQ, dQ + 0x01000000, dQ + 0x02000000, None, None, None, None, None,
                                   None, 1, 2, 640, 64, 32, la.SANA_DT_BF16, 1e-6, None, dQ, nb, None) == E
    npj = la.project_state_workspace_bytes(1, 2, 1000, 64)
    assert L.sana_linattn_project_state(A, Bp, C, Dp, Dp + 8192, 1, 2, 1000, 64, 32, la.SANA_DT_BF16, None, A + 512,
                                        npj, None) == E    # inside x


def test_strided_layout_validation():
    """Layout errors come back before anything is launched; a valid packed
    layout passes the checks and is stopped by the undersized workspace."""
    L = la.lib()
    B, H, N, D = 1, 4, 256, 32
    packed = la.sana_layout(N * 3 * H * D, D, 3 * H * D)      # q/k/v of a [B, N, 3, H, D] buffer
    bnhd = la.sana_layout(N * H * D, D, H * D)                 # [B, N, H, D]
    QKV = 0x10000000
    q, k, v = QKV, QKV + H * D * 2, QKV + 2 * H * D * 2
    O = 0x20000000
    def fwd(lin, lout, o=O, nbytes=16):
        return L.sana_linattn_forward_strided(q, k, v, o, ctypes.byref(lin) if lin else None,
                                              ctypes.byref(lout) if lout else None, B, H, N, D, la.SANA_DT_BF16,
                                              1e-6, None, WS, nbytes, None)

    assert fwd(packed, bnhd) == la.SANA_ERR_WORKSPACE          # accepted, then stopped by the workspace
    assert fwd(None, None, o=0x30000000) == la.SANA_ERR_WORKSPACE  # inputs may overlap one another
    assert fwd(la.sana_layout(N * 3 * H * D, D, 16), bnhd) == la.SANA_ERR_INVALID      # token stride < D
    assert fwd(la.sana_layout(N * 3 * H * D, D, 3 * H * D + 1), bnhd) == la.SANA_ERR_INVALID   # rows not 16-B aligned
    assert fwd(la.sana_layout(N * 3 * H * D, 33, 3 * H * D), bnhd) == la.SANA_ERR_INVALID      # head stride unaligned
    assert fwd(la.sana_layout(-1, D, 3 * H * D), bnhd) == la.SANA_ERR_INVALID          # negative stride
    assert fwd(la.sana_layout(0, D, 1 << 24), bnhd) == la.SANA_ERR_INVALID             # 32 MiB row stride
    assert fwd(packed, la.sana_layout(N * H * D, 0, H * D)) == la.SANA_ERR_INVALID      # heads of o alias
    assert fwd(packed, la.sana_layout(N * H * D, D, D)) == la.SANA_ERR_INVALID          # tokens of o overlap heads
    assert fwd(packed, bnhd, o=QKV + 64) == la.SANA_ERR_INVALID                         # o inside the inputs' span


def test_forward_launches_follows_the_geometry():
    """The launch-count query: one launch when every head is one chunk of one
    split (the Sana-0.6B 1024 px layer: 144 heads of 1024 tokens; any head of
    at most 256 tokens) with dense bf16 and no full-table RoPE; two (the state
    pass and an apply that sums the partials itself) for one chunk in 2-16
    splits over 32-128 heads with dense bf16 and no full-table RoPE (the 4096
    px layer, the 480p video chunk, the 720p layer); otherwise the state pass and the apply, plus the
    finalize when a head has several partials."""
    bf16, f32 = la.SANA_DT_BF16, la.SANA_DT_F32
    assert la.forward_launches(4, 36, 1024) == 1
    assert la.forward_launches(4, 36, 1024, rope_form=2) == 1
    assert la.forward_launches(4, 36, 1024, rope_form=1) == 2
    assert la.forward_launches(4, 36, 1024, dense=False) == 2
    assert la.forward_launches(4, 36, 1024, dtype=f32) == 2
    assert la.forward_launches(1, 3, 200) == 1
    assert la.forward_launches(1, 70, 16384) == 2
    assert la.forward_launches(1, 70, 4680) == 2
    assert la.forward_launches(1, 70, 4680, rope_form=2) == 2
    assert la.forward_launches(1, 70, 4680, rope_form=1) == 3       # full-table RoPE keeps three
    assert la.forward_launches(1, 70, 4680, dense=False) == 3
    assert la.forward_launches(1, 70, 4680, dtype=f32) == 3
    assert la.forward_launches(1, 31, 4680) == 3        # too few heads to fill half the CUs
    assert la.forward_launches(1, 32, 4680) == 2
    assert la.forward_launches(1, 130, 4680) == 3       # one workgroup per head would fit an XCD
    assert la.forward_launches(1, 70, 46800, chunk=4680) == 3
    assert la.forward_launches(1, 70, 512, chunk=256) == 3
    assert la.forward_launches(1, 2, 0) == 0
    assert la.forward_launches(1, 2, 100, D=64) == 0
    assert la.forward_launches(1, 2, 100, rope_form=3) == 0
    assert bf16 != f32



def test_library_was_built_from_these_sources():
    """The library reports the hash of the kernel sources it was compiled
    from; the loader refuses one built from other sources."""
    from linear_attention_diffusion_amd import build
    assert la.binding.lib().sana_linattn_source_hash().decode() == build.source_hash()
