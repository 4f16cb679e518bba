"""The entry points only enqueue kernels on the caller's stream: no allocation,
copy, memset or synchronisation inside.  So a caller can capture a sequence of
calls in a HIP graph (here through torch.cuda.CUDAGraph) and replay it.  The
graph is replayed several times, with the program's own eager work and
synchronisations between the replays, and every replay must equal the eager
result bit for bit."""

import pytest

import linear_attention_diffusion_amd as la
from gpu_util import device, torch_mod

pytestmark = pytest.mark.gpu


def _same(torch, got, want, what):
    it = torch.int16 if got.dtype == torch.bfloat16 else torch.int32
    assert bool((got.view(it) == want.view(it)).all()), f"{what} differs from the eager result"


def test_graph_replays_equal_eager():
    """A forward with the per-axis 3D RoPE, then a block-causal chain of two
    chunks over strided views with in-place commits of the state."""
    torch = torch_mod()
    dev = device()
    g = torch.Generator().manual_seed(12)
    B, H, N, L = 1, 6, 2000, 1000
    q, k, v = ((torch.randn(B, H, N, 32, generator=g) * 0.5).to(torch.bfloat16).to(dev) for _ in range(3))
    rope = la.rope3d_axes_device(5, 20, 20, dev)                 # 2000 positions
    ws = la.make_workspace(B, H, N, dev, has_rope=True)
    wsb = la.make_workspace(B, H, L, dev)
    o_f, o_b = torch.empty_like(q), torch.empty_like(q)
    kv = torch.empty(B, H, 32, 32, device=dev)
    z = torch.empty(B, H, 32, device=dev)

    def work():
        la.sana_linattn_forward(q, k, v, o=o_f, rope=rope, workspace=ws)
        kv.zero_()                                               # a fill kernel, not a memset node
        z.zero_()
        for c in range(N // L):
            sl = slice(c * L, (c + 1) * L)
            la.sana_linattn_block_forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], o=o_b[:, :, sl], kv_in=kv,
                                          ksum_in=z, kv_out=kv, ksum_out=z, workspace=wsb)

    print("case graph: eager reference", flush=True)
    work()
    torch.cuda.synchronize()
    outs = (o_f, o_b, kv, z)
    names = ("forward O", "block-causal O", "committed S", "committed z")
    ref = [t.clone() for t in outs]

    print("case graph: capture", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    for r in range(3):
        print(f"case graph: replay {r}", flush=True)
        for t in outs:
            t.fill_(float("nan"))                                # eager work between the replays
        la.sana_linattn_forward(k, q, v, rope=rope)              # and an unrelated eager call
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip(outs, ref, names):
            _same(torch, got, want, f"replay {r}: {what}")
