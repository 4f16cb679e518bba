#!/usr/bin/env python3
"""Benchmark of SANA's ReLU linear attention on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
feature map and split-N state contraction of K, V; reduction of the partial
states (plus the carried state in block mode); apply + normalise + store of O.
For the block-causal workload one step is the whole 10-chunk loop, committing
the state after every chunk.

Default workload: the Sana-1.6B layer at 4096 px (B=1, H=70, N=16384, D=32,
bf16), the configuration the headline metric is quoted on.

Inputs are resident in HBM before timing starts.  Several input/output sets
(at least 1.5 GiB in total) are cycled so that no step finds its inputs in the
256 MB Infinity Cache left there by the step before.

Prints ONE JSON line.  `roofline` describes the dominant kernel, the apply
pass (apply_bf16): after the main timed region it is launched on its own,
through sana_linattn_apply on the state the forward computes, in the same
launch configuration, and timed with HIP events on the launch stream.  When
the library runs each call as one kernel (every head one chunk of one split:
sana_linattn_forward_launches returns 1), the dominant kernel is that one,
forward_whole_bf16, and `roofline` takes the call's own bytes and time; the
apply-alone figures are then in `apply_alone`.
`cpu_baseline` times the float64 oracle on the host cores, in a child process
whose BLAS/OpenMP thread counts are set, before NumPy loads, to the cores this
process may run on.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import WORKLOADS, generate  # noqa: E402

METRIC = "linear-attn tokens·heads/s + achieved HBM GB/s (% peak), Sana-1.6B 4096px layer"
UNIT = "tokens·heads/s"
HBM_PEAK_GBPS = 8000.0
KERNEL_DIR = "linear_attention_diffusion_amd/csrc"


def kernel_source_hash():
    """sha256[:16] over every kernel source (csrc/*.h and *.hip, by name)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_DIR)
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes the method must move: Q, K, V read once and O written once per
    token-head; in block mode also the fp32 state read and written per chunk."""
    b = w.token_heads * w.bytes_per_token_head()
    if w.mode == "block":
        b += w.n_chunks * w.B * w.H * 2 * (32 * 32 + 32) * 4
    return b


def stored_traffic(name, kernel=None):
    """HBM bytes per launch of the dominant kernel (of the forward, or of the
    backward for names "backward_<workload>"), from committed rocprofv3
    counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
    reads for a copy kernel of known size), if they were taken on the current
    kernel sources (and, when `kernel` is given, for that kernel); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    if kernel is not None and rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def make_rope(la, w, dev, form):
    """The workload's 3D RoPE on the device (None without RoPE)."""
    if w.mode != "rope":
        return None
    return la.rope3d_axes_device(*w.grid, dev) if form == "axes" else la.rope3d_device(*w.grid, dev)


def cpu_model():
    """The host CPU's model string, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, budget_s):
    """Time the float64 oracle on the host: a child process (this script with
    --cpu-worker) runs it with OMP/OpenBLAS/MKL thread counts set, before NumPy
    is imported, to the cores this process may use.  Input generation is not
    timed; the result is the median run, over at least 3 runs and about
    `budget_s` seconds (one run if a run takes more than 10 s)."""
    cores = len(os.sched_getaffinity(0))
    env = dict(os.environ, OMP_NUM_THREADS=str(cores), OPENBLAS_NUM_THREADS=str(cores), MKL_NUM_THREADS=str(cores))
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-worker",
                          json.dumps(dict(spec, budget_s=budget_s))],
                         env=env, capture_output=True, text=True, timeout=30 * budget_s + 600)
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline worker failed ({res.returncode}):\n{res.stderr[-2000:]}")
    out = json.loads(res.stdout.strip().splitlines()[-1])
    out.update(cores=out.pop("threads"), cpu=cpu_model(), affinity_cores=cores)
    return out


def cpu_worker(spec):
    """Child process of cpu_baseline: times the oracle on one workload and prints
    one JSON line."""
    import numpy as np

    import oracle
    from workloads import PROJECTIONS, generate_projection, reduced
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: the thread count the environment asks for
        threads = int(os.environ.get("OPENBLAS_NUM_THREADS", "1"))
    if spec["kind"] == "attention":
        w = WORKLOADS[spec["workload"]]
        f = generate(w).f64
        angles = oracle.rope3d_angles(*w.grid) if w.mode == "rope" else None

        def run():
            if w.mode == "block":
                oracle.block_causal(f["q"], f["k"], f["v"], w.chunk, w.eps)
            else:
                oracle.linattn(f["q"], f["k"], f["v"], w.eps, angles=angles)
        units = w.token_heads
        what = f"the whole workload ({w.B * w.H} heads x {w.N} tokens)"
    else:
        p = reduced(PROJECTIONS["sana16b_4096px_kv_proj"], name=spec["name"], N=spec["N"])
        angles = oracle.rope3d_angles(*spec["grid"]) if spec["grid"] else None
        query = spec["query"]
        f = generate_projection(p, names=("x", "w_q") if query else ("x", "w_k", "w_v")).f64
        heads = 2
        counter = {"run": 0}
        if query:
            wq = f["w_q"].reshape(p.H, 32, p.C).transpose(0, 2, 1)
            rng = np.random.default_rng(1)
            S = rng.standard_normal((p.B, heads, 32, 32)) * 50
            z = rng.random((p.B, heads, 32)) * 4000 + 10
        else:
            wk = f["w_k"].reshape(p.H, 32, p.C).transpose(0, 2, 1)
            wv = f["w_v"].reshape(p.H, 32, p.C).transpose(0, 2, 1)

        def run():
            h0 = (counter["run"] * heads) % p.H
            counter["run"] += 1
            if query:
                oracle.projected_apply(f["x"], wq[h0:h0 + heads], S, z, 1e-6, angles)
            else:
                oracle.projected_kv_state(f["x"], wk[h0:h0 + heads], wv[h0:h0 + heads], angles)
        units = p.B * heads * p.N
        what = f"{heads} heads x {p.N} tokens (C={p.C}) of this layer per run"
    times = []
    while len(times) < 3 or (sum(times) < spec["budget_s"] and len(times) < 2000):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        if len(times) == 1 and times[0] > 10.0:
            break
    med = statistics.median(times)
    print(json.dumps({"value": units / med, "unit": UNIT, "threads": threads, "kind": "oracle",
                      "runs": len(times), "median_run_s": med,
                      "sample": f"float64 oracle over {what}; median of {len(times)} runs "
                                f"({sum(times):.1f} s of CPU work), input generation not timed"}), flush=True)


def step_percentiles(step, steps, first, stream):
    """p10/p50/p90 of single steps, each between its own pair of events, in a
    separate loop after the timed region (per-step events add their own marker
    packets, so the headline time comes from the single event pair)."""
    import torch
    times = []
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(first + i)
        b.record(stream)
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)

    def pct(p):
        return ms[min(len(ms) - 1, int(round(p / 100.0 * (len(ms) - 1))))]

    return {"p10": pct(10), "p50": pct(50), "p90": pct(90)}


def copy_probe(steps, warmup, nbytes=2 ** 30):
    """HBM ceilings of this part, each on buffers far larger than the 256 MB
    MALL: a plain 1 GiB device copy (torch copy_: reads and writes `nbytes`;
    also the kernel whose FETCH_SIZE / WRITE_SIZE counters scale the traffic
    figures), a pure 1 GiB write (torch fill_), a 1 GiB read reduced to one
    number (torch sum), and this library's read-only state pass over a large
    K, V (70 heads x 65536 tokens, 587 MB, sana_linattn_state_update).  Also
    the floor of a dependent launch: 500 back-to-back fills of a 1 KB buffer
    (one workgroup) and of a 2 MB buffer (torch's fill kernel, 512 workgroups of
    256), each waiting for the one before, as the passes of one call do,
    replayed from a HIP graph so that the host's per-call cost does not enter."""
    import torch

    import linear_attention_diffusion_amd as la
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def timed(fn, n=steps):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms_copy = timed(lambda: dst.copy_(src))
    ms_fill = timed(lambda: dst.fill_(2.0))
    ms_sum = timed(lambda: src.sum())
    def graph_launch_us(t, n=500):
        # n dependent fills captured once and replayed, so that the host's
        # per-call cost does not enter; fill_ with a non-zero value is a kernel
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            t.fill_(3.0)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(n):
                    t.fill_(3.0)
        return timed(graph.replay, n=4) * 1e3 / n

    launch_us_1 = graph_launch_us(torch.empty(256, dtype=torch.float32, device=dev))
    launch_us_512 = graph_launch_us(torch.empty(512 * 1024, dtype=torch.float32, device=dev))
    H, N = 70, 65536
    g = torch.Generator(device="cpu").manual_seed(1)
    kv = [tuple((torch.randn(1, H, N, 32, generator=g) * 0.5).to(torch.bfloat16).to(dev) for _ in range(2))
          for _ in range(2)]
    S = torch.zeros(1, H, 32, 32, device=dev)
    z = torch.zeros(1, H, 32, device=dev)
    ws = la.make_workspace(1, H, N, dev)
    it = [0]

    def state():
        k, v = kv[it[0] % 2]
        it[0] += 1
        la.sana_linattn_state_update(k, v, S, z, workspace=ws)
    ms_state = timed(state)
    kv_bytes = 2 * H * N * 32 * 2

    def gbps(b, ms):
        return b / (ms / 1e3) / 1e9
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "ms_per_copy": ms_copy, "gbps_read_plus_write": gbps(2 * nbytes, ms_copy),
                      "fill_gbps_write": gbps(nbytes, ms_fill), "sum_gbps_read": gbps(nbytes, ms_sum),
                      "state_pass_gbps_read": gbps(kv_bytes, ms_state), "state_pass_bytes": kv_bytes,
                      "state_pass_ms": ms_state, "dependent_launch_us_1kb_fill": launch_us_1,
                      "dependent_launch_us_2mb_fill": launch_us_512}), flush=True)


def conv_bench(args, dev, stream):
    """Time the temporal convolution of block inference with its cache
    (sana_linattn_temporal_conv3, reading the previous chunk's last frame and
    committing the new one in place) on one 480p chunk: 3 latent frames of
    30 x 52 tokens, at the Mix-FFN's hidden width (2.5 x 2240 = 5600 channels
    for Sana-1.6B), bf16.  Algorithmic bytes: x read and y written once, the
    cache read and written once."""
    import torch

    import linear_attention_diffusion_amd as la

    B, F, S, C = 1, 3, 30 * 52, 5600
    g = torch.Generator(device="cpu").manual_seed(7)
    x0 = (torch.randn(B, F, S, C, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    w = (torch.randn(C, 3, generator=g) * 0.3).to(dev)
    b = (torch.randn(C, generator=g) * 0.1).to(dev)
    set_bytes = 2 * x0.numel() * 2
    n_sets = max(2, min(64, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    sets = [(x0.clone(), torch.empty_like(x0), torch.zeros(B, S, C, dtype=torch.bfloat16, device=dev))
            for _ in range(n_sets)]
    L = la.lib()
    P = ctypes.c_void_p
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    calls = [(P(x.data_ptr()), P(y.data_ptr()), P(w.data_ptr()), P(b.data_ptr()), P(c.data_ptr()), P(c.data_ptr()),
              B, F, S, C, la.SANA_DT_BF16, st_ptr) for x, y, c in sets]

    def step(i):
        rc = L.sana_linattn_temporal_conv3(*calls[i % n_sets])
        if rc:
            raise la.SanaError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    alg = 2 * B * F * S * C * 2 + 2 * B * S * C * 2
    achieved = alg / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "temporal conv (block-inference conv cache) GB/s",
        "value": achieved, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)x0.5 bf16 activations, random filters",
        "config": {"workload": "480p chunk at Mix-FFN width", "pass": "conv", "B": B, "frames": F, "spatial": S,
                   "channels": C, "input_sets_cycled": n_sets},
        "roofline": {"bound": "hbm", "kernel": "temporal_conv3", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": stored_traffic("conv_480p_chunk"),
                     "algorithmic_bytes_per_launch": alg, "avg_launch_ms": ms},
        "kernel_source_hash": kernel_source_hash(),
    }), flush=True)


def block_infer_bench(args, dev, stream):
    """Time one chunk of block linear diffusion inference ("SANA-Video" paper
    notes, section 4): T denoising passes that read the cache, then the commit
    pass, through one synthetic layer (QKV projection + attention through the
    cache, output projection + residual, temporal conv through its cache) at
    the 480p chunk: 3 latent frames of 30 x 52 tokens, 70 heads of 32, the
    Sana-1.6B width C = 2240, bf16.  T = 4 (the pages give no step count).
    Timed with the fused projection kernels (project_state + project_apply)
    and, beside it, the unfused path (one torch GEMM for Q, K, V, then
    block_forward), alternating, the second round reported.  Chunk inputs are
    cycled; the layer's weights stay the same, as in inference."""
    import torch

    from linear_attention_diffusion_amd import block_infer

    B, H, C, F, S, T = 1, 70, 2240, 3, 30 * 52, 4
    N = F * S
    layers = {fused: [block_infer.SyntheticLayer(C, H, dev, seed=1, fused=fused)] for fused in (True, False)}
    g = torch.Generator(device="cpu").manual_seed(5)
    n_sets = 8
    noise = [(torch.randn(B, N, C, generator=g)).to(torch.bfloat16).to(dev) for _ in range(n_sets)]
    step_noise = [[(torch.randn(B, N, C, generator=g)).to(torch.bfloat16).to(dev) for _ in range(T - 1)]
                  for _ in range(n_sets)]
    timesteps = [(j + 1) / T for j in range(T)]

    def chunk(fused, i, caches):
        x = noise[i % n_sets]
        for j in range(T, 0, -1):
            y0 = block_infer.run_model(layers[fused], caches, x, F, commit=False)
            if j == 1:
                block_infer.run_model(layers[fused], caches, y0, F, commit=True)
            else:
                t = timesteps[j - 2]
                x = (1.0 - t) * y0 + t * step_noise[i % n_sets][T - j]

    def timed(fused):
        caches = [block_infer.BlockCache(B, H, S, C, torch.bfloat16, dev)]
        for i in range(args.warmup):
            chunk(fused, i, caches)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            chunk(fused, args.warmup + i, caches)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = {}
    for _ in range(2):
        for fused in (True, False):
            ms[fused] = timed(fused)
    print(json.dumps({
        "metric": "block-inference chunk (T denoising passes + commit, 1 synthetic layer) latent tokens/s",
        "value": N / (ms[True] / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms[True], "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 chunk noise, N(0,1/C) bf16 weights, random conv filters",
        "config": {"workload": "480p chunk, one layer", "pass": "block_infer", "B": B, "H": H, "C": C, "frames": F,
                   "spatial": S, "T": T, "input_sets_cycled": n_sets},
        "per_chunk_ms": {"fused_projections": ms[True], "unfused_gemm_then_block_forward": ms[False]},
        "fused_speedup": ms[False] / ms[True],
        "kernel_source_hash": kernel_source_hash(),
    }), flush=True)


def project_bench(args, dev, stream):
    """Time sana_linattn_project_state, the key/value projection fused with the
    state update, on the Sana-1.6B 4096 px layer (x [1, 16384, 2240] bf16,
    W_k and W_v [2240, 2240] bf16, 70 heads), one call per step, cycling input
    sets (x and both weights) past the Infinity Cache.  Beside it, the same
    work as two passes on the same stream: a bf16 library GEMM (torch.matmul,
    hipBLASLt) writing K and V as [N, 2 x 2240], then sana_linattn_state_update
    reading them.  The fused call and the GEMM are timed in two alternating
    rounds and the second is reported.  With --workload video720p_rope3d: the
    same width over the SANA-Video 720p layer's 18480 tokens, keys rotated by
    its 3D RoPE (--rope-form), in both paths.  Algorithmic flops: 2 N C (2 H D) for the projection plus
    2 N H D (D + 1) for the state."""
    import numpy as np
    import torch

    import linear_attention_diffusion_amd as la
    from workloads import PROJECTIONS, generate_projection

    p = PROJECTIONS["sana16b_4096px_kv_proj"]
    w = WORKLOADS[args.workload]
    rope = None
    if w.mode == "rope":
        # the video layer's keys: the same width, its tokens and 3D RoPE
        from workloads import reduced
        p = reduced(p, name=f"{w.name}_kv_proj", N=w.N)
        rope = make_rope(la, w, dev, args.rope_form)
    elif w.name != "sana16b_4096px":
        raise SystemExit("--pass project runs on the sana16b_4096px layer or, with RoPE, video720p_rope3d")
    rope_ref = None if rope is None else ctypes.byref(rope.struct())
    x = generate_projection(p, with_f64=False)

    def td(raw):
        return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)

    x0, wk0, wv0 = td(x.raw["x"]), td(x.raw["w_k"]), td(x.raw["w_v"])
    set_bytes = (x0.numel() + wk0.numel() + wv0.numel()) * 2
    n_sets = max(2, min(32, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    sets = [(x0.clone(), wk0.clone(), wv0.clone()) for _ in range(n_sets)]
    kv = torch.zeros(p.B, p.H, 32, 32, device=dev)
    z = torch.zeros(p.B, p.H, 32, device=dev)
    nb = la.project_state_workspace_bytes(p.B, p.H, p.N, p.C)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    L = la.lib()
    P = ctypes.c_void_p
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    calls = [(P(a.data_ptr()), P(b.data_ptr()), P(c.data_ptr()), P(kv.data_ptr()), P(z.data_ptr()), p.B, p.H, p.N,
              p.C, 32, la.SANA_DT_BF16, rope_ref, P(ws.data_ptr()), nb, st_ptr) for a, b, c in sets]

    def step(i):
        rc = L.sana_linattn_project_state(*calls[i % n_sets])
        if rc:
            raise la.SanaError(rc)

    def timed(fn, first):
        for i in range(args.warmup):
            fn(first + i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(first + args.warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # the two-pass path on the same sets
    wkv = [torch.cat([b, c], 0) for _, b, c in sets]
    out = torch.empty(p.B * p.N, 2 * p.H * 32, dtype=torch.bfloat16, device=dev)
    k = torch.empty(p.B, p.H, p.N, 32, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    ws2 = la.make_workspace(p.B, p.H, p.N, dev, has_rope=rope is not None)

    def gemm(i):
        torch.matmul(sets[i % n_sets][0].view(p.B * p.N, p.C), wkv[i % n_sets].t(), out=out)

    def state(i):
        la.sana_linattn_state_update(k, v, kv, z, rope=rope, workspace=ws2, stream=stream)

    # Both paths are timed twice, alternating, and the second round is
    # reported: on this part a matrix-core kernel's first few hundred
    # microseconds of sustained load run slower (clock ramp), which would
    # otherwise fall on whichever path is timed first.
    for _ in range(2):
        ms = timed(step, 0)
        ms_gemm = timed(gemm, 0)
    k.copy_(out[:, :p.H * 32].view(p.B, p.N, p.H, 32).permute(0, 2, 1, 3))
    v.copy_(out[:, p.H * 32:].view(p.B, p.N, p.H, 32).permute(0, 2, 1, 3))
    ms_state = timed(state, 0)
    pct = step_percentiles(step, min(args.steps, 20), 0, stream)

    flops = 2.0 * p.B * p.N * p.C * (2 * p.H * 32) + 2.0 * p.B * p.N * p.H * 32 * 33
    rope_name = None if rope is None else ("3D RoPE, per-axis tables" if rope.grid else "3D RoPE, full tables")
    tflops = flops / (ms / 1e3) / 1e12
    th = p.B * p.N * p.H
    rec = {
        "metric": "fused K/V projection + linear-attn state, tokens·heads/s (" +
                  ("Sana-1.6B 4096px layer)" if rope is None else "SANA-Video 720p layer, 3D RoPE)"),
        "value": th / (ms / 1e3), "unit": "tokens·heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "step_ms_percentiles": pct, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 activations, N(0,1/C) bf16 weights",
        "config": {"workload": p.name, "pass": "project_state", "B": p.B, "N": p.N, "C": p.C, "H": p.H, "D": p.D,
                   "rope": rope_name, "input_sets_cycled": n_sets},
        "roofline": {"bound": "mfma", "kernel": "project_state_bf16", "achieved": tflops, "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": tflops / 2500.0, "traffic": stored_traffic("project_4096px" if rope is None else "project_720p_rope3d"),
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": ms},
        "two_pass": {"gemm_ms": ms_gemm, "state_update_ms": ms_state, "total_ms": ms_gemm + ms_state,
                     "gemm_tflops": 2.0 * p.B * p.N * p.C * (2 * p.H * 32) / (ms_gemm / 1e3) / 1e12,
                     "fused_speedup": (ms_gemm + ms_state) / ms},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline({"kind": "project", "query": False, "name": p.name, "N": p.N,
                                            "grid": list(w.grid) if rope is not None else None}, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def project_apply_bench(args, dev, stream):
    """Time sana_linattn_project_apply, the query projection fused with the
    apply step, on the Sana-1.6B 4096 px layer (x [1, 16384, 2240] bf16, W_q
    [2240, 2240] bf16, 70 heads, a given fp32 state), one call per step,
    cycling input sets (x and W_q) past the Infinity Cache; with --workload
    video720p_rope3d the 720p layer's 18480 tokens with its 3D RoPE.  Beside
    it, the unfused path on the same stream: a bf16 library GEMM (torch.matmul,
    hipBLASLt) writing Q as [N, 2240], then sana_linattn_apply reading Q
    [B, H, N, D] (the regrouping copy between the two is not counted).  Timed
    in two alternating rounds, the second reported.  Algorithmic flops:
    2 N C H D for the projection plus 2 N H D (D + 1) for the apply."""
    import numpy as np
    import torch

    import linear_attention_diffusion_amd as la
    from workloads import PROJECTIONS, generate_projection, reduced

    p = reduced(PROJECTIONS["sana16b_4096px_kv_proj"], name="sana16b_4096px_q_proj")
    w = WORKLOADS[args.workload]
    rope = None
    if w.mode == "rope":
        p = reduced(p, name=f"{w.name}_q_proj", N=w.N)
        rope = make_rope(la, w, dev, args.rope_form)
    elif w.name != "sana16b_4096px":
        raise SystemExit("--pass project_apply runs on the sana16b_4096px layer or, with RoPE, video720p_rope3d")
    rope_ref = None if rope is None else ctypes.byref(rope.struct())
    x = generate_projection(p, with_f64=False, names=("x", "w_q"))

    def td(raw):
        return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)

    x0, wq0 = td(x.raw["x"]), td(x.raw["w_q"])
    set_bytes = (x0.numel() + wq0.numel()) * 2 + p.B * p.N * p.H * 32 * 2
    n_sets = max(2, min(32, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    sets = [(x0.clone(), wq0.clone(), torch.empty(p.B, p.H, p.N, 32, dtype=torch.bfloat16, device=dev))
            for _ in range(n_sets)]
    g = torch.Generator(device="cpu").manual_seed(1)
    kv = (torch.randn(p.B, p.H, 32, 32, generator=g) * 50).to(dev)
    z = (torch.rand(p.B, p.H, 32, generator=g) * 4000 + 10).to(dev)
    L = la.lib()
    P = ctypes.c_void_p
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    calls = [(P(a.data_ptr()), P(b.data_ptr()), P(o.data_ptr()), None, P(kv.data_ptr()), P(z.data_ptr()), p.B, p.H,
              p.N, p.C, 32, la.SANA_DT_BF16, 1e-6, rope_ref, st_ptr) for a, b, o in sets]

    def step(i):
        rc = L.sana_linattn_project_apply(*calls[i % n_sets])
        if rc:
            raise la.SanaError(rc)

    def timed(fn, first):
        for i in range(args.warmup):
            fn(first + i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(first + args.warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    out = torch.empty(p.B * p.N, p.H * 32, dtype=torch.bfloat16, device=dev)
    q = torch.empty(p.B, p.H, p.N, 32, dtype=torch.bfloat16, device=dev)

    def gemm(i):
        torch.matmul(sets[i % n_sets][0].view(p.B * p.N, p.C), sets[i % n_sets][1].t(), out=out)

    def apply(i):
        la.sana_linattn_apply(q, kv, z, o=sets[i % n_sets][2], rope=rope, stream=stream)

    # alternating rounds, the second reported (matrix-core clock ramp)
    for _ in range(2):
        ms = timed(step, 0)
        ms_gemm = timed(gemm, 0)
    q.copy_(out.view(p.B, p.N, p.H, 32).permute(0, 2, 1, 3))
    ms_apply = timed(apply, 0)
    pct = step_percentiles(step, min(args.steps, 20), 0, stream)

    flops = 2.0 * p.B * p.N * p.C * (p.H * 32) + 2.0 * p.B * p.N * p.H * 32 * 33
    rope_name = None if rope is None else ("3D RoPE, per-axis tables" if rope.grid else "3D RoPE, full tables")
    tflops = flops / (ms / 1e3) / 1e12
    th = p.B * p.N * p.H
    rec = {
        "metric": "fused Q projection + linear-attn apply, tokens·heads/s (" +
                  ("Sana-1.6B 4096px layer)" if rope is None else "SANA-Video 720p layer, 3D RoPE)"),
        "value": th / (ms / 1e3), "unit": "tokens·heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "step_ms_percentiles": pct, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 activations, N(0,1/C) bf16 weights, random fp32 state",
        "config": {"workload": p.name, "pass": "project_apply", "B": p.B, "N": p.N, "C": p.C, "H": p.H, "D": p.D,
                   "rope": rope_name, "input_sets_cycled": n_sets},
        "roofline": {"bound": "mfma", "kernel": "project_apply_bf16", "achieved": tflops, "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": tflops / 2500.0,
                     "traffic": stored_traffic("project_apply_4096px" if rope is None else "project_apply_720p_rope3d"),
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": ms},
        "two_pass": {"gemm_ms": ms_gemm, "apply_ms": ms_apply, "total_ms": ms_gemm + ms_apply,
                     "gemm_tflops": 2.0 * p.B * p.N * p.C * (p.H * 32) / (ms_gemm / 1e3) / 1e12,
                     "fused_speedup": (ms_gemm + ms_apply) / ms},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline({"kind": "project", "query": True, "name": p.name, "N": p.N,
                                            "grid": list(w.grid) if rope is not None else None}, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def backward_bench(w, args, dev, stream):
    """Time sana_linattn_backward: one call per step (dQ, dK, dV from dO; the
    chunk states are recomputed from K, V), the block-causal workload as one
    whole-sequence call.  Algorithmic bytes per token-head: Q, K, V, dO read by
    the passes that need them (K, V twice: state recompute and key pass; Q, dO
    once) and dQ, dK, dV written once: 9 tensors x 64 B in bf16."""
    import numpy as np
    import torch

    import linear_attention_diffusion_amd as la

    x = generate(w, with_f64=False, names=("q", "k", "v", "dout"))

    def to_dev(raw):
        if w.dtype == "bf16":
            return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(raw).to(dev)

    base = {n: to_dev(x.raw[n]) for n in ("q", "k", "v", "dout")}
    set_bytes = 7 * base["q"].numel() * base["q"].element_size()
    n_sets = max(2, min(16, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    packed = args.layout == "packed"
    if packed and w.mode == "block":
        raise SystemExit("--layout packed covers the non-causal and RoPE workloads")
    sets = []
    for i in range(n_sets):
        if packed:
            # q, k, v, dO as [B, H, N, D] views of one [B, N, 4, H, D] buffer;
            # dQ, dK, dV as views of [B, N, H, D] buffers
            buf = torch.empty(w.B, w.N, 4, w.H, w.D, dtype=base["q"].dtype, device=dev)
            s = {}
            for j, n in enumerate(("q", "k", "v", "dout")):
                buf[:, :, j] = base[n].permute(0, 2, 1, 3)
                s[n] = buf[:, :, j].permute(0, 2, 1, 3)
            for n in ("dq", "dk", "dv"):
                s[n] = torch.empty(w.B, w.N, w.H, w.D, dtype=base["q"].dtype, device=dev).permute(0, 2, 1, 3)
        else:
            s = {n: (t if i == 0 else t.clone()) for n, t in base.items()}
            for n in ("dq", "dk", "dv"):
                s[n] = torch.empty_like(base["q"])
        sets.append(s)
    chunk = w.chunk if w.mode == "block" else w.N
    rope = make_rope(la, w, dev, args.rope_form)
    dt = la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32
    nb = la.backward_workspace_bytes(w.B, w.H, w.N, chunk, dtype=dt, has_rope=rope is not None)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    L = la.lib()
    P = ctypes.c_void_p
    rope_ref = None if rope is None else ctypes.byref(rope.struct())
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    if packed:
        lin = la.sana_layout(*sets[0]["q"].stride()[:3])
        lout = la.sana_layout(*sets[0]["dq"].stride()[:3])
        calls = [(P(s["q"].data_ptr()), P(s["k"].data_ptr()), P(s["v"].data_ptr()), P(s["dout"].data_ptr()),
                  P(s["dq"].data_ptr()), P(s["dk"].data_ptr()), P(s["dv"].data_ptr()), ctypes.byref(lin),
                  ctypes.byref(lout), None, None, None, None, None, None, w.B, w.H, w.N, chunk, w.D, dt, w.eps,
                  rope_ref, P(ws.data_ptr()), ws.numel(), st_ptr) for s in sets]
        entry = L.sana_linattn_backward_strided
    else:
        calls = [(P(s["q"].data_ptr()), P(s["k"].data_ptr()), P(s["v"].data_ptr()), P(s["dout"].data_ptr()),
                  P(s["dq"].data_ptr()), P(s["dk"].data_ptr()), P(s["dv"].data_ptr()), None, None, None, None, None,
                  None, w.B, w.H, w.N, chunk, w.D, dt, w.eps, rope_ref, P(ws.data_ptr()), ws.numel(), st_ptr)
                 for s in sets]
        entry = L.sana_linattn_backward

    def step(i):
        rc = entry(*calls[i % n_sets])
        if rc:
            raise la.SanaError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = e0.elapsed_time(e1) / args.steps
    step_pct = step_percentiles(step, args.steps, args.warmup + args.steps, stream)
    elem = 2 if w.dtype == "bf16" else 4
    alg_bytes = w.token_heads * 9 * w.D * elem

    # roofline of the dominant kernel: the key pass (dK, dV from a state
    # gradient), launched alone through sana_linattn_state_update_backward on
    # the whole sequence, timed with one event pair on the launch stream
    g = torch.Generator(device="cpu").manual_seed(5)
    dkv = torch.randn(w.B, w.H, 32, 32, generator=g).to(dev)
    dksum = torch.randn(w.B, w.H, 32, generator=g).to(dev)
    # (contiguous K, V, dK, dV: the key pass on its own takes no layout views)
    key_sets = sets if not packed else [{"k": base["k"], "v": base["v"], "dk": torch.empty_like(base["k"]),
                                         "dv": torch.empty_like(base["v"])}]
    key_calls = [(P(s["k"].data_ptr()), P(s["v"].data_ptr()), P(dkv.data_ptr()), P(dksum.data_ptr()),
                  P(s["dk"].data_ptr()), P(s["dv"].data_ptr()), w.B, w.H, w.N, w.D, dt, rope_ref, st_ptr)
                 for s in key_sets]
    for i in range(args.warmup):
        L.sana_linattn_state_update_backward(*key_calls[i % len(key_calls)])
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        rc = L.sana_linattn_state_update_backward(*key_calls[i % len(key_calls)])
        if rc:
            raise la.SanaError(rc)
    k1.record(stream)
    torch.cuda.synchronize()
    key_ms = k0.elapsed_time(k1) / args.steps
    key_bytes = w.token_heads * 4 * w.D * elem + w.B * w.H * (32 * 32 + 32) * 4
    train = None if packed else train_step_timing(w, args, sets, n_sets, chunk, rope_ref, dt, nb, dev, stream)

    # fp32 multiply-adds per token-head of the backward: the forward state
    # recompute (S, z: 32*32 + 32), the query pass (num, den, S dnum, dS, dz:
    # 3*32*32 + 2*32) and the key pass (G V, G^T phi~(K): 2*32*32), 2 flop each
    flops = w.token_heads * 2 * (6 * 32 * 32 + 3 * 32)
    rec = {
        "metric": "linear-attn backward tokens·heads/s (dQ, dK, dV)",
        "value": w.token_heads * args.steps / (ms * args.steps / 1e3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1)x0.5 bf16 tensors at the workload's latent shape (dO drawn after Q, K, V)",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "mode": w.mode, "chunk": chunk, "grid": w.grid, "input_sets_cycled": n_sets,
                   "layout": args.layout, "rope_form": args.rope_form if w.mode == "rope" else None},
        "roofline": {
            "bound": "hbm",
            "kernel": "bwd_key_bf16" if w.dtype == "bf16" else "bwd_key_vec",
            "achieved": key_bytes / (key_ms / 1e3) / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": key_bytes / (key_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": stored_traffic("backward_" + w.name),
            "algorithmic_bytes_per_launch": key_bytes,
            "avg_launch_ms": key_ms,
            "tokens_per_launch": w.token_heads,
        },
        "call": {"entry_point": ("sana_linattn_backward_strided (packed [B,N,4,H,D] in, [B,N,H,D] out)" if packed
                                 else "sana_linattn_backward"),
                 "kernels": "state pass + finalize + query pass + reverse finalize + key pass",
                 "avg_ms": ms, "algorithmic_bytes": alg_bytes,
                 "achieved_gbps": alg_bytes / (ms / 1e3) / 1e9,
                 "frac_of_hbm_peak": alg_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                 "flops": flops, "achieved_tflops": flops / (ms / 1e3) / 1e12},
        "train_step": train,
        "step_ms_percentiles": step_pct,
        "wall_s_timed_region": wall,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(rec), flush=True)


def train_step_timing(w, args, sets, n_sets, chunk, rope_ref, dt, nb, dev, stream):
    """A training step's attention: the forward (block_causal for the chunked
    workload, else forward), then its backward either recomputing the chunk
    states (sana_linattn_backward) or reading the ones the forward left in its
    workspace (sana_linattn_backward_saved).  Each input set has its own
    workspace and output; each variant is timed over the same steps."""
    import torch

    import linear_attention_diffusion_amd as la

    L = la.lib()
    P = ctypes.c_void_p
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    for s in sets:
        s["o"] = torch.empty_like(s["q"])
        s["ws"] = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

    def forward(s):
        ptrs = [P(s[n].data_ptr()) for n in ("q", "k", "v", "o")]
        ws = P(s["ws"].data_ptr())
        if w.mode == "block":
            return L.sana_linattn_block_causal(*ptrs, None, None, None, None, w.B, w.H, w.N, chunk, w.D, dt, w.eps,
                                               rope_ref, ws, s["ws"].numel(), st_ptr)
        return L.sana_linattn_forward(*ptrs, w.B, w.H, w.N, w.D, dt, w.eps, rope_ref, ws, s["ws"].numel(), st_ptr)

    def grads(s):
        return [P(s[n].data_ptr()) for n in ("q", "k", "v", "dout", "dq", "dk", "dv")]

    def recompute(s):
        return L.sana_linattn_backward(*grads(s), None, None, None, None, None, None, w.B, w.H, w.N, chunk, w.D,
                                       dt, w.eps, rope_ref, P(s["ws"].data_ptr()), s["ws"].numel(), st_ptr)

    def saved(s):
        return L.sana_linattn_backward_saved(*grads(s), None, None, None, None, None, None, w.B, w.H, w.N, chunk,
                                             w.D, dt, w.eps, rope_ref, P(s["ws"].data_ptr()), s["ws"].numel(),
                                             st_ptr)

    def timed(calls):
        def one(i):
            for c in calls:
                rc = c(sets[i % n_sets])
                if rc:
                    raise la.SanaError(rc)
        for i in range(args.warmup):
            one(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            one(args.warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    fwd_ms = timed([forward])
    rec_ms = timed([forward, recompute])
    sav_ms = timed([forward, saved])
    return {"forward_ms": fwd_ms, "forward_plus_backward_ms": rec_ms, "forward_plus_backward_saved_ms": sav_ms,
            "backward_saved_ms": sav_ms - fwd_ms,
            "entry_points": "forward/block_causal, then sana_linattn_backward or sana_linattn_backward_saved"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sana16b_4096px", choices=list(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-mode", choices=["chunks", "sequence"], default="chunks",
                    help="block-causal workload: one block_forward call per chunk (inference, the default) or "
                         "one block_causal call over the whole sequence (all chunks known at once)")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "conv", "project", "project_apply",
                                                     "block_infer"], default="forward",
                    help="forward (the default; the headline metric) or backward: one sana_linattn_backward "
                         "call per step (dQ, dK, dV; whole sequence in block-causal chunks for that workload); "
                         "conv: the block-inference temporal conv; project: the key/value projection fused "
                         "with the state update (Sana-1.6B 4096 px layer, or video720p_rope3d with its RoPE); "
                         "project_apply: the query projection fused with the apply step (same layers); "
                         "block_infer: one chunk of block inference (denoising passes + commit) through a "
                         "synthetic layer, fused projections against the unfused path")
    ap.add_argument("--layout", choices=["bhnd", "packed"], default="bhnd",
                    help="bhnd = contiguous [B, H, N, D] (the default); packed = Q, K, V (and dO for the backward) "
                         "read as strided views of one [B, N, 3 (4), H, D] projection-style buffer and O (dQ, dK, "
                         "dV) written to [B, N, H, D] (the *_strided entry points; non-causal and RoPE workloads)")
    ap.add_argument("--rope-form", choices=["table", "axes"], default="axes",
                    help="RoPE workload: axes = the 3D RoPE's per-axis tables, staged in LDS by each workgroup (the "
                         "default); table = full [pos][16] cos/sin tables, streamed per head")
    ap.add_argument("--cpu-worker", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (HBM reference and counter scale)")
    args = ap.parse_args()
    if args.cpu_worker is not None:
        cpu_worker(json.loads(args.cpu_worker))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(every head is independent; see the sharding notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_attention_diffusion_amd as la

    if args.copy_probe:
        copy_probe(args.steps, args.warmup)
        return

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    la.lib()
    stream = torch.cuda.current_stream(dev)
    if args.which == "backward":
        backward_bench(w, args, dev, stream)
        return
    if args.which == "conv":
        conv_bench(args, dev, stream)
        return
    if args.which == "project":
        project_bench(args, dev, stream)
        return
    if args.which == "project_apply":
        project_apply_bench(args, dev, stream)
        return
    if args.which == "block_infer":
        block_infer_bench(args, dev, stream)
        return

    x = generate(w, with_f64=False)

    def to_dev(raw):
        if w.dtype == "bf16":
            return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(raw).to(dev)

    q0, k0, v0 = (to_dev(x.raw[n]) for n in ("q", "k", "v"))
    set_bytes = 4 * q0.numel() * q0.element_size()
    n_sets = max(2, min(16, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    packed = args.layout == "packed"
    if packed and w.mode == "block":
        raise SystemExit("--layout packed covers the non-causal and RoPE workloads")
    sets = []
    for i in range(n_sets):
        if packed:
            # one [B, N, 3, H, D] buffer holding Q, K, V; O as [B, N, H, D]
            buf = torch.empty(w.B, w.N, 3, w.H, w.D, dtype=q0.dtype, device=dev)
            for j, t in enumerate((q0, k0, v0)):
                buf[:, :, j] = t.permute(0, 2, 1, 3)
            q, k, v = (buf[:, :, j].permute(0, 2, 1, 3) for j in range(3))
            o = torch.empty(w.B, w.N, w.H, w.D, dtype=q0.dtype, device=dev).permute(0, 2, 1, 3)
            sets.append({"q": q, "k": k, "v": v, "o": o, "buf": buf})
            continue
        if i == 0:
            q, k, v = q0, k0, v0
        else:
            q, k, v = q0.clone(), k0.clone(), v0.clone()
        sets.append({"q": q, "k": k, "v": v, "o": torch.empty_like(q)})

    rope = make_rope(la, w, dev, args.rope_form)
    if w.mode == "block":
        Lc = w.chunk
        for s in sets:
            for n in ("q", "k", "v", "o"):
                t = s[n]
                s[n + "_chunks"] = [t[:, :, c:min(w.N, c + Lc)].contiguous() for c in range(0, w.N, Lc)]
            s["kv"] = torch.zeros(w.B, w.H, 32, 32, device=dev)
            s["z"] = torch.zeros(w.B, w.H, 32, device=dev)
        dtc = la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32
        if args.block_mode == "sequence":
            nb = la.block_causal_workspace_bytes(w.B, w.H, w.N, Lc, dtype=dtc)
            ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        else:
            ws = la.make_workspace(w.B, w.H, Lc, dev, dtype=dtc)
    else:
        ws = la.make_workspace(w.B, w.H, w.N, dev, dtype=la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32,
                               has_rope=rope is not None)

    # Pre-marshalled C calls: the timed loop makes no torch calls and no
    # argument checks in Python, so the host stays ahead of the GPU.
    L = la.lib()
    dt = la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32
    ws_ptr, ws_n = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    st_ptr = ctypes.c_void_p(stream.cuda_stream)
    rope_ref = None if rope is None else ctypes.byref(rope.struct())
    P = ctypes.c_void_p
    calls = []
    for s in sets:
        if w.mode == "block" and args.block_mode == "sequence":
            calls.append(("sequence", (P(s["q"].data_ptr()), P(s["k"].data_ptr()), P(s["v"].data_ptr()),
                                       P(s["o"].data_ptr()), None, None, P(s["kv"].data_ptr()), P(s["z"].data_ptr()),
                                       w.B, w.H, w.N, w.chunk, w.D, dt, w.eps, None, ws_ptr, ws_n, st_ptr)))
        elif w.mode == "block":
            seq = []
            for c, (qc, kc, vc, oc) in enumerate(zip(s["q_chunks"], s["k_chunks"], s["v_chunks"], s["o_chunks"])):
                # chunk 0 starts from the zero state (kv_in = NULL); every chunk commits in place
                kv_in = None if c == 0 else P(s["kv"].data_ptr())
                z_in = None if c == 0 else P(s["z"].data_ptr())
                seq.append((P(qc.data_ptr()), P(kc.data_ptr()), P(vc.data_ptr()), P(oc.data_ptr()), kv_in, z_in,
                            P(s["kv"].data_ptr()), P(s["z"].data_ptr()), w.B, w.H, qc.shape[2], w.D, dt, w.eps,
                            None, ws_ptr, ws_n, st_ptr))
            calls.append(("block", seq))
        elif packed:
            lin = la.sana_layout(*s["q"].stride()[:3])
            lout = la.sana_layout(*s["o"].stride()[:3])
            s["layouts"] = (lin, lout)
            calls.append(("strided", (P(s["q"].data_ptr()), P(s["k"].data_ptr()), P(s["v"].data_ptr()),
                                      P(s["o"].data_ptr()), ctypes.byref(lin), ctypes.byref(lout), w.B, w.H, w.N,
                                      w.D, dt, w.eps, rope_ref, ws_ptr, ws_n, st_ptr)))
        else:
            calls.append(("fwd", (P(s["q"].data_ptr()), P(s["k"].data_ptr()), P(s["v"].data_ptr()),
                                  P(s["o"].data_ptr()), w.B, w.H, w.N, w.D, dt, w.eps, rope_ref, ws_ptr, ws_n,
                                  st_ptr)))

    def step(i):
        kind, args = calls[i % n_sets]
        if kind == "sequence":
            rc = L.sana_linattn_block_causal(*args)
            if rc:
                raise la.SanaError(rc)
        elif kind == "strided":
            rc = L.sana_linattn_forward_strided(*args)
            if rc:
                raise la.SanaError(rc)
        elif kind == "block":
            for a in args:
                rc = L.sana_linattn_block_forward(*a)
                if rc:
                    raise la.SanaError(rc)
        else:
            rc = L.sana_linattn_forward(*args)
            if rc:
                raise la.SanaError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps between one pair of events on the launch
    # stream (per-step events would add marker packets to the measured time)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    total_ms = e_start.elapsed_time(e_end)

    ms_per_step = total_ms / args.steps
    value = w.token_heads * args.steps / (total_ms / 1e3)
    step_pct = step_percentiles(step, args.steps, args.warmup, stream)
    alg_bytes = algorithmic_bytes(w)
    launches = w.n_chunks if (w.mode == "block" and args.block_mode == "chunks") else 1
    call_ms = ms_per_step / launches

    # kernels per call, from the library's own geometry: one launch (state and
    # apply of a head in one workgroup) when every head is one chunk of one
    # split; else the state pass and the apply, and the finalize when a head
    # has several partials
    rope_form = 0 if rope is None else (2 if rope.grid else 1)
    if w.mode == "block" and args.block_mode == "chunks":
        n_kernels = la.forward_launches(w.B, w.H, w.chunk, None, w.D, dt, rope_form, not packed)
    else:
        n_kernels = la.forward_launches(w.B, w.H, w.N, w.chunk if w.mode == "block" else None, w.D, dt, rope_form,
                                        not packed)
    kernels = {1: "state pass and apply in one launch (forward_whole_bf16)", 2: "state pass + apply pass",
               3: "state pass + finalize + apply pass"}.get(n_kernels, "none")
    # two launches where a head has several partials: the apply sums them
    # itself (apply_fold_bf16); the same geometry read through a strided view
    # would take three
    n_call = w.chunk if (w.mode == "block" and args.block_mode == "chunks") else w.N
    folded = n_kernels == 2 and la.forward_launches(
        w.B, w.H, n_call, w.chunk if (w.mode == "block" and args.block_mode != "chunks") else None, w.D, dt,
        rope_form, False) == 3
    if folded:
        kernels = "state pass + apply that sums the partials (apply_fold_bf16)"

    # roofline of the dominant kernel: the apply pass, launched alone on the
    # state of its head (one chunk's worth of tokens in block mode)
    n_apply = w.chunk if w.mode == "block" else w.N
    kv_st = torch.empty(w.B, w.H, 32, 32, device=dev)
    z_st = torch.empty(w.B, w.H, 32, device=dev)
    apply_sets = []
    for s in sets:
        qa = s["q_chunks"][0] if w.mode == "block" else s["q"]
        oa = s["o_chunks"][0] if w.mode == "block" else s["o"]
        if packed:  # the apply-alone entry point takes contiguous tensors
            qa, oa = q0, torch.empty_like(q0)
        apply_sets.append((P(qa.data_ptr()), P(oa.data_ptr()), P(kv_st.data_ptr()), P(z_st.data_ptr()), w.B, w.H,
                           n_apply, w.D, dt, w.eps, rope_ref, st_ptr))
    kv_st.zero_()
    z_st.zero_()
    k_state = sets[0]["k_chunks"][0] if w.mode == "block" else (k0 if packed else sets[0]["k"])
    v_state = sets[0]["v_chunks"][0] if w.mode == "block" else (v0 if packed else sets[0]["v"])
    la.sana_linattn_state_update(k_state, v_state, kv_st, z_st, rope=rope, stream=stream)
    for i in range(args.warmup):
        L.sana_linattn_apply(*apply_sets[i % n_sets])
    torch.cuda.synchronize()
    a_start, a_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_start.record(stream)
    for i in range(args.steps):
        rc = L.sana_linattn_apply(*apply_sets[i % n_sets])
        if rc:
            raise la.SanaError(rc)
    a_end.record(stream)
    torch.cuda.synchronize()
    apply_ms = a_start.elapsed_time(a_end) / args.steps
    apply_bytes = w.B * w.H * n_apply * 2 * w.D * (2 if w.dtype == "bf16" else 4) + w.B * w.H * (32 * 32 + 32) * 4
    achieved = apply_bytes / (apply_ms / 1e3) / 1e9
    roof_kernel = "apply_bf16" if w.dtype == "bf16" else "apply_f32"
    roof_bytes, roof_ms, roof_tokens = apply_bytes, apply_ms, w.B * w.H * n_apply
    if n_kernels == 1 or folded:
        # the call is one kernel, or the state pass and the apply that does the
        # finalize's work: the call's own bytes and time (the apply-alone
        # figures stay in the record as `apply_alone`)
        roof_kernel = "forward_whole_bf16" if n_kernels == 1 else "state_bf16+apply_fold_bf16"
        roof_bytes, roof_ms = alg_bytes / launches, call_ms
        roof_tokens = w.token_heads // launches
        achieved = roof_bytes / (roof_ms / 1e3) / 1e9
    traffic = stored_traffic(w.name, roof_kernel)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1)x0.5 bf16 tensors at the workload's latent shape (no dataset, no weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "mode": w.mode,
                   "chunk": w.chunk, "grid": w.grid, "eps": w.eps, "input_sets_cycled": n_sets,
                   "block_calls": args.block_mode if w.mode == "block" else None,
                   "layout": args.layout, "rope_form": args.rope_form if w.mode == "rope" else None},
        "roofline": {
            "bound": "hbm",
            "kernel": roof_kernel,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": roof_bytes,
            "avg_launch_ms": roof_ms,
            "tokens_per_launch": roof_tokens,
        },
        "apply_alone": {"kernel": "apply_bf16" if w.dtype == "bf16" else "apply_f32", "avg_launch_ms": apply_ms,
                        "algorithmic_bytes_per_launch": apply_bytes,
                        "achieved_gbps": apply_bytes / (apply_ms / 1e3) / 1e9},
        "call": {
            "entry_point": ("sana_linattn_forward_strided (packed [B,N,3,H,D] in, [B,N,H,D] out)" if packed else
                            "sana_linattn_forward" if w.mode != "block" else
                            "sana_linattn_block_causal (whole sequence)" if args.block_mode == "sequence" else
                            "sana_linattn_block_forward (per chunk)"),
            "kernels": kernels,
            "avg_ms": call_ms,
            "algorithmic_bytes": alg_bytes / launches,
            "achieved_gbps": (alg_bytes / launches) / (call_ms / 1e3) / 1e9,
            "frac_of_peak": (alg_bytes / launches) / (call_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
        },
        "hbm_gbps_step": alg_bytes / (ms_per_step / 1e3) / 1e9,
        "step_ms_percentiles": step_pct,
        "wall_s_timed_region": wall,
        "input_sha256": x.sha256()[:16],
        "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline({"kind": "attention", "workload": w.name}, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
