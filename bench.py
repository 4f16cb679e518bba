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

Prints ONE JSON line.  `roofline` describes the dominant kernel; `cpu_baseline`
times the float64 oracle on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import WORKLOADS, generate  # noqa: E402

METRIC = "linear-attn tokens·heads/s + achieved HBM GB/s (% peak), Sana-1.6B 4096px layer"
UNIT = "tokens·heads/s"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["linear_attention_diffusion_amd/csrc/la_kernels.h",
                  "linear_attention_diffusion_amd/csrc/sana_linattn.hip"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes the method must move: Q, K, V read once and O written once per
    token-head; in block mode also the fp32 state read and written per chunk."""
    b = w.token_heads * w.bytes_per_token_head()
    if w.mode == "block":
        b += w.n_chunks * w.B * w.H * 2 * (32 * 32 + 32) * 4
    return b


def stored_traffic(name):
    """HBM bytes per step from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_step")


def cpu_baseline(w, x, budget_s):
    """Time the float64 oracle on the host on the same workload's inputs."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity
        threads = len(os.sched_getaffinity(0))
    f = x.f64
    angles = oracle.rope3d_angles(*w.grid) if w.mode == "rope" else None
    # bounded sample: whole heads of the workload, as many as fit the budget
    heads = w.H
    t0 = time.perf_counter()
    done = 0
    runs = 0
    while True:
        h0 = (runs * heads) % w.H
        sl = slice(h0, h0 + heads)
        if w.mode == "block":
            oracle.block_causal(f["q"][:, sl], f["k"][:, sl], f["v"][:, sl], w.chunk, w.eps)
        else:
            oracle.linattn(f["q"][:, sl], f["k"][:, sl], f["v"][:, sl], w.eps, angles=angles)
        done += w.B * heads * w.N
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    return {"value": done / el, "unit": UNIT, "cores": threads, "kind": "oracle",
            "sample": f"{runs} run(s) of the float64 oracle over all {w.H} heads x {w.N} tokens "
                      f"(B={w.B}) of this workload, {el:.1f} s on the host"}


def copy_probe(steps, warmup, nbytes=2 ** 30):
    """A plain copy kernel of known size: reads and writes `nbytes` per launch."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "ms_per_copy": ms, "gbps_read_plus_write": 2 * nbytes / (ms / 1e3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sana16b_4096px", choices=list(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (HBM reference and counter scale)")
    args = ap.parse_args()

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

    x = generate(w, with_f64=False)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(raw):
        if w.dtype == "bf16":
            return torch.from_numpy(raw.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(raw).to(dev)

    q0, k0, v0 = (to_dev(x.raw[n]) for n in ("q", "k", "v"))
    set_bytes = 4 * q0.numel() * q0.element_size()
    n_sets = max(2, min(16, math.ceil(1.5 * 2 ** 30 / set_bytes) + 1))
    sets = []
    for i in range(n_sets):
        if i == 0:
            q, k, v = q0, k0, v0
        else:
            q, k, v = q0.clone(), k0.clone(), v0.clone()
        sets.append({"q": q, "k": k, "v": v, "o": torch.empty_like(q)})

    rope = la.rope3d_device(*w.grid, dev) if w.mode == "rope" else None
    if w.mode == "block":
        L = w.chunk
        for s in sets:
            for n in ("q", "k", "v", "o"):
                t = s[n]
                s[n + "_chunks"] = [t[:, :, c:min(w.N, c + L)].contiguous() for c in range(0, w.N, L)]
            s["kv"] = torch.zeros(w.B, w.H, 32, 32, device=dev)
            s["z"] = torch.zeros(w.B, w.H, 32, device=dev)
        ws = la.make_workspace(w.B, w.H, L, dev, dtype=la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32)
    else:
        ws = la.make_workspace(w.B, w.H, w.N, dev, dtype=la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32,
                               has_rope=rope is not None)

    def step(i):
        s = sets[i % n_sets]
        if w.mode == "block":
            kv, z = s["kv"], s["z"]
            for c, (qc, kc, vc, oc) in enumerate(zip(s["q_chunks"], s["k_chunks"], s["v_chunks"], s["o_chunks"])):
                # chunk 0 starts from the zero state (kv_in = NULL); every chunk commits in place
                la.sana_linattn_block_forward(qc, kc, vc, oc, kv_in=None if c == 0 else kv,
                                              ksum_in=None if c == 0 else z, kv_out=kv, ksum_out=z,
                                              eps=w.eps, workspace=ws, stream=stream)
        else:
            la.sana_linattn_forward(s["q"], s["k"], s["v"], s["o"], eps=w.eps, rope=rope, workspace=ws,
                                    stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, an event pair around each (events on the launch stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(args.warmup + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_step_ms = [a.elapsed_time(b) for a, b in evs]
    total_ms = evs[0][0].elapsed_time(evs[-1][1])

    ms_per_step = total_ms / args.steps
    value = w.token_heads * args.steps / (total_ms / 1e3)
    alg_bytes = algorithmic_bytes(w)
    launches = w.n_chunks if w.mode == "block" else 1
    launch_ms = statistics.mean(per_step_ms) / launches
    achieved = (alg_bytes / launches) / (launch_ms / 1e3) / 1e9
    traffic = stored_traffic(w.name)

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
                   "chunk": w.chunk, "grid": w.grid, "eps": w.eps, "input_sets_cycled": n_sets},
        "roofline": {
            "bound": "hbm",
            "kernel": "sana_linattn_forward call (state partials + finalize + apply)"
                      if w.mode != "block" else "sana_linattn_block_forward call (per chunk)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes / launches,
            "avg_launch_ms": launch_ms,
        },
        "step_ms": {"median": statistics.median(per_step_ms),
                    "p10": float(np.percentile(per_step_ms, 10)),
                    "p90": float(np.percentile(per_step_ms, 90))},
        "hbm_gbps_step": alg_bytes / (ms_per_step / 1e3) / 1e9,
        "wall_s_timed_region": wall,
        "input_sha256": x.sha256()[:16],
        "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        xf = generate(w)
        rec["cpu_baseline"] = cpu_baseline(w, xf, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
