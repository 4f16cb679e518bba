"""Error metrics for comparing the HIP path with the float64 oracle.

rel-L2           ||o - r||_2 / ||r||_2 over the whole tensor, in float64.
floored rel err  |o - r| / max(|r|, 1e-3 * RMS(r)) per element.  Outputs cross
                 zero, so a bare |o - r| / |r| is unbounded even for a correct
                 kernel; the floor at 1e-3 of the tensor's RMS keeps the metric
                 relative for every output that is not tiny compared with the
                 rest.  The number of floored elements is reported beside it.

Tolerances (float32 accumulation everywhere):
  fp32 I/O  rel-L2 <= 1e-5
  bf16 I/O  rel-L2 <= 4e-3 and floored max rel err <= 2e-2
"""

import numpy as np

F32_REL_L2 = 1e-5
BF16_REL_L2 = 4e-3
BF16_MAX_REL = 2e-2
FLOOR = 1e-3


def rel_l2(o, r):
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(o - r) / nr) if nr > 0 else float(np.linalg.norm(o))


def floored_rel(o, r):
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = FLOOR * rms
    denom = np.maximum(np.abs(r), floor)
    with np.errstate(invalid="ignore", divide="ignore"):
        err = np.where(denom > 0, np.abs(o - r) / np.where(denom > 0, denom, 1.0), np.abs(o - r))
    return float(err.max()) if err.size else 0.0, int(np.count_nonzero(np.abs(r) < floor))


def check(o, r, dtype, what=""):
    """Assert the tolerance for `dtype` ("bf16" or "f32"); returns the metrics."""
    l2 = rel_l2(o, r)
    mx, n_floored = floored_rel(o, r)
    info = f"{what}: rel-L2 {l2:.3e}, floored max rel {mx:.3e} ({n_floored} floored)"
    print(info, flush=True)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    if dtype == "f32":
        assert l2 <= F32_REL_L2, info
    else:
        assert l2 <= BF16_REL_L2, info
        assert mx <= BF16_MAX_REL, info
    return l2, mx
