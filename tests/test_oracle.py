"""CPU tests of the float64 oracle against its pins, and mutation tests showing
that each plausible mistake planted in a copy of the oracle fails a pin."""

import inspect
import types

import numpy as np
import pytest

import oracle
import oracle.linattn_oracle as oracle_src
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _mutant(old, new, count=1):
    src = inspect.getsource(oracle_src)
    assert src.count(old) == count, f"mutation anchor {old!r} found {src.count(old)} times"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


# Each mutant is one plausible mistake: (anchor text in the oracle, replacement).
MUTANTS = {
    "relu_also_on_v": ("    v = np.asarray(v, dtype=np.float64)\n    pos = _positions(angles, phik.shape[-2], pos_offset)",
                       "    v = feature_map(v)\n    pos = _positions(angles, phik.shape[-2], pos_offset)"),
    "no_relu": ("return np.maximum(np.asarray(x, dtype=np.float64), 0.0)",
                "return np.asarray(x, dtype=np.float64)"),
    "state_transposed": ("S = np.matmul(np.swapaxes(phik_num, -1, -2), v)",
                         "S = np.swapaxes(np.matmul(np.swapaxes(phik_num, -1, -2), v), -1, -2)"),
    "eps_in_numerator": ("return num / den", "return (num + eps) / den"),
    "eps_dropped": ("den = np.matmul(phiq, z[..., :, None]) + eps", "den = np.matmul(phiq, z[..., :, None])"),
    "rope_in_denominator": ("den = np.matmul(phiq, z[..., :, None]) + eps",
                            "den = np.matmul(phiq_num, z[..., :, None]) + eps"),
    "rope_key_sum": ("z = phik.sum(axis=-2)", "z = phik_num.sum(axis=-2)"),
    "rope_before_relu": ("    phik = feature_map(k)\n    v = np.asarray(v, dtype=np.float64)\n    pos = _positions(angles, phik.shape[-2], pos_offset)\n    phik_num = phik if pos is None else rotate_pairs(phik, pos)",
                         "    phik = feature_map(k)\n    v = np.asarray(v, dtype=np.float64)\n    pos = _positions(angles, phik.shape[-2], pos_offset)\n    phik_num = phik if pos is None else feature_map(rotate_pairs(k, pos))"),
    "rotation_sign": ("out[..., 1::2] = x0 * s + x1 * c", "out[..., 1::2] = -x0 * s + x1 * c"),
    "pairs_not_interleaved": ("x0 = x[..., 0::2]\n    x1 = x[..., 1::2]",
                              "x0 = x[..., :x.shape[-1] // 2].repeat(1, axis=-1)[..., :x.shape[-1] // 2]\n    x1 = x[..., x.shape[-1] // 2:]"),
    "rope_base": ("def rope3d_angles(T, Hl, Wl, D=32, split=(8, 12, 12), base=10000.0):",
                  "def rope3d_angles(T, Hl, Wl, D=32, split=(8, 12, 12), base=1000.0):"),
    "rope_axis_order": ("coords = [tt.reshape(-1), hh.reshape(-1), ww.reshape(-1)]",
                        "coords = [ww.reshape(-1), hh.reshape(-1), tt.reshape(-1)]"),
    "rope_freq_exponent": ("freq = base ** (-2.0 * k / width)", "freq = base ** (-1.0 * k / width)"),
    "block_exclusive_mask": ("M = (idx[None, :] <= idx[:, None])", "M = (idx[None, :] < idx[:, None])"),
    "block_state_not_carried": ("o, S, z = block_forward(q[..., sl, :], k[..., sl, :], v[..., sl, :], S, z,",
                                "o, _S, _z = block_forward(q[..., sl, :], k[..., sl, :], v[..., sl, :], S, z,"),
    "block_uses_previous_state_only": ("    o = apply_state(q, S_new, z_new, eps, angles, pos_offset)",
                                       "    o = apply_state(q, np.asarray(S_in, dtype=np.float64), np.asarray(z_in, dtype=np.float64), eps, angles, pos_offset)"),
    "block_positions_restart": ("eps, angles, start)", "eps, angles, 0)"),
    "bwd_dden_sign": ("dden = -(dout[..., sl, :] * num)", "dden = (dout[..., sl, :] * num)"),
    "bwd_dden_power": ("/ den ** 2", "/ den"),
    "bwd_no_relu_mask_on_q": ("dq[..., sl, :] = dphiq * (q[..., sl, :] > 0)", "dq[..., sl, :] = dphiq"),
    "bwd_relu_mask_inclusive": ("dk[..., sl, :] = dphik * (k[..., sl, :] > 0)",
                                "dk[..., sl, :] = dphik * (k[..., sl, :] >= 0) + 0.0 * (k[..., sl, :] == 0)"),
    "bwd_rotation_not_inverted": ("rotate_pairs(dphiq_num, -pos[sl])", "rotate_pairs(dphiq_num, pos[sl])"),
    "bwd_key_rotation_not_inverted": ("rotate_pairs(dphik_num, -pos[sl])", "rotate_pairs(dphik_num, pos[sl])"),
    "bwd_state_not_transposed": ("dphiq_num = np.matmul(dnum, np.swapaxes(S_c, -1, -2))",
                                 "dphiq_num = np.matmul(dnum, S_c)"),
    "bwd_prefix_not_suffix": ("for c in range(len(chunks) - 1, -1, -1):", "for c in range(len(chunks)):"),
    "bwd_key_sum_gradient_dropped": ("dphik = dphik_rot + Gz[..., None, :]", "dphik = dphik_rot"),
    "bwd_dv_unrotated_keys": ("dv[..., sl, :] = np.matmul(phik_num[..., sl, :], G)",
                              "dv[..., sl, :] = np.matmul(phik[..., sl, :], G)"),
    "bwd_dS_rotation_dropped": ("dS_chunk.append(np.matmul(np.swapaxes(phiq_num[..., sl, :], -1, -2), dnum))",
                                "dS_chunk.append(np.matmul(np.swapaxes(phiq[..., sl, :], -1, -2), dnum))"),
    "bwd_out_gradient_ignored": ("G = np.zeros(lead + (D, D)) if dS_out is None else np.asarray(dS_out, dtype=np.float64)",
                                 "G = np.zeros(lead + (D, D))"),
    "conv_taps_swapped": ("y = x + w[:, 0] * padded[:, :F] + w[:, 1] * padded[:, 1:F + 1] + w[:, 2] * padded[:, 2:F + 2]",
                          "y = x + w[:, 2] * padded[:, :F] + w[:, 1] * padded[:, 1:F + 1] + w[:, 0] * padded[:, 2:F + 2]"),
    "conv_no_shortcut": ("y = x + w[:, 0] * padded[:, :F]", "y = 0 * x + w[:, 0] * padded[:, :F]"),
    "conv_cache_first_frame": ("return y, x[:, F - 1].copy()", "return y, x[:, 0].copy()"),
    "conv_wraps_around": ("padded = np.concatenate([prev[:, None], x, np.zeros((B, 1, S, C))], axis=1)",
                          "padded = np.concatenate([prev[:, None], x, x[:, :1]], axis=1)"),
    "proj_rounding_dropped": ("k = round_bf16(np.matmul(x, np.asarray(w_k, dtype=np.float64)[None]))",
                              "k = np.matmul(x, np.asarray(w_k, dtype=np.float64)[None])"),
    "proj_k_v_swapped": ("return kv_state(k, v, angles, pos_offset)", "return kv_state(v, k, angles, pos_offset)"),
    "proj_round_to_nearest_away": ("return np.ldexp(np.rint(m * 256.0), e - 8)",
                                   "return np.ldexp(np.floor(m * 256.0 + 0.5), e - 8)"),
    "proj_rotation_dropped": ("return kv_state(k, v, angles, pos_offset)", "return kv_state(k, v)"),
    "proj_positions_from_zero": ("return kv_state(k, v, angles, pos_offset)", "return kv_state(k, v, angles, 0)"),
    "papply_rounding_dropped": ("q = round_bf16(np.matmul(x, np.asarray(w_q, dtype=np.float64)[None]))",
                                "q = np.matmul(x, np.asarray(w_q, dtype=np.float64)[None])"),
    "papply_rotation_dropped": ("np.asarray(z, dtype=np.float64), eps, angles, pos_offset)",
                                "np.asarray(z, dtype=np.float64), eps)"),
    "proj_round_7_bits": ("return np.ldexp(np.rint(m * 256.0), e - 8)", "return np.ldexp(np.rint(m * 128.0), e - 7)"),
    "bwd_carried_state_ignored": ("S = np.zeros(lead + (D, D)) if S_in is None else np.asarray(S_in, dtype=np.float64)\n    z = np.zeros(lead + (D,)) if z_in is None else np.asarray(z_in, dtype=np.float64)\n    states = []",
                                  "S = np.zeros(lead + (D, D))\n    z = np.zeros(lead + (D,)) if z_in is None else np.asarray(z_in, dtype=np.float64)\n    states = []"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    mod = _mutant(old, new)
    failures = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, FloatingPointError) as exc:
            failures.append(f"{pin.__name__}: {str(exc).splitlines()[0] if str(exc) else type(exc).__name__}")
    assert failures, f"mutant {name} passed every pin"
