"""The comparison rules themselves, checked on the CPU.

The decode linear's element-wise rule (tests/parity.py, check_quantized_dot)
must accept the float32 arithmetic the product does and reject the mistakes
a kernel could plausibly make.  At the 70B down-projection shape (28672
inputs, 2-bit weights in groups of 64), a float32 emulation of a
group-blocked, split product passes it, while the same emulation with one
split part dropped, or with one group's scale doubled, fails it.  The
16-bit rotation rule rejects a second rounding.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import linear as OL
from oracle import quant as Q
from parity import check_quantized_dot, check_rotation, gamma_tilde, quantized_dot_path

N_IN, GROUP, BITS, SPLIT = 28672, 64, 2, 1024


def _operands(T_, m, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << BITS, size=(m, N_IN)).astype(np.uint8)
    alpha = ((0.5 + rng.random((m, N_IN // GROUP))) * 0.05).astype(np.float32)
    x = rng.standard_normal((T_, N_IN))
    x[:, rng.choice(N_IN, size=N_IN // 200, replace=False)] *= 20.0
    xt = S.storage_to_f64(S.to_storage(x, "f16"), "f16")
    return codes, alpha, xt


def _emulate_f32(codes, alpha, xt, drop_split=None):
    """Z in float32 the way a group-blocked product forms it: per group the
    exact products level * x summed one by one, times fl(alpha / L), groups
    added one by one within a split of SPLIT inputs, then the splits."""
    L = (1 << BITS) - 1
    lev = (2.0 * codes.astype(np.float32) - L).astype(np.float32)          # [m, n]
    xs = xt.astype(np.float32)                                             # [T, n]
    prod = lev[None, :, :] * xs[:, None, :]                                # exact in f32
    T_, m = xs.shape[0], lev.shape[0]
    g = prod.reshape(T_, m, N_IN // GROUP, GROUP)
    gsum = np.cumsum(g, axis=3, dtype=np.float32)[..., -1]                 # sequential
    scale = (alpha / np.float32(L)).astype(np.float32)
    gs = (gsum * scale[None]).astype(np.float32)
    per = SPLIT // GROUP
    parts = np.cumsum(gs.reshape(T_, m, -1, per), axis=3, dtype=np.float32)[..., -1]
    if drop_split is not None:
        parts[:, :, drop_split] = 0
    return np.cumsum(parts, axis=2, dtype=np.float32)[..., -1]


def _reference(codes, alpha, xt):
    w = OL.weight(codes, alpha.astype(np.float64), BITS, GROUP)
    return xt @ w.T, np.abs(xt) @ np.abs(w).T


@pytest.mark.parametrize("T_", [1, 4])
def test_quantized_dot_bound_accepts_f32_and_rejects_planted_faults(T_):
    m = 192
    codes, alpha, xt = _operands(T_, m, 11 + T_)
    z_ref, s_abs = _reference(codes, alpha, xt)
    p = quantized_dot_path(N_IN, GROUP)
    z = _emulate_f32(codes, alpha, xt)
    info = check_quantized_dot(z, z_ref, s_abs, p, "float32 emulation")
    assert info["worst_frac_of_bound"] < 0.2

    # one split part (1024 of 28672 inputs) missing: every output fails
    z_drop = _emulate_f32(codes, alpha, xt, drop_split=5)
    with pytest.raises(AssertionError):
        check_quantized_dot(z_drop, z_ref, s_abs, p, "dropped split")
    tol = gamma_tilde(p) * s_abs
    assert (np.abs(z_drop - z_ref) > tol).mean() > 0.9

    # one group's scale doubled in one output row
    bad_alpha = alpha.copy()
    bad_alpha[37, 101] *= 2
    z_scale = _emulate_f32(codes, bad_alpha, xt)
    with pytest.raises(AssertionError):
        check_quantized_dot(z_scale, z_ref, s_abs, p, "doubled scale")
    # the failure is exactly the planted row
    bad = np.abs(z_scale - z_ref) > 2 * np.abs(z - z_ref).max()
    assert bad[:, 37].all() and not np.delete(bad, 37, axis=1).any()


def test_planted_scale_faults_fail_on_most_rows():
    """Planting the doubled scale in each of 192 rows in turn: the bound
    catches almost all of them (a miss needs the group's own contribution to
    be tiny against the bound)."""
    T_, m = 1, 192
    codes, alpha, xt = _operands(T_, m, 5)
    z_ref, s_abs = _reference(codes, alpha, xt)
    p = quantized_dot_path(N_IN, GROUP)
    tol = gamma_tilde(p) * s_abs[0]
    # the doubled group adds its own contribution once more
    L = (1 << BITS) - 1
    lev = 2.0 * codes[:, 64 * 7:64 * 8].astype(np.float64) - L
    contrib = (lev * xt[0, 64 * 7:64 * 8]).sum(axis=1) * alpha[:, 7] / L
    caught = np.abs(contrib) > tol
    assert caught.mean() > 0.95


def test_sixteen_bit_rule_rejects_double_rounding():
    """A value rounded to float16 twice (through bfloat16 first) lands more
    than one ulp plus the float32 allowance away for some elements; a single
    rounding never does."""
    rng = np.random.default_rng(3)
    y_ref = rng.standard_normal((64, 4096)) * 3.0
    once = y_ref.astype(np.float16).astype(np.float64)
    check_rotation(once, y_ref, "f16", "single rounding")
    twice_bf = S.storage_to_f64(S.to_storage(y_ref, "bf16"), "bf16")
    with pytest.raises(AssertionError):
        check_rotation(twice_bf, y_ref, "f16", "rounded through bf16")
