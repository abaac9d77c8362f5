"""The fp32 attention tolerance, reproduced on the CPU.

The fp32 check (chs_testutil.assert_f32) is |a - b| <= 1e-4 |b| + 1e-6 max|b| elementwise plus rel-L2
<= 1e-4. The absolute floor comes from the arithmetic, not from the GPU: a logit q.k.scale summed in fp32
over d channels is exact to about d 2^-24 |q||k| scale, and an output element that nearly cancels moves
by about that much times the values' scale. Here a plain fp32 implementation written for this test
(channels and keys accumulated one after another, one fp32 rounding per step; it shares nothing with the
GPU kernels) is compared with the oracle's double-precision attention on the fp32 test shapes:

- every case passes the committed tolerance;
- at d = 1024 some output elements of this correct fp32 computation lie beyond a floor of
  1e-7 max|b|, so a floor that tight would reject correct fp32 results;
- the worst excess stays well inside the 1e-6 floor.
"""
import numpy as np

import oracle
from chs_testutil import assert_f32

F32 = np.float32


def _sequential_f32_attend(q, keys, scale):
    """One softmax over keys (keys are also the values), every sum taken in fp32 one term at a time."""
    q = q.astype(F32)
    k = keys.astype(F32)
    H, d = q.shape
    n = k.shape[0]
    dot = np.zeros((H, n), F32)
    for i in range(d):
        dot = (dot + np.outer(q[:, i], k[:, i]).astype(F32)).astype(F32)
    logits = (dot * F32(scale)).astype(F32)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m).astype(F32)
    total = np.zeros((H, 1), F32)
    acc = np.zeros((H, d), F32)
    for j in range(n):
        total = (total + p[:, j:j + 1]).astype(F32)
        acc = (acc + (p[:, j:j + 1] * k[j:j + 1, :]).astype(F32)).astype(F32)
    return (acc / total).astype(F32)


def _excess(got, want, floor):
    """Largest elementwise error beyond 1e-4 |b| + floor max|b|, in units of floor max|b|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = np.abs(want).max()
    return float(((np.abs(got - want) - 1e-4 * np.abs(want)) / (floor * scale)).max())


def test_fp32_attention_error_needs_the_1e6_floor():
    worst7, worst6 = -np.inf, -np.inf
    for seed in range(6):
        rng = np.random.default_rng(seed)
        for H, d, n in ((8, 64, 192), (2, 1024, 40), (3, 36, 700)):
            q = rng.standard_normal((H, d)).astype(F32)
            keys = (rng.standard_normal((n, d)) * 0.5).astype(F32)
            scale = d ** -0.5
            want, _ = oracle.attend(q, keys, scale)
            got = _sequential_f32_attend(q, keys, scale)
            assert_f32(got, want, f"seed {seed} H={H} d={d} n={n}")
            worst7 = max(worst7, _excess(got, want, 1e-7))
            worst6 = max(worst6, _excess(got, want, 1e-6))
    assert worst7 > 1.0, f"no element beyond the 1e-7 floor (worst {worst7:.3f} of it)"
    assert worst6 < 0.5, f"the fp32 error reaches {worst6:.3f} of the 1e-6 floor"
