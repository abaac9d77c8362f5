"""Shared helpers for the GPU parity tests: tolerance checks and small utilities.

Tolerances (stated per output kind):
  fp32 storage: elementwise |a - b| <= 1e-4 |b| + 1e-6 max|b|, and rel-L2 <= 1e-4. The absolute
    floor covers entries that nearly cancel: an fp32 attention logit is exact to about
    d 2^-24 |q||k| scale, which moves an output element by about 1e-6 of the values' scale.
  bf16 storage of a compressed entry: compared with the oracle's unrounded double value b,
    |a - b| <= max(1e-2, ulp_bf16(b)) and rel-L2 <= 5e-3; in addition the kernel's own error
    bound (fp32 arithmetic, one rounding to bf16) is asserted:
    |a - b| <= ulp_bf16(b) + 2e-5 max|b|.
  fp32 outputs computed from bf16 inputs (attention): max-abs <= 1e-2 and rel-L2 <= 5e-3.
  Indices: bit-exact.
"""
import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)


def assert_f32(got, want, what="", rtol=1e-4):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    scale = np.abs(want).max()
    err = np.abs(got - want)
    bound = rtol * np.abs(want) + rtol * 1e-2 * scale
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, f"{what}: {bad.size} elements beyond fp32 tolerance, worst " \
                          f"{err.ravel()[bad[:5]]} at {bad[:5]}"
    assert rel_l2(got, want) <= rtol, f"{what}: rel-L2 {rel_l2(got, want)}"


def ulp_bf16(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_bf16_stored(got, want_double, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want_double, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    err = np.abs(got - want)
    u = ulp_bf16(want)
    bad = np.flatnonzero(err > np.maximum(1e-2, u))
    assert bad.size == 0, f"{what}: {bad.size} beyond max(1e-2, ulp)"
    assert rel_l2(got, want) <= 5e-3, f"{what}: rel-L2 {rel_l2(got, want)}"
    # fp32 accumulation leaves an absolute error of a few 1e-7 of the terms' size, which is
    # larger than a bf16 ulp only where the pooled value nearly cancels to zero.
    bound = u + 2e-5 * np.abs(want).max()
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, f"{what}: {bad.size} elements more than one bf16 ulp from the exact value, " \
                          f"worst {np.max(err / bound)} of the bound"


def assert_bf16_path(got, want, what="", max_abs=1e-2, rl2=5e-3):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    ma = np.abs(got - want).max()
    assert ma <= max_abs, f"{what}: max-abs {ma}"
    r = rel_l2(got, want)
    assert r <= rl2, f"{what}: rel-L2 {r}"


def assert_lse(got, want, what="", tol=1e-3):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    inf_g, inf_w = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(inf_g, inf_w), f"{what}: -inf pattern differs"
    fin = ~inf_w
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= tol * max(1.0, np.abs(want[fin]).max()), f"{what}: lse err {err}"


def check_swaps(gpu_sel, ref_sel, ref_scores, k):
    """End-to-end top-k rule: the GPU set may differ from the oracle's only by candidates whose
    oracle score lies within 1e-6 relative of the oracle's threshold (its k-th largest)."""
    g = set(int(x) for x in gpu_sel if x >= 0)
    r = set(int(x) for x in ref_sel if x >= 0)
    assert len(g) == len(r)
    if g == r:
        return 0
    s = np.asarray(ref_scores, np.float64)
    tau = np.sort(s)[::-1][min(k, s.size) - 1]
    for j in g ^ r:
        assert abs(s[j] - tau) <= 1e-6 * abs(tau), f"swap of {j}: score {s[j]} vs tau {tau}"
    return len(g ^ r) // 2
