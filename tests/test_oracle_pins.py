"""Pins for the CPU oracle, against facts that do not come from the oracle itself:
closed forms, invariants, special cases that reduce to a library routine, brute force on tiny
inputs, and the structural counts the pages print. Each pin is chosen so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand) fails it."""
import itertools
import os

import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_structure.txt")


def _golden():
    vals = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


# ------------------------------------------------------------------ compressor
def _groups(X, m):
    n = (X.shape[0] // m) * m
    return X[:n].astype(np.float64).reshape(-1, m, X.shape[1])


@pytest.mark.parametrize("m", [2, 4, 5, 128])
def test_compress_constant_gate_and_flat_bias_is_mean_pooling(rng, m):
    X = rng.standard_normal((m * 6 + 3, 24)).astype(np.float32)
    Z = np.full_like(X, 0.7)
    B = np.full((m, 24), -1.25, np.float32)   # slot-constant bias: no preference between slots
    C = oracle.compress(X, Z, B, m, [0, X.shape[0]])
    np.testing.assert_allclose(C, _groups(X, m).mean(axis=1), rtol=0, atol=1e-12)


def test_compress_m1_is_identity(rng):
    X = rng.standard_normal((37, 16)).astype(np.float32)
    Z = rng.standard_normal((37, 16)).astype(np.float32) * 3
    B = rng.standard_normal((1, 16)).astype(np.float32)
    C = oracle.compress(X, Z, B, 1, [0, 37])
    assert np.array_equal(C.astype(np.float32), X)


@pytest.mark.parametrize("m", [3, 4, 128])
def test_compress_weights_sum_to_one(rng, m):
    # With every token vector equal to 1, the output is the sum of the weights.
    T = m * 5
    X = np.ones((T, 8), np.float32)
    Z = (rng.standard_normal((T, 8)) * 5).astype(np.float32)
    B = rng.standard_normal((m, 8)).astype(np.float32)
    C = oracle.compress(X, Z, B, m, [0, T])
    assert np.abs(C - 1.0).max() <= 1e-12


def test_compress_shift_invariance(rng):
    m, T, d = 4, 40, 12
    X = rng.standard_normal((T, d)).astype(np.float32)
    # Gates on a 1/64 grid, so adding an integer shift is exact in fp32.
    Z = (np.round(rng.standard_normal((T, d)) * 64) / 64).astype(np.float32)
    B = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
    shift = np.repeat(rng.integers(-8, 8, (T // m, d)), m, axis=0).astype(np.float32)
    C1 = oracle.compress(X, Z, B, m, [0, T])
    C2 = oracle.compress(X, Z + shift, B, m, [0, T])
    np.testing.assert_allclose(C1, C2, rtol=0, atol=1e-12)


def test_compress_dominant_slot_selects_that_token(rng):
    m, T, d = 4, 32, 10
    X = rng.standard_normal((T, d)).astype(np.float32)
    Z = rng.standard_normal((T, d)).astype(np.float32)
    B = np.zeros((m, d), np.float32)
    slot = rng.integers(0, m, (T // m, d))
    for g in range(T // m):
        for c in range(d):
            Z[g * m + slot[g, c], c] += 200.0
    C = oracle.compress(X, Z, B, m, [0, T])
    want = np.array([[X[g * m + slot[g, c], c] for c in range(d)] for g in range(T // m)])
    np.testing.assert_allclose(C, want, rtol=0, atol=1e-12)


def test_compress_m2_logistic_closed_form(rng):
    # For two slots the softmax weight of slot 0 is the logistic function of a0 - a1.
    T, d = 20, 9
    X = rng.standard_normal((T, d)).astype(np.float32)
    Z = (rng.standard_normal((T, d)) * 2).astype(np.float32)
    B = (rng.standard_normal((2, d)) * 0.5).astype(np.float32)
    C = oracle.compress(X, Z, B, 2, [0, T])
    a0 = Z[0::2].astype(np.float64) + B[0]
    a1 = Z[1::2].astype(np.float64) + B[1]
    want = expit(a0 - a1) * X[0::2] + expit(a1 - a0) * X[1::2]
    np.testing.assert_allclose(C, want, rtol=1e-12, atol=1e-14)


def test_compress_bias_is_per_slot_per_channel(rng):
    # Constant gates leave only the bias: weights are softmax over slots of B[:, c].
    m, d = 3, 7   # m != d, so a transposed bias would not even line up
    T = m * 4
    X = rng.standard_normal((T, d)).astype(np.float32)
    Z = np.zeros((T, d), np.float32)
    B = rng.standard_normal((m, d)).astype(np.float32)
    C = oracle.compress(X, Z, B, m, [0, T])
    W = softmax(B.astype(np.float64), axis=0)          # [m, d]
    want = np.einsum("gic,ic->gc", _groups(X, m), W)
    np.testing.assert_allclose(C, want, rtol=1e-12, atol=1e-14)


def test_compress_slot_permutation_invariance(rng):
    m, T, d = 4, 24, 6
    X = rng.standard_normal((T, d)).astype(np.float32)
    Z = rng.standard_normal((T, d)).astype(np.float32)
    B = rng.standard_normal((m, d)).astype(np.float32)
    perm = np.array([2, 0, 3, 1])
    rows = (np.arange(T // m)[:, None] * m + perm[None, :]).ravel()
    C1 = oracle.compress(X, Z, B, m, [0, T])
    C2 = oracle.compress(X[rows], Z[rows], B[perm], m, [0, T])
    np.testing.assert_allclose(C1, C2, rtol=1e-13, atol=1e-14)


def test_compress_varlen_packing_and_tails(rng):
    m, d = 4, 5
    lens = [10, 7, 3, 12, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    X = rng.standard_normal((T, d)).astype(np.float32)
    Z = rng.standard_normal((T, d)).astype(np.float32)
    B = rng.standard_normal((m, d)).astype(np.float32)
    C = oracle.compress(X, Z, B, m, cu)
    assert C.shape[0] == sum(n // m for n in lens) == 7
    parts = [oracle.compress(X[cu[b]:cu[b + 1]], Z[cu[b]:cu[b + 1]], B, m, [0, lens[b]])
             for b in range(len(lens))]
    np.testing.assert_array_equal(C, np.concatenate(parts, axis=0))
    # Tail tokens (the last N_b mod m of each sequence) do not enter any group.
    X2, Z2 = X.copy(), Z.copy()
    for b, n in enumerate(lens):
        tail = range(cu[b] + (n // m) * m, cu[b + 1])
        X2[list(tail)] = 99.0
        Z2[list(tail)] = 50.0
    np.testing.assert_array_equal(C, oracle.compress(X2, Z2, B, m, cu))


def test_compress_group_count_matches_pages():
    g = _golden()
    n, m = int(g["context_tokens"]), int(g["c4_ratio"])
    X = np.zeros((n, 1), np.float32)
    C = oracle.compress(X, X, np.zeros((m, 1), np.float32), m, [0, n])
    assert C.shape[0] == int(g["c4_candidates"])
    C128 = oracle.compress(X, X, np.zeros((int(g["c128_ratio"]), 1), np.float32), int(g["c128_ratio"]), [0, n])
    assert C128.shape[0] == n // int(g["c128_ratio"]) == 8192


# ------------------------------------------------------------------ indexer scores
def test_index_scores_one_hot_weight_is_relu_dot(rng):
    q = rng.standard_normal((3, 16)).astype(np.float32)
    K = rng.standard_normal((50, 16)).astype(np.float32)
    for h in range(3):
        w = np.zeros(3, np.float32)
        w[h] = 1.0
        s = oracle.index_scores(q, w, K)
        np.testing.assert_allclose(s, np.maximum(K.astype(np.float64) @ q[h].astype(np.float64), 0.0),
                                   rtol=1e-13, atol=1e-12)


def test_index_scores_linear_in_weights(rng):
    q = rng.standard_normal((4, 8)).astype(np.float32)
    K = rng.standard_normal((30, 8)).astype(np.float32)
    w1, w2 = rng.random(4).astype(np.float32), rng.random(4).astype(np.float32)
    s12 = oracle.index_scores(q, (w1 + w2).astype(np.float32), K)
    s1, s2 = oracle.index_scores(q, w1, K), oracle.index_scores(q, w2, K)
    # w1 + w2 is rounded to fp32 before the call; compare against that same sum.
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-6, atol=1e-9)


def test_index_scores_odd_part_identity(rng):
    # ReLU(x) - ReLU(-x) = x, so s(q) - s(-q) = sum_h w_h (q_h . k_j): catches a dropped ReLU,
    # a sign error or transposed keys.
    q = rng.standard_normal((4, 12)).astype(np.float32)
    w = rng.random(4).astype(np.float32)
    K = rng.standard_normal((40, 12)).astype(np.float32)
    lhs = oracle.index_scores(q, w, K) - oracle.index_scores(-q, w, K)
    rhs = (K.astype(np.float64) @ q.astype(np.float64).T) @ w.astype(np.float64)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_index_scores_negative_dots_give_zero(rng):
    q = rng.standard_normal((1, 10)).astype(np.float32)
    K = -np.abs(rng.standard_normal((20, 1))).astype(np.float32) * q
    assert np.all(oracle.index_scores(q, np.ones(1, np.float32), K) == 0.0)


def test_index_scores_positive_homogeneity(rng):
    q = rng.standard_normal((2, 6)).astype(np.float32)
    w = rng.random(2).astype(np.float32)
    K = rng.standard_normal((25, 6)).astype(np.float32)
    np.testing.assert_allclose(oracle.index_scores(4.0 * q, w, K), 4.0 * oracle.index_scores(q, w, K),
                               rtol=1e-14, atol=0)


# ------------------------------------------------------------------ top-k
def _is_topk_set(s, S):
    """Brute-force characterisation: every chosen element beats every unchosen one, by value
    or, on equal values, by lower index."""
    out = set(range(len(s))) - set(S)
    return all(s[i] > s[j] or (s[i] == s[j] and i < j) for i in S for j in out)


# ---------------------------------------------------------------- FP8 (E4M3) index keys
def test_decode_e4m3_matches_torch_float8_on_every_code():
    # An independent decoder: torch's float8_e4m3fn (the same OCP format) on all 256 codes.
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(codes[nan]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_e4m3_closed_forms():
    d = oracle.decode_e4m3(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0x81, 0xB8, 0xFE], np.uint8))
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -0.0, -(2.0 ** -9), -1.0, -448.0]
    assert list(d) == want
    assert np.signbit(d[7]) and not np.signbit(d[0])
    # Monotone over the non-negative codes, and a code's negation is its sign bit.
    pos = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(oracle.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos)


# ---------------------------------------------------------------- FP8 (E4M3) encoding and row quantisation
def _torch_e4m3(y):
    import torch
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_grid():
    """The 127 non-negative finite E4M3 values in code order, from torch's decoder."""
    import torch
    return torch.from_numpy(np.arange(0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_encode_e4m3_matches_torch_on_representable_values_midpoints_and_neighbours():
    # An independent encoder: torch's float8_e4m3fn cast (round to nearest even). Inputs: every
    # representable value, every midpoint between neighbours (the ties), and the fp32 neighbours
    # of each midpoint (which must round away from the tie), in both signs, up to 448.
    g = _e4m3_grid()
    mids = (g[:-1] + g[1:]) / 2
    pts = np.concatenate([g, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                          np.nextafter(mids.astype(np.float32), np.float32(-np.inf))]).astype(np.float32)
    pts = np.concatenate([pts, -pts, np.array([0.0, -0.0, 464.0, -464.0], np.float32)])
    assert np.array_equal(oracle.encode_e4m3(pts), _torch_e4m3(pts))


def test_encode_e4m3_matches_torch_on_random_fp32(rng):
    # Wide exponent range, subnormal E4M3 results included (|y| < 2^-6), up to the tie at 464.
    y = (rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 9, 200000))).astype(np.float32)
    y = y[np.abs(y) <= 464]
    assert np.array_equal(oracle.encode_e4m3(y), _torch_e4m3(y))


def test_encode_e4m3_closed_forms_and_saturation():
    y = np.array([0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6, 1.0, 1.0625, 1.1875, 448.0, 460.0, 464.0,
                  470.0, 1e6, np.float32(3.4e38), -448.0, -1e6, 2.0 ** -12, -2.0 ** -12], np.float32)
    want = [0x00, 0x01, 0x00,         # 2^-10 ties between 0 and 2^-9: to the even code 0
            0x02,                     # 3 * 2^-10 ties between codes 1 and 2: to 2
            0x08, 0x38, 0x38,         # 1.0625 ties between 1 and 1.125: to 1.0 (0x38, even)
            0x3A,                     # 1.1875 ties between 1.125 (0x39) and 1.25 (0x3A): to 0x3A
            0x7E, 0x7E, 0x7E,         # 460 rounds to 448; 464 ties 448 / 480 and 480 does not exist: 448
            0x7E, 0x7E, 0x7E,         # beyond 464 the magnitude saturates at 448 (no NaN is produced)
            0xFE, 0xFE, 0x00, 0x80]   # tiny values round to a signed zero
    assert oracle.encode_e4m3(y).tolist() == want


def test_encode_e4m3_round_trip_and_monotone():
    g = _e4m3_grid().astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(g), np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(oracle.encode_e4m3(-g[1:]), (np.arange(1, 0x7F) | 0x80).astype(np.uint8))
    y = np.sort(np.random.default_rng(5).uniform(0, 500, 20000)).astype(np.float32)
    c = oracle.encode_e4m3(y).astype(np.int64)
    assert np.all(np.diff(c) >= 0)


def test_quantize_rows_scale_and_error_bound(rng):
    # The row's largest magnitude maps to 448 exactly; every element decodes within half a step of
    # the E4M3 grid at its magnitude (relative 2^-4 for normals, absolute 2^-10 * scale below 2^-6).
    x = (rng.standard_normal((300, 128)) * np.exp2(rng.uniform(-10, 10, (300, 1)))).astype(np.float32)
    x[7] = 0.0
    x[8, :] = 0.0
    x[8, 3] = -2.5
    codes, scales = oracle.quantize_e4m3(x)
    assert scales[7] == 0.0 and np.all(codes[7] == 0)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scales, (amax.astype(np.float64) / 448.0).astype(np.float32))
    dec = oracle.decode_e4m3(codes)
    j = np.abs(x).argmax(axis=1)
    nz = amax > 0
    assert np.all(np.abs(dec[np.arange(300), j][nz]) == 448.0)
    y = x.astype(np.float64) / np.where(nz, scales, 1.0)[:, None]
    step = np.where(np.abs(y) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3),
                    2.0 ** -9)
    assert np.all(np.abs(dec - y)[nz] <= step[nz] / 2 * (1 + 1e-6))
    assert dec[8, 3] == -448.0 and np.count_nonzero(dec[8]) == 1


def test_quantize_rows_are_independent_and_scale_invariant(rng):
    # Scaling a row by a power of two scales its scale and leaves its codes unchanged; rows do not
    # interact.
    x = rng.standard_normal((20, 64)).astype(np.float32)
    c1, s1 = oracle.quantize_e4m3(x)
    c2, s2 = oracle.quantize_e4m3(x * np.float32(8.0))
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * 8)
    c3, s3 = oracle.quantize_e4m3(x[::-1].copy())
    assert np.array_equal(c3, c1[::-1]) and np.array_equal(s3, s1[::-1])


def test_index_scores_fp8_one_hot_query_reads_one_code(rng):
    # q = e_t picks element t of the row: s = w0 relu(c d) + w1 relu(-c d) = c d (d > 0) or 2 c |d|.
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]
    dim = 16
    K8 = np.resize(codes, (len(codes) // dim + 1) * dim).reshape(-1, dim)
    scale = rng.uniform(0.5, 2.0, K8.shape[0]).astype(np.float32)
    for t in (0, 5, 15):
        q = np.zeros((2, dim), np.float32)
        q[0, t], q[1, t] = 1.0, -1.0
        s = oracle.index_scores_fp8(q, np.array([1.0, 2.0], np.float32), K8, scale)
        d = oracle.decode_e4m3(K8[:, t]) * scale.astype(np.float64)
        assert np.array_equal(s, np.where(d > 0, d, -2.0 * d))


def test_index_scores_fp8_equals_scores_of_the_decoded_keys(rng):
    # With scale 1 (and power-of-two scales, exact in fp32) the FP8 keys are just fp32 keys.
    import torch
    q = rng.standard_normal((4, 32)).astype(np.float32)
    w = rng.uniform(0, 1, 4).astype(np.float32)
    K8 = rng.integers(0, 256, (300, 32)).astype(np.uint8)
    K8[(K8 == 0x7F) | (K8 == 0xFF)] = 0x38
    dec = torch.from_numpy(K8.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in (1.0, 0.25, 8.0):
        scale = np.full(300, c, np.float32)
        assert np.allclose(oracle.index_scores_fp8(q, w, K8, scale), oracle.index_scores(q, w, dec * c),
                           rtol=1e-12, atol=0)


def test_attend_fp8_single_key_returns_the_scaled_row(rng):
    codes = rng.integers(0, 256, (1, 64)).astype(np.uint8)
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0x40
    out, lse = oracle.attend_fp8(rng.standard_normal((3, 64)).astype(np.float32), codes, np.array([0.75], np.float32),
                                 0.125)
    row = 0.75 * oracle.decode_e4m3(codes[0])
    assert np.array_equal(out, np.tile(row, (3, 1)))
    assert np.all(np.isfinite(lse))


def test_attend_fp8_equals_attend_of_decoded_keys(rng):
    import torch
    codes = rng.integers(0, 256, (40, 32)).astype(np.uint8)
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0x38
    dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    scales = (2.0 ** rng.integers(-3, 4, 40)).astype(np.float32)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    o1, l1 = oracle.attend_fp8(q, codes, scales, 0.2)
    o2, l2 = oracle.attend(q, dec * scales[:, None], 0.2)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(l1, l2, rtol=1e-12, atol=0)


def test_topk_exhaustive_tiny(rng):
    values = np.array([-1.0, -0.0, 0.0, 2.0, 3.5], np.float32)
    for n in range(1, 7):
        for _ in range(40):
            s = rng.choice(values, n).astype(np.float32)
            for k in range(1, n + 3):
                got = oracle.topk(s, k)
                c = min(k, n)
                cands = [S for S in itertools.combinations(range(n), c) if _is_topk_set(s, S)]
                assert len(cands) == 1, (s, k)      # the set is unique
                assert list(got[:c]) == list(cands[0]) and all(got[c:] == -1)


@pytest.mark.parametrize("n,k", [(1, 1), (100, 7), (4096, 512), (3000, 2048), (777, 777)])
def test_topk_matches_lexsort(rng, n, k):
    s = rng.integers(-20, 20, n).astype(np.float32) * 0.5    # many ties
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))
    want = np.sort(order[:min(k, n)])
    got = oracle.topk(s, k)
    assert np.array_equal(got[:len(want)], want) and np.all(got[len(want):] == -1)


def test_topk_k1_is_first_argmax(rng):
    s = rng.integers(0, 5, 300).astype(np.float32)
    assert oracle.topk(s, 1)[0] == np.argmax(s)


def test_topk_all_equal_and_k_ge_n():
    assert list(oracle.topk(np.full(10, 2.5, np.float32), 4)) == [0, 1, 2, 3]
    assert list(oracle.topk(np.array([3, 1, 2], np.float32), 5)) == [0, 1, 2, -1, -1]
    assert list(oracle.topk(np.zeros(0, np.float32), 3)) == [-1, -1, -1]


def test_topk_signed_zero_ties():
    assert list(oracle.topk(np.array([-0.0, 0.0, -0.0, -1.0], np.float32), 2)) == [0, 1]


def test_topk_invariant_under_increasing_map(rng):
    s = rng.standard_normal(2000).astype(np.float32)
    t = np.exp(s.astype(np.float64)).astype(np.float32)
    assert np.array_equal(oracle.topk(s, 100), oracle.topk(t, 100))


def test_topk_permutation_equivariance(rng):
    s = rng.permutation(5000).astype(np.float32)
    p = rng.permutation(5000)
    a = oracle.topk(s, 300)
    b = oracle.topk(s[p], 300)
    assert np.array_equal(np.sort(p[b]), a)


def test_topk_rejects_nan():
    with pytest.raises(ValueError):
        oracle.topk(np.array([1.0, np.nan], np.float32), 1)


def test_topk_fraction_matches_pages():
    g = _golden()
    n, k = int(g["c4_candidates"]), int(g["c4_topk"])
    sel = oracle.topk(np.arange(n, dtype=np.float32), k)
    assert np.array_equal(sel, np.arange(n - k, n))
    assert round(100.0 * k / n, 1) == g["c4_touched_percent"]


# ------------------------------------------------------------------ attention
def test_attend_single_key(rng):
    q = rng.standard_normal((3, 8)).astype(np.float32)
    k = rng.standard_normal((1, 8)).astype(np.float32)
    o, lse = oracle.attend(q, k, 0.3)
    np.testing.assert_allclose(o, np.repeat(k.astype(np.float64), 3, 0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q.astype(np.float64) @ k[0].astype(np.float64)), rtol=1e-13)


def test_attend_identical_keys(rng):
    q = rng.standard_normal((2, 6)).astype(np.float32)
    k = rng.standard_normal((1, 6)).astype(np.float32)
    o, lse = oracle.attend(q, np.repeat(k, 9, 0), 0.5)
    np.testing.assert_allclose(o, np.repeat(k.astype(np.float64), 2, 0), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q.astype(np.float64) @ k[0]) + np.log(9.0), rtol=1e-13)


def test_attend_zero_query_is_mean(rng):
    keys = rng.standard_normal((13, 5)).astype(np.float32)
    o, lse = oracle.attend(np.zeros((2, 5), np.float32), keys, 1.0)
    np.testing.assert_allclose(o, np.repeat(keys.astype(np.float64).mean(0, keepdims=True), 2, 0),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(13.0), rtol=1e-14)


def test_attend_two_keys_logistic(rng):
    q = rng.standard_normal((4, 7)).astype(np.float32)
    keys = rng.standard_normal((2, 7)).astype(np.float32)
    sc = 1 / np.sqrt(7)
    o, lse = oracle.attend(q, keys, sc)
    l = sc * (q.astype(np.float64) @ keys.astype(np.float64).T)
    p0 = expit(l[:, 0] - l[:, 1])
    want = p0[:, None] * keys[0] + (1 - p0)[:, None] * keys[1]
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, logsumexp(l, axis=1), rtol=1e-13)


def test_attend_lse_merge_identity(rng):
    # Attention over A u B equals the LSE-weighted merge of attention over A and over B.
    q = rng.standard_normal((5, 16)).astype(np.float32)
    keys = rng.standard_normal((40, 16)).astype(np.float32)
    o, lse = oracle.attend(q, keys, 0.25)
    oa, la = oracle.attend(q, keys[:17], 0.25)
    ob, lb = oracle.attend(q, keys[17:], 0.25)
    L = np.logaddexp(la, lb)
    np.testing.assert_allclose(lse, L, rtol=1e-13)
    np.testing.assert_allclose(o, np.exp(la - L)[:, None] * oa + np.exp(lb - L)[:, None] * ob,
                               rtol=1e-11, atol=1e-13)


def test_attend_key_order_invariance(rng):
    q = rng.standard_normal((3, 8)).astype(np.float32)
    keys = rng.standard_normal((30, 8)).astype(np.float32)
    o1, l1 = oracle.attend(q, keys, 0.35)
    o2, l2 = oracle.attend(q, keys[rng.permutation(30)], 0.35)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_attend_large_logits_pick_argmax(rng):
    q = rng.standard_normal((2, 8)).astype(np.float32) * 1000
    keys = rng.standard_normal((6, 8)).astype(np.float32)
    o, lse = oracle.attend(q, keys, 1.0)
    l = q.astype(np.float64) @ keys.astype(np.float64).T
    np.testing.assert_allclose(o, keys[np.argmax(l, 1)].astype(np.float64), rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_attend_no_keys():
    o, lse = oracle.attend(np.ones((2, 4), np.float32), np.zeros((0, 4), np.float32), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------------------------ the decode step's key set
def test_step_full_selection_equals_dense(rng):
    # k >= number of candidates: the sparse step over all indices equals the dense step.
    X = rng.standard_normal((300, 8)).astype(np.float32)
    comp = rng.standard_normal((75, 8)).astype(np.float32)
    q = rng.standard_normal((4, 8)).astype(np.float32)
    sel = oracle.topk(rng.standard_normal(75).astype(np.float32), 100)   # all 75, padded with -1
    o1, l1 = oracle.decode_step(q, X, 128, comp, sel, 0.3)
    o2, l2 = oracle.decode_step(q, X, 128, comp, None, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_step_window_is_last_w_tokens(rng):
    X = rng.standard_normal((200, 4)).astype(np.float32)
    keys = oracle.step_keys(oracle.window_rows(X, 128), np.zeros((0, 4), np.float32), None)
    assert np.array_equal(keys, X[72:])
    short = X[:50]
    assert np.array_equal(oracle.window_rows(short, 128), short)     # N < W: every token


def test_step_skips_invalid_indices_and_keeps_duplicates(rng):
    win = rng.standard_normal((3, 4)).astype(np.float32)
    comp = rng.standard_normal((5, 4)).astype(np.float32)
    keys = oracle.step_keys(win, comp, np.array([4, -1, 7, 1, 1, 5]))
    assert np.array_equal(keys, np.concatenate([win, comp[[4, 1, 1]]]))
    assert oracle.step_keys(win, np.zeros((0, 4), np.float32), np.array([-1, -1])).shape == (3, 4)


def test_step_c128_reads_every_entry_at_1m():
    g = _golden()
    n, m, W = int(g["context_tokens"]), int(g["c128_ratio"]), int(g["window_tokens"])
    comp = np.zeros((n // m, 2), np.float32)
    keys = oracle.step_keys(np.zeros((W, 2), np.float32), comp, None)
    assert keys.shape[0] == W + 8192


# ------------------------------------------------------------------ per-step append (state ring)
@pytest.mark.parametrize("R", [1, 3, 4, 8])
def test_ring_image_closed_form(R):
    # Token t writes t + 1 into slot t mod R. Slot s < N then holds the last such token:
    # s + R * floor((N - 1 - s) / R), plus one; slots s >= N were never written.
    for N in range(0, 3 * R + 3):
        img, written = oracle.ring_image((np.arange(N, dtype=np.float32) + 1)[:, None], R)
        for s in range(R):
            if s < N:
                assert written[s] and img[s, 0] == s + R * ((N - 1 - s) // R) + 1, (N, R, s)
            else:
                assert not written[s] and img[s, 0] == 0, (N, R, s)


def test_ring_image_short_history_is_the_history(rng):
    X = rng.standard_normal((5, 3)).astype(np.float32)
    img, written = oracle.ring_image(X, 8)
    assert np.array_equal(img[:5], X) and written.tolist() == [True] * 5 + [False] * 3


@pytest.mark.parametrize("N", [0, 1, 50, 127, 128, 129, 300, 1000])
def test_window_ring_holds_the_step_window(rng, N):
    # The written slots of the window ring are, as a set of rows, the decode step's window (the
    # last min(N, W) tokens): attention over a set does not depend on the slot order.
    X = rng.standard_normal((N, 4)).astype(np.float32)
    img, written = oracle.ring_image(X, 128)
    got = img[written]
    want = oracle.window_rows(X, 128)
    assert got.shape == want.shape
    assert np.array_equal(got[np.lexsort(got.T)], want[np.lexsort(want.T)])


@pytest.mark.parametrize("m,W", [(4, 128), (128, 128), (3, 10), (8, 8)])
def test_completed_group_lies_in_the_window_ring(rng, m, W):
    # When a group completes (N a multiple of m) and m <= W, all of its token rows are still in
    # the window ring: an append can read the group's rows there.
    X = rng.standard_normal((5 * W, 2)).astype(np.float32)
    for N in range(m, 5 * W + 1, m):
        img, written = oracle.ring_image(X[:N], W)
        for t in range(N - m, N):
            assert written[t % W] and np.array_equal(img[t % W], X[t]), (N, t)


def test_append_state_counts_and_prefix_stability(rng):
    # One token more changes one window slot, one gate slot, and adds one compressed entry
    # exactly when it completes a group; the entries already there do not change (compress is
    # prefix-stable, the property an append relies on).
    m, W, R, d = 4, 16, 8, 6
    X = rng.standard_normal((70, d)).astype(np.float32)
    Z = rng.standard_normal((70, d)).astype(np.float32) * 2
    B = rng.standard_normal((m, d)).astype(np.float32) * 0.1
    prev = oracle.append_state(X[:0], Z[:0], B, m, W, R)
    assert prev["comp"].shape == (0, d) and prev["n"] == 0 and prev["swa_len"] == 0
    for N in range(1, 71):
        cur = oracle.append_state(X[:N], Z[:N], B, m, W, R)
        assert cur["n"] == N and cur["swa_len"] == min(N, W) and cur["comp_count"] == N // m
        assert cur["comp"].shape[0] == N // m
        assert np.array_equal(cur["comp"][:prev["comp"].shape[0]], prev["comp"])
        diff_w = np.flatnonzero(np.any(cur["swa"] != prev["swa"], axis=1) | (cur["swa_written"] != prev["swa_written"]))
        diff_g = np.flatnonzero(np.any(cur["gate"] != prev["gate"], axis=1) | (cur["gate_written"] != prev["gate_written"]))
        assert set(diff_w) <= {(N - 1) % W} and set(diff_g) <= {(N - 1) % R}
        if N % m == 0:   # the new entry is the pool of the last m tokens alone
            g = X[N - m:N].astype(np.float64)
            a = Z[N - m:N].astype(np.float64) + B
            w = softmax(a, axis=0)
            np.testing.assert_allclose(cur["comp"][-1], (w * g).sum(0), rtol=1e-12, atol=1e-14)
        prev = cur


# ------------------------------------------------------------------ paged pools
def test_paged_rows_page_size_one_is_a_gather(rng):
    pool = rng.standard_normal((40, 3)).astype(np.float32)
    pt = rng.permutation(40)[:25]
    assert np.array_equal(oracle.paged_rows(pool, pt, 1, 25), np.take(pool, pt, axis=0))


@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_paged_rows_identity_table_is_the_pool_prefix(rng, P):
    pool = rng.standard_normal((256, 2)).astype(np.float32)
    n = 200
    assert np.array_equal(oracle.paged_rows(pool, np.arange(256 // P), P, n), pool[:n])


def test_paged_rows_swapped_half_pages_swap_the_halves(rng):
    pool = rng.standard_normal((64, 5)).astype(np.float32)
    got = oracle.paged_rows(pool, [1, 0], 32, 64)
    assert np.array_equal(got, np.concatenate([pool[32:], pool[:32]]))
    part = oracle.paged_rows(pool, [1, 0], 32, 40)          # a ragged tail reads into the second page
    assert np.array_equal(part, np.concatenate([pool[32:], pool[:8]]))


# ------------------------------------------------------------------ storage rounding
def test_round_bf16_matches_integer_rne_of_fp32_values(rng):
    # For doubles that are exactly fp32 values, rounding to bf16 equals the integer RNE on the
    # fp32 bit pattern (an independent construction of the same rounding).
    x = (rng.standard_normal(20000) * 10).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16).astype(np.uint32).view(np.float32)
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), r)


def test_round_bf16_ties_and_exact():
    one = 1.0
    ulp = 2.0 ** -7
    got = oracle.round_bf16(np.array([one, one + ulp / 2, one + 1.5 * ulp, one + ulp / 2 + 1e-12, 3.0]))
    assert list(got) == [1.0, 1.0, 1.0 + 2 * ulp, 1.0 + ulp, 3.0]
