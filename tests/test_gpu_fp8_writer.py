"""The FP8 (E4M3) writers through the C ABI against the oracle's quantiser (oracle.quantize_e4m3,
pinned against torch's float8_e4m3fn cast and closed forms):

- chs_quantize_e4m3: codes and scales bit-exact to the oracle's on the same rows (bf16 and fp32,
  widths from 8 to 4096, zero rows, rows whose scale is a power of two so that the scaled values
  land on E4M3 midpoints (ties) and in the subnormal range);
- chs_compress_fp8: m = 1 pools each token to itself, so codes and scales are bit-exact to the
  oracle's quantisation of the token rows; for other m the entries match the oracle's compressor
  followed by its quantiser within the fp32 pooling error (scales to 1e-5 relative, dequantised
  values within half an E4M3 step plus that error), and for fp32 storage they are bit-identical to
  chs_quantize_e4m3 of chs_compress's fp32 output (the same pooled values);
- chs_append_fp8: over decode-time appends, the window's codes and scales bit-exact to the oracle's
  quantisation of the token rows, the state rings exact copies, entries as for chs_compress_fp8
  (bit-identical to chs_compress_fp8 over the same history for m in {1, 2, 4, 8}), counters exact.

Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (attention kept in FP8); "SGLang 如何为
DeepSeek V4 打造「Day-0」推理加速", 4.3 部署配置建议 (an fp8 KV cache)."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
import synth
from chs_testutil import dev

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _t(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev()).to(dt)


def _round(a, dtype):
    a = np.asarray(a, np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy() if dtype == "bf16" else a


def _grid():
    return torch.from_numpy(np.arange(0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _rows(rng, n, d, dtype):
    x = rng.standard_normal((n, d)) * np.exp2(rng.uniform(-20, 20, (n, 1)))
    if n > 1:
        x[1] = 0.0                                              # a zero row: scale 0, codes 0
    if n > 3:
        # Ties: a row whose maximum is 448 * 2^k has the exact scale 2^k, so values placed on E4M3
        # midpoints (and in the subnormal range) stay there after the division.
        g = _grid()
        mids = (g[:-1] + g[1:]) / 2
        k = 3
        row = rng.choice(np.concatenate([mids, g, -mids]), d)
        row[0] = 448.0
        x[2] = row * 2.0 ** k
        x[3] = rng.choice(mids[:12], d) * 2.0 ** -5              # deep in the subnormal range
        x[3, 0] = 448.0 * 2.0 ** -5
    return _round(x, dtype)


@pytest.mark.parametrize("dtype,n,d", [("bf16", 257, 128), ("bf16", 64, 512), ("bf16", 33, 8), ("bf16", 17, 136),
                                       ("bf16", 9, 4096), ("f32", 100, 64), ("f32", 21, 520), ("f32", 5, 1024),
                                       ("bf16", 4000, 64), ("bf16", 70, 256), ("f32", 77, 256), ("bf16", 45, 512),
                                       ("f32", 3, 128), ("bf16", 1, 64), ("f32", 1, 512), ("bf16", 256, 64)])
def test_quantize_bit_exact(rng, dtype, n, d):
    print(f"case: quantize_e4m3 {dtype} n={n} d={d}", flush=True)
    x = _rows(rng, n, d, dtype)
    codes, scales = chs.quantize_e4m3(_t(x, TD[dtype]))
    want_c, want_s = oracle.quantize_e4m3(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "scales differ"
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: {got_c[tuple(bad[0])]} vs " \
                          f"{want_c[tuple(bad[0])]}"


def _step(v):
    """Half the E4M3 grid spacing at the magnitude of v (values in units of the row scale)."""
    a = np.abs(v)
    return np.where(a >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9) / 2


def _check_entries(codes, scales, want_double, what):
    """Entries quantised from the GPU's fp32 pooled values against the oracle's double ones."""
    codes = np.asarray(codes)
    scales = np.asarray(scales, np.float64)
    want = np.asarray(want_double, np.float64)
    amax = np.abs(want).max(axis=1)
    s_ref = amax / 448.0
    assert np.all(np.abs(scales - s_ref) <= 1e-5 * s_ref + 1e-30), f"{what}: scales"
    dec = oracle.decode_e4m3(codes) * scales[:, None]
    nz = s_ref > 0
    y = want[nz] / s_ref[nz, None]
    err = np.abs(dec[nz] - want[nz]) / s_ref[nz, None]
    bound = _step(y) * (1 + 1e-4) + 2e-5 * 448
    worst = np.max(err - bound) if err.size else 0
    assert worst <= 0, f"{what}: dequantised error beyond half a step, worst excess {worst}"
    ref_codes, _ = oracle.quantize_e4m3(want.astype(np.float32))
    assert np.mean(codes == ref_codes) > 0.99, f"{what}: codes agree on {np.mean(codes == ref_codes):.4f}"


COMPRESS_FP8 = [
    ("bf16", 512, 1, [300, 7]),
    ("f32", 64, 1, [100]),
    ("bf16", 512, 4, [5003, 4, 0, 1031]),
    ("bf16", 128, 8, [1601]),
    ("bf16", 512, 128, [4200, 127, 260]),
    ("bf16", 64, 5, [333, 1000]),
    ("f32", 256, 4, [777, 12]),
    ("f32", 128, 130, [1000, 520]),
    ("bf16", 8, 2, [99]),
]


@pytest.mark.parametrize("dtype,d,m,lens", COMPRESS_FP8)
def test_compress_fp8_matches_oracle(dtype, d, m, lens):
    print(f"case: compress_fp8 {dtype} d={d} m={m} lens={lens}", flush=True)
    bf = dtype == "bf16"
    T = sum(lens)
    X = synth.normal(57, 1, 0, T * d, 0, 1, bf).reshape(T, d)
    Z = synth.normal(57, 2, 0, T * d, 0, 2, bf).reshape(T, d)
    B = synth.normal(57, 3, 0, m * d, 0, 0.1).reshape(m, d)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cug = np.concatenate([[0], np.cumsum([n // m for n in lens])]).astype(np.int64)
    G = int(cug[-1])
    args = (_t(X, TD[dtype]), _t(Z, TD[dtype]), _t(B, torch.float32), m, _t(cu, torch.int64), _t(cug, torch.int64))
    # Guard rows past the packed output stay untouched.
    codes = torch.full((G + 4, d), 0x5A, dtype=torch.uint8, device=dev())
    scales = torch.full((G + 4,), -1.0, dtype=torch.float32, device=dev())
    chs.compress_fp8(*args, max(max(n // m for n in lens), 1), codes, scales)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(gc[G:] == 0x5A) and np.all(gs[G:] == -1.0), "rows past the output were written"
    gc, gs = gc[:G], gs[:G]
    if m == 1:
        wc, ws = oracle.quantize_e4m3(X)
        assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32)) and np.array_equal(gc, wc), "m = 1: not exact"
    want = oracle.compress(X, Z, B, m, cu)
    _check_entries(gc, gs, want, f"compress_fp8 {dtype} m={m}")
    if dtype == "f32":
        pooled = chs.compress(*args)
        qc, qs = chs.quantize_e4m3(pooled)
        assert torch.equal(qc, codes[:G]) and torch.equal(qs, scales[:G]), "not the quantised fp32 compressor output"


APPEND_FP8 = [
    # dtype, d, m, W, R, n0 per sequence, steps
    ("bf16", 512, 4, 128, 8, [0, 3, 130, 1001], 22),
    ("bf16", 128, 1, 128, 8, [5, 64], 10),
    ("bf16", 64, 8, 16, 11, [7, 40], 19),
    ("bf16", 512, 128, 128, 128, [120, 255, 0], 140),
    ("f32", 256, 4, 128, 8, [2, 9], 9),
    ("bf16", 128, 16, 32, 19, [33], 40),
]


@pytest.mark.parametrize("dtype,d,m,W,R,n0,steps", APPEND_FP8)
def test_append_fp8_matches_oracle(rng, dtype, d, m, W, R, n0, steps):
    print(f"case: append_fp8 {dtype} d={d} m={m} W={W} R={R} n0={n0} steps={steps}", flush=True)
    bf = dtype == "bf16"
    tdt = TD[dtype]
    Bn = len(n0)
    N = [n + steps for n in n0]
    X = [_round(rng.standard_normal((n, d)), dtype) for n in N]
    Z = [_round(rng.standard_normal((n, d)) * 2, dtype) for n in N]
    bias = rng.standard_normal((m, d)).astype(np.float32) * 0.1
    cap = max(N) // m + 3
    # The state after each sequence's prefill of n0 tokens (the caller's bookkeeping): the window's
    # codes, the two rings, and a sentinel pool.
    swa_c = np.zeros((Bn, W, d), np.uint8)
    swa_s = np.full((Bn, W), -1.0, np.float32)
    xr = np.zeros((Bn * R, d), np.float32)
    zr = np.zeros((Bn * R, d), np.float32)
    for b in range(Bn):
        img, wr = oracle.ring_image(X[b][:n0[b]], W)
        c, s = oracle.quantize_e4m3(img)
        swa_c[b][wr], swa_s[b][wr] = c[wr], s[wr]
        xr[b * R:(b + 1) * R] = oracle.ring_image(X[b][:n0[b]], R)[0]
        zr[b * R:(b + 1) * R] = oracle.ring_image(Z[b][:n0[b]], R)[0]
    t = dict(swa_c=_t(swa_c, torch.uint8), swa_s=_t(swa_s, torch.float32), xr=_t(xr, tdt), zr=_t(zr, tdt),
             page=torch.arange(Bn, dtype=torch.int32, device=dev()),
             cc=torch.full((Bn * cap, d), 0x5A, dtype=torch.uint8, device=dev()),
             cs=torch.full((Bn * cap,), -1.0, dtype=torch.float32, device=dev()),
             start=torch.arange(0, Bn * cap, cap, dtype=torch.int64, device=dev()),
             n=torch.tensor(n0, dtype=torch.int64, device=dev()),
             sl=torch.zeros(Bn, dtype=torch.int32, device=dev()), cnt=torch.zeros(Bn, dtype=torch.int64, device=dev()))
    bias_t = _t(bias, torch.float32)
    for s in range(steps):
        xs = np.stack([X[b][n0[b] + s] for b in range(Bn)])
        zs = np.stack([Z[b][n0[b] + s] for b in range(Bn)])
        chs.append_fp8(_t(xs, tdt), _t(zs, tdt), bias_t, m, t["n"], t["swa_c"], t["swa_s"], t["xr"], t["zr"],
                       t["page"], t["cc"], t["cs"], t["start"], ring_size=R, swa_len=t["sl"], comp_count=t["cnt"])
    torch.cuda.synchronize()
    swa_c, swa_s = t["swa_c"].cpu().numpy(), t["swa_s"].cpu().numpy()
    cc, cs = t["cc"].cpu().numpy(), t["cs"].cpu().numpy()
    xr, zr = t["xr"].float().cpu().numpy(), t["zr"].float().cpu().numpy()
    assert t["n"].cpu().tolist() == N
    assert t["sl"].cpu().tolist() == [min(n, W) for n in N]
    assert t["cnt"].cpu().tolist() == [n // m for n in N]
    for b in range(Bn):
        # The window: every slot written holds the quantised row of its token, bit for bit.
        img, wr = oracle.ring_image(X[b], W)
        c, sc = oracle.quantize_e4m3(img)
        assert np.array_equal(swa_c[b][wr], c[wr]), f"window codes of sequence {b}"
        assert np.array_equal(swa_s[b][wr].view(np.uint32), sc[wr].view(np.uint32)), f"window scales of {b}"
        # The rings: exact copies of the last R tokens' rows and gates.
        for ring, src in ((xr, X[b]), (zr, Z[b])):
            img, wr = oracle.ring_image(src, R)
            assert np.array_equal(ring[b * R:(b + 1) * R][wr], img[wr]), f"ring of sequence {b}"
        # The entries the appends completed: groups n0 // m .. N // m - 1.
        g0, g1 = n0[b] // m, N[b] // m
        rows = slice(b * cap + g0, b * cap + g1)
        assert np.all(cc[b * cap:b * cap + g0] == 0x5A) and np.all(cc[b * cap + g1:(b + 1) * cap] == 0x5A), \
            f"pool rows outside the appended groups of {b} were written"
        if g1 > g0:
            want = oracle.compress(X[b], Z[b], bias, m, np.array([0, N[b]], np.int64))[g0:g1]
            _check_entries(cc[rows], cs[rows], want, f"append_fp8 entries of {b}")
            if m in (1, 2, 4, 8):
                hc, hs = chs.compress_fp8(_t(X[b], tdt), _t(Z[b], tdt), bias_t, m,
                                          torch.tensor([0, N[b]], dtype=torch.int64, device=dev()))
                assert np.array_equal(cc[rows], hc.cpu().numpy()[g0:g1]), f"entries of {b} differ from the prefill's"
                assert np.array_equal(cs[rows].view(np.uint32), hs.cpu().numpy()[g0:g1].view(np.uint32))
