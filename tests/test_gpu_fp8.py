"""chs_index_topk_fp8 (FP8 E4M3 index keys with per-row scales) against the oracle.

Keys are seeded normals (with the index-key spike of the workloads where noted), quantised per
row on the device: scale = max|k| / 448, code = E4M3(k / scale). That is input preparation, like
the generator; the oracle then decodes the same codes from the format's definition."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import assert_bf16_path, assert_lse, check_swaps, dev
from synth import workloads as W

pytestmark = pytest.mark.gpu

NONNAN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _quantise(keys):
    """Per-row E4M3 codes (uint8) and fp32 scales of fp32/bf16 device keys [n, dim]."""
    k = keys.float()
    scale = (k.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
    codes = (k / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _run(q, w, codes, scale, lens, k):
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev())
    scores = torch.empty(max(int(sum(lens)), 1), dtype=torch.float32, device=dev())[:int(sum(lens))]
    topk, _ = chs.index_topk_fp8(q, w, codes, scale, cu, k, max(lens) if lens else 0, scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), topk.cpu().numpy(), cu.cpu().numpy()


@pytest.mark.parametrize("dim", [16, 128, 512])
def test_fp8_every_code_at_every_byte_is_exact(dim):
    # Heads e_t and -e_t with weights 1 and 2 read element t alone: s = c d (d > 0) or 2 c |d|,
    # one fp32 rounding of an exact product, so the GPU must match the oracle bit for bit.
    print(f"case: fp8 codes, dim {dim}", flush=True)
    rng = np.random.default_rng(dim)
    n = 2 * len(NONNAN)
    K8 = np.stack([np.roll(np.resize(NONNAN, n + dim), r)[:dim] for r in range(n)]).astype(np.uint8)
    scale = rng.uniform(0.5, 2.0, n).astype(np.float32)
    codes = torch.from_numpy(K8).to(dev())
    sc = torch.from_numpy(scale).to(dev())
    w = torch.tensor([[1.0, 2.0]], dtype=torch.float32, device=dev())
    for t in sorted({0, 1, 2, 3, 4, 7, 8, 15, dim // 2, dim - 1}):
        qh = np.zeros((2, dim), np.float32)
        qh[0, t], qh[1, t] = 1.0, -1.0
        q = torch.from_numpy(qh).to(dev()).bfloat16().reshape(1, 2, dim)
        s, _, _ = _run(q, w, codes, sc, [n], 64)
        want = oracle.index_scores_fp8(qh, np.array([1.0, 2.0], np.float32), K8, scale).astype(np.float32)
        assert np.array_equal(s, want), f"t={t}: {np.flatnonzero(s != want)[:8]}"


@pytest.mark.parametrize("nh,dim,lens,k", [
    (4, 128, [5000], 512),
    (4, 128, [1000, 0, 7000, 3], 512),
    (1, 16, [3000], 64),
    (16, 64, [2500], 100),
    (2, 512, [1777], 300),
    (8, 32, [900, 64], 1000),
])
def test_fp8_scores_and_topk_match_oracle(nh, dim, lens, k):
    print(f"case: fp8 nh={nh} dim={dim} lens={lens} k={k}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(nh * 1000 + dim)
    G = int(sum(lens))
    keys = torch.randn(max(G, 1), dim, generator=g, device=dev())[:G] * 3
    codes, scale = _quantise(keys)
    q = torch.randn(len(lens), nh, dim, generator=g, device=dev()).bfloat16()
    w = torch.rand(len(lens), nh, generator=g, device=dev())
    s, t, cu = _run(q, w, codes, scale, lens, k)
    qf, wf, K8, sf = q.float().cpu().numpy(), w.cpu().numpy(), codes.cpu().numpy(), scale.cpu().numpy()
    for b in range(len(lens)):
        lo, hi = cu[b], cu[b + 1]
        ref = oracle.index_scores_fp8(qf[b], wf[b], K8[lo:hi], sf[lo:hi])
        got = s[lo:hi]
        if hi > lo:
            assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max()), f"scores seq {b}"
        assert np.array_equal(t[b], oracle.topk(got, k)), f"top-k seq {b}"
        check_swaps(t[b], oracle.topk(ref.astype(np.float32), k), ref, k)


def test_fp8_workload4_size():
    # The 1M-context candidate count with the workload's spiked index keys, quantised.
    wl = W.workload(4)
    layer = wl.layers[0]
    print("case: fp8 keys, 262144 candidates", flush=True)
    inp = W.device_inputs(wl, layer, dev(), with_tokens=False)
    codes, scale = _quantise(inp["k_idx"])
    G = codes.shape[0]
    s, t, _ = _run(inp["q_idx"], inp["w"], codes, scale, [G], layer.k)
    ref = oracle.index_scores_fp8(inp["q_idx"].float().cpu().numpy()[0], inp["w"].cpu().numpy()[0],
                                  codes.cpu().numpy(), scale.cpu().numpy())
    assert np.all(np.abs(s - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    assert np.array_equal(t[0], oracle.topk(s, layer.k))
    swaps = check_swaps(t[0], oracle.topk(ref.astype(np.float32), layer.k), ref, layer.k)
    print(f"  {swaps} legitimate swaps at the threshold", flush=True)


# ---------------------------------------------------------------- FP8 KV cache (attention)
def _codes_rows(rng, n, d, spread=1.0):
    """Seeded rows quantised per row: E4M3 codes (uint8 [n, d]) and fp32 scales [n]. Values are
    N(0, spread^2), the workloads' range: the bf16-path tolerance allows one bf16 rounding of P,
    whose effect on the output grows with |V| (about 2^-9 |V| for a dominant key)."""
    k = torch.from_numpy((rng.standard_normal((max(n, 1), d)) * spread).astype(np.float32))[:n]
    scale = (k.abs().amax(dim=1) / 448.0).clamp_min(1e-30) if n else torch.zeros(0)
    codes = (k / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8) if n else torch.zeros(0, d, dtype=torch.uint8)
    return codes.numpy(), scale.numpy().astype(np.float32)


@pytest.mark.parametrize("H,d,W,swa_lens,G_list,k,dense", [
    (64, 512, 128, [128], [3000], 512, False),
    (64, 512, 128, [128, 40, 0], [700, 0, 2500], 96, False),
    (8, 128, 64, [64, 13], [900, 333], 64, False),
    (100, 256, 128, [77], [1500], 200, False),
    (16, 64, 32, [32, 32], [400, 1200], 0, True),
    (64, 512, 128, [128, 128], [2048, 1000], 0, True),
    (100, 256, 128, [128, 9], [3000, 500], 0, True),
])
def test_fp8_attention_matches_oracle(H, d, W, swa_lens, G_list, k, dense):
    print(f"case: fp8 attention H={H} d={d} W={W} G={G_list} k={k} dense={dense}", flush=True)
    rng = np.random.default_rng(H * 7 + d + W)
    B = len(G_list)
    q = (rng.standard_normal((B, H, d))).astype(np.float32)
    qb = torch.from_numpy(q).bfloat16()
    qf = qb.float().numpy()
    swa_c, swa_s = _codes_rows(rng, B * W, d)
    swa_c, swa_s = swa_c.reshape(B, W, d), swa_s.reshape(B, W)
    comp_c, comp_s = _codes_rows(rng, sum(G_list), d)
    cu = np.concatenate([[0], np.cumsum(G_list)]).astype(np.int64)
    topk = None
    if not dense:
        topk = np.full((B, k), -1, np.int32)
        for b, G in enumerate(G_list):
            sel = rng.integers(0, max(G, 1), k) if G else np.full(k, -1)
            bad = rng.choice(k, min(5, k), replace=False)
            sel[bad] = rng.choice([-1, -7, G, G + 9], len(bad))
            topk[b] = sel
    t = lambda x, dt=None: torch.from_numpy(np.ascontiguousarray(x)).to(dev()) if dt is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev(), dt)
    comp_dev = t(comp_c) if comp_c.size else torch.zeros(1, d, dtype=torch.uint8, device=dev())
    comp_s_dev = t(comp_s) if comp_s.size else torch.zeros(1, dtype=torch.float32, device=dev())
    out, lse = chs.decode_attn_fp8(qb.to(dev()), t(swa_c), t(swa_s), t(np.array(swa_lens, np.int32)), comp_dev,
                                   comp_s_dev, t(cu), None if dense else t(topk), d ** -0.5, max(G_list))
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        nswa = min(max(swa_lens[b], 0), W)
        lo, hi = cu[b], cu[b + 1]
        rows = list(range(lo, hi)) if dense else [lo + int(j) for j in topk[b] if 0 <= j < hi - lo]
        codes = np.concatenate([swa_c[b, :nswa], comp_c[rows].reshape(-1, d)])
        scales = np.concatenate([swa_s[b, :nswa], comp_s[rows]]).astype(np.float32)
        o_ref, l_ref = oracle.attend_fp8(qf[b], codes, scales, d ** -0.5)
        assert_bf16_path(og[b], o_ref, f"fp8 attn b={b}")
        assert_lse(lg[b], l_ref, f"fp8 lse b={b}", 1e-3)


@pytest.mark.parametrize("B,H,d,W,swa,G_list,Hi,dI,k", [
    (1, 64, 512, 128, [128], [20000], 4, 128, 512),                               # one sequence, 16-head workgroups
    (24, 72, 512, 128, [128, 77, 0, 5] * 6, [1500 + 41 * i for i in range(24)], 4, 128, 64),   # 64-head workgroups
    (3, 16, 128, 64, [64, 10, 64], [300, 0, 2000], 2, 64, 32),                   # small heads, an empty sequence
])
def test_fp8_step_matches_the_two_calls(B, H, d, W, swa, G_list, Hi, dI, k):
    # chs_decode_step_fp8 against chs_index_topk_fp8 followed by chs_decode_attn_fp8 on the same inputs:
    # scores, top-k, out and lse bit for bit (the two calls are checked against the oracle above).
    print(f"case: fp8 step B={B} H={H} d={d} G={sum(G_list)} k={k}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(11)
    G = int(sum(G_list))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(G_list)]), dtype=torch.int64, device=dev())
    kc, ks = chs.quantize_e4m3(torch.randn(G, dI, generator=g, device=dev()).bfloat16())
    cc, cs = chs.quantize_e4m3(torch.randn(G, d, generator=g, device=dev()).bfloat16())
    sc, ss = chs.quantize_e4m3(torch.randn(B * W, d, generator=g, device=dev()).bfloat16())
    sc, ss = sc.view(B, W, d), ss.view(B, W)
    qi = torch.randn(B, Hi, dI, generator=g, device=dev()).bfloat16()
    w = torch.rand(B, Hi, generator=g, device=dev())
    q = torch.randn(B, H, d, generator=g, device=dev()).bfloat16()
    sl = torch.tensor(swa, dtype=torch.int32, device=dev())
    mx = max(G_list)
    s1 = torch.empty(G, dtype=torch.float32, device=dev())
    s2 = torch.empty(G, dtype=torch.float32, device=dev())
    tk1, _ = chs.index_topk_fp8(qi, w, kc, ks, cu, k, mx, s1)
    o1, l1 = chs.decode_attn_fp8(q, sc, ss, sl, cc, cs, cu, tk1, None, mx)
    tk2, o2, l2, _ = chs.decode_step_fp8(qi, w, kc, ks, q, sc, ss, sl, cc, cs, cu, k, None, mx, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2), "scores differ"
    assert torch.equal(tk1, tk2), "top-k differs"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "out differs"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs"
