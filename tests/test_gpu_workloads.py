"""The five workloads end to end at their full sizes, through the C ABI, in the launch
configuration the benchmark times: compress -> index scores + top-k -> attention.

Small workloads are compared with the oracle in full. For the large ones the device generates
the inputs and the oracle recomputes sampled outputs one by one from host-regenerated inputs
(the generator is counter-based, so any row can be regenerated alone with identical bits):
sampled compressed entries, the index scores and top-k of sampled sequences, and the attention
of sampled sequences. The top-k of every sequence is checked bit-exact against the oracle's
top-k of the same scores, and against the oracle's own scores under the swap rule."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import (assert_bf16_path, assert_bf16_stored, assert_f32, assert_lse, check_swaps, dev)
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _sample_groups(rng, G, n):
    if G == 0:
        return np.zeros(0, np.int64)
    return np.unique(np.concatenate([[0, G - 1], rng.integers(0, G, n)])).astype(np.int64)


def _oracle_groups(wl, layer, b, groups):
    """Oracle compressed entries (unrounded doubles) of the given groups of sequence b."""
    m = layer.m
    if len(groups) == 0:
        return np.zeros((0, wl.d))
    X = np.concatenate([W.host_tokens(wl, layer, W.T_X, b, g * m, (g + 1) * m) for g in groups])
    Z = np.concatenate([W.host_tokens(wl, layer, W.T_Z, b, g * m, (g + 1) * m) for g in groups])
    return oracle.compress(X, Z, W.host_bias(wl, layer), m, [0, X.shape[0]])


def _check_compress_sampled(wl, layer, comp, rng, seqs, n):
    cug = wl.cu_groups(layer)
    for b in seqs:
        G = int(cug[b + 1] - cug[b])
        pick = _sample_groups(rng, G, n)
        got = comp[torch.from_numpy(cug[b] + pick).to(dev())].float().cpu().numpy()
        want = _oracle_groups(wl, layer, b, pick)
        (assert_bf16_stored if wl.bf16 else assert_f32)(got, want, f"compress seq {b}")


def _window_rows(wl, layer, b):
    n = wl.lengths[b]
    L = min(n, wl.window)
    return W.host_tokens(wl, layer, W.T_X, b, n - L, n)


def _check_attn_c4(wl, layer, q, sel, out, lse, b):
    """Attention of sequence b over the window plus the GPU's selected entries, recomputed by
    the oracle from its own compressed entries."""
    cug = wl.cu_groups(layer)
    G = int(cug[b + 1] - cug[b])
    valid = sel[(sel >= 0) & (sel < G)]
    groups = np.unique(valid)
    rows = oracle.store(_oracle_groups(wl, layer, b, groups), wl.bf16)
    pos = {int(g): i for i, g in enumerate(groups)}
    comp_sel = rows[[pos[int(j)] for j in valid]] if len(valid) else np.zeros((0, wl.d), np.float32)
    keys = oracle.step_keys(_window_rows(wl, layer, b), comp_sel, None)
    o_ref, l_ref = oracle.attend(q[b], keys, wl.d ** -0.5)
    (assert_bf16_path if wl.bf16 else assert_f32)(out[b], o_ref, f"attention seq {b}")
    assert_lse(lse[b], l_ref, f"lse seq {b}", 1e-3 if wl.bf16 else 1e-5)


def _run_c4(wl, layer, rng, score_seqs, attn_seqs, full=False, fused=False):
    """fused: the decode step as one chs_decode_step call instead of chs_index_topk followed by
    chs_decode_attn."""
    print(f"case: workload {wl.index} ({wl.name}) C4 layer{' (chs_decode_step)' if fused else ''}: "
          "generating inputs", flush=True)
    inp = W.device_inputs(wl, layer, dev())
    cug = wl.cu_groups(layer)
    max_g = int((cug[1:] - cug[:-1]).max())
    comp = chs.compress(inp["X"], inp["Z"], inp["bias"], layer.m, inp["cu_tokens"], inp["cu_groups"], max_g)
    scores = torch.empty(max(int(cug[-1]), 1), dtype=torch.float32, device=dev())[:int(cug[-1])]
    if fused:
        topk, out, lse, _ = chs.decode_step(inp["q_idx"], inp["w"], inp["k_idx"], inp["q"], inp["swa_kv"],
                                            inp["swa_len"], comp, inp["cu_groups"], layer.k, wl.d ** -0.5,
                                            max_g, scores)
    else:
        topk, _ = chs.index_topk(inp["q_idx"], inp["w"], inp["k_idx"], inp["cu_groups"], layer.k, max_g, scores)
        out, lse = chs.decode_attn(inp["q"], inp["swa_kv"], inp["swa_len"], comp, inp["cu_groups"], topk,
                                   wl.d ** -0.5, max_g)
    torch.cuda.synchronize()
    print(f"case: workload {wl.index} C4 layer: checking", flush=True)
    del inp["X"], inp["Z"]
    if full:
        X = W.host_all_tokens(wl, layer, W.T_X)
        Z = W.host_all_tokens(wl, layer, W.T_Z)
        want = oracle.compress(X, Z, W.host_bias(wl, layer), layer.m, wl.cu_tokens())
        (assert_bf16_stored if wl.bf16 else assert_f32)(comp.float().cpu().numpy(), want, "compress")
    else:
        _check_compress_sampled(wl, layer, comp, rng, sorted(set(score_seqs) | {0, wl.batch - 1}), 24)
    sg, tg = scores.cpu().numpy(), topk.cpu().numpy()
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    qi, w, q = W.host_qidx(wl, layer), W.host_w(wl, layer), W.host_q(wl, layer)
    for b in range(wl.batch):     # exact top-k of the GPU's own scores, every sequence
        assert np.array_equal(tg[b], oracle.topk(sg[cug[b]:cug[b + 1]], layer.k)), f"top-k seq {b}"
    for b in score_seqs:
        K = W.host_index_keys(wl, layer, b, 0, int(cug[b + 1] - cug[b]))
        s_ref = oracle.index_scores(qi[b], w[b], K)
        s_gpu = sg[cug[b]:cug[b + 1]]
        assert np.all(np.abs(s_gpu - s_ref) <= 1e-5 * np.abs(s_ref) + 1e-6 * np.abs(s_ref).max()), f"scores {b}"
        swaps = check_swaps(tg[b], oracle.topk(s_ref.astype(np.float32), layer.k), s_ref, layer.k)
        print(f"  seq {b}: scores ok, {swaps} legitimate swaps at the threshold", flush=True)
    for b in attn_seqs:
        _check_attn_c4(wl, layer, q, tg[b], og, lg, b)
    return tg


def _run_c128(wl, layer, rng, attn_seqs):
    print(f"case: workload {wl.index} ({wl.name}) C128 layer: generating inputs", flush=True)
    inp = W.device_inputs(wl, layer, dev(), with_index=False)
    cug = wl.cu_groups(layer)
    max_g = int((cug[1:] - cug[:-1]).max())
    comp = chs.compress(inp["X"], inp["Z"], inp["bias"], layer.m, inp["cu_tokens"], inp["cu_groups"], max_g)
    out, lse = chs.decode_attn(inp["q"], inp["swa_kv"], inp["swa_len"], comp, inp["cu_groups"], None,
                               wl.d ** -0.5, max_g)
    torch.cuda.synchronize()
    del inp["X"], inp["Z"]
    print(f"case: workload {wl.index} C128 layer: checking", flush=True)
    _check_compress_sampled(wl, layer, comp, rng, sorted({0, wl.batch // 2, wl.batch - 1}), 24)
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    q = W.host_q(wl, layer)
    cu = wl.cu_tokens()
    for b in attn_seqs:
        n = wl.lengths[b]
        X = W.host_tokens(wl, layer, W.T_X, b, 0, n)
        Z = W.host_tokens(wl, layer, W.T_Z, b, 0, n)
        C = oracle.store(oracle.compress(X, Z, W.host_bias(wl, layer), layer.m, [0, n]), wl.bf16)
        del Z
        o_ref, l_ref = oracle.decode_step(q[b], X, wl.window, C, None, wl.d ** -0.5)
        assert_bf16_path(og[b], o_ref, f"dense attention seq {b}")
        assert_lse(lg[b], l_ref, f"lse seq {b}", 1e-3)
        assert cu[b + 1] - cu[b] == n


def test_workload1_tiny_c4_f32():
    wl = W.workload(1)
    _run_c4(wl, wl.layers[0], np.random.default_rng(1), [0], [0], full=True)


def test_workload2_c4_128k_bf16():
    wl = W.workload(2)
    _run_c4(wl, wl.layers[0], np.random.default_rng(2), [0], [0], full=True)


def test_workload2_c4_128k_bf16_fused_step():
    wl = W.workload(2)
    _run_c4(wl, wl.layers[0], np.random.default_rng(2), [0], [0], full=True, fused=True)


def test_workload3_c128_1m_bs4_bf16():
    wl = W.workload(3)
    _run_c128(wl, wl.layers[0], np.random.default_rng(3), [3])


def test_workload4_c4_1m_bf16():
    wl = W.workload(4)
    _run_c4(wl, wl.layers[0], np.random.default_rng(4), [0], [0])


def test_workload4_c4_1m_bf16_fused_step():
    wl = W.workload(4)
    _run_c4(wl, wl.layers[0], np.random.default_rng(4), [0], [0], fused=True)


def test_workload4_standalone_topk():
    wl = W.workload(4)
    n = wl.topk_len
    rows = {v: W.topk_scores(wl, v) for v in ("normal", "dup10", "tie64")}
    cu = torch.tensor([0, n], dtype=torch.int64, device=dev())
    ws = chs.index_topk_workspace(1, n, 512, dev())
    for v, s in rows.items():
        print(f"case: c4_1m_bf16 standalone top-k ({v})", flush=True)
        got = chs.topk_from_scores(torch.from_numpy(s).to(dev()), cu, 512, n, ws).cpu().numpy()[0]
        assert np.array_equal(got, oracle.topk(s, 512)), v
    # The 64-row batch the benchmark times.
    batch = np.stack([W.topk_scores(wl, "normal", r) for r in range(64)])
    cu64 = torch.arange(0, 65 * n, n, dtype=torch.int64, device=dev())
    ws64 = chs.index_topk_workspace(64, n, 512, dev())
    got = chs.topk_from_scores(torch.from_numpy(batch.ravel()).to(dev()), cu64, 512, n, ws64).cpu().numpy()
    for r in range(64):
        assert np.array_equal(got[r], oracle.topk(batch[r], 512)), f"row {r}"


def test_workload5_mixed_bs64():
    wl = W.workload(5)
    rng = np.random.default_rng(5)
    c4, c128 = wl.layers
    _run_c4(wl, c4, rng, [0, 17, 40, 63], [0, 33, 63])
    torch.cuda.empty_cache()
    _run_c4(wl, c4, rng, [9], [9, 50], fused=True)
    torch.cuda.empty_cache()
    _run_c128(wl, c128, rng, [5, 63])
