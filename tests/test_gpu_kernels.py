"""Parity of each libchs call with the CPU oracle at sizes the oracle finishes in seconds that
still span several workgroups and a ragged tail, plus the degenerate cases of the method.
All GPU calls go through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
import synth
from chs_testutil import (assert_bf16_path, assert_bf16_stored, assert_f32, assert_lse, check_swaps, dev)

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _to_dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev()).to(dt)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


# ------------------------------------------------------------------ generator (bit-identity)
def test_device_fillers_match_host_fillers():
    print("case: generator bit identity", flush=True)
    n = 1_000_003
    for dt, bf in [(torch.float32, False), (torch.bfloat16, True)]:
        t = synth.gpu_normal(torch.empty(n, dtype=dt, device=dev()), 4321, 3, 999, 0.0, 2.0)
        h = synth.normal(4321, 3, 999, n, 0.0, 2.0, bf16=bf)
        assert np.array_equal(t.float().cpu().numpy().view(np.uint32), h.view(np.uint32))
    u = synth.gpu_uniform(torch.empty(77777, dtype=torch.float32, device=dev()), 5, 6, 10)
    assert np.array_equal(u.cpu().numpy(), synth.uniform(5, 6, 10, 77777))
    U = synth.spike_basis(9, 9, 4, 128)
    for dt, bf in [(torch.float32, False), (torch.bfloat16, True)]:
        kd = synth.gpu_index_keys(torch.empty(3000, 128, dtype=dt, device=dev()), 9, 7, 8, 500,
                                  torch.from_numpy(U).to(dev()), 8.0)
        kh = synth.index_keys(9, 7, 8, 500, 3000, 128, U, 8.0, bf)
        assert np.array_equal(kd.float().cpu().numpy().view(np.uint32), kh.view(np.uint32))


# ------------------------------------------------------------------ chs_compress
COMPRESS_CASES = [
    # dtype, d, m, lengths
    ("f32", 64, 4, [1024]),
    ("f32", 36, 3, [0, 2, 50, 301]),
    ("f32", 128, 128, [700, 129]),
    ("bf16", 512, 4, [5003, 4, 3, 0, 1031]),
    ("bf16", 512, 128, [4200, 127, 260]),
    ("bf16", 136, 5, [333, 1000]),
    ("bf16", 64, 1, [257]),
    ("bf16", 256, 2, [99, 100]),
    ("bf16", 512, 8, [1601]),
    ("bf16", 128, 130, [1000, 520]),
    ("bf16", 64, 1024, [2100]),
    # d above the LDS-staged bias path's limit: the per-thread bias reads
    ("bf16", 1024, 16, [100, 37]),
    ("f32", 640, 6, [50, 13]),
    ("bf16", 1024, 8, [200, 17]),   # wide rows at a compile-time group size
]


@pytest.mark.parametrize("dtype,d,m,lens", COMPRESS_CASES)
def test_compress_matches_oracle(rng, dtype, d, m, lens):
    print(f"case: compress {dtype} d={d} m={m} lens={lens}", flush=True)
    bf = dtype == "bf16"
    T = sum(lens)
    X = synth.normal(17, 1, 0, T * d, 0, 1, bf).reshape(T, d)
    Z = synth.normal(17, 2, 0, T * d, 0, 2, bf).reshape(T, d)
    B = synth.normal(17, 3, 0, m * d, 0, 0.1).reshape(m, d)
    cu = _cu(lens)
    G = sum(n // m for n in lens)
    cug = _cu([n // m for n in lens])
    # Guard rows after the packed output must stay untouched.
    out = torch.full((G + 8, d), 7.0, dtype=TORCH_DT[dtype], device=dev())
    chs.compress(_to_dev(X, TORCH_DT[dtype]), _to_dev(Z, TORCH_DT[dtype]), _to_dev(B, torch.float32), m,
                 _to_dev(cu, torch.int64), _to_dev(cug, torch.int64), max(n // m for n in lens), out)
    got = out.float().cpu().numpy()
    assert np.all(got[G:] == 7.0)
    want = oracle.compress(X, Z, B, m, cu)
    if bf:
        assert_bf16_stored(got[:G], want, "compress")
    else:
        assert_f32(got[:G], want, "compress")


def test_compress_m1_identity_and_mean_pooling():
    print("case: compress identity / mean", flush=True)
    d, T = 512, 999
    X = synth.normal(5, 1, 0, T * d, 0, 1, True).reshape(T, d)
    Z = synth.normal(5, 2, 0, T * d, 0, 3, True).reshape(T, d)
    xd = _to_dev(X, torch.bfloat16)
    cu = _to_dev(_cu([T]), torch.int64)
    c1 = chs.compress(xd, _to_dev(Z, torch.bfloat16), _to_dev(np.zeros((1, d), np.float32), torch.float32), 1, cu)
    assert torch.equal(c1, xd)                       # m = 1 is the identity, bit for bit
    zc = torch.full((T, d), 0.5, dtype=torch.bfloat16, device=dev())
    bias = torch.full((4, d), -2.0, dtype=torch.float32, device=dev())
    c4 = chs.compress(xd, zc, bias, 4, cu).float().cpu().numpy()
    mean = X[:(T // 4) * 4].astype(np.float64).reshape(-1, 4, d).mean(1)
    assert_bf16_stored(c4, mean, "mean pooling")


@pytest.mark.parametrize("d,m", [(64, 4), (64, 6), (512, 128)])
def test_compress_output_offsets_are_caller_controlled(d, m):
    # cu_groups need not be packed: sequence 1 is written after a gap; sequence 2 has room for 3
    # of its 5 groups, so only its first 3 are written; rows outside stay put. m = 4 runs the
    # compile-time group size, m = 6 and 128 the LDS-staged bias path.
    print(f"case: compress offsets d={d} m={m}", flush=True)
    lens = [10 * m, 6 * m + 1, 5 * m]
    T = sum(lens)
    X = synth.normal(8, 1, 0, T * d, 0, 1, True).reshape(T, d)
    Z = synth.normal(8, 2, 0, T * d, 0, 1, True).reshape(T, d)
    B = synth.normal(8, 3, 0, m * d, 0, 0.5).reshape(m, d)
    cug = np.array([0, 12, 18, 21], np.int64)      # room 12 >= 10 groups, 6 for 6, 3 for 5
    out = torch.full((24, d), 3.0, dtype=torch.bfloat16, device=dev())
    chs.compress(_to_dev(X, torch.bfloat16), _to_dev(Z, torch.bfloat16), _to_dev(B, torch.float32), m,
                 _to_dev(_cu(lens), torch.int64), _to_dev(cug, torch.int64), 10, out)
    got = out.float().cpu().numpy()
    want = oracle.compress(X, Z, B, m, _cu(lens))   # packed: 10 + 6 + 5 rows
    assert_bf16_stored(got[0:10], want[0:10])
    assert np.all(got[10:12] == 3.0) and np.all(got[21:] == 3.0)
    assert_bf16_stored(got[12:18], want[10:16])
    assert_bf16_stored(got[18:21], want[16:19])
    # max_groups = 2: groups 2 and later of every sequence are not computed.
    out2 = torch.full((24, d), 3.0, dtype=torch.bfloat16, device=dev())
    chs.compress(_to_dev(X, torch.bfloat16), _to_dev(Z, torch.bfloat16), _to_dev(B, torch.float32), m,
                 _to_dev(_cu(lens), torch.int64), _to_dev(cug, torch.int64), 2, out2)
    got2 = out2.float().cpu().numpy()
    for row0, src0, room in ((0, 0, 12), (12, 10, 6), (18, 16, 3)):
        assert_bf16_stored(got2[row0:row0 + 2], want[src0:src0 + 2])
        assert np.all(got2[row0 + 2:row0 + room] == 3.0)


# ------------------------------------------------------------------ standalone top-k (exact)
def _run_topk(score_rows, k, reps=2):
    lens = [len(s) for s in score_rows]
    flat = np.concatenate([np.asarray(s, np.float32) for s in score_rows]) if sum(lens) else np.zeros(0, np.float32)
    sd = torch.from_numpy(flat).to(dev()) if flat.size else torch.zeros(1, dtype=torch.float32, device=dev())[:0]
    cu = _to_dev(_cu(lens), torch.int64)
    ws = chs.index_topk_workspace(len(lens), max(lens) if lens else 0, k, dev())
    outs = []
    for _ in range(reps):   # the workspace must come back clean: a second call gives the same set
        outs.append(chs.topk_from_scores(sd, cu, k, max(lens), ws).cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    for b, s in enumerate(score_rows):
        want = oracle.topk(np.asarray(s, np.float32), k)
        assert np.array_equal(outs[0][b], want), f"row {b} (n={len(s)}, k={k})"
    return outs[0]


def test_topk_262144_score_rows_exact():
    from synth import workloads as W
    wl = W.workload(4)
    for variant in ("normal", "dup10", "tie64"):
        print(f"case: top-k 512 of 262144 ({variant})", flush=True)
        _run_topk([W.topk_scores(wl, variant)], 512)


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (511, 512), (512, 512), (513, 512), (4095, 64), (100003, 2048),
                                 (262144, 1), (3000, 7)])
def test_topk_sizes(rng, n, k):
    print(f"case: top-k n={n} k={k}", flush=True)
    _run_topk([rng.standard_normal(n).astype(np.float32)], k)


def test_topk_ties_and_special_values(rng):
    print("case: top-k ties / specials", flush=True)
    rows = [
        np.full(5000, 1.5, np.float32),                                   # all equal: indices 0..k-1
        rng.integers(-3, 3, 20000).astype(np.float32) * 0.25,             # heavy ties in the threshold bin
        np.where(rng.random(3000) < 0.5, -0.0, 0.0).astype(np.float32),   # signed zeros tie
        np.concatenate([rng.standard_normal(1000), [np.inf, -np.inf, 1e30, -1e30, 1e-40, -1e-40]]).astype(np.float32),
        np.zeros(0, np.float32),                                          # empty sequence
        rng.standard_normal(700).astype(np.float32),
    ]
    _run_topk(rows, 512)
    _run_topk(rows, 64)


def test_topk_signed_zero_and_denormal_threshold(rng):
    # The k-th value is 0: +0 and -0 tie (lower index first) and the tiniest negative values
    # sit just below them, so every group holding a zero must be read whole.
    print("case: top-k threshold at signed zero", flush=True)
    n = 40000
    s = -(1.0 + np.abs(rng.standard_normal(n))).astype(np.float32)
    z = rng.choice(n, 400, replace=False)
    s[z[:300]] = np.where(rng.random(300) < 0.5, -0.0, 0.0)
    s[z[300:350]] = -1e-45
    s[z[350:]] = -3e-45
    for k in (1, 150, 300, 320, 360):
        _run_topk([s], k)


def test_topk_large_threshold_bin_global_path(rng):
    # 30000 equal values straddle the threshold, so the final selection runs from global memory.
    print("case: top-k global-memory path", flush=True)
    s = np.concatenate([rng.standard_normal(50000) - 10, np.full(30000, 3.0), rng.standard_normal(300) + 10])
    _run_topk([rng.permutation(s).astype(np.float32)], 512)


def test_topk_batched_varlen(rng):
    print("case: top-k batched", flush=True)
    lens = [0, 1, 600, 50000, 511, 4096, 33333]
    _run_topk([rng.standard_normal(n).astype(np.float32) * 3 for n in lens], 512)


def test_topk_wide_batch_ragged_unaligned(rng):
    # 33 rows of about 200K-262K scores: enough work for the 8-loads-per-lane statistics kernel.
    # Ragged lengths give masked tail waves and row starts that are not 16-byte aligned (the
    # fallback path); heavy ties and signed zeros sit in a few rows.
    print("case: top-k wide batch, ragged and unaligned", flush=True)
    lens = [262144, 262143, 262141, 200000, 200001] + list(rng.integers(200000, 262145, 28))
    rows = []
    for i, n in enumerate(lens):
        r = rng.standard_normal(int(n)).astype(np.float32)
        if i % 7 == 3:
            r = (rng.integers(-4, 4, int(n)) * 0.5).astype(np.float32)
        if i % 11 == 5:
            r[rng.choice(int(n), 2000, replace=False)] = np.where(rng.random(2000) < 0.5, -0.0, 0.0)
            r = np.minimum(r, np.float32(0.0))
        rows.append(r)
    _run_topk(rows, 512, reps=1)


# ------------------------------------------------------------------ index scores + top-k
@pytest.mark.parametrize("dtype,nh,dim,lens,k", [
    ("bf16", 4, 128, [32768], 512),
    ("bf16", 4, 128, [1000, 0, 3, 40000], 512),
    ("bf16", 1, 512, [3000], 64),
    ("bf16", 16, 64, [2500], 100),
    ("bf16", 5, 24, [1500], 10),
    ("bf16", 2, 8, [777], 5),
    ("f32", 2, 32, [256], 64),
    ("f32", 3, 100, [5000, 70], 300),
])
def test_index_topk_matches_oracle(dtype, nh, dim, lens, k):
    print(f"case: index_topk {dtype} nh={nh} dim={dim} lens={lens} k={k}", flush=True)
    bf = dtype == "bf16"
    B, G = len(lens), sum(lens)
    q = synth.normal(31, 5, 0, B * nh * dim, 0, 1, bf).reshape(B, nh, dim)
    w = synth.uniform(31, 6, 0, B * nh).reshape(B, nh)
    U = synth.spike_basis(31, 9, 4, dim)
    K = synth.index_keys(31, 7, 8, 0, G, dim, U, 8.0, bf)
    cu = _cu(lens)
    scores = torch.empty(max(G, 1), dtype=torch.float32, device=dev())[:G]
    topk, _ = chs.index_topk(_to_dev(q, TORCH_DT[dtype]), _to_dev(w, torch.float32), _to_dev(K, TORCH_DT[dtype]),
                             _to_dev(cu, torch.int64), k, scores=scores)
    sg = scores.cpu().numpy()
    tg = topk.cpu().numpy()
    # chs_index_scores runs the same score kernel with no selection: bit-identical scores.
    alone = chs.index_scores(_to_dev(q, TORCH_DT[dtype]), _to_dev(w, torch.float32), _to_dev(K, TORCH_DT[dtype]),
                             _to_dev(cu, torch.int64)).cpu().numpy()
    assert np.array_equal(alone.view(np.uint32), sg.view(np.uint32)), "index_scores differs from index_topk's scores"
    for b in range(B):
        s_ref = oracle.index_scores(q[b], w[b], K[cu[b]:cu[b + 1]])
        s_gpu = sg[cu[b]:cu[b + 1]]
        if s_ref.size:
            err = np.abs(s_gpu - s_ref)
            assert np.all(err <= 1e-5 * np.abs(s_ref) + 1e-6 * np.abs(s_ref).max()), f"scores b={b}"
        assert np.array_equal(tg[b], oracle.topk(s_gpu, k))                 # exact given the same scores
        check_swaps(tg[b], oracle.topk(s_ref.astype(np.float32), k), s_ref, k)


# ------------------------------------------------------------------ decode attention
def _attn_case(rng, dtype, B, H, d, W, swa_lens, G_list, k, dense, n_bad=0, scale=None):
    bf = dtype == "bf16"
    q = synth.normal(77, 4, 0, B * H * d, 0, 1, bf).reshape(B, H, d)
    swa = synth.normal(77, 1, 0, B * W * d, 0, 1, bf).reshape(B, W, d)
    Gt = sum(G_list)
    # At least one row is allocated so the buffer pointer is never NULL; cu_comp says how many count.
    comp = (synth.normal(77, 20, 0, max(Gt, 1) * d, 0, 0.5, bf)).reshape(max(Gt, 1), d)
    cu = _cu(G_list)
    topk = None
    if not dense:
        topk = np.full((B, k), -1, np.int32)
        for b, G in enumerate(G_list):
            sel = rng.integers(0, max(G, 1), k) if G else np.full(k, -1)
            if n_bad:
                bad = rng.choice(k, n_bad, replace=False)
                sel[bad] = rng.choice([-1, -5, G, G + 100], n_bad)
            topk[b] = sel
    sc = scale if scale is not None else d ** -0.5
    out, lse = chs.decode_attn(_to_dev(q, TORCH_DT[dtype]), _to_dev(swa, TORCH_DT[dtype]),
                               _to_dev(np.array(swa_lens, np.int32), torch.int32),
                               _to_dev(comp, TORCH_DT[dtype]), _to_dev(cu, torch.int64),
                               None if dense else _to_dev(topk, torch.int32), sc)
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        keys = oracle.step_keys(swa[b, :min(max(swa_lens[b], 0), W)], comp[cu[b]:cu[b + 1]],
                                None if dense else topk[b])
        o_ref, l_ref = oracle.attend(q[b], keys, sc)
        if bf:
            assert_bf16_path(og[b], o_ref, f"attn b={b}")
        else:
            assert_f32(og[b], o_ref, f"attn b={b}")
        assert_lse(lg[b], l_ref, f"lse b={b}", 1e-3 if bf else 1e-5)
    return og, lg


@pytest.mark.parametrize("H", [64, 16, 8, 100, 128])
def test_attn_c4_bf16_heads(rng, H):
    print(f"case: attn c4 bf16 H={H}", flush=True)
    _attn_case(rng, "bf16", 2, H, 512, 128, [128, 77], [3000, 40], 512, False, n_bad=9)


def test_attn_c4_bf16_many_sequences(rng):
    # Enough sequences that the 16-head workgroups would outnumber the CUs: the selected entries go
    # through the 64-head d = 512 kernel (its second head group partly past H), with invalid and
    # duplicate indices, ragged and empty windows, and an empty sequence.
    print("case: attn c4 bf16 many sequences", flush=True)
    G = [500 + 41 * i for i in range(23)] + [0]
    _attn_case(rng, "bf16", 24, 72, 512, 128, [128, 77, 0, 5] * 6, G, 64, False, n_bad=9)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_attn_dense_bf16_dims(rng, d):
    print(f"case: attn dense bf16 d={d}", flush=True)
    _attn_case(rng, "bf16", 3, 64, d, 128, [128, 5, 0], [1000, 1, 2100], 0, True)


@pytest.mark.parametrize("H,d", [(72, 512), (100, 128), (128, 256)])
def test_attn_dense_bf16_many_heads(rng, H, d):
    # More than 64 heads: a second 64-head workgroup whose last heads are masked; several chunks
    # per split.
    print(f"case: attn dense bf16 H={H} d={d}", flush=True)
    _attn_case(rng, "bf16", 2, H, d, 128, [128, 50], [4000, 700], 0, True)


@pytest.mark.parametrize("B,L", [(1, 8192), (2, 5000), (6, 6000), (8, 6000), (12, 4000), (4, 8704)])
def test_attn_dense512_split_counts(rng, B, L):
    # Dense d = 512 over 64 heads at batch sizes whose split plans reach every many-split merge form:
    # 130 and 81 splits (the merge sized to 512 splits), 32, 24, 13 and 46 splits (8, 6, 4 and 12
    # partial loads per lane). Sequence lengths vary around L, windows are ragged.
    print(f"case: attn dense d=512 B={B} L={L}", flush=True)
    G = [L - 37 * i for i in range(B)]
    _attn_case(rng, "bf16", B, 64, 512, 128, [(128, 100, 0, 31)[i % 4] for i in range(B)], G, 0, True)


def test_attn_f32(rng):
    print("case: attn f32", flush=True)
    _attn_case(rng, "f32", 2, 8, 64, 128, [128, 30], [256, 300], 64, False, n_bad=3)
    _attn_case(rng, "f32", 2, 3, 36, 16, [16, 0], [700, 5], 0, True)
    _attn_case(rng, "f32", 1, 2, 1024, 8, [8], [40], 16, False)


def test_attn_degenerate(rng):
    print("case: attn degenerate", flush=True)
    # No keys at all: out = 0, lse = -inf.
    og, lg = _attn_case(rng, "bf16", 2, 16, 64, 128, [0, 0], [0, 0], 8, False)
    assert np.all(og == 0) and np.all(np.isneginf(lg))
    # Window only (no compressed entries).
    _attn_case(rng, "bf16", 1, 64, 512, 128, [100], [0], 0, True)
    # A single key: out equals it.
    og, _ = _attn_case(rng, "bf16", 1, 64, 512, 4, [1], [0], 0, True)
    # Window longer than the window buffer is clamped to it.
    _attn_case(rng, "bf16", 1, 64, 128, 32, [500], [64], 16, False)


def test_attn_sparse_with_every_index_equals_dense(rng):
    # Selecting every entry reduces the sparse call to the dense one. The two calls run different
    # kernels whose splits and chunks differ, so P is rounded to bf16 against different running
    # maxima: both meet the bf16-path tolerance against the oracle, and each other within it.
    print("case: attn sparse == dense", flush=True)
    d, H, G = 512, 64, 300
    q = torch.from_numpy(synth.normal(3, 4, 0, H * d, 0, 1, True).reshape(1, H, d)).to(dev()).bfloat16()
    swa = torch.from_numpy(synth.normal(3, 1, 0, 128 * d, 0, 1, True).reshape(1, 128, d)).to(dev()).bfloat16()
    comp = torch.from_numpy(synth.normal(3, 2, 0, G * d, 0, 1, True).reshape(G, d)).to(dev()).bfloat16()
    sl = torch.tensor([128], dtype=torch.int32, device=dev())
    cu = torch.tensor([0, G], dtype=torch.int64, device=dev())
    sel = torch.full((1, 512), -1, dtype=torch.int32, device=dev())
    sel[0, :G] = torch.arange(G, dtype=torch.int32, device=dev())
    o1, l1 = chs.decode_attn(q, swa, sl, comp, cu, sel)
    o2, l2 = chs.decode_attn(q, swa, sl, comp, cu, None)
    keys = np.concatenate([swa[0].float().cpu().numpy(), comp.float().cpu().numpy()])
    o_ref, l_ref = oracle.attend(q[0].float().cpu().numpy(), keys, d ** -0.5)
    for o, l, what in ((o1, l1, "sparse"), (o2, l2, "dense")):
        assert_bf16_path(o[0].cpu().numpy(), o_ref, what)
        assert_lse(l[0].cpu().numpy(), l_ref, what)
    assert_bf16_path(o1.cpu().numpy(), o2.cpu().numpy(), "sparse vs dense")
    assert_lse(l1.cpu().numpy(), l2.cpu().numpy(), "sparse vs dense lse")


def test_attn_is_deterministic():
    # No float atomics on the output path: identical inputs give bitwise identical results.
    print("case: attn determinism", flush=True)
    a = _attn_case(np.random.default_rng(5), "bf16", 2, 64, 512, 128, [128, 128], [5000, 800], 512, False)
    b = _attn_case(np.random.default_rng(5), "bf16", 2, 64, 512, 128, [128, 128], [5000, 800], 512, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
