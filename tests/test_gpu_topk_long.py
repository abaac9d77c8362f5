"""Exact top-k past one pass of the selection block: rows of more than 8192 groups of candidates
(more than 262,144 scores at 32 per group, more than 65,536 at 8 per group for the widest keys).
The selection then ranks every tile's group maxima for its bound and walks the tiles to build the
superset; sorted rows defeat the bound and take the selection from global memory. Every index set
is compared bit for bit with the oracle's full sort of the same scores.

Sources: "DeepSeek-V4 本地部署，SGLang 把活做絕了", Kernel 層一堆狠活 (top-512 of 256K candidates at 1M
context; longer contexts have more) and "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2
(the threshold is found from radix histograms, with no global sort)."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
import synth
from chs_testutil import check_swaps, dev

pytestmark = pytest.mark.gpu


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _row(rng, variant, n):
    if variant == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if variant == "ascending":
        return np.sort(rng.standard_normal(n)).astype(np.float32)
    if variant == "descending":
        return np.sort(rng.standard_normal(n))[::-1].astype(np.float32).copy()
    if variant == "dup10":
        s = rng.standard_normal(n).astype(np.float32)
        perm = rng.permutation(n)
        nd = n // 10
        chosen, rest = perm[:nd], perm[nd:]
        s[chosen] = s[rest[rng.integers(0, rest.size, nd)]]
        return s
    if variant == "ties":
        return (rng.integers(-8, 8, n) * 0.25).astype(np.float32)
    if variant == "spike":
        # A few large values far in, so the largest scores sit in a late tile only.
        s = rng.standard_normal(n).astype(np.float32)
        s[n - n // 7 + rng.permutation(n // 7)[:3000]] += 6.0
        return s
    raise ValueError(variant)


def _select(rows, k):
    lens = [len(r) for r in rows]
    flat = torch.from_numpy(np.concatenate(rows)).to(dev())
    cu = torch.from_numpy(_cu(lens)).to(dev())
    ws = chs.index_topk_workspace(len(rows), max(lens), k, dev())
    got = chs.topk_from_scores(flat, cu, k, max(lens), ws)
    again = chs.topk_from_scores(flat, cu, k, max(lens), ws)
    torch.cuda.synchronize()
    assert torch.equal(got, again), "a second call on the same workspace differs"
    return got.cpu().numpy()


@pytest.mark.parametrize("n", [1 << 20, 1 << 22])
@pytest.mark.parametrize("variant", ["normal", "ascending", "descending", "dup10", "ties", "spike"])
def test_topk_long_rows_exact(rng, n, variant):
    print(f"case: top-k long row n={n} {variant}", flush=True)
    s = _row(rng, variant, n)
    for k in (512, 2048):
        got = _select([s], k)
        assert np.array_equal(got[0], oracle.topk(s, k)), f"n={n} {variant} k={k}"


def test_topk_long_rows_batched_varlen(rng):
    # Rows of one, several and many tiles in one call, with ragged lengths.
    lens = [1 << 20, 300001, 5, 262145, (1 << 22) - 3, 700000]
    print(f"case: top-k long rows batched {lens}", flush=True)
    rows = [_row(rng, v, n) for v, n in zip(["normal", "dup10", "normal", "spike", "normal", "ties"], lens)]
    got = _select(rows, 512)
    for b, s in enumerate(rows):
        assert np.array_equal(got[b], oracle.topk(s, 512)), f"row {b} (n={lens[b]})"


@pytest.mark.parametrize("dtype,nh,dim,lens,k", [
    # score_kernel with one key row per wave-wide load: groups of 8, so 65,536 candidates per tile
    ("bf16", 2, 512, [150000], 512),
    ("f32", 3, 256, [70000, 3000], 256),
    # the MFMA score kernel past one tile of 8192 groups of 32
    ("bf16", 4, 128, [600000, 1000], 512),
])
def test_index_topk_long_matches_oracle(dtype, nh, dim, lens, k):
    print(f"case: index_topk long {dtype} nh={nh} dim={dim} lens={lens} k={k}", flush=True)
    bf = dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    B, G = len(lens), sum(lens)
    q = synth.normal(41, 5, 0, B * nh * dim, 0, 1, bf).reshape(B, nh, dim)
    w = synth.uniform(41, 6, 0, B * nh).reshape(B, nh)
    U = synth.spike_basis(41, 9, 4, dim)
    K = synth.index_keys(41, 7, 8, 0, G, dim, U, 8.0, bf)
    cu = _cu(lens)
    scores = torch.empty(G, dtype=torch.float32, device=dev())
    topk, _ = chs.index_topk(torch.from_numpy(q).to(dev()).to(tdt), torch.from_numpy(w).to(dev()),
                             torch.from_numpy(K).to(dev()).to(tdt), torch.from_numpy(cu).to(dev()), k, scores=scores)
    sg, tg = scores.cpu().numpy(), topk.cpu().numpy()
    for b in range(B):
        s_ref = oracle.index_scores(q[b], w[b], K[cu[b]:cu[b + 1]])
        s_gpu = sg[cu[b]:cu[b + 1]]
        err = np.abs(s_gpu - s_ref)
        assert np.all(err <= 1e-5 * np.abs(s_ref) + 1e-6 * np.abs(s_ref).max()), f"scores b={b}"
        assert np.array_equal(tg[b], oracle.topk(s_gpu, k)), f"top-k b={b}"   # exact given the same scores
        check_swaps(tg[b], oracle.topk(s_ref.astype(np.float32), k), s_ref, k)
