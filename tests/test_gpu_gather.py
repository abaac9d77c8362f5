"""chs_gather_selected (HiSparse-style working-set gather): the gathered rows are the selected
entries (from the device cache where resident, else from the mirror, in device or pinned host
memory), and attention over the working set is bit-identical to attention over the pool and
within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import assert_bf16_path, assert_lse, dev

pytestmark = pytest.mark.gpu


def _round(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt)


def _selection(rng, G_list, k):
    topk = np.full((len(G_list), k), -1, np.int32)
    for b, G in enumerate(G_list):
        sel = rng.integers(0, max(G, 1), k) if G else np.full(k, -1)
        bad = rng.choice(k, min(5, k), replace=False)
        sel[bad] = rng.choice([-1, -7, G, G + 9], len(bad))
        topk[b] = sel
    return topk


@pytest.mark.parametrize("where,cached", [("device", False), ("host", False), ("host", True), ("device", True)])
@pytest.mark.parametrize("dt,d,G_list,k", [
    (torch.bfloat16, 512, [3000, 0, 700], 512),
    (torch.float32, 64, [256, 77], 64),
])
def test_gather_matches_selection_and_attention(where, cached, dt, d, G_list, k):
    print(f"case: gather {where} cached={cached} {dt} d={d} G={G_list} k={k}", flush=True)
    rng = np.random.default_rng(d + k + len(where) + cached)
    B = len(G_list)
    G = sum(G_list)
    rows = _round(rng.standard_normal((max(G, 1), d)), dt)[:G]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(G_list)]), dtype=torch.int64, device=dev())
    topk_np = _selection(rng, G_list, k)
    topk = torch.from_numpy(topk_np).to(dev())
    if where == "host":
        mirror = torch.empty(rows.shape, dtype=dt, pin_memory=True)
        mirror.copy_(rows)
    else:
        mirror = rows.to(dev())
    cache = resident = None
    res_np = np.full(G, -1, np.int32)
    cache_np = None
    if cached:
        # Half of the entries are resident, at shuffled cache rows holding different values, so
        # the test can tell which copy each slot took.
        nres = G // 2
        ids = rng.choice(G, nres, replace=False)
        res_np[ids] = rng.permutation(nres + 3)[:nres]
        cache_np = rng.standard_normal((nres + 3, d)).astype(np.float32)
        cache = _round(cache_np, dt).to(dev())
        resident = torch.from_numpy(res_np).to(dev())
    work, work_topk, cu_work = chs.gather_selected(mirror, cu, topk, cache, resident)
    torch.cuda.synchronize()
    w, wt = work.float().cpu().numpy(), work_topk.cpu().numpy()
    src = rows.float().numpy()
    cache_f = None if cache is None else cache.float().cpu().numpy()
    cuh = cu.cpu().numpy()
    for b in range(B):
        for i in range(k):
            j = topk_np[b, i]
            if 0 <= j < G_list[b]:
                assert wt[b, i] == i
                e = cuh[b] + j
                want = cache_f[res_np[e]] if cached and res_np[e] >= 0 else src[e]
                assert np.array_equal(w[b * k + i], want), (b, i, j)
            else:
                assert wt[b, i] == -1
    if dt != torch.bfloat16 or cached:
        return
    # Attention over the working set equals attention over the pool, bit for bit, and the oracle.
    H, W = 16, 128
    q = _round(rng.standard_normal((B, H, d)), dt).to(dev())
    swa = _round(rng.standard_normal((B, W, d)), dt).to(dev())
    swa_len = torch.full((B,), W, dtype=torch.int32, device=dev())
    o1, l1 = chs.decode_attn(q, swa, swa_len, rows.to(dev()) if G else torch.zeros(1, d, dtype=dt, device=dev()), cu,
                             topk, d ** -0.5, max(G_list))
    o2, l2 = chs.decode_attn(q, swa, swa_len, work, cu_work, work_topk, d ** -0.5, k)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for b in range(B):
        comp_b = src[cuh[b]:cuh[b + 1]]
        o_ref, l_ref = oracle.attend(q[b].float().cpu().numpy(),
                                     oracle.step_keys(swa[b].float().cpu().numpy(), comp_b, topk_np[b]), d ** -0.5)
        assert_bf16_path(o2[b].cpu().numpy(), o_ref, f"b={b}")
        assert_lse(l2[b].cpu().numpy(), l_ref, f"lse b={b}", 1e-3)

