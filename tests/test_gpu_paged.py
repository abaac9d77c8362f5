"""Paged pools: chs_decode_attn_paged and chs_append_paged against the oracle, which reads the
pools through its own paged_rows definition, and against the contiguous calls on the same rows.

Pools are filled by scattering seeded rows to random pages (input preparation); pages no
sequence owns hold a sentinel."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import assert_bf16_path, assert_bf16_stored, assert_f32, assert_lse, dev

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _t(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev(), dt)


def _round(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).float().numpy()


def _paged_pool(rng, rows_per_seq, P, d, dt, extra_pages=3):
    """Scatter each sequence's logical rows to shuffled pages. Returns (pool rows fp32 as stored,
    page table [B, stride] int32)."""
    need = [(len(r) + P - 1) // P for r in rows_per_seq]
    stride = max(1, max(need))
    total = sum(need) + extra_pages
    pages = rng.permutation(total)
    pool = np.full((total * P, d), SENTINEL, np.float32)
    pt = np.full((len(rows_per_seq), stride), -1, np.int32)
    k = 0
    for b, rows in enumerate(rows_per_seq):
        for i in range(need[b]):
            pt[b, i] = pages[k]
            k += 1
        for j in range(len(rows)):
            pool[pt[b, j // P] * P + j % P] = rows[j]
    return _round(pool, dt), pt


@pytest.mark.parametrize("dt,H,d,W,P,G_list,k,dense", [
    (torch.bfloat16, 64, 512, 128, 64, [3000, 0, 700], 512, False),
    # many sequences: the selected entries go through the 64-head d = 512 kernel
    (torch.bfloat16, 72, 512, 128, 64, [400 + 37 * i for i in range(24)], 64, False),
    (torch.bfloat16, 64, 512, 128, 128, [2048, 1000], 0, True),
    (torch.bfloat16, 16, 128, 32, 1, [300, 45], 40, False),        # page size 1: a gather per entry
    (torch.bfloat16, 100, 256, 128, 256, [5000], 200, False),
    (torch.bfloat16, 100, 256, 128, 64, [3000, 900], 0, True),
    (torch.float32, 8, 64, 128, 16, [256, 77], 64, False),
    (torch.float32, 8, 64, 16, 32, [100, 40], 0, True),
])
def test_paged_attention_matches_oracle_and_contiguous(dt, H, d, W, P, G_list, k, dense):
    print(f"case: paged attention {dt} H={H} d={d} W={W} P={P} G={G_list} k={k} dense={dense}", flush=True)
    rng = np.random.default_rng(H + d + W + P)
    B = len(G_list)
    q = _round(rng.standard_normal((B, H, d)), dt)
    logical = [_round(rng.standard_normal((G, d)), dt) for G in G_list]
    pool, pt = _paged_pool(rng, logical, P, d, dt)
    swa_pages = B + 2
    swa_page = rng.permutation(swa_pages)[:B].astype(np.int32)
    swa_pool = _round(rng.standard_normal((swa_pages, W, d)), dt)
    swa_len = rng.integers(0, W + 1, B).astype(np.int32)
    swa_len[0] = W
    topk = None
    if not dense:
        topk = np.full((B, k), -1, np.int32)
        for b, G in enumerate(G_list):
            sel = rng.integers(0, max(G, 1), k) if G else np.full(k, -1)
            bad = rng.choice(k, min(5, k), replace=False)
            sel[bad] = rng.choice([-1, -7, G, G + 9], len(bad))
            topk[b] = sel
    comp_len = np.array(G_list, np.int64)
    out, lse = chs.decode_attn_paged(_t(q, dt), _t(swa_pool, dt), torch.from_numpy(swa_page).to(dev()),
                                     torch.from_numpy(swa_len).to(dev()), _t(pool, dt), P,
                                     torch.from_numpy(pt).to(dev()), torch.from_numpy(comp_len).to(dev()),
                                     None if dense else torch.from_numpy(topk).to(dev()), d ** -0.5, max(G_list))
    # The same rows, contiguous.
    cu = torch.tensor(np.concatenate([[0], np.cumsum(G_list)]), dtype=torch.int64, device=dev())
    comp_c = _t(np.concatenate(logical) if sum(G_list) else np.zeros((1, d)), dt)
    swa_c = _t(np.stack([swa_pool[p] for p in swa_page]), dt)
    out_c, lse_c = chs.decode_attn(_t(q, dt), swa_c, torch.from_numpy(swa_len).to(dev()), comp_c, cu,
                                   None if dense else torch.from_numpy(topk).to(dev()), d ** -0.5, max(G_list))
    torch.cuda.synchronize()
    assert torch.equal(out, out_c) and torch.equal(lse, lse_c), "paged and contiguous calls differ"
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    for b, G in enumerate(G_list):
        comp_rows = oracle.paged_rows(pool, pt[b], P, G)
        win = swa_pool[swa_page[b]][:swa_len[b]]
        o_ref, l_ref = oracle.attend(q[b], oracle.step_keys(win, comp_rows, None if dense else topk[b]), d ** -0.5)
        if dt == torch.bfloat16:
            assert_bf16_path(og[b], o_ref, f"paged attention b={b}")
            assert_lse(lg[b], l_ref, f"paged lse b={b}", 1e-3)
        else:
            assert_f32(og[b], o_ref, f"paged attention b={b}")
            assert_lse(lg[b], l_ref, f"paged lse b={b}", 1e-5)


def test_paged_attention_skips_bad_pages_and_caps_lengths():
    # An entry whose page is outside the pool is skipped; a window page outside the window pool
    # drops the window; comp_len beyond the page table's reach is capped.
    print("case: paged attention with bad pages", flush=True)
    rng = np.random.default_rng(9)
    dt, H, d, W, P = torch.bfloat16, 16, 128, 32, 16
    logical = [_round(rng.standard_normal((64, d)), dt), _round(rng.standard_normal((48, d)), dt)]
    pool, pt = _paged_pool(rng, logical, P, d, dt)
    pool_pages = pool.shape[0] // P
    pt[0, 1] = pool_pages + 3                 # entries 16..31 of sequence 0: skipped
    q = _round(rng.standard_normal((2, H, d)), dt)
    swa_pool = _round(rng.standard_normal((2, W, d)), dt)
    swa_page = np.array([0, 5], np.int32)     # sequence 1's window page is outside [0, 2)
    swa_len = np.array([W, W], np.int32)
    comp_len = np.array([64, 1000], np.int64)  # sequence 1: capped at stride * P = 64; its 4th page is -1
    out, lse = chs.decode_attn_paged(_t(q, dt), _t(swa_pool, dt), torch.from_numpy(swa_page).to(dev()),
                                     torch.from_numpy(swa_len).to(dev()), _t(pool, dt), P,
                                     torch.from_numpy(pt).to(dev()), torch.from_numpy(comp_len).to(dev()), None,
                                     d ** -0.5, 1000)
    torch.cuda.synchronize()
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    keys0 = np.concatenate([swa_pool[0], logical[0][:16], logical[0][32:]])
    assert pt[1, 3] == -1                     # entries 48..63 of the capped length: skipped
    rows1 = oracle.paged_rows(pool, pt[1], P, 48)
    for b, keys in ((0, keys0), (1, rows1)):
        o_ref, l_ref = oracle.attend(q[b], keys, d ** -0.5)
        assert_bf16_path(og[b], o_ref, f"b={b}")
        assert_lse(lg[b], l_ref, f"lse b={b}", 1e-3)


@pytest.mark.parametrize("dt,d,m,W,R,P,n0,steps", [
    (torch.bfloat16, 512, 4, 128, 8, 64, [0, 3, 130, 1001], 13),
    (torch.bfloat16, 256, 128, 128, 128, 16, [0, 127, 300], 130),
    (torch.float32, 64, 4, 16, 4, 1, [5, 6, 70], 9),
])
def test_paged_append_matches_oracle(dt, d, m, W, R, P, n0, steps):
    print(f"case: paged append {dt} d={d} m={m} W={W} R={R} P={P} n0={n0}", flush=True)
    rng = np.random.default_rng(d + m + P)
    B = len(n0)
    X = [_round(rng.standard_normal((n + steps, d)), dt) for n in n0]
    Z = [_round(rng.standard_normal((n + steps, d)) * 2, dt) for n in n0]
    bias = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
    swa_pages = B + 2
    swa_page = rng.permutation(swa_pages)[:B].astype(np.int32)
    swa_pool = np.zeros((swa_pages, W, d), np.float32)
    ring = np.full((swa_pages * R, d), SENTINEL, np.float32)
    for b in range(B):
        img, wr = oracle.ring_image(X[b][:n0[b]], W)
        swa_pool[swa_page[b]][wr] = img[wr]
        img, wr = oracle.ring_image(Z[b][:n0[b]], R)
        ring[swa_page[b] * R:(swa_page[b] + 1) * R][wr] = img[wr]
    caps = [(n + steps) // m + 1 for n in n0]
    placeholder = [np.zeros((c, d), np.float32) for c in caps]
    pool, pt = _paged_pool(rng, placeholder, P, d, dt)
    pool[:] = SENTINEL
    swa_t, ring_t, pool_t = _t(swa_pool, dt), _t(ring, dt), _t(pool, dt)
    n_t = torch.tensor(n0, dtype=torch.int64, device=dev())
    sl = torch.zeros(B, dtype=torch.int32, device=dev())
    cc = torch.zeros(B, dtype=torch.int64, device=dev())
    page_t, pt_t, bias_t = torch.from_numpy(swa_page).to(dev()), torch.from_numpy(pt).to(dev()), _t(bias, torch.float32)
    for s in range(steps):
        xs = np.stack([X[b][n0[b] + s] for b in range(B)])
        zs = np.stack([Z[b][n0[b] + s] for b in range(B)])
        chs.append_paged(_t(xs, dt), _t(zs, dt), bias_t, m, n_t, swa_t, page_t, ring_t, pool_t, P, pt_t, swa_len=sl,
                         comp_count=cc)
    torch.cuda.synchronize()
    swa_g, ring_g, pool_g = swa_t.float().cpu().numpy(), ring_t.float().cpu().numpy(), pool_t.float().cpu().numpy()
    for b in range(B):
        N = n0[b] + steps
        want = oracle.append_state(X[b][:N], Z[b][:N], bias, m, W, R)
        assert n_t[b].item() == N and sl[b].item() == want["swa_len"] and cc[b].item() == want["comp_count"]
        wr = want["swa_written"]
        assert np.array_equal(swa_g[swa_page[b]][wr], want["swa"][wr]), f"window page of sequence {b}"
        gw = want["gate_written"]
        assert np.array_equal(ring_g[swa_page[b] * R:(swa_page[b] + 1) * R][gw], want["gate"][gw])
        entries = oracle.paged_rows(pool_g, pt[b], P, N // m)
        new = slice(n0[b] // m, N // m)
        if new.stop > new.start:
            if dt == torch.bfloat16:
                assert_bf16_stored(entries[new], want["comp"][new], f"entries of sequence {b}")
            else:
                assert_f32(entries[new], want["comp"][new], f"entries of sequence {b}")
        assert np.all(entries[:new.start] == SENTINEL)


def test_paged_decode_loop_dense():
    # A dense (C128-style) layer over paged pools: each step appends the token (its window page,
    # its gate ring, an entry every m tokens through the page table) and attends over the window
    # and every entry; comp_count feeds comp_len directly.
    print("case: paged decode loop", flush=True)
    rng = np.random.default_rng(31)
    dt, m, W, R, P, d, H = torch.bfloat16, 8, 16, 16, 4, 128, 16
    n0, steps = 37, 30
    N1 = n0 + steps
    X = _round(rng.standard_normal((N1, d)), dt)
    Z = _round(rng.standard_normal((N1, d)) * 2, dt)
    bias = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
    cap = N1 // m + 1
    pool, pt = _paged_pool(rng, [np.zeros((cap, d), np.float32)], P, d, dt)
    pre = oracle.store(oracle.compress(X[:n0], Z[:n0], bias, m, np.array([0, n0])), True)
    for j in range(n0 // m):
        pool[pt[0, j // P] * P + j % P] = pre[j]
    swa_pool = np.zeros((3, W, d), np.float32)
    swa_page = np.array([2], np.int32)
    img, wr = oracle.ring_image(X[:n0], W)
    swa_pool[2][wr] = img[wr]
    ring = np.zeros((3 * R, d), np.float32)
    img, wr = oracle.ring_image(Z[:n0], R)
    ring[2 * R:3 * R][wr] = img[wr]
    swa_t, ring_t, pool_t = _t(swa_pool, dt), _t(ring, dt), _t(pool, dt)
    n_t = torch.tensor([n0], dtype=torch.int64, device=dev())
    sl = torch.zeros(1, dtype=torch.int32, device=dev())
    clen = torch.tensor([n0 // m], dtype=torch.int64, device=dev())
    page_t, pt_t, bias_t = torch.from_numpy(swa_page).to(dev()), torch.from_numpy(pt).to(dev()), _t(bias, torch.float32)
    for s in range(steps):
        t = n0 + s
        N = t + 1
        chs.append_paged(_t(X[t:t + 1], dt), _t(Z[t:t + 1], dt), bias_t, m, n_t, swa_t, page_t, ring_t, pool_t, P, pt_t,
                         swa_len=sl, comp_count=clen)
        q = _round(rng.standard_normal((1, H, d)), dt)
        out, lse = chs.decode_attn_paged(_t(q, dt), swa_t, page_t, sl, pool_t, P, pt_t, clen, None, d ** -0.5, cap)
        torch.cuda.synchronize()
        assert clen.item() == N // m and sl.item() == min(N, W)
        cref = oracle.store(oracle.compress(X[:N], Z[:N], bias, m, np.array([0, N])), True)
        o_ref, l_ref = oracle.decode_step(q[0], X[:N], W, cref, None, d ** -0.5)
        assert_bf16_path(out[0].cpu().numpy(), o_ref, f"step {s}")
        assert_lse(lse[0].cpu().numpy(), l_ref, f"step {s} lse")


@pytest.mark.parametrize("nh,dim,P,lens,k", [
    (4, 128, 64, [5000], 512),
    (4, 128, 128, [1000, 0, 7000, 3], 512),
    (16, 64, 64, [2500, 640], 100),
    (2, 256, 1024, [1777], 300),
    (8, 128, 256, [900, 64], 1000),
])
def test_paged_index_topk_matches_oracle_and_contiguous(nh, dim, P, lens, k):
    print(f"case: paged index top-k nh={nh} dim={dim} P={P} lens={lens} k={k}", flush=True)
    rng = np.random.default_rng(nh * 100 + dim + P)
    B = len(lens)
    bf = torch.bfloat16
    logical = [_round(rng.standard_normal((n, dim)) * 3, bf) for n in lens]
    pool, pt = _paged_pool(rng, logical, P, dim, bf)
    q = _round(rng.standard_normal((B, nh, dim)), bf)
    w = rng.random((B, nh)).astype(np.float32)
    max_cand = max(lens)
    scores = torch.full((B, max_cand), -5.0, dtype=torch.float32, device=dev())
    topk, _ = chs.index_topk_paged(_t(q, bf), _t(w, torch.float32), _t(pool, bf), P, torch.from_numpy(pt).to(dev()),
                                   torch.tensor(lens, dtype=torch.int64, device=dev()), k, max_cand, scores)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev())
    keys_c = _t(np.concatenate(logical) if sum(lens) else np.zeros((1, dim)), bf)
    sc_c = torch.empty(max(sum(lens), 1), dtype=torch.float32, device=dev())
    topk_c, _ = chs.index_topk(_t(q, bf), _t(w, torch.float32), keys_c, cu, k, max_cand, sc_c)
    torch.cuda.synchronize()
    assert torch.equal(topk, topk_c), "paged and contiguous top-k differ"
    sg, cuh = scores.cpu().numpy(), cu.cpu().numpy()
    for b, n in enumerate(lens):
        assert np.array_equal(sg[b, :n], sc_c[cuh[b]:cuh[b + 1]].cpu().numpy()), f"scores of sequence {b}"
        assert np.all(sg[b, n:] == -5.0), "scores written past the sequence"
        ref = oracle.index_scores(q[b], w[b], oracle.paged_rows(pool, pt[b], P, n))
        if n:
            assert np.all(np.abs(sg[b, :n] - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max())
        assert np.array_equal(topk[b].cpu().numpy(), oracle.topk(sg[b, :n], k))


def test_paged_decode_loop_c4():
    # The whole step over paged pools, batch 2: appends of the KV row and of the index key (one page
    # table for both pools: they share the entry numbering), the paged top-k and the paged attention;
    # comp_count feeds comp_len / cand_len.
    print("case: paged C4 decode loop", flush=True)
    rng = np.random.default_rng(41)
    bf = torch.bfloat16
    m, W, R, P, d, H, dI, nhI, k = 4, 32, 8, 64, 128, 16, 64, 2, 32
    n0 = [300, 517]
    steps = 9
    B = len(n0)
    N1 = [n + steps for n in n0]
    X = [_round(rng.standard_normal((n, d)), bf) for n in N1]
    Z = [_round(rng.standard_normal((n, d)) * 2, bf) for n in N1]
    XI = [rng.integers(-8, 9, (n, dI)).astype(np.float32) for n in N1]   # equal-weight pooling: exact keys
    Bkv = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
    BI = np.zeros((m, dI), np.float32)
    caps = [n // m + 2 for n in N1]
    _, pt = _paged_pool(rng, [np.zeros((c, 1), np.float32) for c in caps], P, 1, torch.float32)
    pool_rows = (pt.max() + 1 + 3) * P
    kv_pool = np.zeros((pool_rows, d), np.float32)
    key_pool = np.zeros((pool_rows, dI), np.float32)
    for b in range(B):
        pre = oracle.store(oracle.compress(X[b][:n0[b]], Z[b][:n0[b]], Bkv, m, np.array([0, n0[b]])), True)
        prek = oracle.store(oracle.compress(XI[b][:n0[b]], np.zeros((n0[b], dI), np.float32), BI, m,
                                            np.array([0, n0[b]])), True)
        for j in range(n0[b] // m):
            kv_pool[pt[b, j // P] * P + j % P] = pre[j]
            key_pool[pt[b, j // P] * P + j % P] = prek[j]
    swa_page = np.array([3, 1], np.int32)
    swa_pool = np.zeros((4, W, d), np.float32)
    swaI_pool = np.zeros((4, 8, dI), np.float32)
    ring = np.zeros((4 * R, d), np.float32)
    ringI = np.zeros((4 * R, dI), np.float32)
    for b in range(B):
        img, wr = oracle.ring_image(X[b][:n0[b]], W)
        swa_pool[swa_page[b]][wr] = img[wr]
        img, wr = oracle.ring_image(Z[b][:n0[b]], R)
        ring[swa_page[b] * R:(swa_page[b] + 1) * R][wr] = img[wr]
        img, wr = oracle.ring_image(XI[b][:n0[b]], 8)
        swaI_pool[swa_page[b]][wr] = img[wr]
    t = {name: _t(a, bf) for name, a in
         dict(kv=kv_pool, key=key_pool, swa=swa_pool, swaI=swaI_pool, ring=ring, ringI=ringI).items()}
    n_kv = torch.tensor(n0, dtype=torch.int64, device=dev())
    n_ix = n_kv.clone()
    sl = torch.zeros(B, dtype=torch.int32, device=dev())
    clen = torch.tensor([n // m for n in n0], dtype=torch.int64, device=dev())
    page_t, pt_t = torch.from_numpy(swa_page).to(dev()), torch.from_numpy(pt).to(dev())
    bkv, bix = _t(Bkv, torch.float32), _t(BI, torch.float32)
    max_cand = max(caps)
    for s in range(steps):
        xs = np.stack([X[b][n0[b] + s] for b in range(B)])
        zs = np.stack([Z[b][n0[b] + s] for b in range(B)])
        xis = np.stack([XI[b][n0[b] + s] for b in range(B)])
        chs.append_paged(_t(xs, bf), _t(zs, bf), bkv, m, n_kv, t["swa"], page_t, t["ring"], t["kv"], P, pt_t,
                         swa_len=sl, comp_count=clen)
        chs.append_paged(_t(xis, bf), torch.zeros(B, dI, dtype=bf, device=dev()), bix, m, n_ix, t["swaI"], page_t,
                         t["ringI"], t["key"], P, pt_t)
        q = _round(rng.standard_normal((B, H, d)), bf)
        qI = _round(rng.standard_normal((B, nhI, dI)), bf)
        w = rng.random((B, nhI)).astype(np.float32)
        scores = torch.zeros((B, max_cand), dtype=torch.float32, device=dev())
        topk, _ = chs.index_topk_paged(_t(qI, bf), _t(w, torch.float32), t["key"], P, pt_t, clen, k, max_cand, scores)
        out, lse = chs.decode_attn_paged(_t(q, bf), t["swa"], page_t, sl, t["kv"], P, pt_t, clen, topk, d ** -0.5,
                                         max_cand)
        torch.cuda.synchronize()
        for b in range(B):
            N = n0[b] + s + 1
            G = N // m
            assert clen[b].item() == G and sl[b].item() == min(N, W)
            kref = oracle.store(oracle.compress(XI[b][:N], np.zeros((N, dI), np.float32), BI, m, np.array([0, N])), True)
            sref = oracle.index_scores(qI[b], w[b], kref)
            sg = scores[b, :G].cpu().numpy()
            assert np.all(np.abs(sg - sref) <= 1e-5 * np.abs(sref) + 1e-6 * np.abs(sref).max()), f"step {s} b={b}"
            sel = topk[b].cpu().numpy()
            assert np.array_equal(sel, oracle.topk(sg, k)), f"step {s} b={b}: top-k"
            cref = oracle.store(oracle.compress(X[b][:N], Z[b][:N], Bkv, m, np.array([0, N])), True)
            o_ref, l_ref = oracle.decode_step(q[b], X[b][:N], W, cref, sel, d ** -0.5)
            assert_bf16_path(out[b].cpu().numpy(), o_ref, f"step {s} b={b}: attention")
            assert_lse(lse[b].cpu().numpy(), l_ref, f"step {s} b={b}: lse")


def _quantise_rows(x):
    """Per-row E4M3 codes (uint8) and fp32 scales of fp32 device rows (input preparation)."""
    scale = (x.abs().amax(dim=-1) / 448.0).clamp_min(1e-30)
    codes = (x / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _scatter_pages(rows, pt, P, n_rows):
    """Logical rows of each sequence (a list) into a pool of n_rows rows through the page table."""
    pool = torch.zeros((n_rows,) + tuple(rows[0].shape[1:]), dtype=rows[0].dtype, device=dev())
    for b, r in enumerate(rows):
        j = torch.arange(r.shape[0], device=dev())
        phys = pt[b][j // P].long() * P + j % P
        pool[phys] = r
    return pool


@pytest.mark.parametrize("nh,dim,P,lens,k", [(4, 128, 64, [5000, 700], 512), (16, 64, 128, [3000], 100),
                                             (2, 256, 32, [1500, 0, 333], 300)])
def test_paged_fp8_index_equals_contiguous(nh, dim, P, lens, k):
    print(f"case: paged fp8 index nh={nh} dim={dim} P={P} lens={lens}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(dim + P)
    rows = [torch.randn(n, dim, generator=g, device=dev()) * 3 for n in lens]
    qc = [_quantise_rows(r) for r in rows]
    need = [(n + P - 1) // P for n in lens]
    stride = max(1, max(need))
    total = sum(need) + 2
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(1)).to(torch.int32)
    pt = torch.full((len(lens), stride), -1, dtype=torch.int32)
    o = 0
    for b, nb in enumerate(need):
        pt[b, :nb] = perm[o:o + nb]
        o += nb
    pt = pt.to(dev())
    codes_pool = _scatter_pages([c for c, _ in qc], pt, P, total * P)
    scale_pool = _scatter_pages([s for _, s in qc], pt, P, total * P)
    q = torch.randn(len(lens), nh, dim, generator=g, device=dev()).bfloat16()
    w = torch.rand(len(lens), nh, generator=g, device=dev())
    max_cand = max(lens)
    sp = torch.full((len(lens), max_cand), -5.0, device=dev())
    tp, _ = chs.index_topk_fp8_paged(q, w, codes_pool, scale_pool, P, pt, torch.tensor(lens, device=dev()), k,
                                     max_cand, sp)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev())
    codes_c = torch.cat([c for c, _ in qc]) if sum(lens) else torch.zeros(1, dim, dtype=torch.uint8, device=dev())
    scales_c = torch.cat([s for _, s in qc]) if sum(lens) else torch.zeros(1, device=dev())
    sc = torch.empty(max(sum(lens), 1), device=dev())
    tc, _ = chs.index_topk_fp8(q, w, codes_c, scales_c, cu, k, max_cand, sc)
    torch.cuda.synchronize()
    assert torch.equal(tp, tc)
    cuh = cu.cpu().numpy()
    for b, n in enumerate(lens):
        assert torch.equal(sp[b, :n], sc[cuh[b]:cuh[b + 1]]), f"scores of sequence {b}"


@pytest.mark.parametrize("H,d,W,P,G_list,k,dense", [(64, 512, 128, 64, [3000, 700], 512, False),
                                                    (16, 128, 32, 16, [400, 1200], 0, True),
                                                    (64, 512, 128, 64, [2500, 600], 0, True)])
def test_paged_fp8_attention_equals_contiguous_and_oracle(H, d, W, P, G_list, k, dense):
    print(f"case: paged fp8 attention H={H} d={d} P={P} G={G_list} dense={dense}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(H + d + P)
    B = len(G_list)
    rows = [torch.randn(G, d, generator=g, device=dev()) for G in G_list]
    qc = [_quantise_rows(r) for r in rows]
    need = [(G + P - 1) // P for G in G_list]
    stride = max(need)
    total = sum(need) + 1
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(2)).to(torch.int32)
    pt = torch.full((B, stride), -1, dtype=torch.int32)
    o = 0
    for b, nb in enumerate(need):
        pt[b, :nb] = perm[o:o + nb]
        o += nb
    pt = pt.to(dev())
    cpool = _scatter_pages([c for c, _ in qc], pt, P, total * P)
    spool = _scatter_pages([s for _, s in qc], pt, P, total * P)
    swa_pages = B + 1
    swa_codes, swa_scales = _quantise_rows(torch.randn(swa_pages, W, d, generator=g, device=dev()))
    swa_page = torch.tensor([2, 0], dtype=torch.int32, device=dev())[:B]
    swa_len = torch.tensor([W, W // 3], dtype=torch.int32, device=dev())[:B]
    q = torch.randn(B, H, d, generator=g, device=dev()).bfloat16()
    topk = None
    if not dense:
        topk = torch.stack([torch.randint(-2, G + 3, (k,), generator=g, device=dev()) for G in G_list]).int()
    clen = torch.tensor(G_list, dtype=torch.int64, device=dev())
    op, lp = chs.decode_attn_fp8_paged(q, swa_codes, swa_scales, swa_page, swa_len, cpool, spool, P, pt, clen, topk,
                                       d ** -0.5, max(G_list))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(G_list)]), dtype=torch.int64, device=dev())
    oc, lc = chs.decode_attn_fp8(q, swa_codes[swa_page.long()].contiguous(), swa_scales[swa_page.long()].contiguous(),
                                 swa_len, torch.cat([c for c, _ in qc]), torch.cat([s for _, s in qc]), cu, topk,
                                 d ** -0.5, max(G_list))
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc), "paged and contiguous FP8 calls differ"
    b = 0
    nsw = int(swa_len[b])
    sel = [int(j) for j in (range(G_list[b]) if dense else topk[b].tolist()) if 0 <= j < G_list[b]]
    codes = torch.cat([swa_codes[int(swa_page[b]), :nsw], qc[b][0][sel]]).cpu().numpy()
    scales = torch.cat([swa_scales[int(swa_page[b]), :nsw], qc[b][1][sel]]).cpu().numpy()
    o_ref, l_ref = oracle.attend_fp8(q[b].float().cpu().numpy(), codes, scales, d ** -0.5)
    assert_bf16_path(op[b].cpu().numpy(), o_ref, "paged fp8 attention")
    assert_lse(lp[b].cpu().numpy(), l_ref, "paged fp8 lse", 1e-3)


@pytest.mark.parametrize("B,H,d,W,P,G_list,Hi,dI,k", [
    (3, 64, 512, 128, 64, [3000, 0, 700], 4, 128, 512),                          # 16-head fused workgroups
    (24, 72, 512, 128, 64, [400 + 37 * i for i in range(24)], 4, 128, 64),       # many sequences: the 64-head kernel
    (2, 16, 128, 32, 128, [900, 2500], 2, 64, 40),
])
def test_paged_step_matches_the_two_calls_and_the_contiguous_step(B, H, d, W, P, G_list, Hi, dI, k):
    # chs_decode_step_paged against chs_index_topk_paged + chs_decode_attn_paged (one page table for the
    # key pool and the entry pool) and against chs_decode_step on the same rows stored contiguously:
    # scores, top-k, out and lse bit for bit.
    print(f"case: paged step B={B} H={H} d={d} P={P} G={sum(G_list)} k={k}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    gen = np.random.default_rng(9)
    G = int(sum(G_list))
    keys = torch.randn(G, dI, generator=g, device="cuda").bfloat16()
    comp = torch.randn(G, d, generator=g, device="cuda").bfloat16()
    need = [(n + P - 1) // P for n in G_list]
    stride = max(1, max(need))
    pages = torch.from_numpy(gen.permutation(sum(need) + 2).astype(np.int64)).cuda()
    pt = torch.full((B, stride), -1, dtype=torch.int32, device="cuda")
    kpool = torch.zeros((sum(need) + 2) * P, dI, dtype=torch.bfloat16, device="cuda")
    cpool = torch.zeros((sum(need) + 2) * P, d, dtype=torch.bfloat16, device="cuda")
    c0, p0 = 0, 0
    for b, n in enumerate(G_list):
        for i in range(need[b]):
            pg = int(pages[p0 + i])
            pt[b, i] = pg
            lo, hi = i * P, min(n, (i + 1) * P)
            kpool[pg * P:pg * P + hi - lo] = keys[c0 + lo:c0 + hi]
            cpool[pg * P:pg * P + hi - lo] = comp[c0 + lo:c0 + hi]
        c0 += n
        p0 += need[b]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(G_list)]), dtype=torch.int64, device="cuda")
    clen = torch.tensor(G_list, dtype=torch.int64, device="cuda")
    swa_pages = B + 3
    swa_page = torch.from_numpy(gen.permutation(swa_pages)[:B].astype(np.int32)).cuda()
    swa_pool = torch.randn(swa_pages, W, d, generator=g, device="cuda").bfloat16()
    swa = swa_pool[swa_page.long()].contiguous()
    sl = torch.tensor([W, W // 2, 0, 7][:B] + [W] * max(0, B - 4), dtype=torch.int32, device="cuda")
    qi = torch.randn(B, Hi, dI, generator=g, device="cuda").bfloat16()
    w = torch.rand(B, Hi, generator=g, device="cuda")
    q = torch.randn(B, H, d, generator=g, device="cuda").bfloat16()
    mx = max(G_list)
    s1 = torch.empty(B, mx, dtype=torch.float32, device="cuda")
    s2 = torch.empty(B, mx, dtype=torch.float32, device="cuda")
    tk1, _ = chs.index_topk_paged(qi, w, kpool, P, pt, clen, k, mx, s1)
    o1, l1 = chs.decode_attn_paged(q, swa_pool, swa_page, sl, cpool, P, pt, clen, tk1, None, mx)
    tk2, o2, l2, _ = chs.decode_step_paged(qi, w, kpool, q, swa_pool, swa_page, sl, cpool, P, pt, clen, k, mx,
                                           None, s2)
    tk3, o3, l3, _ = chs.decode_step(qi, w, keys, q, swa, sl, comp, cu, k, None, mx)
    torch.cuda.synchronize()
    for b, n in enumerate(G_list):
        assert torch.equal(s1[b, :n], s2[b, :n]), f"scores differ in sequence {b}"
    assert torch.equal(tk1, tk2) and torch.equal(tk2, tk3), "top-k differs"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "out differs from the two paged calls"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs from the two paged calls"
    assert torch.equal(o2.view(torch.int32), o3.view(torch.int32)), "out differs from the contiguous step"
    assert torch.equal(l2.view(torch.int32), l3.view(torch.int32)), "lse differs from the contiguous step"
