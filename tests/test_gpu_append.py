"""chs_append (one decode-time token per sequence into the window ring and the gate state ring,
pooling a group the token completes) against the oracle's append_state, and a decode loop of
append + index top-k + attention against the oracle's definitions of the grown context.

Inputs are seeded normals rounded to the storage dtype (torch's RNE cast, input preparation).
The GPU's starting state is what the rings hold after a prefill of n0 tokens: the ring images
the oracle defines (ring_image replays the writes), i.e. the caller's prefill bookkeeping."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import assert_bf16_path, assert_bf16_stored, assert_f32, assert_lse, check_swaps, dev

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _t(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev(), dt)


def _round(a, dt):
    """Values as stored in dt (fp32 or bf16), as fp32 numpy."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).float().numpy()


class Streams:
    """Per-sequence token histories and the GPU buffers of the window, the gate ring pages and a
    compressed pool with one region per sequence (plus a guard row after each)."""

    def __init__(self, rng, dt, d, m, W, R, n0, steps, pages_extra=2, bad_page=None):
        self.dt, self.d, self.m, self.W, self.R, self.n0, self.steps = dt, d, m, W, R, list(n0), steps
        B = len(n0)
        self.X = [_round(rng.standard_normal((n + steps, d)), dt) for n in n0]
        self.Z = [_round(rng.standard_normal((n + steps, d)) * 2.0, dt) for n in n0]
        self.bias = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
        pages = B + pages_extra
        perm = rng.permutation(pages)[:B].astype(np.int32)
        if bad_page is not None:
            perm[bad_page] = pages          # outside [0, pages): that sequence's ring is skipped
        self.page = perm
        swa = np.zeros((B, W, d), np.float32)
        ring = np.full((pages * R, d), SENTINEL, np.float32)
        for b in range(B):
            img, wr = oracle.ring_image(self.X[b][:n0[b]], W)
            swa[b][wr] = img[wr]
            if 0 <= perm[b] < pages:
                img, wr = oracle.ring_image(self.Z[b][:n0[b]], R)
                ring[perm[b] * R:(perm[b] + 1) * R][wr] = img[wr]
        caps = [(n + steps) // m + 1 for n in n0]
        self.start = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
        self.rows = int(sum(caps))
        self.swa = _t(swa, dt)
        self.ring = _t(ring, dt)
        self.comp = torch.full((self.rows, d), SENTINEL, dtype=dt, device=dev())
        self.n = torch.tensor(n0, dtype=torch.int64, device=dev())
        self.swa_len = torch.full((B,), -5, dtype=torch.int32, device=dev())
        self.count = torch.full((B,), -5, dtype=torch.int64, device=dev())
        self.page_t = torch.from_numpy(perm).to(dev())
        self.start_t = torch.from_numpy(self.start).to(dev())
        self.bias_t = torch.from_numpy(self.bias).to(dev())

    def step(self, s):
        B = len(self.n0)
        xs = np.stack([self.X[b][self.n0[b] + s] for b in range(B)])
        zs = np.stack([self.Z[b][self.n0[b] + s] for b in range(B)])
        chs.append(_t(xs, self.dt), _t(zs, self.dt), self.bias_t, self.m, self.n, self.swa, self.ring, self.page_t,
                   self.comp, self.start_t, ring_size=self.R, swa_len=self.swa_len, comp_count=self.count)


def _check_state(S, upto, bad=()):
    """Compare every buffer with the oracle's state after `upto` appended tokens per sequence."""
    torch.cuda.synchronize()
    B = len(S.n0)
    n = S.n.cpu().numpy()
    swa = S.swa.float().cpu().numpy()
    ring = S.ring.float().cpu().numpy()
    comp = S.comp.float().cpu().numpy()
    pages = ring.shape[0] // S.R
    used = set()
    for b in range(B):
        N = S.n0[b] + upto
        want = oracle.append_state(S.X[b][:N], S.Z[b][:N], S.bias, S.m, S.W, S.R)
        assert n[b] == want["n"], (b, n[b], want["n"])
        assert S.swa_len[b].item() == want["swa_len"] and S.count[b].item() == want["comp_count"]
        wr = want["swa_written"]
        assert np.array_equal(swa[b][wr], want["swa"][wr]), f"window ring of sequence {b}"
        p = int(S.page[b])
        lo = S.start[b]
        new = range(S.n0[b] // S.m, N // S.m)
        if b in bad:
            assert np.all(comp[lo:lo + N // S.m + 1] == SENTINEL), f"skipped sequence {b} wrote entries"
            continue
        used.add(p)
        gw = want["gate_written"]
        assert np.array_equal(ring[p * S.R:(p + 1) * S.R][gw], want["gate"][gw]), f"gate ring of sequence {b}"
        if len(new):
            got = comp[lo + new.start:lo + new.stop]
            ref = want["comp"][new.start:new.stop]
            if S.dt == torch.bfloat16:
                assert_bf16_stored(got, ref, f"entries of sequence {b}")
            else:
                assert_f32(got, ref, f"entries of sequence {b}")
        # rows before the appended ones (prefill's) and the guard row after them are untouched
        assert np.all(comp[lo:lo + new.start] == SENTINEL) and np.all(comp[lo + N // S.m] == SENTINEL)
    for p in range(pages):
        if p not in used:
            assert np.all(ring[p * S.R:(p + 1) * S.R] == SENTINEL), f"page {p} of no sequence was written"


@pytest.mark.parametrize("dt,d,m,W,R,n0,steps", [
    (torch.bfloat16, 512, 4, 128, 8, [0, 3, 127, 128, 1001, 4096], 13),      # C4, ring of 8
    (torch.bfloat16, 512, 128, 128, 128, [0, 127, 200, 1024], 130),          # C128
    (torch.float32, 64, 4, 128, 4, [5, 6, 7, 8], 9),                           # the tiny fp32 layer
    (torch.bfloat16, 128, 3, 10, 7, [0, 1, 2, 50, 61], 20),                   # W, R not multiples of m
    (torch.float32, 32, 200, 256, 200, [0, 199, 399], 202),                   # m > 8, not a power of two
    (torch.bfloat16, 1024, 1, 128, 1, [0, 9], 3),                              # m = 1: every token is an entry
    (torch.bfloat16, 64, 8, 8, 16, [7, 15, 100], 17),                          # W = m, ring of 2m
    (torch.bfloat16, 4096, 16, 16, 16, [15, 31], 2),                           # widest rows, two passes of chunks
])
def test_append_state_matches_oracle(dt, d, m, W, R, n0, steps):
    print(f"case: append {dt} d={d} m={m} W={W} R={R} n0={n0} steps={steps}", flush=True)
    rng = np.random.default_rng(d + 7 * m + W + R)
    S = Streams(rng, dt, d, m, W, R, n0, steps)
    for s in range(steps):
        S.step(s)
        if s == 0 or s == steps - 1 or (steps > 20 and s % 37 == 0):
            _check_state(S, s + 1)


def test_append_skips_a_page_outside_the_pool():
    print("case: append with one ring page out of range", flush=True)
    rng = np.random.default_rng(3)
    S = Streams(rng, torch.bfloat16, 128, 4, 128, 8, [3, 10, 0], 6, bad_page=0)
    for s in range(6):
        S.step(s)
    _check_state(S, 6, bad=(0,))


def test_append_negative_count_reads_as_empty():
    print("case: append with a negative token count", flush=True)
    rng = np.random.default_rng(4)
    S = Streams(rng, torch.float32, 32, 2, 8, 2, [0], 4)
    S.n.fill_(-3)
    for s in range(4):
        S.step(s)
    _check_state(S, 4)


@pytest.mark.parametrize("dt,m", [(torch.bfloat16, 1), (torch.bfloat16, 2), (torch.bfloat16, 4), (torch.bfloat16, 8),
                                  (torch.float32, 4)])
def test_append_entries_are_the_prefill_bits(dt, m):
    # For m <= 8 the append pools a group with the compressor's own function and order.
    print(f"case: append vs compress bits, {dt} m={m}", flush=True)
    rng = np.random.default_rng(11 + m)
    d, W, R = 512, 128, 2 * m
    S = Streams(rng, dt, d, m, W, R, [0, 5, 64], 3 * m + 1)
    for s in range(S.steps):
        S.step(s)
    torch.cuda.synchronize()
    comp = S.comp.cpu()
    for b in range(3):
        N = S.n0[b] + S.steps
        X, Z = _t(S.X[b][:N], dt), _t(S.Z[b][:N], dt)
        ref = chs.compress(X, Z, S.bias_t, m, torch.tensor([0, N], dtype=torch.int64, device=dev())).cpu()
        lo, g0 = S.start[b], S.n0[b] // m
        assert torch.equal(comp[lo + g0:lo + N // m], ref[g0:N // m]), f"sequence {b}"


def test_decode_loop_with_append_matches_oracle():
    # One C4 layer, batch 1: after a prefill of n0 tokens, every step appends the token's KV row
    # (and its index-key row on the indexer's own stream), selects the top-k of the grown
    # candidate set and attends. comp_count points into cu (its element 1), so the top-k and the
    # attention see each new entry without a host update.
    print("case: decode loop with append", flush=True)
    rng = np.random.default_rng(21)
    m, W, R, d, H, dI, nhI, k = 4, 128, 8, 256, 16, 64, 2, 64
    n0, steps = 602, 11
    N1 = n0 + steps
    bf = torch.bfloat16
    X = _round(rng.standard_normal((N1, d)), bf)
    Z = _round(rng.standard_normal((N1, d)) * 2.0, bf)
    Bkv = (rng.standard_normal((m, d)) * 0.1).astype(np.float32)
    # Index keys pooled with equal weights from small integers, so every stored key is exact and
    # both sides score the same keys.
    XI = rng.integers(-8, 9, (N1, dI)).astype(np.float32)
    ZI = np.zeros((N1, dI), np.float32)
    BI = np.zeros((m, dI), np.float32)
    cap = N1 // m + 4
    cu = torch.tensor([0, n0 // m], dtype=torch.int64, device=dev())
    comp = torch.zeros((cap, d), dtype=bf, device=dev())
    keys = torch.zeros((cap, dI), dtype=bf, device=dev())
    cu_tok = torch.tensor([0, n0], dtype=torch.int64, device=dev())
    chs.compress(_t(X[:n0], bf), _t(Z[:n0], bf), _t(Bkv, torch.float32), m, cu_tok, out=comp[:n0 // m])
    chs.compress(_t(XI[:n0], bf), _t(ZI[:n0], bf), _t(BI, torch.float32), m, cu_tok, out=keys[:n0 // m])
    swa_np = np.zeros((1, W, d), np.float32)
    img, wr = oracle.ring_image(X[:n0], W)
    swa_np[0][wr] = img[wr]
    swa = _t(swa_np, bf)
    ring_np = np.zeros((R, d), np.float32)
    img, wr = oracle.ring_image(Z[:n0], R)
    ring_np[wr] = img[wr]
    ring = _t(ring_np, bf)
    WI = 8
    swaI_np = np.zeros((1, WI, dI), np.float32)
    img, wr = oracle.ring_image(XI[:n0], WI)
    swaI_np[0][wr] = img[wr]
    swaI = _t(swaI_np, bf)
    ringI = torch.zeros((R, dI), dtype=bf, device=dev())
    n_kv = torch.tensor([n0], dtype=torch.int64, device=dev())
    n_ix = torch.tensor([n0], dtype=torch.int64, device=dev())
    swa_len = torch.zeros(1, dtype=torch.int32, device=dev())
    page = torch.zeros(1, dtype=torch.int32, device=dev())
    start = torch.zeros(1, dtype=torch.int64, device=dev())
    bkv, bix = _t(Bkv, torch.float32), _t(BI, torch.float32)
    ws = chs.index_topk_workspace(1, cap, k, dev())
    for s in range(steps):
        t = n0 + s
        N = t + 1
        chs.append(_t(X[t:t + 1], bf), _t(Z[t:t + 1], bf), bkv, m, n_kv, swa, ring, page, comp, start, ring_size=R,
                   swa_len=swa_len, comp_count=cu[1:])
        chs.append(_t(XI[t:t + 1], bf), _t(ZI[t:t + 1], bf), bix, m, n_ix, swaI, ringI, page, keys, start,
                   ring_size=R)
        q = _round(rng.standard_normal((1, H, d)), bf)
        qI = _round(rng.standard_normal((1, nhI, dI)), bf)
        w = rng.random((1, nhI)).astype(np.float32)
        scores = torch.empty(cap, dtype=torch.float32, device=dev())
        topk, _ = chs.index_topk(_t(qI, bf), _t(w, torch.float32), keys, cu, k, max_cand=cap, scores=scores,
                                 workspace=ws)
        out, lse = chs.decode_attn(_t(q, bf), swa, swa_len, comp, cu, topk, d ** -0.5, max_comp=cap)
        torch.cuda.synchronize()
        G = N // m
        assert cu[1].item() == G and n_kv.item() == N and n_ix.item() == N and swa_len.item() == min(N, W)
        kref = oracle.store(oracle.compress(XI[:N], ZI[:N], BI, m, np.array([0, N])), True)
        assert np.array_equal(keys[:G].float().cpu().numpy(), kref), f"step {s}: index keys"
        sref = oracle.index_scores(qI[0], w[0], kref)
        sg = scores[:G].cpu().numpy()
        assert np.all(np.abs(sg - sref) <= 1e-5 * np.abs(sref) + 1e-6 * np.abs(sref).max()), f"step {s}: scores"
        sel = topk[0].cpu().numpy()
        assert np.array_equal(sel, oracle.topk(sg, k)), f"step {s}: top-k of the GPU's scores"
        check_swaps(sel, oracle.topk(sref.astype(np.float32), k), sref, k)
        cref = oracle.store(oracle.compress(X[:N], Z[:N], Bkv, m, np.array([0, N])), True)
        o_ref, l_ref = oracle.decode_step(q[0], X[:N], W, cref, sel, d ** -0.5)
        assert_bf16_path(out[0].cpu().numpy(), o_ref, f"step {s}: attention")
        assert_lse(lse[0].cpu().numpy(), l_ref, f"step {s}: lse")


@pytest.mark.parametrize("m,streams", [
    (4, [(torch.bfloat16, 512, 128, 8, False), (torch.bfloat16, 128, 8, 8, False)]),    # KV + index keys (C4)
    (4, [(torch.bfloat16, 256, 32, 8, True), (torch.bfloat16, 64, 8, 4, False), (torch.bfloat16, 128, 16, 4, True)]),
    (128, [(torch.bfloat16, 512, 128, 128, False), (torch.bfloat16, 128, 128, 128, True)]),  # split path
])
def test_append_multi_equals_single_streams(m, streams):
    # chs_append_multi over several streams (contiguous and paged mixed) leaves every buffer
    # bit-identical to one chs_append / chs_append_paged call per stream.
    print(f"case: append multi m={m} streams={[(s[1], s[4]) for s in streams]}", flush=True)
    rng = np.random.default_rng(m + len(streams))
    B, steps = 3, (m + 3 if m > 8 else 2 * m + 1)
    n0 = [0, m - 1, 5 * m + 2]

    def build():
        out = []
        for dt, d, W, R, paged in streams:
            g = np.random.default_rng(d * 7 + W + R + paged)
            st = dict(dt=dt, d=d, paged=paged, R=R,
                      x=[_t(g.standard_normal((B, d)), dt) for _ in range(steps)],
                      z=[_t(g.standard_normal((B, d)) * 2, dt) for _ in range(steps)],
                      bias=_t(g.standard_normal((m, d)) * 0.1, torch.float32),
                      n=torch.tensor(n0, dtype=torch.int64, device=dev()),
                      sl=torch.zeros(B, dtype=torch.int32, device=dev()),
                      cc=torch.zeros(B, dtype=torch.int64, device=dev()))
            pages = B + 1
            st["swa"] = _t(g.standard_normal((pages if paged else B, W, d)), dt)
            st["ring"] = _t(g.standard_normal(((pages if paged else B) * R, d)), dt)
            cap = (n0[-1] + steps) // m + 2
            if paged:
                P = 4
                st["P"] = P
                st["pt"] = torch.from_numpy(g.permutation(B * ((cap + P - 1) // P)).reshape(B, -1).astype(np.int32)).to(dev())
                st["comp"] = torch.zeros(B * ((cap + P - 1) // P) * P, d, dtype=dt, device=dev())
                st["page"] = torch.from_numpy(g.permutation(pages)[:B].astype(np.int32)).to(dev())
            else:
                st["comp"] = torch.zeros(B * cap, d, dtype=dt, device=dev())
                st["page"] = torch.arange(B, dtype=torch.int32, device=dev())
                st["start"] = torch.arange(0, B * cap, cap, dtype=torch.int64, device=dev())
            out.append(st)
        return out

    def single(st, s):
        if st["paged"]:
            chs.append_paged(st["x"][s], st["z"][s], st["bias"], m, st["n"], st["swa"], st["page"], st["ring"], st["comp"],
                             st["P"], st["pt"], swa_len=st["sl"], comp_count=st["cc"])
        else:
            chs.append(st["x"][s], st["z"][s], st["bias"], m, st["n"], st["swa"], st["ring"], st["page"], st["comp"],
                       st["start"], ring_size=st["R"], swa_len=st["sl"], comp_count=st["cc"])

    def desc(st, s):
        if st["paged"]:
            return chs.append_stream(st["x"][s], st["z"][s], st["bias"], st["n"], st["swa"], st["ring"], st["comp"],
                                     swa_len=st["sl"], comp_count=st["cc"], swa_page=st["page"], page_table=st["pt"],
                                     page_size=st["P"])
        return chs.append_stream(st["x"][s], st["z"][s], st["bias"], st["n"], st["swa"], st["ring"], st["comp"],
                                 ring_page=st["page"], comp_start=st["start"], ring_size=st["R"], swa_len=st["sl"],
                                 comp_count=st["cc"])

    A, Bs = build(), build()
    for s in range(steps):
        for st in A:
            single(st, s)
        chs.append_multi(m, [desc(st, s) for st in Bs])
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(A, Bs)):
        for key in ("n", "sl", "cc", "swa", "ring", "comp"):
            assert torch.equal(a[key], b[key]), f"stream {i}: {key} differs"
