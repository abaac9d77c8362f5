"""The calls under HIP graph capture: a replayed graph gives, replay after replay, exactly what the
same calls give when launched eagerly (with unrelated eager work and synchronisations between the
replays). The per-token step advances its counters in place, so its graph replays token after
token; new token rows are copied into the captured input buffers before each replay."""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
from chs_testutil import dev

pytestmark = pytest.mark.gpu


def _randn(g, *shape, dt=torch.bfloat16, scale=1.0):
    return (torch.randn(*shape, generator=g, device=dev()) * scale).to(dt)


def _eager_noise():
    # Unrelated eager work between replays (a reduction and a copy), then a synchronisation.
    x = torch.randn(1 << 20, device=dev())
    _ = (x * 2).sum()
    torch.cuda.synchronize()


def test_graph_replays_decode_step_bitwise():
    print("case: graph decode step", flush=True)
    g = torch.Generator(device=dev()).manual_seed(7)
    B, H, d, W, k, nh, dI = 2, 64, 512, 128, 512, 4, 128
    lens = [30000, 9000]
    G = sum(lens)
    cu = torch.tensor([0, lens[0], G], dtype=torch.int64, device=dev())
    keys = _randn(g, G, dI, scale=3.0)
    comp = _randn(g, G, d)
    q, qI = _randn(g, B, H, d), _randn(g, B, nh, dI)
    w = torch.rand(B, nh, generator=g, device=dev())
    swa = _randn(g, B, W, d)
    swa_len = torch.tensor([W, 77], dtype=torch.int32, device=dev())
    scores = torch.empty(G, dtype=torch.float32, device=dev())
    topk = torch.empty(B, k, dtype=torch.int32, device=dev())
    out = torch.empty(B, H, d, dtype=torch.float32, device=dev())
    lse = torch.empty(B, H, dtype=torch.float32, device=dev())
    ws_t = chs.index_topk_workspace(B, max(lens), k, dev())
    ws_a = chs.decode_attn_workspace(torch.bfloat16, B, H, d, W, k, max(lens), dev())

    def step():
        chs.index_topk(qI, w, keys, cu, k, max(lens), scores, ws_t, topk)
        chs.decode_attn(q, swa, swa_len, comp, cu, topk, d ** -0.5, max(lens), ws_a, out, lse)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (scores, topk, out, lse)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        for t in (scores, out, lse):
            t.fill_(float("nan"))
        topk.fill_(-9)
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("scores", "topk", "out", "lse"), (scores, topk, out, lse), want):
            assert torch.equal(got, ref), f"replay {r}: {name} differs from the eager call"


@pytest.mark.parametrize("paged", [False, True])
def test_graph_replays_per_token_step_bitwise(paged):
    # Twin states: A runs every token eagerly, B replays one captured per-token step. Both get the
    # same token rows; after each token every buffer must agree bit for bit.
    print(f"case: graph per-token step paged={paged}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(11)
    m, W, R, d, H, dI, nh, k, P = 4, 32, 8, 128, 16, 64, 2, 64, 64
    n0, steps = 1001, 9
    cap = (n0 + steps) // m + P

    def state():
        gg = torch.Generator(device=dev()).manual_seed(3)
        s = dict(n=torch.tensor([n0], dtype=torch.int64, device=dev()), ni=torch.tensor([n0], dtype=torch.int64,
                                                                                          device=dev()),
                 swa=_randn(gg, 2 if paged else 1, W, d), swaI=_randn(gg, 2 if paged else 1, 8, dI),
                 ring=_randn(gg, (2 if paged else 1) * R, d), ringI=_randn(gg, (2 if paged else 1) * R, dI),
                 comp=_randn(gg, cap, d), keys=_randn(gg, cap, dI, scale=3.0),
                 sl=torch.zeros(1, dtype=torch.int32, device=dev()),
                 cu=torch.tensor([0, n0 // m], dtype=torch.int64, device=dev()),
                 scores=torch.zeros(cap, dtype=torch.float32, device=dev()),
                 topk=torch.zeros(1, k, dtype=torch.int32, device=dev()),
                 out=torch.zeros(1, H, d, dtype=torch.float32, device=dev()),
                 lse=torch.zeros(1, H, dtype=torch.float32, device=dev()))
        s["clen"] = s["cu"][1:]
        return s

    x_tok, z_tok = _randn(g, 1, d), _randn(g, 1, d)
    xi_tok, zi_tok = _randn(g, 1, dI), _randn(g, 1, dI)
    bias = torch.randn(m, d, generator=g, device=dev()) * 0.1
    bias_i = torch.zeros(m, dI, device=dev())
    q, qI = _randn(g, 1, H, d), _randn(g, 1, nh, dI)
    w = torch.rand(1, nh, generator=g, device=dev())
    zero32 = torch.zeros(1, dtype=torch.int32, device=dev())
    one32 = torch.ones(1, dtype=torch.int32, device=dev())
    zero64 = torch.zeros(1, dtype=torch.int64, device=dev())
    pt = torch.randperm(cap // P, generator=torch.Generator().manual_seed(5)).to(torch.int32)[None, :].contiguous()
    pt = pt.to(dev())
    ws_t = chs.index_topk_workspace(1, cap, k, dev())
    ws_a = chs.decode_attn_workspace(torch.bfloat16, 1, H, d, W, k, cap, dev())

    def streams(s):
        if paged:
            return [chs.append_stream(x_tok, z_tok, bias, s["n"], s["swa"], s["ring"], s["comp"], swa_len=s["sl"],
                                      comp_count=s["clen"], swa_page=one32, page_table=pt, page_size=P),
                    chs.append_stream(xi_tok, zi_tok, bias_i, s["ni"], s["swaI"], s["ringI"], s["keys"],
                                      swa_page=one32, page_table=pt, page_size=P)]
        return [chs.append_stream(x_tok, z_tok, bias, s["n"], s["swa"], s["ring"], s["comp"], ring_page=zero32,
                                  comp_start=zero64, ring_size=R, swa_len=s["sl"], comp_count=s["clen"]),
                chs.append_stream(xi_tok, zi_tok, bias_i, s["ni"], s["swaI"], s["ringI"], s["keys"], ring_page=zero32,
                                  comp_start=zero64, ring_size=R)]

    def step(s, st):
        chs.append_multi(m, st)
        if paged:
            chs.index_topk_paged(qI, w, s["keys"], P, pt, s["clen"], k, cap, s["scores"].view(1, cap), ws_t, s["topk"])
            chs.decode_attn_paged(q, s["swa"], one32, s["sl"], s["comp"], P, pt, s["clen"], s["topk"], d ** -0.5, cap,
                                  ws_a, s["out"], s["lse"])
        else:
            chs.index_topk(qI, w, s["keys"], s["cu"], k, cap, s["scores"], ws_t, s["topk"])
            chs.decode_attn(q, s["swa"], s["sl"], s["comp"], s["cu"], s["topk"], d ** -0.5, cap, ws_a, s["out"],
                            s["lse"])

    A, Bst = state(), state()
    sa, sb = streams(A), streams(Bst)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step(Bst, sb)
    torch.cuda.synchronize()
    # Capture does not run the kernels: both states are still the initial one.
    assert A["n"].item() == Bst["n"].item() == n0
    for t in range(steps):
        for buf in (x_tok, z_tok, xi_tok, zi_tok):
            buf.copy_(torch.randn(buf.shape, generator=g, device=dev()).to(buf.dtype))
        step(A, sa)
        torch.cuda.synchronize()
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        for key in ("n", "ni", "sl", "cu", "swa", "swaI", "ring", "ringI", "comp", "keys", "scores", "topk", "out",
                    "lse"):
            assert torch.equal(A[key], Bst[key]), f"token {t}: {key} differs between eager and replay"
    assert A["n"].item() == n0 + steps


@pytest.mark.parametrize("words", [1, 255, 256, 1000003, 5_000_000])
def test_workspace_clear_eager_and_in_graph(words):
    # chs_workspace_clear zero-fills exactly `bytes` bytes with a kernel (one 4-byte word per
    # element), so it can sit in a captured graph; words past the range keep their values. The
    # graph replays after eager writes of fresh garbage, with eager work between replays.
    print(f"case: workspace clear, {words} words", flush=True)
    g = torch.Generator(device=dev()).manual_seed(words)
    buf = torch.randint(1, 1 << 30, (words + 64,), generator=g, dtype=torch.int32, device=dev())
    tail = buf[words:].clone()
    chs.workspace_clear(buf[:words])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(buf[:words])) == 0
    assert torch.equal(buf[words:], tail)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chs.workspace_clear(buf[:words])
    for r in range(3):
        buf[:words].copy_(torch.randint(1, 1 << 30, (words,), generator=g, dtype=torch.int32, device=dev()))
        torch.cuda.synchronize()
        _eager_noise()
        graph.replay()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(buf[:words])) == 0, f"replay {r}"
        assert torch.equal(buf[words:], tail), f"replay {r}: past the range"
