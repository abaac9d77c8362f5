"""chs_decode_step (the C4 decode step in one call) against the two calls it stands for,
chs_index_topk followed by chs_decode_attn, on the same inputs: scores, top-k, out and lse must
be bit-identical. The two calls are themselves checked against the oracle elsewhere; the
workload tests also check chs_decode_step against the oracle directly. Covered here: several
tiles and ragged tails, head counts that are not a multiple of 16, each bf16 latent width,
sequences with fewer entries than k, with no entries, with a short or empty window, and graph
replay."""
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
from chs_testutil import dev

pytestmark = pytest.mark.gpu


def _randn(g, *shape, scale=1.0):
    return (torch.randn(*shape, generator=g, device=dev()) * scale).to(torch.bfloat16)


def _inputs(seed, lens, H, d, W, k, nh, dI, swa_lens):
    g = torch.Generator(device=dev()).manual_seed(seed)
    B, G = len(lens), sum(lens)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int64, device=dev())
    return dict(
        cu=cu, B=B, G=G, H=H, d=d, W=W, k=k, max_g=max(max(lens), 0),
        keys=_randn(g, max(G, 1), dI, scale=3.0)[:G], comp=_randn(g, max(G, 1), d)[:G],
        q=_randn(g, B, H, d), qI=_randn(g, B, nh, dI), w=torch.rand(B, nh, generator=g, device=dev()),
        swa=_randn(g, B, W, d), swa_len=torch.tensor(swa_lens, dtype=torch.int32, device=dev()))


def _two_calls(x):
    scores = torch.full((x["G"],), float("nan"), dtype=torch.float32, device=dev())
    topk, _ = chs.index_topk(x["qI"], x["w"], x["keys"], x["cu"], x["k"], x["max_g"], scores)
    out, lse = chs.decode_attn(x["q"], x["swa"], x["swa_len"], x["comp"], x["cu"], topk, x["d"] ** -0.5, x["max_g"])
    return scores, topk, out, lse


def _fused(x):
    scores = torch.full((x["G"],), float("nan"), dtype=torch.float32, device=dev())
    topk, out, lse, _ = chs.decode_step(x["qI"], x["w"], x["keys"], x["q"], x["swa"], x["swa_len"], x["comp"],
                                        x["cu"], x["k"], x["d"] ** -0.5, x["max_g"], scores)
    return scores, topk, out, lse


def _same(a, b, what):
    for name, u, v in zip(("scores", "topk", "out", "lse"), a, b):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v), f"{what}: {name} differs"


CASES = [
    # seed, lens, H, d, W, k, idx heads, idx dim, swa_lens
    (1, [256], 8, 64, 128, 64, 2, 32, [128]),
    (2, [30000, 9000], 64, 512, 128, 512, 4, 128, [128, 77]),
    (3, [300, 5000], 64, 512, 128, 512, 4, 128, [128, 128]),
    (4, [0, 4000, 1], 24, 128, 64, 100, 4, 64, [5, 64, 0]),
    (5, [20000], 72, 256, 128, 512, 8, 128, [0]),
    (6, [70000], 64, 512, 128, 2048, 4, 128, [128]),
    # more than one selection tile (8192 groups of 32 candidates) in one sequence
    (7, [300000, 2000], 16, 64, 64, 512, 4, 128, [64, 10]),
    # more selecting workgroups than CUs: one workgroup per 64 heads (the second one partly past H)
    (8, [1000 + 97 * i for i in range(24)], 72, 128, 32, 128, 4, 64, [32, 7, 0, 32] * 6),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_decode_step_equals_two_calls(case):
    seed, lens, H, d, W, k, nh, dI, swa_lens = case
    print(f"case: decode_step seed {seed} lens {lens} H {H} d {d} W {W} k {k}", flush=True)
    x = _inputs(seed, lens, H, d, W, k, nh, dI, swa_lens)
    want = _two_calls(x)
    got = _fused(x)
    torch.cuda.synchronize()
    _same(got, want, f"seed {seed}")
    again = _fused(x)
    _same(again, got, f"seed {seed} repeat")


def test_decode_step_graph_replays_bitwise():
    print("case: decode_step graph replay", flush=True)
    x = _inputs(11, [40000, 12000], 64, 512, 128, 512, 4, 128, [128, 90])
    scores = torch.empty(x["G"], dtype=torch.float32, device=dev())
    topk = torch.empty(x["B"], x["k"], dtype=torch.int32, device=dev())
    out = torch.empty(x["B"], x["H"], x["d"], dtype=torch.float32, device=dev())
    lse = torch.empty(x["B"], x["H"], dtype=torch.float32, device=dev())
    ws = chs.decode_step_workspace(x["B"], x["H"], x["d"], x["W"], x["k"], x["max_g"], dev())

    def step():
        chs.decode_step(x["qI"], x["w"], x["keys"], x["q"], x["swa"], x["swa_len"], x["comp"], x["cu"], x["k"],
                        x["d"] ** -0.5, x["max_g"], scores, ws, topk, out, lse)

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
        y = torch.randn(1 << 20, device=dev())
        _ = (y * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same([scores, topk, out, lse], want, f"replay {r}")
