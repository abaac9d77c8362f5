"""chs_decode_step_noalloc (the decode step for callers that cannot allocate: its scratch is the
library's per-GPU array) against chs_decode_step with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, each bit-identical to chs_decode_step on the same
inputs (the same kernels, so every output matches to the bit); an input whose workspace would
exceed the array is refused before anything is launched."""
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
from chs_testutil import dev

pytestmark = pytest.mark.gpu


def _inputs(seed, lens, H, d, W, k, nh, dI, swa_lens):
    g = torch.Generator(device=dev()).manual_seed(seed)
    r = lambda *s, scale=1.0: (torch.randn(*s, generator=g, device=dev()) * scale).to(torch.bfloat16)  # noqa: E731
    B, G = len(lens), sum(lens)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int64, device=dev())
    return dict(cu=cu, B=B, G=G, H=H, d=d, W=W, k=k, max_g=max(lens), keys=r(G, dI, scale=3.0), comp=r(G, d),
                q=r(B, H, d), qI=r(B, nh, dI), w=torch.rand(B, nh, generator=g, device=dev()), swa=r(B, W, d),
                swa_len=torch.tensor(swa_lens, dtype=torch.int32, device=dev()))


def _run(fn, x, **extra):
    scores = torch.full((x["G"],), float("nan"), dtype=torch.float32, device=dev())
    topk, out, lse, _ = fn(x["qI"], x["w"], x["keys"], x["q"], x["swa"], x["swa_len"], x["comp"], x["cu"], x["k"],
                           x["d"] ** -0.5, x["max_g"], scores, **extra)
    return scores, topk, out, lse


def _same(a, b, what):
    for name, u, v in zip(("scores", "topk", "out", "lse"), a, b):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v), f"{what}: {name} differs"


def test_noalloc_step_equals_step_twice_then_smaller():
    big = _inputs(21, [262144], 64, 512, 128, 512, 4, 128, [128])
    small = _inputs(22, [3000, 0, 777], 24, 128, 64, 100, 4, 64, [64, 0, 13])
    for name, x in (("1M-token step", big), ("smaller step", small)):
        print(f"case: noalloc {name} lens {x['cu'].tolist()}", flush=True)
        want = _run(chs.decode_step, x)
        got = _run(chs.decode_step_noalloc, x)
        torch.cuda.synchronize()
        _same(got, want, name)
    # The second, smaller call left the first call's larger contents behind in the array; the first
    # input again still matches.
    print("case: noalloc 1M-token step again", flush=True)
    _same(_run(chs.decode_step_noalloc, big), _run(chs.decode_step, big), "1M-token step again")
    torch.cuda.synchronize()


def test_noalloc_step_refuses_inputs_beyond_the_scratch():
    print("case: noalloc oversized", flush=True)
    x = _inputs(23, [1000] * 4, 16, 64, 64, 64, 2, 64, [64] * 4)
    limit = 64 << 20
    need = chs.lib().chs_decode_step_workspace_size(4, 16, 64, 64, 64, 1 << 22)
    assert need > limit
    with pytest.raises(chs.ChsError) as e:
        # max_comp (a host bound) sizes the workspace: 4 sequences of up to 4M candidates need more
        chs.decode_step_noalloc(x["qI"], x["w"], x["keys"], x["q"], x["swa"], x["swa_len"], x["comp"], x["cu"], 64,
                                max_comp=1 << 22)
    assert e.value.status == 4   # CHS_ERR_WORKSPACE
    torch.cuda.synchronize()
