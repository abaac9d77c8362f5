"""The binding refuses buffers smaller than what a call addresses, before anything is launched:
an undersized tensor would otherwise be read or written out of bounds on the device."""
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
from chs_testutil import dev

pytestmark = pytest.mark.gpu


def _bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16, device=dev())


def test_undersized_buffers_raise_before_launch():
    print("case: binding size checks", flush=True)
    cu = torch.tensor([0, 100, 300], dtype=torch.int64, device=dev())
    # compress: output rows below cu_groups[-1], tokens below cu_tokens[-1]
    x = _bf(1200, 64)
    cut = torch.tensor([0, 400, 1200], dtype=torch.int64, device=dev())
    cug = torch.tensor([0, 100, 300], dtype=torch.int64, device=dev())
    bias = torch.zeros(4, 64, device=dev())
    with pytest.raises(ValueError):
        chs.compress(x, x, bias, 4, cut, cug, out=_bf(299, 64))
    with pytest.raises(ValueError):
        chs.compress(x[:1100], x[:1100], bias, 4, cut, cug)
    with pytest.raises(ValueError):
        chs.compress(x, x, torch.zeros(3, 64, device=dev()), 4, cut, cug)
    # index_topk: keys and scores below cu[-1], a top-k buffer of the wrong shape
    q = _bf(2, 4, 64)
    w = torch.ones(2, 4, device=dev())
    with pytest.raises(ValueError):
        chs.index_topk(q, w, _bf(299, 64), cu, 16)
    with pytest.raises(ValueError):
        chs.index_topk(q, w, _bf(300, 64), cu, 16, scores=torch.zeros(299, device=dev()))
    with pytest.raises(ValueError):
        chs.index_topk(q, w, _bf(300, 64), cu, 16, out=torch.zeros(2, 15, dtype=torch.int32, device=dev()))
    with pytest.raises(ValueError):
        chs.topk_from_scores(torch.zeros(299, device=dev()), cu, 16)
    # decode_attn: entries below cu[-1], outputs of the wrong shape, a window per sequence
    qa = _bf(2, 16, 64)
    swa = _bf(2, 8, 64)
    sl = torch.full((2,), 8, dtype=torch.int32, device=dev())
    tk = torch.zeros(2, 16, dtype=torch.int32, device=dev())
    with pytest.raises(ValueError):
        chs.decode_attn(qa, swa, sl, _bf(299, 64), cu, tk)
    with pytest.raises(ValueError):
        chs.decode_attn(qa, swa, sl, _bf(300, 64), cu, tk, out=torch.zeros(2, 16, 63, device=dev()))
    with pytest.raises(ValueError):
        chs.decode_attn(qa, swa[:1], sl, _bf(300, 64), cu, tk)
    with pytest.raises(ValueError):
        chs.decode_attn(qa, swa, sl, _bf(300, 64), cu, tk[:, :8].contiguous()[:1])
    # decode_step: keys below cu[-1]
    with pytest.raises(ValueError):
        chs.decode_step(q, w, _bf(299, 64), qa, swa, sl, _bf(300, 64), cu, 16)
    # gather: a working set of the wrong shape
    with pytest.raises(ValueError):
        chs.gather_selected(_bf(300, 64), cu, tk, work=_bf(31, 64))
    torch.cuda.synchronize()
    # the same calls with correct sizes run
    chs.decode_attn(qa, swa, sl, _bf(300, 64), cu, tk)
    chs.index_topk(q, w, _bf(300, 64), cu, 16)
    torch.cuda.synchronize()
