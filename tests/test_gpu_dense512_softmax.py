"""The running maximum of the d = 512, many-head attention kernel under crafted logit profiles.

That kernel moves a head's reference maximum only when a 32-key chunk exceeds it by more than 8
(base-2 logits), and its consumers skip the rescale whenever every factor is 1. These cases drive
that rule through its branches, against the oracle at the bf16-path tolerances:
- a spike of large logits in a late chunk (some heads far above the reference, others far below);
- a ramp, the logits rising across the whole sequence, so the reference moves many times;
- a spike in the first chunk and nothing near it afterwards (every later P underflows);
- the spike inside the window rows;
- the same through paged pools, and for the selected entries at many sequences (the 64-head
  selected form), the selection holding the spike rows.

Construction: u is a fixed unit vector; head h's query is N(0, 1) plus gamma_h u with gamma_h spread
over [-30, 30], so a key beta u adds about 0.064 beta gamma_h to the head's base-2 logit (scale
1 / sqrt(512)). Background keys are N(0, 0.3^2) per element. Values stay of order 1, so the bf16
path's absolute tolerance applies as everywhere else.
"""
import numpy as np
import pytest
import torch

import compressed_hybrid_sparse_amd as chs
import oracle
from chs_testutil import assert_bf16_path, assert_lse, dev

pytestmark = pytest.mark.gpu

D, W = 512, 128


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).bfloat16()


def _queries(rng, B, H, u):
    gamma = np.linspace(-30.0, 30.0, H)
    rng.shuffle(gamma)
    return rng.standard_normal((B, H, D)) + gamma[None, :, None] * u[None, None, :]


def _keys(rng, n, u, profile):
    k = 0.3 * rng.standard_normal((n, D))
    if profile == "late_spike":
        a = int(n * 0.6)
        k[a:a + 5] += 22.0 * u
    elif profile == "ramp":
        k += (22.0 * np.arange(n) / max(n - 1, 1))[:, None] * u[None, :]
    elif profile == "early_spike":
        k[1:4] += 22.0 * u
    elif profile == "flat":
        pass
    else:
        raise ValueError(profile)
    return k


def _reference_moves(q, keys):
    """How often, walking the keys in 32-key chunks, a head's chunk maximum exceeds its reference
    maximum by more than 8 (base 2) after the first chunk: the inputs must drive that branch."""
    x = (q @ keys.T) * D ** -0.5 * 1.4426950408889634
    ref = x[:, :32].max(1)
    moves = 0
    for c0 in range(32, x.shape[1], 32):
        cm = x[:, c0:c0 + 32].max(1)
        up = cm > ref + 8.0
        moves += int(up.sum())
        ref = np.where(up, cm, ref)
    return moves


def _check(out, lse, q, swa_rows, comp_rows, sel, what):
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(q.shape[0]):
        keys = oracle.step_keys(swa_rows[b], comp_rows[b], None if sel is None else sel[b])
        o_ref, l_ref = oracle.attend(q[b], keys, D ** -0.5)
        assert_bf16_path(og[b], o_ref, f"{what} b={b}")
        assert_lse(lg[b], l_ref, f"{what} lse b={b}")


@pytest.mark.parametrize("H", [64, 100])
def test_dense512_logit_profiles(H):
    print(f"case: dense d=512 logit profiles H={H}", flush=True)
    rng = np.random.default_rng(512 + H)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    # 32 sequences, so each split holds several 32-key chunks (4 to 18) and the running maximum
    # evolves inside a split, not only across the merge.
    profiles = ["late_spike", "ramp", "early_spike", "flat"] * 8
    lens = [int(x) for x in rng.integers(1200, 2000, 32)]
    lens[3], lens[7] = 33, 0
    B = len(lens)
    q = _bf(_queries(rng, B, H, u))
    win = 0.3 * rng.standard_normal((B, W, D))
    win[3, 50:52] += 22.0 * u                          # the spike in the window rows
    swa = _bf(win)
    comp = _bf(np.concatenate([_keys(rng, n, u, p) for n, p in zip(lens, profiles)]))
    sl = torch.tensor([W if b % 5 else 37 for b in range(B)], dtype=torch.int32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    out, lse = chs.decode_attn(q.to(dev()), swa.to(dev()), sl.to(dev()), comp.to(dev()), cu.to(dev()), None)
    torch.cuda.synchronize()
    qh, sh, ch = q.float().numpy(), swa.float().numpy(), comp.float().numpy()
    cuh = cu.numpy()
    assert sum(_reference_moves(qh[b], np.concatenate([sh[b, :int(sl[b])], ch[cuh[b]:cuh[b + 1]]]))
               for b in range(B)) > 100
    _check(out, lse, qh, [sh[b, :int(sl[b])] for b in range(B)], [ch[cuh[b]:cuh[b + 1]] for b in range(B)], None,
           f"dense H={H}")


def test_dense512_logit_profiles_paged():
    print("case: dense d=512 logit profiles, paged", flush=True)
    rng = np.random.default_rng(7)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    H, P = 64, 64
    profiles = ["ramp", "late_spike", "early_spike", "flat"] * 4
    lens = [int(x) for x in rng.integers(300, 1600, 16)]
    B = len(lens)
    q = _bf(_queries(rng, B, H, u))
    swa = _bf(0.3 * rng.standard_normal((B, W, D)))
    rows = [_keys(rng, n, u, p) for n, p in zip(lens, profiles)]
    need = [(n + P - 1) // P for n in lens]
    npages = sum(need) + 3
    perm = rng.permutation(npages)
    pool = np.zeros((npages * P, D))
    pt = np.full((B, max(need)), -1, np.int32)
    p0 = 0
    for b, n in enumerate(lens):
        for i in range(need[b]):
            pg = int(perm[p0 + i])
            pt[b, i] = pg
            e = min(n, (i + 1) * P)
            pool[pg * P:pg * P + e - i * P] = rows[b][i * P:e]
        p0 += need[b]
    poolb = _bf(pool)
    sl = torch.full((B,), W, dtype=torch.int32)
    out, lse = chs.decode_attn_paged(q.to(dev()), swa.to(dev()), torch.arange(B, dtype=torch.int32).to(dev()),
                                     sl.to(dev()), poolb.to(dev()), P, torch.from_numpy(pt).to(dev()),
                                     torch.tensor(lens, dtype=torch.int64).to(dev()), None, None, max(lens))
    torch.cuda.synchronize()
    ph = poolb.float().numpy()
    comp_rows = []
    for b, n in enumerate(lens):
        comp_rows.append(np.concatenate([ph[int(pt[b, i]) * P:int(pt[b, i]) * P + P] for i in range(need[b])])[:n])
    _check(out, lse, q.float().numpy(), [swa.float().numpy()[b] for b in range(B)], comp_rows, None, "paged dense")


def test_dense512_selected_profiles_many_sequences():
    # 24 sequences of 72 heads: the selected entries go through the 64-head d = 512 kernel (the
    # second head group partly past H). Each selection holds its sequence's spike rows at scattered
    # positions, so a late chunk of the selected list carries the spike.
    print("case: dense d=512 selected entries, logit profiles, 24 sequences", flush=True)
    rng = np.random.default_rng(24)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    B, H, k = 24, 72, 320
    lens = [900 + 37 * i for i in range(B)]
    profiles = ["late_spike", "ramp", "early_spike", "flat"]
    q = _bf(_queries(rng, B, H, u))
    swa = _bf(0.3 * rng.standard_normal((B, W, D)))
    comp = _bf(np.concatenate([_keys(rng, n, u, profiles[b % 4]) for b, n in enumerate(lens)]))
    cu = np.concatenate([[0], np.cumsum(lens)])
    sel = np.stack([np.sort(rng.choice(n, k, replace=False)) for n in lens]).astype(np.int32)
    for b, n in enumerate(lens):
        if profiles[b % 4] == "late_spike":
            a = int(n * 0.6)
            sel[b, -8:-3] = np.arange(a, a + 5)          # the spike rows, late in the list
        elif profiles[b % 4] == "early_spike":
            sel[b, :3] = [1, 2, 3]
    sl = torch.tensor([W - (b % 3) * 40 for b in range(B)], dtype=torch.int32)
    out, lse = chs.decode_attn(q.to(dev()), swa.to(dev()), sl.to(dev()), comp.to(dev()),
                               torch.from_numpy(cu).to(dev()), torch.from_numpy(sel).to(dev()))
    torch.cuda.synchronize()
    qh, sh, ch = q.float().numpy(), swa.float().numpy(), comp.float().numpy()
    _check(out, lse, qh, [sh[b, :int(sl[b])] for b in range(B)], [ch[cu[b]:cu[b + 1]] for b in range(B)], sel,
           "selected")
