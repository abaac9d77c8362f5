"""The five synthetic workloads the tests and the benchmark run, and their seeded inputs.

Shapes follow the pages' statement of the method (sources, by page title and section):
  "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥: a 128-token sliding window per
  layer, with either 4:1 compression plus top-512 selection (C4) or 128:1 compression attended
  densely (C128); Kernel 層一堆狠活: at 1M context the indexer picks 512 of 256K candidates.
The remaining sizes and distributions (heads, latent width, indexer heads and width, value
distributions, batch mixes) are this project's workload definitions, stated per workload below.

Tensor ids inside one layer (offset by the layer's tensor_base):
  1 token vectors X, 2 gate logits Z, 3 per-slot bias B, 4 queries q, 5 indexer queries q_I,
  6 indexer head weights w, 7 index-key noise, 8 spike loadings A, 9 spike basis U.
Workload-level ids: 10 length jitter, 11 duplicate positions, 12 duplicate sources,
  13 standalone scores, 14 tie positions.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

from . import (gpu_index_keys, gpu_normal, gpu_uniform, index_keys, normal, permutation_prefix,
               spike_basis, uniform, uniform01_f64)

T_X, T_Z, T_B, T_Q, T_QI, T_W, T_KN, T_KA, T_KU = 1, 2, 3, 4, 5, 6, 7, 8, 9
T_JITTER, T_DUPPOS, T_DUPSRC, T_SCORES, T_TIEPOS = 10, 11, 12, 13, 14
N_SPIKE = 4


@dataclass(frozen=True)
class Layer:
    kind: str                 # "c4" (top-k selected) or "c128" (dense)
    m: int                    # compression ratio (group size)
    k: Optional[int]          # top-k for C4 layers; None for dense layers
    tensor_base: int = 0


@dataclass(frozen=True)
class Workload:
    index: int                # 1-based workload number
    name: str
    dtype: str                # "f32" or "bf16": storage type of X, Z, q, q_I, K_I, compressed KV
    lengths: Tuple[int, ...]  # tokens per sequence, N_b
    window: int               # sliding-window length W
    heads: int                # query heads H
    d: int                    # shared latent width (K = V)
    idx_heads: int            # indexer heads
    idx_dim: int              # indexer key width
    gate_std: float
    bias_std: float
    spike_alpha: float        # 0: index keys are plain N(0,1)
    layers: Tuple[Layer, ...]
    topk_len: int = 0         # length of the standalone top-k score rows (0: none)
    note: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def batch(self) -> int:
        return len(self.lengths)

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    def cu_tokens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)

    def groups(self, layer: Layer) -> np.ndarray:
        return np.array([n // layer.m for n in self.lengths], dtype=np.int64)

    def cu_groups(self, layer: Layer) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.groups(layer))]).astype(np.int64)

    def swa_len(self) -> np.ndarray:
        return np.array([min(n, self.window) for n in self.lengths], dtype=np.int32)


def _jittered(seed: int, n: int, base: int, frac: float) -> Tuple[int, ...]:
    u = uniform01_f64(seed, T_JITTER, 0, n)
    return tuple(int(np.floor(base * (1.0 + (ui * 2.0 - 1.0) * frac) + 0.5)) for ui in u)


def workload(i: int) -> Workload:
    """Workload i (1..5)."""
    if i == 1:
        return Workload(1, "tiny_c4_f32", "f32", (1024,), 128, 8, 64, 2, 32, 1.0, 0.1, 0.0,
                        (Layer("c4", 4, 64),),
                        note="fp32; N=1024, m=4 -> 256 entries; top-64; H=8, d=64; indexer 2x32")
    if i == 2:
        return Workload(2, "c4_128k_bf16", "bf16", (131072,), 128, 64, 512, 4, 128, 2.0, 0.1, 8.0,
                        (Layer("c4", 4, 512),),
                        note="bf16; N=131072 -> 32768 entries; top-512; H=64, d=512; indexer 4x128")
    if i == 3:
        return Workload(3, "c128_1m_bs4_bf16", "bf16", (1048576,) * 4, 128, 64, 512, 4, 128, 2.0, 0.1,
                        8.0, (Layer("c128", 128, None),),
                        note="bf16; 4 x 1M tokens, m=128 -> 4 x 8192 entries, all attended")
    if i == 4:
        return Workload(4, "c4_1m_bf16", "bf16", (1048576,), 128, 64, 512, 4, 128, 2.0, 0.1, 8.0,
                        (Layer("c4", 4, 512),), topk_len=262144,
                        note="bf16; 1M tokens -> 262144 candidates; top-512; H=64, d=512; indexer 4x128")
    if i == 5:
        return Workload(5, "mixed_bs64_200k_bf16", "bf16", _jittered(1005, 64, 200000, 0.05), 128, 64,
                        512, 4, 128, 2.0, 0.1, 8.0,
                        (Layer("c4", 4, 512, 0), Layer("c128", 128, None, 100)),
                        note="bf16; 64 sequences of 200000 +-5% tokens; one C4 and one C128 layer")
    raise ValueError(f"no workload {i}")


def small_workload(dtype: str, lengths, m: int, k: Optional[int], window=128, heads=8, d=64,
                   idx_heads=2, idx_dim=32, seed_index=90, gate_std=1.0, spike_alpha=0.0) -> Workload:
    """A reduced workload for parity tests at sizes the oracle finishes in seconds."""
    layer = Layer("c4" if k is not None else "c128", m, k)
    return Workload(seed_index, f"small_{dtype}_{m}", dtype, tuple(int(n) for n in lengths), window,
                    heads, d, idx_heads, idx_dim, gate_std, 0.1, spike_alpha, (layer,))


# ------------------------------------------------------------------ host inputs (numpy)
def host_tokens(wl: Workload, layer: Layer, which: int, b: int, t0: int, t1: int) -> np.ndarray:
    """Rows [t0, t1) of sequence b of X (which=T_X) or Z (which=T_Z), as fp32 [t1-t0, d]."""
    cu = wl.cu_tokens()
    t0, t1 = int(t0), int(t1)      # Python ints: no fixed-width overflow in the offsets
    std = 1.0 if which == T_X else wl.gate_std
    start = (int(cu[b]) + t0) * wl.d
    return normal(wl.seed, layer.tensor_base + which, start, (t1 - t0) * wl.d, 0.0, std,
                  wl.bf16).reshape(t1 - t0, wl.d)


def host_all_tokens(wl: Workload, layer: Layer, which: int) -> np.ndarray:
    T = int(wl.cu_tokens()[-1])
    std = 1.0 if which == T_X else wl.gate_std
    return normal(wl.seed, layer.tensor_base + which, 0, T * wl.d, 0.0, std, wl.bf16).reshape(T, wl.d)


def host_bias(wl: Workload, layer: Layer) -> np.ndarray:
    return normal(wl.seed, layer.tensor_base + T_B, 0, layer.m * wl.d, 0.0, wl.bias_std,
                  False).reshape(layer.m, wl.d)


def host_q(wl: Workload, layer: Layer) -> np.ndarray:
    return normal(wl.seed, layer.tensor_base + T_Q, 0, wl.batch * wl.heads * wl.d, 0.0, 1.0,
                  wl.bf16).reshape(wl.batch, wl.heads, wl.d)


def host_qidx(wl: Workload, layer: Layer) -> np.ndarray:
    return normal(wl.seed, layer.tensor_base + T_QI, 0, wl.batch * wl.idx_heads * wl.idx_dim, 0.0,
                  1.0, wl.bf16).reshape(wl.batch, wl.idx_heads, wl.idx_dim)


def host_w(wl: Workload, layer: Layer) -> np.ndarray:
    return uniform(wl.seed, layer.tensor_base + T_W, 0, wl.batch * wl.idx_heads, 0.0,
                   1.0).reshape(wl.batch, wl.idx_heads)


def host_basis(wl: Workload, layer: Layer) -> np.ndarray:
    return spike_basis(wl.seed, layer.tensor_base + T_KU, N_SPIKE, wl.idx_dim)


def host_index_keys(wl: Workload, layer: Layer, b: int, j0: int, j1: int) -> np.ndarray:
    """Rows [j0, j1) of sequence b's index keys, fp32 [j1-j0, idx_dim]."""
    j0, j1 = int(j0), int(j1)
    row0 = int(wl.cu_groups(layer)[b]) + j0
    if wl.spike_alpha == 0.0:
        return normal(wl.seed, layer.tensor_base + T_KN, row0 * wl.idx_dim, (j1 - j0) * wl.idx_dim,
                      0.0, 1.0, wl.bf16).reshape(j1 - j0, wl.idx_dim)
    return index_keys(wl.seed, layer.tensor_base + T_KN, layer.tensor_base + T_KA, row0, j1 - j0,
                      wl.idx_dim, host_basis(wl, layer), wl.spike_alpha, wl.bf16)


def topk_scores(wl: Workload, variant: str, row: int = 0) -> np.ndarray:
    """A standalone fp32 score row of length wl.topk_len.
    variant "normal": N(0,1). "dup10": 10% of positions (distinct, seeded shuffle) take the
    value of a uniformly chosen position outside that set, so they are bitwise duplicates.
    "tie64": 64 positions take the value of the 512th largest score of the "normal" row."""
    n = wl.topk_len
    s = normal(wl.seed, T_SCORES, row * n, n)
    if variant == "normal":
        return s
    if variant == "dup10":
        nd = n // 10
        perm = permutation_prefix(wl.seed, T_DUPPOS + 16 * row, n, nd)
        chosen, rest = perm[:nd], perm[nd:]
        src = rest[(uniform01_f64(wl.seed, T_DUPSRC + 16 * row, 0, nd) * len(rest)).astype(np.int64)]
        s[chosen] = s[src]
        return s
    if variant == "tie64":
        tau = np.sort(s)[::-1][511]
        pos = permutation_prefix(wl.seed, T_TIEPOS + 16 * row, n, 64)[:64]
        s[pos] = tau
        return s
    raise ValueError(variant)


# ------------------------------------------------------------------ device inputs (torch)
def device_inputs(wl: Workload, layer: Layer, device="cuda", with_tokens=True, with_index=True):
    """Generate one layer's inputs directly in device memory (same bits as the host fillers).
    Returns a dict of torch tensors; token and index tensors are packed over the batch."""
    import torch
    dt = torch.bfloat16 if wl.bf16 else torch.float32
    cu = wl.cu_tokens()
    T = int(cu[-1])
    out = {"cu_tokens": torch.tensor(cu, dtype=torch.int64, device=device)}
    cug = wl.cu_groups(layer)
    out["cu_groups"] = torch.tensor(cug, dtype=torch.int64, device=device)
    tb = layer.tensor_base
    if with_tokens:
        out["X"] = gpu_normal(torch.empty(T, wl.d, dtype=dt, device=device), wl.seed, tb + T_X)
        out["Z"] = gpu_normal(torch.empty(T, wl.d, dtype=dt, device=device), wl.seed, tb + T_Z, 0, 0.0,
                              wl.gate_std)
    out["bias"] = torch.from_numpy(host_bias(wl, layer)).to(device)
    out["q"] = gpu_normal(torch.empty(wl.batch, wl.heads, wl.d, dtype=dt, device=device), wl.seed, tb + T_Q)
    # The window holds the last min(N_b, W) tokens of each sequence, generated straight from X's
    # stream at the same element indices.
    swa = torch.zeros(wl.batch, wl.window, wl.d, dtype=dt, device=device)
    swa_len = wl.swa_len()
    for b, n in enumerate(wl.lengths):
        L = int(swa_len[b])
        if L:
            start = (int(cu[b]) + n - L) * wl.d
            view = torch.empty(L, wl.d, dtype=dt, device=device)
            gpu_normal(view, wl.seed, tb + T_X, start)
            swa[b, :L] = view
    out["swa_kv"] = swa
    out["swa_len"] = torch.tensor(swa_len, dtype=torch.int32, device=device)
    if with_index and layer.k is not None:
        G = int(cug[-1])
        out["q_idx"] = gpu_normal(torch.empty(wl.batch, wl.idx_heads, wl.idx_dim, dtype=dt, device=device),
                                  wl.seed, tb + T_QI)
        out["w"] = gpu_uniform(torch.empty(wl.batch, wl.idx_heads, dtype=torch.float32, device=device),
                               wl.seed, tb + T_W)
        keys = torch.empty(max(G, 1), wl.idx_dim, dtype=dt, device=device)[:G]
        if G:
            if wl.spike_alpha == 0.0:
                gpu_normal(keys, wl.seed, tb + T_KN)
            else:
                U = torch.from_numpy(host_basis(wl, layer)).to(device)
                gpu_index_keys(keys, wl.seed, tb + T_KN, tb + T_KA, 0, U, wl.spike_alpha)
        out["k_idx"] = keys
    return out
