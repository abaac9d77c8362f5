"""CPU oracle for one decode step of one hybrid-sparse-attention layer.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package. The GPU library never calls it, and it never calls the GPU library.

The arithmetic lives in oracle.c (plain C loops in double precision). This module marshals
numpy arrays and assembles the key set of one decode step (window rows plus the selected
compressed entries), which is a matter of choosing rows, not of arithmetic.

Sources (web pages, cited by title and section):
  "DeepSeek-V4 本地部署，SGLang 把活做絕了", V4 到底改了啥 (SWA of 128 tokens plus C4 top-512 or
  C128 dense per layer) and Kernel 層一堆狠活 (one attention call over window and compressed
  entries); "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 2 (compressor stages;
  threshold top-k) and 创新 3 (every C128 entry is read each step).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        # CHS_ORACLE_LIB names another build of oracle.c: the mutation tests load copies with a
        # planted mistake to show that the pins catch it.
        path = os.environ.get("CHS_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run oracle/build.py")
        lib = ctypes.CDLL(path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_compress.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _p, _p, _p, _p, _p]
        lib.oracle_index_scores.argtypes = [ctypes.c_int32, ctypes.c_int32, _p, _p, ctypes.c_int64, _p, _p]
        lib.oracle_decode_e4m3_n.argtypes = [ctypes.c_int64, _p, _p]
        lib.oracle_index_scores_fp8.argtypes = [ctypes.c_int32, ctypes.c_int32, _p, _p, ctypes.c_int64, _p, _p, _p]
        lib.oracle_attend_fp8.argtypes = [ctypes.c_int32, ctypes.c_int32, _p, ctypes.c_int64, _p, _p, ctypes.c_double,
                                          _p, _p]
        lib.oracle_topk.argtypes = [_p, ctypes.c_int64, ctypes.c_int32, _p]
        lib.oracle_topk.restype = ctypes.c_int32
        lib.oracle_attend.argtypes = [ctypes.c_int32, ctypes.c_int32, _p, ctypes.c_int64, _p, ctypes.c_double,
                                      _p, _p]
        lib.oracle_round_bf16.argtypes = [_p, ctypes.c_int64, _p]
        lib.oracle_encode_e4m3_n.argtypes = [ctypes.c_int64, _p, _p]
        lib.oracle_quantize_e4m3_rows.argtypes = [ctypes.c_int64, ctypes.c_int32, _p, _p, _p]
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def compress(X, Z, B, m: int, cu_tokens) -> np.ndarray:
    """Group softmax-pool of every complete group (see oracle.c). X, Z: [T, d]; B: [m, d];
    cu_tokens: [batch+1]. Returns the unrounded double rows [sum_b floor(N_b/m), d]."""
    X, Z, B = _f32(X), _f32(Z), _f32(B)
    cu = np.ascontiguousarray(cu_tokens, dtype=np.int64)
    T, d = X.shape
    assert Z.shape == (T, d) and B.shape == (m, d) and cu[-1] <= T and 1 <= m <= 1024
    G = int(sum((cu[b + 1] - cu[b]) // m for b in range(len(cu) - 1)))
    out = np.zeros((G, d), dtype=np.float64)
    _load().oracle_compress(len(cu) - 1, d, m, _ptr(X), _ptr(Z), _ptr(B), _ptr(cu), _ptr(out))
    return out


def round_bf16(x) -> np.ndarray:
    """Double -> nearest bfloat16 (ties to even), returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    _load().oracle_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def store(x, bf16: bool) -> np.ndarray:
    """The value a compressed entry holds once stored in the input precision."""
    return round_bf16(x) if bf16 else np.asarray(x, dtype=np.float64).astype(np.float32)


def index_scores(q, w, K) -> np.ndarray:
    """s_j = sum_h w_h ReLU(q_h . K_j) in double. q: [nh, dim]; w: [nh]; K: [n, dim]."""
    q, w, K = _f32(q), _f32(w), _f32(K)
    nh, dim = q.shape
    n = K.shape[0]
    assert w.shape == (nh,) and (n == 0 or K.shape[1] == dim)
    s = np.zeros(n, dtype=np.float64)
    _load().oracle_index_scores(nh, dim, _ptr(q), _ptr(w), n, _ptr(K.reshape(max(n, 0), dim)), _ptr(s))
    return s


def decode_e4m3(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8 array) as doubles; see oracle.c."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_decode_e4m3_n(c.size, _ptr(c), _ptr(out))
    return out


def encode_e4m3(y) -> np.ndarray:
    """fp32 values -> E4M3 codes: nearest value, ties to the even code, saturating at +-448."""
    y = _f32(y)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_encode_e4m3_n(y.size, _ptr(y), _ptr(out))
    return out


def quantize_e4m3(rows):
    """Per-row E4M3 quantisation of fp32 rows [n, d] (see oracle.c): returns (codes [n, d] uint8,
    scales [n] fp32), row r = scales[r] * decode(codes[r])."""
    x = _f32(rows)
    n, d = x.shape
    codes = np.empty((n, d), dtype=np.uint8)
    scales = np.empty(n, dtype=np.float32)
    _load().oracle_quantize_e4m3_rows(n, d, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def index_scores_fp8(q, w, K8, scale) -> np.ndarray:
    """s_j = sum_h w_h ReLU(q_h . (scale_j * decode(K8_j))) in double. K8: [n, dim] uint8 E4M3
    codes; scale: [n] fp32."""
    q, w = _f32(q), _f32(w)
    K8 = np.ascontiguousarray(K8, dtype=np.uint8)
    scale = _f32(scale)
    nh, dim = q.shape
    n = K8.shape[0]
    assert w.shape == (nh,) and scale.shape == (n,) and (n == 0 or K8.shape[1] == dim)
    s = np.zeros(n, dtype=np.float64)
    _load().oracle_index_scores_fp8(nh, dim, _ptr(q), _ptr(w), n, _ptr(K8.reshape(max(n, 0), dim)), _ptr(scale),
                                    _ptr(s))
    return s


def topk(scores, k: int) -> np.ndarray:
    """The k largest scores (ties to the lower index), ascending, padded with -1."""
    s = _f32(scores)
    out = np.empty(k, dtype=np.int32)
    cnt = _load().oracle_topk(_ptr(s), s.size, k, _ptr(out))
    if cnt < 0:
        raise ValueError("NaN score: outside the top-k contract")
    return out


def attend(q, keys, scale: float):
    """One softmax over `keys` (which are also the values) for every query row.
    q: [H, d]; keys: [n, d]. Returns (out [H, d] double, lse [H] double)."""
    q, keys = _f32(q), _f32(keys)
    H, d = q.shape
    n = keys.shape[0]
    out = np.zeros((H, d), dtype=np.float64)
    lse = np.zeros(H, dtype=np.float64)
    _load().oracle_attend(H, d, _ptr(q), n, _ptr(keys.reshape(max(n, 0), d)), scale, _ptr(out), _ptr(lse))
    return out, lse


def attend_fp8(q, codes, scales, scale: float):
    """attend() over FP8 key rows: key row i is scales[i] * decode(codes[i]) (exact, in double).
    q: [H, d]; codes: [n, d] uint8 E4M3; scales: [n] fp32."""
    q = _f32(q)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _f32(scales)
    H, d = q.shape
    n = codes.shape[0]
    out = np.zeros((H, d), dtype=np.float64)
    lse = np.zeros(H, dtype=np.float64)
    _load().oracle_attend_fp8(H, d, _ptr(q), n, _ptr(codes.reshape(max(n, 0), d)), _ptr(scales), scale, _ptr(out),
                              _ptr(lse))
    return out, lse


def step_keys(window_rows, comp_rows, sel=None) -> np.ndarray:
    """Key set of one decode step: the window rows (the last min(N_b, W) raw tokens, current
    token included) followed by the compressed entries comp_rows[j] for every j in `sel` with
    0 <= j < len(comp_rows) (entries outside that range, -1 padding included, are skipped), or
    all compressed entries when sel is None (dense C128 layer). A multiset: no deduplication."""
    window_rows = _f32(window_rows)
    comp_rows = _f32(comp_rows)
    G = comp_rows.shape[0]
    if sel is None:
        extra = comp_rows
    else:
        idx = [int(j) for j in np.asarray(sel).ravel() if 0 <= int(j) < G]
        extra = comp_rows[idx] if idx else np.zeros((0, window_rows.shape[1]), np.float32)
    return np.concatenate([window_rows, extra.reshape(-1, window_rows.shape[1])], axis=0)


def window_rows(X_seq, window: int) -> np.ndarray:
    """The last min(N, W) rows of one sequence's token vectors."""
    n = X_seq.shape[0]
    return X_seq[max(0, n - window):n]


def decode_step(q, X_seq, window: int, comp_rows, sel, scale: float):
    """Attention of one sequence's decode step (see step_keys and attend)."""
    return attend(q, step_keys(window_rows(X_seq, window), comp_rows, sel), scale)


# ---------------------------------------------------------------- per-step append (state ring)
def ring_image(rows, ring_size: int):
    """What a ring of `ring_size` row slots holds after the rows of a token history were written
    to it one token at a time, in order, token t into slot t mod ring_size. Returns (image
    [ring_size, d] float32, written [ring_size] bool); slots no token reached hold zeros.

    Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", ShadowRadix (the compression state ring sits
    inside the SWA page: slot address = page * ring size + position mod ring size). Writing tokens
    before N - ring_size only puts rows that a later token of the same residue overwrites, so the
    replay starts there."""
    rows = _f32(rows)
    N, d = rows.shape
    img = np.zeros((ring_size, d), np.float32)
    written = np.zeros(ring_size, bool)
    for t in range(max(0, N - ring_size), N):
        img[t % ring_size] = rows[t]
        written[t % ring_size] = True
    return img, written


def append_state(X_seq, Z_seq, B, m: int, window: int, ring_size: int) -> dict:
    """The state one sequence's decode-time appends must leave after its history of N tokens
    (X_seq, Z_seq: [N, d], token rows and gate logits), whatever mix of prefill and one-token
    appends produced it:
      swa / swa_written:   the window ring, token t's row at slot t mod window;
      gate / gate_written: the gate state ring, token t's gate at slot t mod ring_size;
      comp:                the compressed entries of every complete group (unrounded doubles),
                           i.e. compress() of the whole history;
      n, swa_len, comp_count: N, min(N, window) and floor(N / m).
    Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", ShadowRadix (state rings nested in the SWA
    pages) and V4 到底改了啥 (window of 128; C4 and C128 groups)."""
    X_seq, Z_seq = _f32(X_seq), _f32(Z_seq)
    N = X_seq.shape[0]
    swa, swa_w = ring_image(X_seq, window)
    gate, gate_w = ring_image(Z_seq, ring_size)
    comp = compress(X_seq, Z_seq, B, m, np.array([0, N], np.int64))
    return dict(swa=swa, swa_written=swa_w, gate=gate, gate_written=gate_w, comp=comp, n=N,
                swa_len=min(N, window), comp_count=N // m)


# ---------------------------------------------------------------- paged pools
def paged_rows(pool, page_table, page_size: int, n: int) -> np.ndarray:
    """The first n logical rows of one sequence stored in a paged pool: logical row j lives at
    pool row page_table[j // page_size] * page_size + j % page_size.
    Source: "DeepSeek-V4 本地部署，SGLang 把活做絕了", ShadowRadix, and "SGLang 如何为 DeepSeek V4
    打造「Day-0」推理加速", 创新 1 (the SWA, C4 and C128 pools are managed as physical pools that
    a per-request index maps into; slot address = page * size + position mod size)."""
    pool = np.asarray(pool)
    out = np.empty((n,) + pool.shape[1:], dtype=pool.dtype)
    for j in range(n):
        out[j] = pool[int(page_table[j // page_size]) * page_size + j % page_size]
    return out
