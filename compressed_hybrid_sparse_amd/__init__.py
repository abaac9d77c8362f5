"""Python binding of libchs.so: one decode step of one hybrid-sparse-attention layer on MI355X.

Argument marshalling only. Every step of the path runs in the library's HIP kernels; torch
supplies device memory (outputs and workspaces are torch tensors) and the current stream.
There is no fallback: if libchs.so is missing or a call fails, an exception is raised.

The functions mirror the C ABI in include/chs.h (chs_compress, chs_append, chs_index_topk,
chs_decode_attn and their FP8 forms); see that header for the definitions and the pages they
follow.
"""
import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime first; libchs binds to the same libamdhip64)

HERE = os.path.dirname(os.path.abspath(__file__))
# CHS_LIB names another build of the library (the CPU sanitizer test loads a host-only build with
# AddressSanitizer and UndefinedBehaviorSanitizer).
LIB_PATH = os.environ.get("CHS_LIB") or os.path.join(HERE, "libchs.so")

CHS_F32, CHS_BF16 = 0, 1
_STATUS = {0: "CHS_OK", 1: "CHS_ERR_NULL", 2: "CHS_ERR_SHAPE", 3: "CHS_ERR_DTYPE",
           4: "CHS_ERR_WORKSPACE", 5: "CHS_ERR_UNSUPPORTED", 6: "CHS_ERR_LAUNCH"}
EXPORTS = ("chs_version", "chs_status_string", "chs_workspace_clear", "chs_compress",
           "chs_index_topk_workspace_size", "chs_index_topk", "chs_decode_attn_workspace_size",
           "chs_decode_attn", "chs_index_topk_fp8", "chs_decode_attn_fp8", "chs_append",
           "chs_decode_attn_paged", "chs_append_paged", "chs_index_topk_paged", "chs_gather_selected",
           "chs_append_multi", "chs_index_topk_fp8_paged", "chs_decode_attn_fp8_paged",
           "chs_decode_step_workspace_size", "chs_decode_step", "chs_index_scores", "chs_decode_step_noalloc",
           "chs_quantize_e4m3", "chs_compress_fp8", "chs_append_fp8", "chs_decode_step_fp8",
           "chs_decode_step_paged")

_lib = None
_i32, _i64, _sz, _p, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class AppendStream(ctypes.Structure):
    """chs_append_stream: one compressor stream of chs_append_multi (field for field as in chs.h)."""
    _fields_ = [("d", ctypes.c_int32), ("window", ctypes.c_int32), ("ring_size", ctypes.c_int32),
                ("x_new", ctypes.c_void_p), ("z_new", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("n_tokens", ctypes.c_void_p), ("swa_kv", ctypes.c_void_p), ("swa_len", ctypes.c_void_p),
                ("gate_ring", ctypes.c_void_p), ("ring_page", ctypes.c_void_p), ("ring_pages", ctypes.c_int64),
                ("comp_kv", ctypes.c_void_p), ("comp_start", ctypes.c_void_p), ("comp_rows", ctypes.c_int64),
                ("comp_count", ctypes.c_void_p), ("swa_page", ctypes.c_void_p), ("swa_pages", ctypes.c_int64),
                ("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("pool_pages", ctypes.c_int64)]


class ChsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {_STATUS.get(status, status)}")


def lib():
    """The loaded libchs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with compressed_hybrid_sparse_amd/build.py "
                              "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        L.chs_version.restype = _i32
        L.chs_status_string.restype = ctypes.c_char_p
        L.chs_status_string.argtypes = [ctypes.c_int]
        L.chs_workspace_clear.argtypes = [_p, _sz, _p]
        L.chs_compress.argtypes = [ctypes.c_int, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i64, _p, _p]
        L.chs_index_topk_workspace_size.restype = _sz
        L.chs_index_topk_workspace_size.argtypes = [_i32, _i64, _i32]
        L.chs_index_topk.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _i64, _p, _p, _p,
                                     _sz, _p]
        L.chs_decode_attn_workspace_size.restype = _sz
        L.chs_decode_attn_workspace_size.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i64]
        L.chs_decode_attn.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _f, _p, _p, _p, _p, _p, _p,
                                      _i64, _p, _p, _p, _sz, _p]
        L.chs_index_scores.argtypes = [ctypes.c_int, _i32, _i32, _i32, _p, _p, _p, _p, _i64, _p, _p, _sz, _p]
        L.chs_index_topk_fp8.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i64, _p, _p, _p, _sz, _p]
        L.chs_decode_attn_fp8.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _p,
                                          _p, _p, _sz, _p]
        L.chs_append.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _p,
                                 _p, _i64, _p, _p]
        L.chs_decode_attn_paged.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _f, _p, _p, _p, _i64, _p, _p,
                                            _i64, _i32, _p, _i32, _p, _p, _i64, _p, _p, _p, _sz, _p]
        L.chs_append_paged.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _i64, _p, _p,
                                       _p, _i64, _i32, _p, _i32, _p, _p]
        L.chs_index_topk_fp8_paged.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _i64, _i32, _p, _i32, _p, _i64,
                                               _p, _p, _p, _sz, _p]
        L.chs_decode_attn_fp8_paged.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _p, _p, _p, _p, _i64, _p, _p, _p,
                                                _i64, _i32, _p, _i32, _p, _p, _i64, _p, _p, _p, _sz, _p]
        L.chs_decode_step_workspace_size.restype = _sz
        L.chs_decode_step_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64]
        L.chs_decode_step.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                                      _i64, _p, _p, _p, _p, _p, _sz, _p]
        L.chs_decode_step_noalloc.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                                              _p, _i64, _p, _p, _p, _p, _p]
        L.chs_decode_step_fp8.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                                          _p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _sz, _p]
        L.chs_decode_step_paged.argtypes = [_i32, _i32, _i32, _i32, _i32, _f, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                            _i64, _p, _p, _i64, _i32, _p, _i32, _p, _i64, _p, _p, _p, _p, _p, _sz,
                                            _p]
        L.chs_quantize_e4m3.argtypes = [ctypes.c_int, _i64, _i32, _p, _p, _p, _p]
        L.chs_compress_fp8.argtypes = [ctypes.c_int, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i64, _p, _p, _p]
        L.chs_append_fp8.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _i64, _p, _p, _p, _i64, _p, _p]
        L.chs_append_multi.argtypes = [ctypes.c_int, _i32, _i32, _i32, ctypes.POINTER(AppendStream), _p]
        L.chs_gather_selected.argtypes = [ctypes.c_int, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _i64, _p, _p, _p]
        L.chs_index_topk_paged.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _p, _p, _p, _i64, _i32, _p, _i32, _p,
                                           _i64, _p, _p, _p, _sz, _p]
        for fn in ("chs_workspace_clear", "chs_compress", "chs_index_topk", "chs_index_scores", "chs_decode_step_noalloc",
                   "chs_decode_step_fp8", "chs_decode_step_paged",
                   "chs_quantize_e4m3", "chs_compress_fp8", "chs_append_fp8",
                   "chs_decode_step", "chs_decode_attn", "chs_index_topk_fp8",
                   "chs_decode_attn_fp8", "chs_append", "chs_decode_attn_paged", "chs_append_paged",
                   "chs_index_topk_paged", "chs_gather_selected", "chs_append_multi", "chs_index_topk_fp8_paged",
                   "chs_decode_attn_fp8_paged"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return CHS_BF16
    if t.dtype == torch.float32:
        return CHS_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(status: int, what: str):
    if status != 0:
        raise ChsError(status, what)


def _need(t, name, dtype=None, dim=None):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")


def _host_max_diff(cu):
    """max_b (cu[b+1] - cu[b]) of an int64 prefix array (a host round trip if cu is on the GPU)."""
    d = cu[1:] - cu[:-1]
    return int(d.max().item()) if d.numel() else 0


def _host_cu(cu):
    """(max_b (cu[b+1] - cu[b]), cu[-1]) read on the host in one transfer."""
    h = cu.cpu()
    d = h[1:] - h[:-1]
    return (int(d.max()) if d.numel() else 0), int(h[-1]) if h.numel() else 0


def _shape(t, shape, name):
    """t must have exactly `shape` (checked before any launch: an undersized buffer would be
    read or written out of bounds on the device)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t, n, name):
    """t must hold at least n rows (dimension 0)."""
    if t.shape[0] < n:
        raise ValueError(f"{name} has {t.shape[0]} rows, the call addresses {n}")


def _cu_sizes(cu, max_given):
    """The (max per-sequence count, total) of a cu prefix array. When the caller passes the
    maximum, the array is not read (no device round trip, so the call can be captured in a graph)
    and the total is None: buffers sized from cu[-1] are then the caller's responsibility."""
    if max_given is None:
        return _host_cu(cu)
    return int(max_given), None


def workspace_clear(ws):
    _check(lib().chs_workspace_clear(_ptr(ws), ws.numel() * ws.element_size(), _stream()), "chs_workspace_clear")


def version() -> int:
    return int(lib().chs_version())


# ---------------------------------------------------------------- chs_compress
def compress(x, gate, bias, m: int, cu_tokens, cu_groups=None, max_groups=None, out=None):
    """Group softmax-pool of every complete group of m tokens (chs_compress).
    x, gate: [T, d] (bf16 or fp32); bias: [m, d] fp32; cu_tokens: [B+1] int64 (CUDA).
    cu_groups: [B+1] int64 output offsets (default: packed, prefix sums of floor(N_b/m)).
    Returns out [cu_groups[-1], d] in x's dtype."""
    _need(x, "x", dim=2)
    _need(gate, "gate", x.dtype, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(cu_tokens, "cu_tokens", torch.int64, 1)
    if cu_groups is None:
        lens = cu_tokens[1:] - cu_tokens[:-1]
        cu_groups = torch.zeros_like(cu_tokens)
        cu_groups[1:] = torch.cumsum(torch.div(lens, m, rounding_mode="floor"), 0)
    _need(cu_groups, "cu_groups", torch.int64, 1)
    if cu_groups.numel() != cu_tokens.numel():
        raise ValueError("cu_groups and cu_tokens must have the same length")
    _shape(gate, x.shape, "gate")
    _shape(bias, (m, x.shape[1]), "bias")
    max_groups, n_out = _cu_sizes(cu_groups, max_groups)
    if n_out is not None:
        _rows(x, int(cu_tokens[-1].item()), "x")
    if out is None:
        out = torch.empty(n_out if n_out is not None else int(cu_groups[-1].item()), x.shape[1], dtype=x.dtype,
                          device=x.device)
    _need(out, "out", x.dtype, 2)
    if out.shape[1] != x.shape[1]:
        raise ValueError(f"out must have {x.shape[1]} columns")
    if n_out is not None:
        _rows(out, n_out, "out")
    _check(lib().chs_compress(_dtype_code(x), cu_tokens.numel() - 1, x.shape[1], m, _ptr(x), _ptr(gate),
                              _ptr(bias), _ptr(cu_tokens), _ptr(cu_groups), int(max_groups), _ptr(out),
                              _stream()), "chs_compress")
    return out


# ---------------------------------------------------------------- FP8 writers
def quantize_e4m3(rows, codes=None, scales=None):
    """Per-row E4M3 codes and fp32 scales of rows [n, d] (bf16 or fp32) (chs_quantize_e4m3).
    Returns (codes [n, d] uint8, scales [n] fp32)."""
    _need(rows, "rows", dim=2)
    n, d = rows.shape
    if codes is None:
        codes = torch.empty(n, d, dtype=torch.uint8, device=rows.device)
    if scales is None:
        scales = torch.empty(n, dtype=torch.float32, device=rows.device)
    _need(codes, "codes", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 1)
    _shape(codes, (n, d), "codes")
    _shape(scales, (n,), "scales")
    _check(lib().chs_quantize_e4m3(_dtype_code(rows), n, d, _ptr(rows), _ptr(codes), _ptr(scales), _stream()),
           "chs_quantize_e4m3")
    return codes, scales


def compress_fp8(x, gate, bias, m: int, cu_tokens, cu_groups=None, max_groups=None, codes=None, scales=None):
    """chs_compress with E4M3 output (chs_compress_fp8): returns (codes [G, d] uint8, scales [G] fp32)."""
    _need(x, "x", dim=2)
    _need(gate, "gate", x.dtype, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(cu_tokens, "cu_tokens", torch.int64, 1)
    if cu_groups is None:
        lens = cu_tokens[1:] - cu_tokens[:-1]
        cu_groups = torch.zeros_like(cu_tokens)
        cu_groups[1:] = torch.cumsum(torch.div(lens, m, rounding_mode="floor"), 0)
    _need(cu_groups, "cu_groups", torch.int64, 1)
    if cu_groups.numel() != cu_tokens.numel():
        raise ValueError("cu_groups and cu_tokens must have the same length")
    _shape(gate, x.shape, "gate")
    _shape(bias, (m, x.shape[1]), "bias")
    max_groups, n_out = _cu_sizes(cu_groups, max_groups)
    if n_out is not None:
        _rows(x, int(cu_tokens[-1].item()), "x")
    rows = n_out if n_out is not None else int(cu_groups[-1].item())
    if codes is None:
        codes = torch.empty(rows, x.shape[1], dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 1)
    if codes.shape[1] != x.shape[1] or scales.shape[0] < codes.shape[0]:
        raise ValueError("codes must have d columns and scales one entry per code row")
    if n_out is not None:
        _rows(codes, n_out, "codes")
    _check(lib().chs_compress_fp8(_dtype_code(x), cu_tokens.numel() - 1, x.shape[1], m, _ptr(x), _ptr(gate),
                                  _ptr(bias), _ptr(cu_tokens), _ptr(cu_groups), int(max_groups), _ptr(codes),
                                  _ptr(scales), _stream()), "chs_compress_fp8")
    return codes, scales


def append_fp8(x_new, z_new, bias, m: int, n_tokens, swa_codes, swa_scale, x_ring, gate_ring, ring_page, comp_codes,
               comp_scale, comp_start, ring_size=None, swa_len=None, comp_count=None):
    """chs_append over an FP8 cache (chs_append_fp8): the new token's row quantised into the window
    (swa_codes [B, W, d] uint8, swa_scale [B, W] fp32), its row and gate into the state rings (x_ring,
    gate_ring [pages * ring_size, d], the storage type), a completed group pooled from the rings and
    quantised into comp_codes [rows, d] uint8 / comp_scale [rows] fp32; counters advanced in place."""
    _need(x_new, "x_new", dim=2)
    dt = x_new.dtype
    B, d = x_new.shape
    _need(z_new, "z_new", dt, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(n_tokens, "n_tokens", torch.int64, 1)
    _need(swa_codes, "swa_codes", torch.uint8, 3)
    _need(swa_scale, "swa_scale", torch.float32, 2)
    _need(x_ring, "x_ring", dt, 2)
    _need(gate_ring, "gate_ring", dt, 2)
    _need(ring_page, "ring_page", torch.int32, 1)
    _need(comp_codes, "comp_codes", torch.uint8, 2)
    _need(comp_scale, "comp_scale", torch.float32, 1)
    _need(comp_start, "comp_start", torch.int64, 1)
    _shape(z_new, (B, d), "z_new")
    _shape(bias, (m, d), "bias")
    _shape(n_tokens, (B,), "n_tokens")
    if swa_codes.shape[0] != B or swa_codes.shape[2] != d:
        raise ValueError(f"swa_codes must be [{B}, W, {d}]")
    W = swa_codes.shape[1]
    _shape(swa_scale, (B, W), "swa_scale")
    _shape(gate_ring, x_ring.shape, "gate_ring")
    _shape(ring_page, (B,), "ring_page")
    _shape(comp_start, (B,), "comp_start")
    if x_ring.shape[1] != d or comp_codes.shape[1] != d or comp_scale.numel() < comp_codes.shape[0]:
        raise ValueError("rings and pool must have d columns, comp_scale one entry per pool row")
    for t, name in ((swa_len, "swa_len"), (comp_count, "comp_count")):
        if t is not None and t.numel() < B:
            raise ValueError(f"{name} must hold {B} entries")
    if ring_size is None:
        ring_size = x_ring.shape[0] // B
    pages = x_ring.shape[0] // ring_size
    _check(lib().chs_append_fp8(_dtype_code(x_new), B, d, m, W, int(ring_size), _ptr(x_new), _ptr(z_new), _ptr(bias),
                                _ptr(n_tokens), _ptr(swa_codes), _ptr(swa_scale), _ptr(swa_len), _ptr(x_ring),
                                _ptr(gate_ring), _ptr(ring_page), pages, _ptr(comp_codes), _ptr(comp_scale),
                                _ptr(comp_start), comp_codes.shape[0], _ptr(comp_count), _stream()), "chs_append_fp8")


# ---------------------------------------------------------------- chs_append
def append(x_new, z_new, bias, m: int, n_tokens, swa_kv, gate_ring, ring_page, comp_kv, comp_start,
           ring_size=None, swa_len=None, comp_count=None):
    """One decode-time token per sequence (chs_append): writes x_new into the window ring and z_new
    into the gate state ring, pools a group the token completes into comp_kv, and advances the
    counters in place.
    x_new, z_new: [B, d]; bias: [m, d] fp32; n_tokens: [B] int64 (in/out); swa_kv: [B, W, d];
    gate_ring: [pages * ring_size, d]; ring_page: [B] int32; comp_kv: [rows, d];
    comp_start: [B] int64; swa_len: [B] int32 or None; comp_count: [B] int64 or None (outputs).
    ring_size defaults to gate_ring.shape[0] // the number of pages when that is 1 page per
    sequence; pass it explicitly otherwise."""
    _need(x_new, "x_new", dim=2)
    dt = x_new.dtype
    _need(z_new, "z_new", dt, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(n_tokens, "n_tokens", torch.int64, 1)
    _need(swa_kv, "swa_kv", dt, 3)
    _need(gate_ring, "gate_ring", dt, 2)
    _need(ring_page, "ring_page", torch.int32, 1)
    _need(comp_kv, "comp_kv", dt, 2)
    _need(comp_start, "comp_start", torch.int64, 1)
    if swa_len is not None:
        _need(swa_len, "swa_len", torch.int32, 1)
    if comp_count is not None:
        if comp_count.dtype != torch.int64 or not comp_count.is_cuda:
            raise TypeError("comp_count must be an int64 CUDA tensor")
    B, d = x_new.shape
    _shape(z_new, (B, d), "z_new")
    _shape(bias, (m, d), "bias")
    _shape(n_tokens, (B,), "n_tokens")
    if swa_kv.shape[0] != B or swa_kv.shape[2] != d:
        raise ValueError(f"swa_kv must be [{B}, W, {d}], got {tuple(swa_kv.shape)}")
    _shape(ring_page, (B,), "ring_page")
    _shape(comp_start, (B,), "comp_start")
    if gate_ring.shape[1] != d or comp_kv.shape[1] != d:
        raise ValueError("gate_ring and comp_kv must have d columns")
    for t, name in ((swa_len, "swa_len"), (comp_count, "comp_count")):
        if t is not None and t.numel() < B:
            raise ValueError(f"{name} must hold {B} entries")
    if ring_size is None:
        ring_size = gate_ring.shape[0] // B
    pages = gate_ring.shape[0] // ring_size
    _check(lib().chs_append(_dtype_code(x_new), B, d, m, swa_kv.shape[1], int(ring_size), _ptr(x_new), _ptr(z_new),
                            _ptr(bias), _ptr(n_tokens), _ptr(swa_kv), _ptr(swa_len), _ptr(gate_ring),
                            _ptr(ring_page), pages, _ptr(comp_kv), _ptr(comp_start), comp_kv.shape[0],
                            _ptr(comp_count), _stream()), "chs_append")


# ---------------------------------------------------------------- chs_index_topk
def index_topk_workspace(batch: int, max_cand: int, k: int, device="cuda"):
    n = lib().chs_index_topk_workspace_size(batch, max_cand, k)
    return torch.zeros(max(n, 4), dtype=torch.uint8, device=device)


def index_topk(q_idx, w, k_idx, cu_cand, k: int, max_cand=None, scores=None, workspace=None, out=None):
    """Indexer scores and exact top-k (chs_index_topk).
    q_idx: [B, Hi, dim]; w: [B, Hi] fp32; k_idx: [G, dim]; cu_cand: [B+1] int64.
    If q_idx is None, `scores` ([G] fp32) is the input and w, k_idx are ignored.
    Returns (topk [B, k] int32, scores or None)."""
    _need(cu_cand, "cu_cand", torch.int64, 1)
    batch = cu_cand.numel() - 1
    max_cand, total = _cu_sizes(cu_cand, max_cand)
    if workspace is None:
        workspace = index_topk_workspace(batch, max_cand, k, cu_cand.device)
    if out is None:
        out = torch.empty(batch, k, dtype=torch.int32, device=cu_cand.device)
    _need(out, "topk", torch.int32, 2)
    _shape(out, (batch, k), "topk")
    if q_idx is not None:
        _need(q_idx, "q_idx", dim=3)
        _need(w, "w", torch.float32, 2)
        _need(k_idx, "k_idx", q_idx.dtype, 2)
        dt, nh, dim = _dtype_code(q_idx), q_idx.shape[1], q_idx.shape[2]
        if q_idx.shape[0] != batch:
            raise ValueError(f"q_idx must have {batch} rows (one per sequence)")
        _shape(w, (batch, nh), "w")
        if k_idx.shape[1] != dim:
            raise ValueError(f"k_idx must have {dim} columns")
        if scores is not None:
            _need(scores, "scores", torch.float32, 1)
        if total is not None:
            _rows(k_idx, total, "k_idx")
            if scores is not None:
                _rows(scores, total, "scores")
    else:
        _need(scores, "scores", torch.float32, 1)
        dt, nh, dim = CHS_F32, 0, 0
        if total is not None:
            _rows(scores, total, "scores")
    _check(lib().chs_index_topk(dt, batch, nh, dim, k, _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(cu_cand),
                                int(max_cand), _ptr(scores), _ptr(out), _ptr(workspace),
                                workspace.numel(), _stream()), "chs_index_topk")
    return out, scores


def index_scores(q_idx, w, k_idx, cu_cand, max_cand=None, scores=None, workspace=None):
    """The indexer scores alone (chs_index_scores): the values index_topk computes, no selection.
    q_idx: [B, Hi, dim]; w: [B, Hi] fp32; k_idx: [G, dim]; cu_cand: [B+1] int64. Returns scores [G]
    fp32."""
    _need(cu_cand, "cu_cand", torch.int64, 1)
    _need(q_idx, "q_idx", dim=3)
    _need(w, "w", torch.float32, 2)
    _need(k_idx, "k_idx", q_idx.dtype, 2)
    batch = cu_cand.numel() - 1
    nh, dim = q_idx.shape[1], q_idx.shape[2]
    if q_idx.shape[0] != batch or k_idx.shape[1] != dim:
        raise ValueError("q_idx must be [B, Hi, dim] and k_idx [G, dim]")
    _shape(w, (batch, nh), "w")
    max_cand, total = _cu_sizes(cu_cand, max_cand)
    if scores is None:
        scores = torch.empty(total if total is not None else k_idx.shape[0], dtype=torch.float32,
                             device=q_idx.device)
    _need(scores, "scores", torch.float32, 1)
    if total is not None:
        _rows(k_idx, total, "k_idx")
        _rows(scores, total, "scores")
    if workspace is None:
        workspace = index_topk_workspace(batch, max_cand, 1, cu_cand.device)
    _check(lib().chs_index_scores(_dtype_code(q_idx), batch, nh, dim, _ptr(q_idx), _ptr(w), _ptr(k_idx),
                                  _ptr(cu_cand), int(max_cand), _ptr(scores), _ptr(workspace), workspace.numel(),
                                  _stream()), "chs_index_scores")
    return scores


def topk_from_scores(scores, cu_cand, k: int, max_cand=None, workspace=None, out=None):
    """Standalone exact top-k over given fp32 scores (chs_index_topk with q_idx = NULL)."""
    return index_topk(None, None, None, cu_cand, k, max_cand, scores, workspace, out)[0]


# ---------------------------------------------------------------- chs_decode_attn
def _attn_shapes(q, swa_kv, swa_len, comp_kv, cu_comp):
    """The shapes every attention call shares: q [B, H, d], swa_kv [B or pages, W, d] (d codes for
    FP8), swa_len [B], comp_kv [*, d], cu_comp [B + 1] (or per-sequence counts [B])."""
    B, H, d = q.shape
    if swa_kv.shape[2] != d or comp_kv.shape[1] != d:
        raise ValueError(f"swa_kv and comp_kv rows must have {d} elements")
    _shape(swa_len, (B,), "swa_len")
    if cu_comp is not None and cu_comp.numel() not in (B, B + 1):
        raise ValueError(f"cu_comp / comp_len must have {B + 1} / {B} entries")


def _attn_outputs(q, out, lse):
    """out [B, H, d] fp32 and lse [B, H] fp32, allocated if not given, checked if given."""
    B, H, d = q.shape
    if out is None:
        out = torch.empty(B, H, d, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32)
    _shape(out, (B, H, d), "out")
    _shape(lse, (B, H), "lse")
    return out, lse


def decode_attn_workspace(dtype, batch, n_heads, d, window, k, max_comp, device="cuda"):
    code = CHS_BF16 if dtype == torch.bfloat16 else CHS_F32
    n = lib().chs_decode_attn_workspace_size(code, batch, n_heads, d, window, k, max_comp)
    return torch.zeros(max(n, 4), dtype=torch.uint8, device=device)


def decode_attn(q, swa_kv, swa_len, comp_kv, cu_comp, topk=None, scale=None, max_comp=None,
                workspace=None, out=None, lse=None):
    """One softmax over the window rows and the selected (topk) or all (topk=None) compressed
    entries, keys doubling as values (chs_decode_attn).
    q: [B, H, d]; swa_kv: [B, W, d]; swa_len: [B] int32; comp_kv: [G, d]; cu_comp: [B+1] int64;
    topk: [B, k] int32 or None. Returns (out [B, H, d] fp32, lse [B, H] fp32)."""
    _need(q, "q", dim=3)
    _need(swa_kv, "swa_kv", q.dtype, 3)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_kv, "comp_kv", q.dtype, 2)
    _need(cu_comp, "cu_comp", torch.int64, 1)
    B, H, d = q.shape
    W = swa_kv.shape[1]
    k = 0
    if topk is not None:
        _need(topk, "topk", torch.int32, 2)
        k = topk.shape[1]
        _shape(topk, (B, k), "topk")
    _attn_shapes(q, swa_kv, swa_len, comp_kv, cu_comp)
    if swa_kv.shape[0] != B:
        raise ValueError(f"swa_kv must have {B} windows")
    max_comp, total = _cu_sizes(cu_comp, max_comp)
    if total is not None:
        _rows(comp_kv, total, "comp_kv")
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = decode_attn_workspace(q.dtype, B, H, d, W, k, max_comp, q.device)
    out, lse = _attn_outputs(q, out, lse)
    _check(lib().chs_decode_attn(_dtype_code(q), B, H, d, W, k, float(scale), _ptr(q), _ptr(swa_kv),
                                 _ptr(swa_len), _ptr(comp_kv), _ptr(cu_comp), _ptr(topk), int(max_comp),
                                 _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()),
           "chs_decode_attn")
    return out, lse


# ---------------------------------------------------------------- chs_decode_step
def decode_step_workspace(batch, n_heads, d, window, k, max_comp, device="cuda"):
    n = lib().chs_decode_step_workspace_size(batch, n_heads, d, window, k, max_comp)
    return torch.zeros(max(n, 4), dtype=torch.uint8, device=device)


def decode_step(q_idx, w, k_idx, q, swa_kv, swa_len, comp_kv, cu_comp, k: int, scale=None, max_comp=None,
                scores=None, workspace=None, topk=None, out=None, lse=None):
    """The C4 decode step in one call (chs_decode_step, bf16): the indexer scores and exact top-k
    of index_topk over the compressed entries, then decode_attn over the window and the selected
    entries, with bit-identical results. q_idx: [B, Hi, dim]; w: [B, Hi] fp32; k_idx: [G, dim];
    q: [B, H, d]; swa_kv: [B, W, d]; swa_len: [B] int32; comp_kv: [G, d]; cu_comp: [B+1] int64.
    Returns (topk [B, k] int32, out [B, H, d] fp32, lse [B, H] fp32, scores or None)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(k_idx, "k_idx", torch.bfloat16, 2)
    _need(q, "q", torch.bfloat16, 3)
    _need(swa_kv, "swa_kv", torch.bfloat16, 3)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_kv, "comp_kv", torch.bfloat16, 2)
    _need(cu_comp, "cu_comp", torch.int64, 1)
    B, H, d = q.shape
    W = swa_kv.shape[1]
    _attn_shapes(q, swa_kv, swa_len, comp_kv, cu_comp)
    if swa_kv.shape[0] != B or cu_comp.numel() != B + 1:
        raise ValueError(f"swa_kv must have {B} windows and cu_comp {B + 1} entries")
    if q_idx.shape[0] != B or k_idx.shape[1] != q_idx.shape[2]:
        raise ValueError("q_idx must be [B, Hi, dim] and k_idx [G, dim]")
    _shape(w, q_idx.shape[:2], "w")
    max_comp, total = _cu_sizes(cu_comp, max_comp)
    if scale is None:
        scale = d ** -0.5
    if scores is not None:
        _need(scores, "scores", torch.float32, 1)
    if total is not None:
        _rows(comp_kv, total, "comp_kv")
        _rows(k_idx, total, "k_idx")
        if scores is not None:
            _rows(scores, total, "scores")
    if workspace is None:
        workspace = decode_step_workspace(B, H, d, W, k, max_comp, q.device)
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=q.device)
    out, lse = _attn_outputs(q, out, lse)
    _need(topk, "topk", torch.int32, 2)
    _shape(topk, (B, k), "topk")
    _check(lib().chs_decode_step(B, H, d, W, k, float(scale), q_idx.shape[1], q_idx.shape[2], _ptr(q_idx), _ptr(w),
                                 _ptr(k_idx), _ptr(q), _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv), _ptr(cu_comp),
                                 int(max_comp), _ptr(scores), _ptr(topk), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel(), _stream()), "chs_decode_step")
    return topk, out, lse, scores


def decode_step_fp8(q_idx, w, k_codes, k_scale, q, swa_codes, swa_scale, swa_len, comp_codes, comp_scale, cu_comp,
                    k: int, scale=None, max_comp=None, scores=None, workspace=None, topk=None, out=None, lse=None):
    """The C4 decode step over FP8 storage in one call (chs_decode_step_fp8): index_topk_fp8 then
    decode_attn_fp8, with bit-identical results. q_idx: [B, Hi, dim] bf16; w: [B, Hi] fp32;
    k_codes: [G, dim] uint8 (or float8_e4m3fn) with k_scale [G] fp32; q: [B, H, d] bf16;
    swa_codes: [B, W, d] with swa_scale [B, W]; swa_len: [B] int32; comp_codes: [G, d] with
    comp_scale [G]; cu_comp: [B+1] int64. Returns (topk, out, lse, scores or None)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    k_codes = k_codes.view(torch.uint8) if k_codes.dtype != torch.uint8 else k_codes
    swa_codes = swa_codes.view(torch.uint8) if swa_codes.dtype != torch.uint8 else swa_codes
    comp_codes = comp_codes.view(torch.uint8) if comp_codes.dtype != torch.uint8 else comp_codes
    _need(k_codes, "k_codes", torch.uint8, 2)
    _need(k_scale, "k_scale", torch.float32, 1)
    _need(q, "q", torch.bfloat16, 3)
    _need(swa_codes, "swa_codes", torch.uint8, 3)
    _need(swa_scale, "swa_scale", torch.float32, 2)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_codes, "comp_codes", torch.uint8, 2)
    _need(comp_scale, "comp_scale", torch.float32, 1)
    _need(cu_comp, "cu_comp", torch.int64, 1)
    B, H, d = q.shape
    W = swa_codes.shape[1]
    _attn_shapes(q, swa_codes, swa_len, comp_codes, cu_comp)
    if swa_codes.shape[0] != B or cu_comp.numel() != B + 1:
        raise ValueError(f"swa_codes must have {B} windows and cu_comp {B + 1} entries")
    if q_idx.shape[0] != B or k_codes.shape[1] != q_idx.shape[2]:
        raise ValueError("q_idx must be [B, Hi, dim] and k_codes [G, dim]")
    _shape(w, q_idx.shape[:2], "w")
    _shape(swa_scale, (B, W), "swa_scale")
    if k_scale.numel() != k_codes.shape[0] or comp_scale.numel() != comp_codes.shape[0]:
        raise ValueError("k_scale and comp_scale must hold one scale per row")
    max_comp, total = _cu_sizes(cu_comp, max_comp)
    if scale is None:
        scale = d ** -0.5
    if scores is not None:
        _need(scores, "scores", torch.float32, 1)
    if total is not None:
        _rows(comp_codes, total, "comp_codes")
        _rows(k_codes, total, "k_codes")
        if scores is not None:
            _rows(scores, total, "scores")
    if workspace is None:
        workspace = decode_step_workspace(B, H, d, W, k, max_comp, q.device)
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=q.device)
    out, lse = _attn_outputs(q, out, lse)
    _need(topk, "topk", torch.int32, 2)
    _shape(topk, (B, k), "topk")
    _check(lib().chs_decode_step_fp8(B, H, d, W, k, float(scale), q_idx.shape[1], q_idx.shape[2], _ptr(q_idx),
                                     _ptr(w), _ptr(k_codes), _ptr(k_scale), _ptr(q), _ptr(swa_codes),
                                     _ptr(swa_scale), _ptr(swa_len), _ptr(comp_codes), _ptr(comp_scale),
                                     _ptr(cu_comp), int(max_comp), _ptr(scores), _ptr(topk), _ptr(out), _ptr(lse),
                                     _ptr(workspace), workspace.numel(), _stream()), "chs_decode_step_fp8")
    return topk, out, lse, scores


def decode_step_noalloc(q_idx, w, k_idx, q, swa_kv, swa_len, comp_kv, cu_comp, k: int, scale=None, max_comp=None,
                        scores=None, topk=None, out=None, lse=None):
    """decode_step without a workspace (chs_decode_step_noalloc): the library's per-GPU scratch array
    (CHS_NOALLOC_SCRATCH_BYTES) serves instead, so the C call allocates nothing. Calls that overlap on
    one GPU race on that array. Arguments and results as decode_step; outputs not given are allocated
    here by torch, before the call."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(k_idx, "k_idx", torch.bfloat16, 2)
    _need(q, "q", torch.bfloat16, 3)
    _need(swa_kv, "swa_kv", torch.bfloat16, 3)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_kv, "comp_kv", torch.bfloat16, 2)
    _need(cu_comp, "cu_comp", torch.int64, 1)
    B, H, d = q.shape
    W = swa_kv.shape[1]
    _attn_shapes(q, swa_kv, swa_len, comp_kv, cu_comp)
    if swa_kv.shape[0] != B or cu_comp.numel() != B + 1:
        raise ValueError(f"swa_kv must have {B} windows and cu_comp {B + 1} entries")
    if q_idx.shape[0] != B or k_idx.shape[1] != q_idx.shape[2]:
        raise ValueError("q_idx must be [B, Hi, dim] and k_idx [G, dim]")
    _shape(w, q_idx.shape[:2], "w")
    max_comp, total = _cu_sizes(cu_comp, max_comp)
    if scale is None:
        scale = d ** -0.5
    if scores is not None:
        _need(scores, "scores", torch.float32, 1)
    if total is not None:
        _rows(comp_kv, total, "comp_kv")
        _rows(k_idx, total, "k_idx")
        if scores is not None:
            _rows(scores, total, "scores")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=q.device)
    out, lse = _attn_outputs(q, out, lse)
    _need(topk, "topk", torch.int32, 2)
    _shape(topk, (B, k), "topk")
    _check(lib().chs_decode_step_noalloc(B, H, d, W, k, float(scale), q_idx.shape[1], q_idx.shape[2], _ptr(q_idx),
                                         _ptr(w), _ptr(k_idx), _ptr(q), _ptr(swa_kv), _ptr(swa_len), _ptr(comp_kv),
                                         _ptr(cu_comp), int(max_comp), _ptr(scores), _ptr(topk), _ptr(out), _ptr(lse),
                                         _stream()), "chs_decode_step_noalloc")
    return topk, out, lse, scores


def index_topk_fp8(q_idx, w, k_codes, k_scale, cu_cand, k: int, max_cand=None, scores=None, workspace=None,
                   out=None):
    """Indexer scores with FP8 E4M3 keys and per-row scales, then the exact top-k
    (chs_index_topk_fp8). q_idx: [B, Hi, dim] bf16; w: [B, Hi] fp32; k_codes: [G, dim] uint8 or
    torch.float8_e4m3fn; k_scale: [G] fp32; cu_cand: [B+1] int64. Returns (topk [B, k] int32,
    scores or None)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    if k_codes.dtype != torch.uint8:
        k_codes = k_codes.view(torch.uint8)
    _need(k_codes, "k_codes", torch.uint8, 2)
    _need(k_scale, "k_scale", torch.float32, 1)
    _need(cu_cand, "cu_cand", torch.int64, 1)
    batch = cu_cand.numel() - 1
    nh, dim = q_idx.shape[1], q_idx.shape[2]
    if q_idx.shape[0] != batch or k_codes.shape[1] != dim:
        raise ValueError("q_idx must be [B, Hi, dim] and k_codes [G, dim]")
    _shape(w, (batch, nh), "w")
    if k_scale.numel() != k_codes.shape[0]:
        raise ValueError("k_scale must hold one scale per key row")
    max_cand, total = _cu_sizes(cu_cand, max_cand)
    if total is not None:
        _rows(k_codes, total, "k_codes")
        if scores is not None:
            _rows(scores, total, "scores")
    if scores is not None:
        _need(scores, "scores", torch.float32, 1)
    if workspace is None:
        workspace = index_topk_workspace(batch, max_cand, k, cu_cand.device)
    if out is None:
        out = torch.empty(batch, k, dtype=torch.int32, device=cu_cand.device)
    _need(out, "topk", torch.int32, 2)
    _shape(out, (batch, k), "topk")
    _check(lib().chs_index_topk_fp8(batch, nh, dim, k, _ptr(q_idx), _ptr(w), _ptr(k_codes), _ptr(k_scale),
                                    _ptr(cu_cand), int(max_cand), _ptr(scores), _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream()),
           "chs_index_topk_fp8")
    return out, scores


def decode_attn_fp8(q, swa_codes, swa_scale, swa_len, comp_codes, comp_scale, cu_comp, topk=None, scale=None,
                    max_comp=None, workspace=None, out=None, lse=None):
    """decode_attn over an FP8 E4M3 KV cache with per-row scales (chs_decode_attn_fp8).
    q: [B, H, d] bf16; swa_codes: [B, W, d] uint8 (or float8_e4m3fn); swa_scale: [B, W] fp32;
    swa_len: [B] int32; comp_codes: [G, d]; comp_scale: [G] fp32; cu_comp: [B+1] int64;
    topk: [B, k] int32 or None. Returns (out [B, H, d] fp32, lse [B, H] fp32)."""
    _need(q, "q", torch.bfloat16, 3)
    swa_codes = swa_codes.view(torch.uint8) if swa_codes.dtype != torch.uint8 else swa_codes
    comp_codes = comp_codes.view(torch.uint8) if comp_codes.dtype != torch.uint8 else comp_codes
    _need(swa_codes, "swa_codes", torch.uint8, 3)
    _need(swa_scale, "swa_scale", torch.float32, 2)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_codes, "comp_codes", torch.uint8, 2)
    _need(comp_scale, "comp_scale", torch.float32, 1)
    _need(cu_comp, "cu_comp", torch.int64, 1)
    B, H, d = q.shape
    W = swa_codes.shape[1]
    k = 0
    if topk is not None:
        _need(topk, "topk", torch.int32, 2)
        k = topk.shape[1]
        _shape(topk, (B, k), "topk")
    _attn_shapes(q, swa_codes, swa_len, comp_codes, cu_comp)
    if swa_codes.shape[0] != B:
        raise ValueError(f"swa_codes must have {B} windows")
    _shape(swa_scale, (B, W), "swa_scale")
    if comp_scale.numel() != comp_codes.shape[0]:
        raise ValueError("comp_scale must hold one scale per entry row")
    max_comp, total = _cu_sizes(cu_comp, max_comp)
    if total is not None:
        _rows(comp_codes, total, "comp_codes")
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = decode_attn_workspace(torch.bfloat16, B, H, d, W, k, max_comp, q.device)
    out, lse = _attn_outputs(q, out, lse)
    _check(lib().chs_decode_attn_fp8(B, H, d, W, k, float(scale), _ptr(q), _ptr(swa_codes), _ptr(swa_scale),
                                     _ptr(swa_len), _ptr(comp_codes), _ptr(comp_scale), _ptr(cu_comp), _ptr(topk),
                                     int(max_comp), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                     _stream()),
           "chs_decode_attn_fp8")
    return out, lse


# ---------------------------------------------------------------- paged pools
def decode_attn_paged(q, swa_pool, swa_page, swa_len, comp_pool, page_size: int, page_table, comp_len, topk=None,
                      scale=None, max_comp=None, workspace=None, out=None, lse=None):
    """chs_decode_attn over paged pools (chs_decode_attn_paged).
    q: [B, H, d]; swa_pool: [swa_pages, W, d]; swa_page: [B] int32; swa_len: [B] int32;
    comp_pool: [pool_rows, d] (pool_rows a multiple of page_size); page_table: [B, pt_stride] int32;
    comp_len: [B] int64; topk: [B, k] int32 or None. Returns (out [B, H, d] fp32, lse [B, H] fp32)."""
    _need(q, "q", dim=3)
    _need(swa_pool, "swa_pool", q.dtype, 3)
    _need(swa_page, "swa_page", torch.int32, 1)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_pool, "comp_pool", q.dtype, 2)
    _need(page_table, "page_table", torch.int32, 2)
    _need(comp_len, "comp_len", torch.int64, 1)
    B, H, d = q.shape
    W = swa_pool.shape[1]
    k = 0
    if topk is not None:
        _need(topk, "topk", torch.int32, 2)
        k = topk.shape[1]
        _shape(topk, (B, k), "topk")
    _attn_shapes(q, swa_pool, swa_len, comp_pool, comp_len)
    _shape(swa_page, (B,), "swa_page")
    _shape(comp_len, (B,), "comp_len")
    if page_table.shape[0] != B:
        raise ValueError("page_table must have B rows")
    if max_comp is None:
        max_comp = int(comp_len.max().item()) if comp_len.numel() else 0
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = decode_attn_workspace(q.dtype, B, H, d, W, k, max_comp, q.device)
    out, lse = _attn_outputs(q, out, lse)
    _check(lib().chs_decode_attn_paged(_dtype_code(q), B, H, d, W, k, float(scale), _ptr(q), _ptr(swa_pool),
                                       _ptr(swa_page), swa_pool.shape[0], _ptr(swa_len), _ptr(comp_pool),
                                       comp_pool.shape[0] // page_size, page_size, _ptr(page_table),
                                       page_table.shape[1], _ptr(comp_len), _ptr(topk), int(max_comp), _ptr(out),
                                       _ptr(lse), _ptr(workspace), workspace.numel(), _stream()),
           "chs_decode_attn_paged")
    return out, lse


def append_paged(x_new, z_new, bias, m: int, n_tokens, swa_pool, swa_page, gate_ring, comp_pool, page_size: int,
                 page_table, swa_len=None, comp_count=None):
    """chs_append over paged pools (chs_append_paged). swa_pool: [swa_pages, W, d]; gate_ring:
    [swa_pages * ring_size, d] (the ring of page p is rows p * ring_size ..); comp_pool:
    [pool_rows, d]; page_table: [B, pt_stride] int32."""
    _need(x_new, "x_new", dim=2)
    dt = x_new.dtype
    _need(z_new, "z_new", dt, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(n_tokens, "n_tokens", torch.int64, 1)
    _need(swa_pool, "swa_pool", dt, 3)
    _need(swa_page, "swa_page", torch.int32, 1)
    _need(gate_ring, "gate_ring", dt, 2)
    _need(comp_pool, "comp_pool", dt, 2)
    _need(page_table, "page_table", torch.int32, 2)
    if swa_len is not None:
        _need(swa_len, "swa_len", torch.int32, 1)
    if comp_count is not None and (comp_count.dtype != torch.int64 or not comp_count.is_cuda):
        raise TypeError("comp_count must be an int64 CUDA tensor")
    B, d = x_new.shape
    pages = swa_pool.shape[0]
    ring_size = gate_ring.shape[0] // pages
    _check(lib().chs_append_paged(_dtype_code(x_new), B, d, m, swa_pool.shape[1], ring_size, _ptr(x_new), _ptr(z_new),
                                  _ptr(bias), _ptr(n_tokens), _ptr(swa_pool), _ptr(swa_page), pages, _ptr(swa_len),
                                  _ptr(gate_ring), _ptr(comp_pool), comp_pool.shape[0] // page_size, page_size,
                                  _ptr(page_table), page_table.shape[1], _ptr(comp_count), _stream()),
           "chs_append_paged")


def index_topk_paged(q_idx, w, key_pool, page_size: int, page_table, cand_len, k: int, max_cand: int, scores=None,
                     workspace=None, out=None):
    """chs_index_topk over a paged key pool (chs_index_topk_paged). q_idx: [B, Hi, dim] bf16;
    w: [B, Hi] fp32; key_pool: [pool_rows, dim] bf16; page_table: [B, pt_stride] int32;
    cand_len: [B] int64; scores: [B, max_cand] fp32 or None. Returns (topk [B, k] int32, scores)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(key_pool, "key_pool", torch.bfloat16, 2)
    _need(page_table, "page_table", torch.int32, 2)
    _need(cand_len, "cand_len", torch.int64, 1)
    B, nh, dim = q_idx.shape
    _shape(w, (B, nh), "w")
    _shape(cand_len, (B,), "cand_len")
    if key_pool.shape[1] != dim or page_table.shape[0] != B:
        raise ValueError("key_pool must have dim columns and page_table B rows")
    if scores is not None:
        _need(scores, "scores", torch.float32, 2)
        _shape(scores, (B, max_cand), "scores")
    if workspace is None:
        workspace = index_topk_workspace(B, max_cand, k, q_idx.device)
    if out is None:
        out = torch.empty(B, k, dtype=torch.int32, device=q_idx.device)
    _need(out, "topk", torch.int32, 2)
    _shape(out, (B, k), "topk")
    _check(lib().chs_index_topk_paged(CHS_BF16, B, nh, dim, k, _ptr(q_idx), _ptr(w), _ptr(key_pool),
                                      key_pool.shape[0] // page_size, page_size, _ptr(page_table), page_table.shape[1],
                                      _ptr(cand_len), int(max_cand), _ptr(scores), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream()), "chs_index_topk_paged")
    return out, scores


def decode_step_paged(q_idx, w, key_pool, q, swa_pool, swa_page, swa_len, comp_pool, page_size: int, page_table,
                      comp_len, k: int, max_comp: int, scale=None, scores=None, workspace=None, topk=None, out=None,
                      lse=None):
    """The C4 decode step over paged pools in one call (chs_decode_step_paged): index_topk_paged then
    decode_attn_paged with one page table for the key pool and the entry pool, bit-identical results.
    q_idx: [B, Hi, dim] bf16; w: [B, Hi] fp32; key_pool: [pool_rows, dim] bf16; q: [B, H, d] bf16;
    swa_pool: [swa_pages, W, d]; swa_page, swa_len: [B] int32; comp_pool: [pool_rows, d];
    page_table: [B, pt_stride] int32; comp_len: [B] int64; scores: [B, max_comp] fp32 or None.
    Returns (topk [B, k] int32, out [B, H, d] fp32, lse [B, H] fp32, scores)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(key_pool, "key_pool", torch.bfloat16, 2)
    _need(q, "q", torch.bfloat16, 3)
    _need(swa_pool, "swa_pool", torch.bfloat16, 3)
    _need(swa_page, "swa_page", torch.int32, 1)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_pool, "comp_pool", torch.bfloat16, 2)
    _need(page_table, "page_table", torch.int32, 2)
    _need(comp_len, "comp_len", torch.int64, 1)
    B, H, d = q.shape
    W = swa_pool.shape[1]
    Bi, nh, dim = q_idx.shape
    _attn_shapes(q, swa_pool, swa_len, comp_pool, comp_len)
    _shape(swa_page, (B,), "swa_page")
    _shape(comp_len, (B,), "comp_len")
    _shape(w, (B, nh), "w")
    if Bi != B or key_pool.shape[1] != dim or page_table.shape[0] != B:
        raise ValueError("q_idx must be [B, Hi, dim], key_pool [rows, dim] and page_table [B, pt_stride]")
    if key_pool.shape[0] != comp_pool.shape[0]:
        raise ValueError("key_pool and comp_pool must hold the same number of rows (one page table serves both)")
    if scores is not None:
        _need(scores, "scores", torch.float32, 2)
        _shape(scores, (B, max_comp), "scores")
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = decode_step_workspace(B, H, d, W, k, max_comp, q.device)
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=q.device)
    _need(topk, "topk", torch.int32, 2)
    _shape(topk, (B, k), "topk")
    out, lse = _attn_outputs(q, out, lse)
    _check(lib().chs_decode_step_paged(B, H, d, W, k, float(scale), nh, dim, _ptr(q_idx), _ptr(w), _ptr(key_pool),
                                       _ptr(q), _ptr(swa_pool), _ptr(swa_page), swa_pool.shape[0], _ptr(swa_len),
                                       _ptr(comp_pool), comp_pool.shape[0] // page_size, page_size, _ptr(page_table),
                                       page_table.shape[1], _ptr(comp_len), int(max_comp), _ptr(scores), _ptr(topk),
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()),
           "chs_decode_step_paged")
    return topk, out, lse, scores


# ---------------------------------------------------------------- working-set gather
def gather_selected(mirror, cu_comp, topk, cache=None, resident=None, work=None, work_topk=None, cu_work=None):
    """The selected entries of each sequence gathered into a dense device working set
    (chs_gather_selected). mirror: [G, d] on the device, or a pinned host tensor (pin_memory=True);
    cu_comp: [B+1] int64; topk: [B, k] int32; cache: [rows, d] and resident: [G] int32 (device), both or
    neither. Returns (work [B*k, d], work_topk [B, k] int32, cu_work [B+1] int64 = {0, k, 2k, ..}; pass
    cu_work to reuse one)."""
    if mirror.dim() != 2 or not mirror.is_contiguous():
        raise ValueError("mirror must be a contiguous 2-D tensor")
    on_host = not mirror.is_cuda
    if on_host and not mirror.is_pinned():
        raise ValueError("a host mirror must be pinned (pin_memory=True)")
    _need(cu_comp, "cu_comp", torch.int64, 1)
    _need(topk, "topk", torch.int32, 2)
    B, k = topk.shape
    d = mirror.shape[1]
    if cu_comp.numel() != B + 1:
        raise ValueError(f"cu_comp must have {B + 1} entries")
    if cache is not None or resident is not None:
        _need(cache, "cache", mirror.dtype, 2)
        _need(resident, "resident", torch.int32, 1)
        if cache.shape[1] != d:
            raise ValueError(f"cache rows must have {d} elements")
    if work is None:
        work = torch.empty(B * k, d, dtype=mirror.dtype, device=topk.device)
    if work_topk is None:
        work_topk = torch.empty(B, k, dtype=torch.int32, device=topk.device)
    _need(work, "work", mirror.dtype, 2)
    _need(work_topk, "work_topk", torch.int32, 2)
    _shape(work, (B * k, d), "work")
    _shape(work_topk, (B, k), "work_topk")
    _check(lib().chs_gather_selected(_dtype_code(mirror), B, d, k, _ptr(mirror), int(on_host), _ptr(cu_comp), _ptr(topk),
                                     _ptr(cache), _ptr(resident), 0 if cache is None else cache.shape[0], _ptr(work),
                                     _ptr(work_topk), _stream()), "chs_gather_selected")
    if cu_work is None:
        cu_work = torch.arange(0, (B + 1) * k, k, dtype=torch.int64, device=topk.device)
    return work, work_topk, cu_work


# ---------------------------------------------------------------- several compressor streams
def append_stream(x_new, z_new, bias, n_tokens, swa_kv, gate_ring, comp_kv, ring_page=None, comp_start=None,
                  ring_size=None, swa_len=None, comp_count=None, swa_page=None, page_table=None, page_size=1):
    """One stream for append_multi: contiguous (ring_page, comp_start; as chs.append) or paged
    (swa_page, page_table, page_size; as chs.append_paged). Keeps the tensors alive with it."""
    dt = x_new.dtype
    _need(x_new, "x_new", dim=2)
    _need(z_new, "z_new", dt, 2)
    _need(bias, "bias", torch.float32, 2)
    _need(n_tokens, "n_tokens", torch.int64, 1)
    _need(gate_ring, "gate_ring", dt, 2)
    _need(comp_kv, "comp_kv", dt, 2)
    B, d = x_new.shape
    st = AppendStream()
    st.d = d
    st.x_new, st.z_new, st.bias, st.n_tokens = (x_new.data_ptr(), z_new.data_ptr(), bias.data_ptr(),
                                                n_tokens.data_ptr())
    st.swa_kv, st.gate_ring, st.comp_kv = swa_kv.data_ptr(), gate_ring.data_ptr(), comp_kv.data_ptr()
    st.swa_len = swa_len.data_ptr() if swa_len is not None else None
    st.comp_count = comp_count.data_ptr() if comp_count is not None else None
    if page_table is None:
        _need(swa_kv, "swa_kv", dt, 3)
        st.window = swa_kv.shape[1]
        st.ring_size = int(ring_size if ring_size is not None else gate_ring.shape[0] // B)
        st.ring_page, st.ring_pages = ring_page.data_ptr(), gate_ring.shape[0] // st.ring_size
        st.comp_start, st.comp_rows = comp_start.data_ptr(), comp_kv.shape[0]
    else:
        _need(swa_kv, "swa_pool", dt, 3)
        _need(page_table, "page_table", torch.int32, 2)
        st.window = swa_kv.shape[1]
        st.swa_page, st.swa_pages = swa_page.data_ptr(), swa_kv.shape[0]
        st.ring_size = gate_ring.shape[0] // swa_kv.shape[0]
        st.page_table, st.pt_stride, st.page_size = page_table.data_ptr(), page_table.shape[1], page_size
        st.pool_pages = comp_kv.shape[0] // page_size
    st._keep = (x_new, z_new, bias, n_tokens, swa_kv, gate_ring, comp_kv, ring_page, comp_start, swa_len, comp_count,
                swa_page, page_table)
    return st


def append_multi(m: int, streams):
    """chs_append_multi: the new token of every sequence appended to each stream (a list of
    append_stream(...) descriptions) in one launch. Streams share dtype, batch and m."""
    arr = (AppendStream * len(streams))(*streams)
    x0 = streams[0]._keep[0]
    _check(lib().chs_append_multi(_dtype_code(x0), x0.shape[0], m, len(streams), arr, _stream()), "chs_append_multi")


def index_topk_fp8_paged(q_idx, w, code_pool, scale_pool, page_size: int, page_table, cand_len, k: int, max_cand: int,
                         scores=None, workspace=None, out=None):
    """chs_index_topk_fp8 over paged pools of E4M3 key codes ([rows, dim] uint8) and their fp32
    row scales ([rows]) (chs_index_topk_fp8_paged). Returns (topk [B, k] int32, scores)."""
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(w, "w", torch.float32, 2)
    _need(code_pool, "code_pool", torch.uint8, 2)
    _need(scale_pool, "scale_pool", torch.float32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(cand_len, "cand_len", torch.int64, 1)
    B, nh, dim = q_idx.shape
    _shape(w, (B, nh), "w")
    _shape(cand_len, (B,), "cand_len")
    if code_pool.shape[1] != dim or page_table.shape[0] != B:
        raise ValueError("code_pool must have dim columns and page_table B rows")
    if scale_pool.numel() != code_pool.shape[0]:
        raise ValueError("scale_pool must hold one scale per pool row")
    if scores is not None:
        _need(scores, "scores", torch.float32, 2)
        _shape(scores, (B, max_cand), "scores")
    if workspace is None:
        workspace = index_topk_workspace(B, max_cand, k, q_idx.device)
    if out is None:
        out = torch.empty(B, k, dtype=torch.int32, device=q_idx.device)
    _need(out, "topk", torch.int32, 2)
    _shape(out, (B, k), "topk")
    _check(lib().chs_index_topk_fp8_paged(B, nh, dim, k, _ptr(q_idx), _ptr(w), _ptr(code_pool), _ptr(scale_pool),
                                          code_pool.shape[0] // page_size, page_size, _ptr(page_table),
                                          page_table.shape[1], _ptr(cand_len), int(max_cand), _ptr(scores), _ptr(out),
                                          _ptr(workspace), workspace.numel(), _stream()), "chs_index_topk_fp8_paged")
    return out, scores


def decode_attn_fp8_paged(q, swa_codes, swa_scales, swa_page, swa_len, comp_codes, comp_scales, page_size: int,
                          page_table, comp_len, topk=None, scale=None, max_comp=None, workspace=None, out=None,
                          lse=None):
    """chs_decode_attn_fp8 over paged pools (chs_decode_attn_fp8_paged). swa_codes: [swa_pages, W, d]
    uint8, swa_scales: [swa_pages, W] fp32; comp_codes: [rows, d] uint8, comp_scales: [rows] fp32."""
    _need(q, "q", torch.bfloat16, 3)
    _need(swa_codes, "swa_codes", torch.uint8, 3)
    _need(swa_scales, "swa_scales", torch.float32, 2)
    _need(swa_page, "swa_page", torch.int32, 1)
    _need(swa_len, "swa_len", torch.int32, 1)
    _need(comp_codes, "comp_codes", torch.uint8, 2)
    _need(comp_scales, "comp_scales", torch.float32, 1)
    _need(page_table, "page_table", torch.int32, 2)
    _need(comp_len, "comp_len", torch.int64, 1)
    B, H, d = q.shape
    W = swa_codes.shape[1]
    k = 0
    if topk is not None:
        _need(topk, "topk", torch.int32, 2)
        k = topk.shape[1]
        _shape(topk, (B, k), "topk")
    _attn_shapes(q, swa_codes, swa_len, comp_codes, comp_len)
    _shape(swa_page, (B,), "swa_page")
    _shape(comp_len, (B,), "comp_len")
    _shape(swa_scales, swa_codes.shape[:2], "swa_scales")
    if comp_scales.numel() != comp_codes.shape[0]:
        raise ValueError("comp_scales must hold one scale per pool row")
    if page_table.shape[0] != B:
        raise ValueError("page_table must have B rows")
    if max_comp is None:
        max_comp = int(comp_len.max().item()) if comp_len.numel() else 0
    if scale is None:
        scale = d ** -0.5
    if workspace is None:
        workspace = decode_attn_workspace(torch.bfloat16, B, H, d, W, k, max_comp, q.device)
    out, lse = _attn_outputs(q, out, lse)
    _check(lib().chs_decode_attn_fp8_paged(B, H, d, W, k, float(scale), _ptr(q), _ptr(swa_codes), _ptr(swa_scales),
                                           _ptr(swa_page), swa_codes.shape[0], _ptr(swa_len), _ptr(comp_codes),
                                           _ptr(comp_scales), comp_codes.shape[0] // page_size, page_size,
                                           _ptr(page_table), page_table.shape[1], _ptr(comp_len), _ptr(topk),
                                           int(max_comp), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                           _stream()), "chs_decode_attn_fp8_paged")
    return out, lse
