"""Seeded synthetic inputs, shared by the GPU tests, the oracle checks and the benchmark.

This module only draws numbers (see gen_core.h); it holds none of the attention method's
arithmetic. Host fillers return numpy arrays; device fillers write into torch CUDA tensors
and produce the same bits as the host fillers for the same (seed, tensor, index).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_c_u64, _c_i64, _c_i32, _c_d, _c_p = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_double, ctypes.c_void_p)
_cpu = None
_gpu = None


def _load_cpu():
    global _cpu
    if _cpu is None:
        path = os.path.join(HERE, "libsynth_cpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run synth/build.py")
        lib = ctypes.CDLL(path)
        lib.syn_stream_of.restype = _c_u64
        lib.syn_stream_of.argtypes = [_c_u64, _c_u64]
        lib.syn_fill_bits.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_p]
        lib.syn_fill_normal_f32.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_d, _c_d, ctypes.c_int, _c_p]
        lib.syn_fill_normal_bf16.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_d, _c_d, _c_p]
        lib.syn_fill_uniform_f32.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_d, _c_d, _c_p]
        lib.syn_fill_normal_f64.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_p]
        lib.syn_spike_basis.argtypes = [_c_u64, _c_u64, _c_i32, _c_i32, _c_p]
        lib.syn_fill_index_keys.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_i64, _c_i32, _c_i32,
                                            _c_p, _c_d, ctypes.c_int, _c_p]
        _cpu = lib
    return _cpu


def _load_gpu():
    global _gpu
    if _gpu is None:
        import torch  # noqa: F401  (torch's HIP runtime must be the one this library binds to)
        path = os.path.join(HERE, "libsynth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run synth/build.py")
        lib = ctypes.CDLL(path)
        lib.syn_gpu_fill_normal.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_d, _c_d, ctypes.c_int, _c_p, _c_p]
        lib.syn_gpu_fill_uniform.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_d, _c_d, _c_p, _c_p]
        lib.syn_gpu_fill_index_keys.argtypes = [_c_u64, _c_u64, _c_u64, _c_i64, _c_i64, _c_i32, _c_i32,
                                                _c_p, _c_d, ctypes.c_int, _c_p, _c_p]
        for f in (lib.syn_gpu_fill_normal, lib.syn_gpu_fill_uniform, lib.syn_gpu_fill_index_keys):
            f.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_c_p)


# ---------------------------------------------------------------- host fillers
def bits(seed: int, tensor: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _load_cpu().syn_fill_bits(seed, tensor, start, count, _ptr(out))
    return out


def normal(seed: int, tensor: int, start: int, count: int, mean: float = 0.0, std: float = 1.0,
           bf16: bool = False) -> np.ndarray:
    """fp32 values of N(mean, std^2); with bf16=True, values rounded to bfloat16 (RNE)."""
    out = np.empty(count, dtype=np.float32)
    _load_cpu().syn_fill_normal_f32(seed, tensor, start, count, mean, std, int(bf16), _ptr(out))
    return out


def normal_bf16_bits(seed: int, tensor: int, start: int, count: int, mean: float = 0.0,
                     std: float = 1.0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    _load_cpu().syn_fill_normal_bf16(seed, tensor, start, count, mean, std, _ptr(out))
    return out


def uniform(seed: int, tensor: int, start: int, count: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _load_cpu().syn_fill_uniform_f32(seed, tensor, start, count, lo, hi, _ptr(out))
    return out


def uniform01_f64(seed: int, tensor: int, start: int, count: int) -> np.ndarray:
    """Uniforms in [0, 1) with 53 random bits (used for length jitter)."""
    return (bits(seed, tensor, start, count) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def spike_basis(seed: int, tensor: int, nspike: int, dim: int) -> np.ndarray:
    U = np.empty((nspike, dim), dtype=np.float64)
    _load_cpu().syn_spike_basis(seed, tensor, nspike, dim, _ptr(U))
    return U


def index_keys(seed: int, t_noise: int, t_load: int, row_start: int, nrows: int, dim: int,
               U: np.ndarray, alpha: float, bf16: bool) -> np.ndarray:
    U = np.ascontiguousarray(U, dtype=np.float64)
    out = np.empty((nrows, dim), dtype=np.float32)
    _load_cpu().syn_fill_index_keys(seed, t_noise, t_load, row_start, nrows, dim, U.shape[0],
                                    _ptr(U), alpha, int(bf16), _ptr(out))
    return out


def permutation_prefix(seed: int, tensor: int, n: int, count: int) -> np.ndarray:
    """First `count` entries of a seeded Fisher-Yates shuffle of range(n)."""
    perm = np.arange(n, dtype=np.int64)
    r = bits(seed, tensor, 0, count)
    for i in range(count):
        j = i + int(r[i] % np.uint64(n - i))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


# ---------------------------------------------------------------- device fillers
def _stream_ptr(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} launch failed with hipError {rc}")


def gpu_normal(out, seed: int, tensor: int, start: int = 0, mean: float = 0.0, std: float = 1.0):
    import torch
    lib = _load_gpu()
    assert out.is_cuda and out.is_contiguous() and out.dtype in (torch.float32, torch.bfloat16)
    _check(lib.syn_gpu_fill_normal(seed, tensor, start, out.numel(), mean, std,
                                   int(out.dtype == torch.bfloat16), ctypes.c_void_p(out.data_ptr()),
                                   _stream_ptr(torch)), "syn_gpu_fill_normal")
    return out


def gpu_uniform(out, seed: int, tensor: int, start: int = 0, lo: float = 0.0, hi: float = 1.0):
    import torch
    lib = _load_gpu()
    assert out.is_cuda and out.is_contiguous() and out.dtype == torch.float32
    _check(lib.syn_gpu_fill_uniform(seed, tensor, start, out.numel(), lo, hi,
                                    ctypes.c_void_p(out.data_ptr()), _stream_ptr(torch)),
           "syn_gpu_fill_uniform")
    return out


def gpu_index_keys(out, seed: int, t_noise: int, t_load: int, row_start: int, U_dev, alpha: float):
    """out: CUDA tensor [nrows, dim] (fp32 or bf16); U_dev: CUDA float64 tensor [nspike, dim]."""
    import torch
    lib = _load_gpu()
    assert out.is_cuda and out.is_contiguous() and out.dim() == 2
    assert U_dev.is_cuda and U_dev.dtype == torch.float64 and U_dev.shape[1] == out.shape[1]
    _check(lib.syn_gpu_fill_index_keys(seed, t_noise, t_load, row_start, out.shape[0], out.shape[1],
                                       U_dev.shape[0], ctypes.c_void_p(U_dev.data_ptr()), alpha,
                                       int(out.dtype == torch.bfloat16), ctypes.c_void_p(out.data_ptr()),
                                       _stream_ptr(torch)), "syn_gpu_fill_index_keys")
    return out
