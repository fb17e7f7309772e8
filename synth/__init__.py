"""Seeded synthetic inputs shared by the GPU tests, the benchmark and the oracle.

This package holds no arithmetic of the layer itself: it only produces input
tensors (bf16 bit patterns, fp32 router logits) from a counter-based generator
whose definition is written out in ``gen.c``.  A host build (``gen.c``) and a
device build (``gen_gpu.hip``) produce identical bits for the same tensor key
and row block, so the oracle can regenerate any rows it needs on the CPU while
the GPU path generates multi-gigabyte weights in device memory.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_gpu = None


def _load_host():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run synth/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        i64, u64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        lib.synth_normal_bf16_rows.argtypes = [vp, u64, ctypes.c_double, i64, i64, i64]
        lib.synth_normal_f32_rows.argtypes = [vp, u64, i64, i64, i64]
        lib.synth_ternary_bf16_rows.argtypes = [vp, u64, i64, i64, i64]
        lib.synth_affine_bf16_rows.argtypes = [vp, u64, ctypes.c_double, ctypes.c_double, i64, i64, i64]
        lib.synth_keep_bits_rows.argtypes = [vp, i64, u64, ctypes.c_double, i64, i64, i64]
        lib.synth_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        lib.synth_splitmix64_next.restype = ctypes.c_uint64
        _host = lib
    return _host


def _load_gpu():
    global _gpu
    if _gpu is None:
        path = os.path.join(_HERE, "libsynth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run synth/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        i64, u64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        lib.synth_gpu_normal_bf16.argtypes = [vp, i64, u64, ctypes.c_double, i64, i64, i64, vp]
        lib.synth_gpu_ternary_bf16.argtypes = [vp, i64, u64, i64, i64, i64, vp]
        lib.synth_gpu_normal_f32.argtypes = [vp, i64, u64, i64, i64, i64, vp]
        for f in (lib.synth_gpu_normal_bf16, lib.synth_gpu_ternary_bf16, lib.synth_gpu_normal_f32):
            f.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def splitmix64_stream(seed: int, n: int) -> list[int]:
    """First n outputs of a SplitMix64 generator seeded with ``seed`` (for known-answer tests)."""
    lib = _load_host()
    st = ctypes.c_uint64(seed)
    return [int(lib.synth_splitmix64_next(ctypes.byref(st))) for _ in range(n)]


# ----------------------------------------------------------------------------- host generation
def normal_bf16(seed: int, rows: int, cols: int, sigma: float, r0: int = 0) -> np.ndarray:
    """Rows [r0, r0+rows) of the (.. x cols) bf16 tensor with key ``seed``; uint16 bit patterns."""
    out = np.empty((rows, cols), dtype=np.uint16)
    if rows:
        _load_host().synth_normal_bf16_rows(out.ctypes.data, seed, float(sigma), cols, r0, rows)
    return out


def normal_f32(seed: int, rows: int, cols: int, r0: int = 0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    if rows:
        _load_host().synth_normal_f32_rows(out.ctypes.data, seed, cols, r0, rows)
    return out


def ternary_bf16(seed: int, rows: int, cols: int, r0: int = 0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    if rows:
        _load_host().synth_ternary_bf16_rows(out.ctypes.data, seed, cols, r0, rows)
    return out


def affine_bf16(seed: int, rows: int, cols: int, mean: float, sigma: float, r0: int = 0) -> np.ndarray:
    """bf16 values (float)(mean + z sigma), z the tensor's N(0,1)-like stream (norm scales near one)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    if rows:
        _load_host().synth_affine_bf16_rows(out.ctypes.data, seed, float(mean), float(sigma), cols, r0, rows)
    return out


def keep_bits(seed: int, rows: int, cols: int, p: float, ldk: int | None = None, r0: int = 0) -> np.ndarray:
    """Dropout keep mask, kept with probability 1 - p: uint8 [rows x ldk], column c in bit c % 8 of byte c // 8."""
    ldk = (cols + 7) // 8 if ldk is None else ldk
    assert ldk >= (cols + 7) // 8 and 0.0 <= p < 1.0
    out = np.empty((rows, ldk), dtype=np.uint8)
    if rows:
        _load_host().synth_keep_bits_rows(out.ctypes.data, ldk, seed, float(p), cols, r0, rows)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- device generation
def _stream_ptr(torch, t):
    return torch.cuda.current_stream(t.device).cuda_stream


def gpu_normal_bf16_(t, seed: int, sigma: float, r0: int = 0):
    """Fill a 2-D (or 1-D) cuda tensor of 2-byte elements in place with rows [r0, ..) of tensor ``seed``."""
    import torch
    v = t if t.dim() == 2 else t.view(1, -1)
    assert v.element_size() == 2 and v.stride(1) == 1
    rc = _load_gpu().synth_gpu_normal_bf16(v.data_ptr(), v.stride(0), seed, float(sigma), v.shape[1], r0,
                                          v.shape[0], _stream_ptr(torch, v))
    if rc:
        raise RuntimeError(f"synth_gpu_normal_bf16 failed ({rc})")
    return t


def gpu_ternary_bf16_(t, seed: int, r0: int = 0):
    import torch
    v = t if t.dim() == 2 else t.view(1, -1)
    assert v.element_size() == 2 and v.stride(1) == 1
    rc = _load_gpu().synth_gpu_ternary_bf16(v.data_ptr(), v.stride(0), seed, v.shape[1], r0, v.shape[0],
                                           _stream_ptr(torch, v))
    if rc:
        raise RuntimeError(f"synth_gpu_ternary_bf16 failed ({rc})")
    return t


def gpu_normal_f32_(t, seed: int, r0: int = 0):
    import torch
    v = t if t.dim() == 2 else t.view(1, -1)
    assert v.dtype == torch.float32 and v.stride(1) == 1
    rc = _load_gpu().synth_gpu_normal_f32(v.data_ptr(), v.stride(0), seed, v.shape[1], r0, v.shape[0],
                                         _stream_ptr(torch, v))
    if rc:
        raise RuntimeError(f"synth_gpu_normal_f32 failed ({rc})")
    return t


def device_inputs(workload, device="cuda"):
    """Allocate and fill every input tensor of a workload (synth.configs) on the GPU, bit-identical to the host
    generator.  1-D tensors (biases) are generated as one row."""
    import torch
    out = {}
    for name, spec in workload.tensors.items():
        if spec.kind == "f32":
            t = torch.empty(spec.shape, dtype=torch.float32, device=device)
            gpu_normal_f32_(t, spec.seed)
        else:
            t = torch.empty(spec.shape, dtype=torch.bfloat16, device=device)
            gpu_normal_bf16_(t, spec.seed, spec.sigma)
        out[name] = t
    return out


def host_rows(spec, rows=None):
    """Rows of one workload tensor on the host (all rows by default): uint16 bf16 bits, or float32 for 'f32'."""
    shape = spec.shape if len(spec.shape) == 2 else (1, spec.shape[0])
    if rows is None:
        rows = range(shape[0])
    rows = list(rows)
    gen = (lambda r0, n: normal_f32(spec.seed, n, shape[1], r0)) if spec.kind == "f32" else \
        (lambda r0, n: normal_bf16(spec.seed, n, shape[1], spec.sigma, r0))
    if rows == list(range(rows[0], rows[0] + len(rows))):
        out = gen(rows[0], len(rows))
    else:
        out = np.concatenate([gen(r, 1) for r in rows], axis=0)
    return out if len(spec.shape) == 2 else out.reshape(-1)


def prenorm_inputs(workload, p_drop: float = 0.1) -> dict:
    """Host inputs of the pre-norm layer composition of a TP = 1 workload, beyond its GEMM operands: the
    two norms' scales (bf16 near one) and shifts, and the two dropout keep masks (the random draws of the
    attention and MLP bias-dropout-add).  Keys 1000 * workload + 50 .. 55."""
    d = workload.dims
    M, H = d["M"], d["H"]
    base = 1000 * (2 if workload.name.startswith("gpt345m") else 9) + 50
    return dict(g1=affine_bf16(base, 1, H, 1.0, 0.1)[0], beta1=normal_bf16(base + 1, 1, H, 0.1)[0],
                g2=affine_bf16(base + 2, 1, H, 1.0, 0.1)[0], beta2=normal_bf16(base + 3, 1, H, 0.1)[0],
                keep1=keep_bits(base + 4, M, H, p_drop), keep2=keep_bits(base + 5, M, H, p_drop), p_drop=p_drop)
