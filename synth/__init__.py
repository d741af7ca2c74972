"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

Everything here is a pure function of (workload seed, step, worker, tensor,
element): gradients as bfloat16 bits and initial parameters as fp32.  The
numbers come from the C generator in ``synth_gen.c`` (Philox4x32-10, see that
file's header); this module only marshals arrays.  No optimizer arithmetic
lives here.

Flat arrays follow a caller-supplied layout (per-tensor offsets and padded
length), so the same generator serves any consumer's layout; padding elements
are zero.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import configs
from .configs import (ADVERSARIAL, GPT345M, LLAMA055, LLAMA175, SINGLE, WORKLOADS,  # noqa: F401
                      Workload, ragged, reduced)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")
_lib = None
_gpu_lib = None


def build(force: bool = True) -> str:
    """Compile the generator (gcc, OpenMP)."""
    import subprocess
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
               os.path.join(_HERE, "synth_gen.c"), "-o", LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def build_gpu(force: bool = True) -> str:
    """Compile the GPU twin of the generator (hipcc, gfx950)."""
    import subprocess
    if force or not os.path.exists(GPU_LIB_PATH):
        cmd = ["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
               "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", os.path.join(_HERE, "synth_gen.hip"), "-o", GPU_LIB_PATH + ".tmp"]
        subprocess.run(cmd, check=True, capture_output=True)
        os.replace(GPU_LIB_PATH + ".tmp", GPU_LIB_PATH)
    return GPU_LIB_PATH


def gpu_lib():
    global _gpu_lib
    if _gpu_lib is None:
        if not os.path.exists(GPU_LIB_PATH):
            raise RuntimeError(f"{GPU_LIB_PATH} is not built (synth.build_gpu())")
        L = ctypes.CDLL(GPU_LIB_PATH)
        u32, u64, f32, i32, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
        L.synth_gpu_grad_bf16.argtypes = [u32, u32, u32, u32, i32, f32, i32, u64, u64, vp, vp]
        L.synth_gpu_grad_bf16.restype = i32
        L.synth_gpu_param_f32.argtypes = [u32, u32, f32, u64, u64, vp, vp]
        L.synth_gpu_param_f32.restype = i32
        _gpu_lib = L
    return _gpu_lib


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u32, u64, f32, f64, i32 = (ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
                                   ctypes.c_double, ctypes.c_int)
        vp = ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_philox4x32_10.restype = None
        L.synth_normal_scale.argtypes = [f64]
        L.synth_normal_scale.restype = f32
        L.synth_tensor_sigma.argtypes = [u32, u32]
        L.synth_tensor_sigma.restype = f64
        L.synth_grad_bf16.argtypes = [u32, u32, u32, u32, i32, f32, i32, u64, u64, vp]
        L.synth_grad_bf16.restype = None
        L.synth_param_f32.argtypes = [u32, u32, f32, u64, u64, vp]
        L.synth_param_f32.restype = None
        L.synth_u32.argtypes = [u32, u32, u32, u32, u32, u64, u64, vp]
        L.synth_u32.restype = None
        _lib = L
    return _lib


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


def tensor_sigma(wl: Workload, tensor: int) -> float:
    """Gradient standard deviation of one tensor under the workload's recipe."""
    if wl.grad_kind == "iid":
        return float(wl.sigma)
    if wl.grad_kind == "loguniform":
        return float(lib().synth_tensor_sigma(wl.seed, tensor))
    return float("nan")  # Student-t: scale given by t_scale


def grad_tensor(wl: Workload, step: int, worker: int, tensor: int, e0: int = 0,
                n: Optional[int] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """bfloat16 bits (uint16) of elements [e0, e0+n) of one tensor's gradient."""
    numel = wl.tensors[tensor].numel
    if n is None:
        n = numel - e0
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size >= n and out.flags.c_contiguous
    if n == 0:
        return out
    kind, scale = grad_recipe(wl, tensor)
    lib().synth_grad_bf16(wl.seed, tensor, step, worker, kind, scale,
                          1 if wl.quantised(tensor) else 0, e0, n, out.ctypes.data)
    return out


def grad_recipe(wl: Workload, tensor: int):
    """(kind, fp32 scale) of a tensor's gradient: kind 0 normal, 1 Student-t(2)."""
    if wl.grad_kind == "student2":
        return 1, float(np.float32(wl.t_scale))
    return 0, float(lib().synth_normal_scale(tensor_sigma(wl, tensor)))


def param_tensor(wl: Workload, tensor: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    n = wl.tensors[tensor].numel
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.size >= n and out.flags.c_contiguous
    scale = lib().synth_normal_scale(wl.param_sigma)
    lib().synth_param_f32(wl.seed, tensor, scale, 0, n, out.ctypes.data)
    return out


def grads_flat(wl: Workload, offsets: Sequence[int], n_pad: int, step: int, worker: int,
               tensors: Optional[Sequence[int]] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """One worker's gradient for one step, laid out flat at ``offsets``.

    ``tensors`` selects which workload tensors to generate (default: all), in
    which case ``offsets[i]`` is the flat offset of ``tensors[i]``.
    """
    if tensors is None:
        tensors = range(len(wl.tensors))
    if out is None:
        out = np.zeros(n_pad, dtype=np.uint16)
    for off, t in zip(offsets, tensors):
        n = wl.tensors[t].numel
        grad_tensor(wl, step, worker, t, 0, n, out[off:off + n])
    return out


def params_flat(wl: Workload, offsets: Sequence[int], n_pad: int,
                tensors: Optional[Sequence[int]] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    if tensors is None:
        tensors = range(len(wl.tensors))
    if out is None:
        out = np.zeros(n_pad, dtype=np.float32)
    for off, t in zip(offsets, tensors):
        n = wl.tensors[t].numel
        param_tensor(wl, t, out[off:off + n])
    return out


def uniform_u32(seed: int, purpose: int, n: int, tensor: int = 0, step: int = 0,
                worker: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    if n:
        lib().synth_u32(seed, purpose, tensor, step, worker, 0, n, out.ctypes.data)
    return out


# ----------------------------------------------------------------------------
# GPU twin: the same numbers written straight into device tensors


def _gpu_stream(stream):
    import torch
    return (stream or torch.cuda.current_stream()).cuda_stream


def grads_flat_gpu(wl: Workload, offsets: Sequence[int], out, step: int, worker: int,
                   tensors: Optional[Sequence[int]] = None, stream=None) -> None:
    """Fill a device tensor (int16/uint16/bfloat16 view, n_pad long) with one
    worker's gradient for one step, bit-identical to ``grads_flat``.  Padding
    is left as it is."""
    if tensors is None:
        tensors = range(len(wl.tensors))
    if not out.is_contiguous():
        raise ValueError("the generator writes a contiguous flat tensor")
    base = out.data_ptr()
    st = _gpu_stream(stream)
    for off, t in zip(offsets, tensors):
        n = wl.tensors[t].numel
        kind, scale = grad_recipe(wl, t)
        rc = gpu_lib().synth_gpu_grad_bf16(wl.seed, t, step, worker, kind, scale, 1 if wl.quantised(t) else 0,
                                           0, n, base + 2 * int(off), st)
        if rc:
            raise RuntimeError(f"synth_gpu_grad_bf16 failed: hipError {rc}")


def params_flat_gpu(wl: Workload, offsets: Sequence[int], out, tensors: Optional[Sequence[int]] = None,
                    stream=None) -> None:
    if tensors is None:
        tensors = range(len(wl.tensors))
    if not out.is_contiguous():  # a strided view (x inside (x, v) pairs): through a contiguous copy
        tmp = out.contiguous()
        params_flat_gpu(wl, offsets, tmp, tensors, stream)
        out.copy_(tmp)
        return
    base = out.data_ptr()
    st = _gpu_stream(stream)
    scale = lib().synth_normal_scale(wl.param_sigma)
    for off, t in zip(offsets, tensors):
        n = wl.tensors[t].numel
        rc = gpu_lib().synth_gpu_param_f32(wl.seed, t, scale, 0, n, base + 4 * int(off), st)
        if rc:
            raise RuntimeError(f"synth_gpu_param_f32 failed: hipError {rc}")
