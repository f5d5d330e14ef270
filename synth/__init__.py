"""Seeded, counter-based synthetic inputs shared by the oracle side and the GPU side.

This package generates inputs only; it holds none of the MoGE layer's arithmetic.
The generator is defined in ``synth_def.h`` (SplitMix64 words -> twelve 16-bit
uniforms -> an approximately N(0,1) variate -> one binary32 multiply by the
standard deviation -> optional round-to-nearest-even bf16).  Three
implementations of that one definition live here:

* ``libsynth_cpu.so`` (C + OpenMP): used to feed the CPU oracle;
* ``libsynth_gpu.so`` (HIP kernel): fills device buffers for the GPU path;
* :func:`normal_np` (NumPy): a slow transcription used only to test the C one.

All three give identical bytes for the same ``(seed, tensor_id, index)``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

_cpu = None
_gpu = None

GAMMA = 0x9E3779B97F4A7C15
SEED_SALT = 0x5851F42D4C957F2D
_M64 = (1 << 64) - 1


def _load_cpu():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            raise RuntimeError(f"{CPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(CPU_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        for name, ptr in (("synth_fill_f32", ctypes.c_void_p), ("synth_fill_bf16", ctypes.c_void_p)):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ptr]
        _cpu = lib
    return _cpu


def _load_gpu():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        lib.synth_fill_device.restype = ctypes.c_int
        lib.synth_fill_device.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        _gpu = lib
    return _gpu


def normal_host(seed: int, tensor_id: int, n: int, std: float, bf16: bool, start: int = 0) -> np.ndarray:
    """Elements ``[start, start+n)`` of stream ``(seed, tensor_id)`` on the host.

    Returns uint16 bf16 bit patterns when ``bf16`` else float32 values."""
    lib = _load_cpu()
    if bf16:
        out = np.empty(n, dtype=np.uint16)
        lib.synth_fill_bf16(seed, tensor_id, start, n, float(np.float32(std)), out.ctypes.data)
    else:
        out = np.empty(n, dtype=np.float32)
        lib.synth_fill_f32(seed, tensor_id, start, n, float(np.float32(std)), out.ctypes.data)
    return out


def fill_device(tensor, seed: int, tensor_id: int, std: float, start: int = 0) -> None:
    """Fills a contiguous CUDA/HIP torch tensor (bfloat16 or float32) in place on its current stream."""
    import torch

    if not tensor.is_contiguous():
        raise ValueError("fill_device needs a contiguous tensor")
    if tensor.dtype == torch.bfloat16:
        as_bf16 = 1
    elif tensor.dtype == torch.float32:
        as_bf16 = 0
    else:
        raise ValueError(f"unsupported dtype {tensor.dtype}")
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _load_gpu().synth_fill_device(seed, tensor_id, start, tensor.numel(), float(np.float32(std)),
                                       tensor.data_ptr(), as_bf16, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_device failed with hipError {rc}")


# ---------------------------------------------------------------------------
# NumPy transcription of the same definition (slow; used to test the C filler)
# ---------------------------------------------------------------------------

def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def key_int(seed: int, tensor_id: int) -> int:
    return _mix_int(_mix_int(seed ^ SEED_SALT) + (tensor_id + 1) * GAMMA)


def normal_np(seed: int, tensor_id: int, n: int, std: float, bf16: bool, start: int = 0) -> np.ndarray:
    key = np.uint64(key_int(seed, tensor_id))
    i = np.arange(start, start + n, dtype=np.uint64)
    s = np.zeros(n, dtype=np.int64)
    with np.errstate(over="ignore"):
        for j in range(3):
            w = _mix_np(key + (np.uint64(3) * i + np.uint64(j + 1)) * np.uint64(GAMMA))
            for sh in (0, 16, 32, 48):
                s += ((w >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.int64)
    s -= 393210
    c = np.float32(std) * np.float32(1.0 / 65536.0)
    v = s.astype(np.float32) * c
    if not bf16:
        return v
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
