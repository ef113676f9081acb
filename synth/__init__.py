"""Seeded synthetic inputs (counter-based SplitMix64), shared by the oracle's
tests and the HIP library's tests and benchmark.

Holds no arithmetic of the decode method itself: only random draws and their
rounding to storage types.  See ``synth.c`` for the generator's definition.
The workload recipes (which tensor ids and distributions each workload uses)
live in :mod:`synth.recipes`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``libsynth.so`` with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-D_GNU_SOURCE", "-shared", "-fPIC", os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, dbl, ptr = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.synth_u64.argtypes = [u64, u64, u64, u64, i64, ptr]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, i64, dbl, dbl, ctypes.c_int, ptr]
    lib.synth_normal_f16.argtypes = [u64, u64, u64, u64, i64, dbl, dbl, ctypes.c_int, ptr]
    lib.synth_uniform_i32.argtypes = [u64, u64, u64, u64, i64, i32, i32, ptr]
    lib.synth_uniform_f64.argtypes = [u64, u64, u64, u64, i64, ptr]
    lib.synth_q4k_fields.argtypes = [u64, u64, i32, i32, i32, i32, dbl, ptr, ptr, ptr, ptr, ptr]
    lib.synth_gdn_step_inputs.argtypes = [u64, u64, i32, i32, i32, i32, ptr, ptr, ptr, ptr, ptr]
    lib.synth_f64_to_f16.argtypes = [dbl]
    lib.synth_f64_to_f16.restype = ctypes.c_uint16
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def u64(seed, tensor, sub, n, start=0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_u64(seed, tensor, sub, start, n, _p(out))
    return out


def normal_f32(seed, tensor, sub, n, mean=0.0, std=1.0, start=0, absval=False) -> np.ndarray:
    out = np.empty(n, np.float32)
    _load().synth_normal_f32(seed, tensor, sub, start, n, mean, std, int(absval), _p(out))
    return out


def normal_f16(seed, tensor, sub, n, mean=0.0, std=1.0, start=0, absval=False) -> np.ndarray:
    """fp16 values as their uint16 bit patterns."""
    out = np.empty(n, np.uint16)
    _load().synth_normal_f16(seed, tensor, sub, start, n, mean, std, int(absval), _p(out))
    return out


def uniform_i32(seed, tensor, sub, n, lo, hi, start=0) -> np.ndarray:
    out = np.empty(n, np.int32)
    _load().synth_uniform_i32(seed, tensor, sub, start, n, lo, hi, _p(out))
    return out


def uniform_f64(seed, tensor, sub, n, start=0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform_f64(seed, tensor, sub, start, n, _p(out))
    return out


def f64_to_f16_bits(x: float) -> int:
    return int(_load().synth_f64_to_f16(float(x)))


def q4k_fields(seed, tensor, n_out, n_in, r0=0, r1=None, d_std=0.01, out=None) -> dict:
    """Field arrays of a Q4_K-style matrix (rows [r0, r1)).

    Returns d, dmin (uint16 fp16 bits, [rows][n_in/256]), sc, m (uint8 0..63,
    [rows][n_in/256][8]) and q (uint8 0..15, [rows][n_in]).  `out` may hold
    arrays of those shapes from an earlier call, which are then refilled.
    """
    if n_in % 256:
        raise ValueError("n_in must be a multiple of 256")
    r1 = n_out if r1 is None else r1
    rows, nsb = r1 - r0, n_in // 256
    shapes = {"d": ((rows, nsb), np.uint16), "dmin": ((rows, nsb), np.uint16), "sc": ((rows, nsb, 8), np.uint8),
              "m": ((rows, nsb, 8), np.uint8), "q": ((rows, n_in), np.uint8)}
    f = {}
    for k, (shp, dt) in shapes.items():
        a = None if out is None else out.get(k)
        f[k] = a if a is not None and a.shape == shp and a.dtype == dt and a.flags["C_CONTIGUOUS"] else np.empty(shp, dt)
    _load().synth_q4k_fields(seed, tensor, n_out, n_in, r0, r1, d_std, _p(f["d"]), _p(f["dmin"]), _p(f["sc"]),
                             _p(f["m"]), _p(f["q"]))
    f.update(n_out=rows, n_in=n_in)
    return f


def gdn_step_inputs(seed, tensor, T, nh, dk, dv) -> dict:
    """q, k (L2-normalised), v, g = sigmoid(N(2, .5)), beta = sigmoid(N(0, 1))."""
    if dk > 512:
        raise ValueError("dk must be <= 512")
    q = np.empty((T, nh, dk), np.float32)
    k = np.empty((T, nh, dk), np.float32)
    v = np.empty((T, nh, dv), np.float32)
    g = np.empty((T, nh), np.float32)
    beta = np.empty((T, nh), np.float32)
    _load().synth_gdn_step_inputs(seed, tensor, T, nh, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta))
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta}
