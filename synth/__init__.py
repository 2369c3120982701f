"""Seeded synthetic inputs shared by the fp64 oracle and the GPU library.

This module draws random numbers and rounds them to a storage format. It holds
none of the MoE layer's arithmetic. Every element is a pure function of
``(seed, tensor_id, index)`` (SplitMix64 counters into Box-Muller, see
``synth.c``), so any slice of any tensor can be regenerated independently.

Stored values are returned as numpy arrays of the storage type:
``uint16`` bit patterns for bf16, ``float32`` for fp32, for fp8 weights an
``Fp8Rows`` pair of ``uint8`` E4M3 codes with one ``float32`` scale per row,
and for MXFP4 weights an ``MxFp4Rows`` pair of packed E2M1 codes with one
E8M0 scale byte per 32 values.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

# Tensor ids: one independent random stream per logical tensor of a layer.
TID_U = 1
TID_W_ROUTE = 2
TID_W_GATE = 3
TID_W_UP = 4
TID_W_DOWN = 5
TID_W_LDOWN = 6
TID_W_LUP = 7
TID_WS_GATE = 8
TID_WS_UP = 9
TID_WS_DOWN = 10
TID_U_NOISE = 11  # noise of the planted-routing token vectors


def build() -> str:
    """Compile libsynth.so with gcc (OpenMP). Always recompiles."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _SO, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, dbl, ptr = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_f64.argtypes = [u64, u64, u64, u64, dbl, dbl, ptr]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, dbl, ptr]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, dbl, ptr]
        lib.synth_round_bf16.argtypes = [ptr, u64, ptr]
        lib.synth_round_f32.argtypes = [ptr, u64, ptr]
        lib.synth_f64_to_bf16.argtypes = [dbl]
        lib.synth_f64_to_bf16.restype = ctypes.c_uint16
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_splitmix64.argtypes = [u64, u64]
        lib.synth_splitmix64.restype = u64
        lib.synth_f64_to_e4m3.argtypes = [dbl]
        lib.synth_f64_to_e4m3.restype = ctypes.c_uint8
        lib.synth_normal_e4m3_rows.argtypes = [u64, u64, u64, u64, u64, dbl, ptr, ptr]
        lib.synth_f64_to_e2m1.argtypes = [dbl]
        lib.synth_f64_to_e2m1.restype = ctypes.c_uint8
        lib.synth_normal_mxfp4_rows.argtypes = [u64, u64, u64, u64, u64, dbl, ptr, ptr]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f64(seed: int, tid: int, count: int, std: float = 1.0,
               start: int = 0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(int(count), dtype=np.float64)
    _load().synth_normal_f64(seed, tid, start, int(count), mean, std, _ptr(out))
    return out


def normal_stored(seed: int, tid: int, count: int, std: float, dtype: str,
                  start: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Draw ``std * N(0,1)`` elements [start, start+count) rounded to ``dtype``."""
    count = int(count)
    if dtype == "bf16":
        if out is None:
            out = np.empty(count, dtype=np.uint16)
        _load().synth_normal_bf16(seed, tid, start, count, std, _ptr(out))
    elif dtype == "f32":
        if out is None:
            out = np.empty(count, dtype=np.float32)
        _load().synth_normal_f32(seed, tid, start, count, std, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype (nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    if dtype == "bf16":
        out = np.empty(flat.size, dtype=np.uint16)
        _load().synth_round_bf16(_ptr(flat), flat.size, _ptr(out))
    elif dtype == "f32":
        out = np.empty(flat.size, dtype=np.float32)
        _load().synth_round_f32(_ptr(flat), flat.size, _ptr(out))
    else:
        raise ValueError(dtype)
    return out.reshape(x.shape)


def f64_to_bf16_bits(x: float) -> int:
    return int(_load().synth_f64_to_bf16(float(x)))


def splitmix64(key: int, n: int) -> int:
    return int(_load().synth_splitmix64(key, n))


def stream_key(seed: int, tid: int) -> int:
    return int(_load().synth_stream_key(seed, tid))


@dataclasses.dataclass(frozen=True)
class Fp8Rows:
    """A matrix stored as OCP FP8 E4M3 codes with one fp32 scale per row:
    row r holds scale[r] times the E4M3 value of each code."""
    codes: np.ndarray   # uint8 [..., rows, cols]
    scale: np.ndarray   # float32 [..., rows]

    @property
    def shape(self):
        return self.codes.shape


def f64_to_e4m3(x: float) -> int:
    return int(_load().synth_f64_to_e4m3(float(x)))


def normal_fp8_rows(seed: int, tid: int, rows: int, cols: int, std: float,
                    start: int = 0, codes: np.ndarray | None = None,
                    scale: np.ndarray | None = None) -> Fp8Rows:
    """``std * N(0,1)`` elements [start, start + rows*cols) as E4M3 rows: the
    same draws as ``normal_stored`` with the same arguments, each row scaled by
    max|row| / 448 (rounded to fp32) and rounded to E4M3, nearest-even."""
    rows, cols = int(rows), int(cols)
    if codes is None:
        codes = np.empty(rows * cols, dtype=np.uint8)
    if scale is None:
        scale = np.empty(rows, dtype=np.float32)
    _load().synth_normal_e4m3_rows(seed, tid, start, rows, cols, std, _ptr(codes), _ptr(scale))
    return Fp8Rows(codes.reshape(rows, cols), scale.reshape(rows))


@dataclasses.dataclass(frozen=True)
class MxFp4Rows:
    """A matrix stored as OCP MXFP4: E2M1 codes packed two per byte (element
    2i in the low nibble of byte i of its row) and one E8M0 scale byte per
    32 consecutive elements of a row (value 2^(s - 127))."""
    packed: np.ndarray        # uint8 [..., rows, cols / 2]
    block_scale: np.ndarray   # uint8 [..., rows, cols / 32]

    @property
    def shape(self):
        return self.packed.shape[:-1] + (self.packed.shape[-1] * 2,)


def f64_to_e2m1(x: float) -> int:
    return int(_load().synth_f64_to_e2m1(float(x)))


def normal_mxfp4_rows(seed: int, tid: int, rows: int, cols: int, std: float,
                      start: int = 0, packed: np.ndarray | None = None,
                      scale: np.ndarray | None = None) -> MxFp4Rows:
    """``std * N(0,1)`` elements [start, start + rows*cols) as MXFP4 rows: the
    same draws as ``normal_stored``, each run of 32 scaled by 2^e with
    e = floor(log2 max|v|) - 2 and rounded to E2M1 nearest-even."""
    rows, cols = int(rows), int(cols)
    assert cols % 32 == 0
    if packed is None:
        packed = np.empty(rows * cols // 2, dtype=np.uint8)
    if scale is None:
        scale = np.empty(rows * cols // 32, dtype=np.uint8)
    _load().synth_normal_mxfp4_rows(seed, tid, start, rows, cols, std, _ptr(packed), _ptr(scale))
    return MxFp4Rows(packed.reshape(rows, cols // 2), scale.reshape(rows, cols // 32))
