"""Build and load the C oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None
# storage format codes the C oracle takes
KV_FORMATS = {"bf16": 0, "fp8": 1, "mxfp4": 2}


def build_oracle(force: bool = False) -> str:
    """Compile attention.c with gcc (portable x86-64 code, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_attention.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.c_double, P, P, P, P,
                                         P, P, P, P, i, i, i, i, P, P]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_decode_bf16.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_decode_e4m3.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_decode_e2m1.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_decode_e8m0.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def oracle_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attention(w, rows=None, key_lo: int = 0, key_hi: int = 2**31 - 1):
    """fp64 attention for workload `w` (see workloads.synth for the layout).

    rows: None for every (p, i, h), else an int array [n][3] of (p, i, h).
    Returns (out, lse): out [P][W][Hq][D] / [n][D], lse [P][W][Hq] / [n] (float64).
    """
    lib = _load()
    if rows is None:
        out = np.zeros((w.P, w.W, w.Hq, w.D), dtype=np.float64)
        lse = np.zeros((w.P, w.W, w.Hq), dtype=np.float64)
        rows_arr, n = None, 0
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
        n = rows_arr.shape[0]
        out = np.zeros((n, w.D), dtype=np.float64)
        lse = np.zeros((n,), dtype=np.float64)
    fmt = KV_FORMATS[w.kv]
    scaled = fmt != 0
    if getattr(w, "v_layout", 0) == 1:     # token-major value pages (bf16 only)
        if w.kv != "bf16":
            raise ValueError("token-major value pages are a bf16 layout")
        fmt = 3
    arrs = [np.ascontiguousarray(a) if a is not None else None
            for a in (w.q, w.k_pool, w.v_pool, w.k_scale if scaled else None,
                      w.v_scale if scaled else None, w.block_table, w.seq_lens)]
    rc = lib.oracle_attention(w.P, w.W, w.Hq, w.Hkv, w.D, w.num_pages, w.block_table.shape[1],
                              int(w.causal), fmt, float(w.scale), *[_ptr(a) for a in arrs],
                              _ptr(rows_arr), n, int(key_lo), int(key_hi),
                              int(getattr(w, "window_left", 0)), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    return out, lse


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(bits, dtype=np.uint16)
    dst = np.empty(src.shape, dtype=np.float64)
    _load().oracle_decode_bf16(_ptr(src), _ptr(dst), src.size)
    return dst


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    dst = np.empty(src.shape, dtype=np.float64)
    _load().oracle_decode_e4m3(_ptr(src), _ptr(dst), src.size)
    return dst


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """One E2M1 code per element (its low nibble) -> float64."""
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    dst = np.empty(src.shape, dtype=np.float64)
    _load().oracle_decode_e2m1(_ptr(src), _ptr(dst), src.size)
    return dst


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    dst = np.empty(src.shape, dtype=np.float64)
    _load().oracle_decode_e8m0(_ptr(src), _ptr(dst), src.size)
    return dst


if __name__ == "__main__":
    print(build_oracle(force="--force" in sys.argv))
