"""ctypes front end of the fp64 C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark). The arithmetic lives in oracle.c; this file only builds it,
marshals numpy arrays and converts adapter dictionaries into the oracle's
concatenated storage (A_s rows, then B_s rows, slot after slot).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc: -O2, OpenMP, no fast-math, no FP contraction
    (sums stay in source order)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            sig = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
            lib.oracle_lora_rows.argtypes = sig + [_I, _P, _P, _P, _I, _P]
            lib.oracle_lora_rows.restype = _I
            lib.oracle_lora_merged.argtypes = sig + [_P]
            lib.oracle_lora_merged.restype = _I
            lib.oracle_lora_grouped.argtypes = sig + [_P]
            lib.oracle_lora_grouped.restype = _I
            lib.oracle_decode_bf16.argtypes = [_P, _P, ctypes.c_int64]
            lib.oracle_decode_bf16.restype = None
            lib.oracle_threads.restype = _I
            lib.oracle_set_threads.argtypes = [_I]
            _lib = lib
    return _lib


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_bf16(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def _ptr(a):
    return a.ctypes.data


def _pack(dtype, S, d_in, d_out, adapters):
    """adapters: {slot: object with rank, alpha, A [r, d_in], B [d_out, r]}."""
    npdt = np.uint16 if dtype == "bf16" else np.float32
    rank = np.zeros(S, np.int32)
    alpha = np.zeros(S, np.float64)
    A_parts, B_parts = [], []
    for s in range(S):
        a = adapters.get(s)
        if a is None or a.rank == 0:
            continue
        rank[s] = a.rank
        alpha[s] = a.alpha
        A_parts.append(np.ascontiguousarray(a.A, npdt).reshape(a.rank, d_in))
        B_parts.append(np.ascontiguousarray(a.B, npdt).reshape(d_out, a.rank))
    A_cat = np.concatenate([p.ravel() for p in A_parts]) if A_parts else np.zeros(1, npdt)
    B_cat = np.concatenate([p.ravel() for p in B_parts]) if B_parts else np.zeros(1, npdt)
    return rank, alpha, A_cat, B_cat


def _args(dtype, x, W, S, adapters, slot_ids):
    npdt = np.uint16 if dtype == "bf16" else np.float32
    x = np.ascontiguousarray(x, npdt)
    W = np.ascontiguousarray(W, npdt)
    T, d_in = x.shape
    d_out = W.shape[0]
    assert W.shape[1] == d_in
    slot_ids = np.ascontiguousarray(slot_ids, np.int32)
    assert slot_ids.shape == (T,)
    rank, alpha, A_cat, B_cat = _pack(dtype, S, d_in, d_out, adapters)
    keep = (x, W, rank, alpha, A_cat, B_cat, slot_ids)
    head = [1 if dtype == "bf16" else 0, T, d_in, d_out, S,
            _ptr(x), _ptr(W), _ptr(rank), _ptr(alpha), _ptr(A_cat), _ptr(B_cat), _ptr(slot_ids)]
    return head, keep, T, d_out, int(rank.max(initial=0))


def lora_rows(dtype, x, W, S, adapters, slot_ids, rows=None, want_h=False, h_width=None, want_base=False):
    """fp64 y for the requested rows (all rows if None); optionally h and the
    base term x W^T of the same rows (from the same pass over W).

    Returns y [n, d_out], then h [n, h_width] if want_h, then base [n, d_out]
    if want_base (a tuple when either is asked for)."""
    head, keep, T, d_out, rmax = _args(dtype, x, W, S, adapters, slot_ids)
    if rows is None:
        rows_arr, n, rows_p = None, T, None
    else:
        rows_arr = np.ascontiguousarray(rows, np.int32)
        n, rows_p = len(rows_arr), _ptr(rows_arr)
    y = np.empty((n, d_out), np.float64)
    hw = int(h_width if h_width is not None else max(rmax, 1))
    h = np.empty((n, hw), np.float64) if want_h else None
    base = np.empty((n, d_out), np.float64) if want_base else None
    rc = _load().oracle_lora_rows(*head, n, rows_p, _ptr(y), _ptr(h) if want_h else None, hw,
                                  _ptr(base) if want_base else None)
    if rc != 0:
        raise ValueError("oracle: slot id or row index out of range")
    del keep, rows_arr
    out = (y,) + ((h,) if want_h else ()) + ((base,) if want_base else ())
    return out if len(out) > 1 else y


def lora_merged(dtype, x, W, S, adapters, slot_ids):
    head, keep, T, d_out, _ = _args(dtype, x, W, S, adapters, slot_ids)
    y = np.empty((T, d_out), np.float64)
    if _load().oracle_lora_merged(*head, _ptr(y)) != 0:
        raise ValueError("oracle: slot id out of range")
    del keep
    return y


def lora_grouped(dtype, x, W, S, adapters, slot_ids):
    head, keep, T, d_out, _ = _args(dtype, x, W, S, adapters, slot_ids)
    y = np.empty((T, d_out), np.float64)
    if _load().oracle_lora_grouped(*head, _ptr(y)) != 0:
        raise ValueError("oracle: slot id out of range")
    del keep
    return y
