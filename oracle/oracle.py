"""ctypes binding of the CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It never touches the HIP library and the HIP library never
touches it; the two meet only in tests, through inputs from
``mla_tree_verify_02_amd.inputs``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "mtv_oracle.c")]
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (IEEE double, no contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", *CFLAGS, "-o", tmp, *SOURCES, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.mtv_oracle_run.restype = ctypes.c_int
        lib.mtv_oracle_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, P, P, P, P, P, ctypes.c_double,
                                       P, ctypes.c_int64, P, P, P, P, ctypes.c_int]
        lib.mtv_oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.mtv_oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.mtv_oracle_bf16_to_f64.restype = ctypes.c_double
        lib.mtv_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def run(q: np.ndarray, kv_pool: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
        tree_mask: np.ndarray, scale: float, *, rows: Optional[Sequence[int]] = None,
        threads: int = 0, want_f64: bool = False):
    """Compute the verify attention on the CPU.

    q         uint16 (bf16 bits) [B, N, H, 576]
    kv_pool   uint16 (bf16 bits) [P, 576]
    page_table int32 [B, max_kv]; seq_lens int32 [B]; tree_mask uint32 [B, N, W]
    rows      optional flat row ids (b*N + i)*H + h; others are left as zeros/NaN
    Returns (out_bf16 uint16 [B,N,H,512], lse float32 [B,N,H]) and, with
    want_f64, the unrounded (out float64, lse float64) as well.
    """
    lib = load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv_pool = np.ascontiguousarray(kv_pool, dtype=np.uint16)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tree_mask = np.ascontiguousarray(tree_mask, dtype=np.uint32)
    B, N, H, D = q.shape
    if D != 576 or kv_pool.ndim != 2 or kv_pool.shape[1] != 576:
        raise ValueError("q and kv_pool rows must be 576 wide")
    max_kv = page_table.shape[1]
    W = (N + 31) // 32
    if page_table.shape[0] != B or seq_lens.shape != (B,) or tree_mask.shape != (B, N, W):
        raise ValueError("shape mismatch")
    out = np.zeros((B, N, H, 512), dtype=np.uint16)
    lse = np.full((B, N, H), np.nan, dtype=np.float32)
    out64 = np.zeros((B, N, H, 512), dtype=np.float64) if want_f64 else None
    lse64 = np.full((B, N, H), np.nan, dtype=np.float64) if want_f64 else None
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    if threads <= 0:
        threads = os.cpu_count() or 1
    rc = lib.mtv_oracle_run(B, N, H, max_kv, kv_pool.shape[0], _ptr(q), _ptr(kv_pool),
                            _ptr(page_table), _ptr(seq_lens), _ptr(tree_mask), float(scale),
                            _ptr(rows_arr), 0 if rows_arr is None else len(rows_arr),
                            _ptr(out), _ptr(lse), _ptr(out64), _ptr(lse64), int(threads))
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")
    if want_f64:
        return out, lse, out64, lse64
    return out, lse


def run_workload(wl, **kw):
    """Convenience: run the oracle on an ``inputs.Workload`` (copied to host)."""
    return run(wl.np_q(), wl.np_kv(), wl.np_page_table(), wl.np_seq_lens(), wl.np_mask(),
               wl.scale, **kw)


def f64_to_bf16(x: float) -> int:
    return int(load().mtv_oracle_f64_to_bf16(float(x)))


def bf16_to_f64(bits: int) -> float:
    return float(load().mtv_oracle_bf16_to_f64(int(bits) & 0xFFFF))
