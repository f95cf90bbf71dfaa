"""Plain CPU fp64 oracle for tree-masked MLA verify attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and
its binding) never imports this package, and this package never imports the
product.  The arithmetic lives in ``verify_attn_oracle.c`` (plain C, fp64);
this module only builds it with gcc and marshals numpy arrays.

What the oracle computes is stated in the header comment of the C file:
masked softmax attention written out from its definition, per row, with no
splitting and no online softmax (the operation the pages call MLA-absorb
attention with a custom tree mask).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "verify_attn_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

D_QK = 576
D_V = 512


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math: sums stay in order)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        lib = ctypes.CDLL(str(_LIB_PATH))
        P = ctypes.c_void_p
        lib.oracle_verify_attn.restype = ctypes.c_int
        lib.oracle_verify_attn.argtypes = [
            ctypes.c_int32, ctypes.c_int32, P, P, P, P, ctypes.c_int64, ctypes.c_int32,
            P, P, P, ctypes.c_double, P, P, P, P, ctypes.c_int64, ctypes.c_int32,
        ]
        lib.oracle_tree_visibility.restype = ctypes.c_int
        lib.oracle_tree_visibility.argtypes = [P, ctypes.c_int32, P]
        lib.oracle_attend.restype = ctypes.c_int
        lib.oracle_attend.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int64,
                                      ctypes.c_double, P, P, P]
        lib.oracle_lse_merge.restype = ctypes.c_int
        lib.oracle_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P]
        assert lib.oracle_d_qk() == D_QK and lib.oracle_d_v() == D_V
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def tree_visibility(parent) -> np.ndarray:
    """vis[i, j] is True when draft node j is node i or one of its ancestors."""
    parent = _c(parent, np.int32)
    T = parent.shape[0]
    vis = np.zeros((T, T), dtype=np.uint8)
    rc = _load().oracle_tree_visibility(_ptr(parent), T, _ptr(vis))
    if rc != 0:
        raise OracleError(f"oracle_tree_visibility failed ({rc})")
    return vis.astype(bool)


def attend(q, kv_pool, slots, sm_scale):
    """Unmasked softmax attention of one fp64 query row over explicit pool slots.

    Returns (o [512] fp64, lse float, p [n] fp64)."""
    q = _c(q, np.float64)
    kv_pool = _c(kv_pool, np.uint16)
    slots = _c(slots, np.int32)
    n = slots.shape[0]
    o = np.zeros(D_V, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    p = np.zeros(max(n, 1), dtype=np.float64)
    rc = _load().oracle_attend(_ptr(q), _ptr(kv_pool), kv_pool.shape[0], kv_pool.shape[1],
                               _ptr(slots), n, float(sm_scale), _ptr(o), _ptr(lse), _ptr(p))
    if rc != 0:
        raise OracleError(f"oracle_attend failed ({rc})")
    return o, float(lse[0]), p[:n]


def lse_merge(o_parts, lse_parts):
    """Merge per-part (o_j, lse_j) into the result over the union of the parts."""
    o_parts = _c(o_parts, np.float64)
    lse_parts = _c(lse_parts, np.float64)
    S, d = o_parts.shape
    o = np.zeros(d, dtype=np.float64)
    lse = np.zeros(1, dtype=np.float64)
    rc = _load().oracle_lse_merge(S, d, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse))
    if rc != 0:
        raise OracleError(f"oracle_lse_merge failed ({rc})")
    return o, float(lse[0])


def verify_attn(num_heads, num_tree, prefix_len, q, kv_pool, slot_table, slot_indptr, parent,
                sm_scale, rows=None, return_probs=False, num_threads=0):
    """Tree-masked verify attention in fp64.

    q: uint16 bf16 bits [sum T, H, 576]; kv_pool: uint16 [num_slots, stride>=576];
    slot_table int32 (concatenated per request, prefix then draft slots);
    slot_indptr int32 [B+1]; parent int32 [sum T] (request-local).
    rows: optional iterable of flat row indices ((tree index) * H + head) to compute;
    other rows are returned as NaN.
    Returns out fp64 [sum T, H, 512], lse fp64 [sum T, H] (+ probs [rows, max n]).
    """
    num_tree = _c(num_tree, np.int32)
    prefix_len = _c(prefix_len, np.int32)
    q = _c(q, np.uint16)
    kv_pool = _c(kv_pool, np.uint16)
    slot_table = _c(slot_table, np.int32)
    slot_indptr = _c(slot_indptr, np.int32)
    parent = _c(parent, np.int32)
    B = num_tree.shape[0]
    total_tree = int(num_tree.sum())
    H = int(num_heads)
    assert q.shape == (total_tree, H, D_QK), q.shape
    out = np.full((total_tree, H, D_V), np.nan, dtype=np.float64)
    lse = np.full((total_tree, H), np.nan, dtype=np.float64)
    sel = None
    if rows is not None:
        sel = np.zeros(total_tree * H, dtype=np.uint8)
        sel[np.asarray(list(rows), dtype=np.int64)] = 1
    probs = None
    stride = 0
    if return_probs:
        stride = int((prefix_len + num_tree).max())
        probs = np.zeros((total_tree * H, stride), dtype=np.float64)
    rc = _load().oracle_verify_attn(
        B, H, _ptr(num_tree), _ptr(prefix_len), _ptr(q), _ptr(kv_pool), kv_pool.shape[0],
        kv_pool.shape[1], _ptr(slot_table), _ptr(slot_indptr), _ptr(parent), float(sm_scale),
        _ptr(out), _ptr(lse), _ptr(sel), _ptr(probs), stride, int(num_threads))
    if rc != 0:
        raise OracleError(f"oracle_verify_attn failed ({rc})")
    if return_probs:
        return out, lse, probs
    return out, lse


def verify_attn_workload(wl, **kw):
    """Convenience: run the oracle on a workload object from the seeded input module."""
    return verify_attn(wl.num_heads, wl.num_tree, wl.prefix_len, wl.q, wl.kv_pool, wl.slot_table,
                       wl.slot_indptr, wl.parent, wl.sm_scale, **kw)
