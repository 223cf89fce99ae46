"""fp64 CPU oracle for Bole tree verification and accepted-path commit.

TEST INFRASTRUCTURE ONLY. The test-suite, the smoke entry and the benchmark's CPU-baseline
leg are its only callers. The GPU library never imports, loads or calls anything here.
The two share no code: what they have in common is the seeded inputs from ``workloads``.

Every input is widened to float64 from the exact values the GPU reads: bf16 and fp32
both widen exactly. The arithmetic is in ``bole_oracle.c`` (the naive serial walk per
node, one full state per node) and in ``closed_form.py`` (the fp64 closed form, test-only).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p


def configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    lib.oracle_topology.argtypes = [_i64, _i64, _p, _p, _p, _p, _p]
    lib.oracle_cumlog.argtypes = [_i64, _i64, _i64, _i64, _int, _p, _p, _p, _p]
    lib.oracle_verify_serial.argtypes = [_i64, _i64, _i64, _i64, _i64, _int,
                                         _p, _p, _p, _p, _p, _p, _p, _p, _p]
    lib.oracle_commit_serial.argtypes = [_i64, _i64, _i64, _i64, _i64, _int, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _i64, _p, _p]
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = _int
    lib.oracle_set_threads.argtypes = [_int]
    lib.oracle_set_threads.restype = None
    for f in (lib.oracle_topology, lib.oracle_cumlog, lib.oracle_verify_serial,
              lib.oracle_commit_serial):
        f.restype = _int
    return lib


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("BOLE_ORACLE_LIB", _build.LIB)  # another build, e.g. sanitized
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _lib = configure(ctypes.CDLL(path))
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on (timing only: every result is
    computed per (sequence, head) and does not depend on the thread count)."""
    _load().oracle_set_threads(int(n))


def f64(x) -> np.ndarray:
    """Exact widening of a torch tensor (any float dtype) or array to contiguous float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def topology(parent, node_offsets, total_nodes=None):
    """Depth (int32[T]), ancestor-or-self mask (uint64[T]) and per-tree status (int32[B]).

    Nodes of a bad-size tree keep the sentinel -1 / 0xFF..FF (never written)."""
    parent, offs = i32(parent), i32(node_offsets)
    T = int(parent.shape[0]) if total_nodes is None else int(total_nodes)
    B = int(offs.shape[0]) - 1
    depth = np.full(max(T, 1), -1, np.int32)
    mask = np.full(max(T, 1), np.iinfo(np.uint64).max, np.uint64)
    status = np.zeros(max(B, 1), np.int32)
    _load().oracle_topology(B, T, _ptr(offs), _ptr(parent), _ptr(depth), _ptr(mask),
                            _ptr(status))
    return depth[:T], mask[:T], status[:B]


def cumlog(gate, parent, node_offsets, heads, d_k, vector_gate):
    """Cumulative log-decay per node, fp64: [T, H] or [T, H, d_k]."""
    gate, parent, offs = f64(gate), i32(parent), i32(node_offsets)
    T = int(parent.shape[0])
    B = int(offs.shape[0]) - 1
    shape = (T, heads, d_k) if vector_gate else (T, heads)
    out = np.full(shape, np.nan)
    _load().oracle_cumlog(B, heads, d_k, T, int(bool(vector_gate)), _ptr(gate), _ptr(parent),
                          _ptr(offs), _ptr(out))
    return out


def verify_serial(H0, q, k, v, gate, parent, node_offsets, vector_gate):
    """Naive serial verify in fp64. Returns (out [T, H, d_v] float64, status int32[B])."""
    H0, q, k, v, gate = f64(H0), f64(q), f64(k), f64(v), f64(gate)
    parent, offs = i32(parent), i32(node_offsets)
    B, H, d_k, d_v = H0.shape
    T = int(q.shape[0])
    out = np.full((T, H, d_v), np.nan)
    status = np.zeros(max(B, 1), np.int32)
    _load().oracle_verify_serial(B, H, d_k, d_v, T, int(bool(vector_gate)), _ptr(H0), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(gate), _ptr(parent), _ptr(offs),
                                 _ptr(out), _ptr(status))
    return out, status[:B]


def commit_serial(H0, k, v, gate, parent, node_offsets, accepted_idx, accepted_len,
                  vector_gate):
    """Serial commit in fp64. Returns (new H0 float64, path_nodes int32[B, max_path],
    status int32[B]). The input H0 is not modified."""
    H = f64(H0).copy()
    k, v, gate = f64(k), f64(v), f64(gate)
    parent, offs = i32(parent), i32(node_offsets)
    acc_idx, acc_len = i32(accepted_idx), i32(accepted_len)
    B, Hh, d_k, d_v = H.shape
    T = int(k.shape[0])
    max_path = int(acc_idx.shape[1]) if acc_idx.ndim == 2 else 0
    path_nodes = np.full((max(B, 1), max(max_path, 1)), -7, np.int32)
    status = np.zeros(max(B, 1), np.int32)
    acc_idx = np.ascontiguousarray(acc_idx.reshape(B, max_path))
    _load().oracle_commit_serial(B, Hh, d_k, d_v, T, int(bool(vector_gate)), _ptr(H), _ptr(k),
                                 _ptr(v), _ptr(gate), _ptr(parent), _ptr(offs), _ptr(acc_idx),
                                 _ptr(acc_len), max_path, _ptr(path_nodes), _ptr(status))
    return H, path_nodes[:B, :max_path], status[:B]
