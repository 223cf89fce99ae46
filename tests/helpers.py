"""Small shared helpers for the test-suite (no verify/commit arithmetic)."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hand_case_arrays(case):
    """fp64 arrays in the library layouts (one sequence, one head) for a golden case."""
    n = len(case["parent"])
    d_k, d_v = case["d_k"], case["d_v"]
    H0 = np.asarray(case["H0"], np.float64).reshape(1, 1, d_k, d_v)
    q = np.asarray(case["q"], np.float64).reshape(n, 1, d_k)
    k = np.asarray(case["k"], np.float64).reshape(n, 1, d_k)
    v = np.asarray(case["v"], np.float64).reshape(n, 1, d_v)
    g = np.asarray(case["gate"], np.float64)
    gate = g.reshape(n, 1, d_k) if case["vector_gate"] else g.reshape(n, 1)
    parent = np.asarray(case["parent"], np.int32)
    offs = np.array([0, n], np.int32)
    return H0, q, k, v, gate, parent, offs


def rel_err_rows(got, ref):
    """Worst per-row normwise relative error: max_c |got-ref| / max_c |ref| per row."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    den = np.abs(r).max(axis=1)
    num = np.abs(g - r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def rel_err_states(got, ref):
    """Worst per-(sequence, head) normwise relative error of d_k x d_v states."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    g = got.reshape(-1, got.shape[-2] * got.shape[-1])
    r = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def layer_f64(layer):
    """fp64 numpy copies of a workload layer (exact widening)."""
    f = lambda t: t.to(torch.float64).numpy()
    return f(layer.H0), f(layer.q), f(layer.k), f(layer.v), f(layer.gate)
