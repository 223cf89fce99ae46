"""Pins of the fp64 oracle against what the pages and plain mathematics fix (CPU only).

The oracle (oracle/bole_oracle.c) walks every root-to-node path serially. It is checked
here against facts that do not come from it:
  - hand-derived values (tests/golden/hand_trees.json), for the recurrence of the Bole
    summary page, section 1 "Tree-Structured Closed Form", and the path restore of
    section 2 "Token-Level Factor Encoding";
  - chain == sequential scan, through the decayed-attention dual form built from
    cumulative sums and a lower-triangular mask, and the plain causal linear-attention
    identity O = tril(QK^T) V when a == 1 and H0 == 0;
  - single node == one recurrence step;
  - brute force over every parent array with N <= 6: serial walk == dense closed form
    (built from the transitive closure of the parent relation);
  - exact rational arithmetic (fractions.Fraction) on tiny dyadic inputs;
  - commit == restored closed form, and verify -> commit -> verify resumes exactly;
  - invariants: equal-channel vector gate == scalar gate, joint linearity in (H0, v),
    relabelling invariance, identical siblings, extreme gates stay finite.
Each check is a function, so that the mutation test at the end can run all of them
against deliberately broken copies of the oracle and see that each mistake is caught.
"""
import ctypes
import itertools
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import closed_form as cf
import workloads as W
from tests.helpers import hand_case_arrays, load_golden, rel_err_rows, rel_err_states, layer_f64

TOL64 = 1e-12


# ----------------------------------------------------------------------------- checks

def check_golden():
    g = load_golden("hand_trees.json")
    for case in g["cases"]:
        H0, q, k, v, gate, parent, offs = hand_case_arrays(case)
        vec = case["vector_gate"]
        out, st = oracle.verify_serial(H0, q, k, v, gate, parent, offs, vec)
        assert st.tolist() == [0]
        np.testing.assert_array_equal(out[:, 0, :], np.asarray(case["out"]), err_msg=case["name"])
        depth, mask, st = oracle.topology(parent, offs)
        assert depth.tolist() == case["depth"] and mask.tolist() == case["mask"], case["name"]
        for cm in case["commits"]:
            mp = 3
            idx = np.full((1, mp), -1, np.int32)
            idx[0, :len(cm["path"])] = cm["path"]
            Hn, pn, st = oracle.commit_serial(H0, k, v, gate, parent, offs, idx,
                                              np.array([len(cm["path"])], np.int32), vec)
            assert st.tolist() == [cm["status"]], (case["name"], cm["path"])
            np.testing.assert_array_equal(Hn[0, 0], np.asarray(cm["H0"], np.float64),
                                          err_msg=f"{case['name']} {cm['path']}")
            want = [p for p in cm["path"]] if cm["status"] == 0 else []
            assert pn[0].tolist() == want + [-1] * (mp - len(want))


def check_status_cases():
    g = load_golden("hand_trees.json")
    for sc in g["status_cases"]:
        sizes = sc["sizes"]
        if "parent" in sc:
            parent = np.asarray(sc["parent"], np.int32)
        else:
            parent = np.full(sum(sizes), -1, np.int32)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        _, _, st = oracle.topology(parent, offs)
        assert st.tolist() == sc["status"], sc["name"]
        T, B = int(offs[-1]), len(sizes)
        H0 = np.ones((B, 1, 2, 2))
        q = np.ones((T, 1, 2))
        gate = np.full((T, 1), 0.5)
        out, st2 = oracle.verify_serial(H0, q, q, q, gate, parent, offs, False)
        assert st2.tolist() == sc["status"], sc["name"]
        for b in range(B):
            rows = out[offs[b]:offs[b + 1]]
            if sc["status"][b] == 2:
                assert np.isnan(rows).all()
            elif sc["status"][b] == 0:
                assert np.isfinite(rows).all()


def _dual_form_chain(H0, Q, K, V, a):
    """Sequential scan of a chain as the decayed-attention dual form (one head):
    O = diag(D) Q H0 + (tril(Q K^T) * Gamma) V, D_t = prod_{s<=t} a_s,
    Gamma_ts = prod_{s<u<=t} a_u. Scalar a [n] or per-channel a [n, d_k]."""
    n = Q.shape[0]
    if a.ndim == 1:
        cs = np.cumsum(np.log(a))
        Gam = np.exp(cs[:, None] - cs[None, :])
        return np.exp(cs)[:, None] * (Q @ H0) + (np.tril(Q @ K.T) * np.tril(Gam)) @ V
    cs = np.cumsum(np.log(a), axis=0)                        # [n, d_k]
    S = np.einsum("tc,sc,tsc->ts", Q, K, np.exp(cs[:, None, :] - cs[None, :, :]))
    return (np.exp(cs) * Q) @ H0 + np.tril(S) @ V


def check_chain_scan(seed=0):
    rng = np.random.default_rng(seed)
    for vec in (False, True):
        for n in (1, 2, 7, 33, 64):
            d_k, d_v = 5, 3
            H0 = rng.standard_normal((1, 1, d_k, d_v))
            q, k = rng.standard_normal((2, n, 1, d_k))
            v = rng.standard_normal((n, 1, d_v))
            gate = np.exp(-np.logaddexp(0, rng.standard_normal((n, 1, d_k) if vec else (n, 1))))
            parent = np.arange(-1, n - 1, dtype=np.int32)
            offs = np.array([0, n], np.int32)
            out, _ = oracle.verify_serial(H0, q, k, v, gate, parent, offs, vec)
            ref = _dual_form_chain(H0[0, 0], q[:, 0], k[:, 0], v[:, 0], gate[:, 0])
            assert rel_err_rows(out[:, 0], ref) < TOL64, (vec, n)
    # causal linear attention: a == 1, H0 == 0  ->  O = tril(Q K^T) V
    n, d_k, d_v = 40, 6, 4
    q, k = rng.standard_normal((2, n, 1, d_k))
    v = rng.standard_normal((n, 1, d_v))
    out, _ = oracle.verify_serial(np.zeros((1, 1, d_k, d_v)), q, k, v, np.ones((n, 1)),
                                  np.arange(-1, n - 1, dtype=np.int32),
                                  np.array([0, n], np.int32), False)
    ref = np.tril(q[:, 0] @ k[:, 0].T) @ v[:, 0]
    assert rel_err_rows(out[:, 0], ref) < TOL64


def check_single_node(seed=1):
    rng = np.random.default_rng(seed)
    for vec in (False, True):
        B, Hn, d_k, d_v = 3, 2, 4, 5
        H0 = rng.standard_normal((B, Hn, d_k, d_v))
        q, k = rng.standard_normal((2, B, Hn, d_k))
        v = rng.standard_normal((B, Hn, d_v))
        gate = rng.uniform(0.1, 1.0, (B, Hn, d_k) if vec else (B, Hn))
        out, _ = oracle.verify_serial(H0, q, k, v, gate, np.full(B, -1, np.int32),
                                      np.arange(B + 1, dtype=np.int32), vec)
        for b in range(B):
            for h in range(Hn):
                g = gate[b, h] if vec else gate[b, h] * np.ones(d_k)
                ref = H0[b, h].T @ (g * q[b, h]) + (q[b, h] @ k[b, h]) * v[b, h]
                assert np.max(np.abs(out[b, h] - ref)) < 1e-13


def all_parent_arrays(n):
    return itertools.product(*[range(-1, i) for i in range(n)])


def check_bruteforce_closed_form(seed=2, max_n=6):
    rng = np.random.default_rng(seed)
    for vec in (False, True):
        parents = [np.array(p, np.int32) for n in range(1, max_n + 1) for p in all_parent_arrays(n)]
        sizes = [len(p) for p in parents]
        parent = np.concatenate(parents)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        B, T, Hn, d_k, d_v = len(parents), int(offs[-1]), 2, 3, 2
        H0 = rng.standard_normal((B, Hn, d_k, d_v))
        q, k = rng.standard_normal((2, T, Hn, d_k))
        v = rng.standard_normal((T, Hn, d_v))
        gate = rng.uniform(0.05, 1.0, (T, Hn, d_k) if vec else (T, Hn))
        out, st = oracle.verify_serial(H0, q, k, v, gate, parent, offs, vec)
        assert (st == 0).all()
        ref = cf.verify_closed_form(H0, q, k, v, gate, parent, offs, vec)
        assert rel_err_rows(out, ref) < TOL64, vec


def _rational_states(parent, H0, k, v, gate, vec):
    """H_i for every node by exact rational recursion over parents (memoised)."""
    n = len(parent)
    d_k, d_v = len(H0), len(H0[0])
    states = []
    for i in range(n):
        base = H0 if parent[i] < 0 else states[parent[i]]
        Hi = [[(gate[i][r] if vec else gate[i]) * base[r][c] + k[i][r] * v[i][c]
               for c in range(d_v)] for r in range(d_k)]
        states.append(Hi)
    return states


def check_exact_rational(seed=3):
    rng = np.random.default_rng(seed)
    for vec in (False, True):
        for _ in range(6):
            n, d_k, d_v = int(rng.integers(1, 9)), 3, 2
            parent = W.random_tree(rng, n, "random")
            dy = lambda *s: rng.integers(-8, 9, size=s) / 4.0        # dyadic values
            H0, q, k, v = dy(d_k, d_v), dy(n, d_k), dy(n, d_k), dy(n, d_v)
            gate = rng.choice([0.25, 0.5, 0.75, 1.0], size=(n, d_k) if vec else n)
            F = lambda x: [[Fraction(float(y)) for y in row] for row in np.atleast_2d(x)]
            gateF = F(gate) if vec else [Fraction(float(y)) for y in gate]
            st = _rational_states(parent, F(H0), F(k), F(v), gateF, vec)
            qF = F(q)
            exact = np.array([[float(sum(st[i][r][c] * qF[i][r] for r in range(d_k)))
                               for c in range(d_v)] for i in range(n)])
            out, _ = oracle.verify_serial(H0[None, None], q[:, None], k[:, None], v[:, None],
                                          gate[:, None], parent, np.array([0, n], np.int32), vec)
            assert rel_err_rows(out[:, 0], exact) < 1e-14


def check_commit_restore(seed=4):
    for vec in (False, True):
        wl = W.make_random(seed, batch=12, heads=3, d_k=8, d_v=5, kind="deep", vector_gate=vec,
                           factor_dtype=torch.float32, max_path=64)
        H0, q, k, v, gate = layer_f64(wl.layers[0])
        Hn, pn, st = oracle.commit_serial(H0, k, v, gate, wl.parent, wl.node_offsets,
                                          wl.accepted_idx, wl.accepted_len, vec)
        assert (st == 0).all()
        ref = cf.restore_closed_form(H0, k, v, gate, wl.node_offsets, wl.accepted_idx,
                                     wl.accepted_len, vec)
        assert rel_err_states(Hn, ref) < TOL64
        for b in range(wl.batch):
            L = wl.accepted_len[b]
            assert pn[b, :L].tolist() == (wl.node_offsets[b] + wl.accepted_idx[b, :L]).tolist()
            assert (pn[b, L:] == -1).all()


def check_resume(seed=5):
    """verify(tree t) on the state committed after path p == verify(p, then t hung
    below p's last node) on the old state."""
    rng = np.random.default_rng(seed)
    for vec in (False, True):
        Hn, d_k, d_v = 2, 4, 3
        L, m = 3, 6
        p_par = np.arange(-1, L - 1, dtype=np.int32)               # accepted chain
        t_par = W.random_tree(rng, m, "random")                    # next tree
        joint = np.concatenate([p_par, np.where(t_par < 0, L - 1, t_par + L)]).astype(np.int32)
        n = L + m
        H0 = rng.standard_normal((1, Hn, d_k, d_v))
        q, k = rng.standard_normal((2, n, Hn, d_k))
        v = rng.standard_normal((n, Hn, d_v))
        gate = rng.uniform(0.2, 1.0, (n, Hn, d_k) if vec else (n, Hn))
        out_joint, _ = oracle.verify_serial(H0, q, k, v, gate, joint, np.array([0, n], np.int32), vec)
        H1, _, st = oracle.commit_serial(H0, k[:L], v[:L], gate[:L], p_par, np.array([0, L], np.int32),
                                         np.arange(L, dtype=np.int32)[None], np.array([L], np.int32), vec)
        out_next, _ = oracle.verify_serial(H1, q[L:], k[L:], v[L:], gate[L:], t_par,
                                           np.array([0, m], np.int32), vec)
        assert rel_err_rows(out_next, out_joint[L:]) < TOL64


def check_invariants(seed=6):
    rng = np.random.default_rng(seed)
    wl = W.make_random(seed, batch=6, heads=2, d_k=6, d_v=4, kind="random",
                       factor_dtype=torch.float32)
    H0, q, k, v, a = layer_f64(wl.layers[0])
    par, offs = wl.parent, wl.node_offsets
    base, _ = oracle.verify_serial(H0, q, k, v, a, par, offs, False)
    # equal channels: vector gate == scalar gate
    g = np.repeat(a[:, :, None], 6, axis=2)
    vec_out, _ = oracle.verify_serial(H0, q, k, v, g, par, offs, True)
    assert rel_err_rows(vec_out, base) < TOL64
    # joint linearity in (H0, v)
    H0b, vb = rng.standard_normal(H0.shape), rng.standard_normal(v.shape)
    o2, _ = oracle.verify_serial(H0b, q, k, vb, a, par, offs, False)
    o3, _ = oracle.verify_serial(2.0 * H0 - 3.0 * H0b, q, k, 2.0 * v - 3.0 * vb, a, par, offs, False)
    assert rel_err_rows(o3, 2.0 * base - 3.0 * o2) < 1e-10
    # a == 1, H0 == 0 on a general tree: O = ((Q K^T) * M) V with the ancestor mask
    depth, mask, _ = oracle.topology(par, offs)
    o4, _ = oracle.verify_serial(np.zeros_like(H0), q, k, v, np.ones_like(a), par, offs, False)
    for b in range(wl.batch):
        lo, hi = offs[b], offs[b + 1]
        n = hi - lo
        M = np.array([[(int(mask[lo + i]) >> j) & 1 for j in range(n)] for i in range(n)], float)
        assert (M.sum(axis=1) == depth[lo:hi]).all()
        for h in range(2):
            ref = ((q[lo:hi, h] @ k[lo:hi, h].T) * M) @ v[lo:hi, h]
            assert rel_err_rows(o4[lo:hi, h], ref) < TOL64
    # relabelling invariance under a random topological renumbering (tree 0)
    lo, hi = offs[0], offs[1]
    n = hi - lo
    p0 = par[lo:hi]
    order, ready = [], [i for i in range(n) if p0[i] < 0]
    while ready:
        x = ready.pop(int(rng.integers(len(ready))))
        order.append(x)
        ready += [i for i in range(n) if p0[i] == x]
    new_of = {old: new for new, old in enumerate(order)}
    p_new = np.array([-1 if p0[o] < 0 else new_of[p0[o]] for o in order], np.int32)
    assert all(p_new[i] < i for i in range(n))
    sel = lo + np.array(order)
    o5, _ = oracle.verify_serial(H0[:1], q[sel], k[sel], v[sel], a[sel], p_new,
                                 np.array([0, n], np.int32), False)
    assert rel_err_rows(o5, base[sel]) < TOL64
    # identical siblings give identical outputs
    sib = np.array([-1, 0, 0], np.int32)
    qs, ks = rng.standard_normal((2, 3, 1, 4))
    vs = rng.standard_normal((3, 1, 3))
    gs = rng.uniform(0.1, 1, (3, 1))
    for arr in (qs, ks, vs, gs):
        arr[2] = arr[1]
    o6, _ = oracle.verify_serial(rng.standard_normal((1, 1, 4, 3)), qs, ks, vs, gs, sib,
                                 np.array([0, 3], np.int32), False)
    np.testing.assert_array_equal(o6[1], o6[2])


def check_extreme_gates(seed=7):
    for vec in (False, True):
        wl = W.make_random(seed, batch=4, heads=2, d_k=8, d_v=4, sizes=[64, 40, 10, 64],
                           kind="deep", vector_gate=vec, factor_dtype=torch.float32,
                           gate_shift=6.0)
        H0, q, k, v, gate = layer_f64(wl.layers[0])
        out, _ = oracle.verify_serial(H0, q, k, v, gate, wl.parent, wl.node_offsets, vec)
        assert np.isfinite(out).all()
        ref = cf.verify_closed_form(H0, q, k, v, gate, wl.parent, wl.node_offsets, vec)
        assert rel_err_rows(out, ref) < 1e-9


def check_cumlog(seed=8):
    wl = W.make_random(seed, batch=5, heads=3, d_k=4, d_v=2, kind="random", vector_gate=True,
                       factor_dtype=torch.float32)
    gate = wl.layers[0].gate.double().numpy()
    L = oracle.cumlog(gate, wl.parent, wl.node_offsets, 3, 4, True)
    for b in range(wl.batch):
        lo, hi = wl.node_offsets[b], wl.node_offsets[b + 1]
        M = cf.ancestor_matrix(wl.parent[lo:hi]).astype(float)
        ref = np.einsum("ij,jhc->ihc", M, np.log(gate[lo:hi]))
        assert np.max(np.abs(L[lo:hi] - ref)) < 1e-12


ALL_CHECKS = [check_golden, check_status_cases, check_chain_scan, check_single_node,
              check_bruteforce_closed_form, check_exact_rational, check_commit_restore,
              check_resume, check_invariants, check_extreme_gates, check_cumlog]


# ----------------------------------------------------------------------------- tests

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


def test_config1_topology_by_hand():
    wl = W.make_config(1)
    depth, mask, st = oracle.topology(wl.parent, wl.node_offsets)
    assert depth.tolist() == [1, 2, 2, 3, 3, 3, 3]
    assert mask.tolist() == [0x1, 0x3, 0x5, 0xB, 0x13, 0x25, 0x45]
    chain = np.arange(-1, 63, dtype=np.int32)
    d, m, _ = oracle.topology(chain, np.array([0, 64], np.int32))
    assert d.tolist() == list(range(1, 65))
    assert [int(x) for x in m] == [(1 << (i + 1)) - 1 for i in range(64)]


def test_topology_matches_closure():
    wl = W.make_random(11, batch=40, heads=1, d_k=2, d_v=2, kind="bestfirst")
    depth, mask, st = oracle.topology(wl.parent, wl.node_offsets)
    assert (st == 0).all()
    for b in range(wl.batch):
        lo, hi = wl.node_offsets[b], wl.node_offsets[b + 1]
        M = cf.ancestor_matrix(wl.parent[lo:hi])
        for i in range(hi - lo):
            assert int(mask[lo + i]) == sum(1 << j for j in np.nonzero(M[i])[0])
            assert depth[lo + i] == M[i].sum()


# --------------------------------------------------------------- mutation self-test

MUTANTS = {
    "output_before_own_update": ("for (int t = 0; t < d; ++t)\n                    or_step",
                                 "for (int t = 0; t < d - 1; ++t)\n                    or_step"),
    "gate_on_update_too": ("H[r * d_v + c] = s * H[r * d_v + c] + kj[r] * vj[c];",
                           "H[r * d_v + c] = s * (H[r * d_v + c] + kj[r] * vj[c]);"),
    "leaf_first_order": ("path[m] = rev[d - 1 - m];", "path[m] = rev[m];"),
    "wrong_query_index": ("acc += H[r * d_v + c] * qi[r];",
                          "acc += H[r * d_v + c] * qi[(r + 1) % d_k];"),
    "wrong_gate_channel": ("gate[(gj * heads + h) * d_k + r]",
                           "gate[(gj * heads + h) * d_k + (d_k - 1 - r)]"),
    "commit_drops_last": ("for (int32_t m = 0; m < accepted_len[b]; ++m) {\n                int64_t gj",
                          "for (int32_t m = 0; m + 1 < accepted_len[b]; ++m) {\n                int64_t gj"),
    "mask_off_by_one": ("m |= (uint64_t)1 << path[t];", "m |= (uint64_t)1 << (path[t] + 1);"),
    "parent_check_allows_minus_two": ("if (p < -1 || p >= i) return OR_BAD_PARENT;",
                                      "if (p < -2 || p >= i) return OR_BAD_PARENT;"),
    "cumlog_skips_root": ("for (int t = 0; t < d; ++t)\n                        acc += log",
                          "for (int t = 1; t < d; ++t)\n                        acc += log"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch, tmp_path):
    """Plants one plausible mistake in a copy of the oracle (CPU only) and requires at
    least one pin to fail on it."""
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "bole_oracle.c")).read()
    assert src.count(old) == 1, name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", str(path), "-o",
                    str(lib), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.configure(ctypes.CDLL(str(lib))))
    caught = []
    for check in ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
