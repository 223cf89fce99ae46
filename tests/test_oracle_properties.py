"""Property tests of the fp64 oracle over random forests, drawn and shrunk by hypothesis
(CPU only). Each property follows from the recurrence of the Bole summary page, section 1
("Tree-Structured Closed Form"), H_i = diag(a_i) H_parent(i) + k_i v_i^T, o_i = H_i^T q_i,
which ties a node's output to its own root path and to nothing else:
  - the serial walk equals the dense closed form built from the transitive closure of the
    parent relation;
  - renumbering a tree in another topological order permutes its outputs and changes
    nothing else;
  - outputs are jointly linear in (H0, v);
  - a per-channel gate with all channels equal gives the scalar gate's outputs;
  - adding a leaf anywhere leaves every other node's output unchanged, bit for bit (the
    serial walk reads only a node's own path).
A tree is any parent array with parent[i] < i; nodes with parent -1 hang from the
verified context, so a tree may have several roots.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle import closed_form as cf
from tests.helpers import rel_err_rows

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None)


@st.composite
def forests(draw):
    """(parent, node_offsets, heads, d_k, d_v, vector_gate, seed)"""
    B = draw(st.integers(1, 3))
    sizes = [draw(st.integers(0, 10)) for _ in range(B)]
    parent = []
    for n in sizes:
        parent += [draw(st.integers(-1, i - 1)) for i in range(n)]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return (np.asarray(parent, np.int32), offs, draw(st.integers(1, 2)), draw(st.integers(1, 5)),
            draw(st.integers(1, 4)), draw(st.booleans()), draw(st.integers(0, 2 ** 31 - 1)))


def inputs(f):
    parent, offs, H, dk, dv, vec, seed = f
    rng = np.random.default_rng(seed)
    B, T = len(offs) - 1, len(parent)
    H0 = rng.standard_normal((B, H, dk, dv))
    q, k = rng.standard_normal((2, T, H, dk))
    v = rng.standard_normal((T, H, dv))
    gate = rng.uniform(0.05, 1.5, (T, H, dk) if vec else (T, H))
    return H0, q, k, v, gate, parent, offs, vec


def serial(H0, q, k, v, gate, parent, offs, vec):
    out, status = oracle.verify_serial(H0, q, k, v, gate, parent, offs, vec)
    assert (status == 0).all()
    return out


@SETTINGS
@given(forests())
def test_serial_walk_equals_the_closed_form(f):
    args = inputs(f)
    if len(args[5]) == 0:
        return
    assert rel_err_rows(serial(*args), cf.verify_closed_form(*args)) < 1e-10


@SETTINGS
@given(forests(), st.integers(0, 2 ** 31 - 1))
def test_topological_relabelling_permutes_the_outputs(f, seed):
    H0, q, k, v, gate, parent, offs, vec = inputs(f)
    base = serial(H0, q, k, v, gate, parent, offs, vec)
    rng = np.random.default_rng(seed)
    sel, p_new = [], []
    for b in range(len(offs) - 1):
        lo, hi = int(offs[b]), int(offs[b + 1])
        p0 = parent[lo:hi]
        order, ready = [], [i for i in range(hi - lo) if p0[i] < 0]
        while ready:  # any node whose parent is already placed may come next
            x = ready.pop(int(rng.integers(len(ready))))
            order.append(x)
            ready += [i for i in range(hi - lo) if p0[i] == x]
        new_of = {old: new for new, old in enumerate(order)}
        p_new += [-1 if p0[o] < 0 else new_of[int(p0[o])] for o in order]
        sel += [lo + o for o in order]
    sel = np.asarray(sel, np.int64)
    p_new = np.asarray(p_new, np.int32)
    out = serial(H0, q[sel], k[sel], v[sel], gate[sel], p_new, offs, vec)
    np.testing.assert_array_equal(out, base[sel])


@SETTINGS
@given(forests(), st.floats(-3, 3), st.floats(-3, 3))
def test_outputs_are_jointly_linear_in_the_state_and_values(f, alpha, beta):
    H0, q, k, v, gate, parent, offs, vec = inputs(f)
    if len(parent) == 0:
        return
    rng = np.random.default_rng(len(parent))
    H0b, vb = rng.standard_normal(H0.shape), rng.standard_normal(v.shape)
    o1 = serial(H0, q, k, v, gate, parent, offs, vec)
    o2 = serial(H0b, q, k, vb, gate, parent, offs, vec)
    o3 = serial(alpha * H0 + beta * H0b, q, k, alpha * v + beta * vb, gate, parent, offs, vec)
    ref = alpha * o1 + beta * o2
    scale = max(1.0, float(np.abs(o1).max()) * abs(alpha), float(np.abs(o2).max()) * abs(beta))
    assert float(np.abs(o3 - ref).max()) <= 1e-11 * scale


@SETTINGS
@given(forests())
def test_equal_channels_give_the_scalar_gate(f):
    parent, offs, H, dk, dv, _, seed = f
    H0, q, k, v, gate, parent, offs, _ = inputs((parent, offs, H, dk, dv, False, seed))
    o_s = serial(H0, q, k, v, gate, parent, offs, False)
    o_v = serial(H0, q, k, v, np.repeat(gate[:, :, None], dk, axis=2), parent, offs, True)
    np.testing.assert_allclose(o_v, o_s, rtol=1e-13, atol=1e-13)


@SETTINGS
@given(forests(), st.data())
def test_a_new_leaf_changes_no_other_output(f, data):
    H0, q, k, v, gate, parent, offs, vec = inputs(f)
    base = serial(H0, q, k, v, gate, parent, offs, vec)
    b = data.draw(st.integers(0, len(offs) - 2))
    lo, hi = int(offs[b]), int(offs[b + 1])
    if hi - lo >= 64:
        return
    # the new node is appended to tree b, under any of its nodes or the context
    p_leaf = data.draw(st.integers(-1, hi - lo - 1))
    rng = np.random.default_rng(hi)
    ins = lambda a, x: np.concatenate([a[:hi], x[None], a[hi:]])
    parent2 = ins(parent, np.int32(p_leaf))
    offs2 = offs.copy()
    offs2[b + 1:] += 1
    q2, k2 = ins(q, rng.standard_normal(q.shape[1:])), ins(k, rng.standard_normal(k.shape[1:]))
    v2 = ins(v, rng.standard_normal(v.shape[1:]))
    g2 = ins(gate, rng.uniform(0.05, 1.5, gate.shape[1:]))
    out = serial(H0, q2, k2, v2, g2, parent2, offs2, vec)
    keep = np.r_[0:hi, hi + 1:len(parent2)]
    np.testing.assert_array_equal(out[keep], base)
