"""GPU parity on workloads drawn by hypothesis: the batch, head count, tree sizes and kinds,
widths, gate kind, factor dtype, decay strength and gate range are all drawn
(derandomised, so every run draws the same cases), and each workload must meet the
oracle's bars through the C ABI: statuses, path gathers and topology bit-exact, outputs and
committed states within 2e-3 (bf16 factors) or 1e-5 (fp32), normwise per row and per
(sequence, head)."""
import os

import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

# BOLE_DRAWS=n: n times as many cases, drawn afresh on each run (a wider search than the
# fixed cases the suite runs by default)
_SCALE = int(os.environ.get("BOLE_DRAWS", "0"))


def drawn(n):
    return settings(max_examples=n * max(1, _SCALE), deadline=None, derandomize=_SCALE == 0,
                    database=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])

import workloads as W
from tests.test_gpu_parity import check_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bole():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_speculative_decoding_02_amd import bole as b
    return b


@drawn(30)
@given(st.data())
def test_drawn_workloads_meet_the_oracle_bars(bole, data):
    B = data.draw(st.integers(1, 6), label="batch")
    H = data.draw(st.integers(1, 4), label="heads")
    vec = data.draw(st.booleans(), label="vector_gate")
    dk = data.draw(st.sampled_from([64, 128]), label="d_k")
    dv = data.draw(st.sampled_from([32, 64, 128]), label="d_v")
    kind = data.draw(st.sampled_from(["random", "chain", "star", "deep", "bestfirst"]), label="kind")
    sizes = data.draw(st.lists(st.integers(0, 64), min_size=B, max_size=B), label="sizes")
    dtype = data.draw(st.sampled_from([torch.bfloat16, torch.float32]), label="dtype")
    shift = data.draw(st.sampled_from([0.0, 0.0, 3.0]), label="gate_shift")
    # gates up to about 2.5 (state growing along a path), or all exactly 1
    scale = data.draw(st.sampled_from([1.0, 1.0, 2.5]), label="gate_scale")
    value = data.draw(st.sampled_from([None, None, None, 1.0]), label="gate_value")
    seed = data.draw(st.integers(0, 10 ** 6), label="seed")
    print(f"[case] drawn B={B} H={H} vec={vec} dk={dk} dv={dv} kind={kind} sizes={sizes} "
          f"dtype={dtype} shift={shift} scale={scale} value={value} seed={seed}", flush=True)
    wl = W.make_random(seed, batch=B, heads=H, d_k=dk, d_v=dv, sizes=sizes, kind=kind,
                       vector_gate=vec, factor_dtype=dtype, max_path=64, gate_shift=shift,
                       gate_scale=scale, gate_value=value)
    # the caller's 32-node budget (its own launch shapes) when every tree fits it
    le32 = max(sizes) <= 32 and data.draw(st.booleans(), label="trees_le_32")
    check_workload(bole, wl, paths=("auto",), trees_le_32=le32)


@drawn(25)
@given(st.data())
def test_drawn_lazy_steps_match_two_calls_and_the_oracle(bole, data):
    """The one-pass decode step (the previous step's commit folded into this step's
    verify) on drawn previous trees, accepted paths and current trees: statuses and path
    rows as the two separate calls, bit for bit; states within 1e-6 and outputs within
    1e-5 of them; and within the bars of the oracle's commit then verify."""
    import numpy as np

    import oracle
    from tests.helpers import rel_err_rows, rel_err_states
    from tests.test_gpu_parity import TOL, _lazy_vs_separate, to_dev
    B = data.draw(st.integers(1, 5), label="batch")
    H = data.draw(st.integers(1, 3), label="heads")
    vec = data.draw(st.booleans(), label="vector_gate")
    dk = data.draw(st.sampled_from([64, 128]), label="d_k")
    dv = data.draw(st.sampled_from([32, 64, 128]), label="d_v")
    dtype = data.draw(st.sampled_from([torch.bfloat16, torch.bfloat16, torch.float32]), label="dtype")
    prev_sizes = data.draw(st.lists(st.integers(0, 64), min_size=B, max_size=B), label="prev_sizes")
    cur_sizes = data.draw(st.lists(st.integers(0, 64), min_size=B, max_size=B), label="cur_sizes")
    kinds = ["random", "chain", "deep", "bestfirst"]
    kp, kc = data.draw(st.sampled_from(kinds), label="prev_kind"), data.draw(st.sampled_from(kinds), label="cur_kind")
    seed = data.draw(st.integers(0, 10 ** 6), label="seed")
    le32 = max(prev_sizes) <= 32 and data.draw(st.booleans(), label="prev_trees_le_32")
    print(f"[case] drawn lazy B={B} H={H} vec={vec} dk={dk} dv={dv} dtype={dtype} prev={prev_sizes} "
          f"{kp} cur={cur_sizes} {kc} le32={le32} seed={seed}", flush=True)
    common = dict(batch=B, heads=H, d_k=dk, d_v=dv, vector_gate=vec, factor_dtype=dtype, max_path=64)
    wp = W.make_random(seed, sizes=prev_sizes, kind=kp, **common)
    wc = W.make_random(seed + 1, sizes=cur_sizes, kind=kc, **common)
    tp, tc = to_dev(wp), to_dev(wc)
    (Ha, oa, psa, pna, sa), (Hb, ob, psb, pnb, sb) = _lazy_vs_separate(bole, tp, tc, prev_trees_le_32=le32)
    np.testing.assert_array_equal(psb, psa)
    np.testing.assert_array_equal(pnb, pna)
    np.testing.assert_array_equal(sb, sa)
    assert rel_err_states(Hb.astype(np.float64), Ha.astype(np.float64)) <= 1e-6
    assert rel_err_rows(ob.astype(np.float64), oa.astype(np.float64)) <= 1e-5
    lp, lc = wp.layers[0], wc.layers[0]
    Href, pnref, pstref = oracle.commit_serial(lp.H0, lp.k, lp.v, lp.gate, wp.parent, wp.node_offsets,
                                               wp.accepted_idx, wp.accepted_len, vec)
    oref, stref = oracle.verify_serial(Href, lc.q, lc.k, lc.v, lc.gate, wc.parent, wc.node_offsets, vec)
    assert psb.tolist() == pstref.tolist() and sb.tolist() == stref.tolist()
    np.testing.assert_array_equal(pnb, pnref)
    assert rel_err_states(Hb.astype(np.float64), Href) <= TOL[dtype]
    assert rel_err_rows(ob.astype(np.float64), oref) <= TOL[dtype]


@drawn(25)
@given(st.data())
def test_drawn_builder_inputs_match_the_oracle(bole, data):
    """The draft-tree builder on drawn marginals: vocabularies from 1 token up and around
    the 4,096-token chunks, flat, tied and peaked rows, any budget, with and without a cost
    table; trees, tokens, path scores and speedups bit for bit the oracle's."""
    from tests.test_gpu_tree_build import primer_cost, run_and_compare
    B = data.draw(st.integers(1, 6), label="batch")
    D = data.draw(st.integers(1, 8), label="depth")
    V = data.draw(st.one_of(st.sampled_from([1, 2, 10, 63, 64, 65, 4095, 4096, 4097, 8192, 12289]),
                            st.integers(1, 40000)), label="vocab")
    n_max = data.draw(st.integers(1, 64), label="n_max")
    std = data.draw(st.sampled_from([0.0, 0.01, 0.5, 2.0, 4.0]), label="logit_std")
    grid = data.draw(st.sampled_from([None, None, 2.0 ** -10, 2.0 ** -14]), label="grid")
    alpha = data.draw(st.sampled_from([0.0, 0.02, 0.1]), label="alpha")
    fixed = data.draw(st.booleans(), label="fixed")
    seed = data.draw(st.integers(0, 10 ** 6), label="seed")
    print(f"[case] drawn builder B={B} D={D} V={V} n_max={n_max} std={std} grid={grid} "
          f"alpha={alpha} fixed={fixed} seed={seed}", flush=True)
    m = W.make_marginals(seed, B, D, V, logit_std=std, grid=grid)
    run_and_compare(bole, m, None if fixed else primer_cost(n_max, alpha), n_max, fixed=fixed)


@drawn(25)
@given(st.data())
def test_drawn_trees_accept_as_the_oracle(bole, data):
    """Tree acceptance on drawn trees, vocabularies, path limits, agreement and peakedness,
    greedy and sampling: statuses equal; accepted paths, lengths and bonus tokens bit for
    bit wherever the oracle's smallest decision margin is clear (every greedy tree)."""
    import numpy as np

    from tests.test_gpu_tree_accept import make_case, run
    B = data.draw(st.integers(1, 6), label="batch")
    sizes = data.draw(st.lists(st.integers(0, 64), min_size=B, max_size=B), label="sizes")
    kind = data.draw(st.sampled_from(["random", "chain", "star", "deep", "bestfirst"]), label="kind")
    V = data.draw(st.one_of(st.sampled_from([64, 65, 4096, 4097, 131073]), st.integers(64, 40000)), label="vocab")
    max_path = data.draw(st.integers(1, 64), label="max_path")
    sample = data.draw(st.booleans(), label="sample")
    agree = data.draw(st.sampled_from([0.0, 0.7, 1.0]), label="agree")
    peaked = data.draw(st.sampled_from([0.5, 2.0, 4.0]), label="peaked")
    seed = data.draw(st.integers(0, 10 ** 6), label="seed")
    print(f"[case] drawn accept B={B} sizes={sizes} {kind} V={V} max_path={max_path} sample={sample} "
          f"agree={agree} peaked={peaked} seed={seed}", flush=True)
    c = make_case(seed, B, V, sizes, kind, agree=agree, peaked=peaked)
    got, ref = run(bole, c, max_path, sample)
    np.testing.assert_array_equal(got["status"], ref["status"])
    clear = ref["margin"] > 1e-9 if sample else np.ones(B, bool)
    for k in ("accepted_idx", "accepted_len", "bonus"):
        np.testing.assert_array_equal(got[k][clear], ref[k][clear], err_msg=k)


@drawn(15)
@given(st.data())
def test_drawn_layer_stacks_equal_layer_by_layer(bole, data):
    """Layer stacks (verify, commit and the lazy step, up to 20 layers, so past one
    launch's 16) on drawn shapes and trees: bit for bit the single-layer calls on every
    layer, and the lazy stack within the oracle's bars."""
    from tests.test_gpu_parity import test_layer_stack_equals_layer_by_layer
    n_layers = data.draw(st.integers(1, 20), label="layers")
    B = data.draw(st.integers(1, 5), label="batch")
    kw = dict(batch=B, heads=data.draw(st.integers(1, 4), label="heads"),
              d_k=data.draw(st.sampled_from([64, 128]), label="d_k"),
              d_v=data.draw(st.sampled_from([32, 64, 128]), label="d_v"),
              sizes=data.draw(st.lists(st.integers(0, 64), min_size=B, max_size=B), label="sizes"),
              kind=data.draw(st.sampled_from(["random", "chain", "deep", "bestfirst"]), label="kind"),
              vector_gate=data.draw(st.booleans(), label="vector_gate"),
              factor_dtype=data.draw(st.sampled_from([torch.bfloat16, torch.bfloat16, torch.float32]),
                                     label="dtype"),
              max_path=64)
    name = f"drawn_stack_{data.draw(st.integers(0, 10 ** 6), label='name')}"
    print(f"[case] drawn stack {name} layers={n_layers} {kw}", flush=True)
    test_layer_stack_equals_layer_by_layer(bole, name, n_layers, kw)


@drawn(15)
@given(st.data())
def test_drawn_new_leaves_change_no_other_output(bole, data):
    """Leaves appended to drawn trees (any tree, under any node or the context) leave every
    other node's output as it was: within twice the oracle's bar, the bound that both
    calls meeting that bar implies, whichever size class or path each call takes."""
    import numpy as np

    from tests.helpers import rel_err_rows
    from tests.test_gpu_parity import TOL
    from tests.test_gpu_properties import run
    B = data.draw(st.integers(1, 5), label="batch")
    kw = dict(batch=B, heads=data.draw(st.integers(1, 3), label="heads"),
              d_k=data.draw(st.sampled_from([64, 128]), label="d_k"),
              d_v=data.draw(st.sampled_from([32, 64, 128]), label="d_v"),
              vector_gate=data.draw(st.booleans(), label="vector_gate"),
              factor_dtype=data.draw(st.sampled_from([torch.bfloat16, torch.bfloat16, torch.float32]),
                                     label="dtype"))
    sizes = data.draw(st.lists(st.integers(0, 63), min_size=B, max_size=B), label="sizes")
    grow = data.draw(st.lists(st.booleans(), min_size=B, max_size=B), label="grow")
    kind = data.draw(st.sampled_from(["random", "chain", "star", "deep", "bestfirst"]), label="kind")
    seed = data.draw(st.integers(0, 10 ** 6), label="seed")
    print(f"[case] drawn new leaves sizes={sizes} grow={grow} {kind} {kw} seed={seed}", flush=True)
    wl = W.make_random(seed, sizes=sizes, kind=kind, **kw)
    lay = wl.layers[0]
    ref = W.make_random(seed + 1, sizes=[1] * B, kind="random", **kw).layers[0]
    base = run(bole, lay.H0, lay.q, lay.k, lay.v, lay.gate, wl.parent, wl.node_offsets)
    q, k, v, gate = lay.q, lay.k, lay.v, lay.gate
    parent, offs = wl.parent.copy(), wl.node_offsets.copy()
    keep = np.arange(wl.total_nodes)               # new packed row of each old row
    for b in reversed(range(B)):                   # later trees first: earlier offsets hold
        if not grow[b]:
            continue
        hi = int(offs[b + 1])
        p_leaf = data.draw(st.integers(-1, sizes[b] - 1), label=f"leaf_parent_{b}")
        ins = lambda t, x: torch.cat([t[:hi], x[b:b + 1], t[hi:]])
        q, k, v, gate = ins(q, ref.q), ins(k, ref.k), ins(v, ref.v), ins(gate, ref.gate)
        parent = np.concatenate([parent[:hi], [p_leaf], parent[hi:]]).astype(np.int32)
        offs[b + 1:] += 1
        keep[keep >= hi] += 1
    out = run(bole, lay.H0, q, k, v, gate, parent, offs)
    assert out.shape[0] == wl.total_nodes + sum(grow)
    assert rel_err_rows(out[torch.from_numpy(keep)].double().numpy(), base.double().numpy()) \
        <= 2 * TOL[kw["factor_dtype"]]
