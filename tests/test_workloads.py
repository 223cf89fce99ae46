"""Input generator checks (CPU): the best-first draft trees follow the BASTION summary
page's builder (gist.science, "Method" section 2: repeatedly add the valid node with the
highest path score), and every workload is deterministic and well formed."""
import itertools

import numpy as np
import pytest

import workloads as W


def test_best_first_is_global_top_n():
    """Best-first expansion == the N highest path scores among all candidate paths
    (brute force over every path of a small candidate space)."""
    rng = np.random.default_rng(0)
    for trial in range(20):
        D, C, N = 3, 4, int(rng.integers(1, 30))
        marg = W.draft_marginals(rng, D, C)
        parent, rho, depth, cand = W.best_first_from_marginals(marg, N)
        paths = [p for d in range(1, D + 1) for p in itertools.product(range(C), repeat=d)]
        score = {p: float(np.prod([marg[i, c] for i, c in enumerate(p)])) for p in paths}
        top = sorted(paths, key=lambda p: -score[p])[:N]
        got = []
        for i in range(len(parent)):
            p, x = [], i
            while x >= 0:
                p.append(int(cand[x]))
                x = parent[x]
            got.append(tuple(reversed(p)))
        assert set(got) == set(top)
        np.testing.assert_allclose(rho, [score[p] for p in got], rtol=1e-12)


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_config_trees_well_formed(cid):
    wl = W.make_config(cid)
    offs = wl.node_offsets
    assert offs[0] == 0 and (np.diff(offs) >= 0).all() and (np.diff(offs) <= 64).all()
    for b in range(wl.batch):
        p = wl.parent[offs[b]:offs[b + 1]]
        assert all(-1 <= p[i] < i for i in range(len(p)))
        r = wl.rho[offs[b]:offs[b + 1]]
        if cid > 1:
            assert (np.diff(r) <= 0).all()               # insertion order = score order
            for i in range(len(p)):                      # prefix-closed, scores shrink
                if p[i] >= 0:
                    assert r[i] <= r[p[i]]
        L = wl.accepted_len[b]
        path = wl.accepted_idx[b, :L]
        assert L == 0 or p[path[0]] == -1
        assert all(p[path[m]] == path[m - 1] for m in range(1, L))
    lay = wl.layers[0]
    assert lay.q.shape == (wl.total_nodes, wl.heads, wl.d_k)
    assert lay.v.shape == (wl.total_nodes, wl.heads, wl.d_v)
    assert lay.H0.shape == (wl.batch, wl.heads, wl.d_k, wl.d_v)
    g = lay.gate.numpy()
    assert ((g > 0) & (g < 1)).all()


def test_configs_deterministic():
    a, b = W.make_config(2), W.make_config(2)
    assert (a.parent == b.parent).all() and (a.accepted_len == b.accepted_len).all()
    assert bool((a.layers[0].q == b.layers[0].q).all())
    assert bool((a.layers[0].H0 == b.layers[0].H0).all())


def test_config_shapes_match_plan():
    assert W.make_config(2).tree_sizes.tolist() == [32] * 8
    c4 = W.make_config(4)
    assert set(c4.tree_sizes.tolist()) <= {4, 8, 16, 32, 64} and c4.batch == 128
    c5 = W.make_config(5, n_layers=2)
    assert c5.batch == 64 and c5.heads == 32 and len(c5.layers) == 2
    assert c5.total_nodes == 64 * 32
    assert W.make_config(3).vector_gate and W.make_config(3).layers[0].gate.shape[-1] == 128
