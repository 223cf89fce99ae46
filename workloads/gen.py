"""Seeded synthetic workloads for Bole tree verification and path commit.

This module generates inputs only: draft trees, per-token factors, gates, committed
states and accepted paths. It holds none of the verify/commit arithmetic. The fp64
oracle and the GPU library both consume exactly the tensors returned here: the same
bf16/fp32 values, cast once from fp64 draws with round-to-nearest-even.

Draft trees follow the prefix-tree builder of the BASTION summary page (gist.science,
"Method" section 1, "tree-based block-diffusion drafting", and section 2, "acceptance
surrogate and best-first expansion"):
  - the drafter emits one marginal q_k over candidate tokens for each depth k;
  - a node x at depth d scores rho(x) = prod_{k=1..d} q_k(x_k) along its path;
  - best-first expansion repeatedly adds the highest-scoring node whose parent is
    already in the tree.
Nodes are numbered in insertion order, so parent[i] < i and every tree is prefix-closed.

Configuration ids 1-5 are the five workloads of the benchmark plan:
  1 tiny fp32 tree;
  2 Mamba-2-style scalar decay;
  3 GLA/RWKV-6-style vector gate;
  4 large-batch ragged trees;
  5 eight-layer hybrid stack.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def best_first_from_marginals(marg: np.ndarray, n_nodes: int):
    """Best-first prefix tree over given position-wise marginals ``marg[depth-1, cand]``.

    Returns (parent int32[n], rho float64[n], depth int32[n], cand int32[n]). Ties in
    rho break by depth, then candidate id, then insertion order."""
    max_depth, n_cand = marg.shape
    heap = []
    seq = 0
    for c in range(n_cand):
        heapq.heappush(heap, (-marg[0, c], 1, c, seq, -1))
        seq += 1
    parent, rho, depth, cand = [], [], [], []
    while len(parent) < n_nodes and heap:
        neg_r, d, c, _, par = heapq.heappop(heap)
        idx = len(parent)
        parent.append(par)
        rho.append(-neg_r)
        depth.append(d)
        cand.append(c)
        if d < max_depth:
            for cc in range(n_cand):
                heapq.heappush(heap, (neg_r * marg[d, cc], d + 1, cc, seq, idx))
                seq += 1
    return (np.asarray(parent, np.int32), np.asarray(rho, np.float64),
            np.asarray(depth, np.int32), np.asarray(cand, np.int32))


def draft_marginals(rng: np.random.Generator, max_depth: int, n_cand: int = 64,
                    logit_std: float = 2.0) -> np.ndarray:
    """One drafter marginal per depth: softmax of N(0, logit_std) logits over candidates."""
    logits = rng.standard_normal((max_depth, n_cand)) * logit_std
    marg = np.exp(logits - logits.max(axis=1, keepdims=True))
    return marg / marg.sum(axis=1, keepdims=True)


def best_first_tree(rng: np.random.Generator, n_nodes: int, max_depth: int,
                    n_cand: int = 64, logit_std: float = 2.0):
    """Draft tree of ``n_nodes`` nodes by best-first expansion over freshly drawn
    marginals. Returns (parent int32[n], rho float64[n], depth int32[n])."""
    marg = draft_marginals(rng, max_depth, n_cand, logit_std)
    parent, rho, depth, _ = best_first_from_marginals(marg, n_nodes)
    return parent, rho, depth


def greedy_branch(parent: np.ndarray, rho: np.ndarray) -> List[int]:
    """Highest-score branch: from the best root, step to the best child until a leaf
    (ties go to the lower index). Returns tree-local indices, root first."""
    n = len(parent)
    children: List[List[int]] = [[] for _ in range(n)]
    roots = []
    for i, p in enumerate(parent):
        (roots if p < 0 else children[p]).append(i)
    branch, cand = [], roots
    while cand:
        best = max(cand, key=lambda i: (rho[i], -i))
        branch.append(best)
        cand = children[best]
    return branch


@dataclass
class Layer:
    H0: torch.Tensor          # float32 [B, H, d_k, d_v]
    q: torch.Tensor           # [T, H, d_k], bf16 or fp32
    k: torch.Tensor           # [T, H, d_k]
    v: torch.Tensor           # [T, H, d_v]
    gate: torch.Tensor        # float32 [T, H] (scalar) or [T, H, d_k] (vector)


@dataclass
class Workload:
    name: str
    batch: int
    heads: int
    d_k: int
    d_v: int
    vector_gate: bool
    factor_dtype: torch.dtype
    parent: np.ndarray        # int32 [T], tree-local, -1 = child of the committed state
    node_offsets: np.ndarray  # int32 [B + 1]
    rho: np.ndarray           # float64 [T] path scores (1.0 where not defined)
    accepted_idx: np.ndarray  # int32 [B, max_path], tree-local, -1 padded
    accepted_len: np.ndarray  # int32 [B]
    layers: List[Layer] = field(default_factory=list)
    recipe: str = ""

    @property
    def total_nodes(self) -> int:
        return int(self.node_offsets[-1])

    @property
    def max_path(self) -> int:
        return int(self.accepted_idx.shape[1])

    @property
    def tree_sizes(self) -> np.ndarray:
        return np.diff(self.node_offsets)


def _cast(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).contiguous()


def _layer(ss: np.random.SeedSequence, B, H, T, d_k, d_v, fdt, vector_gate, qkv_std, h0_std,
           gate_shift=0.0, gate_scale=1.0, gate_value=None) -> Layer:
    rq, rk, rv, rg, rh = (np.random.default_rng(s) for s in ss.spawn(5))
    q = _cast(rq.standard_normal((T, H, d_k)) * qkv_std, fdt)
    k = _cast(rk.standard_normal((T, H, d_k)) * qkv_std, fdt)
    v = _cast(rv.standard_normal((T, H, d_v)) * qkv_std, fdt)
    gshape = (T, H, d_k) if vector_gate else (T, H)
    gate = _cast(gate_scale * np.exp(-softplus(rg.standard_normal(gshape) + gate_shift)),
                 torch.float32)
    if gate_value is not None:  # every gate the same value (1.0: no decay at all)
        gate = torch.full(gshape, float(gate_value), dtype=torch.float32)
    H0 = _cast(rh.standard_normal((B, H, d_k, d_v)) * h0_std, torch.float32)
    return Layer(H0=H0, q=q, k=k, v=v, gate=gate)


def _accept_paths(rng, parents, rhos, max_path, geom_p=0.2):
    """Accepted length ~ Geometric(p) on {0, 1, ...} (accepted drafts before the first
    rejection), truncated to the greedy branch; the path is that branch's prefix."""
    B = len(parents)
    idx = np.full((B, max_path), -1, np.int32)
    lens = np.zeros(B, np.int32)
    for b in range(B):
        branch = greedy_branch(parents[b], rhos[b]) if len(parents[b]) else []
        L = min(int(rng.geometric(geom_p)) - 1, len(branch), max_path)
        lens[b] = L
        idx[b, :L] = branch[:L]
    return idx, lens


def _pack(parents: Sequence[np.ndarray]):
    offs = np.zeros(len(parents) + 1, np.int32)
    offs[1:] = np.cumsum([len(p) for p in parents])
    parent = np.concatenate(parents).astype(np.int32) if parents else np.zeros(0, np.int32)
    return parent, offs


CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "mamba2_scalar",
    3: "gla_vector",
    4: "ragged_large_batch",
    5: "hybrid_stack",
}


def make_config(cid: int, n_layers: Optional[int] = None) -> Workload:
    """The five benchmark workloads (seed = SeedSequence(1000 + cid)).

    Configuration 5 has 8 layers that share one tree per sequence; ``n_layers`` limits
    how many are generated (for tests)."""
    root = np.random.SeedSequence(1000 + cid)
    if cid == 1:
        tree_ss, acc_ss, lay_ss = root.spawn(3)
        parent = np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
        offs = np.array([0, 7], np.int32)
        lay = _layer(lay_ss, 1, 1, 7, 16, 16, torch.float32, False, 1.0 / 4.0, 0.1)
        acc_idx = np.array([[0, 1, 3]], np.int32)
        acc_len = np.array([3], np.int32)
        return Workload(CONFIG_NAMES[1], 1, 1, 16, 16, False, torch.float32, parent, offs,
                        np.ones(7), acc_idx, acc_len, [lay],
                        "B=1 H=1 d=16 fp32; parent [-1,0,0,1,1,2,2]; a=exp(-softplus(N(0,1))); "
                        "q,k,v~N(0,1)/4; H0~N(0,0.1); commit [0,1,3]")
    spec = {
        2: dict(B=8, H=32, d_k=128, d_v=64, vec=False, sizes="fixed", N=32, D=8, layers=1),
        3: dict(B=16, H=16, d_k=128, d_v=128, vec=True, sizes="fixed", N=64, D=10, layers=1),
        4: dict(B=128, H=32, d_k=128, d_v=64, vec=False, sizes="budget", N=None, D=8,
                layers=1),
        5: dict(B=64, H=32, d_k=128, d_v=64, vec=False, sizes="fixed", N=32, D=8, layers=8),
    }[cid]
    L = spec["layers"] if n_layers is None else min(n_layers, spec["layers"])
    tree_ss, acc_ss, *lay_ss = root.spawn(2 + spec["layers"])
    trng = np.random.default_rng(tree_ss)
    parents, rhos = [], []
    for _ in range(spec["B"]):
        n = spec["N"] if spec["sizes"] == "fixed" else int(trng.choice([4, 8, 16, 32, 64]))
        p, r, _ = best_first_tree(trng, n, spec["D"])
        parents.append(p)
        rhos.append(r)
    parent, offs = _pack(parents)
    T = int(offs[-1])
    acc_idx, acc_len = _accept_paths(np.random.default_rng(acc_ss), parents, rhos, spec["D"])
    std = 1.0 / np.sqrt(spec["d_k"])
    layers = [_layer(lay_ss[l], spec["B"], spec["H"], T, spec["d_k"], spec["d_v"],
                     torch.bfloat16, spec["vec"], std, 0.05) for l in range(L)]
    recipe = (f"B={spec['B']} H={spec['H']} d_k={spec['d_k']} d_v={spec['d_v']} bf16 q,k,v "
              f"~N(0,1)/sqrt({spec['d_k']}); H0 fp32 ~N(0,0.05); "
              f"{'vector' if spec['vec'] else 'scalar'} gate exp(-softplus(N(0,1))); "
              f"best-first trees N={'U{4,8,16,32,64}' if spec['N'] is None else spec['N']} "
              f"D={spec['D']} over 64 candidates, softmax(N(0,2)) marginals; accepted length "
              f"Geometric(0.2)-1 truncated to the greedy branch; {spec['layers']} layer(s)")
    return Workload(CONFIG_NAMES[cid], spec["B"], spec["H"], spec["d_k"], spec["d_v"],
                    spec["vec"], torch.bfloat16, parent, offs, np.concatenate(rhos), acc_idx,
                    acc_len, layers, recipe)


def make_marginals(seed: int, batch: int, depth: int, vocab: int, logit_std: float = 2.0,
                   grid: Optional[float] = None) -> np.ndarray:
    """Synthetic drafter output for the tree builder: for each sequence and position
    k = 1..depth, q_k = softmax(logits), logits ~ N(0, logit_std) over the vocabulary
    (the shape of a block-diffusion drafter's position-wise marginals). float32
    [batch][depth][vocab]. grid: round every probability down to a multiple of it (many
    exact ties, for tie-order tests)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x7ee5]))
    z = rng.normal(0.0, logit_std, size=(batch, depth, vocab))
    z -= z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=-1, keepdims=True)
    if grid is not None:
        p = np.floor(p / grid) * grid
    return p.astype(np.float32)


def make_accept_inputs(parent: np.ndarray, node_offsets: np.ndarray, vocab: int, seed: int,
                       device, agree: float = 0.7):
    """Synthetic target and draft rows for tree acceptance, built on `device` with a seeded
    torch generator: draft logits N(0, 2) for every node and for each tree's verified
    context; each node's children carry the draft row's top tokens in order; target
    logits = draft + N(0, 1), with the first child's token raised by 8 at a fraction
    `agree` of the nodes (so that paths of several nodes are accepted); uniforms U[0, 1).
    Returns a dict of tensors: p_ctx, q_ctx [B, V], p_node, q_node [T, V], token [T],
    u_node [T], u_bonus [B] (float32 / int32)."""
    T, B = int(parent.shape[0]), int(node_offsets.shape[0]) - 1
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    zq = torch.randn((T + B, vocab), generator=gen, device=device) * 2.0
    top = torch.topk(zq, min(64, vocab), dim=1).indices.cpu().numpy()
    tok = np.zeros(T, np.int32)
    rng = np.random.default_rng(seed)
    raise_at = []
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        for cur in [-1] + list(range(hi - lo)):
            kids = [i for i in range(hi - lo) if parent[lo + i] == cur]
            row = T + b if cur < 0 else lo + cur
            for r, c in enumerate(kids):
                tok[lo + c] = top[row, r]
            if kids and rng.random() < agree:
                raise_at.append((row, int(tok[lo + kids[0]])))
    zp = zq + torch.randn(zq.shape, generator=gen, device=device)
    if raise_at:
        ri = torch.tensor([r for r, _ in raise_at], device=device)
        ci = torch.tensor([c for _, c in raise_at], device=device)
        zp[ri, ci] += 8.0
    p, q = torch.softmax(zp, dim=1), torch.softmax(zq, dim=1)
    del zp, zq
    out = {"p_node": p[:T].contiguous(), "p_ctx": p[T:].contiguous(),
           "q_node": q[:T].contiguous(), "q_ctx": q[T:].contiguous(),
           "token": torch.from_numpy(tok).to(device),
           "u_node": torch.rand(T, generator=gen, device=device),
           "u_bonus": torch.rand(B, generator=gen, device=device)}
    return out


def random_tree(rng: np.random.Generator, n: int, kind: str) -> np.ndarray:
    """Tree-local parent array of n nodes, parent[i] < i. Kinds: 'random' (uniform
    parent in [-1, i)), 'chain', 'star' (all roots), 'bestfirst', 'deep' (mostly chains)."""
    if n == 0:
        return np.zeros(0, np.int32)
    if kind == "chain":
        return np.arange(-1, n - 1, dtype=np.int32)
    if kind == "star":
        return np.full(n, -1, np.int32)
    if kind == "bestfirst":
        return best_first_tree(rng, n, 10)[0]
    if kind == "deep":
        p = np.arange(-1, n - 1, dtype=np.int32)
        jumps = rng.random(n) < 0.15
        for i in np.nonzero(jumps)[0]:
            if i > 0:
                p[i] = rng.integers(-1, i)
        return p
    return np.array([rng.integers(-1, i) if i > 0 else -1 for i in range(n)], np.int32)


def make_random(seed: int, batch: int, heads: int, d_k: int, d_v: int,
                sizes: Optional[Sequence[int]] = None, kind: str = "random",
                vector_gate: bool = False, factor_dtype: torch.dtype = torch.bfloat16,
                max_path: int = 16, gate_shift: float = 0.0, h0_std: float = 0.05,
                gate_scale: float = 1.0, gate_value: Optional[float] = None) -> Workload:
    """Seeded workload with arbitrary shapes for parity and edge-case tests.
    ``sizes`` gives each tree's node count (default: uniform in [1, 64]). Gates are
    ``gate_scale * exp(-softplus(x + gate_shift))`` with x ~ N(0, 1): a scale above 1
    gives gates above 1 as well (the state grows along a path). ``gate_value`` sets every
    gate to one value instead."""
    root = np.random.SeedSequence(seed)
    tree_ss, acc_ss, lay_ss = root.spawn(3)
    trng = np.random.default_rng(tree_ss)
    if sizes is None:
        sizes = trng.integers(1, 65, size=batch)
    parents = [random_tree(trng, int(n), kind) for n in sizes]
    parent, offs = _pack(parents)
    T = int(offs[-1])
    arng = np.random.default_rng(acc_ss)
    rhos = [arng.random(len(p)) for p in parents]
    acc_idx = np.full((batch, max_path), -1, np.int32)
    acc_len = np.zeros(batch, np.int32)
    for b in range(batch):
        branch = greedy_branch(parents[b], rhos[b]) if len(parents[b]) else []
        L = int(arng.integers(0, min(len(branch), max_path) + 1))
        acc_len[b] = L
        acc_idx[b, :L] = branch[:L]
    lay = _layer(lay_ss, batch, heads, T, d_k, d_v, factor_dtype, vector_gate,
                 1.0 / np.sqrt(d_k), h0_std, gate_shift, gate_scale, gate_value)
    return Workload(f"random_{kind}_{seed}", batch, heads, d_k, d_v, vector_gate, factor_dtype,
                    parent, offs, np.concatenate(rhos) if rhos else np.zeros(0), acc_idx,
                    acc_len, [lay], f"random {kind} trees, seed {seed}")
