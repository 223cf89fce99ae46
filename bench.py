#!/usr/bin/env python3
"""Benchmark of the Bole tree-verify hot path on one MI355X.

Workload: the hybrid layer stack. There are 64 sequences, each with one best-first
draft tree of 32 nodes, and 8 linear-recurrence layers of 32 heads (d_k=128, d_v=64).
q/k/v are bf16; the scalar gate and the committed state H0 are fp32. The 8 layers see
the same draft tokens, so they share the trees and the accepted paths.

One decode step does, for every layer, one accepted-path commit and one tree verify. The
headline step runs them as the decode loop would in steady state: one launch for the
8-layer stack (bole_tree_verify_lazy_commit_layers) that commits the previous step's
accepted path into each layer's H0 and verifies this step's tree against the result, so
H0 is read once and written once per step. The previous step is the same synthetic
batch (same trees, paths and factors), so every timed step does exactly one commit and
one verify per layer. The same work as two passes (bole_tree_verify_layers, then
bole_commit_path_layers: H0 read twice, written once) is timed beside it. All inputs are
resident in HBM before the timed region starts. The 8 layers hold 1 GB, four times the
256 MB last-level cache, so every layer is read cold.

The program prints one JSON line:
  - value: draft nodes verified (and committed) through the whole stack per second;
  - roofline: for the step's kernel, its algorithmic bytes per launch over its average
    launch time (one HIP event pair on the launch stream around the timed steps, which
    hold nothing but back-to-back launches), against the 8 TB/s HBM peak;
  - cpu_baseline: the fp64 CPU oracle timed on this host on whole steps of the same
    workload.
"""
import argparse
import json
import os
import sys
import time

METRIC = "tree-verify draft nodes/s + achieved HBM GB/s (B=64, 32 heads, N=32)"
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
_CSRC = os.path.join(ROOT, "tree_speculative_decoding_02_amd", "csrc")
# sources that determine each kernel's memory traffic
_VERIFY_SOURCES = [os.path.join(_CSRC, f) for f in ("verify_mfma.hip", "mfma_util.h",
                                                   "bole_device.h")]
KERNEL_SOURCES = {
    "lazy": _VERIFY_SOURCES,
    "verify": _VERIFY_SOURCES,
    "commit": [os.path.join(_CSRC, f) for f in ("commit.hip", "bole_device.h")],
    "topk": [os.path.join(_CSRC, f) for f in ("tree_build.hip", "bole_device.h")],
}
# FETCH_SIZE / WRITE_SIZE record of the last counter runs (calibrated bytes per launch)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hybrid_stack_hbm_traffic.md")


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch from the committed counter record, or None when there is no
    record or the kernel's sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            line = next(l for l in f if l.startswith("TRAFFIC_JSON "))
        rec = json.loads(line[len("TRAFFIC_JSON "):])["kernels"][kernel]
    except (OSError, StopIteration, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec["traffic_bytes"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time for the oracle baseline (whole steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-layer-forms", action="store_true",
                    help="also time both forms with one launch per layer (the same kernels "
                         "as the stacked forms, so leave it off in profiled runs)")
    ap.add_argument("--no-builder", action="store_true",
                    help="skip timing the draft-tree builder")
    ap.add_argument("--no-calibration", action="store_true",
                    help="feed the tree builder's controller the LLM Primer's cost model "
                         "instead of timing the lazy step at several tree sizes (keeps "
                         "profiled runs to the benchmark's own launches)")
    ap.add_argument("--no-accept", action="store_true",
                    help="skip timing tree acceptance")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip timing the naive serial-walk baseline")
    ap.add_argument("--config-sweep", action="store_true",
                    help="instead of the benchmark, time verify and commit on each of the five "
                         "workloads (one JSON line each)")
    ap.add_argument("--sweep-configs", default="1,2,3,4,5",
                    help="workloads the sweep covers (comma-separated ids)")
    return ap.parse_args()


def verify_bytes(wl, s_f=2):
    """Algorithmic HBM bytes of one verify launch (one layer): H0 read once, every
    node's q, k, v, gate read once, out written once, plus parent and offsets."""
    B, H, dk, dv, T = wl.batch, wl.heads, wl.d_k, wl.d_v, wl.total_nodes
    s_g = 4 * (dk if wl.vector_gate else 1)
    return (4 * B * H * dk * dv + T * H * ((2 * dk + dv) * s_f + s_g) + 4 * T * H * dv
            + 4 * T + 4 * (B + 1))


def commit_bytes(wl, s_f=2):
    """Algorithmic HBM bytes of one commit launch: for each sequence with an accepted
    path (L > 0), H0 read and written once and the path's k, v, gate read once."""
    H, dk, dv = wl.heads, wl.d_k, wl.d_v
    s_g = 4 * (dk if wl.vector_gate else 1)
    tot = 0
    for b in range(wl.batch):
        L = int(wl.accepted_len[b])
        if L > 0:
            tot += H * (8 * dk * dv + L * ((dk + dv) * s_f + s_g))
    return tot + 4 * wl.batch * (wl.max_path + 1) + 4 * wl.total_nodes + 4 * (wl.batch + 1)


def lazy_bytes(wl, s_f=2):
    """Algorithmic HBM bytes of one layer of a lazy launch (the previous step's commit
    folded into this step's verify): verify's and commit's bytes, less the second read of
    H_0 that the two-pass form makes for every (sequence, head) with a non-empty path."""
    with_path = int((wl.accepted_len > 0).sum())
    return verify_bytes(wl, s_f) + commit_bytes(wl, s_f) - 4 * wl.heads * wl.d_k * wl.d_v * with_path


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(verify and commit shard by sequence or head with no communication); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from tree_speculative_decoding_02_amd import bole

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config_sweep:
        config_sweep(dev, configs=tuple(int(c) for c in args.sweep_configs.split(",")))
        return
    wl = W.make_config(5)
    L = len(wl.layers)
    print(f"[bench] workload {wl.name}: B={wl.batch} layers={L} H={wl.heads} d_k={wl.d_k} "
          f"d_v={wl.d_v} T={wl.total_nodes}", file=sys.stderr, flush=True)
    g = lambda t: t.to(dev)
    # transient memory per layer, measured: what Bole keeps per node between verify and
    # commit is the factors (k, v, gate) and no workspace (bole_workspace_bytes = 0)
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated(dev)
    kept = [g(wl.layers[0].k), g(wl.layers[0].v), g(wl.layers[0].gate)]
    bole_kept_bytes = torch.cuda.memory_allocated(dev) - m0 + bole.bole_workspace_bytes()
    del kept
    parent = torch.from_numpy(wl.parent).to(dev)
    offs = torch.from_numpy(wl.node_offsets).to(dev)
    acc_idx = torch.from_numpy(wl.accepted_idx).to(dev)
    acc_len = torch.from_numpy(wl.accepted_len).to(dev)
    layers = []
    for l in wl.layers:
        y = dict(H0=g(l.H0), q=g(l.q), k=g(l.k), v=g(l.v), gate=g(l.gate),
                 out=torch.empty((wl.total_nodes, wl.heads, wl.d_v), dtype=torch.float32,
                                 device=dev))
        y.update(prev_k=y["k"], prev_v=y["v"], prev_gate=y["gate"])  # previous step: same batch
        layers.append(y)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    kw = dict(stream=stream, trees_le_32=True)

    # arguments are checked and marshalled once; the timed loops only enqueue launches
    lazy = bole.bind_tree_verify_lazy_commit_layers(layers, parent, offs, acc_idx, acc_len, parent,
                                                    offs, prev_trees_le_32=True, **kw)
    vstack = bole.bind_tree_verify_layers(layers, parent, offs, **kw)
    cstack = bole.bind_commit_path_layers(layers, parent, offs, acc_idx, acc_len, **kw)

    def timed(groups, steps, warmup):
        """Runs `steps` steps of the launch groups (a step runs every group once, in
        order); returns (ms per step, average ms of each group's launches, wall seconds).
        Every time is one event pair around back-to-back launches with nothing between
        them (an event between two launches costs the stream several microseconds): the
        step time around all steps, and a group's time around `steps` runs of that group
        alone (with one group, the step time itself)."""
        def run(gs, n):
            for _ in range(n):
                for grp in gs:
                    for f in grp:
                        f()

        def span(gs, n):
            t0, t1 = ev(), ev()
            torch.cuda.synchronize()
            t0.record(stream)
            run(gs, n)
            t1.record(stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / n

        run(groups, warmup)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ms = span(groups, steps)
        wall = time.perf_counter() - w0
        if len(groups) == 1:
            return ms, [ms], wall
        return ms, [span([grp], steps) for grp in groups], wall

    # headline: the lazy step, one launch for the stack
    ms_per_step, l_ms, wall = timed([[lazy]], args.steps, args.warmup)
    # the same work in two passes, one launch each for the stack
    tp_ms, tp_group_ms, _ = timed([[vstack], [cstack]], args.steps, args.warmup)
    # the lazy step for a caller that states no tree budget: trees of up to 64 nodes may
    # come, so the fused launch runs (two wavefronts per unit, the second idle for trees
    # of up to 32 nodes)
    lazy_any = bole.bind_tree_verify_lazy_commit_layers(layers, parent, offs, acc_idx, acc_len,
                                                        parent, offs, stream=stream)
    la_ms, _, _ = timed([[lazy_any]], args.steps, args.warmup)
    # the memory-only reference for the lazy step: the same bytes in the same pieces
    ref_launch = lazy_traffic_launch(probe_lib(), layers, wl, offs, acc_idx, acc_len, stream)
    ref_ms, _, _ = timed([[ref_launch]], args.steps, args.warmup)

    nodes = wl.total_nodes
    lb, vb, cb = lazy_bytes(wl), verify_bytes(wl), commit_bytes(wl)

    def kernel_rec(launch_ms, nbytes, what):
        us = 1e3 * launch_ms
        gbs = L * nbytes / (us * 1e3)
        return {"avg_us_per_launch": us, "layers_per_launch": L, "avg_us_per_layer": us / L,
                # the draft nodes of one layer (every head) over one layer's share of the time
                "layer_nodes_per_s": wl.total_nodes / (us / L * 1e-6),
                "bytes_per_launch": L * nbytes, "bytes_per_layer": nbytes, "GB_s": gbs,
                "frac_hbm_peak": gbs / HBM_PEAK_GBS, "what": what}

    kernels = {
        "lazy": kernel_rec(l_ms[0], lb, "verify_mfma_tree_kernel<128,64,1,lazy>: previous "
                           "path committed into H0, this tree verified, 8 layers"),
        "verify": kernel_rec(tp_group_ms[0], vb, "verify_mfma_tree_kernel<128,64,1>: two-pass "
                             "form, verify of 8 layers"),
        "commit": kernel_rec(tp_group_ms[1], cb, "commit_stream_kernel<bf16,scalar>: two-pass "
                             "form, commit of 8 layers"),
    }
    kd = kernels["lazy"]
    ref_gbs = L * lb / (ref_ms * 1e6)
    lazy_reference = {"avg_us_per_launch": 1e3 * ref_ms, "GB_s": ref_gbs,
                      "frac_hbm_peak": ref_gbs / HBM_PEAK_GBS,
                      "lazy_rate_of_reference": ref_ms / l_ms[0],
                      "what": "memory-only kernel moving exactly the lazy launch's bytes (8 "
                              "layers: H0 read and written back, path and tree rows, out) in "
                              "the same row pieces, no arithmetic"}
    naive = wl.heads * wl.total_nodes * wl.d_k * wl.d_v * 4
    bole_transient = sum(int(layers[0][n].numel() * layers[0][n].element_size())
                         for n in ("k", "v", "gate"))
    result = {
        "metric": METRIC,
        "value": nodes / (ms_per_step * 1e-3),
        "unit": "draft nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hybrid_stack: 64 sequences x 8 linear-recurrence layers x 32 "
                               "heads, d_k=128, d_v=64, 32-node best-first draft trees, bf16 "
                               "q/k/v, fp32 scalar gate and state; per step and layer one "
                               "accepted-path commit and one tree verify, run as one launch "
                               "for the stack that commits the previous step's path and "
                               "verifies this step's tree in one pass over H0",
                   "batch": wl.batch, "layers": L, "heads": wl.heads, "d_k": wl.d_k,
                   "d_v": wl.d_v, "nodes_per_tree": 32, "step_form": "lazy_commit_stacked",
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "kernel": "lazy", "achieved": kd["GB_s"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kd["frac_hbm_peak"],
                     "traffic": recorded_traffic("lazy")},
        "kernels": kernels,
        "forms": {
            "lazy_commit_stacked": {"ms_per_step": ms_per_step,
                                    "value": nodes / (ms_per_step * 1e-3), "launches_per_step": 1},
            "two_pass_stacked": {"ms_per_step": tp_ms, "value": nodes / (tp_ms * 1e-3),
                                 "launches_per_step": 2},
            "lazy_commit_stacked_no_tree_budget": {"ms_per_step": la_ms,
                                                   "value": nodes / (la_ms * 1e-3),
                                                   "launches_per_step": 1},
        },
        "lazy_traffic_reference": lazy_reference,
        "hbm_GB_s_step": L * lb / (ms_per_step * 1e6),
        "wall_ms_per_step": 1e3 * wall / args.steps,
        "transient_bytes_per_layer": {"naive_state_per_node": naive,
                                      "bole_factors": bole_transient,
                                      "bole_measured": bole_kept_bytes,
                                      "reduction": 1.0 - bole_kept_bytes / naive},
    }
    if args.per_layer_forms:
        v1 = [bole.bind_tree_verify(y["H0"], y["q"], y["k"], y["v"], y["gate"], parent, offs,
                                    y["out"], **kw) for y in layers]
        c1 = [bole.bind_commit_path(y["H0"], y["k"], y["v"], y["gate"], parent, offs, acc_idx,
                                    acc_len, **kw) for y in layers]
        l1 = [bole.bind_tree_verify_lazy_commit(
            y["H0"], (y["k"], y["v"], y["gate"], parent, offs), acc_idx, acc_len, y["q"], y["k"],
            y["v"], y["gate"], parent, offs, y["out"], prev_trees_le_32=True, **kw) for y in layers]
        for name, groups in (("lazy_commit_per_layer", [l1]), ("two_pass_per_layer", [v1, c1])):
            ms, _, _ = timed(groups, args.steps, args.warmup)
            result["forms"][name] = {"ms_per_step": ms, "value": nodes / (ms * 1e-3),
                                     "launches_per_step": L * len(groups)}
    v_us = kernels["verify"]["avg_us_per_layer"]

    # the draft-tree builder on the same batch: 64 sequences x 8 drafted positions over a
    # 128256-token vocabulary (Llama-3.1's), best-first up to 64 nodes, with the budget
    # controller's cost C(N) from this GPU: the lazy step of the same stack is timed at
    # tree sizes N, the roofline form T(N) = t0 + t1 N fitted to it, L_AR = T(1) (one node
    # per sequence is an autoregressive step through these layers) and
    # C(N) = T_draft + T(N) with T_draft = 0.1 L_AR
    if not args.no_builder:
        Bb, Db, Vb, nb = wl.batch, 8, 128256, 64
        if args.no_calibration:
            # the speedup model of the LLM Primer (chapter 9.3), in autoregressive steps:
            # C(N) = T_draft/T_AR + 1 + 0.05 N
            t0, t1, l_ar = 1.0, 0.05, 1.0
        else:
            calib = calibrate_verify_cost(bole, W, wl, dev, stream, timed)
            t0, t1 = calib["fit_us"]["t0"], calib["fit_us"]["t1"]
            l_ar = t0 + t1
            result["controller_calibration"] = calib
        marg = torch.from_numpy(W.make_marginals(2024, Bb, Db, Vb)).to(dev)
        cost = torch.tensor([0.1 * l_ar + t0 + t1 * n for n in range(1, nb + 1)],
                            dtype=torch.float32, device=dev)
        build = bole.bind_build_tree(marg, cost, l_ar, n_max=nb, stream=stream)
        b_ms, _, _ = timed([[build]], args.steps, args.warmup)
        b_us = 1e3 * b_ms
        b_bytes = Bb * Db * Vb * 4   # the marginals, read once; the rest is < 0.1 %
        torch.cuda.synchronize()
        n_kept = build.out["node_offsets"][-1].item()
        result["tree_builder"] = {
            "avg_us_per_call": b_us,
            "bytes_per_call": b_bytes, "GB_s": b_bytes / (b_us * 1e3),
            "frac_hbm_peak": b_bytes / (b_us * 1e3) / HBM_PEAK_GBS, "nodes_kept": n_kept,
            "topk_kernel_traffic": recorded_traffic("topk"),
            "what": "bole_build_tree: top-64 per position, best-first tree, budget controller "
                    "and packing for 64 sequences x 8 positions x 128256 tokens (3 launches)"}
        del marg

    # tree acceptance on the same trees: target and draft rows over a 128256-token
    # vocabulary for the context and every node (synthetic, generated on the GPU: draft
    # logits N(0, 2), target = draft + N(0, 1) with the first child's token raised by 8
    # at 70 % of the nodes; each node's children carry the draft row's top tokens)
    if not args.no_accept:
        Va = 128256
        ai = W.make_accept_inputs(wl.parent, wl.node_offsets, Va, 2025, dev)
        p_ctx, p_node, q_ctx, q_node = ai["p_ctx"], ai["p_node"], ai["q_ctx"], ai["q_node"]
        tok, u_node, u_bonus = ai["token"], ai["u_node"], ai["u_bonus"]
        del ai
        acc = {}
        for mode in ("greedy", "sample"):
            f = bole.bind_tree_accept(p_ctx, p_node, parent, tok, offs, wl.max_path,
                                      sample=mode == "sample", q_ctx=q_ctx, q_node=q_node,
                                      u_node=u_node, u_bonus=u_bonus, stream=stream)
            a_ms, _, _ = timed([[f]], args.steps, args.warmup)
            torch.cuda.synchronize()
            lens = f.out["accepted_len"][:wl.batch].cpu().numpy()
            us = 1e3 * a_ms
            rec = {"avg_us_per_call": us, "mean_accepted_len": float(lens.mean())}
            if mode == "greedy":
                # the walk reads one target row per visited node (the path and its end)
                nb = int((lens + 1).sum()) * Va * 4
                rec.update({"bytes_per_call": nb, "GB_s": nb / (us * 1e3),
                            "frac_hbm_peak": nb / (us * 1e3) / HBM_PEAK_GBS})
            acc[mode] = rec
        acc["what"] = ("bole_tree_accept on the benchmark's 64 trees of 32 nodes, target and "
                       "draft rows over 128256 tokens")
        result["tree_accept"] = acc
        del p_node, p_ctx, q_node, q_ctx

    # the naive serial walk on layer 0 (one materialised state per node): the baseline the
    # closed form is measured against, timed after the benchmark proper
    if not args.no_naive:
        x = layers[0]
        torch.cuda.synchronize()
        m0 = torch.cuda.memory_allocated(dev)
        states = torch.empty((wl.total_nodes, wl.heads, wl.d_k, wl.d_v), dtype=torch.float32,
                             device=dev)
        states_bytes = torch.cuda.memory_allocated(dev) - m0
        nout = torch.empty_like(x["out"])
        naive = lambda: bole.bole_tree_verify_naive(x["H0"], x["q"], x["k"], x["v"], x["gate"],
                                                    parent, offs, out=nout, states=states,
                                                    stream=stream)
        naive()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(5):
            naive()
        b.record(stream)
        torch.cuda.synchronize()
        n_us = a.elapsed_time(b) * 1e3 / 5
        result["naive_serial_walk"] = {
            "avg_us_per_layer": n_us, "closed_form_speedup": n_us / v_us,
            "states_bytes_measured": states_bytes,
            "what": "bole_tree_verify_naive: every node's state materialised in tree order, "
                    "layer 0 of the same workload, 5 launches"}
        del states, nout

    # a plain 512 MiB device copy: a practical streaming rate (one byte read per byte
    # written) beside the 8 TB/s peak; under rocprofv3 counters its launches also calibrate
    # FETCH_SIZE and WRITE_SIZE against bytes known exactly
    n = 512 * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 8 * n / (a.elapsed_time(b) * 1e6)
    result["copy_reference"] = {"read_bytes": 4 * n, "write_bytes": 4 * n, "GB_s": copy_gbs,
                                "lazy_kernel_frac_of_copy": kd["GB_s"] / copy_gbs}
    del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def calibrate_verify_cost(bole, W, wl, dev, stream, timed, sizes=(1, 4, 8, 16, 32, 64)):
    """The lazy step of the benchmark's stack (64 sequences, 8 layers x 32 heads,
    d_k=128, d_v=64) timed with every tree of N nodes, for each N in `sizes`; the
    least-squares line T(N) = t0 + t1 N through the times (us per step)."""
    import numpy as np
    import torch
    ts = []
    for n in sizes:
        w = W.make_random(900 + n, batch=wl.batch, heads=wl.heads, d_k=wl.d_k, d_v=wl.d_v,
                          sizes=[n] * wl.batch, kind="bestfirst", max_path=wl.max_path)
        lay = w.layers[0]
        g = lambda x: x.to(dev)
        par, offs = g(torch.from_numpy(w.parent)), g(torch.from_numpy(w.node_offsets))
        ai, al = g(torch.from_numpy(w.accepted_idx)), g(torch.from_numpy(w.accepted_len))
        q, k, v, gate = g(lay.q), g(lay.k), g(lay.v), g(lay.gate)
        layers = [dict(H0=g(lay.H0).clone(), q=q, k=k, v=v, gate=gate, prev_k=k, prev_v=v,
                       prev_gate=gate,
                       out=torch.empty((w.total_nodes, w.heads, w.d_v), dtype=torch.float32,
                                       device=dev)) for _ in range(len(wl.layers))]
        step = bole.bind_tree_verify_lazy_commit_layers(
            layers, par, offs, ai, al, par, offs, stream=stream, trees_le_32=n <= 32,
            prev_trees_le_32=n <= 32)
        ms, _, _ = timed([[step]], 20, 3)
        ts.append(1e3 * ms)
        del layers, step
    A = np.stack([np.ones(len(sizes)), np.array(sizes, float)], axis=1)
    (t0, t1), *_ = np.linalg.lstsq(A, np.array(ts), rcond=None)
    return {"N": list(sizes), "T_us": ts, "fit_us": {"t0": float(t0), "t1": float(t1)},
            "what": "lazy step of the 8-layer stack with every tree of N nodes; "
                    "C(N) = 0.1 L_AR + t0 + t1 N, L_AR = t0 + t1"}


ROTATE_BYTES = 512 * 2 ** 20   # input sets rotated per launch kind: at least this much


def sweep_sets(wl, dev, rotate_bytes=ROTATE_BYTES, max_sets=64):
    """Copies of one workload layer's whole input set (H0, q, k, v, gate, out, trees and
    paths) on the GPU, enough of them that consecutive launches over the copies read at
    least `rotate_bytes`: twice the 256 MB last-level cache, so every launch reads its
    inputs from HBM."""
    import torch
    lay = wl.layers[0]
    tensors = [lay.H0, lay.q, lay.k, lay.v, lay.gate]
    foot = sum(t.numel() * t.element_size() for t in tensors) + 4 * wl.total_nodes * wl.heads * wl.d_v
    n = int(min(max_sets, max(1, -(-rotate_bytes // foot))))
    g = lambda t: t.to(dev).clone()
    sets = []
    for _ in range(n):
        sets.append(dict(H0=g(lay.H0), q=g(lay.q), k=g(lay.k), v=g(lay.v), gate=g(lay.gate),
                         out=torch.empty((wl.total_nodes, wl.heads, wl.d_v), dtype=torch.float32,
                                         device=dev),
                         par=g(torch.from_numpy(wl.parent)), offs=g(torch.from_numpy(wl.node_offsets)),
                         ai=g(torch.from_numpy(wl.accepted_idx)), al=g(torch.from_numpy(wl.accepted_len))))
    return sets, foot


def time_rotated(fs, stream, reps=20, warm=2, min_launches=100, min_warm=20):
    """Median time of one launch (us): the launches `fs` (one per input set) run in turn
    under one event pair, `reps` times; each time is that span over len(fs). At least
    `min_launches` timed launches after at least `min_warm` untimed ones."""
    import numpy as np
    import torch
    reps = max(reps, -(-min_launches // len(fs)))
    warm = max(warm, -(-min_warm // len(fs)))
    for _ in range(warm):
        for f in fs:
            f()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        for f in fs:
            f()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 / len(fs) for a, b in evs]))


def probe_lib():
    """The memory-only reference kernels (libbole_probe.so, built with the library)."""
    import ctypes
    import os

    from tree_speculative_decoding_02_amd import bole
    path = os.path.join(os.path.dirname(bole.LIB_PATH), "libbole_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    common = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 5
    lib.probe_verify_traffic_scalar.argtypes = common + [ctypes.c_int, ctypes.c_void_p]
    lib.probe_verify_traffic_vector.argtypes = common + [ctypes.c_void_p]
    lib.probe_lazy_traffic_scalar.argtypes = ([ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4
                                              + [ctypes.c_int] * 7 + [ctypes.c_void_p])
    lib.probe_lazy_traffic_vector.argtypes = lib.probe_lazy_traffic_scalar.argtypes
    return lib


def lazy_traffic_launch(lib, layers, wl, parent_offs, acc_idx, acc_len, stream):
    """A launcher for the memory-only kernel that moves exactly the lazy step's bytes for
    the layer stack (the same stack, trees and paths; the previous step's tree is this
    step's, as in the benchmark), in the lazy launch's shape for scalar gates (d_k = 128,
    d_v = 64) or per-channel gates (d_k = d_v = 128). H0 is written back unchanged; out
    gets arbitrary values."""
    import ctypes

    class ProbeLayer(ctypes.Structure):
        _fields_ = [(n, ctypes.c_void_p) for n in ("H0", "q", "k", "v", "gate", "out", "prev_k",
                                                   "prev_v", "prev_gate")]
    arr = (ProbeLayer * len(layers))()
    for i, y in enumerate(layers):
        for n, _ in ProbeLayer._fields_:
            setattr(arr[i], n, y[n].data_ptr())
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = (arr, len(layers), P(parent_offs), P(parent_offs), P(acc_idx), P(acc_len), wl.batch,
            wl.heads, wl.d_k, wl.d_v, wl.total_nodes, wl.total_nodes, int(acc_idx.shape[1]),
            ctypes.c_void_p(stream.cuda_stream))

    probe = lib.probe_lazy_traffic_vector if wl.vector_gate else lib.probe_lazy_traffic_scalar

    def launch():
        rc = probe(*args)
        if rc != 0:
            raise RuntimeError(f"lazy traffic probe failed: {rc}")
    launch.keep = arr
    return launch


def traffic_reference(lib, wl, sets, stream, verify_us, nbytes, reps):
    """A memory-only launch that moves exactly the verify's bytes, in the same pieces, on
    the same cold input sets: the time this access pattern takes by itself. Scalar gates:
    the best of 1, 2 and 4 units per workgroup. None for shapes it does not take."""
    import ctypes

    import torch
    vec = bool(wl.vector_gate)
    if wl.layers[0].q.dtype != torch.bfloat16 or wl.d_k != 128 or wl.d_v != (128 if vec else 64):
        return None
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(stream.cuda_stream)

    def launch(x, nu):
        args = (P(x["H0"]), P(x["q"]), P(x["k"]), P(x["v"]), P(x["gate"]), P(x["out"]),
                P(x["offs"]), wl.batch, wl.heads, wl.d_k, wl.d_v, wl.total_nodes)
        rc = (lib.probe_verify_traffic_vector(*args, st) if vec
              else lib.probe_verify_traffic_scalar(*args, nu, st))
        if rc != 0:
            raise RuntimeError(f"traffic probe failed: {rc}")

    best = None
    for nu in ((1,) if vec else (1, 2, 4)):
        us = time_rotated([lambda x=x: launch(x, nu) for x in sets], stream, reps)
        if best is None or us < best[0]:
            best = (us, nu)
    us, nu = best
    return {"median_us": us, "GB_s": nbytes / (us * 1e3),
            "frac_hbm_peak": nbytes / (us * 1e3) / HBM_PEAK_GBS,
            "verify_rate_of_reference": us / verify_us,
            "units_per_workgroup": nu if not vec else 1,
            "what": "memory-only kernel moving the verify's bytes in the same row pieces "
                    "(no arithmetic), the same cold input sets"}


def config_sweep(dev, reps=20, configs=(1, 2, 3, 4, 5)):
    """Verify and commit on each workload, one layer. Each launch kind cycles through
    copies of the whole input set (sweep_sets: at least 512 MB per cycle), so every launch
    reads cold HBM. No flags: a caller without a known tree budget takes the general
    launch. Workloads whose trees have at most 32 nodes are also timed as a caller with
    that budget runs them (BOLE_FLAG_TREES_LE_32), under "verify_budget32"."""
    import numpy as np
    import torch

    import workloads as W
    from tree_speculative_decoding_02_amd import bole
    stream = torch.cuda.current_stream()
    plib = probe_lib()
    names = {1: "tiny_fp32", 2: "mamba2_scalar", 3: "gla_vector", 4: "ragged_large_batch",
             5: "hybrid_stack_one_layer"}
    for cid in configs:
        wl = W.make_config(cid, n_layers=1) if cid == 5 else W.make_config(cid)
        lay = wl.layers[0]
        sets, foot = sweep_sets(wl, dev)
        launches = {"verify": [bole.bind_tree_verify(x["H0"], x["q"], x["k"], x["v"], x["gate"],
                                                     x["par"], x["offs"], x["out"], stream=stream)
                               for x in sets],
                    "commit": [bole.bind_commit_path(x["H0"], x["k"], x["v"], x["gate"], x["par"],
                                                     x["offs"], x["ai"], x["al"], stream=stream)
                               for x in sets],
                    # one decode step in one call: the set's own path committed (as the
                    # previous step's) and its tree verified against the new state
                    "lazy": [bole.bind_tree_verify_lazy_commit(
                        x["H0"], (x["k"], x["v"], x["gate"], x["par"], x["offs"]), x["ai"],
                        x["al"], x["q"], x["k"], x["v"], x["gate"], x["par"], x["offs"], x["out"],
                        stream=stream) for x in sets]}
        s_f = 2 if lay.q.dtype == torch.bfloat16 else 4
        nbytes = {"verify": verify_bytes(wl, s_f), "commit": commit_bytes(wl, s_f),
                  "lazy": lazy_bytes(wl, s_f)}
        if int(np.diff(wl.node_offsets).max()) <= 32:
            launches["verify_budget32"] = [bole.bind_tree_verify(
                x["H0"], x["q"], x["k"], x["v"], x["gate"], x["par"], x["offs"], x["out"],
                stream=stream, trees_le_32=True) for x in sets]
            nbytes["verify_budget32"] = nbytes["verify"]
            launches["lazy_budget32"] = [bole.bind_tree_verify_lazy_commit(
                x["H0"], (x["k"], x["v"], x["gate"], x["par"], x["offs"]), x["ai"], x["al"],
                x["q"], x["k"], x["v"], x["gate"], x["par"], x["offs"], x["out"], stream=stream,
                trees_le_32=True, prev_trees_le_32=True) for x in sets]
            nbytes["lazy_budget32"] = nbytes["lazy"]
        rec = {"kind": "config_sweep", "config": cid, "workload": names[cid], "batch": wl.batch,
               "heads": wl.heads, "d_k": wl.d_k, "d_v": wl.d_v, "total_nodes": wl.total_nodes,
               "vector_gate": bool(wl.vector_gate), "factor_dtype": str(lay.q.dtype),
               "input_sets": len(sets), "bytes_per_set": foot}
        for name, fs in launches.items():
            us = time_rotated(fs, stream, reps)
            gbs = nbytes[name] / (us * 1e3)
            rec[name] = {"median_us": us, "bytes": nbytes[name], "GB_s": gbs,
                         "frac_hbm_peak": gbs / HBM_PEAK_GBS}
            if name.startswith("verify"):
                # draft nodes verified per second, every head of the layer
                rec[name]["nodes_per_s"] = wl.total_nodes / (us * 1e-6)
        ref = traffic_reference(plib, wl, sets, stream, rec["verify"]["median_us"],
                                nbytes["verify"], reps)
        if ref is not None:
            rec["verify_traffic_reference"] = ref
        if ref is not None:
            # the lazy step's bytes, moved by the memory-only kernel on the same sets
            lfs = [lazy_traffic_launch(plib, [dict(H0=x["H0"], q=x["q"], k=x["k"], v=x["v"],
                                                   gate=x["gate"], out=x["out"], prev_k=x["k"],
                                                   prev_v=x["v"], prev_gate=x["gate"])],
                                       wl, x["offs"], x["ai"], x["al"], stream) for x in sets]
            lus = time_rotated(lfs, stream, reps)
            lgbs = nbytes["lazy"] / (lus * 1e3)
            rec["lazy_traffic_reference"] = {
                "median_us": lus, "GB_s": lgbs, "frac_hbm_peak": lgbs / HBM_PEAK_GBS,
                "lazy_rate_of_reference": lus / rec["lazy"]["median_us"],
                "what": "memory-only kernel moving the lazy step's bytes (H0 read and written "
                        "back, path and tree rows, out) in the same row pieces"}
        print(json.dumps(rec), flush=True)
        del sets, launches
    if 3 in configs:
        vector_stack(dev, stream, reps)


def vector_stack(dev, stream, reps, n_layers=8):
    """8 layers of workload 3's shape (16 sequences x 16 heads, d_k = d_v = 128,
    per-channel gates, 64-node trees) sharing one tree per sequence: the verify stack and
    the lazy stack, one launch each (8 layers x 46 MB of inputs, read cold)."""
    import numpy as np
    import torch

    import workloads as W
    from tree_speculative_decoding_02_amd import bole
    wl = W.make_config(3)
    kw = dict(batch=wl.batch, heads=wl.heads, d_k=wl.d_k, d_v=wl.d_v,
              sizes=np.diff(wl.node_offsets).tolist(), kind="bestfirst", vector_gate=True)
    lays = [wl.layers[0]] + [W.make_random(5300 + l, **kw).layers[0] for l in range(n_layers - 1)]
    g = lambda t: t.to(dev)
    par, offs = g(torch.from_numpy(wl.parent)), g(torch.from_numpy(wl.node_offsets))
    ai, al = g(torch.from_numpy(wl.accepted_idx)), g(torch.from_numpy(wl.accepted_len))
    layers = []
    for l in lays:
        y = dict(H0=g(l.H0), q=g(l.q), k=g(l.k), v=g(l.v), gate=g(l.gate),
                 out=torch.empty((wl.total_nodes, wl.heads, wl.d_v), dtype=torch.float32,
                                 device=dev))
        y.update(prev_k=y["k"], prev_v=y["v"], prev_gate=y["gate"])
        layers.append(y)
    fv = bole.bind_tree_verify_layers(layers, par, offs, stream=stream)
    fl = bole.bind_tree_verify_lazy_commit_layers(layers, par, offs, ai, al, par, offs,
                                                  stream=stream)
    rec = {"kind": "vector_stack", "workload": "gla_vector x 8 layers", "layers": n_layers,
           "batch": wl.batch, "heads": wl.heads, "d_k": wl.d_k, "d_v": wl.d_v,
           "total_nodes": wl.total_nodes}
    for name, f, nb in (("verify", fv, verify_bytes(wl)), ("lazy", fl, lazy_bytes(wl))):
        us = time_rotated([f] * 4, stream, reps)
        gbs = n_layers * nb / (us * 1e3)
        rec[name] = {"median_us": us, "bytes": n_layers * nb, "GB_s": gbs,
                     "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                     "nodes_per_s": n_layers * wl.total_nodes / (us * 1e-6)}
    # the stack's lazy-step bytes moved by the memory-only kernel, one launch of 8 layers
    lref = lazy_traffic_launch(probe_lib(), layers, wl, offs, ai, al, stream)
    lus = time_rotated([lref] * 4, stream, reps)
    lgbs = rec["lazy"]["bytes"] / (lus * 1e3)
    rec["lazy_traffic_reference"] = {
        "median_us": lus, "GB_s": lgbs, "frac_hbm_peak": lgbs / HBM_PEAK_GBS,
        "lazy_rate_of_reference": lus / rec["lazy"]["median_us"],
        "what": "memory-only kernel moving the lazy stack's bytes in the same row pieces"}
    print(json.dumps(rec), flush=True)


def cpu_baseline(wl, min_seconds):
    """The fp64 CPU oracle (serial walk per node) on the same workload: verify of every
    layer, then commit of every layer, as one step. Run with every core of this process's
    affinity set and with one thread, three samples each, the median reported. All-core
    samples are whole steps, repeated to about min_seconds / 6 each; one-thread samples
    are one layer each, scaled to a step (layers are alike in cost). Inputs are widened to
    fp64 before the clock starts."""
    import numpy as np

    import oracle
    L = len(wl.layers)
    lays = [[oracle.f64(t) for t in (l.H0, l.q, l.k, l.v, l.gate)] for l in wl.layers]

    def step(layers):
        for H0, q, k, v, gate in layers:
            oracle.verify_serial(H0, q, k, v, gate, wl.parent, wl.node_offsets, False)
        for H0, q, k, v, gate in layers:
            oracle.commit_serial(H0, k, v, gate, wl.parent, wl.node_offsets, wl.accepted_idx,
                                 wl.accepted_len, False)

    cores = len(os.sched_getaffinity(0))
    out = {}
    for threads in (cores, 1):
        oracle.set_threads(threads)
        used = oracle.threads()
        samples, total = [], 0.0
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                step(lays if threads > 1 else lays[:1])
                reps += 1
                el = time.perf_counter() - t0
                if threads == 1 or el >= min_seconds / 6:
                    break
            total += el
            samples.append(el / reps * (1 if threads > 1 else L))
        out[threads] = (float(np.median(samples)), used, total)
    oracle.set_threads(cores)
    t_all, used_all, s_all = out[cores]
    t_one, _, s_one = out[1]
    return {"value": wl.total_nodes / t_all, "unit": "draft nodes/s", "cores": used_all,
            "kind": "oracle",
            "sample": f"verify + commit of {L} layers ({wl.total_nodes} nodes x {wl.heads} "
                      f"heads per layer), fp64: median of 3 samples of whole steps on "
                      f"{used_all} threads ({s_all:.1f} s in all), and of 3 one-layer samples "
                      f"on 1 thread scaled to a step ({s_one:.1f} s in all)",
            "ms_per_step": 1e3 * t_all,
            "one_thread": {"value": wl.total_nodes / t_one, "ms_per_step": 1e3 * t_one},
            "affinity_cores": cores}


if __name__ == "__main__":
    main()
