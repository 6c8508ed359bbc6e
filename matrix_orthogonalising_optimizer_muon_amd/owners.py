"""Owner assignment over ranks from measured per-shape costs (argument marshalling over
``muon_prepare`` and ``muon_owner_plan``; every measurement and the search run in the
library).

DMuon summary (gist.science), section 2.3: at initialisation the update time of several
batch sizes is measured for each distinct matrix shape, and each matrix gets one owner rank
so that the predicted makespan is least. ``measure_shape_costs`` times synthetic updates
(``muon_prepare``: W, G and M are not needed) of k same-shape matrices for the given batch
sizes; ``plan_owners`` hands the table to the planner.

Run as a module to print the plan of a workload for several rank counts, e.g.
``python -m matrix_orthogonalising_optimizer_muon_amd.owners --workload dense_7b_28layers
--ranks 2 4 8`` (one GPU measures; the plan is for N ranks of the same GPU type).
"""

from __future__ import annotations

import argparse
import json
import sys

from . import binding as B


def canonical(rows: int, cols: int) -> tuple:
    return (min(rows, cols), max(rows, cols))


def default_batches(n: int) -> list:
    """1, 2, 4, ... below n, then n itself."""
    out, b = [], 1
    while b < n:
        out.append(b)
        b *= 2
    out.append(n)
    return out


def measure_shape_costs(ctx, shapes: dict, hp, batches=None, stream_ptr=None) -> dict:
    """{(m, n): [(batch, ms), ...]} for every canonical shape in ``shapes`` (shape ->
    matrices in the list), one synthetic update of ``batch`` matrices per point."""
    import torch

    costs = {}
    for shape, count in shapes.items():
        pts = []
        sizes = batches(count) if callable(batches) else (list(batches) if batches else default_batches(count))
        for b in sizes:
            raw = [(0, 0, 0, shape[0], shape[1])] * b
            nbytes = B.muon_workspace_size(ctx, raw, hp)
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            ms = B.muon_prepare(ctx, raw, hp, ws.data_ptr(), nbytes, stream_ptr)
            pts.append((b, ms))
            del ws
            print(f"[owners] {shape[0]}x{shape[1]} batch {b}: {ms:.3f} ms", file=sys.stderr, flush=True)
        costs[shape] = pts
    return costs


def plan_owners(matrix_shapes: list, costs: dict, ranks: int, greedy: bool = False, max_nodes: int = 0) -> dict:
    """Plan for a list of (rows, cols); ``costs`` as from ``measure_shape_costs``."""
    keys = sorted(costs)
    index = {k: i for i, k in enumerate(keys)}
    shape_of = [index[canonical(r, c)] for r, c in matrix_shapes]
    out = B.muon_owner_plan(shape_of, [costs[k] for k in keys], ranks, greedy=greedy, max_nodes=max_nodes)
    out["shapes"] = [f"{k[0]}x{k[1]}" for k in keys]
    return out


def round_robin_makespan(matrix_shapes: list, costs: dict, ranks: int) -> float:
    """Predicted makespan of owner i mod N under the same cost model (the naive plan the
    pages compare against), computed by the planner itself on the fixed assignment: each
    rank's load is the planned load of a one-rank problem over its matrices."""
    loads = []
    for r in range(ranks):
        mine = [s for i, s in enumerate(matrix_shapes) if i % ranks == r]
        loads.append(plan_owners(mine, costs, 1)["makespan_ms"] if mine else 0.0)
    return max(loads)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="dense_7b_28layers")
    ap.add_argument("--ranks", type=int, nargs="+", default=[2, 4, 8])
    ap.add_argument("--mode", default="auto")
    args = ap.parse_args()
    import torch

    from . import workloads as wl
    w = wl.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    ctx = B.muon_init(0)
    hp = B.make_hparams(lr=w.lr, momentum=w.mu, weight_decay=w.wd, mode=args.mode, w_dtype=w.w_dtype,
                        g_dtype=w.g_dtype, m_dtype=w.m_dtype, ns_dtype=w.ns_dtype)
    mshapes = [(s.rows, s.cols) for s in w.matrices]
    shapes = {}
    for r, c in mshapes:
        shapes[canonical(r, c)] = shapes.get(canonical(r, c), 0) + 1
    costs = measure_shape_costs(ctx, shapes, hp)
    result = {"workload": w.name, "costs_ms": {f"{k[0]}x{k[1]}": v for k, v in costs.items()}, "plans": {}}
    for n in args.ranks:
        p = plan_owners(mshapes, costs, n)
        result["plans"][n] = {"makespan_ms": round(p["makespan_ms"], 3), "optimal": p["optimal"],
                              "rank_ms": [round(x, 3) for x in p["rank_ms"]],
                              "round_robin_ms": round(round_robin_makespan(mshapes, costs, n), 3),
                              "one_rank_ms": round(plan_owners(mshapes, costs, 1)["makespan_ms"], 3)}
    B.muon_destroy(ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
