"""Graph-replayed timing of table entries on given shapes (factory tuning).

    python -m dense_mixed_precision_amd.sweep --shapes 512x512,1024x2048 --ks 256,2048,8192 \\
        --configs 35,36,41 [--candidates] [--rounds 5] [--in f16|bf16] [--layout rr|cr|rc|cc]
    python -m dense_mixed_precision_amd.sweep --triples 5907x1622x137,652x11198x66 --configs 3,5,6
    python -m dense_mixed_precision_amd.sweep --triples 256x256x8192 --splits 0,1,4,8,16,32

For every M x N x K it captures, per forced table entry, a HIP graph of
back-to-back launches of that entry (FP16 or BF16 operands, each row- or
column-major, uniform inputs, alpha 1, beta 0), replays the graphs in
alternating rounds and
prints one line per shape: the median per-launch time of each entry, the
factory's own choice and the fastest entry.  With ``--splits`` the variants
are split-K piece counts instead (0: the automatic plan, 1: one piece),
each launched through the split-K entry with a workspace of its plan's size.  Launch overhead on the host is
outside the graphs, so microsecond-scale kernels are timed as the GPU runs
them back to back.
"""
from __future__ import annotations

import argparse
import itertools
import json


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--shapes", help="comma-separated MxN pairs (with --ks)")
    p.add_argument("--ks", help="comma-separated K values (with --shapes)")
    p.add_argument("--triples", help="comma-separated MxNxK products (instead of --shapes and --ks)")
    p.add_argument("--configs", help="comma-separated table entries to force")
    p.add_argument("--splits", help="comma-separated split-K piece counts to force (instead of --configs)")
    p.add_argument("--candidates", action="store_true", help="load the candidates build")
    p.add_argument("--rounds", type=int, default=5)
    p.add_argument("--seed", type=int, default=7)
    p.add_argument("--in", dest="in_type", choices=("f16", "bf16"), default="f16", help="input format")
    p.add_argument("--layout", choices=("rr", "cr", "rc", "cc"), default="rr",
                   help="storage orders of A and B (r: row-major, c: column-major)")
    return p.parse_args()


def main():
    args = parse()
    import torch

    import dense_mixed_precision_amd as mp
    from dense_mixed_precision_amd.workloads import make_inputs

    mp.load(mp.CANDIDATES_PATH if args.candidates else None)
    dev = torch.device("cuda:0")
    if args.triples:
        products = [tuple(int(x) for x in t.split("x")) for t in args.triples.split(",")]
    elif args.shapes and args.ks:
        shapes = [tuple(int(x) for x in s.split("x")) for s in args.shapes.split(",")]
        ks = [int(k) for k in args.ks.split(",")]
        products = [(M, N, K) for (M, N), K in itertools.product(shapes, ks)]
    else:
        raise SystemExit("give --triples, or --shapes and --ks")
    if bool(args.configs) == bool(args.splits):
        raise SystemExit("give one of --configs and --splits")
    cfgs = [int(c) for c in (args.configs or args.splits).split(",")]
    for M, N, K in products:
        dtype = torch.bfloat16 if args.in_type == "bf16" else torch.float16
        A, B, _ = make_inputs(M, N, K, "uniform", seed=args.seed, dtype=dtype)
        # a column-major operand is stored transposed and passed as the transposed view
        A = A.t().contiguous().to(dev).t() if args.layout[0] == "c" else A.to(dev)
        B = B.t().contiguous().to(dev).t() if args.layout[1] == "c" else B.to(dev)
        C = torch.empty(M, N, device=dev)
        if args.splits:
            factory = 0
            plans = {c: mp.splitk_plan_for(A, B, C, c) for c in cfgs}
            ws = {c: torch.empty(max(plans[c]["workspace_bytes"] // 4, 1), device=dev) for c in cfgs}

            def launch(c):
                mp.gemm_splitk(A, B, C, 1.0, 0.0, splits=c, workspace=ws[c])
        else:
            factory = mp.query_for(A, B, C)["id"]

            def launch(c):
                mp.gemm(A, B, C, 1.0, 0.0, config=c)
        # about 0.4 ms of work per graph at 1 PFLOP/s, 4..40 launches
        per = max(4, min(40, int(4e5 / (2 * M * N * K / 1e6 + 1))))
        side = torch.cuda.Stream()
        graphs = {}
        for c in cfgs:
            with torch.cuda.stream(side):
                for _ in range(2):
                    launch(c)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(per):
                    launch(c)
            graphs[c] = g
        torch.cuda.synchronize()
        times = {c: [] for c in cfgs}
        for _ in range(args.rounds):
            for c in cfgs:
                graphs[c].replay()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                graphs[c].replay()
                e1.record()
                torch.cuda.synchronize()
                times[c].append(e0.elapsed_time(e1) * 1e3 / per)
        med = {c: sorted(v)[len(v) // 2] for c, v in times.items()}
        best = min(med, key=med.get)
        line = {"M": M, "N": N, "K": K, "factory": factory, "best": best,
                "factory_over_best": round(med[factory] / med[best], 3) if factory in med else None,
                "us": {str(c): round(v, 3) for c, v in med.items()}}
        if args.splits:
            line["pieces"] = {str(c): plans[c]["splits"] for c in cfgs}
            line["config"] = {str(c): plans[c]["config_id"] for c in cfgs}
            del ws
        print(json.dumps(line), flush=True)
        del graphs, A, B, C


if __name__ == "__main__":
    main()
