"""Per-workload parity record: every workload at full size through the library, every sequence,
tree or sampler row compared with the oracle (tests/parity.py), and the band counts written out.

    python tests/record_parity.py [--out profiles/parity_bands.md]

For each workload it prints one JSON line: the rows checked, how many matched the oracle exactly,
how many fell inside the accept band (|u - min(1, p/q)| < 1e-6, the Speculative Sampling
explainer's Step 3 test) or the edge band (u * W within 1e-6 * W of a bucket edge of the
inverse-CDF draw, modified rejection sampling), how many took the fallback, and how many band
rows the GPU resolved differently from the oracle's own outcome (always inside the allowed set,
or the script stops with the mismatch).  The band counts are a property of the inputs and the
oracle; band_differs is the GPU's.  Test infrastructure: it calls only the oracle (through
tests/parity.py) and the library (through the binding), on the calls the benchmark makes.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (HERE, ROOT):
    if p not in sys.path:
        sys.path.insert(0, p)

# (kind, workload, entry-point options)
RECORDS = [
    ("chain", "gauss_b1_g4_v1000_f32", {}),
    ("chain", "gauss_b1_g4_v32000_bf16", {}),
    ("chain", "gauss_b1_g5_v32000_bf16", {}),
    ("chain", "gauss_b1_g6_v32000_bf16", {}),
    ("chain", "gauss_b1_g7_v32000_bf16", {}),
    ("chain", "zipf_b64_g4_v128256_bf16", {}),
    ("chain", "gauss_b256_g7_v152064_f32", {}),
    ("chain", "gauss_b256_g7_v152064_f32", {"lazy": True}),
    ("tree", "tree_16x64_v32000_bf16", {}),
    ("sample", "sample_b256_v152064_f32", {}),
    ("sample", "sample_b64_v128256_bf16", {}),
]


def record(kind, name, opts):
    import torch

    from parity import chain_refs, check_chain, check_sample, check_tree
    from rejection_sampling_verify_chain_amd import binding as BD
    from rejection_sampling_verify_chain_amd import inputs as I

    def host(out):
        torch.cuda.synchronize()
        return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}

    t0 = time.perf_counter()
    if kind == "chain":
        b = I.CHAIN_WORKLOADS[name]()
        d = BD.chain_to_device(b)
        out = host(BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                      d["temperature"], **opts))
        counts = check_chain(b, out, lazy=bool(opts.get("lazy")), refs=chain_refs(b))
        n = b.B
        unit = "sequences"
    elif kind == "tree":
        b = I.TREE_WORKLOADS[name]()
        d = BD.tree_to_device(b)
        out = host(BD.sv_verify_tree(d["logits"], d["parents"], d["node_tokens"]))
        ks = check_tree(b, out)
        n = len(ks)
        counts = {"exact": n, "accept_band": 0, "edge_band": 0, "fallback": 0, "band_differs": 0,
                  "accepted_per_tree": ks}
        unit = "trees"
    else:
        b = I.SAMPLE_WORKLOADS[name]()
        d = BD.sample_to_device(b)
        out = host(BD.sv_sample(d["logits"], d["temperature"], d["uniforms"]))
        counts = check_sample(b, out)
        counts["accept_band"] = 0
        n = b.rows
        unit = "rows"
    entry = {"chain": "sv_verify_chain_lazy" if opts.get("lazy") else "sv_verify_chain",
             "tree": "sv_verify_tree", "sample": "sv_sample"}[kind]
    return {"workload": name, "entry_point": entry, "checked": n, "unit": unit,
            "mismatches": 0, **counts, "seconds": round(time.perf_counter() - t0, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=None, help="also write the records as a markdown summary")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("record_parity.py needs a GPU")
    from rejection_sampling_verify_chain_amd import binding as BD
    lines = []
    for kind, name, opts in RECORDS:
        print(f"[record] {kind} {name} {opts}", file=sys.stderr, flush=True)
        rec = record(kind, name, opts)
        lines.append(rec)
        print(json.dumps(rec), flush=True)
    if args.out:
        cmd = "python tests/record_parity.py --out " + args.out
        with open(args.out, "w") as f:
            f.write("# Parity against the oracle, per workload, with band counts\n\n")
            f.write(f"Command: `{cmd}` ({BD.version()}, {torch.cuda.get_device_name(0)}).\n\n")
            f.write("Every sequence (tree, sampler row) of each workload at full size, through the "
                    "entry point the benchmark calls, against the oracle. Band rows are "
                    "counted, not excluded: each must lie in its allowed set.\n\n")
            f.write("| workload | entry point | checked | exact | accept band | edge band | "
                    "fallback | band rows resolved differently | mismatches |\n")
            f.write("|---|---|---|---|---|---|---|---|---|\n")
            for r in lines:
                f.write(f"| {r['workload']} | `{r['entry_point']}` | {r['checked']} {r['unit']} | "
                        f"{r['exact']} | {r['accept_band']} | {r['edge_band']} | "
                        f"{r['fallback']} | {r['band_differs']} | {r['mismatches']} |\n")
            f.write("\nRecords:\n\n```\n")
            for r in lines:
                f.write(json.dumps(r) + "\n")
            f.write("```\n")


if __name__ == "__main__":
    main()
