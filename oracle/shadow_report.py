"""Disagreement counts between the binary32 reading and the exact-quotient readings.

Runs the oracle's shadow comparison (oracle.shadow_compare) over the five synthetic
workloads at full size, for every run each workload lists, with alpha rounded to
binary32 ("after alpha") and with alpha = amax / (6*M) exact ("fully exact"), and
prints one table row per run.  Test infrastructure: it calls only the oracle and
the input generators.

    python -m oracle.shadow_report [--threads N] [--workloads tiny,weight,...]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from nvfp4_block_scaled_amax_amd import workloads as W  # noqa: E402

# the runs of each workload, plus rtn6 where the workload lists only Four Over Six
EXTRA = {"act": (("rtn6", "mse", "fakequant"),), "moe": (("rtn6", "mse", "packed"),)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--workloads", default="tiny,weight,act,large,moe")
    args = ap.parse_args()
    cols = ("blocks", "block_diff", "code_diff", "scale_diff", "choice_diff", "y_diff",
            "exact_ties", "inexact")
    print("| workload | mode / rule | alpha | " + " | ".join(cols) + " |")
    print("|" + "---|" * (3 + len(cols)))
    for name in args.workloads.split(","):
        wl = W.WORKLOADS[name]
        x = W.bits(W.generate(name))
        for mode, rule, _ in wl.runs + EXTRA.get(name, ()):
            for exact_alpha in (False, True):
                t0 = time.time()
                c = oracle.shadow_compare(x, mode, rule, exact_alpha, nthreads=args.threads)
                print("| %s | %s | %s | %s |" % (
                    name, mode if mode == "rtn6" else "4/6 " + rule,
                    "fully exact" if exact_alpha else "after alpha",
                    " | ".join(str(c[k]) for k in cols)), flush=True)
                print("  (%.1f s)" % (time.time() - t0), file=sys.stderr, flush=True)
        del x


if __name__ == "__main__":
    main()
