"""Write tests/golden/chain64_dag.txt: the 64-node random elementwise chain.

The generic pointwise workload is a seeded random DAG of 64 elementwise nodes
(add, mul, exp, gelu, sqrt of abs, tanh, pow2; about a fifth of the values
read twice) over three f32 inputs A [16384,16384], B [16384,1], C [1,16384],
values U(-1,1).  The structure is drawn by ``synth.dag.random_chain_dag``;
this script keeps the first seed whose DAG is well posed, judged by the
oracle alone:

  (i)  interval arithmetic over inputs in [-1, 1] keeps every node within
       [-1e4, 1e4], so no value can overflow or turn into NaN;
  (ii) on 2^20 elements (64 sampled rows of the full-size inputs) the f32
       oracle stays within a quarter of the parity tolerance
       (1e-7 + 2e-6 |ref|) of a float64 evaluation of the same DAG, so the
       chain is conditioned well enough for that tolerance.

Run:  python tests/golden/make_chain64_dag.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import configs  # noqa: E402
from synth.dag import format_dag, random_chain_dag  # noqa: E402

N = 16384
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "chain64_dag.txt")


def sample_inputs(rows):
    A, B, C = configs.chain_inputs(N, N)
    A, B, C = A.numpy(), B.numpy(), C.numpy()
    return np.ascontiguousarray(A[rows]), np.ascontiguousarray(B[rows]), C


def accept(nodes, inputs):
    bounds = oracle.interval_bounds(nodes, [(-1.0, 1.0)] * 3)
    worst = max(max(abs(lo), abs(hi)) for lo, hi in bounds)
    if worst > 1e4:
        return False, f"interval bound {worst:.3g}"
    A, B, C = inputs
    got = oracle.eval_group(nodes, [A, B, C], A.shape).astype(np.float64)
    ref = oracle.eval_group_f64(nodes, [A, B, C], A.shape)
    slack = np.abs(got - ref) / (1e-7 + 2e-6 * np.abs(ref))
    if not np.all(np.isfinite(got)) or slack.max() > 0.25:
        return False, f"f32 vs f64 slack {slack.max():.3g}"
    return True, f"interval bound {worst:.3g}, f32 vs f64 worst {slack.max():.3f} of tolerance"


def main():
    rows = np.random.default_rng(configs.CHAIN_DAG_SEED).choice(N, 64, replace=False)
    rows.sort()
    inputs = sample_inputs(rows)
    seed = configs.CHAIN_DAG_SEED
    for k in range(2000):
        nodes = random_chain_dag(seed + k)
        ok, why = accept(nodes, inputs)
        print(f"seed {seed + k}: {'accept' if ok else 'reject'} ({why})", flush=True)
        if ok:
            twice = sum(1 for i in range(len(nodes)) if sum(a == i for nd in nodes for a in nd.args) == 2)
            with open(OUT, "w") as f:
                f.write(f"# 64-node elementwise chain over A [16384,16384], B [16384,1], C [1,16384]\n")
                f.write(f"# drawn by synth.dag.random_chain_dag(seed={seed + k}); {twice} values read twice\n")
                f.write(f"# accepted by tests/golden/make_chain64_dag.py: {why}\n")
                f.write(format_dag(nodes))
            print("wrote", OUT)
            return
    raise SystemExit("no seed accepted")


if __name__ == "__main__":
    main()
