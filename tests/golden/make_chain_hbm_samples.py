"""Writes chain_hbm_samples.json: seeded entries of OzII-RescaleBE chains
with large tensor sides (n = 128, batch 2; n = 256, batch 1; s = 16, depth
3, the directions in turn), computed by the CPU oracle (oracle/rescale_be.py,
"You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products",
Algorithm 7) from the seeded inputs of workloads.py.  Only the oracle and the
input generators are called.  Run from the repository root:

    python tests/golden/make_chain_hbm_samples.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import rescale_be as rb  # noqa: E402

CASES = [
    # n, s, batch, operator seed, tensor seed, sampled entries per tensor
    (128, 16, 2, 9700, 9701, 1024),
    (256, 16, 1, 9800, 9801, 2048),
]


def main():
    out = []
    for n, s, batch, ops_seed, x_seed, per in CASES:
        t0 = time.time()
        ops = [workloads.real_matrix(n, n, ops_seed + q) for q in range(3)]
        X = workloads.tensor_batch(n, batch, x_seed)
        plan = rb.prepare_chain(ops, n, s)
        n3 = n ** 3
        rng = np.random.default_rng(x_seed + 1)
        index, value = [], []
        for t in range(batch):
            Y = rb.chain_tensor(X[t * n3:(t + 1) * n3], plan)
            picks = np.unique(np.concatenate([[0, n3 - 1], rng.choice(n3, per, replace=False)]))
            index += [int(t * n3 + i) for i in picks]
            value += [float(Y[i]).hex() for i in picks]
        out.append(dict(n=n, s=s, batch=batch, ops_seed=ops_seed, x_seed=x_seed, b=plan["b"], g=plan["g"],
                        index=index, value=value))
        print(f"n={n}: b={plan['b']} g={plan['g']} {len(index)} entries, {time.time() - t0:.0f} s", flush=True)
    doc = dict(source="oracle/rescale_be.py chain_tensor (Algorithm 7 of the chain page)",
               inputs="workloads.real_matrix(n, n, ops_seed + q) for q = 0, 1, 2; workloads.tensor_batch(n, batch, x_seed)",
               cases=out)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "chain_hbm_samples.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
