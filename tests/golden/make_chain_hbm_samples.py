"""Writes chain_hbm_samples.json: seeded entries of OzII-RescaleBE chains
with large tensor sides, computed by the CPU oracle (oracle/rescale_be.py,
"You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products",
Algorithm 7) from the seeded inputs of workloads.py.  Only the oracle and the
input generators are called.  The sides cover the product kernels' staged
form with 2, 3 and 4 pairs of k chunks (n = 100, 128, 136, 200, 256), other
mode orders than the directions in turn, and (n = 256) blocks of 8
wavefronts.  A case already in the file with the same parameters is kept,
not recomputed.  Run from the repository root:

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
    # n, s, batch, operator seed, tensor seed, sampled entries per tensor,
    # directions of the products (1-based; None: 1, 2, 3 in turn)
    (128, 16, 2, 9700, 9701, 1024, None),
    (256, 16, 1, 9800, 9801, 2048, None),
    (100, 12, 2, 9900, 9901, 1024, None),
    (100, 12, 1, 9905, 9906, 1024, [2, 2, 1, 3]),
    (136, 15, 1, 9910, 9911, 1024, None),
    (200, 10, 1, 9920, 9921, 1024, [3, 1, 2]),
]
PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "chain_hbm_samples.json")
KEYS = ("n", "s", "batch", "ops_seed", "x_seed", "per", "modes")


def _key(n, s, batch, ops_seed, x_seed, per, modes):
    return (n, s, batch, ops_seed, x_seed, per, None if modes is None else tuple(modes))


def main():
    old = {}
    if os.path.exists(PATH):
        with open(PATH) as f:
            for c in json.load(f)["cases"]:
                old[_key(*(c.get(k) for k in KEYS))] = c
    out = []
    for n, s, batch, ops_seed, x_seed, per, modes in CASES:
        key = _key(n, s, batch, ops_seed, x_seed, per, modes)
        if key in old:
            out.append(old[key])
            print(f"n={n} modes={modes}: kept", flush=True)
            continue
        t0 = time.time()
        d = 3 if modes is None else len(modes)
        ops = [workloads.real_matrix(n, n, ops_seed + q) for q in range(d)]
        X = workloads.tensor_batch(n, batch, x_seed)
        plan = rb.prepare_chain(ops, n, s, None if modes is None else [m - 1 for m in modes])
        n3 = n ** 3
        rng = np.random.default_rng(x_seed + 1)
        index, value = [], []
        for t in range(batch):
            Y = rb.chain_tensor(X[t * n3:(t + 1) * n3], plan)
            picks = np.unique(np.concatenate([[0, n3 - 1], rng.choice(n3, per, replace=False)]))
            index += [int(t * n3 + i) for i in picks]
            value += [float(Y[i]).hex() for i in picks]
        out.append(dict(n=n, s=s, batch=batch, ops_seed=ops_seed, x_seed=x_seed, per=per, modes=modes,
                        b=plan["b"], g=plan["g"], index=index, value=value))
        print(f"n={n} modes={modes}: b={plan['b']} g={plan['g']} {len(index)} entries, {time.time() - t0:.0f} s",
              flush=True)
    doc = dict(source="oracle/rescale_be.py chain_tensor (Algorithm 7 of the chain page)",
               inputs="workloads.real_matrix(n, n, ops_seed + q) for q = 0 .. d - 1; "
                      "workloads.tensor_batch(n, batch, x_seed)",
               cases=out)
    with open(PATH, "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
