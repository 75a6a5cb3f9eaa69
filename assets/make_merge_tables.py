"""Write the merge tables for the five workloads.

Each table is the oracle trainer's output (most frequent pair first, ties to
the smallest pair, stop at the workload's merge count or when no pair occurs
twice) on the workload's seeded training corpus.  The tables are model
assets, like a shipped merges file: the GPU library only loads them.

    python assets/make_merge_tables.py [workload ...]

writes assets/merges_<workload>.npy (int32 [R, 2], rank order) and refreshes
assets/SHA256SUMS.  Only the oracle and the workload generator run here.
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle as O  # noqa: E402
from workloads import WORKLOADS, make_lexicon, training_corpus  # noqa: E402


def table_path(name: str) -> str:
    return os.path.join(HERE, f"merges_{name}.npy")


def main(argv):
    ks = list(argv) or list(WORKLOADS)
    for k in ks:
        cfg = WORKLOADS[k]
        t0 = time.time()
        tc = training_corpus(cfg, make_lexicon(cfg))
        merges, counts = O.train(tc.data, tc.doc_off, cfg.n_merges)
        np.save(table_path(k), merges.astype(np.int32), allow_pickle=False)
        print(f"{k}: {merges.shape[0]} merges (asked {cfg.n_merges}), "
              f"last count {counts[-1] if counts.size else None}, {time.time() - t0:.1f}s", flush=True)
    with open(os.path.join(HERE, "SHA256SUMS"), "w") as f:
        for k in WORKLOADS:
            p = table_path(k)
            if os.path.exists(p):
                f.write(f"{hashlib.sha256(open(p, 'rb').read()).hexdigest()}  merges_{k}.npy\n")


if __name__ == "__main__":
    main(sys.argv[1:])
