"""Pre-token statistics of a workload's encode input, from the oracle: per
4 KiB chunk (the encode's unit of work), the pre-tokens that start in it,
the share that run the merge loop (not a single byte and not one whole
token), what those are, and the merges each takes.

    python tests/workload_stats.py [workload] [n_docs]

A pre-token "hits" when it is a single byte or when the oracle encodes it to
one token of at most 24 bytes (the load-time word tables hold exactly such
tokens); every other pre-token is a merge-loop entry.  Test infrastructure:
it runs the oracle only.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from workloads import WORKLOADS, encode_batch_input, make_lexicon  # noqa: E402


def main(argv):
    name = argv[0] if argv else "throughput"
    n_docs = int(argv[1]) if len(argv) > 1 else 64
    cfg = WORKLOADS[name]
    batch = encode_batch_input(cfg, make_lexicon(cfg), n_docs=n_docs)
    table = O.Table(np.load(os.path.join(ROOT, "assets", f"merges_{name}.npy")))
    n_pt = 0
    kinds = {"lower": 0, "capital": 0, "digits": 0, "other": 0}
    misses = merges = 0
    lengths = []
    for d in range(batch.n_docs):
        doc = batch.data[batch.doc_off[d]:batch.doc_off[d + 1]].tobytes()
        for w in O.split(doc):
            n_pt += 1
            lengths.append(len(w))
            if len(w) == 1:
                continue
            t = table.encode_word(w)
            if len(t) == 1 and len(w) <= 24:
                continue
            misses += 1
            merges += len(w) - len(t)
            core = w[1:] if w[:1] == b" " else w
            if core.isdigit():
                kinds["digits"] += 1
            elif core[:1].isupper():
                kinds["capital"] += 1
            elif core.isalpha() and core.islower():
                kinds["lower"] += 1
            else:
                kinds["other"] += 1
    chunks = batch.n_bytes / 4096
    print(f"{name}: {batch.n_docs} documents, {batch.n_bytes} bytes")
    print(f"pre-tokens per 4 KiB chunk: {n_pt / chunks:.1f} (mean length {np.mean(lengths):.2f} bytes)")
    print(f"merge-loop entries: {100 * misses / n_pt:.1f}% of pre-tokens "
          f"({misses / chunks:.1f} per chunk), {merges / max(1, misses):.2f} merges each")
    print("of which: " + ", ".join(f"{k} {100 * v / max(1, misses):.0f}%" for k, v in kinds.items()))


if __name__ == "__main__":
    main(sys.argv[1:])
