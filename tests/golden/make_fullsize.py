"""Write tests/golden/fullsize.json: the oracle's whole-batch encode of every
workload, as the token count T and two 64-bit FNV-1a checksums.

For each workload the script generates the full encode input with the seeded
generator (``workloads``), loads the workload's merge table from ``assets/``,
encodes every document with the oracle (``oracle``, the plain C encoder) and
records

    T                T = id_off[n_docs], the number of IDs of the batch
    ids_fnv1a64      FNV-1a 64 over the IDs as little-endian int32, in order
    id_off_fnv1a64   FNV-1a 64 over id_off[0..n_docs] as little-endian int64

(the benchmark protocol of "Hugging Face Tokenizers v1: encoding up to 30x
faster", section "Benchmarks", checks a run by the FNV-1a of its output IDs;
the checksum over the offsets extends that to the document boundaries).

Documents are independent (a merge never crosses a pre-token, and every
document start is a pre-token start), so the documents are split into
contiguous shards that worker processes encode with the oracle's batch call;
the shards' IDs are joined in document order and their offsets shifted by the
IDs before them.  Nothing but the oracle and the generator runs here.

    python tests/golden/make_fullsize.py [workload ...] [--procs N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from workloads import WORKLOADS, encode_batch_input, make_lexicon  # noqa: E402

OUT = os.path.join(HERE, "fullsize.json")

# set in the parent before the workers fork, read by them
_BATCH = None
_MERGES = None


def merges_path(name: str) -> str:
    return os.path.join(ROOT, "assets", f"merges_{name}.npy")


def _encode_shard(span):
    d0, d1 = span
    data, doc_off = _BATCH
    a, b = int(doc_off[d0]), int(doc_off[d1])
    table = O.Table(_MERGES)
    ids, off = table.encode_batch(data[a:b], doc_off[d0:d1 + 1] - a)
    return d0, ids, off


def oracle_encode_all(data: np.ndarray, doc_off: np.ndarray, merges: np.ndarray, procs: int):
    """The oracle's IDs and offsets for the whole batch, shard by shard."""
    global _BATCH, _MERGES
    _BATCH, _MERGES = (data, doc_off), merges
    D = doc_off.size - 1
    # shards of about equal bytes, at most 64 per process
    n_sh = max(1, min(D, 64 * procs))
    cuts = np.searchsorted(doc_off, np.linspace(0, data.size, n_sh + 1)[1:-1]).tolist()
    bounds = sorted(set([0] + [int(c) for c in cuts if 0 < c < D] + [D]))
    spans = list(zip(bounds[:-1], bounds[1:]))
    parts = {}
    if procs > 1 and len(spans) > 1:
        with mp.get_context("fork").Pool(procs) as pool:
            for d0, ids, off in pool.imap_unordered(_encode_shard, spans):
                parts[d0] = (ids, off)
    else:
        for s in spans:
            d0, ids, off = _encode_shard(s)
            parts[d0] = (ids, off)
    id_off = np.zeros(D + 1, dtype=np.int64)
    chunks = []
    t = 0
    for d0, d1 in spans:
        ids, off = parts[d0]
        id_off[d0:d1 + 1] = off + t
        t += int(off[-1])
        chunks.append(ids)
    ids = np.concatenate(chunks) if chunks else np.zeros(0, np.int32)
    assert ids.size == t == id_off[-1]
    return ids, id_off


def main(argv):
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*")
    ap.add_argument("--procs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args(argv)
    names = args.workloads or list(WORKLOADS)
    golden = {}
    if os.path.exists(OUT):
        golden = json.load(open(OUT))
    for name in names:
        cfg = WORKLOADS[name]
        t0 = time.time()
        batch = encode_batch_input(cfg, make_lexicon(cfg))
        t1 = time.time()
        merges = np.load(merges_path(name), allow_pickle=False)
        ids, id_off = oracle_encode_all(batch.data, batch.doc_off, merges, args.procs)
        t2 = time.time()
        golden[name] = {
            "n_bytes": int(batch.n_bytes),
            "n_docs": int(batch.doc_off.size - 1),
            "input_fnv1a64": f"{O.fnv1a64(batch.data):016x}",
            "merges_sha256": hashlib.sha256(open(merges_path(name), "rb").read()).hexdigest(),
            "T": int(id_off[-1]),
            "ids_fnv1a64": f"{O.ids_fnv(ids):016x}",
            "id_off_fnv1a64": f"{O.fnv1a64(np.ascontiguousarray(id_off, dtype='<i8')):016x}",
        }
        print(f"{name}: N={batch.n_bytes} D={batch.doc_off.size - 1} T={int(id_off[-1])} "
              f"ids {golden[name]['ids_fnv1a64']} (generate {t1 - t0:.1f}s, "
              f"oracle {t2 - t1:.1f}s on {args.procs} processes)", flush=True)
        del ids, id_off, batch
        with open(OUT, "w") as f:
            json.dump({"about": "oracle whole-batch encode of each workload; written by "
                                "tests/golden/make_fullsize.py (oracle and generator only)",
                       **{k: v for k, v in golden.items() if k != "about"}}, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
