"""The stored whole-batch checksums (tests/golden/fullsize.json) against the
oracle: the tiny workload is encoded again here by the same recipe as
tests/golden/make_fullsize.py, and every entry names the merge table it was
made with."""
import hashlib
import json
import os

import numpy as np

import oracle as O
from workloads import WORKLOADS, encode_batch_input, make_lexicon

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "fullsize.json")))


def test_every_workload_has_an_entry():
    for name in WORKLOADS:
        g = GOLDEN[name]
        path = os.path.join(ROOT, "assets", f"merges_{name}.npy")
        assert hashlib.sha256(open(path, "rb").read()).hexdigest() == g["merges_sha256"]
        assert 0 < g["T"] <= g["n_bytes"]


def test_tiny_entry_is_the_oracles():
    cfg = WORKLOADS["tiny"]
    batch = encode_batch_input(cfg, make_lexicon(cfg))
    g = GOLDEN["tiny"]
    assert f"{O.fnv1a64(batch.data):016x}" == g["input_fnv1a64"]
    merges = np.load(os.path.join(ROOT, "assets", "merges_tiny.npy"), allow_pickle=False)
    ids, off = O.Table(merges).encode_batch(batch.data, batch.doc_off)
    assert int(off[-1]) == g["T"] == ids.size
    assert f"{O.ids_fnv(ids):016x}" == g["ids_fnv1a64"]
    assert f"{O.fnv1a64(np.ascontiguousarray(off, dtype='<i8')):016x}" == g["id_off_fnv1a64"]
