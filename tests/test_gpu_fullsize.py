"""Full-size encode of every workload, in the launch configuration bench.py
times: one bpe_encode_batch call over the whole batch.

The whole batch is checked against the oracle's whole-batch encode, stored in
tests/golden/fullsize.json by tests/golden/make_fullsize.py (the oracle and
the generator only): the ID count T, the FNV-1a 64 of all IDs and the FNV-1a
64 of all document offsets must be equal ("Hugging Face Tokenizers v1:
encoding up to 30x faster", section "Benchmarks": a run is checked by the
FNV-1a of its output IDs).  A seeded sample of documents is also compared
with the oracle element by element, which names the first differing document
if the checksums ever disagree, and decode(encode(x)) == x is checked over the
whole batch.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import Model
from workloads import WORKLOADS, encode_batch_input, make_lexicon

from gpu_util import ROOT, device, merges_for

pytestmark = pytest.mark.gpu

SAMPLE_DOCS = 24
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "fullsize.json")))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_workload(name):
    dev = device()
    torch.cuda.set_device(dev)
    cfg = WORKLOADS[name]
    gold = GOLDEN[name]
    print(f"[fullsize] {name}: generating", flush=True)
    batch = encode_batch_input(cfg, make_lexicon(cfg))
    assert batch.n_bytes == gold["n_bytes"] and batch.n_docs == gold["n_docs"]
    assert f"{O.fnv1a64(batch.data):016x}" == gold["input_fnv1a64"], "generator output changed"
    merges = merges_for(name)
    model = Model(merges)
    N, D = batch.n_bytes, batch.n_docs
    print(f"[fullsize] {name}: {N} bytes, {D} documents, encoding", flush=True)
    data = torch.from_numpy(batch.data).to(dev)
    doc_off = torch.from_numpy(batch.doc_off).to(dev)
    ids = torch.empty(N, dtype=torch.int32, device=dev)
    id_off = torch.empty(D + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(model.encode_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    model.encode_batch_into(data, doc_off, ids, id_off, ws, status)
    torch.cuda.synchronize()
    del ws
    assert int(status.item()) == 0
    off = id_off.cpu().numpy()
    T = int(off[-1])
    ids_host = ids[:T].cpu().numpy()

    # the whole batch against the oracle's whole-batch checksums
    got = {"T": T, "ids_fnv1a64": f"{O.ids_fnv(ids_host):016x}",
           "id_off_fnv1a64": f"{O.fnv1a64(np.ascontiguousarray(off, dtype='<i8')):016x}"}
    print(f"[fullsize] {name}: T = {T}, ids {got['ids_fnv1a64']}, offsets "
          f"{got['id_off_fnv1a64']}", flush=True)
    whole_ok = all(got[k] == gold[k] for k in got)

    # sampled documents against the oracle, element by element
    table = O.Table(merges)
    rng = np.random.default_rng(4242)
    picks = sorted(set(rng.choice(D, size=min(D, SAMPLE_DOCS), replace=False).tolist()) | {0, D - 1})
    for d in picks:
        a, b = int(batch.doc_off[d]), int(batch.doc_off[d + 1])
        want = np.asarray(table.encode(batch.data[a:b].tobytes()), dtype=np.int32)
        g = ids_host[off[d]:off[d + 1]] if off[d + 1] <= T else None
        assert g is not None and np.array_equal(g, want), \
            f"{name}: document {d} differs from the oracle"
    assert whole_ok, f"{name}: whole batch differs from the oracle: {got} vs {gold}"
    print(f"[fullsize] {name}: whole batch equals the oracle (T, ID and offset checksums); "
          f"{len(picks)} sampled documents equal element by element", flush=True)

    # decode(encode(x)) == x over the whole batch
    out = torch.empty(N, dtype=torch.uint8, device=dev)
    byte_off = torch.empty(D + 1, dtype=torch.int64, device=dev)
    dws = torch.empty(max(1, model.decode_workspace_bytes(T, D)), dtype=torch.uint8, device=dev)
    dstat = torch.full((1,), -1, dtype=torch.int32, device=dev)
    model.decode_batch_into(ids[:T], id_off, out, byte_off, dws, dstat)
    torch.cuda.synchronize()
    assert int(dstat.item()) == 0
    assert torch.equal(out, data) and torch.equal(byte_off, doc_off)
    print(f"[fullsize] {name}: round trip equal", flush=True)
    del data, doc_off, ids, id_off, out, byte_off, dws, model
    torch.cuda.empty_cache()
