"""Full-size encode of every workload, in the launch configuration bench.py
times: one bpe_encode_batch call over the whole batch.

The oracle cannot encode a whole 1 GiB batch in seconds, so the check is
split.  A seeded sample of documents is compared with the oracle element by
element; what holds at any size is checked on everything: the status word,
the offsets, and decode(encode(x)) == x over the whole batch.
"""
import numpy as np
import pytest
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import Model
from workloads import WORKLOADS, encode_batch_input, make_lexicon

from gpu_util import device, merges_for

pytestmark = pytest.mark.gpu

SAMPLE_DOCS = 24


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_workload(name):
    dev = device()
    torch.cuda.set_device(dev)
    cfg = WORKLOADS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    batch = encode_batch_input(cfg, make_lexicon(cfg))
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
    assert off[0] == 0 and 0 < T <= N and np.all(np.diff(off) >= 0)
    # a non-empty document yields at least one ID, and no document more IDs than bytes
    doc_len = np.diff(batch.doc_off)
    tok_len = np.diff(off)
    assert np.all(tok_len <= doc_len) and np.all((tok_len > 0) == (doc_len > 0))

    # sampled documents against the oracle, element by element
    table = O.Table(merges)
    rng = np.random.default_rng(4242)
    picks = sorted(set(rng.choice(D, size=min(D, SAMPLE_DOCS), replace=False).tolist()) | {0, D - 1})
    ids_host = ids[:T].cpu().numpy()
    for d in picks:
        a, b = int(batch.doc_off[d]), int(batch.doc_off[d + 1])
        want = np.asarray(table.encode(batch.data[a:b].tobytes()), dtype=np.int32)
        got = ids_host[off[d]:off[d + 1]]
        assert np.array_equal(got, want), f"{name}: document {d} differs from the oracle"
        assert O.ids_fnv(got) == O.ids_fnv(want)
    print(f"[fullsize] {name}: {len(picks)} sampled documents equal the oracle; T = {T}", flush=True)

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
