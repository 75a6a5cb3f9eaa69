"""bpe_encode_batch_noalloc (the encode on the library's static scratch)
against bpe_encode_batch (the same pipeline on a caller workspace), through
the C ABI: two calls in a row, the second with a smaller input, each compared
element by element (IDs, offsets, status) with the workspace call on the same
input; then the host-side rejection of an input too large for the scratch."""
import ctypes as C

import numpy as np
import pytest
import torch

from byte_level_bpe_pretokenize_amd import Model, _lib
from workloads import WORKLOADS, make_lexicon, small_batch

from gpu_util import device, merges_for

pytestmark = pytest.mark.gpu


def _run(model, batch, noalloc):
    dev = model.device
    N, D = batch.n_bytes, batch.n_docs
    data = torch.from_numpy(batch.data).to(dev)
    doc_off = torch.from_numpy(batch.doc_off).to(dev)
    ids = torch.full((N,), -7, dtype=torch.int32, device=dev)
    id_off = torch.full((D + 1,), -7, dtype=torch.int64, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    if noalloc:
        model.encode_batch_noalloc_into(data, doc_off, ids, id_off, status)
    else:
        ws = torch.empty(model.encode_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
        model.encode_batch_into(data, doc_off, ids, id_off, ws, status)
    torch.cuda.synchronize()
    off = id_off.cpu().numpy()
    return ids.cpu().numpy(), off, int(status.item())


@pytest.mark.parametrize("name", ["throughput", "multilingual"])
def test_noalloc_matches_workspace_encode(name):
    dev = device()
    torch.cuda.set_device(dev)
    cfg = WORKLOADS[name]
    lex = make_lexicon(cfg)
    model = Model(merges_for(name))
    # two calls in a row on the shared scratch, the second smaller than the first
    shapes = [(48, 65536, 11), (5, 3000, 12)]
    for n_docs, doc_bytes, seed in shapes:
        batch = small_batch(cfg, n_docs=n_docs, doc_bytes=doc_bytes, seed=seed, lex=lex)
        need = model.encode_workspace_bytes(batch.n_bytes, batch.n_docs)
        assert need <= _lib.NOALLOC_SCRATCH_BYTES, need
        print(f"[noalloc] {name}: {batch.n_docs} docs, {batch.n_bytes} bytes", flush=True)
        want_ids, want_off, want_st = _run(model, batch, noalloc=False)
        got_ids, got_off, got_st = _run(model, batch, noalloc=True)
        assert want_st == 0 and got_st == 0
        T = int(want_off[-1])
        assert np.array_equal(got_off, want_off)
        assert np.array_equal(got_ids[:T], want_ids[:T])
        # nothing written past the IDs
        assert np.all(got_ids[T:] == -7)


def test_noalloc_rejects_inputs_over_the_scratch():
    dev = device()
    torch.cuda.set_device(dev)
    model = Model(merges_for("tiny"))
    L = _lib.load()
    # the smallest size whose workspace exceeds the scratch (checked on the host,
    # before any pointer is read or anything is queued)
    n = 1 << 20
    while model.encode_workspace_bytes(n, 1) <= _lib.NOALLOC_SCRATCH_BYTES:
        n *= 2
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    id_off = torch.zeros(2, dtype=torch.int64, device=dev)
    rc = L.bpe_encode_batch_noalloc(model._h, C.c_void_p(16), n, C.c_void_p(id_off.data_ptr()), 1,
                                    C.c_void_p(16), n, C.c_void_p(id_off.data_ptr()),
                                    C.c_void_p(status.data_ptr()), None)
    assert rc == _lib.BPE_ESCRATCH
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and id_off.cpu().tolist() == [0, 0]
