"""Reserved IDs around each document (post-processing) on the GPU, against the
oracle, element by element: bpe_encode_batch_special and
bpe_decode_batch_special through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import BPEError, Model, _lib
from workloads import WORKLOADS, make_lexicon, small_batch

from gpu_util import batch_from_docs, device, merges_for

pytestmark = pytest.mark.gpu

_models = {}


def model_pair(k):
    if k not in _models:
        m = merges_for(k)
        _models[k] = (Model(m), O.Table(m))
    return _models[k]


@pytest.fixture(scope="module")
def dev():
    d = device()
    torch.cuda.set_device(d)
    return d


def gpu_encode_special(model, data, doc_off, bos, eos, cap=None, guard=64):
    """Encode with reserved IDs; returns (ids[:T], id_off, status, guard region)."""
    dev = model.device
    n, nd = data.size, doc_off.size - 1
    per = int(bos >= 0) + int(eos >= 0)
    cap = n + nd * per if cap is None else cap
    buf = torch.full((cap + guard,), -7, dtype=torch.int32, device=dev)
    ids = buf[:cap]
    d_data = torch.from_numpy(data).to(dev) if n else torch.zeros(0, dtype=torch.uint8, device=dev)
    d_off = torch.from_numpy(np.ascontiguousarray(doc_off)).to(dev)
    id_off = torch.full((nd + 1,), -7, dtype=torch.int64, device=dev)
    wsb = model.encode_special_workspace_bytes(n, nd)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    model.encode_batch_special_into(d_data, d_off, bos, eos, ids, id_off, ws, status)
    torch.cuda.synchronize()
    st = int(status.item())
    off = id_off.cpu().numpy()
    T = int(off[-1]) if st == 0 else cap
    return buf[:min(T, cap)].cpu().numpy(), off, st, buf[cap:].cpu().numpy()


def check_special(model, table, data, doc_off, bos, eos):
    got, got_off, st, guard = gpu_encode_special(model, data, doc_off, bos, eos)
    assert st == 0, f"device status {st:#x}"
    want, want_off = table.encode_batch_special(data, doc_off, bos, eos)
    assert np.array_equal(got_off, want_off)
    assert np.array_equal(got, want)
    assert (guard == -7).all()
    return got, got_off


@pytest.mark.parametrize("bos,eos", [(-1, -1), (0, -1), (-1, 1), (0, 1)])
def test_special_small_docs(dev, bos, eos):
    model, table = model_pair("tiny")
    V = model.vocab_size
    b = None if bos < 0 else V + 3 + bos
    e = None if eos < 0 else V + 10 + eos
    docs = [b"Hello world!", b"", b"the 42 cats sat", b"", b"", b"x", "Grüße 🐈".encode()]
    data, off = batch_from_docs(docs)
    check_special(model, table, data, off, -1 if b is None else b, -1 if e is None else e)


@pytest.mark.parametrize("k", ["throughput", "serving"])
def test_special_workload_batches(dev, k):
    # many documents per chunk (serving) and documents spanning chunks (throughput)
    cfg = WORKLOADS[k]
    model, table = model_pair(k)
    nd, sz = (24, 6000) if k == "throughput" else (400, 0)
    b = small_batch(cfg, n_docs=nd, doc_bytes=sz, seed=77, lex=make_lexicon(cfg))
    V = model.vocab_size
    ids, off = check_special(model, table, b.data, b.doc_off, V, V + 1)
    # and back: the reserved IDs decode to no bytes
    out, boff = gpu_decode_special(model, ids, off, (V, V + 1))
    assert out.tobytes() == b.data.tobytes() and np.array_equal(boff, b.doc_off)


def test_special_empty_input(dev):
    model, table = model_pair("tiny")
    V = model.vocab_size
    data = np.zeros(0, np.uint8)
    off = np.zeros(4, np.int64)
    got, got_off, st, guard = gpu_encode_special(model, data, off, V + 2, V + 5)
    assert st == 0
    assert got.tolist() == [V + 2, V + 5] * 3
    assert got_off.tolist() == [0, 2, 4, 6]
    assert (guard == -7).all()


def test_special_capacity(dev):
    model, table = model_pair("tiny")
    V = model.vocab_size
    docs = [b"alpha beta", b"gamma", b""]
    data, off = batch_from_docs(docs)
    want, want_off = table.encode_batch_special(data, off, V, V + 1)
    cap = int(want.size) - 3
    got, got_off, st, guard = gpu_encode_special(model, data, off, V, V + 1, cap=cap)
    assert st & _lib.STATUS_IDS_CAPACITY
    assert (guard == -7).all()          # nothing written past the capacity
    assert np.array_equal(got[:cap], want[:cap])


def test_special_rejects_symbol_ids(dev):
    model, _ = model_pair("tiny")
    V = model.vocab_size
    data, off = batch_from_docs([b"abc"])
    for bad in (65, V - 1, -2, _lib.MAX_ID + 1):
        with pytest.raises(BPEError):
            model.encode_batch_special(torch.from_numpy(data).to(dev),
                                       torch.from_numpy(off).to(dev), bad, -1)
    with pytest.raises(BPEError):
        gpu_decode_special(model, np.array([97], np.int32), np.array([0, 1]), (97, -1))


def test_special_with_id_map(dev):
    m = merges_for("tiny")
    V = 256 + m.shape[0]
    rng = np.random.default_rng(5)
    id_map = (rng.permutation(V) + 10).astype(np.int32)   # IDs 10 .. V + 9
    model, table = Model(m, id_map), O.Table(m, id_map)
    docs = [b"one two three", b"", b"4567 !!"]
    data, off = batch_from_docs(docs)
    check_special(model, table, data, off, 3, V + 10)     # 3 and V + 10: no symbol's ID
    with pytest.raises(BPEError):                          # 10 is some symbol's ID
        model.encode_batch_special(torch.from_numpy(data).to(dev), torch.from_numpy(off).to(dev),
                                   int(id_map[0]), -1)


def test_decode_without_skip_flags_reserved_ids(dev):
    model, table = model_pair("tiny")
    V = model.vocab_size
    data, off = batch_from_docs([b"abc def"])
    ids, id_off, st, _ = gpu_encode_special(model, data, off, V, V + 1)
    assert st == 0
    _, _, st2 = gpu_decode_plain(model, ids, id_off)
    assert st2 & _lib.STATUS_BAD_ID


def gpu_decode_special(model, ids, id_off, skip):
    dev = model.device
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev)
    d_off = torch.from_numpy(np.ascontiguousarray(id_off, dtype=np.int64)).to(dev)
    out, boff = model.decode_batch(d_ids, d_off, skip=skip)
    return out.cpu().numpy(), boff.cpu().numpy()


def gpu_decode_plain(model, ids, id_off):
    from gpu_util import gpu_decode
    return gpu_decode(model, ids, id_off)


def test_special_many_documents_per_chunk(dev):
    # more document starts in one chunk than k_emit stages in LDS (512), with
    # empty documents among them
    model, table = model_pair("tiny")
    V = model.vocab_size
    rng = np.random.default_rng(21)
    alphabet = np.frombuffer(b"ab c1!", dtype=np.uint8)
    docs = [rng.choice(alphabet, size=int(rng.integers(0, 4))).tobytes() for _ in range(3000)]
    data, off = batch_from_docs(docs)
    check_special(model, table, data, off, V, V + 1)
    check_special(model, table, data, off, -1, V + 1)


def test_special_long_pretokens(dev):
    # pre-tokens that run past a chunk's window (wave-merged, written straight
    # to the output) next to document starts
    model, table = model_pair("adversarial")
    V = model.vocab_size
    docs = [b"x " + b"a" * 9000 + b" tail", b"", b"7" * 3000, b"short one", b"b" * 4100]
    data, off = batch_from_docs(docs)
    check_special(model, table, data, off, V + 5, V + 9)


@pytest.mark.parametrize("name", ["throughput", "serving"])
def test_special_full_size(dev, name):
    # the whole batch at its full size, in the launch configuration bench.py
    # times: with the reserved IDs taken out the IDs are the plain encode's,
    # and every document is [bos] ... [eos] at the plain offset + 2 d
    from workloads import encode_batch_input
    cfg = WORKLOADS[name]
    batch = encode_batch_input(cfg, make_lexicon(cfg))
    model, _ = model_pair(name)
    V = model.vocab_size
    data = torch.from_numpy(batch.data).to(dev)
    off = torch.from_numpy(batch.doc_off).to(dev)
    plain, plain_off = model.encode_batch(data, off)
    ids, id_off = model.encode_batch_special(data, off, V, V + 1)
    D = batch.n_docs
    assert torch.equal(id_off, plain_off + 2 * torch.arange(D + 1, device=dev))
    keep = (ids != V) & (ids != V + 1)
    assert torch.equal(ids[keep], plain)
    assert bool((ids[id_off[:-1]] == V).all()) and bool((ids[id_off[1:] - 1] == V + 1).all())
    assert int((~keep).sum()) == 2 * D
