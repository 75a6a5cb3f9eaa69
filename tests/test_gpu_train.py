"""The GPU trainer (bpe_train) against the oracle's trainer: the same merges
in the same order with the same counts, bit for bit."""
import os
import time

import numpy as np
import pytest
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import BPEError, _lib, train
from workloads import WORKLOADS, make_lexicon, training_corpus

from gpu_util import batch_from_docs, device

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def dev():
    torch.cuda.set_device(device())


def check_train(data, off, n):
    got_m, got_c = train(data, off, n)
    want_m, want_c = O.train(data, off, n)
    assert got_m.shape == want_m.shape, (got_m.shape, want_m.shape)
    assert np.array_equal(got_m, want_m)
    assert np.array_equal(got_c, want_c)
    return got_m


def test_train_tiny_corpus():
    cfg = WORKLOADS["tiny"]
    tc = training_corpus(cfg, make_lexicon(cfg))
    m = check_train(tc.data, tc.doc_off, cfg.n_merges)
    # and the table stored for the tiny workload (made by the oracle's trainer)
    assert np.array_equal(m, np.load(os.path.join(ROOT, "assets", "merges_tiny.npy")))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_train_runs_and_ties(seed):
    # repeated letters (positional counts of (x, x)), equal counts (ties to
    # the smallest pair), a space before letters, digits and punctuation, an
    # empty document; more merges asked for than the text allows
    rng = np.random.default_rng(seed)
    words = [b"aaaa", b"abab", b" ab", b"ba", b"!!", b"123", b"\t\t", b"aaab", b"bbbb", b"x"]
    docs = [b" ".join(words[i] for i in rng.integers(0, len(words), size=int(rng.integers(1, 40))))
            for _ in range(12)] + [b""]
    data, off = batch_from_docs(docs)
    check_train(data, off, 200)


def test_train_edges():
    data, off = batch_from_docs([b"hello hello", b""])
    assert train(data, off, 0)[0].shape == (0, 2)
    assert train(np.zeros(0, np.uint8), np.zeros(1, np.int64), 10)[0].shape == (0, 2)
    with pytest.raises(BPEError) as e:
        train(data, np.array([0, 5, 3], np.int64), 10)
    assert e.value.code == _lib.BPE_EINVAL


def test_train_throughput_corpus():
    # the 16 MiB training corpus of the throughput workload, 32,000 merges:
    # the same table the oracle's trainer stored for it
    cfg = WORKLOADS["throughput"]
    tc = training_corpus(cfg, make_lexicon(cfg))
    t0 = time.perf_counter()
    m, c = train(tc.data, tc.doc_off, cfg.n_merges)
    dt = time.perf_counter() - t0
    print(f"bpe_train: {tc.data.size} bytes, {m.shape[0]} merges in {dt:.2f} s")
    assert np.array_equal(m, np.load(os.path.join(ROOT, "assets", "merges_throughput.npy")))


@pytest.mark.parametrize("name", ["multilingual", "serving", "adversarial"])
def test_train_reproduces_stored_tables(name):
    # the larger workloads' training corpora (32-64 MiB, 50,000-128,000
    # merges): the tables the oracle's trainer stored in assets/
    cfg = WORKLOADS[name]
    tc = training_corpus(cfg, make_lexicon(cfg))
    t0 = time.perf_counter()
    m, c = train(tc.data, tc.doc_off, cfg.n_merges)
    dt = time.perf_counter() - t0
    print(f"bpe_train {name}: {tc.data.size} bytes, {m.shape[0]} merges in {dt:.2f} s")
    assert np.array_equal(m, np.load(os.path.join(ROOT, "assets", f"merges_{name}.npy")))
    # the chosen counts never increase
    assert np.all(np.diff(c) <= 0) and c[-1] >= 2
