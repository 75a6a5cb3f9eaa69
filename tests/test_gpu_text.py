"""A model loaded from the text form (merges file and vocabulary JSON) encodes
and decodes exactly as the oracle with the same table and ID map."""
import numpy as np
import pytest
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import Model
from workloads import WORKLOADS, make_lexicon, small_batch

from gpu_util import check_encode, device, gpu_decode, merges_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", ["tiny", "throughput"])
def test_model_from_text(k):
    torch.cuda.set_device(device())
    m = merges_for(k)
    rng = np.random.default_rng(11)
    id_map = (rng.permutation(256 + m.shape[0]) + 3).astype(np.int32)
    model = Model.from_text(O.merges_to_text(m), O.vocab_to_json(m, id_map, ensure_ascii=False))
    table = O.Table(m, id_map)
    cfg = WORKLOADS[k]
    b = small_batch(cfg, n_docs=6, doc_bytes=5000, seed=31, lex=make_lexicon(cfg))
    ids, off = check_encode(model, table, b.data, b.doc_off)
    out, boff, st = gpu_decode(model, ids, off)
    assert st == 0 and np.array_equal(out, b.data) and np.array_equal(boff, b.doc_off)
