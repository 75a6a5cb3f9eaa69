"""The C ABI without a GPU: the library loads, exports every function that
include/bpe.h declares, and its host-side checks answer before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from byte_level_bpe_pretokenize_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bpe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bpe_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SYMBOLS)


def test_library_exports_every_symbol():
    L = _lib.load()
    for name in declared_functions():
        assert hasattr(L, name), name


def _load(merges, id_map=None):
    L = _lib.load()
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
    h = C.c_void_p()
    im = None if id_map is None else np.ascontiguousarray(id_map, dtype=np.int32)
    rc = L.bpe_load_merges(m.ctypes.data_as(C.c_void_p) if m.size else None, m.shape[0],
                           im.ctypes.data_as(C.c_void_p) if im is not None else None, None,
                           C.byref(h))
    return rc


@pytest.mark.parametrize("merges,code", [
    ([[97, 98], [97, 98]], _lib.BPE_EMERGES),     # repeated pair
    ([[97, 300]], _lib.BPE_EMERGES),              # operand out of range
    ([[-1, 97]], _lib.BPE_EMERGES),
    ([[256, 97]], _lib.BPE_EMERGES),              # symbol built from itself
    ([[257, 97], [256, 98]], _lib.BPE_EMERGES),   # 256 -> 257 -> 256
])
def test_load_rejects_bad_tables(merges, code):
    assert _load(merges) == code


def test_load_rejects_bad_id_maps():
    m = [[97, 98]]
    dup = np.arange(257)
    dup[3] = 4
    assert _load(m, dup) == _lib.BPE_EIDMAP
    neg = np.arange(257)
    neg[0] = -1
    assert _load(m, neg) == _lib.BPE_EIDMAP
    big = np.arange(257)
    big[0] = _lib.MAX_ID + 1
    assert _load(m, big) == _lib.BPE_EIDMAP


def test_load_argument_checks():
    L = _lib.load()
    h = C.c_void_p()
    assert L.bpe_load_merges(None, -1, None, None, C.byref(h)) == _lib.BPE_EINVAL
    assert L.bpe_load_merges(None, 3, None, None, C.byref(h)) == _lib.BPE_EINVAL
    assert L.bpe_load_merges(None, _lib.MAX_MERGES + 1, None, None, C.byref(h)) == _lib.BPE_EINVAL
    assert L.bpe_load_merges(None, 0, None, None, None) == _lib.BPE_EINVAL


def test_null_model_calls():
    L = _lib.load()
    assert L.bpe_vocab_size(None) == -1
    assert L.bpe_max_token_bytes(None) == -1
    assert L.bpe_encode_batch(None, None, 0, None, 0, None, 0, None, None, 0, None, None) == _lib.BPE_EINVAL
    assert L.bpe_decode_batch(None, None, 0, None, 0, None, 0, None, None, 0, None, None) == _lib.BPE_EINVAL
    assert L.bpe_encode_batch_noalloc(None, None, 0, None, 0, None, 0, None, None, None) == _lib.BPE_EINVAL
    assert b"scratch" in L.bpe_strerror(_lib.BPE_ESCRATCH)
    assert L.bpe_encode_batch_special(None, None, 0, None, 0, -1, -1, None, 0, None, None, 0, None,
                                      None) == _lib.BPE_EINVAL
    assert L.bpe_decode_batch_special(None, None, 0, None, 0, -1, -1, None, 0, None, None, 0, None,
                                      None) == _lib.BPE_EINVAL
    L.bpe_free(None)


def test_workspace_sizes():
    L = _lib.load()
    assert L.bpe_encode_workspace_bytes(None, 0, 0) == 0
    assert L.bpe_decode_workspace_bytes(None, 0, 0) == 0
    n = 1 << 20
    ws = L.bpe_encode_workspace_bytes(None, n, 16)
    assert ws >= 8 * n                       # position-indexed scratch for long pre-tokens
    # about 28.7 bytes per input byte (the regions are sized for each chunk's
    # worst case)
    for big in (1 << 20, 1 << 28):
        assert L.bpe_encode_workspace_bytes(None, big, 4096) <= 29 * big
    assert L.bpe_encode_workspace_bytes(None, n + 1, 16) > ws
    assert L.bpe_decode_workspace_bytes(None, 5000, 3) > 0
    # the special encode writes its reserved IDs in the encode's own kernels
    assert L.bpe_encode_special_workspace_bytes(None, n, 16) == ws
    assert L.bpe_encode_special_workspace_bytes(None, 0, 5) == 0


def test_stage_timing_queries():
    L = _lib.load()
    assert L.bpe_stage_count(_lib.OP_ENCODE) == 10
    assert L.bpe_stage_count(_lib.OP_DECODE) == 4
    assert L.bpe_stage_count(7) == -1
    names = [L.bpe_stage_name(_lib.OP_ENCODE, k).decode() for k in range(10)]
    assert names == ["k_docs", "k_find", "k_dedup", "k_merge", "k_merge_wide", "k_merge_long",
                     "k_dupfill", "k_offsets", "k_bscan", "k_emit"]
    assert L.bpe_stage_name(_lib.OP_ENCODE, 10) is None
    assert L.bpe_stage_name(_lib.OP_DECODE, -1) is None
    assert L.bpe_stage_timing(None, 1) == _lib.BPE_EINVAL
    ms = (C.c_double * 10)()
    n = C.c_int64()
    assert L.bpe_stage_times(None, _lib.OP_ENCODE, ms, 10, C.byref(n)) == _lib.BPE_EINVAL


def test_strerror():
    L = _lib.load()
    for code in range(-7, 1):
        assert len(L.bpe_strerror(code)) > 3
