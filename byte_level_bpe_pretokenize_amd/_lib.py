"""ctypes declarations for libbpe.so (the C ABI in include/bpe.h)."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbpe.so")

# every symbol include/bpe.h declares
SYMBOLS = (
    "bpe_load_merges", "bpe_parse_merges_text", "bpe_parse_vocab_json", "bpe_train",
    "bpe_free", "bpe_vocab_size", "bpe_max_token_bytes",
    "bpe_encode_workspace_bytes", "bpe_encode_batch", "bpe_encode_batch_noalloc",
    "bpe_encode_special_workspace_bytes", "bpe_encode_batch_special",
    "bpe_decode_workspace_bytes", "bpe_decode_batch", "bpe_decode_batch_special",
    "bpe_stage_timing", "bpe_stage_count", "bpe_stage_name", "bpe_stage_times",
    "bpe_strerror",
)

BPE_OK, BPE_EINVAL, BPE_EMERGES, BPE_EIDMAP, BPE_EWORKSPACE, BPE_EHIP, BPE_ENOMEM, BPE_ENOTSUP, \
    BPE_EFORMAT, BPE_ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
NOALLOC_SCRATCH_BYTES = 128 << 20
STATUS_BAD_DOC_OFFSETS, STATUS_IDS_CAPACITY, STATUS_BAD_ID, STATUS_BYTES_CAPACITY, \
    STATUS_BAD_ID_OFFSETS = 1, 2, 4, 8, 16
OP_ENCODE, OP_DECODE = 0, 1
MAX_MERGES = 1 << 20
MAX_ID = (1 << 24) - 1

_lib = None


def load() -> C.CDLL:
    """Load the in-tree libbpe.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m byte_level_bpe_pretokenize_amd.build`")
    L = C.CDLL(LIB_PATH)
    p, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
    L.bpe_load_merges.argtypes = [p, i64, p, p, C.POINTER(p)]
    L.bpe_load_merges.restype = i32
    L.bpe_parse_merges_text.argtypes = [p, i64, p, i64, C.POINTER(C.c_int64)]
    L.bpe_parse_merges_text.restype = i32
    L.bpe_parse_vocab_json.argtypes = [p, i64, p, i64, p]
    L.bpe_parse_vocab_json.restype = i32
    L.bpe_train.argtypes = [p, i64, p, i64, i64, p, p, C.POINTER(C.c_int64), p]
    L.bpe_train.restype = i32
    L.bpe_free.argtypes = [p]
    L.bpe_free.restype = None
    L.bpe_vocab_size.argtypes = [p]
    L.bpe_vocab_size.restype = i64
    L.bpe_max_token_bytes.argtypes = [p]
    L.bpe_max_token_bytes.restype = i64
    L.bpe_encode_workspace_bytes.argtypes = [p, i64, i64]
    L.bpe_encode_workspace_bytes.restype = sz
    L.bpe_encode_batch.argtypes = [p, p, i64, p, i64, p, i64, p, p, sz, p, p]
    L.bpe_encode_batch.restype = i32
    L.bpe_encode_batch_noalloc.argtypes = [p, p, i64, p, i64, p, i64, p, p, p]
    L.bpe_encode_batch_noalloc.restype = i32
    L.bpe_encode_special_workspace_bytes.argtypes = [p, i64, i64]
    L.bpe_encode_special_workspace_bytes.restype = sz
    L.bpe_encode_batch_special.argtypes = [p, p, i64, p, i64, i32, i32, p, i64, p, p, sz, p, p]
    L.bpe_encode_batch_special.restype = i32
    L.bpe_decode_batch_special.argtypes = [p, p, i64, p, i64, i32, i32, p, i64, p, p, sz, p, p]
    L.bpe_decode_batch_special.restype = i32
    L.bpe_decode_workspace_bytes.argtypes = [p, i64, i64]
    L.bpe_decode_workspace_bytes.restype = sz
    L.bpe_decode_batch.argtypes = [p, p, i64, p, i64, p, i64, p, p, sz, p, p]
    L.bpe_decode_batch.restype = i32
    L.bpe_stage_timing.argtypes = [p, i32]
    L.bpe_stage_timing.restype = i32
    L.bpe_stage_count.argtypes = [i32]
    L.bpe_stage_count.restype = i32
    L.bpe_stage_name.argtypes = [i32, i32]
    L.bpe_stage_name.restype = C.c_char_p
    L.bpe_stage_times.argtypes = [p, i32, C.POINTER(C.c_double), i32, C.POINTER(C.c_int64)]
    L.bpe_stage_times.restype = i32
    L.bpe_strerror.argtypes = [i32]
    L.bpe_strerror.restype = C.c_char_p
    _lib = L
    return L
