"""ctypes wrapper over the plain C oracle in ``bpe_oracle.c``.

Test infrastructure: see the header of ``bpe_oracle.c`` for the sources and
the readings the oracle follows.  Nothing here runs on a GPU.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bpe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CLS_L, CLS_D, CLS_W, CLS_P = 0, 1, 2, 3
ORA_OK, ORA_EINVAL, ORA_EDUP, ORA_ERANGE, ORA_ECYCLE, ORA_EIDMAP = 0, -1, -2, -3, -4, -5

_lib = None


def build() -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                    "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    L = C.CDLL(LIB)
    i64, i32, p = C.c_int64, C.c_int32, C.c_void_p
    L.ora_byte_class.argtypes = [C.c_int]
    L.ora_byte_class.restype = C.c_int
    L.ora_split.argtypes = [p, i64, p]
    L.ora_split.restype = i64
    L.ora_byte_to_unicode.argtypes = [C.c_int]
    L.ora_byte_to_unicode.restype = C.c_int
    L.ora_utf8_encode.argtypes = [C.c_uint32, p]
    L.ora_utf8_encode.restype = C.c_int
    L.ora_fnv1a64.argtypes = [p, i64]
    L.ora_fnv1a64.restype = C.c_uint64
    L.ora_validate.argtypes = [p, i64, p]
    L.ora_validate.restype = C.c_int
    L.ora_table_new.argtypes = [p, i64, p]
    L.ora_table_new.restype = p
    L.ora_table_free.argtypes = [p]
    L.ora_table_free.restype = None
    L.ora_encode_word.argtypes = [p, p, i64, p]
    L.ora_encode_word.restype = i64
    L.ora_encode_batch.argtypes = [p, p, i64, p, i64, p, i64, p]
    L.ora_encode_batch.restype = i64
    L.ora_decode_batch.argtypes = [p, p, i64, p, i64, p, i64, p]
    L.ora_decode_batch.restype = i64
    L.ora_train.argtypes = [p, i64, p, i64, i64, p, p, C.c_int]
    L.ora_train.restype = i64
    L.ora_replay_merges.argtypes = [p, i64, p, i64, p]
    L.ora_replay_merges.restype = i64
    _lib = L
    return L


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def byte_class(b: int) -> int:
    return lib().ora_byte_class(b)


def split(s: bytes) -> list[bytes]:
    """Pre-tokens of one document (readings R1, R2)."""
    a = np.frombuffer(s, dtype=np.uint8) if s else np.zeros(0, np.uint8)
    starts = np.zeros(len(s) + 1, dtype=np.int64)
    k = lib().ora_split(_ptr(a), len(s), _ptr(starts))
    starts[k] = len(s)
    return [s[starts[i]:starts[i + 1]] for i in range(k)]


def byte_to_unicode(b: int) -> str:
    return chr(lib().ora_byte_to_unicode(b))


def utf8_encode(cp: int) -> bytes:
    out = np.zeros(4, dtype=np.uint8)
    n = lib().ora_utf8_encode(cp, _ptr(out))
    return out[:n].tobytes()


def fnv1a64(buf: bytes | np.ndarray) -> int:
    a = np.frombuffer(buf, dtype=np.uint8) if isinstance(buf, (bytes, bytearray)) else \
        np.ascontiguousarray(buf).view(np.uint8).reshape(-1)
    return int(lib().ora_fnv1a64(_ptr(a), a.size))


def ids_fnv(ids: np.ndarray) -> int:
    """FNV-1a 64 over the little-endian int32 ID stream (reading R12)."""
    return fnv1a64(np.ascontiguousarray(ids, dtype="<i4"))


def _merges_array(merges) -> np.ndarray:
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
    return m


def validate(merges, id_map=None) -> int:
    m = _merges_array(merges)
    im = None if id_map is None else np.ascontiguousarray(id_map, dtype=np.int32)
    return lib().ora_validate(_ptr(m), m.shape[0], _ptr(im))


class Table:
    """A validated merge table held by the oracle."""

    def __init__(self, merges, id_map=None):
        self.merges = _merges_array(merges)
        self.R = int(self.merges.shape[0])
        self.id_map = None if id_map is None else np.ascontiguousarray(id_map, dtype=np.int32)
        rc = validate(self.merges, self.id_map)
        if rc != ORA_OK:
            raise ValueError(f"merge table rejected by the oracle (code {rc})")
        self._h = lib().ora_table_new(_ptr(self.merges), self.R, _ptr(self.id_map))
        if not self._h:
            raise ValueError("merge table rejected by the oracle")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.ora_table_free(h)
            self._h = None

    def encode_word(self, w: bytes) -> list[int]:
        """Symbols of one pre-token (reading R4), before any ID map."""
        a = np.frombuffer(w, dtype=np.uint8) if w else np.zeros(0, np.uint8)
        out = np.zeros(max(1, len(w)), dtype=np.int32)
        n = lib().ora_encode_word(self._h, _ptr(a), len(w), _ptr(out))
        return out[:n].tolist()

    def encode_batch(self, data: np.ndarray, doc_off: np.ndarray):
        """IDs and per-document offsets for a batch of documents."""
        data = np.ascontiguousarray(data, dtype=np.uint8)
        doc_off = np.ascontiguousarray(doc_off, dtype=np.int64)
        nd = doc_off.size - 1
        ids = np.zeros(max(1, data.size), dtype=np.int32)
        id_off = np.zeros(nd + 1, dtype=np.int64)
        T = lib().ora_encode_batch(self._h, _ptr(data), data.size, _ptr(doc_off), nd,
                                   _ptr(ids), ids.size, _ptr(id_off))
        if T < 0:
            raise ValueError(f"oracle encode failed ({T})")
        return ids[:T].copy(), id_off

    def encode(self, s: bytes) -> list[int]:
        ids, _ = self.encode_batch(np.frombuffer(s, dtype=np.uint8) if s else np.zeros(0, np.uint8),
                                   np.array([0, len(s)], dtype=np.int64))
        return ids.tolist()

    def decode_batch(self, ids: np.ndarray, id_off: np.ndarray):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        id_off = np.ascontiguousarray(id_off, dtype=np.int64)
        nd = id_off.size - 1
        byte_off = np.zeros(nd + 1, dtype=np.int64)
        n = lib().ora_decode_batch(self._h, _ptr(ids), ids.size, _ptr(id_off), nd, None,
                                   np.iinfo(np.int64).max, _ptr(byte_off))
        if n < 0:
            raise ValueError(f"oracle decode failed ({n})")
        out = np.zeros(max(1, n), dtype=np.uint8)
        n2 = lib().ora_decode_batch(self._h, _ptr(ids), ids.size, _ptr(id_off), nd, _ptr(out),
                                    out.size, _ptr(byte_off))
        assert n2 == n
        return out[:n].copy(), byte_off

    def encode_batch_special(self, data: np.ndarray, doc_off: np.ndarray, bos: int = -1,
                             eos: int = -1):
        """Post-processing with reserved IDs ("Characters, bytes and subwords",
        section "Special tokens are their own IDs"): each document's IDs with
        bos before and eos after them (-1: none), one document at a time."""
        ids, id_off = self.encode_batch(data, doc_off)
        out, off = [], [0]
        for d in range(id_off.size - 1):
            seq = ids[id_off[d]:id_off[d + 1]].tolist()
            if bos >= 0:
                seq = [bos] + seq
            if eos >= 0:
                seq = seq + [eos]
            out += seq
            off.append(off[-1] + len(seq))
        return np.array(out, dtype=np.int32), np.array(off, dtype=np.int64)

    def decode_batch_special(self, ids: np.ndarray, id_off: np.ndarray, skip=(-1, -1)):
        """Decode with the reserved IDs in skip dropped first (on output they
        may be skipped, same section)."""
        ids = np.asarray(ids, dtype=np.int32)
        id_off = np.asarray(id_off, dtype=np.int64)
        keep = np.ones(ids.size, dtype=bool)
        for x in skip:
            if x >= 0:
                keep &= ids != x
        new_off = np.zeros(id_off.size, dtype=np.int64)
        csum = np.concatenate([[0], np.cumsum(keep)])
        new_off[:] = csum[id_off]
        return self.decode_batch(ids[keep], new_off)

    def decode(self, ids) -> bytes:
        a = np.asarray(ids, dtype=np.int32)
        out, _ = self.decode_batch(a, np.array([0, a.size], dtype=np.int64))
        return out.tobytes()


def train(data: np.ndarray, doc_off: np.ndarray, n_merges: int, naive: bool = False):
    """Merges (R x 2 int32, rank order) and their pair counts (reading R7)."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    doc_off = np.ascontiguousarray(doc_off, dtype=np.int64)
    merges = np.zeros((max(1, n_merges), 2), dtype=np.int32)
    counts = np.zeros(max(1, n_merges), dtype=np.int64)
    r = lib().ora_train(_ptr(data), data.size, _ptr(doc_off), doc_off.size - 1, n_merges,
                        _ptr(merges), _ptr(counts), 1 if naive else 0)
    return merges[:r].copy(), counts[:r].copy()


def train_text(texts: list[bytes], n_merges: int, naive: bool = False):
    data = np.frombuffer(b"".join(texts), dtype=np.uint8) if any(texts) else np.zeros(0, np.uint8)
    off = np.zeros(len(texts) + 1, dtype=np.int64)
    np.cumsum([len(t) for t in texts], out=off[1:])
    return train(data, off, n_merges, naive)


def replay_merges(merges, w: bytes) -> list[int]:
    """Apply the recorded merges in rank order to one pre-token: the
    trainer's own final segmentation of it."""
    m = _merges_array(merges)
    a = np.frombuffer(w, dtype=np.uint8) if w else np.zeros(0, np.uint8)
    out = np.zeros(max(1, len(w)), dtype=np.int32)
    n = lib().ora_replay_merges(_ptr(m), m.shape[0], _ptr(a), len(w), _ptr(out))
    return out[:n].tolist()


# ---- the text form of a table ("Tokenization LLM: details of building an
# inference engine in C++", sections "Byte-level encoding" and "Vocabulary
# lookup": each byte prints as one character, so merges and vocabularies are
# stored as text; reading R8 for the character of each byte) ----

def _expansions(merges) -> list[bytes]:
    """Bytes of every symbol: a byte, or its merge's two operands' bytes."""
    m = np.asarray(merges, dtype=np.int64).reshape(-1, 2)
    exp: list[bytes | None] = [bytes([b]) for b in range(256)] + [None] * m.shape[0]
    todo = True
    while todo:
        todo = False
        for r, (a, b) in enumerate(m.tolist()):
            if exp[256 + r] is None and exp[a] is not None and exp[b] is not None:
                exp[256 + r] = exp[a] + exp[b]
                todo = True
    assert all(e is not None for e in exp), "operand out of range or a cycle"
    return exp


_printed = None


def _print_table():
    global _printed
    if _printed is None:
        chars = [byte_to_unicode(x) for x in range(256)]
        _printed = (chars, {ch: x for x, ch in enumerate(chars)})
    return _printed


def bytes_to_text(b: bytes) -> str:
    chars, _ = _print_table()
    return "".join(chars[x] for x in b)


def text_to_bytes(t: str) -> bytes:
    _, inv = _print_table()
    return bytes(inv[ch] for ch in t)


def merges_to_text(merges) -> str:
    """A merges file: a version line, then "left right" per merge in rank order."""
    exp = _expansions(merges)
    m = np.asarray(merges).reshape(-1, 2)
    return "#version: 0.2\n" + "".join(f"{bytes_to_text(exp[a])} {bytes_to_text(exp[b])}\n"
                                       for a, b in m.tolist())


def parse_merges_text(text: str) -> np.ndarray:
    """The integer table of a merges file: each line's operands looked up by
    their bytes among the bytes and the earlier lines' results."""
    sym = {bytes([b]): b for b in range(256)}
    out = []
    lines = text.split("\n")
    for n, line in enumerate(lines):
        line = line[:-1] if line.endswith("\r") else line
        if not line or (n == 0 and line.startswith("#version")):
            continue
        left, right = line.split(" ")
        lb, rb = text_to_bytes(left), text_to_bytes(right)
        assert lb + rb not in sym, "two lines give the same bytes"
        out.append((sym[lb], sym[rb]))
        sym[lb + rb] = 256 + len(out) - 1
    return np.array(out, dtype=np.int32).reshape(-1, 2)


def vocab_to_json(merges, id_map, ensure_ascii: bool = True, extra: dict | None = None) -> str:
    import json
    exp = _expansions(merges)
    d = {bytes_to_text(e): int(i) for e, i in zip(exp, np.asarray(id_map).tolist())}
    d.update(extra or {})
    return json.dumps(d, ensure_ascii=ensure_ascii)


def parse_vocab_json(text: str, merges) -> np.ndarray:
    """Each symbol's ID: the vocabulary's entry for the text of its bytes."""
    import json
    d = json.loads(text)
    return np.array([d[bytes_to_text(e)] for e in _expansions(merges)], dtype=np.int32)
