"""Python binding over libbpe's C ABI (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of
encode and decode runs in the library's HIP kernels.  There is no CPU path:
without libbpe.so or a GPU, these calls raise.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib


class BPEError(RuntimeError):
    def __init__(self, code: int, what: str):
        msg = _lib.load().bpe_strerror(code).decode()
        super().__init__(f"{what}: {msg} ({code})")
        self.code = code


def _stream_handle(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def parse_merges_text(text: bytes | str) -> np.ndarray:
    """A merges file (text form) as the (R, 2) int32 table: bpe_parse_merges_text."""
    b = text.encode() if isinstance(text, str) else bytes(text)
    cap = b.count(b"\n") + 1
    out = np.zeros((cap, 2), dtype=np.int32)
    n = C.c_int64()
    rc = _lib.load().bpe_parse_merges_text(b, len(b), out.ctypes.data_as(C.c_void_p), cap, C.byref(n))
    if rc != _lib.BPE_OK:
        raise BPEError(rc, "bpe_parse_merges_text")
    return out[:n.value].copy()


def parse_vocab_json(text: bytes | str, merges) -> np.ndarray:
    """Each symbol's ID from a vocabulary (JSON text form): bpe_parse_vocab_json."""
    b = text.encode() if isinstance(text, str) else bytes(text)
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
    out = np.zeros(256 + m.shape[0], dtype=np.int32)
    rc = _lib.load().bpe_parse_vocab_json(b, len(b), m.ctypes.data_as(C.c_void_p) if m.size else None,
                                          m.shape[0], out.ctypes.data_as(C.c_void_p))
    if rc != _lib.BPE_OK:
        raise BPEError(rc, "bpe_parse_vocab_json")
    return out


def train(data, doc_off, n_merges: int, stream=None):
    """Train a merge table on the current GPU (bpe_train): data (uint8 bytes,
    host) and doc_off (int64, host); returns (merges (R, 2) int32, counts)."""
    if not torch.cuda.is_available():
        raise RuntimeError("libbpe needs a HIP device; none is visible")
    d = np.ascontiguousarray(np.frombuffer(data, dtype=np.uint8) if isinstance(data, (bytes, bytearray))
                             else np.asarray(data, dtype=np.uint8))
    off = np.ascontiguousarray(np.asarray(doc_off, dtype=np.int64))
    merges = np.zeros((max(1, n_merges), 2), dtype=np.int32)
    counts = np.zeros(max(1, n_merges), dtype=np.int64)
    made = C.c_int64()
    rc = _lib.load().bpe_train(d.ctypes.data_as(C.c_void_p) if d.size else None, d.size,
                               off.ctypes.data_as(C.c_void_p), off.size - 1, int(n_merges),
                               merges.ctypes.data_as(C.c_void_p), counts.ctypes.data_as(C.c_void_p),
                               C.byref(made), C.c_void_p(_stream_handle(stream)))
    if rc != _lib.BPE_OK:
        raise BPEError(rc, "bpe_train")
    return merges[:made.value].copy(), counts[:made.value].copy()


class Model:
    """A merge table resident on the current GPU (bpe_load_merges)."""

    @classmethod
    def from_text(cls, merges_text: bytes | str, vocab_json: bytes | str | None = None,
                  stream=None) -> "Model":
        """Load a table from its text form (merges file, and optionally the
        vocabulary that gives the output IDs)."""
        m = parse_merges_text(merges_text)
        return cls(m, None if vocab_json is None else parse_vocab_json(vocab_json, m), stream)

    def __init__(self, merges, id_map=None, stream=None):
        if not torch.cuda.is_available():
            raise RuntimeError("libbpe needs a HIP device; none is visible")
        L = _lib.load()
        m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
        im = None if id_map is None else np.ascontiguousarray(np.asarray(id_map, dtype=np.int32))
        if im is not None and im.size != 256 + m.shape[0]:
            raise ValueError("id_map must have 256 + n_merges entries")
        h = C.c_void_p()
        rc = L.bpe_load_merges(m.ctypes.data_as(C.c_void_p) if m.size else None, m.shape[0],
                               im.ctypes.data_as(C.c_void_p) if im is not None else None,
                               C.c_void_p(_stream_handle(stream)), C.byref(h))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_load_merges")
        self._h = h
        self.n_merges = int(m.shape[0])
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self):
        if getattr(self, "_h", None):
            _lib.load().bpe_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def vocab_size(self) -> int:
        return int(_lib.load().bpe_vocab_size(self._h))

    @property
    def max_token_bytes(self) -> int:
        return int(_lib.load().bpe_max_token_bytes(self._h))

    # ---- stage timing (bpe_stage_timing / bpe_stage_times) -------------------
    def stage_timing(self, enable: bool = True) -> None:
        rc = _lib.load().bpe_stage_timing(self._h, 1 if enable else 0)
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_stage_timing")

    def stage_times(self, op: str = "encode") -> tuple[dict[str, float], int]:
        """Total milliseconds per kernel over the timed calls since the last
        read, and the number of those calls (waits for their events)."""
        L = _lib.load()
        code = {"encode": _lib.OP_ENCODE, "decode": _lib.OP_DECODE}[op]
        n = L.bpe_stage_count(code)
        ms = (C.c_double * n)()
        calls = C.c_int64()
        rc = L.bpe_stage_times(self._h, code, ms, n, C.byref(calls))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_stage_times")
        return {L.bpe_stage_name(code, k).decode(): float(ms[k]) for k in range(n)}, int(calls.value)

    # ---- encode -------------------------------------------------------------
    def encode_workspace_bytes(self, n_bytes: int, n_docs: int) -> int:
        return int(_lib.load().bpe_encode_workspace_bytes(self._h, n_bytes, n_docs))

    def encode_batch_into(self, data: torch.Tensor, doc_off: torch.Tensor, ids: torch.Tensor,
                          id_off: torch.Tensor, workspace: torch.Tensor | None,
                          status: torch.Tensor, stream=None) -> None:
        """bpe_encode_batch on caller-owned device buffers (no allocation, no
        synchronization)."""
        n_bytes = int(data.numel())
        n_docs = int(doc_off.numel()) - 1
        if data.dtype != torch.uint8 or doc_off.dtype != torch.int64 or ids.dtype != torch.int32 \
                or id_off.dtype != torch.int64 or status.dtype != torch.int32:
            raise TypeError("dtypes: data uint8, doc_off int64, ids int32, id_off int64, status int32")
        if n_docs < 0 or id_off.numel() != n_docs + 1:
            raise ValueError("doc_off and id_off need n_docs + 1 entries")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = _lib.load().bpe_encode_batch(
            self._h, _dptr(data) if n_bytes else None, n_bytes, _dptr(doc_off), n_docs,
            _dptr(ids) if ids.numel() else None, int(ids.numel()), _dptr(id_off),
            _dptr(workspace) if ws_bytes else None, ws_bytes, _dptr(status),
            C.c_void_p(_stream_handle(stream)))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_encode_batch")

    def encode_batch_noalloc_into(self, data: torch.Tensor, doc_off: torch.Tensor,
                                  ids: torch.Tensor, id_off: torch.Tensor, status: torch.Tensor,
                                  stream=None) -> None:
        """bpe_encode_batch_noalloc: as encode_batch_into, with the library's
        static scratch as the workspace (inputs up to NOALLOC_SCRATCH_BYTES of
        workspace; calls on one GPU must not overlap)."""
        n_bytes = int(data.numel())
        n_docs = int(doc_off.numel()) - 1
        if data.dtype != torch.uint8 or doc_off.dtype != torch.int64 or ids.dtype != torch.int32 \
                or id_off.dtype != torch.int64 or status.dtype != torch.int32:
            raise TypeError("dtypes: data uint8, doc_off int64, ids int32, id_off int64, status int32")
        if n_docs < 0 or id_off.numel() != n_docs + 1:
            raise ValueError("doc_off and id_off need n_docs + 1 entries")
        rc = _lib.load().bpe_encode_batch_noalloc(
            self._h, _dptr(data) if n_bytes else None, n_bytes, _dptr(doc_off), n_docs,
            _dptr(ids) if ids.numel() else None, int(ids.numel()), _dptr(id_off), _dptr(status),
            C.c_void_p(_stream_handle(stream)))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_encode_batch_noalloc")

    def encode_batch(self, data: torch.Tensor, doc_off: torch.Tensor, ids_capacity: int | None = None,
                     stream=None):
        """Allocate outputs, encode, synchronize, and return (ids[:T], id_off)."""
        dev = data.device
        n_bytes = int(data.numel())
        n_docs = int(doc_off.numel()) - 1
        cap = n_bytes if ids_capacity is None else ids_capacity
        ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)[:cap]
        id_off = torch.empty(n_docs + 1, dtype=torch.int64, device=dev)
        ws = torch.empty(max(1, self.encode_workspace_bytes(n_bytes, n_docs)), dtype=torch.uint8,
                         device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.encode_batch_into(data, doc_off, ids, id_off, ws, status, stream)
        st = int(status.item())
        if st:
            raise RuntimeError(f"bpe_encode_batch device status {st:#x}")
        T = int(id_off[-1].item())
        return ids[:T], id_off

    # ---- encode with reserved IDs around each document --------------------------
    def encode_special_workspace_bytes(self, n_bytes: int, n_docs: int) -> int:
        return int(_lib.load().bpe_encode_special_workspace_bytes(self._h, n_bytes, n_docs))

    def encode_batch_special_into(self, data: torch.Tensor, doc_off: torch.Tensor, bos_id: int,
                                  eos_id: int, ids: torch.Tensor, id_off: torch.Tensor,
                                  workspace: torch.Tensor | None, status: torch.Tensor,
                                  stream=None) -> None:
        """bpe_encode_batch_special on caller-owned device buffers (bos_id / eos_id:
        -1 for none)."""
        n_bytes = int(data.numel())
        n_docs = int(doc_off.numel()) - 1
        if data.dtype != torch.uint8 or doc_off.dtype != torch.int64 or ids.dtype != torch.int32 \
                or id_off.dtype != torch.int64 or status.dtype != torch.int32:
            raise TypeError("dtypes: data uint8, doc_off int64, ids int32, id_off int64, status int32")
        if n_docs < 0 or id_off.numel() != n_docs + 1:
            raise ValueError("doc_off and id_off need n_docs + 1 entries")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = _lib.load().bpe_encode_batch_special(
            self._h, _dptr(data) if n_bytes else None, n_bytes, _dptr(doc_off), n_docs,
            int(bos_id), int(eos_id), _dptr(ids) if ids.numel() else None, int(ids.numel()),
            _dptr(id_off), _dptr(workspace) if ws_bytes else None, ws_bytes, _dptr(status),
            C.c_void_p(_stream_handle(stream)))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_encode_batch_special")

    def encode_batch_special(self, data: torch.Tensor, doc_off: torch.Tensor, bos_id: int = -1,
                             eos_id: int = -1, ids_capacity: int | None = None, stream=None):
        """Allocate outputs, encode with bos_id / eos_id around each document,
        synchronize, and return (ids[:T], id_off)."""
        dev = data.device
        n_bytes = int(data.numel())
        n_docs = int(doc_off.numel()) - 1
        per_doc = int(bos_id >= 0) + int(eos_id >= 0)
        cap = n_bytes + n_docs * per_doc if ids_capacity is None else ids_capacity
        ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)[:cap]
        id_off = torch.empty(n_docs + 1, dtype=torch.int64, device=dev)
        ws = torch.empty(max(1, self.encode_special_workspace_bytes(n_bytes, n_docs)),
                         dtype=torch.uint8, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.encode_batch_special_into(data, doc_off, bos_id, eos_id, ids, id_off, ws, status, stream)
        st = int(status.item())
        if st:
            raise RuntimeError(f"bpe_encode_batch_special device status {st:#x}")
        T = int(id_off[-1].item())
        return ids[:T], id_off

    # ---- decode -------------------------------------------------------------
    def decode_workspace_bytes(self, n_ids: int, n_docs: int) -> int:
        return int(_lib.load().bpe_decode_workspace_bytes(self._h, n_ids, n_docs))

    def decode_batch_into(self, ids: torch.Tensor, id_off: torch.Tensor, out: torch.Tensor,
                          byte_off: torch.Tensor, workspace: torch.Tensor | None,
                          status: torch.Tensor, stream=None, skip=(-1, -1)) -> None:
        """bpe_decode_batch (bpe_decode_batch_special when skip names reserved
        IDs that decode to no bytes)."""
        n_ids = int(ids.numel())
        n_docs = int(id_off.numel()) - 1
        if ids.dtype != torch.int32 or id_off.dtype != torch.int64 or out.dtype != torch.uint8 \
                or byte_off.dtype != torch.int64 or status.dtype != torch.int32:
            raise TypeError("dtypes: ids int32, id_off int64, out uint8, byte_off int64, status int32")
        if n_docs < 0 or byte_off.numel() != n_docs + 1:
            raise ValueError("id_off and byte_off need n_docs + 1 entries")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        skip_a, skip_b = (int(x) for x in skip)
        L = _lib.load()
        if skip_a == -1 and skip_b == -1:
            rc = L.bpe_decode_batch(
                self._h, _dptr(ids) if n_ids else None, n_ids, _dptr(id_off), n_docs,
                _dptr(out) if out.numel() else None, int(out.numel()), _dptr(byte_off),
                _dptr(workspace) if ws_bytes else None, ws_bytes, _dptr(status),
                C.c_void_p(_stream_handle(stream)))
        else:
            rc = L.bpe_decode_batch_special(
                self._h, _dptr(ids) if n_ids else None, n_ids, _dptr(id_off), n_docs, skip_a,
                skip_b, _dptr(out) if out.numel() else None, int(out.numel()), _dptr(byte_off),
                _dptr(workspace) if ws_bytes else None, ws_bytes, _dptr(status),
                C.c_void_p(_stream_handle(stream)))
        if rc != _lib.BPE_OK:
            raise BPEError(rc, "bpe_decode_batch")

    def decode_batch(self, ids: torch.Tensor, id_off: torch.Tensor, bytes_capacity: int | None = None,
                     stream=None, skip=(-1, -1)):
        """Allocate outputs, decode, synchronize, and return (bytes[:N], byte_off)."""
        dev = ids.device
        n_ids = int(ids.numel())
        n_docs = int(id_off.numel()) - 1
        cap = n_ids * max(1, self.max_token_bytes) if bytes_capacity is None else bytes_capacity
        out = torch.empty(max(cap, 1), dtype=torch.uint8, device=dev)[:cap]
        byte_off = torch.empty(n_docs + 1, dtype=torch.int64, device=dev)
        ws = torch.empty(max(1, self.decode_workspace_bytes(n_ids, n_docs)), dtype=torch.uint8,
                         device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.decode_batch_into(ids, id_off, out, byte_off, ws, status, stream, skip)
        st = int(status.item())
        if st:
            raise RuntimeError(f"bpe_decode_batch device status {st:#x}")
        N = int(byte_off[-1].item())
        return out[:N], byte_off
