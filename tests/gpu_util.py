"""Helpers for the GPU parity tests: device buffers, oracle comparison."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle as O
from byte_level_bpe_pretokenize_amd import Model, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def merges_for(name: str) -> np.ndarray:
    return np.load(os.path.join(ROOT, "assets", f"merges_{name}.npy"), allow_pickle=False)


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a visible HIP device"
    return torch.device("cuda", 0)


def batch_from_docs(docs: list[bytes]):
    data = np.frombuffer(b"".join(docs), dtype=np.uint8).copy() if any(docs) else np.zeros(0, np.uint8)
    off = np.zeros(len(docs) + 1, dtype=np.int64)
    np.cumsum([len(d) for d in docs], out=off[1:])
    return data, off


def gpu_encode(model: Model, data: np.ndarray, doc_off: np.ndarray, cap: int | None = None,
               data_offset: int = 0):
    """Encode through the C ABI; returns (ids[:min(T,cap)], id_off, status)."""
    dev = model.device
    n = data.size
    if data_offset:
        buf = torch.zeros(n + data_offset, dtype=torch.uint8, device=dev)
        buf[data_offset:] = torch.from_numpy(data).to(dev)
        d_data = buf[data_offset:]
    else:
        d_data = torch.from_numpy(data).to(dev) if n else torch.zeros(0, dtype=torch.uint8, device=dev)
    d_off = torch.from_numpy(np.ascontiguousarray(doc_off)).to(dev)
    cap = n if cap is None else cap
    ids = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev)[:cap]
    id_off = torch.full((doc_off.size,), -7, dtype=torch.int64, device=dev)
    ws_bytes = model.encode_workspace_bytes(n, doc_off.size - 1)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev) if ws_bytes else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    model.encode_batch_into(d_data, d_off, ids, id_off, ws, status)
    torch.cuda.synchronize()
    st = int(status.item())
    off = id_off.cpu().numpy()
    T = int(off[-1]) if st == 0 else min(cap, n)
    return ids[:min(T, cap)].cpu().numpy(), off, st


def check_encode(model: Model, table: O.Table, data: np.ndarray, doc_off: np.ndarray, **kw):
    got, got_off, st = gpu_encode(model, data, doc_off, **kw)
    assert st == 0, f"device status {st:#x}"
    want, want_off = table.encode_batch(data, doc_off)
    assert np.array_equal(got_off, want_off), _first_diff(got_off, want_off)
    assert got.size == want.size, (got.size, want.size)
    if not np.array_equal(got, want):
        raise AssertionError("ids differ: " + _first_diff(got, want))
    assert O.ids_fnv(got) == O.ids_fnv(want)
    return got, got_off


def _first_diff(a: np.ndarray, b: np.ndarray) -> str:
    n = min(a.size, b.size)
    idx = np.nonzero(a[:n] != b[:n])[0]
    i = int(idx[0]) if idx.size else n
    return f"sizes {a.size}/{b.size}, first difference at {i}: {a[i:i + 8]} vs {b[i:i + 8]}"


def gpu_decode(model: Model, ids: np.ndarray, id_off: np.ndarray, cap: int | None = None):
    dev = model.device
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev) if ids.size else \
        torch.zeros(0, dtype=torch.int32, device=dev)
    d_off = torch.from_numpy(np.ascontiguousarray(id_off, dtype=np.int64)).to(dev)
    if cap is None:
        cap = ids.size * max(1, model.max_token_bytes)
    out = torch.zeros((max(cap, 1),), dtype=torch.uint8, device=dev)[:cap]
    byte_off = torch.full((id_off.size,), -7, dtype=torch.int64, device=dev)
    ws_bytes = model.decode_workspace_bytes(ids.size, id_off.size - 1)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev) if ws_bytes else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    model.decode_batch_into(d_ids, d_off, out, byte_off, ws, status)
    torch.cuda.synchronize()
    st = int(status.item())
    boff = byte_off.cpu().numpy()
    N = int(boff[-1]) if st == 0 else cap
    return out[:min(N, cap)].cpu().numpy(), boff, st


STATUS = _lib
