"""MI355X byte-level BPE encode/decode behind a C ABI (libbpe.so).

Python side: ``Model`` marshals torch device tensors into the C calls.
"""
from .api import BPEError, Model, parse_merges_text, parse_vocab_json, train  # noqa: F401
from . import _lib  # noqa: F401
