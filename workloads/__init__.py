"""Seeded synthetic text workloads for byte-level BPE.

This package only draws random text. It contains none of the tokenizer's
arithmetic (no splitting, no merging, no ID mapping), so both the oracle and
the GPU path may consume its output.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    WorkloadConfig,
    Batch,
    make_lexicon,
    training_corpus,
    encode_batch_input,
    small_batch,
)
