"""The text form of a table (merges file and vocabulary JSON), parsed by the
library on the host (bpe_parse_merges_text, bpe_parse_vocab_json) and by the
oracle, against each other and against what the pages fix ("Tokenization
LLM: details of building an inference engine in C++", sections "Byte-level
encoding": 0xF0 prints as 'ð', and "Vocabulary lookup": " world" is
"Ġworld").  No GPU needed."""
import os

import numpy as np
import pytest

import oracle as O
from byte_level_bpe_pretokenize_amd import BPEError, _lib, parse_merges_text, parse_vocab_json

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def merges_of(name):
    return np.load(os.path.join(ROOT, "assets", f"merges_{name}.npy"), allow_pickle=False)


def code(fn):
    with pytest.raises(BPEError) as e:
        fn()
    return e.value.code


def test_printed_bytes_of_the_pages():
    # " world": the space prints as 'Ġ', so the merge of the space and 'w' is "Ġ w"
    m = parse_merges_text("Ġ w\nĠw o\n")
    assert m.tolist() == [[32, 119], [256, 111]]
    # 0xF0 prints as U+00F0 'ð'
    assert parse_merges_text("ð ð\n").tolist() == [[0xF0, 0xF0]]


@pytest.mark.parametrize("name", ["tiny", "throughput", "serving"])
def test_merges_round_trip(name):
    m = merges_of(name)
    text = O.merges_to_text(m)
    assert np.array_equal(parse_merges_text(text), m)          # the library
    assert np.array_equal(O.parse_merges_text(text), m)        # the oracle
    # CRLF line ends and blank lines read the same
    crlf = text.replace("\n", "\r\n") + "\r\n\r\n"
    assert np.array_equal(parse_merges_text(crlf), m)


@pytest.mark.parametrize("ascii_only", [True, False])
def test_vocab_round_trip(ascii_only):
    m = merges_of("tiny")
    rng = np.random.default_rng(3)
    id_map = (rng.permutation(256 + m.shape[0]) * 3 + 7).astype(np.int32)
    # extra keys: a reserved ID's name (its characters print as bytes, but
    # no symbol has these bytes) and text outside the printable map
    js = O.vocab_to_json(m, id_map, ensure_ascii=ascii_only,
                         extra={"<|endoftext|>": 99999, "一二": 5})
    got = parse_vocab_json(js, m)
    assert np.array_equal(got, id_map)
    assert np.array_equal(O.parse_vocab_json(js, m), id_map)


def test_vocab_ids_of_a_small_table():
    m = parse_merges_text("#version: 0.2\nĠ w\no r\nĠw or\nl d\nĠwor ld\nh e\nl l\nhe ll\nhell o\n")
    V = 256 + m.shape[0]
    vocab = {O.bytes_to_text(bytes([b])): 1000 + b for b in range(256)}
    vocab.update({"Ġw": 1, "or": 2, "Ġwor": 3, "ld": 4, "Ġworld": 1917, "he": 5, "ll": 6,
                  "hell": 7, "hello": 15339})
    import json
    ids = parse_vocab_json(json.dumps(vocab), m)
    assert ids.size == V
    assert ids[256 + 4] == 1917 and ids[256 + 8] == 15339 and ids[32] == 1032


@pytest.mark.parametrize("text,err", [
    ("a b c\n", _lib.BPE_EFORMAT),      # two spaces
    ("ab\n", _lib.BPE_EFORMAT),         # no space
    (" a\n", _lib.BPE_EFORMAT),         # empty operand
    ("一 a\n", _lib.BPE_EFORMAT),       # a character no byte prints as
    ("ab c\n", _lib.BPE_EMERGES),       # "ab" is not a byte nor an earlier result
    ("a b\nb c\nab c\na bc\n", _lib.BPE_EMERGES),  # "abc" twice
])
def test_merges_text_errors(text, err):
    assert code(lambda: parse_merges_text(text)) == err


def test_merges_text_bad_utf8():
    assert code(lambda: parse_merges_text(b"a \xff\n")) == _lib.BPE_EFORMAT


def test_version_line_only_first():
    # "#version" is a header only on the first line; later a '#' is a byte
    m = parse_merges_text("#version: 0.2\n# #\n")
    assert m.tolist() == [[35, 35]]


def test_vocab_json_errors():
    m = parse_merges_text("a b\n")
    full = {O.bytes_to_text(bytes([b])): b for b in range(256)}
    import json
    missing = json.dumps(full)                        # no entry for "ab"
    assert code(lambda: parse_vocab_json(missing, m)) == _lib.BPE_EIDMAP
    full["ab"] = -4                                   # negative ID
    assert code(lambda: parse_vocab_json(json.dumps(full), m)) == _lib.BPE_EIDMAP
    full["ab"] = 300
    ok = json.dumps(full)
    assert parse_vocab_json(ok, m)[256] == 300
    assert code(lambda: parse_vocab_json(ok[:-1], m)) == _lib.BPE_EFORMAT      # unterminated
    assert code(lambda: parse_vocab_json("[1, 2]", m)) == _lib.BPE_EFORMAT
