"""The oracle against what the pages fix, closed forms and library routines.

Every test here runs on the CPU.  Fixtures with their citations live in
tests/golden/pages_pins.json.
"""
import json
import os
import re

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json"),
                      encoding="utf-8"))


# ---------------------------------------------------------------- split ----

def test_split_hello_world():
    g = GOLD["split_hello_world"]
    got = O.split(g["input_utf8"].encode())
    assert got == [p.encode() for p in g["pretokens_utf8"]]


def _class_by_definition(b: int) -> int:
    # reading R1, restated with Python's own character predicates
    ch = bytes([b])
    if b >= 0x80 or ch.isalpha():
        return O.CLS_L
    if ch.isdigit():
        return O.CLS_D
    if ch in b" \t\n\x0b\x0c\r":
        return O.CLS_W
    return O.CLS_P


def test_byte_classes_exhaustive():
    for b in range(256):
        assert O.byte_class(b) == _class_by_definition(b), b


# Reading R2 as a Python regular expression over bytes: a library routine
# with its own matcher, independent of the oracle's hand-written scanner.
_RE = re.compile(rb" ?[A-Za-z\x80-\xff]+|[0-9]+|[^A-Za-z\x80-\xff0-9\t\n\x0b\x0c\r ]+|[\t\n\x0b\x0c\r ]+")


def _re_split(s: bytes):
    out = _RE.findall(s)
    assert b"".join(out) == s
    return out


def test_split_matches_regex_exhaustive_short():
    alphabet = [b"a", b"\xc3", b"\xa9", b"1", b"!", b" ", b"\t"]
    import itertools
    for n in range(0, 6):
        for combo in itertools.product(alphabet, repeat=n):
            s = b"".join(combo)
            assert O.split(s) == _re_split(s), s


def test_split_matches_regex_random():
    rng = np.random.default_rng(7)
    pool = np.frombuffer(b"aZ \t\n09!.,\x00\x7f\x80\xc3\xa9\xe4\xbd\xa0 ", dtype=np.uint8)
    for _ in range(3000):
        n = int(rng.integers(0, 40))
        if rng.random() < 0.5:
            s = rng.integers(0, 256, n).astype(np.uint8).tobytes()
        else:
            s = pool[rng.integers(0, pool.size, n)].tobytes()
        assert O.split(s) == _re_split(s), s


def test_split_covers_document_exactly():
    rng = np.random.default_rng(11)
    for _ in range(200):
        s = rng.integers(0, 256, int(rng.integers(0, 300))).astype(np.uint8).tobytes()
        parts = O.split(s)
        assert b"".join(parts) == s
        assert all(len(p) > 0 for p in parts)


# ------------------------------------------------------ bytes and unicode ----

def test_utf8_nihao():
    g = GOLD["utf8_nihao"]
    got = b"".join(O.utf8_encode(cp) for cp in g["codepoints"])
    assert got.hex() == g["bytes_hex"]


def test_utf8_matches_python_codec():
    rng = np.random.default_rng(3)
    cps = list(range(0, 0x800, 7)) + list(rng.integers(0x800, 0x110000, 4000))
    for cp in cps:
        cp = int(cp)
        if 0xD800 <= cp <= 0xDFFF:
            assert O.utf8_encode(cp) == b""
            continue
        assert O.utf8_encode(cp) == chr(cp).encode("utf-8"), hex(cp)


def test_byte_to_unicode_pins_and_bijection():
    for b, cp in GOLD["byte_to_unicode"]["pairs"]:
        assert O.byte_to_unicode(b) == chr(cp)
    chars = [O.byte_to_unicode(b) for b in range(256)]
    assert len(set(chars)) == 256
    for c in chars:
        assert c.isprintable() and not c.isspace()
    # the remapped code points are exactly U+0100..U+0143, in byte order
    moved = [ord(c) for b, c in enumerate(chars) if ord(c) != b]
    assert moved == list(range(0x100, 0x144))


# ---------------------------------------------------------------- merges ----

def test_aaa_non_overlapping():
    g = GOLD["aaa_non_overlapping"]
    t = O.Table(g["merges"])
    assert t.encode_word(g["input_utf8"].encode()) == g["symbols"]


def _hello_table():
    g = GOLD["hello_ranked_walk"]
    # ranks 0..10; rank 10 = (h,e) -> symbol 266, rank 5 = (266, l) -> 261,
    # rank 3 = (261, l) -> 259; other ranks: digit pairs absent from 'hello'
    merges = [[48 + r, 48] for r in range(11)]
    sym = {"h": ord("h"), "e": ord("e"), "l": ord("l")}
    sym["he"] = 256 + 10
    sym["hel"] = 256 + 5
    for r, (a, b) in g["ranked_pairs"].items():
        merges[int(r)] = [sym[a], sym[b]]
    return merges


def test_hello_ranked_walk():
    g = GOLD["hello_ranked_walk"]
    t = O.Table(_hello_table())
    assert t.encode_word(b"hello") == g["symbols_derived"]
    assert O.replay_merges(_hello_table(), b"hello") == g["merge_order_application_derived"]
    # the expansion of the result spells the input
    assert t.decode(t.encode_word(b"hello")) == b"hello"


def test_all_occurrences_rule_on_out_of_order_table():
    # (a,a)=1 and (aa,a)=0: the first step merges both (a,a) occurrences
    t = O.Table([[257, 97], [97, 97]])
    assert t.encode_word(b"aaaa") == [257, 257]


def test_run_parity_even_and_odd():
    t = O.Table([[97, 97]])
    for n in range(1, 12):
        assert t.encode_word(b"a" * n) == [256] * (n // 2) + [97] * (n % 2)


def test_fnv_vectors():
    for s, h in GOLD["fnv1a64_vectors"]["vectors"]:
        assert O.fnv1a64(s.encode()) == int(h, 16)


# --------------------------------------------------------- table checks ----

@pytest.mark.parametrize("merges,code", [
    ([[97, 98], [97, 98]], O.ORA_EDUP),
    ([[97, 300]], O.ORA_ERANGE),
    ([[-1, 97]], O.ORA_ERANGE),
    ([[256, 97]], O.ORA_ECYCLE),               # symbol 256 built from itself
    ([[257, 97], [256, 98]], O.ORA_ECYCLE),    # 256 -> 257 -> 256
    ([[97, 98], [256, 99]], O.ORA_OK),
    ([], O.ORA_OK),
])
def test_validate(merges, code):
    assert O.validate(np.array(merges, dtype=np.int32).reshape(-1, 2)) == code


def test_validate_id_map():
    m = [[97, 98]]
    assert O.validate(m, np.arange(257)) == O.ORA_OK
    bad = np.arange(257)
    bad[5] = 6
    assert O.validate(m, bad) == O.ORA_EIDMAP
    bad = np.arange(257)
    bad[0] = -3
    assert O.validate(m, bad) == O.ORA_EIDMAP


# ------------------------------------------------------ batch semantics ----

def _trained_tiny():
    from workloads import WORKLOADS, make_lexicon, training_corpus
    cfg = WORKLOADS["tiny"]
    tc = training_corpus(cfg, make_lexicon(cfg))
    merges, _ = O.train(tc.data, tc.doc_off, cfg.n_merges)
    return merges


@pytest.fixture(scope="module")
def tiny_table():
    return O.Table(_trained_tiny())


def test_round_trip_catalogue(tiny_table):
    for s in GOLD["round_trip_catalogue"]["texts_utf8"]:
        b = s.encode("utf-8")
        ids = tiny_table.encode(b)
        assert tiny_table.decode(ids) == b
        assert all(0 <= i < 256 + tiny_table.R for i in ids)


def test_round_trip_random_bytes(tiny_table):
    rng = np.random.default_rng(5)
    for _ in range(300):
        b = rng.integers(0, 256, int(rng.integers(0, 200))).astype(np.uint8).tobytes()
        assert tiny_table.decode(tiny_table.encode(b)) == b


def test_documents_are_boundaries(tiny_table):
    # R3: merges never cross documents; the batch equals per-document calls
    docs = [b"hello", b"", b"world again", b" x", b"", b"12345 ab"]
    data = np.frombuffer(b"".join(docs), dtype=np.uint8)
    off = np.zeros(len(docs) + 1, dtype=np.int64)
    np.cumsum([len(d) for d in docs], out=off[1:])
    ids, id_off = tiny_table.encode_batch(data, off)
    for d, doc in enumerate(docs):
        assert ids[id_off[d]:id_off[d + 1]].tolist() == tiny_table.encode(doc)
    assert id_off[1] == id_off[2]  # empty document


def test_id_map_permutation(tiny_table):
    # IDs are addresses: a permutation renames every output ID and nothing else
    rng = np.random.default_rng(9)
    V = 256 + tiny_table.R
    perm = rng.permutation(V).astype(np.int32)
    tp = O.Table(tiny_table.merges, perm)
    text = b"the quick brown fox 123 !!"
    assert tp.encode(text) == [int(perm[i]) for i in tiny_table.encode(text)]
    assert tp.decode(tp.encode(text)) == text


def test_save_reload_same_encoder(tmp_path, tiny_table):
    p = tmp_path / "merges.npy"
    np.save(p, tiny_table.merges)
    t2 = O.Table(np.load(p, allow_pickle=False))
    text = "Grüße 🐈 and the lexicon words".encode()
    assert t2.encode(text) == tiny_table.encode(text)


def test_special_token_like_text_stays_text(tiny_table):
    ids = tiny_table.encode(b"<assistant>")
    assert all(i < 256 + tiny_table.R for i in ids)
    assert tiny_table.decode(ids) == b"<assistant>"


# ---- reserved IDs around documents ("Characters, bytes and subwords", section
# "Special tokens are their own IDs": reserved IDs are inserted explicitly,
# EOS marks the end of a document, and on output they may be skipped) ----

def test_special_tokens_wrap_each_document(tiny_table):
    docs = [b"Hello world!", b"", b"the 42 cats"]
    data = np.frombuffer(b"".join(docs), dtype=np.uint8).copy()
    off = np.array([0, 12, 12, 23], dtype=np.int64)
    V = 256 + tiny_table.R
    bos, eos = V + 1, V + 7
    ids, id_off = tiny_table.encode_batch_special(data, off, bos, eos)
    for d, doc in enumerate(docs):
        assert ids[id_off[d]:id_off[d + 1]].tolist() == [bos] + tiny_table.encode(doc) + [eos]
    # an empty document is [bos, eos]; offsets move by two per document
    assert ids[id_off[1]:id_off[2]].tolist() == [bos, eos]
    plain_ids, plain_off = tiny_table.encode_batch(data, off)
    assert np.array_equal(id_off, plain_off + 2 * np.arange(len(docs) + 1))
    assert ids.size == plain_ids.size + 2 * len(docs)


@pytest.mark.parametrize("bos,eos", [(-1, -1), (1000, -1), (-1, 1001), (1000, 1001)])
def test_special_tokens_one_side_and_round_trip(tiny_table, bos, eos):
    docs = [b"a", b"  spaces  ", b"", b"\xf0\x9f\x90\x88 cat"]
    data = np.frombuffer(b"".join(docs), dtype=np.uint8).copy()
    off = np.zeros(len(docs) + 1, dtype=np.int64)
    np.cumsum([len(x) for x in docs], out=off[1:])
    ids, id_off = tiny_table.encode_batch_special(data, off, bos, eos)
    plain, plain_off = tiny_table.encode_batch(data, off)
    n = int(bos >= 0) + int(eos >= 0)
    assert np.array_equal(id_off, plain_off + n * np.arange(len(docs) + 1))
    for d in range(len(docs)):
        seg = ids[id_off[d]:id_off[d + 1]].tolist()
        body = seg[1:] if bos >= 0 else seg
        body = body[:-1] if eos >= 0 else body
        assert body == plain[plain_off[d]:plain_off[d + 1]].tolist()
        if bos >= 0:
            assert seg[0] == bos
        if eos >= 0:
            assert seg[-1] == eos
    out, boff = tiny_table.decode_batch_special(ids, id_off, (bos, eos))
    assert out.tobytes() == data.tobytes() and np.array_equal(boff, off)
