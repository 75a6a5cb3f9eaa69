"""Seeded synthetic text for the five byte-level BPE workloads.

Every random draw comes from numpy's PCG64 generator, seeded from the table
in ``WORKLOADS``.  The output is raw bytes plus document offsets; nothing here
splits, merges or maps tokens.

Recipe (one reading of the workload descriptions, stated once here):

* Lexicon: ``lexicon_size`` distinct words, each ``U{1..10}`` codepoints long,
  drawn with the lexicon seed and shared by the training corpus and the text
  to encode.  Alphabet ``ascii_lower`` uses a-z.  Alphabet ``multilingual``
  draws each codepoint as an ASCII letter (A-Z a-z, p=0.60), from
  U+00C0..U+06FF (p=0.15), from U+4E00..U+9FFF (p=0.20) or from
  U+1F300..U+1F5FF (p=0.05).
* Slots: a word (p=0.90, Zipf: P(rank k) proportional to k**-s, the lexicon's
  order being the rank), one of the 32 ASCII punctuation characters (p=0.05),
  or a run of U{1..6} iid decimal digits (p=0.05).  Word occurrences get an
  upper-case first letter with probability ``cap_prob``.  Each slot is
  followed by one space (0x20).
* Pathological slots (encode input only, fraction ``patho_frac`` of slots):
  half are one letter a-z repeated U{64..4096} times, half are runs of
  U{1..2048} iid digits.
* A document of size S takes the next S bytes of the slot stream, backs the
  cut off to a whole UTF-8 codepoint, and pads with 0x20 to exactly S bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KiB = 1 << 10
MiB = 1 << 20

# The 32 printable ASCII characters that are neither letters, digits nor space.
PUNCT = np.frombuffer(b"!\"#$%&'()*+,-./:;<=>?@[\\]^_`{|}~", dtype=np.uint8).copy()
assert PUNCT.size == 32


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    n_merges: int
    train_bytes: int
    lexicon_size: int
    zipf_s: float
    alphabet: str
    cap_prob: float
    lexicon_seed: int
    train_seed: int
    encode_seed: int
    doc_sizes: str          # "fixed" or "lognormal"
    n_docs: int
    doc_bytes: int          # document size when doc_sizes == "fixed"
    patho_frac: float = 0.0


WORKLOADS = {
    "tiny": WorkloadConfig("tiny", 512, 64 * KiB, 2000, 1.10, "ascii_lower", 0.0,
                      101, 201, 301, "fixed", 1, 1 * MiB),
    "throughput": WorkloadConfig("throughput", 32000, 16 * MiB, 50000, 1.05, "ascii_lower", 0.10,
                      102, 202, 302, "fixed", 4096, 64 * KiB),
    "multilingual": WorkloadConfig("multilingual", 50000, 32 * MiB, 50000, 1.05, "multilingual", 0.0,
                      103, 203, 303, "fixed", 16384, 64 * KiB),
    "adversarial": WorkloadConfig("adversarial", 128000, 64 * MiB, 50000, 1.05, "multilingual", 0.0,
                      104, 204, 304, "fixed", 16384, 64 * KiB, patho_frac=0.01),
    "serving": WorkloadConfig("serving", 100000, 64 * MiB, 50000, 1.05, "multilingual", 0.0,
                      105, 205, 305, "lognormal", 65536, 0),
}


@dataclass
class Batch:
    data: np.ndarray     # uint8 [n_bytes], documents back to back
    doc_off: np.ndarray  # int64 [n_docs + 1], doc_off[0] == 0, doc_off[-1] == n_bytes

    @property
    def n_bytes(self) -> int:
        return int(self.data.size)

    @property
    def n_docs(self) -> int:
        return int(self.doc_off.size - 1)

    def doc(self, d: int) -> bytes:
        return self.data[self.doc_off[d]:self.doc_off[d + 1]].tobytes()


@dataclass
class Lexicon:
    blob: np.ndarray     # uint8, all words back to back
    off: np.ndarray      # int64 [V + 1]
    cdf: np.ndarray      # float64 [V], unnormalised cumulative Zipf weights

    @property
    def lens(self) -> np.ndarray:
        return np.diff(self.off)


def _draw_codepoints(rng: np.random.Generator, alphabet: str, n: int) -> list[int]:
    if alphabet == "ascii_lower":
        return list(rng.integers(ord("a"), ord("z") + 1, n))
    cat = rng.choice(4, size=n, p=[0.60, 0.15, 0.20, 0.05])
    out = []
    for c in cat:
        if c == 0:
            k = int(rng.integers(0, 52))
            out.append(ord("A") + k if k < 26 else ord("a") + k - 26)
        elif c == 1:
            out.append(int(rng.integers(0x00C0, 0x06FF + 1)))
        elif c == 2:
            out.append(int(rng.integers(0x4E00, 0x9FFF + 1)))
        else:
            out.append(int(rng.integers(0x1F300, 0x1F5FF + 1)))
    return out


def make_lexicon(cfg: WorkloadConfig) -> Lexicon:
    rng = np.random.Generator(np.random.PCG64(cfg.lexicon_seed))
    seen: set[bytes] = set()
    words: list[bytes] = []
    while len(words) < cfg.lexicon_size:
        n = int(rng.integers(1, 11))
        w = "".join(chr(c) for c in _draw_codepoints(rng, cfg.alphabet, n)).encode("utf-8")
        if w in seen:
            continue
        seen.add(w)
        words.append(w)
    lens = np.fromiter((len(w) for w in words), dtype=np.int64, count=len(words))
    off = np.zeros(len(words) + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    blob = np.frombuffer(b"".join(words), dtype=np.uint8).copy()
    k = np.arange(1, cfg.lexicon_size + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-cfg.zipf_s))
    return Lexicon(blob, off, cdf)


def _ragged_positions(starts: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Flat indices start[i] + j for j < lens[i], concatenated in order."""
    total = int(lens.sum())
    if total == 0:
        return np.zeros(0, dtype=np.int64)
    excl = np.zeros(lens.size, dtype=np.int64)
    np.cumsum(lens[:-1], out=excl[1:])
    return np.repeat(starts - excl, lens) + np.arange(total, dtype=np.int64)


def _slot_block(rng: np.random.Generator, cfg: WorkloadConfig, lex: Lexicon,
                n: int, patho_frac: float) -> np.ndarray:
    """n slots, each followed by one space, as a uint8 array."""
    u_type = rng.random(n)
    u_word = rng.random(n)
    u_cap = rng.random(n) if cfg.cap_prob > 0 else None
    punct_idx = rng.integers(0, 32, n)
    dig_len = rng.integers(1, 7, n)
    is_word = u_type < 0.90
    is_punct = (u_type >= 0.90) & (u_type < 0.95)
    is_dig = u_type >= 0.95
    is_prun = np.zeros(n, dtype=bool)
    is_pdig = np.zeros(n, dtype=bool)
    if patho_frac > 0:
        u_patho = rng.random(n)
        u_kind = rng.random(n)
        letter = rng.integers(0, 26, n)
        run_len = rng.integers(64, 4097, n)
        pdig_len = rng.integers(1, 2049, n)
        patho = u_patho < patho_frac
        is_prun = patho & (u_kind < 0.5)
        is_pdig = patho & (u_kind >= 0.5)
        is_word &= ~patho
        is_punct &= ~patho
        is_dig &= ~patho

    widx = np.searchsorted(lex.cdf, u_word * lex.cdf[-1], side="right")
    np.minimum(widx, lex.cdf.size - 1, out=widx)
    lens = np.ones(n, dtype=np.int64)
    wl = lex.lens
    lens[is_word] = wl[widx[is_word]]
    lens[is_dig] = dig_len[is_dig]
    if patho_frac > 0:
        lens[is_prun] = run_len[is_prun]
        lens[is_pdig] = pdig_len[is_pdig]
    slot_len = lens + 1
    start = np.zeros(n, dtype=np.int64)
    np.cumsum(slot_len[:-1], out=start[1:])
    out = np.full(int(slot_len.sum()), 0x20, dtype=np.uint8)

    # words
    ws = start[is_word]
    wlen = lens[is_word]
    dst = _ragged_positions(ws, wlen)
    src = _ragged_positions(lex.off[widx[is_word]], wlen)
    out[dst] = lex.blob[src]
    if u_cap is not None:
        cap = is_word & (u_cap < cfg.cap_prob)
        out[start[cap]] -= 32  # a-z words: first byte becomes A-Z
    # punctuation
    out[start[is_punct]] = PUNCT[punct_idx[is_punct]]
    # digit runs (regular and pathological)
    dmask = is_dig | is_pdig
    dpos = _ragged_positions(start[dmask], lens[dmask])
    out[dpos] = (48 + rng.integers(0, 10, dpos.size)).astype(np.uint8)
    # single-letter runs
    if is_prun.any():
        rpos = _ragged_positions(start[is_prun], lens[is_prun])
        out[rpos] = np.repeat((97 + letter[is_prun]).astype(np.uint8), lens[is_prun])
    return out


def _stream(rng: np.random.Generator, cfg: WorkloadConfig, lex: Lexicon,
            n_bytes: int, patho_frac: float) -> np.ndarray:
    blocks = []
    have = 0
    block = int(min(1 << 20, max(64, n_bytes // 3)))
    while have < n_bytes:
        b = _slot_block(rng, cfg, lex, block, patho_frac)
        blocks.append(b)
        have += b.size
    s = np.concatenate(blocks) if len(blocks) > 1 else blocks[0]
    return s


def _cut_docs(stream: np.ndarray, sizes: np.ndarray) -> Batch:
    doc_off = np.zeros(sizes.size + 1, dtype=np.int64)
    np.cumsum(sizes, out=doc_off[1:])
    out = np.full(int(doc_off[-1]), 0x20, dtype=np.uint8)
    pos = 0
    for d in range(sizes.size):
        size = int(sizes[d])
        cut = pos + size
        # back the cut off to the first byte of a codepoint
        while cut > pos and cut < stream.size and (stream[cut] & 0xC0) == 0x80:
            cut -= 1
        take = cut - pos
        o = int(doc_off[d])
        out[o:o + take] = stream[pos:cut]
        pos = cut
    return Batch(out, doc_off)


def training_corpus(cfg: WorkloadConfig, lex: Lexicon | None = None) -> Batch:
    """The training text: one document of ``cfg.train_bytes`` bytes."""
    lex = lex if lex is not None else make_lexicon(cfg)
    rng = np.random.Generator(np.random.PCG64(cfg.train_seed))
    stream = _stream(rng, cfg, lex, cfg.train_bytes + 64, 0.0)
    return _cut_docs(stream, np.array([cfg.train_bytes], dtype=np.int64))


def _doc_sizes(rng: np.random.Generator, cfg: WorkloadConfig, n_docs: int,
               doc_bytes: int) -> np.ndarray:
    if cfg.doc_sizes == "lognormal":
        v = np.rint(np.exp(rng.normal(6.0, 1.0, n_docs)))
        return np.clip(v, 32, 8192).astype(np.int64)
    return np.full(n_docs, doc_bytes, dtype=np.int64)


def encode_batch_input(cfg: WorkloadConfig, lex: Lexicon | None = None,
                       n_docs: int | None = None) -> Batch:
    """The text to encode.  ``n_docs`` takes a prefix-shaped subset of the
    documents (same seed, same sizes, fewer of them) for smaller runs."""
    lex = lex if lex is not None else make_lexicon(cfg)
    rng = np.random.Generator(np.random.PCG64(cfg.encode_seed))
    sizes = _doc_sizes(rng, cfg, cfg.n_docs, cfg.doc_bytes)
    if n_docs is not None:
        sizes = sizes[:n_docs]
    stream = _stream(rng, cfg, lex, int(sizes.sum()) + 64, cfg.patho_frac)
    return _cut_docs(stream, sizes)


def small_batch(cfg: WorkloadConfig, n_docs: int, doc_bytes: int, seed: int,
                lex: Lexicon | None = None, patho_frac: float | None = None) -> Batch:
    """A batch in the style of ``cfg`` with a caller-chosen shape and seed."""
    lex = lex if lex is not None else make_lexicon(cfg)
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg.doc_sizes == "lognormal":
        sizes = _doc_sizes(rng, cfg, n_docs, doc_bytes)
    else:
        sizes = np.full(n_docs, doc_bytes, dtype=np.int64)
    pf = cfg.patho_frac if patho_frac is None else patho_frac
    stream = _stream(rng, cfg, lex, int(sizes.sum()) + 64, pf)
    return _cut_docs(stream, sizes)
