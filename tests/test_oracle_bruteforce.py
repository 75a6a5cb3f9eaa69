"""Brute force on tiny inputs, and the trainer against its plain definition.

B1: on consistent tables (every operand made by a lower rank), three
    independently written formulations agree with the oracle's loop:
    the merge-order application of 'Characters, bytes and subwords'
    (section 'Train the tokenizer only on training data': the reference
    encoder applies the learned rules in their order), and the single-merge
    minimum over packed (rank, position) keys of 'Hugging Face Tokenizers v1'
    (section 'Merge-loop rewrite').
B2: every sequence of single merges, enumerated: the oracle's result is a
    reachable terminal state, and the lowest-rank-first restriction leaves
    one result unless a pair (x, x) is involved, where the left-to-right
    choice is the oracle's.
B3: the trainer's own segmentation of each training pre-token equals the
    oracle's encoding of it.
B4: the incremental trainer equals the full-recount trainer bit for bit.
"""
import itertools

import numpy as np
import pytest

import oracle as O

A, B, Cc = 97, 98, 99


def random_consistent_table(rng, n_merges, alphabet=(A, B, Cc)):
    syms = list(alphabet)
    seen = set()
    merges = []
    tries = 0
    while len(merges) < n_merges and tries < 1000:
        tries += 1
        l, r = int(rng.choice(syms)), int(rng.choice(syms))
        if (l, r) in seen:
            continue
        seen.add((l, r))
        merges.append([l, r])
        syms.append(256 + len(merges) - 1)
    return merges


# --- independent formulations (written here, not shared with the oracle) ---

def merge_order_apply(merges, s):
    seq = list(s)
    for r, (l, rt) in enumerate(merges):
        out, i = [], 0
        while i < len(seq):
            if i + 1 < len(seq) and seq[i] == l and seq[i + 1] == rt:
                out.append(256 + r)
                i += 2
            else:
                out.append(seq[i])
                i += 1
        seq = out
    return seq


def packed_min_one_at_a_time(merges, s):
    rank = {(l, r): k for k, (l, r) in enumerate(merges)}
    seq = list(s)
    n = len(seq)
    while True:
        best = (1 << 62)
        for i in range(len(seq) - 1):
            k = rank.get((seq[i], seq[i + 1]))
            if k is not None:
                key = (k << 32) | i          # rank in the high bits
                best = min(best, key)
        if best == (1 << 62):
            return seq
        k, i = best >> 32, best & 0xFFFFFFFF
        seq[i:i + 2] = [256 + k]
        assert len(seq) < n + 1


def all_strings(alphabet, max_len):
    for n in range(max_len + 1):
        for combo in itertools.product(alphabet, repeat=n):
            yield bytes(combo)


def test_b1_three_formulations_agree():
    rng = np.random.default_rng(1)
    strings = list(all_strings((A, B, Cc), 7))
    for trial in range(40):
        merges = random_consistent_table(rng, int(rng.integers(1, 7)))
        t = O.Table(merges)
        for s in strings:
            got = t.encode_word(s)
            assert got == merge_order_apply(merges, s), (merges, s)
            assert got == packed_min_one_at_a_time(merges, s), (merges, s)


def test_b1_detects_a_dropped_rule():
    # a plausible mistake (any one rule that fires, dropped) changes a result
    rng = np.random.default_rng(2)
    strings = list(all_strings((A, B, Cc), 6))
    merges = random_consistent_table(rng, 5)
    t = O.Table(merges)
    checked = 0
    for k in range(len(merges)):
        if not any(256 + k in merge_order_apply(merges, s) for s in strings):
            continue
        broken = merges[:k] + [[1, 1]] + merges[k + 1:]
        assert any(t.encode_word(s) != merge_order_apply(broken, s) for s in strings)
        checked += 1
    assert checked >= 2


# --- B2: enumerate merge orders --------------------------------------------

def terminal_states(merges, s, restrict):
    rank = {(l, r): k for k, (l, r) in enumerate(merges)}
    start = tuple(s)
    seen, out, stack = {start}, set(), [start]
    while stack:
        seq = stack.pop()
        moves = [(rank[(seq[i], seq[i + 1])], i) for i in range(len(seq) - 1)
                 if (seq[i], seq[i + 1]) in rank]
        if not moves:
            out.add(seq)
            continue
        if restrict:
            m = min(k for k, _ in moves)
            moves = [(k, i) for k, i in moves if k == m]
        for k, i in moves:
            nxt = seq[:i] + (256 + k,) + seq[i + 2:]
            if nxt not in seen:
                seen.add(nxt)
                stack.append(nxt)
    return out


def leftmost_min_rank(merges, s):
    rank = {(l, r): k for k, (l, r) in enumerate(merges)}
    seq = list(s)
    while True:
        moves = [(rank[(seq[i], seq[i + 1])], i) for i in range(len(seq) - 1)
                 if (seq[i], seq[i + 1]) in rank]
        if not moves:
            return seq
        k, i = min(moves)
        seq[i:i + 2] = [256 + k]


def test_b2_merge_order_enumeration():
    rng = np.random.default_rng(3)
    strings = [s for s in all_strings((A, B), 6)] + [b"abcabc", b"aaaaa", b"cabbac"]
    n_multi = 0
    for trial in range(25):
        merges = random_consistent_table(rng, int(rng.integers(1, 6)))
        t = O.Table(merges)
        has_xx = any(l == r for l, r in merges)
        for s in strings:
            mine = tuple(t.encode_word(s))
            anyorder = terminal_states(merges, s, restrict=False)
            assert mine in anyorder
            prio = terminal_states(merges, s, restrict=True)
            assert mine in prio
            if not has_xx:
                assert prio == {mine}, (merges, s)
            assert tuple(leftmost_min_rank(merges, s)) == mine
            n_multi += len(anyorder) > 1
    # without the priority rule the result is not unique
    assert n_multi > 0


# --- B3/B4: trainer --------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_corpus():
    from workloads import WORKLOADS, make_lexicon, training_corpus
    cfg = WORKLOADS["tiny"]
    return cfg, training_corpus(cfg, make_lexicon(cfg))


def test_b4_incremental_equals_naive_tiny(tiny_corpus):
    cfg, tc = tiny_corpus
    m1, c1 = O.train(tc.data, tc.doc_off, cfg.n_merges, naive=True)
    m2, c2 = O.train(tc.data, tc.doc_off, cfg.n_merges, naive=False)
    assert m1.shape == (cfg.n_merges, 2)
    assert np.array_equal(m1, m2) and np.array_equal(c1, c2)


def test_b4_incremental_equals_naive_random():
    rng = np.random.default_rng(4)
    for trial in range(30):
        words = [bytes(rng.choice(list(b"ab c"), int(rng.integers(1, 9)))) for _ in range(int(rng.integers(1, 30)))]
        docs = [b" ".join(words[i::3]) for i in range(3)]
        m1, c1 = O.train_text(docs, 40, naive=True)
        m2, c2 = O.train_text(docs, 40, naive=False)
        assert np.array_equal(m1, m2) and np.array_equal(c1, c2), docs


def test_trainer_invariants(tiny_corpus):
    cfg, tc = tiny_corpus
    m, c = O.train(tc.data, tc.doc_off, cfg.n_merges)
    assert np.all(np.diff(c) <= 0)              # best count never rises
    assert np.all(c >= 2)
    for r, (l, rt) in enumerate(m):
        assert l < 256 + r and rt < 256 + r     # consistent by construction
    assert O.validate(m) == O.ORA_OK


def test_trainer_hand_computed_ties():
    # (a,b)=2 and (c,d)=2 tie: the smaller pair (97,98) goes first
    m, c = O.train_text([b"ab", b"ab", b"cd", b"cd"], 10)
    assert m.tolist() == [[97, 98], [99, 100]] and c.tolist() == [2, 2]
    m, c = O.train_text([b"ba", b"ba", b"ab", b"ab"], 10)
    assert m.tolist() == [[97, 98], [98, 97]]
    # positional counts: 'aaa' holds (a,a) twice; after the merge, [aa, a]
    m, c = O.train_text([b"aaa", b"aaa"], 10)
    assert m.tolist() == [[97, 97], [256, 97]] and c.tolist() == [4, 2]
    # counts below 2 stop training
    m, c = O.train_text([b"ab", b"cd"], 10)
    assert m.shape[0] == 0


def test_b3_trainer_and_encoder_agree(tiny_corpus):
    cfg, tc = tiny_corpus
    m, _ = O.train(tc.data, tc.doc_off, cfg.n_merges)
    t = O.Table(m)
    words = set(O.split(tc.data.tobytes()))
    for w in sorted(words)[:3000]:
        assert t.encode_word(w) == O.replay_merges(m, w), w
