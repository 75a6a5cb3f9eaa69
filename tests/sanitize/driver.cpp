// Host-code check under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
// only): the oracle (oracle/bpe_oracle.c), the library's text-form parsers
// (bpe_text.cpp) and its hash-table placement (bpe_tables.cpp) on seeded
// random tables and inputs, their error paths included.  Every placed key
// must be found by the rule the kernels probe with.  Built and run by
// tests/test_sanitizers.py; any report of either sanitizer aborts with a
// non-zero status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <string>
#include <unordered_set>
#include <vector>

#include "bpe.h"
#include "bpe_internal.h"

extern "C" {
int64_t ora_split(const uint8_t *s, int64_t n, int64_t *starts);
int ora_byte_to_unicode(int b);
int ora_utf8_encode(uint32_t cp, uint8_t *out);
uint64_t ora_fnv1a64(const uint8_t *p, int64_t n);
int ora_validate(const int32_t *merges, int64_t R, const int32_t *id_map);
void *ora_table_new(const int32_t *merges, int64_t R, const int32_t *id_map);
void ora_table_free(void *h);
int64_t ora_encode_word(const void *h, const uint8_t *w, int64_t n, int32_t *out);
int64_t ora_encode_batch(const void *h, const uint8_t *data, int64_t n_bytes, const int64_t *doc_off,
                         int64_t n_docs, int32_t *ids, int64_t ids_cap, int64_t *id_off);
int64_t ora_decode_batch(const void *h, const int32_t *ids, int64_t n_ids, const int64_t *id_off,
                         int64_t n_docs, uint8_t *out, int64_t out_cap, int64_t *byte_off);
int64_t ora_train(const uint8_t *data, int64_t n_bytes, const int64_t *doc_off, int64_t n_docs,
                  int64_t n_merges, int32_t *merges_out, int64_t *counts_out, int naive);
int64_t ora_replay_merges(const int32_t *merges, int64_t R, const uint8_t *w, int64_t n,
                          int32_t *out);
}

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      exit(3);                                                        \
    }                                                                 \
  } while (0)

static std::mt19937_64 rng(20261202);

// Random documents from a small alphabet that covers every byte class.
static void random_docs(std::vector<uint8_t> &data, std::vector<int64_t> &off, int n_docs,
                        int max_len) {
  static const uint8_t alpha[] = {'a', 'b', 'a', 'b', 'c', ' ', ' ', '1', '2', '!', '\t', 0xC3, 0xA9};
  data.clear();
  off.assign(1, 0);
  for (int d = 0; d < n_docs; ++d) {
    const int n = (int)(rng() % (uint64_t)(max_len + 1));
    for (int i = 0; i < n; ++i) data.push_back(alpha[rng() % sizeof(alpha)]);
    off.push_back((int64_t)data.size());
  }
}

// The text of symbol v's bytes in the printable map.
static std::string sym_text(const std::vector<std::string> &exp, int32_t v) {
  std::string t;
  for (unsigned char c : exp[(size_t)v]) {
    uint8_t u[4];
    const int k = ora_utf8_encode((uint32_t)ora_byte_to_unicode(c), u);
    t.append((const char *)u, (size_t)k);
  }
  return t;
}

// The word tables' and the rank table's placement: every key is found where
// the kernels look for it (short table: its one slot; long table: its first
// or second slot; rank table: its first bucket, or its second when the first
// bucket's flag is set), and no slot holds two keys.
static void check_tables() {
  for (int n : {1, 7, 300, 5000, 40000}) {
    uint32_t mask = 255;
    while ((int64_t)mask + 1 < 2 * (int64_t)n) mask = 2 * mask + 1;
    int dbits = 0;
    while (((uint64_t)bpe::kShortSlotsPerDisp << dbits) < (uint64_t)mask + 1) ++dbits;
    std::vector<uint32_t> h((size_t)n), st((size_t)n);
    for (int i = 0; i < n; ++i) {
      h[(size_t)i] = (uint32_t)rng();
      st[(size_t)i] = bpe::short_step((uint32_t)rng(), (uint32_t)rng(), (uint32_t)rng());
    }
    std::vector<int32_t> at;
    std::vector<uint8_t> disp;
    CHECK(bpe::place_displaced(h, st, mask, dbits, at, disp));
    CHECK(at.size() == (size_t)mask + 1 && disp.size() == (size_t)1 << dbits);
    int64_t used = 0;
    for (int32_t e : at) used += e >= 0;
    CHECK(used == n);
    for (int i = 0; i < n; ++i) {
      const uint32_t d = disp[h[(size_t)i] >> (32 - dbits)];
      CHECK(at[bpe::short_slot(h[(size_t)i], d, st[(size_t)i], mask)] == i);
    }
    // the long table's two choices, at 2.5 slots per key
    uint32_t lmask = 255;
    while ((int64_t)lmask + 1 < 5 * (int64_t)n / 2) lmask = 2 * lmask + 1;
    CHECK(bpe::place_words(h, lmask, at));
    used = 0;
    for (int32_t e : at) used += e >= 0;
    CHECK(used == n);
    for (int i = 0; i < n; ++i)
      CHECK(at[bpe::word_slot0(h[(size_t)i], lmask)] == i ||
            at[bpe::word_slot1(h[(size_t)i], lmask)] == i);
  }
  // the rank table: distinct pair keys in rank order, at most half full
  for (int n : {1, 100, 20000}) {
    std::vector<uint64_t> keys;
    std::unordered_set<uint64_t> seen;
    while ((int)keys.size() < n) {
      const uint32_t l = (uint32_t)(rng() % 70000), r = (uint32_t)(rng() % 70000);
      const uint64_t k = bpe::pair_key(l, r);
      if (seen.insert(k).second) keys.push_back(k);
    }
    uint32_t mask = 63;
    while ((int64_t)mask + 1 < (int64_t)n) mask = 2 * mask + 1;
    const uint32_t seed = 0x9E3779B9u;
    std::vector<uint64_t> slots;
    CHECK(bpe::build_rank_table(keys, mask, seed, slots));
    for (int r = 0; r < n; ++r) {
      const uint64_t k = keys[(size_t)r];
      const uint32_t x = bpe::pair_mix((uint32_t)(k >> bpe::kSymBits),
                                       (uint32_t)(k & ((1u << bpe::kSymBits) - 1)), seed);
      auto find = [&](uint32_t b) {
        for (int j = 0; j < 2; ++j) {
          const uint64_t v = slots[2 * (size_t)b + j];
          if (v != bpe::kEmptySlot && (v >> bpe::kSymBits) == k)
            return (int64_t)(v & ((1u << 20) - 1));
        }
        return (int64_t)-1;
      };
      const uint32_t b0 = bpe::pair_bucket0(x, mask);
      int64_t got = find(b0);
      if (got < 0 && (slots[2 * (size_t)b0] & bpe::kSlotFlag)) got = find(bpe::pair_bucket1(x, mask));
      CHECK(got == r);
    }
  }
  // window radii: digits '1' '2' -> 256, (256, '3') -> 257 give the digit
  // class radius 3 and the others 1; a merge that uses a later symbol
  // gives 0 everywhere
  {
    const int32_t m[4] = {'1', '2', 256, '3'};
    std::vector<int64_t> len(258, 1);
    len[256] = 2;
    len[257] = 3;
    int32_t wd[4];
    bpe::window_radii(m, 2, len, {256, 257}, wd);
    CHECK(wd[bpe::kD] == 3 && wd[bpe::kL] == 1 && wd[bpe::kW] == 1 && wd[bpe::kP] == 1);
    const int32_t bad[4] = {'1', 257, '2', '3'};
    bpe::window_radii(bad, 2, len, {257, 256}, wd);
    CHECK(wd[0] == 0 && wd[1] == 0 && wd[2] == 0 && wd[3] == 0);
  }
}

int main() {
  check_tables();
  for (int round = 0; round < 40; ++round) {
    // a table trained by the oracle on a random corpus
    std::vector<uint8_t> data;
    std::vector<int64_t> off;
    random_docs(data, off, 20, 200);
    const int64_t want = 1 + (int64_t)(rng() % 60);
    std::vector<int32_t> merges((size_t)(2 * want));
    std::vector<int64_t> counts((size_t)want);
    const int64_t R = ora_train(data.empty() ? nullptr : data.data(), (int64_t)data.size(),
                                off.data(), (int64_t)off.size() - 1, want, merges.data(),
                                counts.data(), (int)(round & 1));
    CHECK(R >= 0 && R <= want);
    merges.resize((size_t)(2 * R));
    CHECK(ora_validate(R ? merges.data() : nullptr, R, nullptr) == 0);
    void *t = ora_table_new(R ? merges.data() : nullptr, R, nullptr);
    CHECK(t != nullptr);

    // encode and decode a fresh batch; the round trip holds
    random_docs(data, off, 30, 300);
    const int64_t nd = (int64_t)off.size() - 1, N = (int64_t)data.size();
    std::vector<int32_t> ids((size_t)(N ? N : 1));
    std::vector<int64_t> ioff((size_t)(nd + 1));
    const int64_t T = ora_encode_batch(t, N ? data.data() : nullptr, N, off.data(), nd, ids.data(),
                                       N, ioff.data());
    CHECK(T >= 0 && T <= N);
    std::vector<uint8_t> back((size_t)(N ? N : 1));
    std::vector<int64_t> boff((size_t)(nd + 1));
    CHECK(ora_decode_batch(t, ids.data(), T, ioff.data(), nd, back.data(), N, boff.data()) == N);
    CHECK(N == 0 || memcmp(back.data(), data.data(), (size_t)N) == 0);
    // too little room, bad offsets and an unknown ID are reported, not overrun
    if (T > 1) {
      CHECK(ora_encode_batch(t, data.data(), N, off.data(), nd, ids.data(), T - 1, ioff.data()) == -1);
      CHECK(ora_decode_batch(t, ids.data(), T, ioff.data(), nd, back.data(), N - 1, boff.data()) == -1);
      std::vector<int32_t> bad(ids.begin(), ids.begin() + T);
      bad[0] = 256 + (int32_t)R + 7;
      CHECK(ora_decode_batch(t, bad.data(), T, ioff.data(), nd, back.data(), N, boff.data()) == -3);
    }
    // each pre-token: the encoder's symbols equal the trainer's replay
    std::vector<int64_t> st((size_t)(N ? N : 1));
    for (int64_t d = 0; d < nd; ++d) {
      const uint8_t *doc = data.data() + off[(size_t)d];
      const int64_t n = off[(size_t)d + 1] - off[(size_t)d];
      const int64_t k = ora_split(doc, n, st.data());
      for (int64_t j = 0; j < k; ++j) {
        const int64_t a = st[(size_t)j], b = j + 1 < k ? st[(size_t)j + 1] : n;
        std::vector<int32_t> x((size_t)(b - a)), y((size_t)(b - a));
        const int64_t nx = ora_encode_word(t, doc + a, b - a, x.data());
        const int64_t ny = ora_replay_merges(R ? merges.data() : nullptr, R, doc + a, b - a, y.data());
        CHECK(nx == ny && memcmp(x.data(), y.data(), sizeof(int32_t) * (size_t)nx) == 0);
      }
    }

    // the text form: a merges file and a vocabulary parsed back by the library
    std::vector<std::string> exp(256 + (size_t)R);
    for (int b = 0; b < 256; ++b) exp[(size_t)b] = std::string(1, (char)b);
    for (int64_t r = 0; r < R; ++r)
      exp[256 + (size_t)r] = exp[(size_t)merges[2 * r]] + exp[(size_t)merges[2 * r + 1]];
    std::string text = "#version: 0.2\n";
    for (int64_t r = 0; r < R; ++r)
      text += sym_text(exp, merges[2 * r]) + " " + sym_text(exp, merges[2 * r + 1]) + "\r\n";
    std::vector<int32_t> parsed((size_t)(2 * (R + 1)));
    int64_t np = -1;
    const int rc = bpe_parse_merges_text(text.data(), (int64_t)text.size(), parsed.data(), R + 1, &np);
    // a table whose two merges give the same bytes has no text form
    if (rc == BPE_OK) {
      CHECK(np == R && memcmp(parsed.data(), merges.data(), sizeof(int32_t) * 2 * (size_t)R) == 0);
      std::string json = "{";
      for (size_t v = 0; v < exp.size(); ++v) {
        json += (v ? ",\"" : "\"");
        for (unsigned char c : sym_text(exp, (int32_t)v)) {
          if (c == '"' || c == '\\') json += '\\';
          json += (char)c;
        }
        json += "\": " + std::to_string(v);
      }
      json += ", \"<|endoftext|>\": 999999}";
      std::vector<int32_t> idm(exp.size());
      CHECK(bpe_parse_vocab_json(json.data(), (int64_t)json.size(), R ? merges.data() : nullptr, R,
                                 idm.data()) == BPE_OK);
      for (size_t v = 0; v < exp.size(); ++v) CHECK(idm[v] == (int32_t)v);
    } else {
      CHECK(rc == BPE_EMERGES);
    }
    // malformed text: random bytes and every prefix of a valid file
    for (int k = 0; k < 20; ++k) {
      std::string junk(rng() % 64, ' ');
      for (char &c : junk) c = (char)(rng() & 0xFF);
      int64_t nn = 0;
      (void)bpe_parse_merges_text(junk.data(), (int64_t)junk.size(), parsed.data(), R + 1, &nn);
      std::vector<int32_t> idm(exp.size());
      (void)bpe_parse_vocab_json(junk.data(), (int64_t)junk.size(), R ? merges.data() : nullptr, R,
                                 idm.data());
    }
    for (size_t cut = 0; cut < text.size(); cut += 1 + text.size() / 17) {
      int64_t nn = 0;
      (void)bpe_parse_merges_text(text.data(), (int64_t)cut, parsed.data(), R + 1, &nn);
    }
    ora_table_free(t);
  }
  uint8_t u[4];
  CHECK(ora_utf8_encode(0x1F408, u) == 4);
  CHECK(ora_fnv1a64(nullptr, 0) == 0xcbf29ce484222325ull);
  printf("sanitized host checks passed\n");
  return 0;
}
