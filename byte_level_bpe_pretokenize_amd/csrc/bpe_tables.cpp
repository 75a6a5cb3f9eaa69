// bpe_tables.cpp -- the host-side placement of the model's hash tables (the
// rank table, the two word tables) and the window radii of the long
// pre-tokens' rounds.  Pure functions of their arguments, with no HIP call,
// so that the CPU tests can run them under the sanitizers.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "bpe_internal.h"

namespace bpe {

// Place every (key, rank) in its first or second bucket (two slots each):
// lower ranks first, each into its first bucket when there is room, else its
// second, else by displacing an occupant to that occupant's other bucket
// (a bounded random walk).  Then set the flag of the first bucket of every
// key that ended in its second.  False if some key found no place.
bool build_rank_table(const std::vector<uint64_t> &keys, uint32_t mask, uint32_t seed,
                      std::vector<uint64_t> &slots) {
  const size_t nb = (size_t)mask + 1;
  slots.assign(2 * nb, kEmptySlot);
  auto place = [&](size_t b, uint64_t item) {
    for (int k = 0; k < 2; ++k)
      if (slots[2 * b + k] == kEmptySlot) {
        slots[2 * b + k] = item;
        return true;
      }
    return false;
  };
  auto buckets = [&](uint64_t item, uint32_t &b0, uint32_t &b1) {
    const uint64_t key = item >> kSymBits;
    const uint32_t x = pair_mix((uint32_t)(key >> kSymBits), (uint32_t)(key & ((1u << kSymBits) - 1)), seed);
    b0 = pair_bucket0(x, mask);
    b1 = pair_bucket1(x, mask);
  };
  uint64_t rng = 0x2545F4914F6CDD1Dull ^ seed;
  const int max_kicks = 500;
  for (size_t r = 0; r < keys.size(); ++r) {
    uint64_t item = (keys[r] << kSymBits) | (uint64_t)r;
    uint32_t b0, b1;
    buckets(item, b0, b1);
    if (place(b0, item) || place(b1, item)) continue;
    uint32_t at = b1;  // bucket the walk evicts from
    bool ok = false;
    for (int kick = 0; kick < max_kicks && !ok; ++kick) {
      rng = rng * 6364136223846793005ull + 1442695040888963407ull;
      const int k = (int)((rng >> 33) & 1u);
      std::swap(item, slots[2 * (size_t)at + k]);
      buckets(item, b0, b1);
      const uint32_t other = (at == b0) ? b1 : b0;
      if (place(other, item)) ok = true;
      else at = other;
    }
    if (!ok) return false;
  }
  // keys in their second bucket move to the first where it has room
  for (size_t b = 0; b < nb; ++b)
    for (int k = 0; k < 2; ++k) {
      const uint64_t item = slots[2 * b + k];
      if (item == kEmptySlot) continue;
      uint32_t b0, b1;
      buckets(item, b0, b1);
      if (b0 != b && place(b0, item)) slots[2 * b + k] = kEmptySlot;
    }
  for (size_t b = 0; b < nb; ++b)
    for (int k = 0; k < 2; ++k) {
      const uint64_t item = slots[2 * b + k];
      if (item == kEmptySlot || item == (kEmptySlot | kSlotFlag)) continue;
      uint32_t b0, b1;
      buckets(item & ~kSlotFlag, b0, b1);
      if (b0 != b) slots[2 * (size_t)b0] |= kSlotFlag;
    }
  return true;
}

// Window radii for the long-pre-token merge, by pre-token class.  A pair
// whose rank is the lowest among all pairs within D symbols on each side is
// merged by the rank-ordered rounds before any other merge touches its
// symbols, provided every merge's operands come from lower ranks (so the
// rounds run in increasing rank) and D is at least the longest token that
// can form inside the pre-token: a merge chain reaching the pair from
// further away would build a longer token.  Merges stay inside a pre-token
// ("Hugging Face Tokenizers v1", section "How v1 works"), so that token's
// bytes belong to the pre-token: digits only, whitespace only, punctuation
// only, or letters after an optional space.  D = 0 where the table is not
// in rank order or a radius exceeds kWinMax.
void window_radii(const int32_t *merges, int64_t R, const std::vector<int64_t> &len,
                  const std::vector<int64_t> &order, int32_t win_d[4]) {
  bool ordered = true;
  for (int64_t r = 0; r < R; ++r)
    if (merges[2 * r] >= 256 + r || merges[2 * r + 1] >= 256 + r) ordered = false;
  const size_t V = (size_t)(256 + R);
  std::vector<uint8_t> first(V), all(V), rest(V);  // first byte; class bits of all / later bytes
  for (uint32_t b = 0; b < 256; ++b) {
    first[b] = (uint8_t)b;
    all[b] = (uint8_t)(1u << byte_class(b));
    rest[b] = 0;
  }
  for (int64_t v : order) {
    const int32_t l = merges[2 * (v - 256)], rt = merges[2 * (v - 256) + 1];
    first[(size_t)v] = first[(size_t)l];
    all[(size_t)v] = all[(size_t)l] | all[(size_t)rt];
    rest[(size_t)v] = rest[(size_t)l] | all[(size_t)rt];
  }
  int64_t d[4] = {1, 1, 1, 1};
  for (size_t v = 0; v < V; ++v) {
    const int64_t n = len[v];
    for (uint32_t c = 0; c < 4; ++c)
      if (all[v] == (1u << c)) d[c] = std::max(d[c], n);
    if (first[v] == 0x20 && (rest[v] & ~(1u << kL)) == 0) d[kL] = std::max(d[kL], n);
  }
  for (int c = 0; c < 4; ++c) win_d[c] = (ordered && d[c] <= kWinMax) ? (int32_t)d[c] : 0;
}

// Two-choice cuckoo placement with one slot per bucket for entries with
// hashes h, in order: each into its first slot when free, else its second,
// else displacing the occupant of its second slot to that occupant's other
// slot, and so on (bounded); then entries move back to a free first slot.
// at[slot] = entry or -1.  False if some entry found no slot.
bool place_words(const std::vector<uint32_t> &h, uint32_t mask, std::vector<int32_t> &at) {
  at.assign((size_t)mask + 1, -1);
  const int max_kicks = 500;
  for (int32_t e = 0; e < (int32_t)h.size(); ++e) {
    int32_t item = e;
    const uint32_t s0 = word_slot0(h[(size_t)item], mask), s1 = word_slot1(h[(size_t)item], mask);
    if (at[s0] < 0) { at[s0] = item; continue; }
    if (at[s1] < 0) { at[s1] = item; continue; }
    uint32_t cur = s1;
    bool ok = false;
    for (int kick = 0; kick < max_kicks && !ok; ++kick) {
      std::swap(item, at[cur]);
      const uint32_t a0 = word_slot0(h[(size_t)item], mask), a1 = word_slot1(h[(size_t)item], mask);
      const uint32_t other = cur == a0 ? a1 : a0;
      if (at[other] < 0) {
        at[other] = item;
        ok = true;
      } else {
        cur = other;
      }
    }
    if (!ok) return false;
  }
  for (uint32_t i = 0; i <= mask; ++i) {
    const int32_t e = at[i];
    if (e < 0) continue;
    const uint32_t s0 = word_slot0(h[(size_t)e], mask);
    if (s0 != i && at[s0] < 0) {
      at[s0] = e;
      at[i] = -1;
    }
  }
  return true;
}

// Displacement placement for keys with hashes h and steps st (the short
// table): the keys are grouped by h >> (32 - dbits); the largest groups
// first, each takes the first displacement d < 256 under which all its keys
// land on distinct free slots short_slot(h, d, st, mask).  at[slot] = key or
// -1, disp[group] = d.  False if some group found no displacement.
bool place_displaced(const std::vector<uint32_t> &h, const std::vector<uint32_t> &st,
                     uint32_t mask, int dbits, std::vector<int32_t> &at,
                     std::vector<uint8_t> &disp) {
  const size_t nb = (size_t)1 << dbits;
  at.assign((size_t)mask + 1, -1);
  disp.assign(nb, 0);
  std::vector<std::vector<int32_t>> group(nb);
  for (int32_t e = 0; e < (int32_t)h.size(); ++e) group[h[(size_t)e] >> (32 - dbits)].push_back(e);
  std::vector<uint32_t> order(nb);
  for (size_t b = 0; b < nb; ++b) order[b] = (uint32_t)b;
  std::stable_sort(order.begin(), order.end(),
                   [&](uint32_t x, uint32_t y) { return group[x].size() > group[y].size(); });
  std::vector<uint32_t> sl;
  for (uint32_t b : order) {
    const std::vector<int32_t> &g = group[b];
    if (g.empty()) break;
    bool ok = false;
    for (uint32_t d = 0; d < 256 && !ok; ++d) {
      sl.clear();
      ok = true;
      for (int32_t e : g) {
        const uint32_t s = short_slot(h[(size_t)e], d, st[(size_t)e], mask);
        if (at[s] >= 0 || std::find(sl.begin(), sl.end(), s) != sl.end()) {
          ok = false;
          break;
        }
        sl.push_back(s);
      }
      if (ok) {
        for (size_t i = 0; i < g.size(); ++i) at[sl[i]] = g[i];
        disp[b] = (uint8_t)d;
      }
    }
    if (!ok) return false;
  }
  return true;
}

}  // namespace bpe
