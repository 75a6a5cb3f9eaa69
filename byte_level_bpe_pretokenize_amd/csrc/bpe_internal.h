// bpe_internal.h -- layouts shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

struct bpe_model;

namespace bpe {

// bpe_encode_batch's argument checks and launches (bpe_api.cpp); `timed`:
// record stage-timing events when the model has them enabled.
int encode_checked(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                   const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids, int64_t ids_capacity,
                   int64_t *d_id_off, void *d_workspace, size_t workspace_bytes, int32_t *d_status,
                   void *hip_stream, bool timed);
// The device a model was loaded on (-1 for NULL).
int model_device(const bpe_model *model);

// Host-side table placement (bpe_tables.cpp).
// The rank table: keys in rank order (pair_key), buckets = mask + 1 of two
// 64-bit slots {key << kSymBits | rank}, the kSlotFlag of a key's first
// bucket set when the key sits in its second.
bool build_rank_table(const std::vector<uint64_t> &keys, uint32_t mask, uint32_t seed,
                      std::vector<uint64_t> &slots);
// The long word table: a two-choice cuckoo placement of hashes h over mask + 1
// slots (word_slot0, word_slot1); at[slot] = entry or -1.
bool place_words(const std::vector<uint32_t> &h, uint32_t mask, std::vector<int32_t> &at);
// The short word table: a displacement per bucket of keys (h >> (32 - dbits))
// under which every key sits at short_slot(h, disp, st, mask), all distinct.
bool place_displaced(const std::vector<uint32_t> &h, const std::vector<uint32_t> &st,
                     uint32_t mask, int dbits, std::vector<int32_t> &at,
                     std::vector<uint8_t> &disp);
// Window radii of the long pre-tokens' rounds by class (0: one rank per
// round); len[v] = bytes of symbol v, order = the symbols >= 256 with their
// operands first.
void window_radii(const int32_t *merges, int64_t R, const std::vector<int64_t> &len,
                  const std::vector<int64_t> &order, int32_t win_d[4]);

// ---- byte classes ---------------------------------------------------------
// The fixed split rule's classes: letters (A-Z, a-z and every byte from 0x80
// up), digits, whitespace (0x09-0x0D, 0x20), punctuation (the rest).
// ("Tokenization LLM: ... C++", section "Technical analysis": words,
// numbers, punctuation and whitespace.)
enum : uint32_t { kL = 0, kD = 1, kW = 2, kP = 3 };

__host__ __device__ inline uint32_t byte_class(uint32_t b) {
  const uint32_t lo = b | 0x20u;
  if ((lo - 'a' <= 'z' - 'a') || b >= 0x80u) return kL;
  if (b - '0' <= 9u) return kD;
  if (b - 9u <= 4u || b == 0x20u) return kW;
  return kP;
}

// ---- rank table --------------------------------------------------------
// Pair-keyed map from a pair of units to its rank ("Tokenization LLM: ...
// C++" (glitch4techs.com), section "Vocabulary lookup"), as a hash table in
// device memory of 16-byte buckets, each two 64-bit slots, so that a bucket
// is one load.  A slot holds key << 21 | rank with key = (left << 21) | right;
// ranks stay below 2^20 (BPE_MAX_MERGES), so bit 20 is free, and bit 20 of a
// bucket's first slot is the bucket's flag: a key whose first bucket this is
// sits in its second bucket.  An empty slot has every bit set but bit 20, so
// its upper bits equal no key.  Every key sits in its first or its second
// bucket: a lookup loads the first bucket, and the second only when the key
// is not in the first and the flag is set.
constexpr int kSymBits = 21;
constexpr uint64_t kSlotFlag = 1ull << 20;
constexpr uint64_t kEmptySlot = ~0ull ^ kSlotFlag;
constexpr uint32_t kRankMask = (1u << 20) - 1;
constexpr int32_t kRankInf = 0x7fffffff;  // "no merge here" compares largest

__host__ __device__ inline uint64_t pair_key(uint32_t l, uint32_t r) {
  return ((uint64_t)l << kSymBits) | (uint64_t)r;
}

// Products of two values below 2^24 (one full-rate multiply on the device).
__host__ __device__ inline uint32_t mul24(uint32_t a, uint32_t b) {
  return (a & 0xFFFFFFu) * (b & 0xFFFFFFu);
}

// A bijection of 32-bit values: the low 24 bits times an odd constant (a
// bijection of the low 24 bits of the product), the top byte carried over.
__host__ __device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x = mul24(x, 0x85EBCBu) ^ (x & 0xFF000000u);
  x ^= x >> 13;
  return x;
}

// 32-bit mix of a pair of symbols (both below 2^21) and the table's seed.
__host__ __device__ inline uint32_t pair_mix(uint32_t l, uint32_t r, uint32_t seed) {
  return mix32(mul24(l ^ seed, 0x9E3779u) ^ r ^ (seed >> 8));
}

// A bit set of the merges' pairs (a one-hash Bloom filter over pair_mix): a
// pair whose bit is clear has no rank, so its probe of the rank table can be
// skipped.  2^18 bits (32 KiB): for 32,000 merges about one clear-pair probe
// in eight still goes to the table.
constexpr int kPairFilterLog2 = 18;
constexpr int kPairFilterWords = (1 << kPairFilterLog2) / 32;
__host__ __device__ inline uint32_t pair_filter_bit(uint32_t x) { return x >> (32 - kPairFilterLog2); }

// First and second bucket of a mix, for a table of mask + 1 buckets (a power
// of two, at least 2); the second differs from the first.
__host__ __device__ inline uint32_t pair_bucket0(uint32_t x, uint32_t mask) { return x & mask; }
__host__ __device__ inline uint32_t pair_bucket1(uint32_t x, uint32_t mask) {
  const uint32_t y = mul24(x >> 8, 0xC2B2AFu) ^ (x >> 21);
  const uint32_t b0 = x & mask, b1 = y & mask;
  return b1 == b0 ? b0 ^ 1u : b1;
}

// ---- word tables ----------------------------------------------------------
// Read-only tables built at load time ("Hugging Face Tokenizers v1", section
// "Word caching": a pre-token seen as a whole skips the merge loop): a
// pre-token whose bytes equal the expansion of symbol s (2..kWordMax bytes),
// where encoding that expansion yields exactly [s], encodes to [s].  Keys are
// the bytes as little-endian words, zero padded.
//
// Short table (2..kShortMax bytes): one probe per lookup.  The keys are
// grouped by the top bits of their hash h into buckets of about four; each
// bucket has a one-byte displacement d, chosen at load so that every key of
// the bucket lands on its own free slot short_slot(h, d, step) with step an
// odd value from the key's words (keys with equal hashes still part).  The
// table has at least two slots per key.  16-byte slots {w0, w1, w2, symbol |
// len << 21}; an empty slot is all zero (its len field matches no key).
//
// Long table (kShortMax + 1..kWordMax bytes): a two-choice cuckoo table with
// one slot per bucket: an entry sits in its first or its second slot, and a
// flag in the first slot says that some entry whose first slot it is sits in
// its second; a lookup loads the first slot, and the second only when the
// key is not in the first and the flag is set.  32-byte slots {tag, symbol |
// flag << 31, w0, w1}, {w2, w3, w4, w5}, tag = (h & ~0xff) | len (0 = empty).
constexpr int kShortMax = 12;
constexpr int kWordMax = 24;
constexpr int kWordWords = kWordMax / 4;
constexpr uint32_t kWordFlag = 1u << 31;
constexpr uint32_t kWordSymMask = (1u << 21) - 1;

// Mix of a short key (w2:w1:w0 zero padded past len bytes): its twelve
// bytes as four 24-bit pieces, each times an odd constant, summed with the
// length and the seed (24-bit multiply-adds on the device), then mixed.
__host__ __device__ inline uint32_t short_mix(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t len,
                                              uint32_t seed) {
  const uint32_t p1 = (w0 >> 24) | (w1 << 8);
  const uint32_t p2 = (w1 >> 16) | (w2 << 16);
  return mix32(mul24(w0, 0x9E3779u) + mul24(p1, 0x85EBCBu) + mul24(p2, 0xC2B2AFu) +
               mul24(w2 >> 8, 0x27D4EBu) + (len << 26) + seed);
}

// The short table's slots per displacement (about four keys per bucket at
// two slots per key), the step of a key (odd, below 2^24), and its slot for
// displacement d < 256 (the product stays below 2^32: one 24-bit
// multiply-add on the device).
constexpr uint32_t kShortSlotsPerDisp = 8;
__host__ __device__ inline uint32_t short_step(uint32_t w0, uint32_t w1, uint32_t w2) {
  return (mul24(w1 ^ (w2 << 7) ^ (w0 >> 9), 0x27D4EBu) >> 8) | 1u;
}
__host__ __device__ inline uint32_t short_slot(uint32_t h, uint32_t d, uint32_t step,
                                               uint32_t mask) {
  return (d * step + h) & mask;
}

__host__ __device__ inline uint32_t word_hash(const uint32_t *w, int len, uint32_t seed) {
  uint32_t h = 0x811C9DC5u ^ ((uint32_t)len * 0x01000193u) ^ seed;
  for (int i = 0; i < kWordWords; ++i) {
    h = (h ^ w[i]) * 0x9E3779B1u;
    h ^= h >> 16;
  }
  return h;
}

__host__ __device__ inline uint32_t word_tag(uint32_t h, int len) {
  return (h & 0xFFFFFF00u) | (uint32_t)len;
}

// The two slots of a key; the second moves off the first when they coincide.
__host__ __device__ inline uint32_t word_slot0(uint32_t h, uint32_t mask) { return h & mask; }
__host__ __device__ inline uint32_t word_slot1(uint32_t h, uint32_t mask) {
  const uint32_t g = mul24(h >> 8, 0xC2B2AFu) ^ (h >> 19);
  const uint32_t s0 = h & mask, s1 = g & mask;
  return s1 == s0 ? s0 ^ 1u : s1;
}

// ---- encode geometry ----------------------------------------------------
constexpr int kEncThreads = 256;     // one workgroup = 4 wave64
constexpr int kChunk = 4096;         // bytes whose pre-token starts a workgroup owns
constexpr int kHalo = 64;            // bytes read past the chunk for the last pre-token
constexpr int kLaneMax = 32;         // longest pre-token one lane merges alone

// ---- decode geometry ----------------------------------------------------
constexpr int kDecThreads = 256;
constexpr int kDecPerThread = 4;
constexpr int kDecChunk = kDecThreads * kDecPerThread;  // IDs per workgroup

inline int64_t enc_chunks(int64_t n_bytes) { return (n_bytes + kChunk - 1) / kChunk; }
inline int64_t dec_chunks(int64_t n_ids) { return (n_ids + kDecChunk - 1) / kDecChunk; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Largest window radius of the multi-rank rounds (longer: one rank per round).
constexpr int kWinMax = 64;

// Per-chunk records of the encode pipeline.
constexpr int kMissBytes = kChunk + kHalo;  // bytes of a chunk's lane-merged pre-tokens, at most
// Their dense region: each entry at a 4-byte aligned offset (at most twice
// its bytes, entries being at least 2 bytes long).
constexpr int kMissSpan = 2 * kMissBytes;
constexpr int kMaxLong = kChunk / (kLaneMax + 1) + 4;  // wave-merged pre-tokens per chunk, at most
// The merge-loop list of a chunk: one region per length bucket (2-8, 9-16,
// 17-32 bytes, then longer or running past the window), each sized for the
// most entries of its least length whose bytes fit in the window.
constexpr int kBuckets = 4;
constexpr int kBucketCap[kBuckets] = {kMissBytes / 2, kMissBytes / 9 + 1, kMissBytes / 17 + 1,
                                      kMaxLong};
constexpr int kBucketBase[kBuckets] = {0, kBucketCap[0], kBucketCap[0] + kBucketCap[1],
                                       kBucketCap[0] + kBucketCap[1] + kBucketCap[2]};
constexpr int kMissMax = kBucketBase[3] + kBucketCap[3];
// The call's entry table covers buckets 1 and 2: their entries' references
// (dref), per chunk.
constexpr int kDrefBase = kBucketBase[1];
constexpr int kDrefCap = kBucketCap[1] + kBucketCap[2];
// meta: 16 int32 per chunk
constexpr int kMetaInts = 16;
constexpr int kMetaPretokens = 0;  // pre-tokens that start in the chunk
constexpr int kMetaMisses = 1;     // of which on the merge-loop list
constexpr int kMetaStatus = 2;     // status bits found by the chunk
constexpr int kMetaBytes = 3;      // span of the lane-merged entries' dense region
constexpr int kMetaBucket = 4;     // 4 entries: list entries per length bucket
constexpr int kMetaOwners = 8;     // 3 entries: of which first of their bytes in the call
                                   // (buckets 0-2)

// Encode workspace, all regions 256-byte aligned:
//   meta      [G][16] i32  pre-tokens, merge-loop pre-tokens, status bits,
//                          lane-merged bytes, list entries per length bucket,
//                          owners per lane-merged bucket
//   tot, off  [G] i64   token count per chunk with its status bits on top,
//                       then the counts' exclusive prefix within its block of
//                       1024 chunks
//   bsum, boff [B] i64  per block of 1024 chunks: its count with the status
//                       bits on top, then the blocks' exclusive prefix
//   doc_rng   [G][2] i64  documents that start in the chunk
//   dfirst    [G] i64   first document whose offset is at or after the byte
//                       before the chunk
//   doc_pt    [D] i32   index of each document's first pre-token in its chunk
//   pv        [G][kChunk] i32    per pre-token: its symbol; -1 - o4 for a
//                                lane-merged one whose bytes start at 4 o4 in
//                                mbytes; -1 - 2^20 - q for the q-th
//                                wave-merged one; -1 - 2^21 - g for a
//                                lane-merged one whose tokens are those of
//                                another entry with the same bytes, at 4 g in
//                                res (g counted from the start of res)
//   cntk      [G][kChunk] u8     token count of each lane-merged pre-token
//   miss      [G][kMissMax] u32  merge-loop list, a region per length bucket
//                                (kBucketBase), in no particular order:
//                                o / 4 | len << 12 | k << 18 (lane-merged,
//                                k the pre-token's index), start | len << 13 |
//                                overhang << 26 (wave-merged)
//   mt        [G][kMaxLong] i32  token count of each wave-merged entry
//   dref      [G][kDrefCap] u32  entry of bucket 1 or 2 (list index minus
//                                kDrefBase): kDrefOwner if it is merged itself,
//                                else the entry-table slot of its bytes
//   olist     [G][kMissMax] u64  the entries merged themselves, per bucket
//                                region: entry | slot << 32 (kNoSlot: none)
//   dstat     u32       entry-table claims of the first (seeding) launch
//   dt        [DS][16] u8  the call's entry table, DS = dedup_slots(G): per
//                          slot the key (u64: hash bits and length above the
//                          owner's offset / 4 in mbytes, counted from its
//                          start), that offset again (u32) and, once the
//                          owner is merged, its token count (u32)
//   mbytes    [G][kMissSpan] u8   bytes of the lane-merged entries, each at a
//                                  4-byte aligned offset o
//   res       [G][kMissSpan] i32  its tokens, from o on
//   gsym      [N] i32   tokens of a wave-merged entry that starts at byte g, from gsym[g] on
//   grank     [N] i32   pair ranks of the wave merge, position-indexed (in olist's
//                       memory: olist is dead by then)
struct EncLayout {
  size_t meta, tot, off, bsum, boff, doc_rng, dfirst, doc_pt, pv, cntk, miss, mt, dref, olist, dstat, dt, mbytes, res, gsym,
      grank, total;
};

// Chunks per workgroup of the first level of the offset scans.
constexpr int kScanBlock = 1024;

// Slots of the call's entry table: a power of two >= 32 per chunk.
inline size_t dedup_slots(size_t G) {
  size_t n = 4096;
  while (n < 32 * G) n *= 2;
  return n;
}
constexpr uint32_t kDrefOwner = 0xFFFFFFFFu;
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;
// pv values below -2^21 address res across chunks; the entry table is used
// only while every such value fits an int32.
constexpr int64_t kDedupMaxChunks = ((1ll << 31) - (1ll << 21)) / (kMissSpan / 4) - 1;
inline EncLayout enc_layout(int64_t n_bytes, int64_t n_docs) {
  EncLayout L;
  const size_t G = (size_t)enc_chunks(n_bytes);
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.meta = take(4 * kMetaInts * G);
  L.tot = take(8 * (G + 16));  // the offset scan reads whole groups of 16
  L.off = take(8 * (G + 16));
  const size_t B = (G + kScanBlock - 1) / kScanBlock;
  L.bsum = take(8 * (B + 16));
  L.boff = take(8 * (B + 16));
  L.doc_rng = take(16 * G);
  L.dfirst = take(8 * G);
  L.doc_pt = take(4 * (size_t)(n_docs + 1));
  L.pv = take(4 * (size_t)kChunk * G);
  L.cntk = take((size_t)kChunk * G);
  L.miss = take(4 * (size_t)kMissMax * G);
  L.mt = take(4 * (size_t)kMaxLong * G);
  L.dref = take(4 * (size_t)kDrefCap * G);
  L.olist = take(8 * (size_t)kMissMax * G);
  L.dstat = take(8);
  L.dt = take(16 * dedup_slots(G));
  L.mbytes = take((size_t)kMissSpan * G + 64);  // word loads read a little past the end
  L.res = take(4 * (size_t)kMissSpan * G + 64);
  L.gsym = take(4 * (size_t)n_bytes);
  // grank is only used by k_merge_long, after the last reader of olist
  // (k_merge_wide): it takes olist's memory
  static_assert(8 * kMissMax >= 4 * kChunk, "olist holds grank");
  L.grank = L.olist;
  L.total = o;
  return L;
}

// Decode workspace: tot, off [G] i64 (byte count per chunk of IDs with the
// chunk's status bits on top, then the counts' exclusive prefix within its
// block of kScanBlock chunks); dlo [G + 1] i64 (the first document whose IDs
// start at or after chunk g's first ID, and after the last ID); bsum, boff
// [B] i64 (per block: its count with the status bits on top, then the blocks'
// exclusive prefix).
struct DecLayout {
  size_t tot, off, dlo, bsum, boff, total;
};
inline DecLayout dec_layout(int64_t n_ids) {
  DecLayout L;
  const size_t G = (size_t)dec_chunks(n_ids);
  const size_t B = (G + kScanBlock - 1) / kScanBlock;
  L.tot = 0;
  L.off = align256(8 * G);
  L.dlo = L.off + align256(8 * G);
  L.bsum = L.dlo + align256(8 * (G + 1));
  L.boff = L.bsum + align256(8 * (B + 16));  // the block scan reads whole groups of 16
  L.total = L.boff + align256(8 * (B + 16));
  return L;
}

struct EncodeArgs {
  const uint8_t *bytes;
  int64_t n_bytes;
  const int64_t *doc_off;
  int64_t n_docs;
  int32_t *ids;
  int64_t ids_cap;
  int64_t *id_off;
  const uint64_t *table;     // rank table: 2 slots per bucket
  uint32_t table_mask;       // buckets - 1
  uint32_t table_seed;
  const int32_t *id_map;     // nullptr = identity
  const int32_t *pair_rank;  // [65536]: rank of the byte pair (a, b) at a * 256 + b
  const uint32_t *pair_filter;  // [kPairFilterWords] bit pair_filter_bit(pair_mix(l, r, table_seed))
                                // set for every merge (l, r)
  int n_cu;                  // compute units (workgroups of the persistent merge kernel)
  int lgroup;                // chunks per lane-merge group (set by the launch)
  const uint4 *words;        // short word table (one uint4 per slot); nullptr = none
  const uint8_t *word_disp;  // its displacement per bucket of keys (hash >> word_dshift)
  uint32_t word_mask;        // slots - 1
  uint32_t word_seed;
  uint32_t word_dshift;
  const uint4 *lwords;       // long word table (two uint4 per slot); nullptr = none
  uint32_t lword_mask;
  uint32_t lword_seed;
  int32_t *meta;
  int64_t *tot;
  int64_t *off;
  int64_t *bsum;
  int64_t *boff;
  int64_t *doc_rng;
  int64_t *dfirst;
  int32_t *doc_pt;
  int32_t *pv;
  uint8_t *cntk;
  uint32_t *miss;
  int32_t *mt;
  uint32_t *dref;
  uint64_t *olist;
  uint32_t *dstat;           // entry-table claims of the seeding launch
  unsigned long long *dt;    // the call's entry table (dedup_slots(n_chunks) slots)
  uint32_t dt_mask;          // slots - 1
  int dedup;                 // 0: every lane-merged entry is merged (no table)
  uint8_t *mbytes;
  int32_t *res;
  int32_t *gsym;
  int32_t *grank;
  int32_t *status;
  int64_t n_chunks;
  int64_t doc_per;           // document offsets checked per chunk (k_docs): ceil((n_docs + 1) / n_chunks)
  // Window radius of the multi-rank rounds for long pre-tokens, by the class
  // of the pre-token's first letter/digit/space/punctuation byte: the longest
  // token whose bytes can occur in such a pre-token; 0 = one rank per round.
  int32_t win_d[4];
  // reserved IDs put before / after each document's IDs (-1: none); with
  // either, k_emit writes every ID at its place in the output with them
  int32_t bos, eos;
};

struct DecodeArgs {
  const int32_t *ids;
  int64_t n_ids;
  const int64_t *id_off;
  int64_t n_docs;
  uint8_t *out;
  int64_t out_cap;
  int64_t *byte_off;
  const int64_t *exp_off;    // [V + 1]
  const uint8_t *exp_bytes;  // expansions back to back
  const uint4 *exp16;        // [V]: the first 16 bytes of each expansion, zero padded
  const uint4 *exp16b;       // [V]: its bytes 16..31, zero padded
  const int32_t *exp_len;    // [V]: each expansion's length
  const int32_t *inv_map;    // nullptr = identity; else [inv_size], -1 = no symbol
  int64_t inv_size;
  int64_t vocab;
  int64_t *tot;
  int64_t *off;
  int64_t *bsum;
  int64_t *boff;
  int64_t *dlo;
  int32_t *status;
  int64_t n_chunks;
  int64_t doc_per;           // document offsets checked per chunk (k_dec_len): ceil((n_docs + 1) / n_chunks)
  int32_t skip0, skip1;      // reserved IDs that decode to no bytes (-1: none)
};

// Reserved IDs around the documents of an empty input (k_special).
struct SpecialArgs {
  int64_t n_docs;
  int32_t bos, eos;          // written before / after each document (-1: none)
  int32_t *ids;
  int64_t ids_cap;
  int64_t *id_off;
  int32_t *status;
};

// Launchers.
// Empty input: clears the status, checks that offs[0..n_docs] are all zero
// (else sets bad_bit) and writes zeros to out_off[0..n_docs]  (bpe_encode.hip).
hipError_t launch_empty(const int64_t *offs, int64_t n_docs, uint32_t bad_bit, int64_t *out_off,
                        int32_t *status, hipStream_t stream);
// The encode pipeline for n_bytes > 0 (bpe_encode.hip).  ev: nullptr, or
// kEncStages + 1 events recorded before the first kernel and after each.
constexpr int kEncStages = 10;
extern const char *const kEncStageNames[kEncStages];
hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream, hipEvent_t *ev);
// Training (bpe_train.hip): the distinct pre-tokens of the corpus with their
// frequencies, their current symbols, and a pair table whose counts are kept
// up to date merge by merge.  The table's slots are summarized in blocks of
// kTrainBlock: each block's largest count and the smallest key with it, kept
// exact for every block a merge touched before the next pick.
constexpr int kTrainBlock = 1024;       // slots per block, at least
constexpr int kTrainLoopBlocks = 8192;  // blocks, at most (the one-workgroup loop keeps them in LDS)
constexpr int kTrainGridMerges = 256;   // merges run as grid-wide kernels before the loop
struct TrainArgs {
  int32_t *sym;              // the pre-tokens' current symbols
  uint4 *wrec;               // per pre-token: its first symbol's index in sym, its
                             // symbol count, its frequency (low, high 32 bits)
  const int32_t *pos_word;   // the pre-token of each original position
  int64_t n_words, n_pos;
  uint64_t *keys;            // pair table: (left << 32 | right) + 1, 0 = empty
  uint32_t *counts;          // its counts (a corpus has fewer than 2^32 bytes)
  uint64_t mask;             // slots - 1 (a power of two, at least 4 n_pos: keys are never removed)
  uint32_t *bmax;            // [nblocks] each block's largest count
  unsigned long long *bkey;  // [nblocks] the smallest key with that count (~0: none)
  uint32_t *dirty;           // [nblocks] 1 while the block is listed in dlist
  uint32_t *dlist;           // [nblocks] blocks touched since their summary
  uint32_t *ndirty;          // [1] entries of dlist
  int64_t nblocks;           // a power of two, at most kTrainLoopBlocks
  uint64_t bsize;            // slots per block: (mask + 1) / nblocks
  // occurrence lists: symbol x's list, pool[lrec[x].x .. + lrec[x].y),
  // holds every pre-token that contains x (and perhaps some that no longer
  // do): for a byte, the pre-tokens with that byte; for 256 + r, the
  // pre-tokens merge r changed, appended at pool_top during the merge
  int32_t *pool;
  uint2 *lrec;               // per symbol: its list's first pool entry, its length
  unsigned long long *pool_top;  // [1] the pool's first free entry
  uint32_t *zcount;          // [1] pre-tokens the last merge changed
  uint64_t *best;            // [3]: the picked count, its key, and the merge's index
  int64_t n_target;          // merges asked for
  int64_t n_grid;            // of which made by the grid-wide kernels (the rest by k_tloop)
  int32_t *stop;             // set once the best count is below 2 or n_target merges are made
  int32_t *merges;           // [n_merges][2] out
  int64_t *out_counts;       // [n_merges] out
  int64_t *made;             // merges made
};
// The initial pair counts and every block's summary.
hipError_t launch_train_init(const TrainArgs &a, hipStream_t stream);
// One merge as grid-wide kernels: pick the best pair, apply it, summarize
// the touched blocks.
hipError_t launch_train_step(const TrainArgs &a, hipStream_t stream);
// The remaining merges in one workgroup.
hipError_t launch_train_loop(const TrainArgs &a, hipStream_t stream);

// The reserved IDs of an empty input, after launch_empty (bpe_encode.hip).
hipError_t launch_special(const SpecialArgs &a, hipStream_t stream);
// The decode pipeline for n_ids > 0 (bpe_decode.hip), events as for encode.
constexpr int kDecStages = 4;
extern const char *const kDecStageNames[kDecStages];
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, hipEvent_t *ev);

}  // namespace bpe
