// bpe_internal.h -- layouts shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpe {

// ---- rank table --------------------------------------------------------
// Open-addressing hash table in device memory, one 64-bit slot per entry:
//   bits 42..62  left symbol, bits 21..41 right symbol, bits 0..20 rank.
// A key is (left << 21) | right, so (slot >> 21) is the key; the empty slot
// is all ones, whose upper bits can equal no key.  Capacity is a power of
// two >= 2 * merges (load <= 1/2), probed linearly from a multiplicative hash
// of the key.  ("Tokenization LLM: ... C++", section "Vocabulary lookup":
// a pair-keyed map from the pair of units to its rank.)
constexpr int kSymBits = 21;
constexpr uint64_t kEmptySlot = ~0ull;
constexpr int32_t kRankInf = 0x7fffffff;  // "no merge here" compares largest

__host__ __device__ inline uint64_t pair_key(uint32_t l, uint32_t r) {
  return ((uint64_t)l << kSymBits) | (uint64_t)r;
}

__host__ __device__ inline uint64_t pair_hash(uint64_t key, int bits) {
  return (key * 0x9E3779B97F4A7C15ull) >> (64 - bits);
}

// ---- word table -----------------------------------------------------------
// Read-only table built at load time: a pre-token whose bytes equal the
// expansion of symbol s (2..kWordMax bytes), where encoding that expansion
// yields exactly [s], encodes to [s] without running the merge loop.  One
// 32-byte slot per entry: {tag, symbol, key[6]}; tag = (hash & ~0xff) | len
// (0 = empty); key = the bytes as six little-endian words, zero padded.
constexpr int kWordMax = 24;
constexpr int kWordWords = kWordMax / 4;

__host__ __device__ inline uint32_t word_hash(const uint32_t *w, int len) {
  uint32_t h = 0x811C9DC5u ^ ((uint32_t)len * 0x01000193u);
  for (int i = 0; i < kWordWords; ++i) {
    h = (h ^ w[i]) * 0x9E3779B1u;
    h ^= h >> 16;
  }
  return h;
}

__host__ __device__ inline uint32_t word_tag(uint32_t h, int len) {
  return (h & 0xFFFFFF00u) | (uint32_t)len;
}

// ---- look-back flags ----------------------------------------------------
// One 64-bit word per chunk: bits 62..63 state, bits 0..61 value.
constexpr uint64_t kFlagAgg = 1ull << 62;     // value = this chunk's count
constexpr uint64_t kFlagPrefix = 2ull << 62;  // value = count up to and including this chunk
constexpr uint64_t kFlagValue = (1ull << 62) - 1;

// ---- encode geometry ----------------------------------------------------
constexpr int kEncThreads = 256;     // one workgroup = 4 wave64
constexpr int kChunk = 4096;         // bytes whose pre-token starts a workgroup owns
constexpr int kHalo = 64;            // bytes read past the chunk for the last pre-token
constexpr int kLaneMax = 32;         // longest pre-token one lane merges alone

// ---- decode geometry ----------------------------------------------------
constexpr int kDecThreads = 256;
constexpr int kDecPerThread = 8;
constexpr int kDecChunk = kDecThreads * kDecPerThread;  // IDs per workgroup

inline int64_t enc_chunks(int64_t n_bytes) { return (n_bytes + kChunk - 1) / kChunk; }
inline int64_t dec_chunks(int64_t n_ids) { return (n_ids + kDecChunk - 1) / kDecChunk; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Encode workspace: [ticket 256 B][flags 8*G][first doc 8*G][symbols 4*N]
// [ranks 4*N].  The symbol/rank regions hold the pre-tokens that run the
// merge loop, each at its own byte position, so no two overlap.
struct EncLayout {
  size_t ticket, flags, first_doc, gsym, grank, total;
};
inline EncLayout enc_layout(int64_t n_bytes) {
  EncLayout L;
  int64_t G = enc_chunks(n_bytes);
  L.ticket = 0;
  L.flags = 256;
  L.first_doc = L.flags + align256(8 * (size_t)G);
  L.gsym = L.first_doc + align256(8 * (size_t)G);
  L.grank = L.gsym + align256(4 * (size_t)n_bytes);
  L.total = L.grank + align256(4 * (size_t)n_bytes);
  return L;
}

struct DecLayout {
  size_t ticket, flags, total;
};
inline DecLayout dec_layout(int64_t n_ids) {
  DecLayout L;
  L.ticket = 0;
  L.flags = 256;
  L.total = L.flags + align256(8 * (size_t)dec_chunks(n_ids));
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
  const uint64_t *table;
  int table_bits;
  const int32_t *id_map;  // nullptr = identity
  const int32_t *pair_rank;  // [65536]: rank of the byte pair (a, b) at a * 256 + b
  const uint4 *words;        // word table: 2 uint4 per slot; nullptr = none
  int word_bits;
  uint32_t *ticket;
  uint64_t *flags;
  const int64_t *first_doc;  // [n_chunks]
  int32_t *gsym;
  int32_t *grank;
  int32_t *status;
  int64_t n_chunks;
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
  const int32_t *inv_map;    // nullptr = identity; else [inv_size], -1 = no symbol
  int64_t inv_size;
  int64_t vocab;
  uint32_t *ticket;
  uint64_t *flags;
  int32_t *status;
  int64_t n_chunks;
};

// Launchers (bpe_kernels.hip).
// Clears the ticket, the status word and n_flags look-back flags; with
// first_doc, also records each chunk's first document (encode).
hipError_t launch_clear(uint32_t *ticket, uint64_t *flags, int64_t n_flags, int32_t *status,
                        int64_t *first_doc, const int64_t *doc_off, int64_t n_docs,
                        hipStream_t stream);
// Empty input: clears the status, checks that offs[0..n_docs] are all zero
// (else sets bad_bit) and writes zeros to out_off[0..n_docs].
hipError_t launch_empty(const int64_t *offs, int64_t n_docs, uint32_t bad_bit, int64_t *out_off,
                        int32_t *status, hipStream_t stream);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace bpe
