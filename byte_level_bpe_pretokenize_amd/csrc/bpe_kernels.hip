// bpe_kernels.hip -- byte-level BPE encode and decode kernels for gfx950.
//
// Encode is one pass over the input.  A workgroup owns a 4 KiB chunk of the
// concatenated documents: every pre-token whose first byte lies in the chunk.
//   1. scan: the chunk (plus a 64-byte halo after it and 2 bytes before) is
//      read once, coalesced, into LDS; each byte gets its class and a start
//      bit from a 3-byte window, and the start bits are packed 16 per lane.
//   2. merge: each lane merges the short pre-tokens that start in its 16
//      bytes, in place in LDS, with ranks probed in the device hash table;
//      longer ones are merged by the whole workgroup (LDS, or global scratch
//      for a pre-token that runs past the halo).
//   3. compaction: surviving symbols are counted per lane, scanned, the
//      chunk's total is chained to the previous chunks by a decoupled
//      look-back over 64-bit flags, and the IDs are written at their final
//      positions together with the per-document offsets.
// Decode uses the same chained-prefix pattern over per-ID byte lengths.
//
// Sources: "Tokenization LLM: ... C++" (glitch4techs.com), sections
// "Technical analysis", "Byte-level encoding", "BPE algorithm", "Vocabulary
// lookup"; "Characters, bytes and subwords" (tokenwerk.deckle.io), section
// "BPE step by step" ([a,a,a] -> [aa,a]); "Hugging Face Tokenizers v1"
// (dothoosh.com), sections "How v1 works", "Bitcannon" (boundaries from
// bit-parallel class masks), "Merge-loop rewrite" (flat symbol arrays,
// 'no merge' as the largest value, batches) and "Road to 1.0.0" (GPU batch
// encode/decode, output positions in parallel).
#include <limits.h>
#include <stdint.h>

#include "bpe_internal.h"
#include "../../include/bpe.h"

namespace bpe {
namespace {

constexpr int WG = kEncThreads;
constexpr int WIN = kChunk + kHalo;        // window positions [0, WIN)
constexpr int SB_HALF = WIN / 16 + 1;      // 16-bit start masks for positions [0, WIN]
constexpr int SB_WORDS = (SB_HALF + 1) / 2 + 1;
constexpr int DB_OFF = 32;                 // doc-start bit of position p is bit p + DB_OFF
constexpr int DB_WORDS = (WIN + DB_OFF) / 32 + 2;
constexpr int kMaxLong = kChunk / (kLaneMax + 1) + 4;
constexpr int kTile = WG * 16;
constexpr int32_t kDead = -1;
constexpr int kNoStart = INT_MAX;

// Byte classes (the fixed split rule): letters (A-Z, a-z and every byte from
// 0x80 up), digits, whitespace (0x09-0x0D, 0x20), punctuation (the rest).
enum : uint32_t { kL = 0, kD = 1, kW = 2, kP = 3 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t byte_class(uint32_t b) {
  const uint32_t lo = b | 0x20u;
  if ((lo - 'a' <= 'z' - 'a') || b >= 0x80u) return kL;
  if (b - '0' <= 9u) return kD;
  if (b - 9u <= 4u || b == 0x20u) return kW;
  return kP;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Rank of the pair (l, r), or kRankInf.  Linear probing from the pair's hash.
__device__ __forceinline__ int32_t rank_of(const uint64_t *__restrict__ tab, int bits, uint32_t l,
                                           uint32_t r) {
  const uint64_t key = pair_key(l, r);
  const uint64_t mask = (1ull << bits) - 1;
  uint64_t h = pair_hash(key, bits);
  for (;;) {
    const uint64_t s = tab[h];
    if ((s >> kSymBits) == key) return (int32_t)(s & ((1u << kSymBits) - 1));
    if (s == kEmptySlot) return kRankInf;
    h = (h + 1) & mask;
  }
}

// ---- wave / workgroup reductions and scans --------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_incl_sum(T v) {
  const int lane = lane_id();
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix sum over the workgroup; *total gets the sum.  Barriers
// inside: every thread must call it.
template <typename T, int NT>
__device__ T block_excl_sum(T v, T *red, T *total) {
  const T inc = wave_incl_sum(v);
  if (lane_id() == 63) red[wave_id()] = inc;
  __syncthreads();
  T wp = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const T x = red[w];
    if (w < wave_id()) wp += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return wp + inc - v;
}

template <int NT>
__device__ int32_t block_min(int32_t v, int32_t *red) {
  for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d, 64));
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  int32_t m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = min(m, red[w]);
  __syncthreads();
  return m;
}

template <int NT>
__device__ int32_t block_max(int32_t v, int32_t *red) {
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, 64));
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  int32_t m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = max(m, red[w]);
  __syncthreads();
  return m;
}

// Exclusive running maximum over the workgroup (identity `lowest`);
// *total gets the maximum of all values.
template <int NT>
__device__ int64_t block_excl_max64(int64_t v, int64_t lowest, int64_t *red, int64_t *total) {
  const int lane = lane_id();
  int64_t inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t o = __shfl_up(inc, d, 64);
    if (lane >= d) inc = max(inc, o);
  }
  int64_t ex = __shfl_up(inc, 1, 64);
  if (lane == 0) ex = lowest;
  if (lane == 63) red[wave_id()] = inc;
  __syncthreads();
  int64_t wp = lowest, tot = lowest;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int64_t x = red[w];
    if (w < wave_id()) wp = max(wp, x);
    tot = max(tot, x);
  }
  __syncthreads();
  *total = tot;
  return max(wp, ex);
}

// First index i in [0, n) with a[i] >= key (n if none), for a sorted array.
// Called by all 64 lanes of one wave; 64-way split per step.  For an array
// that is not sorted the result is still in [0, n].
__device__ int64_t wave_lower_bound(const int64_t *a, int64_t n, int64_t key) {
  const int lane = lane_id();
  int64_t lo = 0, hi = n;  // a[i] < key for i < lo; answer <= hi
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t idx = lo + (int64_t)lane * step;
    const bool ge = idx < hi ? (a[idx] >= key) : true;
    const uint64_t m = __ballot(ge);
    const int first = m ? __ffsll((unsigned long long)m) - 1 : 64;
    const int64_t nlo = first == 0 ? lo : lo + (int64_t)(first - 1) * step + 1;
    const int64_t nhi = first == 64 ? hi : min(hi, lo + (int64_t)first * step);
    lo = nlo;
    hi = max(nhi, nlo);
  }
  const int64_t idx = lo + lane;
  const bool ge = idx < hi ? (a[idx] >= key) : true;
  const uint64_t m = __ballot(ge);
  return m ? lo + (__ffsll((unsigned long long)m) - 1) : hi;
}

// Decoupled look-back over per-chunk flags (called by all lanes of one wave).
// Publishes this chunk's own count, then sums the counts of earlier chunks
// until one with a published running total, publishes its own running total
// and returns the exclusive prefix.
__device__ int64_t wave_lookback(uint64_t *flags, int64_t c, int64_t agg) {
  const int lane = lane_id();
  if (c == 0) {
    if (lane == 0)
      __hip_atomic_store(&flags[0], kFlagPrefix | (uint64_t)agg, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0)
    __hip_atomic_store(&flags[c], kFlagAgg | (uint64_t)agg, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int64_t excl = 0;
  int64_t top = c - 1;
  for (;;) {
    const int64_t idx = top - lane;
    const uint64_t f = idx >= 0 ? __hip_atomic_load(&flags[idx], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                : kFlagPrefix;
    const uint64_t state = f & ~kFlagValue;
    const uint64_t not_ready = __ballot(state == 0);
    const uint64_t pfx = __ballot(state == kFlagPrefix);
    const int kp = pfx ? __ffsll((unsigned long long)pfx) - 1 : 64;
    const uint64_t upto = kp >= 63 ? ~0ull : ((1ull << (kp + 1)) - 1);
    if (not_ready & upto) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    const int64_t v = lane <= kp ? (int64_t)(f & kFlagValue) : 0;
    excl += wave_sum(v);
    if (kp < 64) break;
    top -= 64;
  }
  if (lane == 0)
    __hip_atomic_store(&flags[c], kFlagPrefix | (uint64_t)(excl + agg), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return excl;
}

// ---- encode ---------------------------------------------------------------
constexpr int kPool = 768;  // LDS ints for the merge loop of 17..32-byte pre-tokens

struct EncShared {
  alignas(16) uint8_t B[16 + WIN + 32];  // B[16 + p] = byte at window position p
  uint32_t SB[SB_WORDS];                 // pre-token start bits, positions [0, WIN]
  uint32_t DB[DB_WORDS];                 // document start bits, positions [-32, WIN)
  uint16_t PS[kChunk + 2];               // owned pre-token starts in order, then the end
  int32_t PV[kChunk + 2];                // result of each pre-token (see kPendBase)
  uint16_t miss[kChunk / 2 + 2];         // pre-tokens for the merge loop (list indices)
  int32_t pool[kPool];                   // merge-loop scratch for 17..32-byte pre-tokens
  int32_t pool_used;
  int32_t long_st[kMaxLong];             // long pre-tokens inside the window
  int32_t long_e[kMaxLong];
  int32_t long_nt[kMaxLong];
  uint8_t mflag[WG];
  int32_t red[8];
  int64_t red64[8];
  int32_t n_miss, n_long;
  uint32_t ticket;
  int64_t o_lo, o_hi;
  int64_t base;
  int64_t ov_ntok;
};

__device__ __forceinline__ uint32_t sb16(const EncShared &s, int g) {
  return reinterpret_cast<const uint16_t *>(s.SB)[g];
}

__device__ __forceinline__ bool db_bit(const EncShared &s, int p) {
  const int q = p + DB_OFF;
  return (s.DB[q >> 5] >> (q & 31)) & 1u;
}

// Smallest start position in [from, WIN], or kNoStart.  Whole workgroup.
__device__ int block_next_start(EncShared &s, int from) {
  int cand = kNoStart;
  if (from <= WIN) {
    const int w = (from >> 5) + (int)threadIdx.x;
    if (w <= (WIN >> 5)) {
      uint32_t bits = s.SB[w];
      if (w == (from >> 5)) bits &= ~0u << (from & 31);
      if (bits) {
        const int p = (w << 5) + __ffs(bits) - 1;
        if (p <= WIN) cand = p;
      }
    }
  }
  return block_min<WG>(cand, s.red);
}

// The bytes of the pre-token at window position st (len <= kWordMax) as six
// little-endian words, zero padded.
__device__ __forceinline__ void pretoken_words(const EncShared &s, int st, int len,
                                               uint32_t w[kWordWords]) {
  const int b0 = 16 + st;
  const uint32_t *B32 = reinterpret_cast<const uint32_t *>(s.B);
  const int q = b0 >> 2;
  const uint32_t sh = (uint32_t)(b0 & 3);
  uint32_t raw[kWordWords + 1];
#pragma unroll
  for (int i = 0; i <= kWordWords; ++i) raw[i] = B32[q + i];
#pragma unroll
  for (int i = 0; i < kWordWords; ++i) {
    const uint32_t v = __builtin_amdgcn_alignbyte(raw[i + 1], raw[i], sh);
    const int valid = len - 4 * i;
    const uint32_t m = valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : ((1u << (8 * valid)) - 1u));
    w[i] = v & m;
  }
}

// Symbol stored for these bytes in the word table, or -1.
__device__ __forceinline__ int32_t word_lookup(const uint4 *__restrict__ tab, int bits,
                                               const uint32_t w[kWordWords], int len) {
  const uint32_t h = word_hash(w, len);
  const uint32_t tag = word_tag(h, len);
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t i = h & mask;
  for (;;) {
    const uint4 a = tab[2 * i];
    if (a.x == 0) return -1;
    if (a.x == tag && a.z == w[0] && a.w == w[1]) {
      const uint4 b = tab[2 * i + 1];
      if (b.x == w[2] && b.y == w[3] && b.z == w[4] && b.w == w[5]) return (int32_t)a.y;
    }
    i = (i + 1) & mask;
  }
}

// Merge one short pre-token of len symbols in place at Y[0..len), with RK
// as scratch (one lane; Y and RK are the position-indexed global scratch).
// Each round takes the lowest rank r present and rewrites the sequence left
// to right, merging every pair whose rank is r unless its left symbol was
// just consumed; then only pairs touching the new symbol are probed again.
// Returns the final symbol count.
__device__ int lane_merge(int32_t *Y, int32_t *RK, const int len, const uint64_t *tab,
                          const int bits, const int32_t *__restrict__ pair_rank) {
  // the symbols are still bytes: their ranks come from the direct table
  for (int i = 0; i + 1 < len; ++i) RK[i] = pair_rank[(Y[i] << 8) | Y[i + 1]];
  RK[len - 1] = kRankInf;
  int n = len;
  for (;;) {
    int32_t r = kRankInf;
    for (int i = 0; i + 1 < n; ++i) r = min(r, RK[i]);
    if (r == kRankInf) break;
    const int32_t z = 256 + r;
    int o = 0;
    for (int i = 0; i < n; ++o) {
      if (RK[i] == r) {
        Y[o] = z;
        i += 2;
      } else {
        Y[o] = Y[i];
        RK[o] = RK[i];
        i += 1;
      }
    }
    n = o;
    for (int j = 0; j + 1 < n; ++j)
      if (Y[j] == z || Y[j + 1] == z) RK[j] = rank_of(tab, bits, Y[j], Y[j + 1]);
    RK[n - 1] = kRankInf;
  }
  return n;
}

// Rank of (l, r) continuing the linear probe after slot h (rare path).
__device__ __noinline__ int32_t rank_probe_from(const uint64_t *__restrict__ tab, int bits,
                                                uint64_t key, uint64_t h) {
  const uint64_t mask = (1ull << bits) - 1;
  for (;;) {
    h = (h + 1) & mask;
    const uint64_t s = tab[h];
    if ((s >> kSymBits) == key) return (int32_t)(s & ((1u << kSymBits) - 1));
    if (s == kEmptySlot) return kRankInf;
  }
}

// Merge one pre-token of len <= W bytes (read from LDS at b) in registers
// and write its symbols to out; returns their count.  Same rounds as
// lane_merge, but positions never move: a consumed position is marked dead
// and every pair joins a live position to the next live one, so all
// indexing is static and the arrays stay in registers.  The rank probes of
// a round are issued together, so a round costs one table round trip.
template <int W>
__device__ int reg_merge(const uint8_t *b, const int len, int32_t *out, const uint64_t *tab,
                         const int bits, const int32_t *__restrict__ pair_rank) {
  int32_t sym[W], rk[W];
  uint32_t alive = len >= 32 ? ~0u : ((1u << len) - 1u);
#pragma unroll
  for (int i = 0; i < W; ++i) sym[i] = i < len ? (int32_t)b[i] : 0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    rk[i] = (i + 1 < len) ? pair_rank[(sym[i] << 8) | sym[i + 1]] : kRankInf;
  const uint64_t mask = (1ull << bits) - 1;
  for (;;) {
    int32_t r = kRankInf;
#pragma unroll
    for (int i = 0; i < W; ++i) r = min(r, rk[i]);   // dead and last positions hold kRankInf
    if (r == kRankInf) break;
    const int32_t z = 256 + r;
    bool carry = false;  // the previous live position merged: this one is consumed
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const bool live = (alive >> i) & 1u;
      const bool consumed = live && carry;
      const bool merge = live && !carry && rk[i] == r;
      if (consumed) {
        alive &= ~(1u << i);
        rk[i] = kRankInf;
      }
      if (merge) sym[i] = z;
      carry = live ? merge : carry;
    }
    // pairs touching z get new ranks.  Groups of 8 positions from the top:
    // the next live symbol of each position, then the group's first probes
    // issued together, then examined.
    int32_t ns = -1;  // next live symbol above the current group
#pragma unroll
    for (int g = W / 8 - 1; g >= 0; --g) {
      int32_t nx[8];
      uint32_t need = 0;
#pragma unroll
      for (int j = 7; j >= 0; --j) {
        const int i = 8 * g + j;
        nx[j] = ns;
        const bool live = (alive >> i) & 1u;
        if (live && ns >= 0 && (sym[i] == z || ns == z)) need |= 1u << j;
        if (live && ns < 0) rk[i] = kRankInf;
        if (live) ns = sym[i];
      }
      if (need) {
        uint64_t slot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          slot[j] = kEmptySlot;
          if ((need >> j) & 1u) slot[j] = tab[pair_hash(pair_key(sym[8 * g + j], nx[j]), bits)];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((need >> j) & 1u) {
            const int i = 8 * g + j;
            const uint64_t key = pair_key(sym[i], nx[j]);
            if ((slot[j] >> kSymBits) == key) rk[i] = (int32_t)(slot[j] & ((1u << kSymBits) - 1));
            else if (slot[j] == kEmptySlot) rk[i] = kRankInf;
            else rk[i] = rank_probe_from(tab, bits, key, pair_hash(key, bits) & mask);
          }
        }
      }
    }
  }
  int n = 0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    if ((alive >> i) & 1u) out[n++] = sym[i];
  return n;
}

constexpr int kWgPer = 4;                // positions per thread per tile
constexpr int kWgTile = WG * kWgPer;

// Merge one pre-token of n symbols at Y[0..n) with the whole workgroup; RK is
// scratch of n entries (position-indexed global scratch).  Same rounds as
// lane_merge: the lowest rank r is a workgroup minimum, runs of consecutive
// pairs with rank r (only possible for a pair (x, x)) merge at even offsets
// from the run start, and survivors are compacted in place tile by tile.
// Returns the final symbol count.
__device__ int64_t wg_merge(int32_t *Y, int32_t *RK, int64_t n, const uint64_t *tab, int bits,
                            const int32_t *__restrict__ pair_rank, EncShared &s) {
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < n; i += WG)
    RK[i] = (i + 1 < n) ? pair_rank[(Y[i] << 8) | Y[i + 1]] : kRankInf;
  __syncthreads();
  for (;;) {
    int32_t r = kRankInf;
    for (int64_t i = tid; i < n; i += WG) r = min(r, RK[i]);
    r = block_min<WG>(r, s.red);
    if (r == kRankInf) break;
    const int32_t z = 256 + r;
    int64_t out_base = 0;
    int64_t anchor = -1;  // last position before the tile whose pair rank is not r
    bool prev_m = false;  // the pair just before the tile merged
    for (int64_t t0 = 0; t0 < n; t0 += kWgTile) {
      const int64_t p0 = t0 + kWgPer * (int64_t)tid;
      int32_t y[kWgPer], rk[kWgPer];
      uint32_t f = 0;
      int64_t my_anchor = -1;
#pragma unroll
      for (int j = 0; j < kWgPer; ++j) {
        const int64_t p = p0 + j;
        const bool v = p < n;
        rk[j] = v ? RK[p] : kRankInf;
        y[j] = v ? Y[p] : kDead;
        if (v && rk[j] == r) f |= 1u << j;
        else my_anchor = p;
      }
      int64_t tile_anchor;
      int64_t za = block_excl_max64<WG>(my_anchor, -1, s.red64, &tile_anchor);
      za = max(za, anchor);
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < kWgPer; ++j) {
        const int64_t p = p0 + j;
        if (!((f >> j) & 1u)) za = p;
        else if (((p - 1 - za) & 1) == 0) m |= 1u << j;
      }
      s.mflag[tid] = (m >> (kWgPer - 1)) & 1u;
      __syncthreads();
      const uint32_t mprev = tid ? (uint32_t)s.mflag[tid - 1] : (uint32_t)prev_m;
      const bool tile_last_m = s.mflag[WG - 1] != 0;
      // position p is consumed when the pair at p - 1 merged
      const uint32_t consumed = ((m << 1) | mprev) & ((1u << kWgPer) - 1u);
      uint32_t keep = 0;
#pragma unroll
      for (int j = 0; j < kWgPer; ++j)
        if (p0 + j < n && !((consumed >> j) & 1u)) keep |= 1u << j;
      int tile_kept;
      const int kex = block_excl_sum<int, WG>(__popc(keep), s.red, &tile_kept);
      int64_t o = out_base + kex;
#pragma unroll
      for (int j = 0; j < kWgPer; ++j) {
        if ((keep >> j) & 1u) {
          Y[o] = ((m >> j) & 1u) ? z : y[j];
          RK[o] = rk[j];
          ++o;
        }
      }
      anchor = max(anchor, tile_anchor);
      prev_m = tile_last_m;
      out_base += tile_kept;
      __syncthreads();
    }
    n = out_base;
    for (int64_t i = tid; i < n; i += WG) {
      if (i + 1 < n) {
        const int32_t a = Y[i], b = Y[i + 1];
        if (a == z || b == z) RK[i] = rank_of(tab, bits, a, b);
      } else {
        RK[i] = kRankInf;
      }
    }
    __syncthreads();
  }
  return n;
}

__device__ __forceinline__ int32_t out_id(const int32_t *id_map, int32_t sym) {
  return id_map ? id_map[sym] : sym;
}

// End (exclusive, global) of the pre-token that starts at gs and has no start
// in the window, scanning bytes from `from` on.  Whole workgroup.
__device__ int64_t block_global_end(const EncodeArgs &a, EncShared &s, int64_t gs, int64_t from) {
  const int tid = threadIdx.x;
  if (wave_id() == 0) {
    const int64_t d = wave_lower_bound(a.doc_off, a.n_docs + 1, gs + 1);
    if (lane_id() == 0) {
      int64_t dn = d <= a.n_docs ? a.doc_off[d] : a.n_bytes;
      dn = min(max(dn, gs + 1), a.n_bytes);
      s.red64[4] = dn;
    }
  }
  __syncthreads();
  const int64_t limit = s.red64[4];
  __syncthreads();
  const uint8_t *b = a.bytes;
  // from > gs + 1 always (the pre-token fills the window), so q - 1 > gs is
  // inside the document and is not a document start
  for (int64_t q0 = max(from, gs + 2); q0 < limit; q0 += kTile) {
    int cand = kNoStart;
    for (int j = 0; j < 16; ++j) {
      const int64_t q = q0 + 16 * (int64_t)tid + j;
      if (q >= limit) break;
      const uint32_t c0 = byte_class(b[q]), b1 = b[q - 1], c1 = byte_class(b1);
      const bool attach = c0 == kL && b1 == 0x20u && byte_class(b[q - 2]) != kW;
      if (c0 != c1 && !attach) {
        cand = 16 * tid + j;
        break;
      }
    }
    const int first = block_min<WG>(cand, s.red);
    if (first != kNoStart) return q0 + first;
  }
  return limit;
}

// Result of one pre-token, kept in LDS (PV) between the phases:
//   >= 0                    the pre-token is this one symbol
//   [-kPendBase, -1]        its -v symbols are in the global scratch at its start
//   -2 * kPendBase - 1 - q  long-list entry q (q == kMaxLong: the pre-token past the window)
constexpr int32_t kPendBase = 1 << 20;

// Token count of pre-token k from its PV entry (after the merge phases).
__device__ __forceinline__ int64_t pv_ntok(const EncShared &s, int32_t x) {
  if (x >= 0) return 1;
  if (x < -2 * kPendBase) {
    const int q = -2 * kPendBase - 1 - x;
    return q == kMaxLong ? s.ov_ntok : (int64_t)s.long_nt[q];
  }
  return -(int64_t)x;
}

// One chunk: every pre-token whose first byte lies in [c * kChunk, +kChunk).
__device__ void encode_chunk(const EncodeArgs &a, EncShared &s, const int64_t c) {
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  if (tid == 0) {
    s.n_long = 0;
    s.n_miss = 0;
    s.ov_ntok = 0;
    s.pool_used = 0;
  }
  for (int i = tid; i < DB_WORDS; i += WG) s.DB[i] = 0;
  __syncthreads();
  const int64_t c0 = c * kChunk;
  const int64_t n = a.n_bytes;
  const int nwin = (int)min<int64_t>(WIN, n - c0);
  const int nown = (int)min<int64_t>(kChunk, n - c0);
  const bool win_reaches_end = (c0 + nwin == n);

  // 1. document starts in the window (wave 0, from the chunk's first
  //    document onwards, 64 offsets per load); bytes into LDS (all waves)
  if (wave == 0) {
    int64_t d0 = a.first_doc[c];
    d0 = min(max(d0, (int64_t)0), a.n_docs);
    int64_t olo = d0, ohi = d0;
    for (;;) {
      const int64_t d = d0 + lane;
      const int64_t v = d < a.n_docs ? a.doc_off[d] : INT64_MAX;
      const int64_t p = v - c0;
      if (p >= -1 && p < nwin) atomicOr(&s.DB[(p + DB_OFF) >> 5], 1u << ((p + DB_OFF) & 31));
      olo += __popcll(__ballot(v < c0));
      ohi += __popcll(__ballot(v < c0 + nown));
      if (!(__shfl(v, 63, 64) < c0 + nwin)) break;
      d0 += 64;
    }
    if (lane == 0) {
      s.o_lo = olo;
      s.o_hi = ohi;
    }
  }
  {
    const bool aligned = (((uintptr_t)a.bytes) & 15u) == 0;
    for (int g = tid - 1; g < WIN / 16; g += WG) {
      const int64_t gp = c0 + 16 * (int64_t)g;
      uint8_t *dst = &s.B[16 + 16 * g];
      if (aligned && gp >= 0 && gp + 16 <= n) {
        // streamed once: keep it out of the way of the tables in L2
        *reinterpret_cast<u32x4 *>(dst) =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.bytes + gp));
      } else {
        for (int k = 0; k < 16; ++k) {
          const int64_t q = gp + k;
          dst[k] = (q >= 0 && q < n) ? a.bytes[q] : 0;
        }
      }
    }
  }
  __syncthreads();

  // 2. start bits: a document start, or a class change unless a single space
  //    that follows a non-whitespace byte (or opens the document) leads a
  //    letter run.  Positions past the input end read as starts.
  for (int g = tid; g < SB_HALF; g += WG) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int p = 16 * g + k;
      bool st;
      if (p >= nwin) {
        st = win_reaches_end;
      } else if (db_bit(s, p)) {
        st = true;
      } else {
        const uint32_t b0 = s.B[16 + p], b1 = s.B[16 + p - 1], b2 = s.B[16 + p - 2];
        const uint32_t k0 = byte_class(b0), k1 = byte_class(b1);
        const bool attach = k0 == kL && b1 == 0x20u && (db_bit(s, p - 1) || byte_class(b2) != kW);
        st = k0 != k1 && !attach;
      }
      m |= (uint32_t)st << k;
    }
    reinterpret_cast<uint16_t *>(s.SB)[g] = (uint16_t)m;
  }
  __syncthreads();

  // last owned start and whether its pre-token runs past the window
  uint32_t own = 0;
  if (16 * tid < nown) {
    own = sb16(s, tid);
    const int lim = nown - 16 * tid;
    if (lim < 16) own &= (1u << lim) - 1;
  }
  const int ls = block_max<WG>(own ? 16 * tid + 31 - __clz(own) : -1, s.red);
  const int e_last = ls >= 0 ? block_next_start(s, ls + 1) : -1;
  const bool overhang = ls >= 0 && e_last == kNoStart;

  // 3. the owned pre-token starts as one ordered list (prefix popcount), and
  //    the end of the last one
  int n_pt;
  {
    const int pex = block_excl_sum<int, WG>(__popc(own), s.red, &n_pt);
    uint32_t m = own;
    for (int k = pex; m; ++k, m &= m - 1) s.PS[k] = (uint16_t)(16 * tid + __ffs(m) - 1);
    if (tid == 0) s.PS[n_pt] = (uint16_t)(overhang ? WIN : (ls >= 0 ? e_last : 0));
  }
  __syncthreads();

  // 4. each thread takes a contiguous block of the list.  A single byte is its
  //    own token; a pre-token found in the word table takes its symbol; the
  //    rest go to a shared list for the merge loop, with their symbols in an
  //    LDS pool (or in the global scratch at the pre-token's position).
  const int per = (n_pt + WG - 1) / WG;
  const int k0 = min(n_pt, tid * per), k1 = min(n_pt, k0 + per);
  int32_t *gsym = a.gsym + c0;
  int32_t *grank = a.grank + c0;
  for (int k = k0; k < k1; ++k) {
    const int st = s.PS[k];
    int32_t res = -1;
    if (overhang && k == n_pt - 1) {
      res = -2 * kPendBase - 1 - kMaxLong;
    } else {
      const int len = (int)s.PS[k + 1] - st;
      if (len > kLaneMax) {
        const int q = atomicAdd(&s.n_long, 1);  // < kMaxLong: each is > kLaneMax bytes
        s.long_st[q] = st;
        s.long_e[q] = st + len;
        res = -2 * kPendBase - 1 - q;
      } else if (len == 1) {
        res = s.B[16 + st];
      } else {
        if (a.words && len <= kWordMax) {
          uint32_t w[kWordWords];
          pretoken_words(s, st, len, w);
          res = word_lookup(a.words, a.word_bits, w, len);
        }
        if (res < 0) {
          s.miss[atomicAdd(&s.n_miss, 1)] = (uint16_t)k;  // < kChunk / 2: each is >= 2 bytes
          res = -1;                                       // set by the merge below
        }
      }
    }
    s.PV[k] = res;
  }
  __syncthreads();
  {
    // the merge loop for the list, one pre-token per lane, symbols in registers
    // entry q goes to lane q / 4 of wave q % 4: every wave (SIMD) gets a share
    const int n_miss = s.n_miss;
    const int slot = 4 * lane + wave;
    for (int q = slot; q < n_miss; q += WG) {
      const int k = s.miss[q];
      const int st = s.PS[k], len = (int)s.PS[k + 1] - st;
      int nt;
      if (len <= 8) {
        nt = reg_merge<8>(&s.B[16 + st], len, gsym + st, a.table, a.table_bits, a.pair_rank);
      } else if (len <= 16) {
        nt = reg_merge<16>(&s.B[16 + st], len, gsym + st, a.table, a.table_bits, a.pair_rank);
      } else {
        // 17..32 bytes: symbols and ranks in the LDS pool when it has room
        const int off = atomicAdd(&s.pool_used, 2 * len);
        int32_t *Y = gsym + st, *RK = grank + st;
        if (off + 2 * len <= kPool) {
          Y = s.pool + off;
          RK = Y + len;
        }
        for (int j = 0; j < len; ++j) Y[j] = s.B[16 + st + j];
        nt = lane_merge(Y, RK, len, a.table, a.table_bits, a.pair_rank);
        if (Y != gsym + st)
          for (int j = 0; j < nt; ++j) gsym[st + j] = Y[j];
      }
      s.PV[k] = -nt;
    }
  }

  // 5. workgroup tier: longer pre-tokens inside the window, then the one that
  //    runs past it (both in the global scratch at their positions)
  const int n_long = s.n_long;
  for (int q = 0; q < n_long; ++q) {
    const int st = s.long_st[q], e = s.long_e[q];
    for (int p = st + tid; p < e; p += WG) gsym[p] = s.B[16 + p];
    __syncthreads();
    const int64_t nt = wg_merge(gsym + st, grank + st, e - st, a.table, a.table_bits, a.pair_rank, s);
    if (tid == 0) s.long_nt[q] = (int32_t)nt;
  }
  if (overhang) {
    const int64_t gs = c0 + ls;
    const int64_t ge = block_global_end(a, s, gs, c0 + WIN);
    for (int64_t q = gs + tid; q < ge; q += WG) a.gsym[q] = a.bytes[q];
    __syncthreads();
    const int64_t nt = wg_merge(a.gsym + gs, a.grank + gs, ge - gs, a.table, a.table_bits,
                                a.pair_rank, s);
    if (tid == 0) s.ov_ntok = nt;
  }
  __syncthreads();

  // 6. token counts per thread, chained prefix over the chunks, writes
  int64_t cnt = 0;
  for (int k = k0; k < k1; ++k) cnt += pv_ntok(s, s.PV[k]);
  int64_t total;
  const int64_t ex = block_excl_sum<int64_t, WG>(cnt, s.red64, &total);
  {
    // local token offset at each document start, kept at that position in
    // the rank scratch (free again by now) for the offsets written below
    int64_t run = ex;
    for (int k = k0; k < k1; ++k) {
      const int st = s.PS[k];
      if (db_bit(s, st)) grank[st] = (int32_t)run;
      run += pv_ntok(s, s.PV[k]);
    }
  }
  if (wave == 0) {
    const int64_t base = wave_lookback(a.flags, c, total);
    if (lane == 0) s.base = base;
  }
  __syncthreads();
  const int64_t base = s.base;
  bool overflow = false;
  {
    int64_t w = base + ex;
    for (int k = k0; k < k1; ++k) {
      const int32_t x = s.PV[k];
      if (x >= 0) {
        if (w < a.ids_cap) __builtin_nontemporal_store(out_id(a.id_map, x), &a.ids[w]);
        else overflow = true;
        ++w;
        continue;
      }
      if (x < -2 * kPendBase && -2 * kPendBase - 1 - x == kMaxLong) continue;  // below
      const int st = s.PS[k];
      const int32_t *src = gsym + st;
      int nt;
      if (x < -2 * kPendBase) nt = s.long_nt[-2 * kPendBase - 1 - x];
      else nt = -x;
      for (int q = 0; q < nt; ++q, ++w) {
        if (w < a.ids_cap) __builtin_nontemporal_store(out_id(a.id_map, src[q]), &a.ids[w]);
        else overflow = true;
      }
    }
  }
  if (overhang) {
    const int64_t w0 = base + total - s.ov_ntok;
    for (int64_t q = tid; q < s.ov_ntok; q += WG) {
      const int64_t w = w0 + q;
      if (w < a.ids_cap) __builtin_nontemporal_store(out_id(a.id_map, gsym[ls + q]), &a.ids[w]);
      else overflow = true;
    }
  }
  if (overflow) atomicOr(a.status, (int32_t)BPE_STATUS_IDS_CAPACITY);

  // per-document offsets: a document starting at p begins after every token
  // of the pre-tokens that start before p
  for (int64_t d = s.o_lo + tid; d < s.o_hi; d += WG) {
    const int64_t p = min(max(a.doc_off[d] - c0, (int64_t)0), (int64_t)kChunk - 1);
    a.id_off[d] = base + grank[p];
  }
  if (c == a.n_chunks - 1)
    for (int64_t d = s.o_hi + tid; d <= a.n_docs; d += WG) a.id_off[d] = base + total;
  __syncthreads();
}

// One workgroup per chunk.  Chunks are numbered in the order workgroups
// start (an atomic ticket), so the chunk a look-back waits for always belongs
// to a workgroup that is already running.
__global__ void __launch_bounds__(WG) k_encode(EncodeArgs a) {
  __shared__ EncShared s;
  const int tid = threadIdx.x;
  {
    const int64_t per = (a.n_docs + 1 + gridDim.x - 1) / gridDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * per;
    bool bad = false;
    for (int64_t i = i0 + tid; i < min(i0 + per, a.n_docs + 1); i += WG) {
      const int64_t v = a.doc_off[i];
      if (i == 0 && v != 0) bad = true;
      if (i == a.n_docs && v != a.n_bytes) bad = true;
      if (i < a.n_docs && a.doc_off[i + 1] < v) bad = true;
    }
    if (bad) atomicOr(a.status, (int32_t)BPE_STATUS_BAD_DOC_OFFSETS);
  }
  if (tid == 0)
    s.ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  encode_chunk(a, s, (int64_t)s.ticket);
}

// Clears the ticket, the status word and the look-back flags, and finds each
// chunk's first document: the first d with doc_off[d] >= chunk start - 1.
__global__ void k_clear(uint32_t *ticket, uint64_t *flags, int64_t n_flags, int32_t *status,
                        int64_t *first_doc, const int64_t *doc_off, int64_t n_docs, int64_t chunk) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (gid == 0) {
    *ticket = 0;
    *status = 0;
  }
  for (int64_t i = gid; i < n_flags; i += stride) {
    flags[i] = 0;
    if (first_doc) {
      const int64_t key = i * chunk - 1;
      int64_t lo = 0, hi = n_docs + 1;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (doc_off[mid] < key) lo = mid + 1;
        else hi = mid;
      }
      first_doc[i] = lo;
    }
  }
}

// Empty input (one workgroup): clear the status, then check that every
// offset is zero and write zero offsets.
__global__ void k_empty(const int64_t *offs, int64_t n_docs, uint32_t bad_bit, int64_t *out_off,
                        int32_t *status) {
  if (threadIdx.x == 0) *status = 0;
  __syncthreads();
  bool bad = false;
  for (int64_t i = threadIdx.x; i <= n_docs; i += blockDim.x) {
    if (offs[i] != 0) bad = true;
    out_off[i] = 0;
  }
  if (bad) atomicOr(status, (int32_t)bad_bit);
}

// ---- decode ---------------------------------------------------------------
constexpr int DWG = kDecThreads;
constexpr int DPT = kDecPerThread;

struct DecShared {
  int32_t len[kDecChunk];
  int32_t sym[kDecChunk];
  int64_t excl[DWG];
  int64_t red64[8];
  int64_t chunk;
  int64_t o_lo, o_hi;
  int64_t base;
};

__global__ void __launch_bounds__(DWG) k_decode(DecodeArgs a) {
  __shared__ DecShared s;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  {
    const int64_t per = (a.n_docs + 1 + gridDim.x - 1) / gridDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * per;
    bool bad = false;
    for (int64_t i = i0 + tid; i < min(i0 + per, a.n_docs + 1); i += DWG) {
      const int64_t v = a.id_off[i];
      if (i == 0 && v != 0) bad = true;
      if (i == a.n_docs && v != a.n_ids) bad = true;
      if (i < a.n_docs && a.id_off[i + 1] < v) bad = true;
    }
    if (bad) atomicOr(a.status, (int32_t)BPE_STATUS_BAD_ID_OFFSETS);
  }
  if (tid == 0)
    s.chunk = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int64_t c = s.chunk;
  const int64_t i0 = c * kDecChunk;
  const int cnt = (int)min<int64_t>(kDecChunk, a.n_ids - i0);
  if (wave == 0) {
    const int64_t olo = wave_lower_bound(a.id_off, a.n_docs + 1, i0);
    const int64_t ohi = wave_lower_bound(a.id_off, a.n_docs + 1, i0 + cnt);
    if (lane == 0) {
      s.o_lo = olo;
      s.o_hi = ohi;
    }
  }
  bool bad_id = false;
  int64_t mine = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int k = tid * DPT + j;
    int32_t sym = -1, len = 0;
    if (k < cnt) {
      const int32_t id = a.ids[i0 + k];
      if (a.inv_map) sym = (id >= 0 && id < a.inv_size) ? a.inv_map[id] : -1;
      else sym = (id >= 0 && id < a.vocab) ? id : -1;
      if (sym < 0) bad_id = true;
      else len = (int32_t)(a.exp_off[sym + 1] - a.exp_off[sym]);
    }
    s.sym[k] = sym;
    s.len[k] = len;
    mine += len;
  }
  if (bad_id) atomicOr(a.status, (int32_t)BPE_STATUS_BAD_ID);
  int64_t total;
  const int64_t ex = block_excl_sum<int64_t, DWG>(mine, s.red64, &total);
  s.excl[tid] = ex;
  if (wave == 0) {
    const int64_t base = wave_lookback(a.flags, c, total);
    if (lane == 0) s.base = base;
  }
  __syncthreads();
  const int64_t base = s.base;
  bool overflow = false;
  int64_t w = base + ex;
  for (int j = 0; j < DPT; ++j) {
    const int k = tid * DPT + j;
    const int32_t sym = s.sym[k];
    const int32_t len = s.len[k];
    if (sym >= 0) {
      const uint8_t *src = a.exp_bytes + a.exp_off[sym];
      for (int q = 0; q < len; ++q) {
        if (w + q < a.out_cap) a.out[w + q] = src[q];
        else overflow = true;
      }
    }
    w += len;
  }
  if (overflow) atomicOr(a.status, (int32_t)BPE_STATUS_BYTES_CAPACITY);
  for (int64_t d = s.o_lo + tid; d < s.o_hi; d += DWG) {
    const int64_t k64 = a.id_off[d] - i0;
    const int k = (int)min<int64_t>(max<int64_t>(k64, 0), kDecChunk - 1);
    const int t = k / DPT;
    int64_t before = s.excl[t];
    for (int q = t * DPT; q < k; ++q) before += s.len[q];
    a.byte_off[d] = base + before;
  }
  if (c == a.n_chunks - 1)
    for (int64_t d = s.o_hi + tid; d <= a.n_docs; d += DWG) a.byte_off[d] = base + total;
}

}  // namespace

hipError_t launch_clear(uint32_t *ticket, uint64_t *flags, int64_t n_flags, int32_t *status,
                        int64_t *first_doc, const int64_t *doc_off, int64_t n_docs,
                        hipStream_t stream) {
  int64_t blocks = (n_flags + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(k_clear, dim3((unsigned)blocks), dim3(256), 0, stream, ticket, flags, n_flags,
                     status, first_doc, doc_off, n_docs, (int64_t)kChunk);
  return hipGetLastError();
}

hipError_t launch_empty(const int64_t *offs, int64_t n_docs, uint32_t bad_bit, int64_t *out_off,
                        int32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(256), 0, stream, offs, n_docs, bad_bit, out_off,
                     status);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_encode, dim3((unsigned)a.n_chunks), dim3(WG), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_decode, dim3((unsigned)a.n_chunks), dim3(DWG), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bpe
