// bpe_encode.hip -- byte-level BPE encode for gfx950.
//
// The input is cut into 4 KiB chunks; a chunk owns every pre-token whose
// first byte lies in it.  Ten kernels in order on one stream, none of which
// waits on another workgroup:
//   k_docs        each chunk's first document (a binary search per chunk).
//   k_find        scan a chunk (coalesced bytes into LDS, a byte class and a
//                 start bit per byte from a 3-byte window), list its
//                 pre-tokens in order (prefix popcount), and resolve each one
//                 that is a single byte or a whole entry of a word table; the
//                 others go to the chunk's merge-loop list, by length bucket.
//   k_dedup       the call's table of 9-32 byte entries: the first entry with
//                 given bytes owns them, later ones take its result.
//   k_merge       (persistent) the merge loop for 2-8 byte entries and the
//                 9-16 byte owners, one pre-token per lane in LDS columns.
//   k_merge_wide  the same for the 17-32 byte owners.
//   k_merge_long  longer pre-tokens, one wave each: runs of one byte on
//                 their run lengths; up to 2048 bytes in LDS, with each lane
//                 owning a segment of the symbols (256 bytes on) or every
//                 64th position; longer ones in global scratch.
//   k_dupfill     token counts of the entries that took an owner's result.
//   k_offsets     exclusive scan of the per-chunk token counts within blocks
//                 of 1024 chunks; k_bscan the same over the blocks' counts.
//   k_emit        writes each chunk's IDs at its offset, and the
//                 per-document offsets.
//
// Sources: "Tokenization LLM: ... C++" (glitch4techs.com), sections
// "Technical analysis" (the split into words, numbers, punctuation and
// whitespace), "Byte-level encoding", "BPE algorithm" (lowest rank merges
// first, repeat until no ranked pair) and "Vocabulary lookup";
// "Characters, bytes and subwords" (tokenwerk.deckle.io), section "BPE step
// by step" (left to right without overlap: [a,a,a] -> [aa,a]); "Hugging Face
// Tokenizers v1" (dothoosh.com), sections "How v1 works" (merges stay inside
// a pre-token), "Bitcannon" (pre-token boundaries from bit-parallel class
// masks), "Word caching" (a pre-token seen as a whole skips the merge loop),
// "Merge-loop rewrite" (flat arrays, 'no merge' as the largest value,
// batches) and "Road to 1.0.0" (GPU batch encode, output positions in
// parallel).
#include "../../include/bpe.h"
#include "bpe_device.h"

namespace bpe {
namespace {

constexpr int WG = kEncThreads;             // k_find: 4 waves
constexpr int MWG = 64;                     // threads of a merge wave
constexpr int OWG = 1024;                   // k_bscan: one workgroup
constexpr int WIN = kChunk + kHalo;         // window positions [0, WIN)
constexpr int SB_WORDS = kChunk / 32;       // start bits of the owned positions
constexpr int DB_OFF = 32;                  // document-start bit of position p is bit p + DB_OFF
constexpr int DB_WORDS = (WIN + DB_OFF) / 32 + 2;

// Merge-loop list entry: where (13 bits) | length (13 bits) << 13 | overhang
// << 26.  `where` is the pre-token's start in the chunk for bucket 3, and its
// offset in the chunk's mbytes / res regions for buckets 0-2.  An overhang
// entry is a chunk's last pre-token that runs past the window; its length is
// found by the merge kernel.
// Lane-merged entries (at most kLaneMax bytes) instead: o / 4 (12 bits), the
// entry's 4-byte aligned offset in the dense region | len << 12 | the
// pre-token's index k in the chunk << 18.
__device__ __forceinline__ uint32_t lane_entry(int o4, int len, int k) {
  return (uint32_t)o4 | ((uint32_t)len << 12) | ((uint32_t)k << 18);
}
__device__ __forceinline__ int le_o4(uint32_t e) { return (int)(e & 0xFFFu); }
__device__ __forceinline__ int le_len(uint32_t e) { return (int)((e >> 12) & 0x3Fu); }
__device__ __forceinline__ int le_k(uint32_t e) { return (int)(e >> 18); }

// pv value of a merge-loop pre-token: -1 - u.  A lane-merged entry at dense
// offset 4 o4 has u = o4 (its token count goes to cntk at the pre-token's
// index); the q-th wave-merged entry has u = kPvLong + q.
constexpr int kPvLong = 1 << 20;
// pv of a lane-merged pre-token that takes the tokens of another entry with
// the same bytes: -1 - (kPvDup + g), the tokens at res + 4 g.
constexpr int kPvDup = 1 << 21;
// Buckets kDedupFrom..2 go through the call's entry table (k_dedup); the
// shorter entries below are merged wherever they occur.
constexpr int kDedupFrom = 1;
static_assert(kBucketBase[kDedupFrom] == kDrefBase, "dref covers the deduplicated buckets");
__device__ __forceinline__ bool deduped(int b) { return b >= kDedupFrom && b < 3; }

__device__ __forceinline__ uint32_t miss_entry(int st, int len, bool over) {
  return (uint32_t)st | ((uint32_t)len << 13) | ((uint32_t)over << 26);
}
__device__ __forceinline__ int me_start(uint32_t e) { return (int)(e & 0x1FFFu); }
__device__ __forceinline__ int me_len(uint32_t e) { return (int)((e >> 13) & 0x1FFFu); }
__device__ __forceinline__ bool me_over(uint32_t e) { return (e >> 26) & 1u; }

// Length buckets of the merge-loop list (2-8, 9-16, 17-kLaneMax bytes, then
// longer ones and a chunk's last pre-token when it runs past the window).
// Buckets 0-2 are merged one pre-token per lane, bucket 3 by a whole wave.
__device__ __forceinline__ int bucket_of(int len, bool over) {
  return over ? 3 : (len <= 8 ? 0 : (len <= 16 ? 1 : (len <= kLaneMax ? 2 : 3)));
}

// Scratch for the workgroup reductions and the workgroup merge.
template <int NT>
struct Red {
  int32_t red[NT / 64 + 4];
};

// ---- merge loops ----------------------------------------------------------

// Pair keys of the lane merge: rank << 5 | position, so that the smallest
// key is the leftmost pair of the lowest rank.  A pair made during a round
// with a rank below the round's (possible only when ranks are not in
// creation order) carries kKeyDef until the round ends; keys at or above
// kKeyDone stand for no pair.
constexpr uint32_t kKeyDef = 1u << 25;
constexpr uint32_t kKeyDone = 1u << 26;
constexpr uint32_t kKeyNone = 0xFFFFFFFFu;

// One wave's per-lane arrays in LDS, lane-major: element j of lane l at
// [j][l], so that lanes hit distinct banks whatever their indexes.
template <int W>
struct LaneCols {
  uint32_t s[W][64];      // symbol at each position (bytes at the start)
  uint32_t k[W - 1][64];  // key of the pair (position, next live position)
};

// Rank of a byte pair from the direct table in device memory.
struct GlobalPairs {
  const int32_t *__restrict__ pair_rank;
  __device__ __forceinline__ int32_t operator()(uint32_t x, uint32_t y) const {
    return pair_rank[(x << 8) | y];
  }
};

// The live symbols of a lane's column S (bit j of alive: position j), in
// order, to out; returns their count.  They are first packed to the front of
// the column (in place: the k-th live position is at or after k), then
// stored four to a 16-byte store.  out is 16-byte aligned and has room for
// the pre-token's length rounded up to 4 (an entry's tokens sit at 4 times its
// 4-byte aligned dense offset, in a span four times its rounded length), so
// the stores stay inside it; slots past the count hold leftovers.
template <int W>
__device__ __forceinline__ int emit_alive(uint32_t *S, uint32_t alive, int32_t *out) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < W; ++j)
    if ((alive >> j) & 1u) S[64 * n++] = S[64 * j];
#pragma unroll
  for (int q = 0; q < W / 4; ++q)
    if (n > 4 * q)
      *reinterpret_cast<u32x4 *>(out + 4 * q) =
          u32x4{S[64 * (4 * q)], S[64 * (4 * q + 1)], S[64 * (4 * q + 2)], S[64 * (4 * q + 3)]};
  return n;
}

// Merge one pre-token of len <= W bytes (little-endian words w) by one lane
// and write its symbols to out; returns their count.  A round takes the
// lowest rank r and merges its pairs left to right without overlap; here the
// round's merges are made one at a time, always the leftmost pair of rank r:
// merging (x, y) into 256 + r leaves no pair of rank r that overlaps it (a
// merge never takes its own symbol as an operand), so the pairs of rank r
// still present are exactly the rest of the round's.  Positions never move:
// a consumed position leaves the live mask, and each pair joins a live
// position to the next live one.
template <int W, class Pairs>
__device__ int lane_merge(const uint32_t *w, const int len, LaneCols<W> &L, const RankTable &t,
                          const Pairs &pair_rank, int32_t *out) {
  const int lane = lane_id();
  uint32_t *S = &L.s[0][lane];
  uint32_t *K = &L.k[0][lane];
  uint32_t b[W];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    b[j] = (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    S[64 * j] = b[j];
  }
  // the symbols are still bytes: their pair ranks come from the direct table
  int32_t r0[W - 1];
#pragma unroll
  for (int j = 0; j + 1 < W; ++j)
    r0[j] = (j + 1 < len) ? pair_rank(b[j], b[j + 1]) : kRankInf;
#pragma unroll
  for (int j = 0; j + 1 < W; ++j)
    K[64 * j] = r0[j] == kRankInf ? kKeyNone : (((uint32_t)r0[j] << 5) | (uint32_t)j);
  uint32_t alive = len >= 32 ? ~0u : ((1u << len) - 1u);
  uint32_t rcur = kKeyNone;  // rank of the round in progress
  bool def = false;          // some key carries kKeyDef
  for (;;) {
    uint32_t m = kKeyNone;
#pragma unroll
    for (int j = 0; j + 1 < W; ++j) m = min(m, K[64 * j]);
    if (m >= kKeyDone) break;
    const uint32_t r = m >> 5;
    if (def && r != rcur) {
      // the round is over: pairs it made join the next one
#pragma unroll
      for (int j = 0; j + 1 < W; ++j) K[64 * j] &= ~kKeyDef;
      def = false;
      continue;
    }
    rcur = r;
    const int i = (int)(m & 31u);
    const uint32_t above = alive & (0xFFFFFFFEu << i);  // the pair's right symbol first
    const int q = __builtin_ctz(above);
    const uint32_t rest = above & (above - 1u);
    const uint32_t below = alive & ((1u << i) - 1u);
    alive ^= 1u << q;
    const uint32_t z = 256u + r;
    const bool hp = below != 0, ht = rest != 0;
    const int p = hp ? 31 - __builtin_clz(below) : i;
    const int tt = ht ? __builtin_ctz(rest) : i;
    const uint32_t sp = S[64 * p], st = S[64 * tt];
    S[64 * i] = z;
    if (q < W - 1) K[64 * q] = kKeyNone;  // the last position starts no pair
    // ranks of the new pairs (S[p], z) and (z, S[t]): both first buckets at once
    const uint32_t xl = pair_mix(sp, z, t.seed), xr = pair_mix(z, st, t.seed);
    const uint64_t kl = pair_key(sp, z), kr = pair_key(z, st);
    u64x2 bl = {kEmptySlot, kEmptySlot}, br = {kEmptySlot, kEmptySlot};
    if (hp && pair_maybe(t, xl)) bl = t.b[pair_bucket0(xl, t.mask)];
    if (ht && pair_maybe(t, xr)) br = t.b[pair_bucket0(xr, t.mask)];
    int32_t rl = bucket_rank(bl, kl), rr = bucket_rank(br, kr);
    const bool nl = hp && rl == kRankInf && bucket_flag(bl);
    const bool nr = ht && rr == kRankInf && bucket_flag(br);
    if (nl || nr) {
      if (nl) bl = t.b[pair_bucket1(xl, t.mask)];
      if (nr) br = t.b[pair_bucket1(xr, t.mask)];
      if (nl) rl = bucket_rank(bl, kl);
      if (nr) rr = bucket_rank(br, kr);
    }
    uint32_t vl = rl == kRankInf ? kKeyNone : (((uint32_t)rl << 5) | (uint32_t)p);
    uint32_t vr = rr == kRankInf ? kKeyNone : (((uint32_t)rr << 5) | (uint32_t)i);
    if ((uint32_t)rl < r) {
      vl |= kKeyDef;
      def = true;
    }
    if ((uint32_t)rr < r) {
      vr |= kKeyDef;
      def = true;
    }
    if (hp) K[64 * p] = vl;
    K[64 * i] = vr;  // i < q <= W - 1
  }
  return emit_alive<W>(S, alive, out);
}

// The rounds of lds_merge (multi-rank rounds with window radius D; D == 0:
// the lowest rank of the whole pre-token per round) for a pre-token longer
// than the LDS path takes, by one wave on Y[0..n) and RK (global,
// position-indexed), in place.  Each round:
//  1. a pair that is the lowest within D positions on each side gets the
//     sign bit of its RK entry (the windows read RK without that bit, and
//     each step's reads come before its writes);
//  2. merge flags by the run rule (a run of one pair (x, x) merges at even
//     offsets from its first pair, and only if that first pair is a lowest
//     pair) and compaction, 64 positions per step: every read of a step
//     comes before its writes, which land at or before its positions;
//  3. the pairs that touch a new symbol (RK == -1) are probed.
// Returns the final symbol count.
__device__ __noinline__ int64_t wg_merge(int32_t *Y, int32_t *RK, int64_t n, int D, const RankTable &tab,
                            const int32_t *__restrict__ pair_rank) {
  constexpr int32_t kRankBits = 0x7FFFFFFF;  // RK without the candidate bit
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1;
  for (int64_t i = lane; i < n; i += MWG)
    RK[i] = (i + 1 < n) ? pair_rank[(Y[i] << 8) | Y[i + 1]] : kRankInf;
  __syncthreads();
  while (n > 1) {
    int32_t gmin = kRankInf;
    if (D == 0) {
      for (int64_t i = lane; i < n; i += MWG) gmin = min(gmin, RK[i]);
      gmin = wave_min(gmin);
      if (gmin == kRankInf) break;
    }
    // 1. the lowest pairs of their windows
    for (int64_t i0 = 0; i0 < n; i0 += MWG) {
      const int64_t i = i0 + lane;
      if (i >= n) continue;
      const int32_t r = RK[i] & kRankBits;
      int32_t w = gmin;
      if (D > 0) {
        w = r;
        const int64_t j1 = min(i + D, n - 1);
        for (int64_t j = max(i - D, (int64_t)0); j <= j1; ++j) w = min(w, RK[j] & kRankBits);
      }
      if (r < kRankInf && r == w) RK[i] = r | (int32_t)0x80000000;
    }
    __syncthreads();
    // 2. merge flags and compaction (the carries: the run start in force,
    //    its candidate bit, whether the position before the step merged, and
    //    its rank)
    int64_t run = 0, out = 0;
    bool run_c = false, prevm = false, any = false;
    int32_t prevr = kRankInf;
    for (int64_t i0 = 0; i0 < n; i0 += MWG) {
      const int64_t i = i0 + lane;
      const bool in = i < n;
      const int32_t raw = in ? RK[i] : kRankInf;
      const int32_t y = in ? Y[i] : 0;
      const int32_t r = raw & kRankBits;
      const bool c = in && raw < 0;
      const uint64_t cm = __ballot(c);
      const int32_t rl = wave_shift_up1(r, prevr);
      const bool b = in && (i == 0 || rl != r);
      int64_t st = i;
      bool cs = c;
      if (__ballot(in && !b) != 0) {
        const int sl = wave_incl_max(b ? lane : -1);  // the step's last run start at or before
        st = sl >= 0 ? i0 + sl : run;
        cs = sl >= 0 ? ((cm >> sl) & 1u) != 0 : run_c;
      }
      const bool m = c && cs && ((i - st) & 1) == 0;
      const uint64_t bm = __ballot(m);
      const bool cons = lane == 0 ? prevm : ((bm >> (lane - 1)) & 1u) != 0;
      const bool k = in && !cons;
      const uint64_t bk = __ballot(k);
      if (k) {
        const int64_t o = out + __popcll(bk & below);
        Y[o] = m ? 256 + r : y;
        RK[o] = m ? -1 : r;
      }
      any |= bm != 0;
      out += __popcll(bk);
      prevm = ((bm >> 63) & 1u) != 0;
      prevr = lane_value(r, 63);
      run = lane_value(st, 63);
      run_c = lane_value((int32_t)cs, 63) != 0;
    }
    __syncthreads();
    if (!any) break;
    n = out;
    // 3. ranks of the pairs that touch a new symbol
    for (int64_t i0 = 0; i0 < n; i0 += MWG) {
      const int64_t i = i0 + lane;
      if (i >= n) continue;
      const int32_t r = RK[i];
      const int32_t rn = i + 1 < n ? RK[i + 1] : 0;
      int32_t v = r;
      if (i + 1 >= n) v = kRankInf;
      else if (r == -1 || rn == -1) v = rank_of(tab, (uint32_t)Y[i], (uint32_t)Y[i + 1]);
      RK[i] = v;
    }
    __syncthreads();
  }
  return n;
}

// ---- start bits ------------------------------------------------------------------

// Pre-token start bits of the positions 16g .. 16g + 15 (bit k: position
// 16g + k) from the 20 bytes at positions 16g - 4 .. 16g + 15 (w[0]: the four
// before, then four words in order) and the document-start bits doc (bit
// k + 1: position 16g + k, bit 0: position 16g - 1).  A position starts a
// pre-token when it starts a document, or when its class differs from the
// byte before's, unless it is a letter after a single space that follows a
// non-whitespace byte (or starts its document).  Classes: letters A-Z, a-z
// and bytes >= 0x80; digits; whitespace 0x09-0x0D and 0x20; punctuation, the
// rest.
//
// The 16 bytes are first transposed so that byte j of word k is position
// 4j + k: the byte one position back is then the same byte of word k - 1.
// Class flags live in bit 7 of each byte (range tests by byte-wise adds of
// 7-bit values); the lower bits carry no meaning until the final mask.
__device__ __forceinline__ uint32_t start_bits16(const uint32_t w[5], uint32_t doc) {
  constexpr uint32_t H = 0x80808080u, M7 = 0x7F7F7F7Fu;
  const uint32_t t0 = __builtin_amdgcn_perm(w[2], w[1], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(w[2], w[1], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(w[4], w[3], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(w[4], w[3], 0x07030602u);
  uint32_t x[5];
  x[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  x[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  x[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
  x[4] = w[0];  // positions 16g - 4 .. 16g - 1, in order
  uint32_t L[5], D[5], W[5], S[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const uint32_t v = x[k], z = v & M7;
    const uint32_t y = (v | 0x20202020u) & M7;                   // letters folded to lower case
    L[k] = ((y + 0x1F1F1F1Fu) & ~(y + 0x05050505u)) | v;         // 'a'..'z', or >= 0x80
    D[k] = (z + 0x50505050u) & ~(z + 0x46464646u) & ~v;           // '0'..'9'
    S[k] = (z + 0x60606060u) & ~(z + 0x5F5F5F5Fu) & ~v;           // 0x20
    W[k] = ((z + 0x77777777u) & ~(z + 0x72727272u) & ~v) | S[k]; // 0x09..0x0D, or 0x20
  }
  // the flags one and two positions back: word k - 1 (k - 2), or for the
  // first words the last word shifted up one byte, the earlier bytes first
  uint32_t ne[4], att[4], W2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t L1, D1, W1, S1;
    if (k == 0) {
      L1 = __builtin_amdgcn_alignbyte(L[3], L[4], 3);
      D1 = __builtin_amdgcn_alignbyte(D[3], D[4], 3);
      W1 = __builtin_amdgcn_alignbyte(W[3], W[4], 3);
      S1 = __builtin_amdgcn_alignbyte(S[3], S[4], 3);
      W2[k] = __builtin_amdgcn_alignbyte(W[2], W[4] << 8, 3);
    } else {
      L1 = L[k - 1];
      D1 = D[k - 1];
      W1 = W[k - 1];
      S1 = S[k - 1];
      W2[k] = k == 1 ? __builtin_amdgcn_alignbyte(W[3], W[4], 3) : W[k - 2];
    }
    ne[k] = (L[k] ^ L1) | (D[k] ^ D1) | (W[k] ^ W1);
    att[k] = L[k] & S1;
  }
  uint32_t F[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) F[k] = ne[k] & ~(att[k] & ~W2[k]) & H;
  if (doc) {
    // a document start is a start, and a space that starts its document
    // leads the letter after it
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t d0 = 0, d1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d0 |= ((doc >> (4 * j + k + 1)) & 1u) << (8 * j + 7);
        d1 |= ((doc >> (4 * j + k)) & 1u) << (8 * j + 7);
      }
      F[k] = (d0 | (ne[k] & ~(att[k] & (d1 | ~W2[k])))) & H;
    }
  }
  // bit 8j + k of X is position 4j + k; then the four nibbles side by side
  const uint32_t X = (F[0] >> 7) | (F[1] >> 6) | (F[2] >> 5) | (F[3] >> 4);
  const uint32_t t = X | (X >> 4);
  return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
}

// ---- k_find -------------------------------------------------------------------

constexpr int kFindList = 1024;  // byte copies listed for full waves (more: by their own thread)

struct FindShared {
  alignas(16) uint8_t B[16 + WIN + 32];  // B[16 + p] = byte at window position p
  uint32_t SB[SB_WORDS];                 // pre-token start bits, positions [0, kChunk)
  uint32_t DB[DB_WORDS];                 // document start bits, positions [-32, WIN)
  uint16_t PS[kChunk + 2];               // owned pre-token starts in order, then the end
  uint16_t ML[kFindList];                // the pre-tokens that missed the word tables
  u32x4 LM[kShortMax + 1];               // masks of the first len bytes of three words
  Red<WG> r;
  int64_t o_lo, o_hi;
  int e_last;
  uint64_t tally;                        // the entries placed so far (tally_add, hi:lo)
};

// A merge-loop entry's place, as two 32-bit tallies whose fields never carry
// into each other (the bounds hold for any chunk: the owned pre-tokens start
// at distinct positions below kChunk and are disjoint):
//   lo: entries of 2-8 bytes (bits 0-11, at most kChunk / 2), of 9-16 bytes
//       (bits 12-23, at most kChunk / 9 + 1), of 17-kLaneMax bytes (bits
//       24-31, at most kChunk / 17 + 1 < 256)
//   hi: longer entries and the one past the window (bits 0-15), dense-region
//       bytes of the lane-merged ones, each rounded up to 4 (bits 16-31, at
//       most kMissSpan)
// One 64-bit LDS add of a wave's tallies (hi:lo) places all its entries:
// their slots in their buckets' regions and their dense offsets.
__device__ __forceinline__ void tally_add(uint32_t &lo, uint32_t &hi, int b, int len) {
  if (b < 3) {
    lo += 1u << (12 * b);
    hi += (uint32_t)((len + 3) & ~3) << 16;
  } else {
    hi += 1u;
  }
}
__device__ __forceinline__ int tally_count(uint32_t lo, uint32_t hi, int b) {
  return b == 0 ? (int)(lo & 0xFFFu)
       : b == 1 ? (int)((lo >> 12) & 0xFFFu)
       : b == 2 ? (int)(lo >> 24)
                : (int)(hi & 0xFFFFu);
}
static_assert(kChunk / 2 < 4096 && kChunk / 9 + 1 < 4096 && kChunk / 17 + 1 < 256 &&
              kMissSpan < 65536, "tally fields hold a chunk's counts");

// The len bytes at window position st as words at dst (the last word's bytes
// past len are the window's next bytes: readers take len bytes).
__device__ __forceinline__ void copy_words(const FindShared &s, int st, int len, uint32_t *dst) {
  const uint32_t *B32 = reinterpret_cast<const uint32_t *>(s.B);
  const int q = (16 + st) >> 2;
  const uint32_t sh = (uint32_t)((16 + st) & 3);
  uint32_t prev = B32[q];
  for (int i = 0; 4 * i < len; ++i) {
    const uint32_t next = B32[q + i + 1];
    dst[i] = __builtin_amdgcn_alignbyte(next, prev, sh);
    prev = next;
  }
}

__device__ __forceinline__ bool db_bit(const FindShared &s, int p) {
  const int q = p + DB_OFF;
  return (s.DB[q >> 5] >> (q & 31)) & 1u;
}

__device__ __forceinline__ uint32_t sb16(const FindShared &s, int g) {
  return reinterpret_cast<const uint16_t *>(s.SB)[g];
}

// The bytes of the pre-token at window position st (len <= kWordMax) as six
// little-endian words, zero padded.
__device__ __forceinline__ void pretoken_words(const FindShared &s, int st, int len,
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

// The first kShortMax bytes at window position st as three little-endian
// words, the bytes past len zeroed.
__device__ __forceinline__ void short_words(const FindShared &s, int st, int len, uint32_t &w0,
                                            uint32_t &w1, uint32_t &w2) {
  const int b0 = 16 + st;
  const uint32_t *B32 = reinterpret_cast<const uint32_t *>(s.B);
  const int q = b0 >> 2;
  const uint32_t sh = (uint32_t)(b0 & 3);
  const uint32_t r0 = B32[q], r1 = B32[q + 1], r2 = B32[q + 2], r3 = B32[q + 3];
  const u32x4 m = s.LM[min(len, kShortMax)];
  w0 = __builtin_amdgcn_alignbyte(r1, r0, sh) & m.x;
  w1 = __builtin_amdgcn_alignbyte(r2, r1, sh) & m.y;
  w2 = __builtin_amdgcn_alignbyte(r3, r2, sh) & m.z;
}

// Symbol of a pre-token of 2..kShortMax bytes (words w0..w2) in the short
// word table, or -1: the key's bucket displacement, then its one slot (no
// branch: every lane of a wave takes the same two loads).
__device__ __forceinline__ int32_t short_lookup(const EncodeArgs &a, uint32_t w0, uint32_t w1,
                                                uint32_t w2, int len) {
  const uint32_t x = short_mix(w0, w1, w2, (uint32_t)len, a.word_seed);
  const uint32_t d = a.word_disp[x >> a.word_dshift];
  const u32x4 e = reinterpret_cast<const u32x4 *>(
      a.words)[short_slot(x, d, short_step(w0, w1, w2), a.word_mask)];
  const uint32_t tl = (uint32_t)len << 21;
  return ((e.x ^ w0) | (e.y ^ w1) | (e.z ^ w2) | ((e.w ^ tl) & (0xFu << 21))) == 0
             ? (int32_t)(e.w & kWordSymMask)
             : -1;
}

// Symbol of a pre-token of kShortMax + 1..kWordMax bytes in the long word
// table, or -1.
__device__ __forceinline__ int32_t long_lookup(const FindShared &s, const EncodeArgs &a, int st,
                                               int len) {
  uint32_t w[kWordWords];
  pretoken_words(s, st, len, w);
  const uint32_t h = word_hash(w, len, a.lword_seed);
  const uint32_t tag = word_tag(h, len);
  uint32_t i = word_slot0(h, a.lword_mask);
  const u32x4 *tab = reinterpret_cast<const u32x4 *>(a.lwords);
  for (int k = 0; k < 2; ++k) {
    const u32x4 x = tab[2 * i], y = tab[2 * i + 1];
    if (((x.x ^ tag) | (x.z ^ w[0]) | (x.w ^ w[1]) | (y.x ^ w[2]) | (y.y ^ w[3]) | (y.z ^ w[4]) |
         (y.w ^ w[5])) == 0)
      return (int32_t)(x.y & kWordSymMask);
    if (!(x.y & kWordFlag)) return -1;
    i = word_slot1(h, a.lword_mask);
  }
  return -1;
}

// The first document whose offset is at or after the byte before each
// chunk (a binary search per chunk, one thread each): k_find starts its
// document scan there.  The same grid checks the document offsets (start at
// 0, never decrease, end at the input's length), each block its share, and
// flags a block's first chunk (kDocFirstBad) where the share breaks a rule;
// the check's loads are issued before the search's, so that their latencies
// overlap.  It also clears the call's entry table (k_dedup).
constexpr int64_t kDocFirstBad = (int64_t)1 << 62;
__global__ void __launch_bounds__(256) k_docs(EncodeArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool bad = false;
  {
    const int64_t i0 = (int64_t)blockIdx.x * 256 * a.doc_per;
    const int64_t i1 = min(i0 + 256 * a.doc_per, a.n_docs + 1);
    for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) {
      const int64_t v = a.doc_off[i];
      if (i == 0 && v != 0) bad = true;
      if (i == a.n_docs && v != a.n_bytes) bad = true;
      if (i < a.n_docs && a.doc_off[i + 1] < v) bad = true;
    }
  }
  bad = __syncthreads_or(bad);
  if (a.dedup) {
    // the call's entry table starts empty (one 16-byte slot per store,
    // spread over the grid)
    u64x2 *dt = reinterpret_cast<u64x2 *>(a.dt);
    const uint64_t slots = (uint64_t)a.dt_mask + 1, step = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)c; i < slots; i += step) dt[i] = u64x2{0ull, 0ull};
  }
  if (c >= a.n_chunks) return;
  const int64_t key = c * kChunk - 1;
  int64_t lo = 0, hi = a.n_docs + 1;  // first index in [lo, hi) with doc_off >= key
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a.doc_off[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  a.dfirst[c] = lo | ((bad && threadIdx.x == 0) ? kDocFirstBad : 0);
}

// Eight waves per SIMD.
__global__ void __launch_bounds__(WG, 8) k_find(EncodeArgs a) {
  __shared__ FindShared s;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();

  const int64_t c = blockIdx.x;
  const int64_t dfirst = a.dfirst[c];  // (k_docs) loaded early: used after the window loads
  const int64_t c0 = c * kChunk;
  const int64_t n = a.n_bytes;
  const int nwin = (int)min<int64_t>(WIN, n - c0);
  const int nown = (int)min<int64_t>(kChunk, n - c0);
  const bool win_reaches_end = (c0 + nwin == n);
  for (int i = tid; i < DB_WORDS; i += WG) s.DB[i] = 0;
  if (tid <= kShortMax) {
    // masks of the first tid bytes of three little-endian words
    u32x4 m;
    m.x = tid >= 4 ? ~0u : (1u << (8 * tid)) - 1u;
    m.y = tid >= 8 ? ~0u : (tid <= 4 ? 0u : (1u << (8 * (tid - 4))) - 1u);
    m.z = tid >= 12 ? ~0u : (tid <= 8 ? 0u : (1u << (8 * (tid - 8))) - 1u);
    m.w = 0;
    s.LM[tid] = m;
  }

  // 1. the window's bytes, 16 per load (group g covers positions 16g ..
  //    16g + 15; group -1 is the two bytes before the chunk), issued first so
  //    that their latency overlaps the document search.  Every thread loads
  //    from an address clamped into the input, so that no lane is masked off
  //    and nothing waits for these loads before the search; a group that is
  //    not wholly inside the input is copied byte by byte below.
  const bool vec = (((uintptr_t)a.bytes) & 15u) == 0 && n >= 16;
  constexpr int NG = WIN / 16 + 1;  // groups -1 .. WIN / 16 - 1
  u32x4 reg[2];
  if (vec) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t gp = c0 + 16 * (int64_t)(tid - 1 + r * WG);
      const int64_t q = min(max(gp, (int64_t)0), (n - 16) & ~(int64_t)15);
      // streamed once: keep it out of the way of the tables in L2
      reg[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.bytes + q));
    }
  }
  __syncthreads();

  //    document starts in the window (wave 0: a 64-way search for the first
  //    document at or after the byte before the chunk, then 64 offsets per
  //    load)
  if (wave == 0) {
    int64_t d0 = min(dfirst & (kDocFirstBad - 1), a.n_docs);
    int64_t olo = d0, ohi = d0;
    for (;;) {
      const int64_t d = d0 + lane;
      const int64_t v = d < a.n_docs ? a.doc_off[d] : INT64_MAX;
      const int64_t p = v - c0;
      if (p >= -1 && p < nwin) atomicOr(&s.DB[(p + DB_OFF) >> 5], 1u << ((p + DB_OFF) & 31));
      olo += __popcll(__ballot(v < c0));
      ohi += __popcll(__ballot(v < c0 + nown));
      if (!(lane_value(v, 63) < c0 + nwin)) break;
      d0 += 64;
    }
    if (lane == 0) {
      s.o_lo = olo;
      s.o_hi = ohi;
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = tid - 1 + r * WG;
    if (g + 1 >= NG) continue;
    const int64_t gp = c0 + 16 * (int64_t)g;
    uint8_t *dst = &s.B[16 + 16 * g];
    if (vec && gp >= 0 && gp + 16 <= n) {
      *reinterpret_cast<u32x4 *>(dst) = reg[r];
    } else {
      for (int k = 0; k < 16; ++k) {
        const int64_t q = gp + k;
        dst[k] = (q >= 0 && q < n) ? a.bytes[q] : 0;
      }
    }
  }
  __syncthreads();

  // 2. start bits of the owned positions: a document start, or a class
  //    change unless a single space that follows a non-whitespace byte (or
  //    opens the document) leads a letter run.  Positions past the input end
  //    read as starts.
  for (int g = tid; g < kChunk / 16; g += WG) {
    // this thread's 16 bytes, the 4 before them, and the document-start bits
    // of positions 16g - 1 .. 16g + 15, from LDS in four reads
    const u32x4 cur = *reinterpret_cast<const u32x4 *>(&s.B[16 + 16 * g]);
    const uint32_t before = *reinterpret_cast<const uint32_t *>(&s.B[16 + 16 * g - 4]);
    const int q = 16 * g - 1 + DB_OFF;
    const uint64_t dw = (uint64_t)s.DB[q >> 5] | ((uint64_t)s.DB[(q >> 5) + 1] << 32);
    const uint32_t doc = (uint32_t)(dw >> (q & 31));  // bit k + 1: position 16g + k
    const uint32_t w[5] = {before, cur.x, cur.y, cur.z, cur.w};
    uint32_t m = start_bits16(w, doc);
    // positions at or past the window's end read as starts only at the input's end
    const int lim = nwin - 16 * g;
    if (lim < 16) {
      const uint32_t past = lim <= 0 ? 0xFFFFu : (0xFFFFu << lim) & 0xFFFFu;
      m = (m & ~past) | (win_reaches_end ? past : 0u);
    }
    reinterpret_cast<uint16_t *>(s.SB)[g] = (uint16_t)m;
  }
  __syncthreads();

  // 3. the owned pre-token starts (positions below nown) as one ordered list,
  //    then the end of the last: the first start at or after nown, where the
  //    window still has one (else the pre-token runs past the window)
  uint32_t own = 0;
  if (16 * tid < nown) {
    own = sb16(s, tid);
    const int lim = nown - 16 * tid;
    if (lim < 16) own &= (1u << lim) - 1;
  }
  if (wave == 0) {
    // one position per lane, nown .. nown + 63 (the halo), by the same rule
    const int p = nown + lane;
    bool st;
    if (p >= nwin) {
      st = win_reaches_end;
    } else {
      const uint32_t b0 = s.B[16 + p], b1 = s.B[16 + p - 1], b2 = s.B[16 + p - 2];
      const uint32_t c0 = byte_class(b0), c1 = byte_class(b1);
      const bool d0 = db_bit(s, p), d1 = db_bit(s, p - 1);
      const bool attach = c0 == kL && b1 == 0x20u && (d1 || byte_class(b2) != kW);
      st = d0 || (c0 != c1 && !attach);
    }
    const uint64_t m = __ballot(st);
    if (lane == 0) {
      int e = m ? nown + __ffsll((unsigned long long)m) - 1
                : ((win_reaches_end && nwin == WIN) ? WIN : kNoStart);
      s.e_last = e <= WIN ? e : kNoStart;
    }
  }
  int n_pt;
  {
    const int pex = block_excl_sum<int, WG>(__popc(own), s.r.red, &n_pt);
    uint32_t m = own;
    for (int k = pex; m; ++k, m &= m - 1) s.PS[k] = (uint16_t)(16 * tid + __ffs(m) - 1);
    if (tid == 0) s.PS[n_pt] = (uint16_t)(s.e_last == kNoStart ? WIN : s.e_last);
  }
  __syncthreads();
  const bool overhang = n_pt > 0 && s.e_last == kNoStart;

  // 4. each thread resolves every WG-th pre-token: a single byte is its own
  //    token; a pre-token that is a whole word-table entry takes its symbol;
  //    the others (bit j of `missed`: pre-token tid + j WG) are listed and
  //    then placed 64 to a wave, so that the merge-loop path runs on full
  //    waves
  int32_t *pv = a.pv + c * kChunk;
  uint32_t *ml = a.miss + c * kMissMax;
  uint32_t *mb = reinterpret_cast<uint32_t *>(a.mbytes + c * kMissSpan);
  uint32_t missed = 0;
  for (int k = tid, j = 0; k < n_pt; k += WG, ++j) {
    const bool over = overhang && k == n_pt - 1;
    const int st = s.PS[k];
    const int len = over ? 0 : (int)s.PS[k + 1] - st;
    uint32_t w0, w1, w2;
    short_words(s, st, len, w0, w1, w2);
    int32_t v = -1;
    if (len == 1) {
      v = (int32_t)w0;
    } else if (!over) {
      if (len <= kShortMax) {
        if (a.words) v = short_lookup(a, w0, w1, w2, len);
      } else if (len <= kWordMax && a.lwords) {
        v = long_lookup(s, a, st, len);
      }
    }
    if (v >= 0) pv[k] = v;
    else missed |= 1u << j;
  }
  if (tid == 0) s.tally = 0;
  // an entry's slot and dense offset from the tallies before it (elo, ehi):
  // its entry, its pv value, and its bytes
  auto place = [&](int k, uint32_t elo, uint32_t ehi) {
    const bool over = overhang && k == n_pt - 1;
    const int st = s.PS[k];
    const int len = over ? 0 : (int)s.PS[k + 1] - st;
    const int b = bucket_of(len, over);
    const int idx = tally_count(elo, ehi, b);
    const int base = b == 0 ? kBucketBase[0] : b == 1 ? kBucketBase[1] : b == 2 ? kBucketBase[2] : kBucketBase[3];
    if (b < 3) {
      const int o4 = (int)(ehi >> 18);
      copy_words(s, st, len, mb + o4);
      ml[base + idx] = lane_entry(o4, len, k);
      pv[k] = -1 - o4;
    } else {
      ml[base + idx] = miss_entry(st, len, over);
      pv[k] = -1 - kPvLong - idx;
    }
  };
  int n_miss;
  const int mex = block_excl_sum<int, WG>(__popc(missed), s.r.red, &n_miss);
  {
    int o = mex;
    for (uint32_t m = missed; m; m &= m - 1, ++o)
      if (o < kFindList) s.ML[o] = (uint16_t)(tid + (__ffs(m) - 1) * WG);
  }
  __syncthreads();
  // the listed entries, 64 to a wave: the wave's tallies by two prefix sums,
  // placed by one LDS add
  const int n_list = min(n_miss, kFindList);
  for (int i0 = wave * 64; i0 < n_list; i0 += WG) {
    const int i = i0 + lane;
    const bool act = i < n_list;
    const int k = act ? (int)s.ML[i] : 0;
    uint32_t tlo = 0, thi = 0;
    if (act) {
      const bool over = overhang && k == n_pt - 1;
      const int st = s.PS[k];
      const int len = over ? 0 : (int)s.PS[k + 1] - st;
      tally_add(tlo, thi, bucket_of(len, over), len);
    }
    const uint32_t ilo = (uint32_t)wave_incl_sum((int32_t)tlo);
    const uint32_t ihi = (uint32_t)wave_incl_sum((int32_t)thi);
    uint64_t wb = 0;
    if (lane == 63) wb = atomicAdd(&s.tally, ((uint64_t)ihi << 32) | ilo);
    const uint32_t blo = (uint32_t)lane_value((int32_t)(uint32_t)wb, 63);
    const uint32_t bhi = (uint32_t)lane_value((int32_t)(uint32_t)(wb >> 32), 63);
    if (act) place(k, blo + ilo - tlo, bhi + ihi - thi);
  }
  if (n_miss > kFindList) {  // the rest, each by the thread that found it
    int o = mex;
    for (uint32_t m = missed; m; m &= m - 1, ++o) {
      if (o < kFindList) continue;
      const int k = tid + (__ffs(m) - 1) * WG;
      const bool over = overhang && k == n_pt - 1;
      const int len = over ? 0 : (int)s.PS[k + 1] - (int)s.PS[k];
      uint32_t tlo = 0, thi = 0;
      tally_add(tlo, thi, bucket_of(len, over), len);
      const uint64_t e = atomicAdd(&s.tally, ((uint64_t)thi << 32) | tlo);
      place(k, (uint32_t)e, (uint32_t)(e >> 32));
    }
  }
  __syncthreads();
  const bool any_bad = (dfirst & kDocFirstBad) != 0;
  const uint32_t nlo = (uint32_t)s.tally, nhi = (uint32_t)(s.tally >> 32);
  if (tid == 0) {
    int32_t *m = a.meta + kMetaInts * c;
    int n_miss = 0;
#pragma unroll
    for (int b = 0; b < kBuckets; ++b) {
      const int nb = tally_count(nlo, nhi, b);
      m[kMetaBucket + b] = nb;
      n_miss += nb;
    }
    m[kMetaPretokens] = n_pt;
    m[kMetaMisses] = n_miss;
    m[kMetaStatus] = any_bad ? (int32_t)BPE_STATUS_BAD_DOC_OFFSETS : 0;
    m[kMetaBytes] = (int)(nhi >> 16);
    if (c == 0) a.dstat[0] = 0u;
    a.doc_rng[2 * c] = s.o_lo;
    a.doc_rng[2 * c + 1] = s.o_hi;
  }
  // each document that starts here: the index of its first pre-token
  for (int64_t d = s.o_lo + tid; d < s.o_hi; d += WG) {
    const int p = (int)min(max(a.doc_off[d] - c0, (int64_t)0), (int64_t)kChunk - 1);
    int lo = 0, hi = n_pt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)s.PS[mid] < p) lo = mid + 1;
      else hi = mid;
    }
    a.doc_pt[d] = lo;
  }
}

// Two pre-tokens per lane, merged as lane_merge does, their steps taken side
// by side: both minimums, both pairs' symbols and all four new pairs' first
// buckets are read before any write, so the latencies of the two overlap.
// Entry A (words wa, la bytes) uses columns LA, entry B columns LB; an entry
// with va / vb false is absent.  Returns the token counts in *nta, *ntb.
template <int W, class Pairs>
__device__ void lane_merge2(const uint32_t *wa, int la, bool va, int32_t *outa, int *nta,
                            const uint32_t *wb, int lb, bool vb, int32_t *outb, int *ntb,
                            LaneCols<W> &LA, LaneCols<W> &LB, const RankTable &t,
                            const Pairs &pair_rank) {
  const int lane = lane_id();
  uint32_t *SA = &LA.s[0][lane], *KA = &LA.k[0][lane];
  uint32_t *SB = &LB.s[0][lane], *KB = &LB.k[0][lane];
  if (!va) la = 0;
  if (!vb) lb = 0;
  {
    uint32_t ba[W], bb[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      ba[j] = (wa[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      bb[j] = (wb[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      SA[64 * j] = ba[j];
      SB[64 * j] = bb[j];
    }
    int32_t ra[W - 1], rb[W - 1];
#pragma unroll
    for (int j = 0; j + 1 < W; ++j) {
      ra[j] = (j + 1 < la) ? pair_rank(ba[j], ba[j + 1]) : kRankInf;
      rb[j] = (j + 1 < lb) ? pair_rank(bb[j], bb[j + 1]) : kRankInf;
    }
#pragma unroll
    for (int j = 0; j + 1 < W; ++j) {
      KA[64 * j] = ra[j] == kRankInf ? kKeyNone : (((uint32_t)ra[j] << 5) | (uint32_t)j);
      KB[64 * j] = rb[j] == kRankInf ? kKeyNone : (((uint32_t)rb[j] << 5) | (uint32_t)j);
    }
  }
  uint32_t aliveA = la >= 32 ? ~0u : ((1u << la) - 1u);
  uint32_t aliveB = lb >= 32 ? ~0u : ((1u << lb) - 1u);
  uint32_t rcA = kKeyNone, rcB = kKeyNone;
  bool defA = false, defB = false;
  for (;;) {
    uint32_t mA = kKeyNone, mB = kKeyNone;
#pragma unroll
    for (int j = 0; j + 1 < W; ++j) {
      mA = min(mA, KA[64 * j]);
      mB = min(mB, KB[64 * j]);
    }
    const bool goA = mA < kKeyDone, goB = mB < kKeyDone;
    if (!goA && !goB) break;
    const uint32_t rA = mA >> 5, rB = mB >> 5;
    const bool fixA = defA && goA && rA != rcA, fixB = defB && goB && rB != rcB;
    if (fixA || fixB) {
      // a round is over: pairs it made join the next one
      if (fixA) {
#pragma unroll
        for (int j = 0; j + 1 < W; ++j) KA[64 * j] &= ~kKeyDef;
        defA = false;
      }
      if (fixB) {
#pragma unroll
        for (int j = 0; j + 1 < W; ++j) KB[64 * j] &= ~kKeyDef;
        defB = false;
      }
      continue;
    }
    // positions: the merged pair (i, q), its live neighbours p and t
    const int iA = goA ? (int)(mA & 31u) : 0, iB = goB ? (int)(mB & 31u) : 0;
    const uint32_t abA = aliveA & (0xFFFFFFFEu << iA), abB = aliveB & (0xFFFFFFFEu << iB);
    const int qA = goA ? __builtin_ctz(abA) : 0, qB = goB ? __builtin_ctz(abB) : 0;
    const uint32_t reA = abA & (abA - 1u), reB = abB & (abB - 1u);
    const uint32_t beA = aliveA & ((1u << iA) - 1u), beB = aliveB & ((1u << iB) - 1u);
    const bool hpA = goA && beA != 0, htA = goA && reA != 0;
    const bool hpB = goB && beB != 0, htB = goB && reB != 0;
    const int pA = hpA ? 31 - __builtin_clz(beA) : iA, tA = htA ? __builtin_ctz(reA) : iA;
    const int pB = hpB ? 31 - __builtin_clz(beB) : iB, tB = htB ? __builtin_ctz(reB) : iB;
    const uint32_t spA = SA[64 * pA], stA = SA[64 * tA];
    const uint32_t spB = SB[64 * pB], stB = SB[64 * tB];
    const uint32_t zA = 256u + rA, zB = 256u + rB;
    // the new pairs' ranks: four first buckets at once
    const uint32_t xlA = pair_mix(spA, zA, t.seed), xrA = pair_mix(zA, stA, t.seed);
    const uint32_t xlB = pair_mix(spB, zB, t.seed), xrB = pair_mix(zB, stB, t.seed);
    const uint64_t klA = pair_key(spA, zA), krA = pair_key(zA, stA);
    const uint64_t klB = pair_key(spB, zB), krB = pair_key(zB, stB);
    const u64x2 none = {kEmptySlot, kEmptySlot};
    u64x2 blA = none, brA = none, blB = none, brB = none;
    if (hpA && pair_maybe(t, xlA)) blA = t.b[pair_bucket0(xlA, t.mask)];
    if (htA && pair_maybe(t, xrA)) brA = t.b[pair_bucket0(xrA, t.mask)];
    if (hpB && pair_maybe(t, xlB)) blB = t.b[pair_bucket0(xlB, t.mask)];
    if (htB && pair_maybe(t, xrB)) brB = t.b[pair_bucket0(xrB, t.mask)];
    int32_t rlA = bucket_rank(blA, klA), rrA = bucket_rank(brA, krA);
    int32_t rlB = bucket_rank(blB, klB), rrB = bucket_rank(brB, krB);
    const bool nlA = hpA && rlA == kRankInf && bucket_flag(blA);
    const bool nrA = htA && rrA == kRankInf && bucket_flag(brA);
    const bool nlB = hpB && rlB == kRankInf && bucket_flag(blB);
    const bool nrB = htB && rrB == kRankInf && bucket_flag(brB);
    if (nlA || nrA || nlB || nrB) {
      if (nlA) blA = t.b[pair_bucket1(xlA, t.mask)];
      if (nrA) brA = t.b[pair_bucket1(xrA, t.mask)];
      if (nlB) blB = t.b[pair_bucket1(xlB, t.mask)];
      if (nrB) brB = t.b[pair_bucket1(xrB, t.mask)];
      if (nlA) rlA = bucket_rank(blA, klA);
      if (nrA) rrA = bucket_rank(brA, krA);
      if (nlB) rlB = bucket_rank(blB, klB);
      if (nrB) rrB = bucket_rank(brB, krB);
    }
    if (goA) {
      aliveA ^= 1u << qA;
      SA[64 * iA] = zA;
      if (qA < W - 1) KA[64 * qA] = kKeyNone;
      uint32_t vl = rlA == kRankInf ? kKeyNone : (((uint32_t)rlA << 5) | (uint32_t)pA);
      uint32_t vr = rrA == kRankInf ? kKeyNone : (((uint32_t)rrA << 5) | (uint32_t)iA);
      if ((uint32_t)rlA < rA) {
        vl |= kKeyDef;
        defA = true;
      }
      if ((uint32_t)rrA < rA) {
        vr |= kKeyDef;
        defA = true;
      }
      if (hpA) KA[64 * pA] = vl;
      KA[64 * iA] = vr;
      rcA = rA;
    }
    if (goB) {
      aliveB ^= 1u << qB;
      SB[64 * iB] = zB;
      if (qB < W - 1) KB[64 * qB] = kKeyNone;
      uint32_t vl = rlB == kRankInf ? kKeyNone : (((uint32_t)rlB << 5) | (uint32_t)pB);
      uint32_t vr = rrB == kRankInf ? kKeyNone : (((uint32_t)rrB << 5) | (uint32_t)iB);
      if ((uint32_t)rlB < rB) {
        vl |= kKeyDef;
        defB = true;
      }
      if ((uint32_t)rrB < rB) {
        vr |= kKeyDef;
        defB = true;
      }
      if (hpB) KB[64 * pB] = vl;
      KB[64 * iB] = vr;
      rcB = rB;
    }
  }
  *nta = emit_alive<W>(SA, aliveA, outa);
  *ntb = emit_alive<W>(SB, aliveB, outb);
}

// ---- k_merge, k_merge_wide ---------------------------------------------------

constexpr int kGroup = 4;       // chunks per merge wave: batches of one bucket span them
constexpr int kMergeWaves = 4;  // waves per merge workgroup, each on its own group

struct MergeShared {
  int32_t meta[kGroup][kMetaInts];
  int32_t tok[kGroup];
};

__device__ void load_group(const EncodeArgs &a, MergeShared &s, int64_t cg, int nf) {
  const int lane = lane_id();
  if (lane < kMetaInts * nf) (&s.meta[0][0])[lane] = a.meta[kMetaInts * cg + lane];
  if (lane < kGroup) s.tok[lane] = 0;
  __syncthreads();
}

// The group of one wave of a lane-merge workgroup: its chunk meta read with
// scalar loads.
struct LaneGroup {
  int64_t cg;  // first chunk
  int nf;      // chunks in the group
  int cnt[kGroup][kBuckets];
};

// Group q (chunks lgroup q .., lgroup <= kGroup) of the merge-loop lists;
// false past the last.
// The counts of buckets kDedupFrom..2 are their owners', listed in olist
// (all their entries, in a chunk that did not go through the call's table).
__device__ __forceinline__ bool lane_group(const EncodeArgs &a, int64_t q, LaneGroup &G) {
  G.cg = q * a.lgroup;
  if (G.cg >= a.n_chunks) return false;
  G.nf = (int)min<int64_t>(a.lgroup, a.n_chunks - G.cg);
  // every count loaded (the group's last chunk again past its end), so that
  // all the loads are in flight together
#pragma unroll
  for (int f = 0; f < kGroup; ++f) {
    const int32_t *m = a.meta + kMetaInts * (G.cg + min(f, G.nf - 1));
#pragma unroll
    for (int b = 0; b < kBuckets; ++b) G.cnt[f][b] = m[(deduped(b) ? kMetaOwners : kMetaBucket) + b];
  }
#pragma unroll
  for (int f = 0; f < kGroup; ++f)
#pragma unroll
    for (int b = 0; b < kBuckets; ++b)
      if (f >= G.nf) G.cnt[f][b] = 0;
  return true;
}

// The list entry of bucket b, chunk c at idx: its miss entry and, for an
// owner in the call's entry table, its slot (else kNoSlot).
__device__ __forceinline__ uint64_t group_list_entry(const EncodeArgs &a, int b, int64_t c,
                                                     int idx) {
  return deduped(b) ? a.olist[c * kMissMax + idx]
                    : ((uint64_t)kNoSlot << 32 | a.miss[c * kMissMax + idx]);
}

__device__ __forceinline__ int64_t wave_group(int64_t first) {
  return first + __builtin_amdgcn_readfirstlane(wave_id());
}

// Bucket b of the group's lists, one pre-token per lane with W-wide LDS
// columns, 64 entries per batch.  An entry's bytes are read from its chunk's
// dense mbytes region and its tokens written to res at the same offset (never
// more tokens than bytes, so entries do not overlap), their count to cntk
// at the pre-token's index; the return value holds the tokens per chunk, 16
// bits each.
template <int W, class Pairs>
__device__ uint64_t merge_bucket(const EncodeArgs &a, const LaneGroup &G, int b, LaneCols<W> &L,
                                 const Pairs &pairs, const uint32_t *filt = nullptr) {
  const int lane = lane_id();
  const RankTable t{reinterpret_cast<const u64x2 *>(a.table), a.table_mask, a.table_seed, filt};
  // per chunk: entries of the bucket before the chunk's (uniform across the wave)
  int pre[kGroup];
  int total = 0;
#pragma unroll
  for (int f = 0; f < kGroup; ++f) {
    pre[f] = total;
    total += G.cnt[f][b];
  }
  const int base = kBucketBase[b];
  uint64_t tok = 0;
  for (int s0 = 0; s0 < total; s0 += 64) {
    const int g = s0 + lane;
    if (g >= total) break;
    int f = 0, idx = base + g;
#pragma unroll
    for (int k = 1; k < kGroup; ++k)
      if (g >= pre[k]) {
        f = k;
        idx = base + g - pre[k];
      }
    const int64_t c = G.cg + f;
    const uint64_t ol = group_list_entry(a, b, c, idx);
    const uint32_t e = (uint32_t)ol, slot = (uint32_t)(ol >> 32);
    const int o4 = le_o4(e), o = o4 << 2;  // 4-byte aligned
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.mbytes + c * kMissSpan + o);
    uint32_t w[W / 4];
#pragma unroll
    for (int i = 0; i < W / 4; ++i) w[i] = src[i];
    const int nt = lane_merge<W>(w, le_len(e), L, t, pairs, a.res + c * kMissSpan + o);
    a.cntk[c * kChunk + le_k(e)] = (uint8_t)nt;
    if (slot != kNoSlot) reinterpret_cast<uint32_t *>(a.dt)[4 * (size_t)slot + 3] = (uint32_t)nt;
    tok += (uint64_t)nt << (16 * f);
  }
  return tok;
}

// Bucket b as merge_bucket does, two entries per lane (lane_merge2), 128
// entries per batch; the two column sets share the W-wide region of L2.
template <int W, class Pairs>
__device__ uint64_t merge_bucket2(const EncodeArgs &a, const LaneGroup &G, int b,
                                  LaneCols<2 * W> &L2, const Pairs &pairs,
                                  const uint32_t *filt = nullptr) {
  static_assert(2 * sizeof(LaneCols<W>) <= sizeof(LaneCols<2 * W>), "two column sets fit");
  const int lane = lane_id();
  const RankTable t{reinterpret_cast<const u64x2 *>(a.table), a.table_mask, a.table_seed, filt};
  LaneCols<W> &LA = *reinterpret_cast<LaneCols<W> *>(&L2);
  LaneCols<W> &LB = *(reinterpret_cast<LaneCols<W> *>(&L2) + 1);
  int pre[kGroup];
  int total = 0;
#pragma unroll
  for (int f = 0; f < kGroup; ++f) {
    pre[f] = total;
    total += G.cnt[f][b];
  }
  const int base = kBucketBase[b];
  uint64_t tok = 0;
  for (int s0 = 0; s0 < total; s0 += 128) {
    int f[2], o[2], len[2], kk[2];
    int64_t c[2];
    bool v[2];
    uint32_t sl[2];
    uint32_t w[2][W / 4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = s0 + 64 * h + lane;
      v[h] = g < total;
      f[h] = 0;
      int idx = base + (v[h] ? g : 0);
#pragma unroll
      for (int k = 1; k < kGroup; ++k)
        if (v[h] && g >= pre[k]) {
          f[h] = k;
          idx = base + g - pre[k];
        }
      c[h] = G.cg + f[h];
      const uint64_t ol =
          v[h] ? group_list_entry(a, b, c[h], idx) : ((uint64_t)kNoSlot << 32);
      const uint32_t e = (uint32_t)ol;
      sl[h] = (uint32_t)(ol >> 32);
      o[h] = le_o4(e) << 2;
      len[h] = le_len(e);
      kk[h] = le_k(e);
      const uint32_t *src = reinterpret_cast<const uint32_t *>(a.mbytes + c[h] * kMissSpan + o[h]);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) w[h][i] = v[h] ? src[i] : 0u;
    }
    if (!v[0]) break;
    int nt0 = 0, nt1 = 0;
    lane_merge2<W>(w[0], len[0], v[0], a.res + c[0] * kMissSpan + o[0], &nt0, w[1], len[1], v[1],
                   a.res + c[1] * kMissSpan + o[1], &nt1, LA, LB, t, pairs);
    uint32_t *dt32 = reinterpret_cast<uint32_t *>(a.dt);
    a.cntk[c[0] * kChunk + kk[0]] = (uint8_t)nt0;
    if (sl[0] != kNoSlot) dt32[4 * (size_t)sl[0] + 3] = (uint32_t)nt0;
    tok += (uint64_t)nt0 << (16 * f[0]);
    if (v[1]) {
      a.cntk[c[1] * kChunk + kk[1]] = (uint8_t)nt1;
      if (sl[1] != kNoSlot) dt32[4 * (size_t)sl[1] + 3] = (uint32_t)nt1;
      tok += (uint64_t)nt1 << (16 * f[1]);
    }
  }
  return tok;
}

// Per-chunk token sums of the wave (16 bits each in tok).
__device__ __forceinline__ uint64_t wave_tok_sum(uint64_t tok) {
  return wave_sum(tok);
}

constexpr int kMergePWaves = 16;  // waves of a persistent k_merge workgroup, one per CU

struct PMergeShared {
  LaneCols<16> cols[kMergePWaves];
  uint32_t filt[kPairFilterWords];  // the pair filter: most pairs without a rank stay in the CU
  int next;                         // next group of this workgroup's share
};

// Merge-loop lists of kGroup consecutive chunks per wave, buckets 0 (2-8
// bytes) and 1 (9-16 bytes).  The entries of one bucket are taken 64 at a
// time across the chunks, so every lane of a batch runs the same merge width.
// tot[c] gets the chunk's count so far (its resolved pre-tokens and these
// buckets) with its status bits on top.  One workgroup per compute unit,
// kMergePWaves waves that take the groups of its share (every gridDim.x-th)
// one at a time.  The merges' pair filter is copied to LDS: a new pair whose
// filter bit is clear skips its rank probe.
__global__ void __launch_bounds__(MWG *kMergePWaves) k_merge(EncodeArgs a) {
  __shared__ PMergeShared s;
  const int tid = threadIdx.x, lane = lane_id();
  {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.pair_filter);
    u32x4 *dst = reinterpret_cast<u32x4 *>(s.filt);
    for (int i = tid; i < kPairFilterWords / 4; i += MWG * kMergePWaves) dst[i] = src[i];
    if (tid == 0) s.next = 0;
  }
  __syncthreads();
  const GlobalPairs pairs{a.pair_rank};
  LaneCols<16> &L = s.cols[wave_id()];
  for (;;) {
    int q = 0;
    if (lane == 0) q = atomicAdd(&s.next, 1);
    q = lane_value(q, 0);
    LaneGroup G;
    if (!lane_group(a, (int64_t)blockIdx.x + (int64_t)gridDim.x * q, G)) break;
    uint64_t tok = merge_bucket2<8>(a, G, 0, L, pairs, s.filt);
    tok += merge_bucket<16>(a, G, 1, L, pairs, s.filt);
    tok = wave_tok_sum(tok);
    if (lane < G.nf) {
      const int64_t c = G.cg + lane;
      const int32_t *m = a.meta + kMetaInts * c;
      const int64_t t = (int64_t)(m[kMetaPretokens] - m[kMetaMisses]) +
                        (int64_t)((tok >> (16 * lane)) & 0xFFFFu);
      a.tot[c] = t | ((int64_t)m[kMetaStatus] << kCountBits);
    }
  }
}

// Bucket 2 (17-32 bytes) of the same groups; adds its token counts to tot.
__global__ void __launch_bounds__(MWG *kMergeWaves) k_merge_wide(EncodeArgs a) {
  __shared__ LaneCols<32> cols[kMergeWaves];
  LaneGroup G;
  if (!lane_group(a, wave_group((int64_t)blockIdx.x * kMergeWaves), G)) return;
  int any = 0;
#pragma unroll
  for (int f = 0; f < kGroup; ++f) any += G.cnt[f][2];
  if (any == 0) return;
  uint64_t tok = wave_tok_sum(merge_bucket<32>(a, G, 2, cols[wave_id()], GlobalPairs{a.pair_rank}));
  const int lane = lane_id();
  if (lane < G.nf) {
    const int32_t add = (int32_t)((tok >> (16 * lane)) & 0xFFFFu);
    if (add) a.tot[G.cg + lane] += add;
  }
}

// ---- k_dedup, k_dupfill ----------------------------------------------------
// The pages' word cache ("Hugging Face Tokenizers v1", section "Word
// caching": a pre-token seen before skips the merge loop), built for each call
// from nothing.  The first lane-merged entry with given bytes to claim a slot
// of the call's table owns them and is merged; a later one with the same bytes
// takes, once the owner is merged, the owner's token count and its tokens (pv
// points at them).  Nothing is kept from one call to the next.
//
// A slot is 16 bytes: the claimed key (hash bits and the entry's length, above
// g, the owner's offset / 4 in mbytes), then g again and, once the owner is
// merged, its token count.  A key whose upper half matches is checked against
// the bytes at g.

constexpr int kDedupProbes = 16;  // slots tried before an entry merges itself
constexpr int kDedupSeed = 256;    // chunks of the first, seeding launch

// The bytes (at most 32) at 4-byte offset q of mbytes as eight words, zero
// from byte len on.  All eight are loaded, with no branch between the loads
// (mbytes has room past its last entry for that).
__device__ __forceinline__ void entry_words(const uint8_t *mbytes, uint64_t q, int len,
                                            uint32_t *w) {
  const uint32_t *src = reinterpret_cast<const uint32_t *>(mbytes) + q;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = src[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int valid = len - 4 * i;
    w[i] &= valid >= 4 ? ~0u : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
  }
}

__device__ __forceinline__ uint32_t entry_hash(const uint32_t *w, int len) {
  uint32_t x = mix32((uint32_t)len * 0x9E3779B9u);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (4 * i < len) x = mix32(x ^ w[i]) + (uint32_t)i;
  return x;
}

// List entries of bucket b of a chunk (meta m) that go through the table.
__device__ __forceinline__ int dedup_count(const int32_t *m, int b) {
  return deduped(b) ? m[kMetaBucket + b] : 0;
}

// Entry g of buckets 0-2 of a chunk, taken in bucket order: its list index.
__device__ __forceinline__ int lane_list_index(int g, int n0, int n01, int &b) {
  b = g < n0 ? 0 : (g < n01 ? 1 : 2);
  return b == 0 ? g : (b == 1 ? kBucketBase[1] + g - n0 : kBucketBase[2] + g - n01);
}

// One wave per chunk of [c_lo, c_hi): every lane-merged entry becomes an
// owner (merged itself, listed in olist by bucket) or takes the owner of its
// bytes (dref = the slot); the owner counts go to meta.
__global__ void __launch_bounds__(256) k_dedup(EncodeArgs a, int64_t c_lo, int64_t c_hi,
                                               int seeding) {
  const int64_t c = c_lo + (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave_id());
  if (c >= c_hi) return;
  const int lane = lane_id();
  const int32_t *m = a.meta + kMetaInts * c;
  // after the first kDedupSeed chunks: if at their rate of new byte strings
  // the call's would overfill the table four times over, the text has few
  // repeats, and the rest is merged without the table
  const uint64_t slots = (uint64_t)a.dt_mask + 1;
  const bool use = a.dedup && (seeding || (uint64_t)a.dstat[0] * (uint64_t)a.n_chunks <=
                                              4 * slots * (uint64_t)kDedupSeed);
  int claims = 0;
  const int n0 = dedup_count(m, 0), n01 = n0 + dedup_count(m, 1);
  const int n = n01 + dedup_count(m, 2);
  if (!use) {  // every entry merges itself: the lists as they are
    for (int g = lane; g < n; g += 64) {
      int b;
      const int idx = lane_list_index(g, n0, n01, b);
      a.olist[c * kMissMax + idx] = (uint64_t)a.miss[c * kMissMax + idx] | ((uint64_t)kNoSlot << 32);
    }
    if (lane < 3) a.meta[kMetaInts * c + kMetaOwners + lane] = m[kMetaBucket + lane];
    return;
  }
  const uint32_t q0 = (uint32_t)c * (kMissSpan / 4);  // the chunk's mbytes, in words
  const uint64_t below = (1ull << lane) - 1;
  uint32_t *dt32 = reinterpret_cast<uint32_t *>(a.dt);
  const u64x2 *dt2 = reinterpret_cast<const u64x2 *>(a.dt);
  int own0 = 0, own1 = 0, own2 = 0;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int g = s0 + lane;
    const bool v = g < n;
    int b;
    const int idx = lane_list_index(g, n0, n01, b);
    const uint32_t e = v ? a.miss[c * kMissMax + idx] : 0u;
    bool owner = true;
    uint32_t slot = kNoSlot;
    if (v) {
      const int len = le_len(e);
      const uint32_t gme = q0 + le_o4(e);
      uint32_t w[8];
      entry_words(a.mbytes, gme, len, w);
      const uint32_t h = entry_hash(w, len);
      const uint32_t khi = (h & ~63u) | 0x80000000u | (uint32_t)len;
      const unsigned long long key = (unsigned long long)khi << 32 | gme;
      // linear probing; an empty slot is claimed by a CAS (one that loses
      // reads the slot again), a slot whose key matches a longer entry is
      // checked by its bytes.  The claims and the byte loads of the other
      // lanes are in flight together.
      uint32_t s = mix32(h ^ 0x5BD1E995u) & a.dt_mask;
      bool active = true, need = true;
      unsigned long long x = 0ull;
      for (int p = 0; p < kDedupProbes && active; ++p) {
        if (need) x = dt2[s].x;
        need = true;
        const bool empty = x == 0ull;
        const bool hit = (uint32_t)(x >> 32) == khi;
        unsigned long long old = 1ull;
        if (empty) old = atomicCAS(&a.dt[2 * (size_t)s], 0ull, key);
        uint32_t w2[8];
        if (hit) entry_words(a.mbytes, (uint32_t)x, len, w2);
        if (empty) {
          if (old == 0ull) {
            slot = s;  // this entry owns its bytes
            dt32[4 * (size_t)s + 2] = gme;
            ++claims;
            active = false;
          } else {
            x = old;  // taken meanwhile: look at the key that won
            need = false;
          }
        } else if (hit) {
          uint32_t d = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) d |= w[i] ^ w2[i];
          if (d == 0) {
            owner = false;
            slot = s;
            active = false;
          } else {
            s = (s + 1) & a.dt_mask;
          }
        } else {
          s = (s + 1) & a.dt_mask;
        }
      }
    }
    if (v) a.dref[c * kDrefCap + idx - kDrefBase] = owner ? kDrefOwner : slot;
    const bool ov = v && owner;
    const uint64_t o0 = __ballot(ov && b == 0), o1 = __ballot(ov && b == 1),
                   o2 = __ballot(ov && b == 2);
    if (ov) {
      const int at = b == 0 ? own0 + __popcll(o0 & below)
                            : (b == 1 ? own1 + __popcll(o1 & below) : own2 + __popcll(o2 & below));
      a.olist[c * kMissMax + kBucketBase[b] + at] = (uint64_t)e | ((uint64_t)slot << 32);
    }
    own0 += __popcll(o0);
    own1 += __popcll(o1);
    own2 += __popcll(o2);
  }
  claims = wave_sum(claims);
  if (lane == 0) {
    int32_t *mm = a.meta + kMetaInts * c;
    mm[kMetaOwners + 0] = own0;
    mm[kMetaOwners + 1] = own1;
    mm[kMetaOwners + 2] = own2;
    if (seeding && claims) atomicAdd(&a.dstat[0], (uint32_t)claims);
  }
}

// One wave per chunk, after the owners are merged: each entry that is not an
// owner takes its owner's token count and tokens from the slot; the chunk's
// count grows by theirs.
__global__ void __launch_bounds__(256) k_dupfill(EncodeArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave_id());
  if (c >= a.n_chunks) return;
  const int lane = lane_id();
  const int32_t *m = a.meta + kMetaInts * c;
  const int n0 = dedup_count(m, 0), n01 = n0 + dedup_count(m, 1);
  const int n = n01 + dedup_count(m, 2);
  int owners = 0;
#pragma unroll
  for (int b = kDedupFrom; b < 3; ++b) owners += m[kMetaOwners + b];
  if (owners == n) return;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 *dty = reinterpret_cast<const u32x2 *>(a.dt);
  int sum = 0;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int g = s0 + lane;
    int b;
    const int idx = lane_list_index(g, n0, n01, b);
    if (g < n) {
      const uint32_t r = a.dref[c * kDrefCap + idx - kDrefBase];
      const uint32_t e = a.miss[c * kMissMax + idx];
      if (r != kDrefOwner) {
        const u32x2 y = dty[2 * (size_t)r + 1];  // owner's g, token count
        a.cntk[c * kChunk + le_k(e)] = (uint8_t)y.y;
        a.pv[c * kChunk + le_k(e)] = -1 - (kPvDup + (int32_t)y.x);
        sum += (int)y.y;
      }
    }
  }
  sum = wave_sum(sum);
  if (lane == 0 && sum) a.tot[c] += sum;
}

// End (exclusive, global) of the pre-token that starts at gs and has no start
// in the window, scanning bytes from `from` on (one wave).
__device__ int64_t wave_global_end(const EncodeArgs &a, int64_t gs, int64_t from) {
  const int lane = lane_id();
  const int64_t d = wave_lower_bound(a.doc_off, a.n_docs + 1, gs + 1);
  int64_t limit = d <= a.n_docs ? a.doc_off[d] : a.n_bytes;
  limit = min(max(limit, gs + 1), a.n_bytes);
  const uint8_t *b = a.bytes;
  // from > gs + 1 always (the pre-token fills the window), so q - 1 > gs is
  // inside the document and is not a document start
  for (int64_t q0 = max(from, gs + 2); q0 < limit; q0 += 64 * 16) {
    // the lane's 16 positions and the two bytes before them, loaded together
    const int64_t p0 = q0 + 16 * (int64_t)lane;
    uint32_t v[18];
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      const int64_t q = p0 - 2 + j;
      v[j] = q < limit ? (uint32_t)b[q] : 0u;
    }
    int cand = kNoStart;
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      const int64_t q = p0 + j;
      const uint32_t c0 = byte_class(v[j + 2]), b1 = v[j + 1], c1 = byte_class(b1);
      const bool attach = c0 == kL && b1 == 0x20u && byte_class(v[j]) != kW;
      if (q < limit && c0 != c1 && !attach) cand = 16 * lane + j;
    }
    cand = wave_min(cand);
    if (cand != kNoStart) return q0 + cand;
  }
  return limit;
}

// ---- k_merge_long -------------------------------------------------------------

constexpr int kLdsLong = 2048;    // longest bucket-3 pre-token merged in LDS
constexpr int kProbeGroups = 8;   // groups of 64 positions whose rank probes go together

constexpr int kRPad = 8;          // sentinel ranks on each side of r (window radii up to 8)
constexpr int kFreshMax = 128;    // new symbols of a round listed for their probes (more: a scan)

struct LongShared {
  int32_t y[kLdsLong];                          // symbols
  int32_t rpad[kRPad + kLdsLong + kRPad];       // r(): rank of the pair (y[i], y[i + 1]);
                                                //   -1 = to be found
  uint32_t cand[kLdsLong / 32];                 // bit i: the pair is the lowest in its window
  uint16_t fresh[kFreshMax];                    // positions of a round's new symbols
  __device__ __forceinline__ int32_t *r() { return rpad + kRPad; }
};

// Bits of the pairs whose rank is the lowest within D positions on each side
// (D a compile-time radius up to kRPad): the ranks r[-kRPad .. -1] and
// r[n .. n + kRPad - 1] read as kRankInf, so no window needs a bounds test.
template <int D>
__device__ __forceinline__ void lowest_in_window(LongShared &L, const int32_t *r, int n) {
  static_assert(D >= 1 && D <= kRPad, "radius within the sentinels");
  const int lane = lane_id();
  for (int i0 = 0; i0 < n; i0 += MWG) {
    const int i = i0 + lane;
    bool c = false;
    if (i < n) {
      const int32_t x = r[i];
      int32_t w = x;
#pragma unroll
      for (int dj = 1; dj <= D; ++dj) w = min(w, min(r[i - dj], r[i + dj]));
      c = x < kRankInf && x == w;
    }
    const uint64_t bc = __ballot(c);
    if (lane == 0) {
      L.cand[i0 >> 5] = (uint32_t)bc;
      L.cand[(i0 >> 5) + 1] = (uint32_t)(bc >> 32);
    }
  }
}

// The rounds for one pre-token of n <= kLdsLong symbols (bytes on entry) in
// LDS, by one wave; returns the final count, the symbols left in y.
//  D > 0: each round merges every pair whose rank is the lowest among the
//    pairs within D positions on each side (window_radii on the host gives
//    why the rank-ordered rounds merge it the same way).  A run of one pair
//    (x, x) merges at even offsets from its first pair, and only if that
//    first pair is such a lowest pair: the run's start then cannot move
//    before its round.
//  D == 0: each round merges the lowest rank of the whole pre-token, every
//    occurrence left to right without overlap.
// Position i belongs to lane i % 64; scans run 64 positions at a time with
// a carry.  One wave does all the work, so LDS accesses stay in program
// order and the arrays are rewritten in place.
__device__ __noinline__ int lds_merge(LongShared &L, int n, int D, const RankTable &tab,
                         const int32_t *__restrict__ pair_rank) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1;
  int32_t *const R = L.r();
#pragma unroll 8
  for (int i = lane; i < n; i += MWG)
    R[i] = (i + 1 < n) ? pair_rank[(L.y[i] << 8) | L.y[i + 1]] : kRankInf;
  if (lane < kRPad) {
    R[-1 - lane] = kRankInf;
    R[n + lane] = kRankInf;
  }
  while (n > 1) {
    int32_t gmin = kRankInf;
    if (D == 0) {
      for (int i = lane; i < n; i += MWG) gmin = min(gmin, R[i]);
      gmin = wave_min(gmin);
      if (gmin == kRankInf) break;
    }
    // 1. the lowest pairs of their windows
    switch (D) {
      case 1: lowest_in_window<1>(L, R, n); break;
      case 2: lowest_in_window<2>(L, R, n); break;
      case 3: lowest_in_window<3>(L, R, n); break;
      case 4: lowest_in_window<4>(L, R, n); break;
      case 5: lowest_in_window<5>(L, R, n); break;
      case 6: lowest_in_window<6>(L, R, n); break;
      case 7: lowest_in_window<7>(L, R, n); break;
      case 8: lowest_in_window<8>(L, R, n); break;
      default:
        for (int i0 = 0; i0 < n; i0 += MWG) {
          const int i = i0 + lane;
          bool c = false;
          if (i < n) {
            const int32_t r = R[i];
            int32_t w = gmin;
            if (D > 0) {
              w = r;
              const int j1 = min(n - 1, i + D);
              for (int j = max(0, i - D); j <= j1; ++j) w = min(w, R[j]);
            }
            c = r < kRankInf && r == w;
          }
          const uint64_t bc = __ballot(c);
          if (lane == 0) {
            L.cand[i0 >> 5] = (uint32_t)bc;
            L.cand[(i0 >> 5) + 1] = (uint32_t)(bc >> 32);
          }
        }
    }
    // 2. merge flags (run starts by a running maximum) and compaction: a
    //    symbol whose left neighbour merged is consumed.  Two groups of 64
    //    positions per step, A then B: their scans and ballots do not wait on
    //    each other, only the carries from A into B do.  The next two
    //    groups' symbols, ranks and candidate bits are read before this
    //    step's writes (those land at or before this step's positions), so
    //    each step's reads overlap the one before.
    int run = 0;                // run start in force before this step
    bool run_c = false;         // its candidate bit
    bool prevm = false;         // the position before this step merged
    int32_t prevr = kRankInf;   // and its rank (its slot may already be rewritten)
    int out = 0;                // symbols kept so far
    int nnew = 0;               // new symbols so far
    bool any = false;
    int32_t nrA = lane < n ? R[lane] : kRankInf;
    int32_t nyA = lane < n ? L.y[lane] : 0;
    int32_t nrB = lane + MWG < n ? R[lane + MWG] : kRankInf;
    int32_t nyB = lane + MWG < n ? L.y[lane + MWG] : 0;
    uint64_t ncmA = ((uint64_t)L.cand[1] << 32) | L.cand[0];
    uint64_t ncmB = ((uint64_t)L.cand[3] << 32) | L.cand[2];
    for (int i0 = 0; i0 < n; i0 += 2 * MWG) {
      const int iA = i0 + lane, iB = iA + MWG;
      const bool inA = iA < n, inB = iB < n;
      const int32_t rA = nrA, yA = nyA, rB = nrB, yB = nyB;
      const uint64_t cmA = ncmA, cmB = ncmB;  // candidate bits of positions i0 .., i0 + 64 ..
      if (i0 + 2 * MWG < n) {
        const int jA = iA + 2 * MWG, jB = iB + 2 * MWG;
        nrA = jA < n ? R[jA] : kRankInf;
        nyA = jA < n ? L.y[jA] : 0;
        nrB = jB < n ? R[jB] : kRankInf;
        nyB = jB < n ? L.y[jB] : 0;
        const int w = (i0 >> 5) + 4;  // the word of position i0 + 128
        ncmA = ((uint64_t)L.cand[w + 1] << 32) | L.cand[w];
        ncmB = ((uint64_t)L.cand[w + 3] << 32) | L.cand[w + 2];
      }
      const int32_t rAl = wave_shift_up1(rA, prevr);
      const int32_t rBl = wave_shift_up1(rB, lane_value(rA, 63));
      const bool bA = inA && (iA == 0 || rAl != rA);
      const bool bB = inB && rBl != rB;
      const bool cA = inA && ((cmA >> lane) & 1u), cB = inB && ((cmB >> lane) & 1u);
      // where every position starts a run (no pair repeats its neighbour's
      // rank) each is its own run start
      int stA = iA, stB = iB;
      bool csA = cA, csB = cB;
      if (__ballot((inA && !bA) || (inB && !bB)) != 0) {
        const int sA = wave_incl_max(bA ? iA : -1), sB = wave_incl_max(bB ? iB : -1);
        stA = max(sA, run);
        const int runA = lane_value(stA, 63);
        const bool rcA = runA >= i0 ? ((cmA >> (runA - i0)) & 1u) : run_c;
        stB = max(sB, runA);
        csA = stA >= i0 ? ((cmA >> (stA - i0)) & 1u) : run_c;
        csB = stB >= i0 + MWG ? ((cmB >> (stB - i0 - MWG)) & 1u) : rcA;
      }
      const bool mA = cA && csA && ((iA - stA) & 1) == 0;
      const bool mB = cB && csB && ((iB - stB) & 1) == 0;
      const uint64_t bmA = __ballot(mA), bmB = __ballot(mB);
      const bool consA = lane == 0 ? prevm : ((bmA >> (lane - 1)) & 1u);
      const bool consB = lane == 0 ? ((bmA >> 63) & 1u) : ((bmB >> (lane - 1)) & 1u);
      const bool kA = inA && !consA, kB = inB && !consB;
      const uint64_t bkA = __ballot(kA), bkB = __ballot(kB);
      const int oA = out + __popcll(bkA & below);
      const int oB = out + __popcll(bkA) + __popcll(bkB & below);
      if (kA) {
        L.y[oA] = mA ? 256 + rA : yA;
        R[oA] = mA ? -1 : rA;
      }
      if (kB) {
        L.y[oB] = mB ? 256 + rB : yB;
        R[oB] = mB ? -1 : rB;
      }
      // (a merging position is never consumed: its left neighbour would
      // belong to the same run at an odd offset)
      if (mA) {
        const int q = nnew + __popcll(bmA & below);
        if (q < kFreshMax) L.fresh[q] = (uint16_t)oA;
      }
      if (mB) {
        const int q = nnew + __popcll(bmA) + __popcll(bmB & below);
        if (q < kFreshMax) L.fresh[q] = (uint16_t)oB;
      }
      nnew += __popcll(bmA) + __popcll(bmB);
      any |= (bmA | bmB) != 0;
      out += __popcll(bkA) + __popcll(bkB);
      prevm = (bmB >> 63) & 1u;
      prevr = lane_value(rB, 63);
      const int nrun = lane_value(stB, 63);
      run_c = nrun >= i0 + MWG ? ((cmB >> (nrun - i0 - MWG)) & 1u)
            : nrun >= i0       ? ((cmA >> (nrun - i0)) & 1u)
                               : run_c;
      run = nrun;
    }
    if (!any) break;
    n = out;
    if (lane < kRPad) R[n + lane] = kRankInf;
    // 3. ranks of the pairs that touch a new symbol.  Listed new symbols: a
    //    lane probes both pairs of one, (left neighbour, new) unless the left
    //    neighbour is new too (its own right pair is that pair) and (new,
    //    right neighbour), the two probes in flight together.
    if (nnew <= kFreshMax) {
      for (int k0 = 0; k0 < nnew; k0 += MWG) {
        const int k = k0 + lane;
        const bool act = k < nnew;
        const int o = act ? (int)L.fresh[k] : 0;
        const bool hl = act && o > 0 && R[o - 1] != -1;
        const bool hr = act && o + 1 < n;
        const uint32_t yo = (uint32_t)L.y[o];
        const uint32_t yl = hl ? (uint32_t)L.y[o - 1] : 0u, yr = hr ? (uint32_t)L.y[o + 1] : 0u;
        const uint64_t kl = pair_key(yl, yo), kr = pair_key(yo, yr);
        const uint32_t xl = pair_mix(yl, yo, tab.seed), xr = pair_mix(yo, yr, tab.seed);
        u64x2 bl = u64x2{kEmptySlot, kEmptySlot}, br = bl;
        if (hl) bl = tab.b[pair_bucket0(xl, tab.mask)];
        if (hr) br = tab.b[pair_bucket0(xr, tab.mask)];
        int32_t rl = hl ? bucket_rank(bl, kl) : kRankInf;
        int32_t rr = hr ? bucket_rank(br, kr) : kRankInf;
        const bool l2 = hl && rl == kRankInf && bucket_flag(bl);
        const bool r2 = hr && rr == kRankInf && bucket_flag(br);
        if (l2) bl = tab.b[pair_bucket1(xl, tab.mask)];
        if (r2) br = tab.b[pair_bucket1(xr, tab.mask)];
        if (l2) rl = bucket_rank(bl, kl);
        if (r2) rr = bucket_rank(br, kr);
        if (hl) R[o - 1] = rl;
        if (act) R[o] = rr;
      }
      continue;
    }
    //    More new symbols: every position scanned, the probes of kProbeGroups
    //    groups of 64 positions issued together.
    for (int i0 = 0; i0 < n; i0 += MWG * kProbeGroups) {
      int32_t nv[kProbeGroups];
      uint32_t xs[kProbeGroups];
      uint64_t key[kProbeGroups];
      u64x2 bk[kProbeGroups];
      uint32_t need = 0;
#pragma unroll
      for (int g = 0; g < kProbeGroups; ++g) {
        const int i = i0 + MWG * g + lane;
        nv[g] = kRankInf;
        key[g] = 0;
        xs[g] = 0;
        bk[g] = u64x2{kEmptySlot, kEmptySlot};
        if (i + 1 < n) {
          const int32_t r = R[i];
          nv[g] = r;
          if (r == -1 || R[i + 1] == -1) {
            need |= 1u << g;
            const uint32_t l = (uint32_t)L.y[i], rt = (uint32_t)L.y[i + 1];
            key[g] = pair_key(l, rt);
            xs[g] = pair_mix(l, rt, tab.seed);
            bk[g] = tab.b[pair_bucket0(xs[g], tab.mask)];
          }
        }
      }
      uint32_t need2 = 0;
#pragma unroll
      for (int g = 0; g < kProbeGroups; ++g) {
        if ((need >> g) & 1u) {
          nv[g] = bucket_rank(bk[g], key[g]);
          if (nv[g] == kRankInf && bucket_flag(bk[g])) need2 |= 1u << g;
        }
      }
      if (need2) {
#pragma unroll
        for (int g = 0; g < kProbeGroups; ++g)
          if ((need2 >> g) & 1u) bk[g] = tab.b[pair_bucket1(xs[g], tab.mask)];
#pragma unroll
        for (int g = 0; g < kProbeGroups; ++g)
          if ((need2 >> g) & 1u) nv[g] = bucket_rank(bk[g], key[g]);
      }
#pragma unroll
      for (int g = 0; g < kProbeGroups; ++g) {
        const int i = i0 + MWG * g + lane;
        if (i < n) R[i] = nv[g];
      }
    }
  }
  return n;
}

// ---- segmented rounds -----------------------------------------------------
// The rounds of lds_merge for a window radius 1 <= D <= kRPad, with each
// lane owning a contiguous segment of the symbols instead of every 64th
// position.  A lane walks its own segment one symbol after another, so the
// run rule and the compaction need no scan over the wave; only the segment
// edges are exchanged, once per round:
//  - the window of a symbol near an edge reads the neighbouring lane's
//    ranks (every segment holds at least D symbols, so the window never
//    reaches two lanes away);
//  - a run of one pair that enters a segment from the left takes its start
//    (and that start's window bit) from the nearest lane on the left with a
//    run start, by a running maximum over the lanes;
//  - a merge of a segment's last pair consumes the next segment's first
//    symbol.
// Segments compact in place; when one falls below D symbols, the symbols are
// spread again through the entry's position-indexed scratch (gy, gr).
// Lane l's segment sits at l * kSegStride in LDS (an odd stride: the lanes'
// k-th symbols fall in different banks).

constexpr int kSegCap = 32;              // symbols a lane holds
constexpr int kSegStride = kSegCap + 1;  // LDS words from one lane's segment to the next
// fewest symbols per lane when spread (if n allows): at least the largest
// radius, so that a spread leaves every segment long enough for its windows
constexpr int kSegShare = 8;
static_assert(kSegShare >= kRPad, "a spread segment holds a window's radius");
constexpr int kSegFrom = 256;            // entries this long or longer take the segmented rounds

__device__ __forceinline__ int seg_lanes(int n) { return min(MWG, max(1, n / kSegShare)); }

// Lane l's share of n symbols over Ln lanes: [n l / Ln, n (l + 1) / Ln).
__device__ __forceinline__ void seg_share(int n, int Ln, int lane, int &lo, int &len) {
  lo = lane < Ln ? n * lane / Ln : n;
  len = (lane < Ln ? n * (lane + 1) / Ln : n) - lo;
}

constexpr int kSegBatch = 8;  // symbols a lane loads together
// probes in flight per lane: with 4, the kernel fits in 168 registers (3
// waves per SIMD; LDS then allows 9 per CU); 8 took 243 (2 waves per SIMD)
constexpr int kSegProbe = 4;

// The positions of m's lowest kSegProbe set bits, lowest first (-1 where m
// has fewer); m loses them.
__device__ __forceinline__ void take_bits(uint32_t &m, int (&k)[kSegProbe]) {
#pragma unroll
  for (int g = 0; g < kSegProbe; ++g) {
    k[g] = m ? __builtin_ctz(m) : -1;
    m &= m - 1;
  }
}

template <int D>
__device__ int seg_merge(LongShared &LS, const uint8_t *__restrict__ bytes, int n,
                         const RankTable &tab, const int32_t *__restrict__ pair_rank,
                         int32_t *__restrict__ gy, int32_t *__restrict__ gr) {
  static_assert(D >= 1 && D <= kRPad, "radius");
  static_assert(sizeof(LongShared) >= 2 * MWG * kSegStride * sizeof(int32_t), "segments fit");
  static_assert(MWG * kSegCap >= kLdsLong && MWG * kSegStride >= kLdsLong, "every entry fits");
  static_assert(kSegCap % kSegBatch == 0, "whole batches");
  int32_t *const Y = reinterpret_cast<int32_t *>(&LS);
  int32_t *const R = Y + MWG * kSegStride;
  const int lane = lane_id();
  const int base = lane * kSegStride;
  const int baseL = max(base - kSegStride, 0), baseR = min(base + kSegStride, (MWG - 1) * kSegStride);
  int Ln = seg_lanes(n);
  int lo, len;
  seg_share(n, Ln, lane, lo, len);
  // the bytes in position order (in R, as staging), then each lane's share
  // into its segment, then the pairs' ranks by the byte-pair table
#pragma unroll 8
  for (int i = lane; i < n; i += MWG) R[i] = bytes[i];
  __syncthreads();
  const int32_t nb = lo + len < n ? R[lo + len] : 0;  // the byte after the segment
  for (int c = 0; c < len; c += kSegBatch) {
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (c + j < len) Y[base + c + j] = R[lo + c + j];
  }
  __syncthreads();
  for (int c = 0; c < len; c += kSegBatch) {
    int32_t rk[kSegBatch];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j) {
      const int k = c + j;
      // (bytes here; masked so that a slot past the segment indexes the table too)
      const uint32_t b0 = (uint32_t)Y[base + min(k, kSegCap - 1)] & 0xFFu;
      const uint32_t b1 = (k + 1 < len ? (uint32_t)Y[base + min(k + 1, kSegCap - 1)] : (uint32_t)nb) & 0xFFu;
      rk[j] = pair_rank[(b0 << 8) | b1];
    }
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j) {
      const int k = c + j;
      if (k < len) R[base + k] = lo + k + 1 < n ? rk[j] : kRankInf;
    }
  }
  __syncthreads();
  while (true) {
    const int incl = wave_incl_sum(len);
    const int P = incl - len;  // global index of the segment's first symbol
    const int lenL = wave_shift_up1(len, 0);
    const int lenR = wave_shift_down1(len, 0);
    // rank of pair k of this segment, k >= -D (before the round): an index
    // always inside the arrays, and whether the value counts (kRankInf past
    // either end of the symbols)
    auto rank_at = [&](int k) -> int32_t {
      int idx;
      bool ok;
      if (k < 0) {
        idx = baseL + max(lenL + k, 0);
        ok = lane > 0;
      } else if (k < len) {
        idx = base + k;
        ok = true;
      } else {
        idx = baseR + min(k - len, kSegCap - 1);
        ok = k - len < lenR;
      }
      const int32_t v = R[idx];
      return ok ? v : kRankInf;
    };
    // 1. window bits cm (bit k: pair k is the lowest within D on each side),
    //    and the last run start kls in the segment (-1: none); kSegBatch
    //    pairs at a time, their windows' ranks loaded together
    const int32_t left1 = rank_at(-1);
    const bool cont0 = lane > 0 && len > 0 && rank_at(0) == left1;  // a run enters from the left
    uint32_t cm = 0;
    int kls = -1;
    // w[q]: rank of pair c - D + q; the first 2D carried over from the
    // batch before
    int32_t w[kSegBatch + 2 * D];
#pragma unroll
    for (int q = 0; q < 2 * D; ++q) w[q] = rank_at(q - D);
    for (int c = 0; c < len; c += kSegBatch) {
#pragma unroll
      for (int j = 0; j < kSegBatch; ++j) w[2 * D + j] = rank_at(c + D + j);
#pragma unroll
      for (int j = 0; j < kSegBatch; ++j) {
        const int k = c + j;
        const int32_t x = w[D + j];
        int32_t mn = x;
#pragma unroll
        for (int q = 0; q <= 2 * D; ++q) mn = min(mn, w[j + q]);
        if (k < len) {
          if (x < kRankInf && x == mn) cm |= 1u << k;
          if (k == 0 ? !cont0 : x != w[D + j - 1]) kls = k;
        }
      }
#pragma unroll
      for (int q = 0; q < 2 * D; ++q) w[q] = w[q + kSegBatch];
    }
    // 2. the run start in force at the segment's first symbol, from the
    //    nearest lane on the left with a start: (global index << 1) | window bit
    const int key = kls >= 0 ? ((P + kls) << 1) | (int)((cm >> kls) & 1u) : -1;
    const int carried = wave_incl_max(wave_shift_up1(key, -1));
    int st_last = carried >> 1, cst_last = carried & 1;
    if (kls >= 0) st_last = P + kls, cst_last = (int)((cm >> kls) & 1u);
    const bool m_last = len > 0 && ((cm >> (len - 1)) & 1u) && cst_last &&
                        ((P + len - 1 - st_last) & 1) == 0;
    const bool prevm = wave_shift_up1((int32_t)m_last, 0) != 0;  // my first symbol is consumed
    // 3. merge flags and compaction in place, kSegBatch symbols loaded
    //    together (the writes land at or before them); need: the pairs whose
    //    rank the new symbols change (a new symbol's own pair and the one
    //    before it)
    int st = carried >> 1, cst = carried & 1;
    bool pm = prevm, anym = false, first_new = false;
    int32_t pr = left1;
    int out = 0;
    uint32_t need = 0;
    for (int c = 0; c < len; c += kSegBatch) {
      int32_t xr[kSegBatch], xy[kSegBatch];
#pragma unroll
      for (int j = 0; j < kSegBatch; ++j) {
        xr[j] = R[base + c + j];
        xy[j] = Y[base + c + j];
      }
#pragma unroll
      for (int j = 0; j < kSegBatch; ++j) {
        const int k = c + j;
        if (k < len) {
          const int32_t x = xr[j];
          const int cb = (int)((cm >> k) & 1u);
          if (k == 0 ? !cont0 : x != pr) st = P + k, cst = cb;
          const bool m = cb && cst && ((P + k - st) & 1) == 0;
          if (!pm) {
            Y[base + out] = m ? 256 + x : xy[j];
            R[base + out] = m ? -1 : x;
            if (m) {
              need |= 1u << out;
              if (out > 0) need |= 1u << (out - 1);
              else first_new = true;
            }
            ++out;
          }
          anym |= m;
          pm = m;
          pr = x;
        }
      }
    }
    if (__ballot(anym) == 0) break;
    // the pair before a segment's new first symbol is the last of the lane
    // on the left
    if (wave_shift_down1((int32_t)first_new, 0) != 0 && out > 0) need |= 1u << (out - 1);
    len = out;
    n = lane_value(wave_incl_sum(len), MWG - 1);
    __syncthreads();
    // 4. spread again when a segment is too short for the windows; the new
    //    symbols (rank -1) then mark the pairs to probe
    if (__ballot(lane < Ln && len < (Ln > 1 ? D : 1)) != 0) {
      const int Q = wave_incl_sum(len) - len;
      for (int k = 0; k < len; ++k) {
        gy[Q + k] = Y[base + k];
        gr[Q + k] = R[base + k];
      }
      __syncthreads();
      Ln = seg_lanes(n);
      seg_share(n, Ln, lane, lo, len);
      for (int k = 0; k < len; ++k) {
        Y[base + k] = gy[lo + k];
        R[base + k] = gr[lo + k];
      }
      __syncthreads();
      need = 0;
      const int32_t r0n = lane + 1 < Ln ? R[baseR] : kRankInf;
      for (int k = 0; k < len; ++k) {
        const int32_t rn = k + 1 < len ? R[base + k + 1] : r0n;
        if (R[base + k] == -1 || rn == -1) need |= 1u << k;
      }
      __syncthreads();
    }
    // 5. ranks of the marked pairs, kSegProbe probes in flight per lane; the
    //    next segment's first symbol is read before any lane rewrites it
    //    (the barrier keeps the read ahead of the writes)
    const int32_t ny0 = Y[baseR];
    const bool glast = lane == Ln - 1;
    if (glast && len > 0 && ((need >> (len - 1)) & 1u)) {
      need &= ~(1u << (len - 1));
      R[base + len - 1] = kRankInf;  // the last pair has no right symbol
    }
    __syncthreads();
    while (__ballot(need != 0) != 0) {
      int ks[kSegProbe];
      take_bits(need, ks);
      uint32_t xs[kSegProbe];
      uint64_t kk[kSegProbe];
      u64x2 bk[kSegProbe];
      int32_t nv[kSegProbe];
#pragma unroll
      for (int g = 0; g < kSegProbe; ++g) {
        const int k = max(ks[g], 0);
        const uint32_t l = (uint32_t)Y[base + k];
        const uint32_t rt = k + 1 < len ? (uint32_t)Y[base + min(k + 1, kSegCap - 1)] : (uint32_t)ny0;
        kk[g] = pair_key(l, rt);
        xs[g] = pair_mix(l, rt, tab.seed);
      }
#pragma unroll
      for (int g = 0; g < kSegProbe; ++g)
        bk[g] = ks[g] >= 0 ? tab.b[pair_bucket0(xs[g], tab.mask)] : u64x2{kEmptySlot, kEmptySlot};
      uint32_t need2 = 0;
#pragma unroll
      for (int g = 0; g < kSegProbe; ++g) {
        nv[g] = bucket_rank(bk[g], kk[g]);
        if (ks[g] >= 0 && nv[g] == kRankInf && bucket_flag(bk[g])) need2 |= 1u << g;
      }
      if (need2) {
#pragma unroll
        for (int g = 0; g < kSegProbe; ++g)
          if ((need2 >> g) & 1u) bk[g] = tab.b[pair_bucket1(xs[g], tab.mask)];
#pragma unroll
        for (int g = 0; g < kSegProbe; ++g)
          if ((need2 >> g) & 1u) nv[g] = bucket_rank(bk[g], kk[g]);
      }
#pragma unroll
      for (int g = 0; g < kSegProbe; ++g)
        if (ks[g] >= 0) R[base + ks[g]] = nv[g];
    }
    __syncthreads();
  }
  // the symbols in order, at the entry's positions: gathered in position
  // order in R's memory, then stored by consecutive lanes
  const int P = wave_incl_sum(len) - len;
  for (int k = 0; k < len; ++k) R[P + k] = Y[base + k];
  __syncthreads();
#pragma unroll 8
  for (int i = lane; i < n; i += MWG) gy[i] = R[i];
  return n;
}

__device__ int seg_merge_d(LongShared &LS, const uint8_t *bytes, int n, int D, const RankTable &tab,
                           const int32_t *pair_rank, int32_t *gy, int32_t *gr) {
  switch (D) {
    case 1: return seg_merge<1>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 2: return seg_merge<2>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 3: return seg_merge<3>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 4: return seg_merge<4>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 5: return seg_merge<5>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 6: return seg_merge<6>(LS, bytes, n, tab, pair_rank, gy, gr);
    case 7: return seg_merge<7>(LS, bytes, n, tab, pair_rank, gy, gr);
    default: return seg_merge<8>(LS, bytes, n, tab, pair_rank, gy, gr);
  }
}

// ---- run-length rounds ----------------------------------------------------
// A pre-token made of few runs of one repeated byte (a letter repeated
// hundreds of times, say) is merged on its runs, (symbol, count), instead of
// symbol by symbol.  Each round is an exact R4 round: the lowest rank r of
// the pairs present, all its occurrences left to right without overlap,
// taken on the sequence as it was at the round's start.  The pair of rank r
// is one pair (A, B):
//  - A == B occurs only inside runs of A: a run of k becomes (Z, k / 2) and,
//    for odd k, one A after it;
//  - A != B occurs only where a run of A meets a run of B (no two such
//    occurrences overlap): each side gives up one symbol to a Z between them.
// Z = 256 + r.  Equal neighbouring runs are then joined.  The run list lives
// in LongShared's arrays; a round that would leave more than kRleMax runs
// gives up (false), and the entry is merged symbol by symbol from its bytes.

constexpr int kRleMax = 512;

struct RleView {
  int32_t *sym, *cnt;    // [kRleMax] the runs
  int32_t *rin, *rbd;    // [kRleMax] rank of (sym, sym) inside a run of 2 or more, and of
                         //   (sym[i], sym[i + 1]); kRankInf where none
  int32_t *esym, *ecnt;  // [2 kRleMax] the runs a round emits, before joining
};

__device__ __forceinline__ RleView rle_view(LongShared &L) {
  static_assert(2 * kRleMax + 2 * kRleMax <= kLdsLong, "run arrays fit LongShared");
  return RleView{L.y, L.y + kRleMax, L.r(), L.r() + kRleMax, L.y + 2 * kRleMax, L.r() + 2 * kRleMax};
}

// Wave-wide exclusive prefix of v over the lanes, plus a carry; *all gets
// the wave's sum.
__device__ __forceinline__ int wave_excl(int v, int carry, int *all) {
  const int inc = wave_incl_sum(v);
  *all = lane_value(inc, 63);
  return carry + inc - v;
}

__device__ void rle_ranks(const RleView &V, int R, const RankTable &tab) {
  for (int i = lane_id(); i < R; i += 64) {
    const int32_t x = V.sym[i];
    V.rin[i] = V.cnt[i] >= 2 ? rank_of(tab, (uint32_t)x, (uint32_t)x) : kRankInf;
    V.rbd[i] = i + 1 < R ? rank_of(tab, (uint32_t)x, (uint32_t)V.sym[i + 1]) : kRankInf;
  }
}

// The runs of bytes[0, n) (global), if there are at most kRleMax of them and
// at least 8 bytes per run on average; returns their number, or -1.
// The bytes come 16 per lane per step (1 KiB per wave, all loads of a step in
// flight together); a run starts where a byte differs from the one before.
__device__ __noinline__ int rle_build(const RleView &V, const uint8_t *bytes, int64_t n) {
  const int lane = lane_id();
  int R = 0;
  int32_t prev = -1;
  for (int64_t i0 = 0; i0 < n; i0 += 64 * 16) {
    const int64_t p0 = i0 + 16 * (int64_t)lane;
    int32_t b[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) b[j] = p0 + j < n ? (int32_t)bytes[p0 + j] : -2;
    const int32_t left = wave_shift_up1(b[15], prev);  // the byte before this lane's first
    uint32_t hm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (p0 + j < n && b[j] != (j ? b[j - 1] : left)) hm |= 1u << j;
    // the 16 bytes packed (a head's byte is taken by a shift, not by a
    // register index)
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)(b[4 * q] & 0xFF) | ((uint32_t)(b[4 * q + 1] & 0xFF) << 8) |
             ((uint32_t)(b[4 * q + 2] & 0xFF) << 16) | ((uint32_t)(b[4 * q + 3] & 0xFF) << 24);
    int all;
    int k = wave_excl(__popc(hm), R, &all);
    for (uint32_t m = hm; m; m &= m - 1, ++k) {
      const int j = __ffs(m) - 1;
      const uint32_t wq = j < 8 ? (j < 4 ? w[0] : w[1]) : (j < 12 ? w[2] : w[3]);
      if (k < kRleMax) {
        V.sym[k] = (int32_t)((wq >> (8 * (j & 3))) & 0xFFu);
        V.cnt[k] = (int32_t)(p0 + j);  // start for now
      }
    }
    R += all;
    prev = lane_value(b[15], 63);
    if (R > kRleMax || (int64_t)R * 8 > n) return -1;  // R only grows
  }
  for (int k = lane; k < R; k += 64)
    V.cnt[k] = (int32_t)((k + 1 < R ? (int64_t)V.cnt[k + 1] : n) - V.cnt[k]);
  return R;
}

// Rounds on the R runs in V until no pair has a rank; returns the final
// number of runs, or -1 if a round would leave more than kRleMax.
__device__ __noinline__ int rle_merge(const RleView &V, int R, const RankTable &tab) {
  const int lane = lane_id();
  rle_ranks(V, R, tab);
  for (;;) {
    // the lowest rank, and whether it is a pair of equal symbols
    int32_t r = kRankInf;
    for (int i = lane; i < R; i += 64) r = min(r, min(V.rin[i], V.rbd[i]));
    r = wave_min(r);
    if (r == kRankInf) return R;
    int32_t A = -1, B = -1;
    for (int i0 = 0; i0 < R && A < 0; i0 += 64) {
      const int i = i0 + lane;
      const bool in = i < R && V.rin[i] == r, bd = i < R && V.rbd[i] == r;
      const uint64_t m = __ballot(in || bd);
      if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        const int32_t a_l = in ? V.sym[i] : (bd ? V.sym[i] : -1);
        const int32_t b_l = in ? V.sym[i] : (bd ? V.sym[i + 1] : -1);
        A = lane_value(a_l, src);
        B = lane_value(b_l, src);
      }
    }
    const int32_t Z = 256 + r;
    // emit: every run gives at most two
    int E = 0;
    for (int i0 = 0; i0 < R; i0 += 64) {
      const int i = i0 + lane;
      int32_t s0 = -1, c0 = 0, s1 = -1, c1 = 0;
      if (i < R) {
        const int32_t x = V.sym[i], k = V.cnt[i];
        if (A == B) {
          const bool m = x == A && k >= 2;
          s0 = m ? Z : x;
          c0 = m ? k / 2 : k;
          if (m && (k & 1)) {
            s1 = A;
            c1 = 1;
          }
        } else {
          const int dl = (i > 0 && V.sym[i - 1] == A && x == B) ? 1 : 0;
          const int dr = (i + 1 < R && x == A && V.sym[i + 1] == B) ? 1 : 0;
          if (k - dl - dr > 0) {
            s0 = x;
            c0 = k - dl - dr;
          }
          if (dr) {
            s1 = Z;
            c1 = 1;
          }
        }
      }
      const int ne = (s0 >= 0) + (s1 >= 0);
      int all;
      int o = wave_excl(ne, E, &all);
      if (s0 >= 0) {
        V.esym[o] = s0;
        V.ecnt[o] = c0;
        ++o;
      }
      if (s1 >= 0) {
        V.esym[o] = s1;
        V.ecnt[o] = c1;
      }
      E += all;
    }
    // join equal neighbours: heads take their symbol and the count before
    // them; a head's count is the next head's minus its own
    int Rn = 0, before = 0;
    for (int j0 = 0; j0 < E; j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < E;
      const int32_t x = in ? V.esym[j] : -1;
      const int32_t k = in ? V.ecnt[j] : 0;
      const bool head = in && (j == 0 || V.esym[j - 1] != x);
      int all_h, all_c;
      const int h = wave_excl(head ? 1 : 0, Rn, &all_h);
      const int p = wave_excl(k, before, &all_c);
      if (head && h < kRleMax) {
        V.sym[h] = x;
        V.cnt[h] = p;
      }
      Rn += all_h;
      before += all_c;
    }
    if (Rn > kRleMax) return -1;
    for (int h = lane; h < Rn; h += 64) {
      // groups run in order and every lane reads before it writes: cnt[h + 1]
      // still holds a start here
      const int32_t next = h + 1 < Rn ? V.cnt[h + 1] : before;
      V.cnt[h] = next - V.cnt[h];
    }
    R = Rn;
    rle_ranks(V, R, tab);
  }
}

// The R runs in V written out as symbols to out[0 ..); returns their number.
__device__ __noinline__ int64_t rle_expand(const RleView &V, int R, int32_t *out) {
  int64_t p = 0;
  for (int k = 0; k < R; ++k) {
    const int32_t x = V.sym[k], n = V.cnt[k];
    for (int q = lane_id(); q < n; q += 64) out[p + q] = x;
    p += n;
  }
  return p;
}

// The window radius of the entry at gs if the segmented rounds take it
// (1 .. kRPad), else 0.  The class is the first byte's, or the letter's
// after a leading space.
__device__ __forceinline__ int seg_radius(const EncodeArgs &a, int64_t gs) {
  uint32_t b = a.bytes[gs];
  if (b == 0x20u) b = a.bytes[gs + 1];
  const int D = a.win_d[byte_class(b)];
  return D >= 1 && D <= kRPad ? D : 0;
}

struct LongGroupShared {
  MergeShared g;
  LongShared L;
};

// Bucket 3 of the same groups: one wave per entry, in turn (each merge path
// a function of its own, so that each is given its own registers and the
// kernel's stay within 3 waves per SIMD).  An entry made
// of few runs of one byte is merged on its runs; otherwise one of at most
// kLdsLong bytes is merged in LDS (lds_merge) and a longer one in place in
// the position-indexed gsym / grank (wg_merge), both with the window radius
// of its class.  The tokens end in gsym at the entry's position; adds the
// token counts to tot.
__global__ void __launch_bounds__(MWG) k_merge_long(EncodeArgs a) {
  __shared__ LongGroupShared s;
  const int64_t cg = (int64_t)blockIdx.x * kGroup;
  const int nf = (int)min<int64_t>(kGroup, a.n_chunks - cg);
  load_group(a, s.g, cg, nf);
  int any = 0;
  for (int f = 0; f < nf; ++f) any += s.g.meta[f][kMetaBucket + 3];
  if (any == 0) return;
  const int lane = threadIdx.x;
  const RankTable t{reinterpret_cast<const u64x2 *>(a.table), a.table_mask, a.table_seed};
  for (int f = 0; f < nf; ++f) {
    const int n3 = s.g.meta[f][kMetaBucket + 3];
    const int base = kBucketBase[3];
    const int64_t c = cg + f, c0 = c * kChunk;
    for (int q = 0; q < n3; ++q) {
      const uint32_t e = a.miss[c * kMissMax + base + q];
      const int64_t gs = c0 + me_start(e);
      const int64_t ge = me_over(e) ? wave_global_end(a, gs, c0 + WIN) : gs + me_len(e);
      const int64_t len = ge - gs;
      int64_t nt = -1;
      // a first look at 64 bytes: more than 8 runs there rules out the
      // run-length path for an entry that the LDS paths take
      const int32_t hb = lane < len ? (int32_t)a.bytes[gs + lane] : -1;
      const bool many = __popcll(__ballot(lane < len && hb != wave_shift_up1(hb, -1))) > 8;
      if (!(many && len <= kLdsLong)) {
        // few long runs of one byte: merged on the runs
        const RleView V = rle_view(s.L);
        const int R = rle_build(V, a.bytes + gs, len);
        const int Rf = R > 0 ? rle_merge(V, R, t) : -1;
        if (Rf > 0) nt = rle_expand(V, Rf, a.gsym + gs);
      }
      if (nt >= 0) {
        // done
      } else if (len >= kSegFrom && len <= kLdsLong && seg_radius(a, gs)) {
        nt = seg_merge_d(s.L, a.bytes + gs, (int)len, seg_radius(a, gs), t, a.pair_rank,
                         a.gsym + gs, a.grank + gs);
      } else if (len <= kLdsLong) {
#pragma unroll 8
        for (int i = lane; i < len; i += MWG) s.L.y[i] = a.bytes[gs + i];
        __syncthreads();
        // the pre-token's class: its first byte, or the letter after a leading space
        uint32_t b = (uint32_t)s.L.y[0];
        if (b == 0x20u && len > 1) b = (uint32_t)s.L.y[1];
        nt = lds_merge(s.L, (int)len, a.win_d[byte_class(b)], t, a.pair_rank);
        for (int i = lane; i < nt; i += MWG) a.gsym[gs + i] = s.L.y[i];
      } else {
        for (int64_t p = gs + lane; p < ge; p += MWG) a.gsym[p] = a.bytes[p];
        __syncthreads();
        uint32_t b = a.bytes[gs];
        if (b == 0x20u) b = a.bytes[gs + 1];  // (len > kLdsLong)
        nt = wg_merge(a.gsym + gs, a.grank + gs, len, a.win_d[byte_class(b)], t, a.pair_rank);
      }
      if (lane == 0) {
        a.mt[c * kMaxLong + q] = (int32_t)nt;
        s.g.tok[f] += (int32_t)nt;
      }
      __syncthreads();
    }
  }
  if (lane < nf && s.g.tok[lane] != 0) a.tot[cg + lane] += s.g.tok[lane];
}

// ---- k_offsets ---------------------------------------------------------------

// The first level of the offset scan (block_offsets): blocks of kScanBlock
// chunks.
__global__ void __launch_bounds__(kScanBlock) k_offsets(EncodeArgs a) {
  block_offsets(a.tot, a.off, a.bsum, a.n_chunks);
}

// Exclusive prefix of the blocks' counts, and the status word from their
// status bits (one workgroup).  A chunk's offset is off[c] + boff[c / kScanBlock].
__global__ void __launch_bounds__(OWG) k_bscan(EncodeArgs a) {
  __shared__ int64_t red64[OWG / 64];
  chunk_offsets<OWG>(a.bsum, a.boff, (a.n_chunks + kScanBlock - 1) / kScanBlock, a.status, red64);
}

// ---- k_emit -------------------------------------------------------------------

constexpr int EWG = 256;                 // k_emit threads per chunk
constexpr int kOutCap = kChunk + kHalo;  // chunk-relative token positions staged in LDS
constexpr int kEmitPasses = 4;           // passes of EWG pre-tokens per round

constexpr int kDocLds = 512;             // document starts of a chunk staged in LDS (with reserved IDs)

template <bool SP>
struct EmitShared {
  int32_t out[kOutCap + 1];              // the chunk's symbols at positions below kOutCap;
                                         // stores that place nothing go to out[kOutCap]
  int32_t wtot[kEmitPasses][EWG / 64];   // token counts per pass and wave
  int64_t lw[kMaxLong];                  // wave-merged entries: position, source, count
  int64_t lsrc[kMaxLong];
  int64_t lnt[kMaxLong];
  int32_t n_long;
  int32_t dpos[SP ? kDocLds : 1];        // first position of each document that starts here
};

// Tokens of the lane-merged pre-token with pv value -1 - u: in the chunk's
// own res region, or (u >= kPvDup) in the owner's of the same bytes.
__device__ __forceinline__ const int32_t *entry_res(const EncodeArgs &a, const int32_t *res,
                                                    int u) {
  return u >= kPvDup ? a.res + 4 * (size_t)(uint32_t)(u - kPvDup) : res + ((u & 0xFFF) << 2);
}

// Writes a chunk's IDs at its offset, and the offsets of the documents that
// start in it.  Pre-token k belongs to thread k % EWG; rounds of kEmitPasses
// passes load every pv value of the round, then the token counts and the first
// four tokens of the merge-loop entries, scan the counts and place the
// symbols in LDS; the workgroup then writes the chunk's positions in order.
// A position at or past kOutCap (possible only after a long pre-token that
// runs past the window) is written directly.
//
// SP: reserved IDs around each document ("Characters, bytes and subwords",
// section "Special tokens are their own IDs"; "Hugging Face Tokenizers v1",
// section "How v1 works": post-processing adds the special tokens a model
// expects).  With nb (0 or 1) reserved IDs before and ne after each document,
// the token at plain position p of document d lands at p + d (nb + ne) + nb,
// and document d's IDs start at its plain offset + d (nb + ne): the shift is
// constant between document starts, so no scan changes.  The chunk's
// document starts are placed first (their offsets, BOS and the previous
// document's EOS), then every position is written with the shift of its
// document (a binary search over the starts staged in LDS; a chunk where no
// document starts has one shift for all).
template <bool SP>
__global__ void __launch_bounds__(EWG) k_emit(EncodeArgs a) {
  __shared__ EmitShared<SP> s;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int64_t c = blockIdx.x;
  const int64_t c0 = c * kChunk;
  int32_t *pv = a.pv + c * kChunk;
  const int32_t *res = a.res + c * kMissSpan;
  // loads that need nothing else first: the first round's pv values (pv has
  // room for kChunk entries, so this reads inside it whatever the count), and
  // the first pre-token of the documents that start here.  The IDs (written
  // once) are streamed out with non-temporal stores.
  const uint8_t *cntk = a.cntk + c * kChunk;
  int32_t v0[kEmitPasses], n0[kEmitPasses];
#pragma unroll
  for (int j = 0; j < kEmitPasses; ++j) {
    v0[j] = pv[j * EWG + tid];
    n0[j] = cntk[j * EWG + tid];
  }
  const int64_t dlo = a.doc_rng[2 * c], dhi = a.doc_rng[2 * c + 1];
  const int dk0 = dlo + tid < dhi ? a.doc_pt[dlo + tid] : 0;
  const int n_pt = a.meta[kMetaInts * c + kMetaPretokens];
  const bool docs_here = dhi > dlo;
  const int64_t base = a.off[c] + a.boff[c / kScanBlock];
  if (tid == 0) s.n_long = 0;
  bool overflow = false;
  // SP: the reserved IDs per document, and the output position of plain
  // chunk position w (documents dlo .. dhi - 1 start here, at s.dpos / from
  // their first pre-token's position)
  const int64_t nb = SP && a.bos >= 0 ? 1 : 0, ns = nb + (SP && a.eos >= 0 ? 1 : 0);
  int64_t total = 0;
  auto doc_pos = [&](int64_t d) -> int64_t {
    const int k = min(max(a.doc_pt[d], 0), n_pt);
    return k < n_pt ? (int64_t)pv[k] : total;
  };
  auto out_pos = [&](int64_t w) -> int64_t {
    if (!SP) return base + w;
    const int64_t nd = dhi - dlo;
    int lo = 0, hi = (int)min<int64_t>(nd, kDocLds);  // starts at or before w
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s.dpos[mid] > w) hi = mid;
      else lo = mid + 1;
    }
    int64_t n = lo;
    if (lo == kDocLds && nd > kDocLds) {
      int64_t l2 = kDocLds, h2 = nd;
      while (l2 < h2) {
        const int64_t mid = (l2 + h2) >> 1;
        if (doc_pos(dlo + mid) > w) h2 = mid;
        else l2 = mid + 1;
      }
      n = l2;
    }
    return base + w + ns * max(dlo - 1 + n, (int64_t)0) + nb;
  };
  auto put = [&](int64_t w, int32_t sym) {
    if (w < kOutCap) {
      s.out[w] = sym;
    } else {
      const int64_t o = out_pos(w);
      if (o < a.ids_cap) a.ids[o] = out_id(a.id_map, sym);
      else overflow = true;
    }
  };
  int64_t carry = 0;
  for (int r0 = 0; r0 < n_pt; r0 += EWG * kEmitPasses) {
    // the passes of this round that hold pre-tokens (the same for every thread)
    const int np = min(kEmitPasses, (n_pt - r0 + EWG - 1) / EWG);
    int32_t v[kEmitPasses], cnt[kEmitPasses], inc[kEmitPasses], w0[kEmitPasses];
    u32x4 first[kEmitPasses];
    // a lane-merged entry's count comes from cntk, loaded beside pv, a
    // wave-merged one's from mt; then the first four tokens of each
    // lane-merged entry in one load (other pre-tokens read entry 0: the load
    // stays unconditional), issued last so that the scan below waits for the
    // counts only
#pragma unroll
    for (int j = 0; j < kEmitPasses; ++j) {
      v[j] = INT32_MIN;
      cnt[j] = 0;
      if (j >= np) continue;
      const int k = r0 + j * EWG + tid;
      v[j] = k < n_pt ? (r0 == 0 ? v0[j] : pv[k]) : INT32_MIN;
      const int nk = r0 == 0 ? n0[j] : cntk[k];
      const int u = -1 - v[j];
      const bool neg = v[j] < 0 && v[j] != INT32_MIN;
      const bool lane_merged = neg && (u < kPvLong || u >= kPvDup);
      cnt[j] = v[j] >= 0 ? 1 : (lane_merged ? nk : 0);
      if (neg && !lane_merged) cnt[j] = a.mt[c * kMaxLong + (u - kPvLong)];
    }
#pragma unroll
    for (int j = 0; j < kEmitPasses; ++j) {
      const int u = -1 - v[j];
      const bool lane_merged = v[j] < 0 && v[j] != INT32_MIN && (u < kPvLong || u >= kPvDup);
      first[j] = *reinterpret_cast<const u32x4 *>(entry_res(a, res, lane_merged ? u : 0));
    }
    // positions: every pass of the round is one scan over the workgroup
    // (chunk-relative positions fit 32 bits: only the chunk's last pre-token
    // can run past the window)
#pragma unroll
    for (int j = 0; j < kEmitPasses; ++j) {
      if (j >= np) continue;
      inc[j] = wave_incl_sum(cnt[j]);
      if (lane == 63) s.wtot[j][wave] = inc[j];
    }
    __syncthreads();
    int32_t run = 0;
#pragma unroll
    for (int j = 0; j < kEmitPasses; ++j) {
      if (j >= np) continue;
      int32_t before = 0, all = 0;
#pragma unroll
      for (int ww = 0; ww < EWG / 64; ++ww) {
        const int32_t t = s.wtot[j][ww];
        if (ww < wave) before += t;
        all += t;
      }
      w0[j] = (int32_t)carry + run + before + inc[j] - cnt[j];
      run += all;
    }
#pragma unroll
    for (int j = 0; j < kEmitPasses; ++j) {
      if (j >= np) continue;
      // the tokens of a pre-token that does not run past the window all fall
      // below kOutCap: its first four by unconditional stores (the unused
      // ones to the spare slot), the rest of a longer lane-merged entry after
      const int k = r0 + j * EWG + tid;
      const int32_t x = v[j];
      const int u = -1 - x;
      const bool placed = k < n_pt && (x >= 0 || u < kPvLong || u >= kPvDup);
      const int nt = placed ? cnt[j] : 0;
      const int w = w0[j];
      const u32x4 t = x >= 0 ? u32x4{(uint32_t)x, 0u, 0u, 0u} : first[j];
      s.out[nt > 0 ? w : kOutCap] = (int32_t)t.x;
      s.out[nt > 1 ? w + 1 : kOutCap] = (int32_t)t.y;
      s.out[nt > 2 ? w + 2 : kOutCap] = (int32_t)t.z;
      s.out[nt > 3 ? w + 3 : kOutCap] = (int32_t)t.w;
      if (nt > 4) {
        // the rest four to a 16-byte load: an entry's token span is 16-byte
        // aligned and covers its tokens rounded up to four
        const int32_t *src = entry_res(a, res, u);
        for (int q = 4; q < nt; q += 4) {
          const u32x4 r4 = *reinterpret_cast<const u32x4 *>(src + q);
          s.out[w + q] = (int32_t)r4.x;
          if (q + 1 < nt) s.out[w + q + 1] = (int32_t)r4.y;
          if (q + 2 < nt) s.out[w + q + 2] = (int32_t)r4.z;
          if (q + 3 < nt) s.out[w + q + 3] = (int32_t)r4.w;
        }
      }
      // a chunk where documents start keeps each pre-token's first position
      // in place of its pv value (read by this thread only, and already read)
      if (docs_here && k < n_pt) pv[k] = w;
      if (k < n_pt && x < 0 && u >= kPvLong && u < kPvDup) {
        const int q = u - kPvLong;
        const uint32_t e = a.miss[c * kMissMax + kBucketBase[3] + q];
        const int slot = atomicAdd(&s.n_long, 1);
        s.lw[slot] = w;
        s.lsrc[slot] = c0 + me_start(e);
        s.lnt[slot] = cnt[j];
      }
    }
    carry += run;
    __syncthreads();  // wtot is rewritten by the next round
  }
  total = carry;
  if (SP) {
    // the documents that start here: offsets, their BOS and the previous
    // document's EOS, and their first positions for out_pos
    for (int64_t d = dlo + tid; d < dhi; d += EWG) {
      const int64_t p = doc_pos(d);
      if (d - dlo < kDocLds) s.dpos[d - dlo] = (int32_t)p;
      const int64_t o = base + p + ns * d;
      a.id_off[d] = o;
      if (nb) {
        if (o < a.ids_cap) a.ids[o] = a.bos;
        else overflow = true;
      }
      if (a.eos >= 0 && d >= 1) {
        if (o - 1 < a.ids_cap) a.ids[o - 1] = a.eos;
        else overflow = true;
      }
    }
    __syncthreads();
  }
  // wave-merged entries' symbols, copied by the whole workgroup
  for (int q = 0; q < s.n_long; ++q) {
    const int64_t w0 = s.lw[q], src = s.lsrc[q], nt = s.lnt[q];
    for (int64_t j = tid; j < nt; j += EWG) put(w0 + j, a.gsym[src + j]);
  }
  __syncthreads();
  // the staged positions, in order
  const int nst = (int)min(total, (int64_t)kOutCap);
  if (SP && docs_here) {
    for (int k = tid; k < nst; k += EWG) {
      const int64_t o = out_pos(k);
      if (o < a.ids_cap) a.ids[o] = out_id(a.id_map, s.out[k]);
      else overflow = true;
    }
  } else if (out_pos(0) + nst <= a.ids_cap) {
    // (one shift for the whole chunk)
    const int64_t base = out_pos(0);
    // the positions before the first 16-byte boundary of ids one per thread,
    // then four per thread with 16-byte stores, then the rest
    const int head = min(nst, (int)((4 - ((reinterpret_cast<uintptr_t>(a.ids + base) >> 2) & 3)) & 3));
    const int body = (nst - head) & ~3;
    if (tid < head) a.ids[base + tid] = out_id(a.id_map, s.out[tid]);
    if (a.id_map) {
      for (int k = head + 4 * tid; k < head + body; k += 4 * EWG) {
        uint4 q;
        q.x = (uint32_t)a.id_map[s.out[k]];
        q.y = (uint32_t)a.id_map[s.out[k + 1]];
        q.z = (uint32_t)a.id_map[s.out[k + 2]];
        q.w = (uint32_t)a.id_map[s.out[k + 3]];
        __builtin_nontemporal_store(u32x4{q.x, q.y, q.z, q.w},
                                    reinterpret_cast<u32x4 *>(a.ids + base + k));
      }
    } else {
      // (the symbols are the IDs: the four reads need no branch between them)
      for (int k = head + 4 * tid; k < head + body; k += 4 * EWG)
        __builtin_nontemporal_store(u32x4{(uint32_t)s.out[k], (uint32_t)s.out[k + 1],
                                          (uint32_t)s.out[k + 2], (uint32_t)s.out[k + 3]},
                                    reinterpret_cast<u32x4 *>(a.ids + base + k));
    }
    const int k = head + body + tid;
    if (k < nst) a.ids[base + k] = out_id(a.id_map, s.out[k]);
  } else {
    const int64_t base = out_pos(0);
    for (int k = tid; k < nst; k += EWG) {
      if (base + k < a.ids_cap) a.ids[base + k] = out_id(a.id_map, s.out[k]);
      else overflow = true;
    }
  }
  // per-document offsets: a document starting at pre-token k begins at k's
  // first position (the workgroup's own stores to pv, ordered by the barrier
  // above), one starting after the last pre-token at the chunk's end
  if (!SP) {
    for (int64_t d = dlo + tid; d < dhi; d += EWG) {
      const int k = min(max(d == dlo + tid ? dk0 : a.doc_pt[d], 0), n_pt);
      a.id_off[d] = base + (k < n_pt ? (int64_t)pv[k] : total);
    }
  }
  if (c == a.n_chunks - 1) {
    // documents that start at the input's end (empty), and the end; with
    // reserved IDs their BOS, the EOS before each, and the last document's
    const int64_t end = base + (a.tot[c] & kCountMask);
    for (int64_t d = dhi + tid; d <= a.n_docs; d += EWG) {
      const int64_t o = end + ns * d;
      a.id_off[d] = o;
      if (SP && nb && d < a.n_docs) {
        if (o < a.ids_cap) a.ids[o] = a.bos;
        else overflow = true;
      }
      if (SP && a.eos >= 0 && d >= 1) {
        if (o - 1 < a.ids_cap) a.ids[o - 1] = a.eos;
        else overflow = true;
      }
    }
  }
  if (overflow) atomicOr(a.status, (int32_t)BPE_STATUS_IDS_CAPACITY);
}

// ---- k_special ------------------------------------------------------------------
// Reserved IDs around the documents of an empty input (every document
// empty, as k_empty has checked): document d is [bos, eos] at d (nb + ne).
// One document per thread; every write is checked against the capacity.  (A
// non-empty input gets its reserved IDs from k_emit<true>.)
__global__ void __launch_bounds__(256) k_special(SpecialArgs a) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (d > a.n_docs) return;
  const int64_t nb = a.bos >= 0 ? 1 : 0, ns = nb + (a.eos >= 0 ? 1 : 0);
  const int64_t o = ns * d;
  bool over = false;
  a.id_off[d] = o;
  if (nb && d < a.n_docs) {
    if (o < a.ids_cap) a.ids[o] = a.bos;
    else over = true;
  }
  if (a.eos >= 0 && d >= 1) {
    if (o - 1 < a.ids_cap) a.ids[o - 1] = a.eos;
    else over = true;
  }
  if (over) atomicOr(a.status, (int32_t)BPE_STATUS_IDS_CAPACITY);
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

}  // namespace

hipError_t launch_special(const SpecialArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_special, dim3((unsigned)((a.n_docs + 1 + 255) / 256)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_empty(const int64_t *offs, int64_t n_docs, uint32_t bad_bit, int64_t *out_off,
                        int32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(256), 0, stream, offs, n_docs, bad_bit, out_off,
                     status);
  return hipGetLastError();
}

const char *const kEncStageNames[kEncStages] = {
    "k_docs",       "k_find",    "k_dedup",   "k_merge", "k_merge_wide",
    "k_merge_long", "k_dupfill", "k_offsets", "k_bscan", "k_emit"};

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream, hipEvent_t *ev) {
  const unsigned G = (unsigned)a.n_chunks;
  const unsigned G4 = (G + 3) / 4;
  int st = 0;
  auto mark = [&]() {
    if (ev) (void)hipEventRecord(ev[st++], stream);
  };
  mark();
  hipLaunchKernelGGL(k_docs, dim3((G + 255) / 256), dim3(256), 0, stream, a);
  mark();
  hipLaunchKernelGGL(k_find, dim3(G), dim3(WG), 0, stream, a);
  mark();
  {
    // the first chunks claim the keys they share with most others before the
    // rest start, so that few CAS on one slot at once
    const int64_t seed = min((int64_t)kDedupSeed, a.n_chunks);
    hipLaunchKernelGGL(k_dedup, dim3((unsigned)((seed + 3) / 4)), dim3(256), 0, stream, a,
                       (int64_t)0, seed, 1);
    if (a.n_chunks > seed)
      hipLaunchKernelGGL(k_dedup, dim3((unsigned)((a.n_chunks - seed + 3) / 4)), dim3(256), 0,
                         stream, a, seed, a.n_chunks, 0);
  }
  mark();
  // chunks per lane-merge group: kGroup fills a batch's lanes from several
  // chunks; fewer where that would leave most waves of the persistent
  // k_merge without a group (a small input)
  EncodeArgs m = a;
  m.lgroup = kGroup;
  while (m.lgroup > 1 && 4 * ((G + m.lgroup - 1) / m.lgroup) < (unsigned)a.n_cu * kMergePWaves)
    m.lgroup /= 2;
  const unsigned n_groups = (G + m.lgroup - 1) / m.lgroup;
  const unsigned LG = (n_groups + kMergeWaves - 1) / kMergeWaves;
  hipLaunchKernelGGL(k_merge, dim3(min((unsigned)a.n_cu, n_groups)), dim3(MWG * kMergePWaves), 0,
                     stream, m);
  mark();
  hipLaunchKernelGGL(k_merge_wide, dim3(LG), dim3(MWG * kMergeWaves), 0, stream, m);
  mark();
  hipLaunchKernelGGL(k_merge_long, dim3((G + kGroup - 1) / kGroup), dim3(MWG), 0, stream, a);
  mark();
  hipLaunchKernelGGL(k_dupfill, dim3(G4), dim3(256), 0, stream, a);
  mark();
  hipLaunchKernelGGL(k_offsets, dim3((unsigned)((G + kScanBlock - 1) / kScanBlock)),
                     dim3(kScanBlock), 0, stream, a);
  mark();
  hipLaunchKernelGGL(k_bscan, dim3(1), dim3(OWG), 0, stream, a);
  mark();
  if (a.bos >= 0 || a.eos >= 0) hipLaunchKernelGGL(k_emit<true>, dim3(G), dim3(EWG), 0, stream, a);
  else hipLaunchKernelGGL(k_emit<false>, dim3(G), dim3(EWG), 0, stream, a);
  mark();
  return hipGetLastError();
}

}  // namespace bpe
