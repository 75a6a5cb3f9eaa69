// bpe_train.hip -- training a merge table on the GPU.
//
// "Characters, bytes and subwords", section "BPE step by step": start from
// the bytes, count the adjacent pairs over the training text, take the most
// frequent pair (ties: the smallest IDs), give it the next ID, replace its
// occurrences, and count again, until the requested number of merges or
// until no pair is frequent enough.  "Hugging Face Tokenizers v1", section
// "How v1 works": a merge never crosses a pre-token boundary, so the text is
// counted as its distinct pre-tokens with their frequencies.  Readings: a
// pair is counted at every position (so [a, a, a] counts (a, a) twice, each
// weighted by the pre-token's frequency); ties go to the smallest (left,
// right); training stops when the best count is below 2; replacement is one
// left-to-right pass without overlap, the merge step of encoding.
//
// "Count again" is kept incremental: a merge changes only the pre-tokens
// that hold its pair, and in them only the pairs next to an occurrence.  The
// host collects the distinct pre-tokens (bpe_api.cpp) and the occurrence
// lists of the bytes; the device counts every pair once into an
// open-addressing pair table whose slots are summarized in blocks (each
// block's largest count and the smallest key with it).  A merge is then:
//   pick   the best pair from the block summaries;
//   merge  the pre-tokens on the shorter occurrence list of the pair's two
//          symbols, one per thread: a pre-token that holds the pair subtracts
//          the counts of the pairs the merge changes (times its frequency),
//          replaces the pair left to right, adds the new pairs' counts, and
//          joins the new symbol's occurrence list;
//   sum    the summaries of the blocks the merge may have changed.
// The first merges change many pre-tokens and run as three grid-wide
// kernels each (k_tpick, k_tmerge, k_tsum); the rest run in one resident
// workgroup (k_tloop), whose barriers replace the kernel boundaries.
// A merge cannot raise the best count (a new pair occurs at most as often as
// the pair just merged, and other pairs only lose occurrences), and a pair's
// count, once it falls to 0 after the merge that made the pair possible,
// never rises again, so keys are never removed from the table.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "bpe_internal.h"

namespace bpe {
namespace {

constexpr int TWG = 256;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ uint64_t tkey(int32_t l, int32_t r) {
  return (((uint64_t)(uint32_t)l << 32) | (uint32_t)r) + 1;  // 0 marks an empty slot
}

__device__ __forceinline__ uint64_t tslot(uint64_t key, uint64_t mask) {
  uint64_t x = key * 0x9E3779B97F4A7C15ull;
  return (x >> 29) & mask;
}

__device__ __forceinline__ uint64_t load_key(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The slot of key (linear probing), claimed by a 64-bit CAS when it is not
// there yet.  A plain atomic read that finds the key skips the CAS (the
// frequent pairs' slots are the contended ones).
__device__ uint64_t pair_slot(const TrainArgs &a, uint64_t key) {
  uint64_t s = tslot(key, a.mask);
  for (uint64_t probe = 0; probe <= a.mask; ++probe) {
    unsigned long long old = load_key(&a.keys[s]);
    if (old == 0ull) old = atomicCAS((unsigned long long *)&a.keys[s], 0ull, (unsigned long long)key);
    if (old == 0ull || old == key) return s;
    s = (s + 1) & a.mask;
  }
  return ~0ull;  // a full table (it is sized so that this cannot happen)
}

// (count, key) x better than y: a larger count, or the same count and a
// smaller key.
__device__ __forceinline__ bool better(uint32_t cx, unsigned long long kx, uint32_t cy,
                                       unsigned long long ky) {
  return cx > cy || (cx == cy && kx < ky);
}

// The best (count, key) over a wave, in every lane.
__device__ __forceinline__ void wave_best(uint32_t &c, unsigned long long &k) {
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t c2 = __shfl_xor(c, d, 64);
    const unsigned long long k2 = __shfl_xor(k, d, 64);
    if (better(c2, k2, c, k)) {
      c = c2;
      k = k2;
    }
  }
}

// The best slot of block b, by one wave: its count, and its key (~0 when
// every count is 0).  Per 1024 slots the counts come in one round of loads
// (16 per lane), then only the slots with the largest count load their keys.
__device__ void block_best(const TrainArgs &a, uint64_t b, uint32_t &m, unsigned long long &km) {
  m = 0;
  km = ~0ull;
  const uint64_t s0 = b * a.bsize;
  for (uint64_t c0 = 0; c0 < a.bsize; c0 += 1024) {
    uint32_t c[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = a.counts[s0 + c0 + 64 * j + lane_id()];
    uint32_t cm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) cm = max(cm, c[j]);
    for (int d = 32; d >= 1; d >>= 1) cm = max(cm, (uint32_t)__shfl_xor(cm, d, 64));
    if (cm == 0 || cm < m) continue;
    unsigned long long ck = ~0ull;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (c[j] == cm) ck = min(ck, (unsigned long long)a.keys[s0 + c0 + 64 * j + lane_id()]);
    for (int d = 32; d >= 1; d >>= 1) ck = min(ck, (unsigned long long)__shfl_xor(ck, d, 64));
    if (better(cm, ck, m, km)) {
      m = cm;
      km = ck;
    }
  }
}

// Every adjacent pair of every pre-token, weighted by its frequency (thread
// p: the pair at original position p).
__global__ void __launch_bounds__(TWG) k_tcount(TrainArgs a) {
  const int64_t p = (int64_t)blockIdx.x * TWG + threadIdx.x;
  if (p >= a.n_pos) return;
  const int32_t w = a.pos_word[p];
  const uint4 rec = a.wrec[w];
  const int64_t j = p - (int64_t)rec.x;
  if (j + 1 >= (int64_t)rec.y) return;
  const int32_t *sym = a.sym + rec.x;
  const uint64_t s = pair_slot(a, tkey(sym[j], sym[j + 1]));
  if (s != ~0ull) atomicAdd(&a.counts[s], rec.z);
}

// Block summaries, one block per wave: every block (k_tsum_all), or the
// blocks listed by the last merge (k_tsum).
__global__ void __launch_bounds__(TWG) k_tsum_all(TrainArgs a) {
  const uint64_t b = (uint64_t)blockIdx.x * (TWG / 64) + wave_id();
  if (b >= (uint64_t)a.nblocks) return;
  uint32_t m;
  unsigned long long km;
  block_best(a, b, m, km);
  if (lane_id() == 0) {
    a.bmax[b] = m;
    a.bkey[b] = km;
  }
}

__global__ void __launch_bounds__(TWG) k_tsum(TrainArgs a) {
  if (*a.stop) return;
  const uint32_t n = *a.ndirty;
  for (uint32_t i = blockIdx.x * (TWG / 64) + wave_id(); i < n; i += gridDim.x * (TWG / 64)) {
    const uint32_t b = a.dlist[i];
    uint32_t m;
    unsigned long long km;
    block_best(a, b, m, km);
    if (lane_id() == 0) {
      a.bmax[b] = m;
      a.bkey[b] = km;
      a.dirty[b] = 0u;
    }
  }
}

// ---- the first merges: three grid-wide kernels each ---------------------------

// Lists slot s's block for k_tsum, once per merge.
__device__ __forceinline__ void touch(const TrainArgs &a, uint64_t s) {
  const uint64_t b = s / a.bsize;
  if (__hip_atomic_load(&a.dirty[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u &&
      atomicExch(&a.dirty[b], 1u) == 0u)
    a.dlist[atomicAdd(a.ndirty, 1u)] = (uint32_t)b;
}

constexpr int PWG = 1024;

// The best pair: the largest count over the blocks, then the smallest key
// with it; training stops below a count of 2 or after n_target merges.  One
// workgroup.  It also closes the last merge's occurrence list and empties
// the list of touched blocks (k_tsum has read it).
__global__ void __launch_bounds__(PWG) k_tpick(TrainArgs a) {
  if (*a.stop) return;
  __shared__ uint32_t rc[PWG / 64];
  __shared__ unsigned long long rk[PWG / 64];
  uint32_t m = 0;
  unsigned long long km = ~0ull;
  for (int64_t b = threadIdx.x; b < a.nblocks; b += PWG)
    if (better(a.bmax[b], a.bkey[b], m, km)) {
      m = a.bmax[b];
      km = a.bkey[b];
    }
  wave_best(m, km);
  if (lane_id() == 0) {
    rc[wave_id()] = m;
    rk[wave_id()] = km;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < PWG / 64; ++w)
      if (better(rc[w], rk[w], m, km)) {
        m = rc[w];
        km = rk[w];
      }
    const int64_t r = *a.made;
    *a.ndirty = 0u;
    if (r > 0) {
      // the occurrence list of the last merge's symbol is complete
      const int64_t z = 255 + r;
      const uint32_t nz = *a.zcount;
      a.lrec[z] = uint2{(uint32_t)*a.pool_top, nz};
      *a.pool_top += nz;
      *a.zcount = 0u;
    }
    if (m < 2 || km == ~0ull || r >= a.n_grid) {
      if (m < 2 || km == ~0ull || r >= a.n_target) *a.stop = 1;
      a.best[2] = ~0ull;  // no merge this step
    } else {
      a.best[0] = m;
      a.best[1] = km;
      a.best[2] = (uint64_t)r;
    }
  }
}

// Pre-token w of the merge (L, R) -> z, if it holds the pair: the counts of
// the pairs the merge changes updated (add(l, r, f, dec): count -= f when
// dec, else += f), the pair
// replaced, and w put on z's occurrence list (join(w)).  The changed pairs:
// before, every pair that overlaps an occurrence (positions i - 1, i and
// i + 1 for an occurrence at i, each once); after, every pair next to a new
// symbol.  Every other pair is the same pair at the same place before and
// after.
template <class Add, class Join>
__device__ void merge_word(const TrainArgs &a, int32_t w, int32_t L, int32_t R, int32_t z,
                           Add &&add, Join &&join) {
  const uint4 rec = a.wrec[w];
  int32_t *sym = a.sym + rec.x;
  const int32_t n = (int32_t)rec.y;
  // the first symbols in one go (independent loads), then the rest
  constexpr int HEAD = 8;
  int32_t v[HEAD];
#pragma unroll
  for (int k = 0; k < HEAD; ++k) v[k] = k < n ? sym[k] : -1;
  bool has = false;
#pragma unroll
  for (int k = 0; k + 1 < HEAD; ++k) has |= k + 1 < n && v[k] == L && v[k + 1] == R;
  for (int32_t i = HEAD - 1; i + 1 < n && !has; ++i) has = sym[i] == L && sym[i + 1] == R;
  if (!has) return;
  const uint32_t f = rec.z;
  // the pairs that change, before: subtracted
  int32_t done = -1;  // the last pair index already subtracted
  for (int32_t i = 0; i + 1 < n;) {
    if (sym[i] == L && sym[i + 1] == R) {
      for (int32_t q = max(i - 1, done + 1); q <= min(i + 1, n - 2); ++q)
        add(sym[q], sym[q + 1], f, true);
      done = min(i + 1, n - 2);
      i += 2;
    } else {
      ++i;
    }
  }
  // the replacement, left to right without overlap
  int32_t o = 0;
  for (int32_t i = 0; i < n;) {
    if (i + 1 < n && sym[i] == L && sym[i + 1] == R) {
      sym[o++] = z;
      i += 2;
    } else {
      sym[o++] = sym[i++];
    }
  }
  reinterpret_cast<uint32_t *>(a.wrec)[4 * (int64_t)w + 1] = (uint32_t)o;
  // after: the pairs next to a new symbol, added
  for (int32_t j = 0; j + 1 < o; ++j) {
    const int32_t x = sym[j], y = sym[j + 1];
    if (x == z || y == z) add(x, y, f, false);
  }
  join(w);
}

// Merge r = best[2]: (L, R) -> 256 + r in every pre-token that holds the
// pair (each is on the occurrence lists of both L and R: the shorter list is
// walked, one entry per thread); thread 0 records the merge.
__global__ void __launch_bounds__(TWG) k_tmerge(TrainArgs a) {
  if (*a.stop || a.best[2] == ~0ull) return;
  const uint64_t best = a.best[0], key = a.best[1];
  const int64_t r = (int64_t)a.best[2];
  const int32_t L = (int32_t)((key - 1) >> 32), R = (int32_t)((key - 1) & 0xFFFFFFFFull);
  const int32_t z = 256 + (int32_t)r;
  const int64_t t = (int64_t)blockIdx.x * TWG + threadIdx.x;
  if (t == 0) {
    a.merges[2 * r] = L;
    a.merges[2 * r + 1] = R;
    a.out_counts[r] = (int64_t)best;
    *a.made = r + 1;
  }
  const uint2 ll = a.lrec[L], lr = a.lrec[R];
  const int32_t *lst = a.pool + (ll.y <= lr.y ? ll.x : lr.x);
  const int64_t nlst = min(ll.y, lr.y);
  const unsigned long long zbase = *a.pool_top;
  auto add = [&](int32_t l, int32_t rr, uint32_t f, bool dec) {
    const uint64_t s = pair_slot(a, tkey(l, rr));
    if (s == ~0ull) return;
    atomicAdd(&a.counts[s], dec ? 0u - f : f);
    touch(a, s);
  };
  auto join = [&](int32_t w) { a.pool[zbase + atomicAdd(a.zcount, 1u)] = w; };
  for (int64_t i = t; i < nlst; i += (int64_t)gridDim.x * TWG)
    merge_word(a, lst[i], L, R, z, add, join);
}

// ---- the later merges in one workgroup ------------------------------------------
//
// After the first merges a merge changes few pre-tokens, and a chain of three
// small kernels per merge costs more than its work.  k_tloop runs the rest in
// one resident workgroup: the block summaries sit in LDS, the pick is a scan
// of them, and the phases are separated by workgroup barriers (only this
// workgroup touches the pre-tokens, the pair table and the lists, so its
// barriers order them).  A block's summary is recomputed only when the merge
// may have changed it: a decrement of the slot that holds the block's best,
// or an increment that reaches the block's largest count.

constexpr int LWG = 1024;
constexpr int kLoopUpdates = 2048;   // count updates of a merge gathered in LDS (more: applied in place)
constexpr int kLoopGroup = 64;       // blocks per group of the two-level pick
constexpr int kLoopGroups = kTrainLoopBlocks / kLoopGroup;

struct LoopShared {
  uint32_t bmax[kTrainLoopBlocks];
  unsigned long long bkey[kTrainLoopBlocks];
  uint32_t gmax[kLoopGroups];            // per group of blocks: the best of their summaries
  unsigned long long gkey[kLoopGroups];
  uint32_t dmask[kTrainLoopBlocks / 32];  // blocks marked this merge
  uint16_t dlist[kTrainLoopBlocks];
  int32_t ul[kLoopUpdates], ur[kLoopUpdates];  // the merge's count updates: pair, amount, sign
  uint32_t uf[kLoopUpdates];
  uint8_t udec[kLoopUpdates];
  int ndirty, nupd;
  uint32_t nz, top;  // pre-tokens joined to the new symbol's list; the pool's first free entry
};

__device__ __forceinline__ void loop_mark(LoopShared &s, uint32_t b) {
  const uint32_t bit = 1u << (b & 31);
  if (atomicOr(&s.dmask[b >> 5], bit) & bit) return;
  s.dlist[atomicAdd(&s.ndirty, 1)] = (uint16_t)b;
}

// Group g's summary from its blocks' (one wave).
__device__ __forceinline__ void loop_group(LoopShared &s, int g, int nb) {
  const int b = g * kLoopGroup + lane_id();
  uint32_t m = b < nb ? s.bmax[b] : 0u;
  unsigned long long km = b < nb ? s.bkey[b] : ~0ull;
  wave_best(m, km);
  if (lane_id() == 0) {
    s.gmax[g] = m;
    s.gkey[g] = km;
  }
}

__global__ void __launch_bounds__(LWG) k_tloop(TrainArgs a) {
  if (*a.stop) return;
  __shared__ LoopShared s;
  const int lane = lane_id(), wave = wave_id();
  const int nb = (int)a.nblocks;
  const int ng = (nb + kLoopGroup - 1) / kLoopGroup;
  for (int b = threadIdx.x; b < nb; b += LWG) {
    s.bmax[b] = a.bmax[b];
    s.bkey[b] = a.bkey[b];
  }
  for (int i = threadIdx.x; i < kTrainLoopBlocks / 32; i += LWG) s.dmask[i] = 0u;
  if (threadIdx.x == 0) {
    s.ndirty = 0;
    s.nupd = 0;
    // the occurrence list of the last grid-wide merge's symbol, when no pick
    // has closed it yet
    const int64_t r = *a.made;
    const uint32_t nz = *a.zcount;
    if (r > 0 && nz > 0) {
      a.lrec[255 + r] = uint2{(uint32_t)*a.pool_top, nz};
      *a.pool_top += nz;
      *a.zcount = 0u;
    }
    s.nz = 0u;
    s.top = (uint32_t)*a.pool_top;
  }
  __syncthreads();
  for (int g = wave; g < ng; g += LWG / 64) loop_group(s, g, nb);
  __syncthreads();
  // count(l, r) -= f (dec) or += f, and the block marked when its summary
  // may change
  auto apply = [&](int32_t l, int32_t r, uint32_t f, bool dec) {
    const uint64_t key = tkey(l, r);
    const uint64_t slot = pair_slot(a, key);
    if (slot == ~0ull) return;
    const uint32_t old = atomicAdd(&a.counts[slot], dec ? 0u - f : f);
    const uint32_t b = (uint32_t)(slot / a.bsize);
    if (dec) {
      if (old == s.bmax[b] && key == s.bkey[b]) loop_mark(s, b);
    } else if (old + f >= s.bmax[b]) {
      loop_mark(s, b);
    }
  };
  // an update gathered for the whole workgroup, or applied at once when the
  // list is full
  auto add = [&](int32_t l, int32_t r, uint32_t f, bool dec) {
    const int i = atomicAdd(&s.nupd, 1);
    if (i < kLoopUpdates) {
      s.ul[i] = l;
      s.ur[i] = r;
      s.uf[i] = f;
      s.udec[i] = dec ? 1 : 0;
    } else {
      apply(l, r, f, dec);
    }
  };
  for (int64_t r = *a.made; r < a.n_target; ++r) {
    // pick (every wave, from the group summaries): the largest count, then
    // the smallest key with it
    uint32_t m = 0;
    unsigned long long km = ~0ull;
    for (int g = lane; g < ng; g += 64)
      if (better(s.gmax[g], s.gkey[g], m, km)) {
        m = s.gmax[g];
        km = s.gkey[g];
      }
    wave_best(m, km);
    if (m < 2 || km == ~0ull) {
      if (threadIdx.x == 0) *a.stop = 1;
      break;
    }
    const int32_t L = (int32_t)((km - 1) >> 32), R = (int32_t)((km - 1) & 0xFFFFFFFFull);
    const int32_t z = 256 + (int32_t)r;
    if (threadIdx.x == 0) {
      a.merges[2 * r] = L;
      a.merges[2 * r + 1] = R;
      a.out_counts[r] = (int64_t)m;
      *a.made = r + 1;
    }
    // merge: the shorter occurrence list, one pre-token per thread; the
    // count updates gathered, then applied one per thread
    const uint2 ll = a.lrec[L], lr = a.lrec[R];
    const int32_t *lst = a.pool + (ll.y <= lr.y ? ll.x : lr.x);
    const int32_t nlst = (int32_t)min(ll.y, lr.y);
    const uint32_t zbase = s.top;
    auto join = [&](int32_t w) { a.pool[zbase + atomicAdd(&s.nz, 1u)] = w; };
    for (int32_t i = threadIdx.x; i < nlst; i += LWG) merge_word(a, lst[i], L, R, z, add, join);
    __syncthreads();
    const int nu = min(s.nupd, kLoopUpdates);
    for (int i = threadIdx.x; i < nu; i += LWG) apply(s.ul[i], s.ur[i], s.uf[i], s.udec[i] != 0);
    __syncthreads();
    // the new symbol's list; the marked blocks' summaries (one block per
    // wave), then their groups'
    if (threadIdx.x == 0) {
      const uint32_t nz = s.nz;
      a.lrec[z] = uint2{zbase, nz};
      s.top = zbase + nz;
      s.nz = 0u;
      s.nupd = 0;
    }
    const int nd = s.ndirty;
    for (int i = wave; i < nd; i += LWG / 64) {
      const uint32_t b = s.dlist[i];
      uint32_t bm;
      unsigned long long bk;
      block_best(a, b, bm, bk);
      if (lane == 0) {
        s.bmax[b] = bm;
        s.bkey[b] = bk;
        s.dmask[b >> 5] = 0u;
      }
    }
    __syncthreads();
    for (int i = wave; i < nd; i += LWG / 64) loop_group(s, s.dlist[i] / kLoopGroup, nb);
    __syncthreads();
    if (threadIdx.x == 0) s.ndirty = 0;
    __syncthreads();
  }
}

constexpr unsigned kSumGrid = 128;
constexpr unsigned kMergeGrid = 512;

}  // namespace

hipError_t launch_train_init(const TrainArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_tcount, dim3((unsigned)((a.n_pos + TWG - 1) / TWG)), dim3(TWG), 0, stream, a);
  hipLaunchKernelGGL(k_tsum_all, dim3((unsigned)((a.nblocks + TWG / 64 - 1) / (TWG / 64))), dim3(TWG),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_train_step(const TrainArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_tpick, dim3(1), dim3(PWG), 0, stream, a);
  hipLaunchKernelGGL(k_tmerge, dim3(kMergeGrid), dim3(TWG), 0, stream, a);
  hipLaunchKernelGGL(k_tsum, dim3(kSumGrid), dim3(TWG), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_train_loop(const TrainArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_tloop, dim3(1), dim3(LWG), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bpe
