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
// The host collects the distinct pre-tokens (bpe_api.cpp); each merge is
// then four kernels on the caller's stream with no host round trip: count
// every adjacent pair into the pair table (open addressing, 64-bit CAS
// claims, 64-bit atomic adds), the best count (atomicMax), the smallest pair
// with that count (atomicMin, emptying the table as it reads it), and the
// replacement in every pre-token.
// Once the best count falls below 2 a flag in device memory turns the
// remaining launches into no-ops.
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

__device__ __forceinline__ uint32_t tslot(uint64_t key, uint64_t mask) {
  uint64_t x = key * 0x9E3779B97F4A7C15ull;
  return (uint32_t)((x >> 29) & mask);
}

// Every adjacent pair of every pre-token, weighted by its frequency: thread
// p takes the pair at original position p (positions past a pre-token's
// current length hold nothing).
__global__ void __launch_bounds__(TWG) k_tcount(TrainArgs a) {
  if (*a.stop) return;
  const int64_t p = (int64_t)blockIdx.x * TWG + threadIdx.x;
  if (p == 0) {  // the merge's best count and key start over (read from k_tmax on)
    a.best[0] = 0ull;
    a.best[1] = ~0ull;
  }
  if (p >= a.n_pos) return;
  const int32_t w = a.pos_word[p];
  const int64_t j = p - a.word_off[w];
  if (j + 1 >= a.word_len[w]) return;
  const int32_t *sym = a.sym + a.word_off[w];
  const uint64_t key = tkey(sym[j], sym[j + 1]);
  const unsigned long long f = (unsigned long long)a.word_freq[w];
  uint64_t s = tslot(key, a.mask);
  for (uint64_t probe = 0; probe <= a.mask; ++probe) {
    // a slot goes from empty to its key once per merge: a plain read that
    // finds the key needs no CAS (the frequent pairs' slots are the hot ones)
    unsigned long long old = a.keys[s];
    if (old == 0ull) old = atomicCAS((unsigned long long *)&a.keys[s], 0ull, (unsigned long long)key);
    if (old == 0ull || old == key) {
      atomicAdd((unsigned long long *)&a.counts[s], f);
      return;
    }
    s = (s + 1) & a.mask;
  }
}

// The best count over the table.
__global__ void __launch_bounds__(TWG) k_tmax(TrainArgs a) {
  if (*a.stop) return;
  __shared__ unsigned long long red[TWG / 64];
  unsigned long long m = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * TWG + threadIdx.x; i <= a.mask;
       i += (uint64_t)gridDim.x * TWG)
    m = max(m, (unsigned long long)a.counts[i]);
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (unsigned long long)__shfl_xor(m, d, 64));
  if (lane_id() == 0) red[wave_id()] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < TWG / 64; ++w) m = max(m, red[w]);
    if (m) atomicMax((unsigned long long *)&a.best[0], m);
  }
}

// The smallest pair with the best count; each slot is emptied once read, so
// the table starts the next merge empty.
__global__ void __launch_bounds__(TWG) k_tmin(TrainArgs a) {
  if (*a.stop) return;
  __shared__ unsigned long long red[TWG / 64];
  const uint64_t best = a.best[0];
  unsigned long long m = ~0ull;
  for (uint64_t i = (uint64_t)blockIdx.x * TWG + threadIdx.x; i <= a.mask;
       i += (uint64_t)gridDim.x * TWG) {
    const uint64_t k = a.keys[i];
    if (k == 0ull) continue;
    if (a.counts[i] == best) m = min(m, (unsigned long long)k);
    a.keys[i] = 0ull;
    a.counts[i] = 0ull;
  }
  for (int d = 32; d >= 1; d >>= 1) m = min(m, (unsigned long long)__shfl_xor(m, d, 64));
  if (lane_id() == 0) red[wave_id()] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < TWG / 64; ++w) m = min(m, red[w]);
    if (m != ~0ull) atomicMin((unsigned long long *)&a.best[1], m);
  }
}

// Merge r: (l, r) -> 256 + r in every pre-token, one left-to-right pass
// without overlap, one pre-token per thread; thread 0 records the merge (or,
// below a count of 2, stops training).
__global__ void __launch_bounds__(TWG) k_tapply(TrainArgs a, int64_t r) {
  if (*a.stop) return;
  const uint64_t best = a.best[0], key = a.best[1];
  const int64_t w = (int64_t)blockIdx.x * TWG + threadIdx.x;
  if (best < 2 || key == ~0ull) {
    // every thread reads the flag before any writes it: it is written by
    // the last kernel of this merge, and the next merge's kernels see it
    if (w == 0) *a.stop = 1;
    return;
  }
  const int32_t L = (int32_t)((key - 1) >> 32), R = (int32_t)((key - 1) & 0xFFFFFFFFull);
  if (w == 0) {
    a.merges[2 * r] = L;
    a.merges[2 * r + 1] = R;
    a.out_counts[r] = (int64_t)best;
    *a.made = r + 1;
  }
  if (w >= a.n_words) return;
  int32_t *sym = a.sym + a.word_off[w];
  const int32_t n = a.word_len[w];
  int32_t o = 0;
  for (int32_t i = 0; i < n;) {
    if (i + 1 < n && sym[i] == L && sym[i + 1] == R) {
      sym[o++] = 256 + (int32_t)r;
      i += 2;
    } else {
      sym[o++] = sym[i++];
    }
  }
  a.word_len[w] = o;
}

}  // namespace

hipError_t launch_train_step(const TrainArgs &a, int64_t r, hipStream_t stream) {
  const unsigned red_blocks = (unsigned)std::min<uint64_t>((a.mask + TWG) / TWG, 1024);
  hipLaunchKernelGGL(k_tcount, dim3((unsigned)((a.n_pos + TWG - 1) / TWG)), dim3(TWG), 0, stream, a);
  hipLaunchKernelGGL(k_tmax, dim3(red_blocks), dim3(TWG), 0, stream, a);
  hipLaunchKernelGGL(k_tmin, dim3(red_blocks), dim3(TWG), 0, stream, a);
  hipLaunchKernelGGL(k_tapply, dim3((unsigned)((a.n_words + TWG - 1) / TWG)), dim3(TWG), 0, stream,
                     a, r);
  return hipGetLastError();
}

}  // namespace bpe
