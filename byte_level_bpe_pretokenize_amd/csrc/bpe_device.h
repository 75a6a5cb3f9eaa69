// bpe_device.h -- device helpers shared by the encode and decode kernels:
// byte classes, rank probes, wave / workgroup reductions and scans, a wave-wide
// binary search and the per-chunk offset scan.
#pragma once

#include <limits.h>
#include <stdint.h>

#include "bpe_internal.h"

namespace bpe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNoStart = INT_MAX;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// The rank table as seen by the kernels.
struct RankTable {
  const u64x2 *b;             // buckets
  uint32_t mask;              // buckets - 1
  uint32_t seed;
  const uint32_t *filt = nullptr;  // the pair filter (pair_filter_bit), nullptr = none
};

// False when the pair with mix x certainly has no rank (its filter bit is clear).
__device__ __forceinline__ bool pair_maybe(const RankTable &t, uint32_t x) {
  if (!t.filt) return true;
  const uint32_t k = pair_filter_bit(x);
  return (t.filt[k >> 5] >> (k & 31)) & 1u;
}

// Rank held by a loaded bucket for key, or kRankInf.
__device__ __forceinline__ int32_t bucket_rank(u64x2 b, uint64_t key) {
  if ((b.x >> kSymBits) == key) return (int32_t)((uint32_t)b.x & kRankMask);
  if ((b.y >> kSymBits) == key) return (int32_t)((uint32_t)b.y & kRankMask);
  return kRankInf;
}

// Whether a lookup that missed in this first bucket must load the second.
__device__ __forceinline__ bool bucket_flag(u64x2 b) { return ((uint32_t)b.x & kSlotFlag) != 0; }

// Rank of the pair (l, r), or kRankInf: the first bucket, then the second
// only if the first bucket's flag asks for it.
__device__ __forceinline__ int32_t rank_of(const RankTable &t, uint32_t l, uint32_t r) {
  const uint32_t x = pair_mix(l, r, t.seed);
  const uint64_t key = pair_key(l, r);
  const u64x2 b0 = t.b[pair_bucket0(x, t.mask)];
  int32_t rk = bucket_rank(b0, key);
  if (rk == kRankInf && bucket_flag(b0)) rk = bucket_rank(t.b[pair_bucket1(x, t.mask)], key);
  return rk;
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

// The same for 32-bit values with every lane of the wave active, in six DPP
// adds and no LDS traffic: prefix sums within each row of 16 lanes by row
// shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row add 0), then
// lane 15's sum added to row 1 and row 3 (row broadcast 15), then lane 31's
// to rows 2 and 3 (row broadcast 31).
__device__ __forceinline__ int32_t wave_incl_sum(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The same for 64-bit values: each DPP step moves both 32-bit halves, then
// one 64-bit add.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)v >> 32), CTRL,
                                                            ROW_MASK, 0xF, false);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t wave_incl_sum(int64_t v) {
  v += dpp64<0x111, 0xF>(v);
  v += dpp64<0x112, 0xF>(v);
  v += dpp64<0x114, 0xF>(v);
  v += dpp64<0x118, 0xF>(v);
  v += dpp64<0x142, 0xA>(v);
  v += dpp64<0x143, 0xC>(v);
  return v;
}

// Lane l's value in every lane (l the same in every lane of the wave).
__device__ __forceinline__ int32_t lane_value(int32_t v, int l) {
  return __builtin_amdgcn_readlane(v, l);
}
__device__ __forceinline__ int64_t lane_value(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Each lane gets the value of the lane below it, lane 0 gets fill (DPP wave
// shift; every lane active).
__device__ __forceinline__ int32_t wave_shift_up1(int32_t v, int32_t fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x138, 0xF, 0xF, false);  // wave_shr:1
}

// Each lane gets the value of the lane above it, lane 63 gets fill (DPP
// wave shift; every lane active).
__device__ __forceinline__ int32_t wave_shift_down1(int32_t v, int32_t fill) {
  return __builtin_amdgcn_update_dpp(fill, v, 0x130, 0xF, 0xF, false);  // wave_shl:1
}

// Running maximum over the lanes (lane i gets the maximum of lanes 0..i),
// every lane active: the same DPP steps as wave_incl_sum.
__device__ __forceinline__ int32_t wave_incl_max(int32_t v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x111, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x112, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x114, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x118, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x142, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x143, 0xC, 0xF, false));
  return v;
}

// Minimum and maximum over the wave in every lane (every lane active): a
// running minimum by DPP, then lane 63's.
__device__ __forceinline__ int32_t wave_min(int32_t v) {
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x111, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x112, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x114, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x118, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x142, 0xA, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x143, 0xC, 0xF, false));
  return lane_value(v, 63);
}
__device__ __forceinline__ int32_t wave_max(int32_t v) { return lane_value(wave_incl_max(v), 63); }

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

// Per-chunk totals carry the chunk's status bits above bit kCountBits.
constexpr int kCountBits = 56;
constexpr int kScanSeg = 16;
constexpr int64_t kCountMask = (1ll << kCountBits) - 1;

// Exclusive prefix of the per-chunk counts tot[0..n) (low kCountBits bits)
// into off, and the OR of their status bits into *status.  One workgroup of
// NT threads; thread t owns kScanSeg consecutive chunks of each tile, read
// and written with 16-byte accesses: tot and off are 256-byte aligned and
// hold n rounded up to kScanSeg entries (the extra ones are ignored).
// red64 holds NT / 64 values.
template <int NT>
__device__ void chunk_offsets(const int64_t *__restrict__ tot, int64_t *__restrict__ off,
                              int64_t n, int32_t *status, int64_t *red64) {
  constexpr int64_t TILE = (int64_t)NT * kScanSeg;
  typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
  int64_t carry = 0;
  int64_t bits = 0;
  for (int64_t t0 = 0; t0 < n; t0 += TILE) {
    const int64_t b0 = t0 + (int64_t)threadIdx.x * kScanSeg;
    i64x2 v[kScanSeg / 2];
    int64_t sum = 0;
    if (b0 < n) {
      const i64x2 *p = reinterpret_cast<const i64x2 *>(tot + b0);
#pragma unroll
      for (int j = 0; j < kScanSeg / 2; ++j) v[j] = p[j];
#pragma unroll
      for (int j = 0; j < kScanSeg / 2; ++j) {
        if (b0 + 2 * j >= n) v[j].x = 0;
        if (b0 + 2 * j + 1 >= n) v[j].y = 0;
        bits |= v[j].x | v[j].y;
        v[j].x &= kCountMask;
        v[j].y &= kCountMask;
        sum += v[j].x + v[j].y;
      }
    }
    int64_t total;
    int64_t run = carry + block_excl_sum<int64_t, NT>(sum, red64, &total);
    if (b0 < n) {
      i64x2 *q = reinterpret_cast<i64x2 *>(off + b0);
#pragma unroll
      for (int j = 0; j < kScanSeg / 2; ++j) {
        i64x2 x;
        x.x = run;
        x.y = run + v[j].x;
        run = x.y + v[j].y;
        q[j] = x;
      }
    }
    carry += total;
  }
  int32_t b32 = (int32_t)(bits >> kCountBits);
  for (int d = 32; d >= 1; d >>= 1) b32 |= __shfl_xor(b32, d, 64);
  int32_t *red = reinterpret_cast<int32_t *>(red64);
  if (lane_id() == 0) red[wave_id()] = b32;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t all = 0;
    for (int w = 0; w < NT / 64; ++w) all |= red[w];
    *status = all;
  }
}

// First level of an offset scan: block blockIdx.x of kScanBlock chunks, one
// chunk per thread (coalesced), of the per-chunk counts tot[0..n) (status
// bits above kCountBits): the exclusive prefix within the block into off,
// and the block's count with the OR of its status bits into bsum.  The
// second level is chunk_offsets over bsum.
__device__ void block_offsets(const int64_t *__restrict__ tot, int64_t *__restrict__ off,
                              int64_t *__restrict__ bsum, int64_t n) {
  __shared__ int64_t red64[kScanBlock / 64];
  __shared__ int32_t bits_w[kScanBlock / 64];
  const int64_t c = (int64_t)blockIdx.x * kScanBlock + threadIdx.x;
  const int64_t v = c < n ? tot[c] : 0;
  int64_t total;
  const int64_t ex = block_excl_sum<int64_t, kScanBlock>(v & kCountMask, red64, &total);
  if (c < n) off[c] = ex;
  int32_t b32 = (int32_t)(v >> kCountBits);
  for (int d = 32; d >= 1; d >>= 1) b32 |= __shfl_xor(b32, d, 64);
  if (lane_id() == 0) bits_w[wave_id()] = b32;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t all = 0;
    for (int w = 0; w < kScanBlock / 64; ++w) all |= bits_w[w];
    bsum[blockIdx.x] = total | ((int64_t)all << kCountBits);
  }
}

__device__ __forceinline__ int32_t out_id(const int32_t *id_map, int32_t sym) {
  return id_map ? id_map[sym] : sym;
}

}  // namespace
}  // namespace bpe
