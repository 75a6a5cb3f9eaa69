// bpe_decode.hip -- byte-level BPE decode for gfx950.
//
// Decode maps every ID back to its symbol and writes the symbol's byte
// expansion; the concatenation is the original text.  IDs are cut into
// chunks of kDecChunk; three kernels, none of which waits on another
// workgroup:
//   k_dec_len    per chunk (two a workgroup): the byte count of its IDs and
//                its status bits
//                (an ID outside the vocabulary, bad document offsets).
//   k_dec_scan   exclusive scan of the chunk byte counts within blocks of
//                1024 chunks; k_dec_bscan the same over the blocks' counts,
//                and the status word.
//   k_dec_write  per chunk: the byte offset of each ID in the chunk, the
//                bytes, and the per-document byte offsets.
//
// Sources: "Tokenization LLM: ... C++" (glitch4techs.com), sections
// "Byte-level encoding" (every byte sequence has a representation, so
// decoding returns the exact input bytes) and "Vocabulary lookup" (ID back
// to token); "Hugging Face Tokenizers v1" (dothoosh.com), section "Road to
// 1.0.0" (GPU batch decode).
#include "../../include/bpe.h"
#include "bpe_device.h"

namespace bpe {
namespace {

constexpr int DWG = kDecThreads;
constexpr int DPT = kDecPerThread;
constexpr int SWG = 1024;

// Symbol of an ID, or -1 for an ID with no symbol.
__device__ __forceinline__ int32_t dec_sym(const DecodeArgs &a, int32_t id) {
  if (a.inv_map) return (id >= 0 && id < a.inv_size) ? a.inv_map[id] : -1;
  return (id >= 0 && id < a.vocab) ? id : -1;
}

// The symbols of DPT IDs (dec_sym): the map's loads unconditional (entry 0
// for an ID outside it) and issued together, so that no lane is masked off
// around them and no load waits on another.
__device__ __forceinline__ void dec_syms(const DecodeArgs &a, const int32_t *id, int32_t *sym) {
  if (a.inv_map) {
    int32_t m[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) m[j] = a.inv_map[(id[j] >= 0 && id[j] < a.inv_size) ? id[j] : 0];
#pragma unroll
    for (int j = 0; j < DPT; ++j) sym[j] = (id[j] >= 0 && id[j] < a.inv_size) ? m[j] : -1;
  } else {
#pragma unroll
    for (int j = 0; j < DPT; ++j) sym[j] = (id[j] >= 0 && id[j] < a.vocab) ? id[j] : -1;
  }
}

// kLenChunks chunks per workgroup: DPT IDs per thread and chunk, all loaded
// together.
constexpr int kLenChunks = 2;
__global__ void __launch_bounds__(DWG) k_dec_len(DecodeArgs a) {
  constexpr int LPT = kLenChunks * DPT;  // IDs per thread: chunk j / DPT
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kLenChunks;
  const int64_t i0 = c0 * kDecChunk;
  const int cnt = (int)min<int64_t>(kLenChunks * kDecChunk, a.n_ids - i0);
  bool bad_id = false;
  int64_t mine[kLenChunks] = {};
  // consecutive threads read consecutive IDs; every load is unconditional
  // (the workgroup's last ID again past its end, symbol 0 for an ID with
  // none), so that the loads of all LPT IDs are in flight together
  int32_t id[LPT], sym[LPT], len[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) id[j] = a.ids[i0 + min(j * DWG + tid, cnt - 1)];
#pragma unroll
  for (int f = 0; f < kLenChunks; ++f) dec_syms(a, id + f * DPT, sym + f * DPT);
#pragma unroll
  for (int j = 0; j < LPT; ++j) len[j] = a.exp_len[max(sym[j], 0)];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    if (j * DWG + tid >= cnt) continue;
    // a reserved ID given as skip0 / skip1 decodes to no bytes (k_dec_write
    // writes none for an ID with no symbol)
    if (sym[j] >= 0) mine[j / DPT] += len[j];
    else if (!((a.skip0 >= 0 && id[j] == a.skip0) || (a.skip1 >= 0 && id[j] == a.skip1)))
      bad_id = true;
  }
  // the ID offsets check, spread over the grid (after the loads above)
  bool bad_off = false;
  {
    const int64_t per = a.doc_per;
    const int64_t d0 = c0 * per;
    for (int64_t i = d0 + tid; i < min(d0 + kLenChunks * per, a.n_docs + 1); i += DWG) {
      const int64_t v = a.id_off[i];
      if (i == 0 && v != 0) bad_off = true;
      if (i == a.n_docs && v != a.n_ids) bad_off = true;
      if (i < a.n_docs && a.id_off[i + 1] < v) bad_off = true;
    }
  }
  // per chunk: the wave totals (lane 63 of each inclusive sum) and the
  // waves' status bits through LDS, one barrier
  __shared__ int64_t wtot[DWG / 64][kLenChunks];
  __shared__ int32_t wbits[DWG / 64];
  const int wv = wave_id();
  int64_t inc[kLenChunks];
#pragma unroll
  for (int f = 0; f < kLenChunks; ++f) inc[f] = wave_incl_sum(mine[f]);
  const int bits = (__ballot(bad_id) ? (int)BPE_STATUS_BAD_ID : 0) |
                   (__ballot(bad_off) ? (int)BPE_STATUS_BAD_ID_OFFSETS : 0);
  if (lane_id() == 63) {
#pragma unroll
    for (int f = 0; f < kLenChunks; ++f) wtot[wv][f] = inc[f];
    wbits[wv] = bits;
  }
  __syncthreads();
  if (tid < kLenChunks && c0 + tid < a.n_chunks) {
    int64_t t = 0;
    int b = 0;
#pragma unroll
    for (int w = 0; w < DWG / 64; ++w) t += wtot[w][tid], b |= wbits[w];
    a.tot[c0 + tid] = t | ((int64_t)(tid == 0 ? b : 0) << kCountBits);
  }
  // the first document whose IDs start at or after each chunk's (and, after
  // the last chunk, after the last ID): the documents that start in each
  // chunk.  Searched last: nothing above waits on it.
  if (wv < kLenChunks) {
    if (c0 + wv < a.n_chunks) {
      const int64_t d = wave_lower_bound(a.id_off, a.n_docs + 1, (c0 + wv) * kDecChunk);
      if (lane_id() == 0) a.dlo[c0 + wv] = d;
    }
  } else if (wv == kLenChunks && c0 + kLenChunks >= a.n_chunks) {
    const int64_t d = wave_lower_bound(a.id_off, a.n_docs + 1, a.n_ids);
    if (lane_id() == 0) a.dlo[a.n_chunks] = d;
  }
}

__global__ void __launch_bounds__(kScanBlock) k_dec_scan(DecodeArgs a) {
  block_offsets(a.tot, a.off, a.bsum, a.n_chunks);
}

// A chunk's output offset is off[c] + boff[c / kScanBlock].
__global__ void __launch_bounds__(SWG) k_dec_bscan(DecodeArgs a) {
  __shared__ int64_t red64[SWG / 64];
  chunk_offsets<SWG>(a.bsum, a.boff, (a.n_chunks + kScanBlock - 1) / kScanBlock, a.status, red64);
}

// OR the expansion bytes b (zero from byte len on, len <= 16) into the
// zeroed LDS stage at byte offset w: up to five 32-bit words, shifted across
// word boundaries (tokens never overlap, so every byte is ORed once).
__device__ __forceinline__ void stage_or16(uint32_t *stage32, int w, uint4 b, int len) {
  const uint32_t sh = 32u - 8u * (uint32_t)(w & 3);  // 32: already aligned
  const int nw = ((w & 3) + len + 3) >> 2;
  uint32_t *d = stage32 + (w >> 2);
  auto word = [sh](uint32_t hi, uint32_t lo) {
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
  };
  atomicOr(d, word(b.x, 0u));
  if (nw > 1) atomicOr(d + 1, word(b.y, b.x));
  if (nw > 2) atomicOr(d + 2, word(b.z, b.y));
  if (nw > 3) atomicOr(d + 3, word(b.w, b.z));
  if (nw > 4) atomicOr(d + 4, word(0u, b.w));
}

constexpr int kDecStage = 8192;   // output bytes a chunk may stage in LDS

struct WriteShared {
  int32_t len[kDecChunk];
  int64_t excl[DWG];
  int64_t red64[DWG / 64];
  alignas(16) uint32_t stage32[(kDecStage + 16) / 4];
};

__global__ void __launch_bounds__(DWG) k_dec_write(DecodeArgs a) {
  __shared__ WriteShared s;
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t i0 = c * kDecChunk;
  const int cnt = (int)min<int64_t>(kDecChunk, a.n_ids - i0);
  const int64_t base = a.off[c] + a.boff[c / kScanBlock];
  const int64_t o_lo = a.dlo[c], o_hi = max(o_lo, a.dlo[c + 1]);
  for (int i = tid; i < (kDecStage + 16) / 4; i += DWG) s.stage32[i] = 0u;
  // each thread takes DPT IDs in a row: their symbols, lengths and first 16
  // bytes, all loads in flight together (lengths also to LDS for the
  // document offsets)
  const int k0 = tid * DPT;
  int32_t id[DPT], sym[DPT], len[DPT];
  if (k0 + DPT <= cnt && ((reinterpret_cast<uintptr_t>(a.ids + i0 + k0) & 15u) == 0)) {
    // the thread's four IDs in one 16-byte load
    const int4 p = *reinterpret_cast<const int4 *>(a.ids + i0 + k0);
    id[0] = p.x, id[1] = p.y, id[2] = p.z, id[3] = p.w;
  } else {
#pragma unroll
    for (int j = 0; j < DPT; ++j) id[j] = a.ids[i0 + min(k0 + j, cnt - 1)];
  }
  dec_syms(a, id, sym);
#pragma unroll
  for (int j = 0; j < DPT; ++j)
    if (k0 + j >= cnt) sym[j] = -1;
  // (unconditional loads, symbol 0 for an ID with none: they stay in flight
  // together)
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int32_t n = a.exp_len[max(sym[j], 0)];
    len[j] = sym[j] >= 0 ? n : 0;
  }
  // (named values, not an array: an array of them ends up in scratch; these
  // loads stay conditional: unconditional ones took the kernel past 128
  // VGPRs, to three waves per SIMD)
  auto first16 = [&a](int32_t v) { return v >= 0 ? a.exp16[v] : uint4{0u, 0u, 0u, 0u}; };
  static_assert(DPT == 4, "four IDs per thread");
  const uint4 b0 = first16(sym[0]), b1 = first16(sym[1]), b2 = first16(sym[2]),
              b3 = first16(sym[3]);
  int64_t mine = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    s.len[k0 + j] = len[j];
    mine += len[j];
  }
  int64_t total;
  const int64_t ex = block_excl_sum<int64_t, DWG>(mine, s.red64, &total);
  s.excl[tid] = ex;
  bool overflow = false;
  if (total <= kDecStage) {
    // stage the bytes in LDS at the output's 16-byte phase, then write whole
    // aligned 16-byte blocks (bytes at the two ends)
    const int lead = (int)(((uintptr_t)(a.out + base)) & 15u);
    int w = lead + (int)ex;
    bool longer = false;
    auto put = [&](uint4 b, int32_t n) {
      if (n > 0 && n <= 16) stage_or16(s.stage32, w, b, n);
      longer |= n > 16;
      w += n;
    };
    put(b0, len[0]);
    put(b1, len[1]);
    put(b2, len[2]);
    put(b3, len[3]);
    if (longer) {  // expansions of more than 16 bytes: up to 32 from the two
                   // 16-byte tables, longer ones byte by byte
      w = lead + (int)ex;
      for (int j = 0; j < DPT; ++j) {
        const int32_t n = len[j];
        if (n > 32) {
          const uint8_t *src = a.exp_bytes + a.exp_off[sym[j]];
          for (int q = 0; q < n; ++q)
            atomicOr(&s.stage32[(w + q) >> 2], (uint32_t)src[q] << (8 * ((w + q) & 3)));
        } else if (n > 16) {
          stage_or16(s.stage32, w, a.exp16[sym[j]], 16);
          stage_or16(s.stage32, w + 16, a.exp16b[sym[j]], n - 16);
        }
        w += n;
      }
    }
    __syncthreads();
    const uint8_t *stage = reinterpret_cast<const uint8_t *>(s.stage32);
    const int nblk = (lead + (int)total + 15) >> 4;
    uint8_t *g0 = a.out + base - lead;  // 16-byte aligned
    for (int blk = tid; blk < nblk; blk += DWG) {
      const int lo = 16 * blk;
      const int64_t gpos = base - lead + lo;  // output index of stage[lo]
      if (lo >= lead && lo + 16 <= lead + (int)total && gpos + 16 <= a.out_cap) {
        *reinterpret_cast<u32x4 *>(g0 + lo) = *reinterpret_cast<const u32x4 *>(&stage[lo]);
      } else {
        for (int q = max(lo, lead); q < min(lo + 16, lead + (int)total); ++q) {
          if (base - lead + q < a.out_cap) g0[q] = stage[q];
          else overflow = true;
        }
      }
    }
  } else {
    int64_t w = base + ex;
    for (int j = 0; j < DPT; ++j) {
      const int k = tid * DPT + j;
      const int32_t len = s.len[k];
      if (len > 0) {
        const int32_t sym = dec_sym(a, a.ids[i0 + k]);
        const uint8_t *src = a.exp_bytes + a.exp_off[sym];
        for (int q = 0; q < len; ++q) {
          if (w + q < a.out_cap) a.out[w + q] = src[q];
          else overflow = true;
        }
      }
      w += len;
    }
  }
  if (overflow) atomicOr(a.status, (int32_t)BPE_STATUS_BYTES_CAPACITY);
  __syncthreads();
  for (int64_t d = o_lo + tid; d < o_hi; d += DWG) {
    const int64_t k64 = a.id_off[d] - i0;
    const int k = (int)min<int64_t>(max<int64_t>(k64, 0), kDecChunk - 1);
    const int t = k / DPT;
    int64_t before = s.excl[t];
    for (int q = t * DPT; q < k; ++q) before += s.len[q];
    a.byte_off[d] = base + before;
  }
  if (c == a.n_chunks - 1)
    for (int64_t d = o_hi + tid; d <= a.n_docs; d += DWG) a.byte_off[d] = base + total;
}

}  // namespace

const char *const kDecStageNames[kDecStages] = {"k_dec_len", "k_dec_scan", "k_dec_bscan",
                                                "k_dec_write"};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, hipEvent_t *ev) {
  const unsigned G = (unsigned)a.n_chunks;
  if (ev) (void)hipEventRecord(ev[0], stream);
  hipLaunchKernelGGL(k_dec_len, dim3((G + kLenChunks - 1) / kLenChunks), dim3(DWG), 0, stream, a);
  if (ev) (void)hipEventRecord(ev[1], stream);
  hipLaunchKernelGGL(k_dec_scan, dim3((G + kScanBlock - 1) / kScanBlock), dim3(kScanBlock), 0,
                     stream, a);
  if (ev) (void)hipEventRecord(ev[2], stream);
  hipLaunchKernelGGL(k_dec_bscan, dim3(1), dim3(SWG), 0, stream, a);
  if (ev) (void)hipEventRecord(ev[3], stream);
  hipLaunchKernelGGL(k_dec_write, dim3(G), dim3(DWG), 0, stream, a);
  if (ev) (void)hipEventRecord(ev[4], stream);
  return hipGetLastError();
}

}  // namespace bpe
