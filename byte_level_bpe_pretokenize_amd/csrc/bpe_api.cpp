// bpe_api.cpp -- host side of libbpe: model building, checks, launches.
//
// The model is the merge table of "Tokenization LLM: ... C++"
// (glitch4techs.com), sections "BPE algorithm" and "Vocabulary lookup",
// uploaded once to the device as "Hugging Face Tokenizers v1" (dothoosh.com)
// section "Road to 1.0.0" proposes for GPU batch encoding.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/bpe.h"
#include "bpe_internal.h"

using namespace bpe;

struct bpe_model {
  int64_t R = 0, V = 0;
  int device = 0;
  uint64_t *d_table = nullptr;     // rank table, 2 slots per bucket
  uint32_t table_mask = 0, table_seed = 0;
  int32_t *d_id_map = nullptr;
  int32_t *d_pair_rank = nullptr;   // [65536] ranks of byte pairs
  uint32_t *d_pair_filter = nullptr;  // [kPairFilterWords] bit set of the merges' pairs
  int n_cu = 1;                     // compute units of the device
  uint4 *d_words = nullptr;         // short word table (one uint4 per slot), or nullptr
  uint8_t *d_word_disp = nullptr;   // its displacements, one per bucket of keys
  uint32_t word_mask = 0, word_dshift = 32;
  uint4 *d_lwords = nullptr;        // long word table (two uint4 per slot), or nullptr
  uint32_t lword_mask = 0, lword_seed = 0;
  uint32_t word_seed = 0;
  int64_t n_words = 0;
  // decode tables
  bool decode_ok = false;
  int64_t max_token = 1;
  int64_t *d_exp_off = nullptr;
  uint8_t *d_exp_bytes = nullptr;
  uint4 *d_exp16 = nullptr;     // first 16 bytes of each expansion, zero padded
  uint4 *d_exp16b = nullptr;    // its bytes 16..31, zero padded
  int32_t *d_exp_len = nullptr;
  int32_t *d_inv_map = nullptr;
  int64_t inv_size = 0;
  int32_t win_d[4] = {0, 0, 0, 0};  // window radii by pre-token class (EncodeArgs::win_d)
  std::vector<uint64_t> used;       // with an id_map: bit x set when x is a symbol's output ID
  // stage timing (bpe_stage_timing): events of the calls not yet read, per
  // op, stages + 1 per call; spare events for reuse
  bool timing = false;
  mutable std::vector<hipEvent_t> rec[2];
  mutable std::vector<hipEvent_t> spare;
};

namespace {

constexpr int kStages[2] = {kEncStages, kDecStages};

void drop_events(bpe_model *m) {
  for (auto &r : m->rec) {
    m->spare.insert(m->spare.end(), r.begin(), r.end());
    r.clear();
  }
}

// Events for one timed call of op (nullptr when timing is off or events run out).
hipEvent_t *call_events(const bpe_model *m, int op) {
  if (!m->timing) return nullptr;
  const int n = kStages[op] + 1;
  std::vector<hipEvent_t> &r = m->rec[op];
  for (int i = 0; i < n; ++i) {
    hipEvent_t e = nullptr;
    if (!m->spare.empty()) {
      e = m->spare.back();
      m->spare.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      // give back what this call took
      m->spare.insert(m->spare.end(), r.end() - i, r.end());
      r.resize(r.size() - i);
      return nullptr;
    }
    r.push_back(e);
  }
  return r.data() + r.size() - n;
}

void free_model(bpe_model *m) {
  if (!m) return;
  drop_events(m);
  for (hipEvent_t e : m->spare) (void)hipEventDestroy(e);
  if (m->d_table) (void)hipFree(m->d_table);
  if (m->d_id_map) (void)hipFree(m->d_id_map);
  if (m->d_pair_rank) (void)hipFree(m->d_pair_rank);
  if (m->d_pair_filter) (void)hipFree(m->d_pair_filter);
  if (m->d_words) (void)hipFree(m->d_words);
  if (m->d_word_disp) (void)hipFree(m->d_word_disp);
  if (m->d_lwords) (void)hipFree(m->d_lwords);
  if (m->d_exp_off) (void)hipFree(m->d_exp_off);
  if (m->d_exp_bytes) (void)hipFree(m->d_exp_bytes);
  if (m->d_exp16) (void)hipFree(m->d_exp16);
  if (m->d_exp16b) (void)hipFree(m->d_exp16b);
  if (m->d_exp_len) (void)hipFree(m->d_exp_len);
  if (m->d_inv_map) (void)hipFree(m->d_inv_map);
  delete m;
}

template <typename T>
int upload(T **dst, const T *src, size_t count, hipStream_t stream) {
  if (count == 0) count = 1;
  if (hipMalloc((void **)dst, count * sizeof(T)) != hipSuccess) {
    *dst = nullptr;
    return BPE_ENOMEM;
  }
  if (src && hipMemcpyAsync(*dst, src, count * sizeof(T), hipMemcpyHostToDevice, stream) !=
                 hipSuccess)
    return BPE_EHIP;
  return BPE_OK;
}



bool on_model_device(const bpe_model *m) {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == m->device;
}

// Queue the encode kernels.  `words`: use the model's word tables (else every
// pre-token runs the merge loop); `id_map` the output mapping.
int enqueue_encode(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                   const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids, int64_t ids_capacity,
                   int64_t *d_id_off, void *d_workspace, int32_t *d_status, bool words,
                   const int32_t *id_map, hipStream_t stream, int32_t bos = -1,
                   int32_t eos = -1, bool timed = true) {
  if (n_bytes == 0)
    return launch_empty(d_doc_off, n_docs, BPE_STATUS_BAD_DOC_OFFSETS, d_id_off, d_status,
                        stream) == hipSuccess
               ? BPE_OK
               : BPE_EHIP;
  const EncLayout L = enc_layout(n_bytes, n_docs);
  uint8_t *ws = (uint8_t *)d_workspace;
  EncodeArgs a;
  a.bytes = d_bytes;
  a.n_bytes = n_bytes;
  a.doc_off = d_doc_off;
  a.n_docs = n_docs;
  a.ids = d_ids;
  a.ids_cap = ids_capacity;
  a.id_off = d_id_off;
  a.table = model->d_table;
  a.table_mask = model->table_mask;
  a.table_seed = model->table_seed;
  a.id_map = id_map;
  a.pair_rank = model->d_pair_rank;
  a.pair_filter = model->d_pair_filter;
  a.n_cu = model->n_cu;
  a.lgroup = 1;  // the launch picks the merge kernels' group size
  a.words = words ? model->d_words : nullptr;
  a.word_disp = model->d_word_disp;
  a.word_mask = model->word_mask;
  a.word_seed = model->word_seed;
  a.word_dshift = model->word_dshift;
  a.lwords = words ? model->d_lwords : nullptr;
  a.lword_mask = model->lword_mask;
  a.lword_seed = model->lword_seed;
  a.meta = (int32_t *)(ws + L.meta);
  a.tot = (int64_t *)(ws + L.tot);
  a.off = (int64_t *)(ws + L.off);
  a.bsum = (int64_t *)(ws + L.bsum);
  a.boff = (int64_t *)(ws + L.boff);
  a.doc_rng = (int64_t *)(ws + L.doc_rng);
  a.dfirst = (int64_t *)(ws + L.dfirst);
  a.doc_pt = (int32_t *)(ws + L.doc_pt);
  a.pv = (int32_t *)(ws + L.pv);
  a.cntk = ws + L.cntk;
  a.miss = (uint32_t *)(ws + L.miss);
  a.mt = (int32_t *)(ws + L.mt);
  a.mbytes = ws + L.mbytes;
  a.dref = (uint32_t *)(ws + L.dref);
  a.olist = (uint64_t *)(ws + L.olist);
  a.dstat = (uint32_t *)(ws + L.dstat);
  a.dt = (unsigned long long *)(ws + L.dt);
  a.dt_mask = (uint32_t)(dedup_slots((size_t)enc_chunks(n_bytes)) - 1);
  a.dedup = enc_chunks(n_bytes) <= kDedupMaxChunks ? 1 : 0;
  a.res = (int32_t *)(ws + L.res);
  a.gsym = (int32_t *)(ws + L.gsym);
  a.grank = (int32_t *)(ws + L.grank);
  a.status = d_status;
  a.n_chunks = enc_chunks(n_bytes);
  a.doc_per = (n_docs + 1 + a.n_chunks - 1) / a.n_chunks;
  for (int k = 0; k < 4; ++k) a.win_d[k] = model->win_d[k];
  a.bos = bos;
  a.eos = eos;
  if (launch_encode(a, stream, timed ? call_events(model, BPE_OP_ENCODE) : nullptr) != hipSuccess)
    return BPE_EHIP;
  return BPE_OK;
}

}  // namespace

namespace bpe {

int encode_checked(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                   const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids, int64_t ids_capacity,
                   int64_t *d_id_off, void *d_workspace, size_t workspace_bytes, int32_t *d_status,
                   void *hip_stream, bool timed) {
  if (!model || n_bytes < 0 || n_docs < 0 || ids_capacity < 0 || !d_doc_off || !d_id_off ||
      !d_status || (ids_capacity > 0 && !d_ids) || (n_bytes > 0 && (!d_bytes || !d_workspace)))
    return BPE_EINVAL;
  // a launch holds at most 2^32 - 1 work-items
  if (enc_chunks(n_bytes) * kEncThreads > (int64_t)UINT32_MAX) return BPE_EINVAL;
  if (!on_model_device(model)) return BPE_EINVAL;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (n_bytes > 0 && workspace_bytes < enc_layout(n_bytes, n_docs).total) return BPE_EWORKSPACE;
  return enqueue_encode(model, d_bytes, n_bytes, d_doc_off, n_docs, d_ids, ids_capacity, d_id_off,
                        d_workspace, d_status, true, model->d_id_map, stream, -1, -1, timed);
}

int model_device(const bpe_model *model) { return model ? model->device : -1; }

}  // namespace bpe

namespace {



// The word table: every symbol whose byte expansion (2..kWordMax bytes)
// encodes to exactly that symbol.  The expansions are encoded on the device
// by the same kernels, with the merge loop for every pre-token; the host only
// arranges the results into the hash table.
int build_word_table(bpe_model *m, const std::vector<int64_t> &exp_off,
                     const std::vector<uint8_t> &exp_bytes, hipStream_t stream) {
  std::vector<int32_t> cand;
  std::vector<int64_t> doc_off(1, 0);
  for (int64_t v = 256; v < m->V; ++v) {
    const int64_t n = exp_off[(size_t)v + 1] - exp_off[(size_t)v];
    if (n >= 2 && n <= kWordMax) {
      cand.push_back((int32_t)v);
      doc_off.push_back(doc_off.back() + n);
    }
  }
  if (cand.empty()) return BPE_OK;
  const int64_t N = doc_off.back(), D = (int64_t)cand.size();
  std::vector<uint8_t> text((size_t)N);
  for (int64_t k = 0; k < D; ++k) {
    const int64_t v = cand[(size_t)k];
    std::memcpy(&text[(size_t)doc_off[(size_t)k]], &exp_bytes[(size_t)exp_off[(size_t)v]],
                (size_t)(doc_off[(size_t)k + 1] - doc_off[(size_t)k]));
  }
  const EncLayout L = enc_layout(N, D);
  uint8_t *d_text = nullptr, *d_ws = nullptr;
  int64_t *d_doc = nullptr, *d_ioff = nullptr;
  int32_t *d_ids = nullptr, *d_status = nullptr;
  int rc = BPE_OK;
  if (hipMalloc((void **)&d_text, (size_t)N) != hipSuccess ||
      hipMalloc((void **)&d_doc, sizeof(int64_t) * (size_t)(D + 1)) != hipSuccess ||
      hipMalloc((void **)&d_ioff, sizeof(int64_t) * (size_t)(D + 1)) != hipSuccess ||
      hipMalloc((void **)&d_ids, sizeof(int32_t) * (size_t)N) != hipSuccess ||
      hipMalloc((void **)&d_status, sizeof(int32_t)) != hipSuccess ||
      hipMalloc((void **)&d_ws, L.total) != hipSuccess)
    rc = BPE_ENOMEM;
  std::vector<int64_t> ioff((size_t)D + 1);
  std::vector<int32_t> ids((size_t)N);
  int32_t status = -1;
  if (rc == BPE_OK &&
      (hipMemcpyAsync(d_text, text.data(), (size_t)N, hipMemcpyHostToDevice, stream) != hipSuccess ||
       hipMemcpyAsync(d_doc, doc_off.data(), sizeof(int64_t) * (size_t)(D + 1),
                      hipMemcpyHostToDevice, stream) != hipSuccess))
    rc = BPE_EHIP;
  if (rc == BPE_OK)
    rc = enqueue_encode(m, d_text, N, d_doc, D, d_ids, N, d_ioff, d_ws, d_status, false,
                        nullptr, stream);
  if (rc == BPE_OK &&
      (hipMemcpyAsync(ioff.data(), d_ioff, sizeof(int64_t) * (size_t)(D + 1), hipMemcpyDeviceToHost,
                      stream) != hipSuccess ||
       hipMemcpyAsync(ids.data(), d_ids, sizeof(int32_t) * (size_t)N, hipMemcpyDeviceToHost,
                      stream) != hipSuccess ||
       hipMemcpyAsync(&status, d_status, sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
           hipSuccess ||
       hipStreamSynchronize(stream) != hipSuccess))
    rc = BPE_EHIP;
  (void)hipFree(d_text);
  (void)hipFree(d_doc);
  (void)hipFree(d_ioff);
  (void)hipFree(d_ids);
  (void)hipFree(d_status);
  (void)hipFree(d_ws);
  if (rc != BPE_OK) return rc;
  if (status != 0) return BPE_EHIP;

  // the entries, split by key length: {len, symbol, key[6]}
  std::vector<std::array<uint32_t, 8>> items[2];
  for (int64_t k = 0; k < D; ++k) {
    if (!(ioff[(size_t)k + 1] - ioff[(size_t)k] == 1 && ids[(size_t)ioff[(size_t)k]] == cand[(size_t)k]))
      continue;
    const int len = (int)(doc_off[(size_t)k + 1] - doc_off[(size_t)k]);
    std::array<uint32_t, 8> it{};
    uint32_t *w = &it[2];
    for (int j = 0; j < len; ++j)
      w[j >> 2] |= (uint32_t)text[(size_t)doc_off[(size_t)k] + j] << (8 * (j & 3));
    it[0] = (uint32_t)len;
    it[1] = (uint32_t)cand[(size_t)k];
    items[len <= kShortMax ? 0 : 1].push_back(it);
  }
  for (int t = 0; t < 2; ++t) {
    const std::vector<std::array<uint32_t, 8>> &its = items[t];
    const int64_t n_keep = (int64_t)its.size();
    if (n_keep == 0) continue;
    // capacity a power of two >= 2 entries (short table) or >= 2.5 (long
    // table); on failure another seed, then twice the capacity; after that
    // without this table (its pre-tokens then run the merge loop, with the
    // same result)
    uint32_t mask = 255;
    while ((int64_t)mask + 1 < (t == 0 ? 2 * n_keep : 5 * n_keep / 2)) mask = 2 * mask + 1;
    std::vector<int32_t> at;
    std::vector<uint8_t> disp;
    std::vector<uint32_t> hs((size_t)n_keep), st((size_t)n_keep);
    uint32_t seed = 0;
    int dbits = 0;
    bool placed = false;
    for (int attempt = 0; attempt < 8 && !placed; ++attempt) {
      seed = 0x9E3779B9u * (uint32_t)(attempt + 1);
      for (int64_t e = 0; e < n_keep; ++e) {
        const uint32_t *w = &its[(size_t)e][2];
        const int len = (int)its[(size_t)e][0];
        hs[(size_t)e] = t == 0 ? short_mix(w[0], w[1], w[2], (uint32_t)len, seed)
                               : word_hash(w, len, seed);
        if (t == 0) st[(size_t)e] = short_step(w[0], w[1], w[2]);
      }
      if (t == 0) {
        dbits = 0;
        while (((uint64_t)kShortSlotsPerDisp << dbits) < (uint64_t)mask + 1) ++dbits;
        placed = place_displaced(hs, st, mask, dbits, at, disp);
      } else {
        placed = place_words(hs, mask, at);
      }
      if (!placed && attempt % 2 == 1) mask = 2 * mask + 1;
    }
    if (!placed) continue;
    std::vector<uint32_t> flag((size_t)mask + 1, 0u);
    if (t == 1)
      for (uint32_t i = 0; i <= mask; ++i)
        if (at[i] >= 0 && word_slot0(hs[(size_t)at[i]], mask) != i)
          flag[word_slot0(hs[(size_t)at[i]], mask)] = kWordFlag;
    const int words_per_slot = t == 0 ? 4 : 8;
    std::vector<uint32_t> slots((size_t)words_per_slot * ((size_t)mask + 1), 0u);
    for (uint32_t i = 0; i <= mask; ++i) {
      uint32_t *o = &slots[(size_t)words_per_slot * i];
      if (at[i] < 0) {
        if (t == 0) o[3] = flag[i];
        else o[1] = flag[i];
        continue;
      }
      const std::array<uint32_t, 8> &it = its[(size_t)at[i]];
      const uint32_t len = it[0], sym = it[1];
      if (t == 0) {
        o[0] = it[2];
        o[1] = it[3];
        o[2] = it[4];
        o[3] = sym | (len << 21) | flag[i];
      } else {
        o[0] = word_tag(hs[(size_t)at[i]], (int)len);
        o[1] = sym | flag[i];
        for (int j = 0; j < 6; ++j) o[2 + j] = it[2 + (size_t)j];
      }
    }
    uint4 **dst = t == 0 ? &m->d_words : &m->d_lwords;
    rc = upload(reinterpret_cast<uint32_t **>(dst), slots.data(), slots.size(), stream);
    if (rc != BPE_OK) return rc;
    if (t == 0) {
      rc = upload(&m->d_word_disp, disp.data(), disp.size(), stream);
      if (rc != BPE_OK) return rc;
      m->word_mask = mask;
      m->word_seed = seed;
      m->word_dshift = (uint32_t)(32 - dbits);
    } else {
      m->lword_mask = mask;
      m->lword_seed = seed;
    }
    m->n_words += n_keep;
  }
  return BPE_OK;
}

}  // namespace

extern "C" {

int bpe_load_merges(const int32_t *merges, int64_t n_merges, const int32_t *id_map,
                    void *hip_stream, bpe_model **out) {
  if (!out || n_merges < 0 || n_merges > BPE_MAX_MERGES || (n_merges > 0 && !merges))
    return BPE_EINVAL;
  const int64_t R = n_merges, V = 256 + n_merges;
  hipStream_t stream = (hipStream_t)hip_stream;

  // operands in range, pairs distinct
  std::vector<uint64_t> keys((size_t)R);
  for (int64_t r = 0; r < R; ++r) {
    const int64_t l = merges[2 * r], rt = merges[2 * r + 1];
    if (l < 0 || l >= V || rt < 0 || rt >= V) return BPE_EMERGES;
    keys[(size_t)r] = pair_key((uint32_t)l, (uint32_t)rt);
  }
  {
    std::vector<uint64_t> sorted(keys);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return BPE_EMERGES;
  }

  // Operands before the symbols built from them (Kahn's order); symbols left
  // unordered lie on a cycle.  Byte lengths follow in the same order.
  std::vector<int64_t> len((size_t)V, 1);
  std::vector<int64_t> order;
  order.reserve((size_t)R);
  {
    std::vector<int32_t> indeg((size_t)R, 0);
    std::vector<int64_t> ustart((size_t)V + 1, 0);
    for (int64_t r = 0; r < R; ++r)
      for (int k = 0; k < 2; ++k) {
        const int32_t u = merges[2 * r + k];
        if (u >= 256) {
          ++indeg[(size_t)r];
          ++ustart[(size_t)u + 1];
        }
      }
    for (int64_t v = 0; v < V; ++v) ustart[(size_t)v + 1] += ustart[(size_t)v];
    std::vector<int32_t> users((size_t)ustart[(size_t)V]);
    std::vector<int64_t> fill(ustart.begin(), ustart.end() - 1);
    for (int64_t r = 0; r < R; ++r)
      for (int k = 0; k < 2; ++k) {
        const int32_t u = merges[2 * r + k];
        if (u >= 256) users[(size_t)fill[(size_t)u]++] = (int32_t)(256 + r);
      }
    std::vector<int64_t> queue;
    queue.reserve((size_t)R);
    for (int64_t r = 0; r < R; ++r)
      if (indeg[(size_t)r] == 0) queue.push_back(256 + r);
    const int64_t cap = (int64_t)1 << 62;
    for (size_t qi = 0; qi < queue.size(); ++qi) {
      const int64_t v = queue[qi];
      const int64_t r = v - 256;
      len[(size_t)v] = std::min(cap, len[(size_t)merges[2 * r]] + len[(size_t)merges[2 * r + 1]]);
      order.push_back(v);
      for (int64_t k = ustart[(size_t)v]; k < ustart[(size_t)v + 1]; ++k) {
        const int32_t w = users[(size_t)k];
        if (--indeg[(size_t)(w - 256)] == 0) queue.push_back(w);
      }
    }
    if ((int64_t)order.size() != R) return BPE_EMERGES;
  }

  // id_map: distinct values in [0, BPE_MAX_ID]
  int64_t max_id = V - 1;
  if (id_map) {
    std::vector<uint8_t> seen((size_t)BPE_MAX_ID + 1, 0);
    max_id = 0;
    for (int64_t v = 0; v < V; ++v) {
      const int32_t x = id_map[v];
      if (x < 0 || x > BPE_MAX_ID || seen[(size_t)x]) return BPE_EIDMAP;
      seen[(size_t)x] = 1;
      max_id = std::max<int64_t>(max_id, x);
    }
  }

  // rank table: buckets of two slots, a power-of-two count >= R (load <= 1/2);
  // on failure another seed, then twice the buckets
  uint32_t tmask = 1;
  while ((int64_t)tmask + 1 < R) tmask = 2 * tmask + 1;
  std::vector<uint64_t> table;
  uint32_t tseed = 0;
  for (int attempt = 0;; ++attempt) {
    if (tmask >= (1u << 30)) return BPE_ENOMEM;
    tseed = 0x9E3779B9u * (uint32_t)(attempt + 1);
    if (build_rank_table(keys, tmask, tseed, table)) break;
    if (attempt % 2 == 1) tmask = 2 * tmask + 1;
  }

  bpe_model *m = new (std::nothrow) bpe_model;
  if (!m) return BPE_ENOMEM;
  m->R = R;
  m->V = V;
  if (id_map) {
    m->used.assign(((size_t)max_id + 64) / 64, 0ull);
    for (int64_t v = 0; v < V; ++v) m->used[(size_t)id_map[v] >> 6] |= 1ull << (id_map[v] & 63);
  }
  window_radii(merges, R, len, order, m->win_d);
  m->table_mask = tmask;
  m->table_seed = tseed;
  if (hipGetDevice(&m->device) != hipSuccess) {
    delete m;
    return BPE_EHIP;
  }
  int rc = upload(&m->d_table, table.data(), table.size(), stream);
  if (rc == BPE_OK && id_map) rc = upload(&m->d_id_map, id_map, (size_t)V, stream);
  if (rc == BPE_OK) {
    std::vector<int32_t> pr((size_t)65536, kRankInf);
    for (int64_t r = 0; r < R; ++r)
      if (merges[2 * r] < 256 && merges[2 * r + 1] < 256)
        pr[(size_t)(merges[2 * r] * 256 + merges[2 * r + 1])] = (int32_t)r;
    rc = upload(&m->d_pair_rank, pr.data(), pr.size(), stream);
    if (rc == BPE_OK) {
      std::vector<uint32_t> pf((size_t)kPairFilterWords, 0u);
      for (int64_t r = 0; r < R; ++r) {
        const uint32_t k = pair_filter_bit(
            pair_mix((uint32_t)merges[2 * r], (uint32_t)merges[2 * r + 1], tseed));
        pf[k >> 5] |= 1u << (k & 31);
      }
      rc = upload(&m->d_pair_filter, pf.data(), pf.size(), stream);
    }
  }
  if (rc == BPE_OK) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, m->device) != hipSuccess)
      rc = BPE_EHIP;
    m->n_cu = cu > 0 ? cu : 1;
  }

  // decode tables: byte expansion of every symbol, and the ID -> symbol map
  int64_t total = 0;
  for (int64_t v = 0; v < V && total <= BPE_MAX_EXPANSION; ++v) total += len[(size_t)v];
  std::vector<int64_t> exp_off;
  std::vector<uint8_t> exp_bytes;
  std::vector<int32_t> inv;
  if (rc == BPE_OK && total <= BPE_MAX_EXPANSION) {
    exp_off.resize((size_t)V + 1);
    exp_off[0] = 0;
    for (int64_t v = 0; v < V; ++v) exp_off[(size_t)v + 1] = exp_off[(size_t)v] + len[(size_t)v];
    exp_bytes.resize((size_t)std::max<int64_t>(1, total));
    for (int64_t b = 0; b < 256; ++b) exp_bytes[(size_t)exp_off[(size_t)b]] = (uint8_t)b;
    for (int64_t v : order) {
      const int64_t r = v - 256;
      const int32_t l = merges[2 * r], rt = merges[2 * r + 1];
      uint8_t *dst = &exp_bytes[(size_t)exp_off[(size_t)v]];
      std::memcpy(dst, &exp_bytes[(size_t)exp_off[(size_t)l]], (size_t)len[(size_t)l]);
      std::memcpy(dst + len[(size_t)l], &exp_bytes[(size_t)exp_off[(size_t)rt]],
                  (size_t)len[(size_t)rt]);
    }
    m->max_token = *std::max_element(len.begin(), len.end());
    rc = upload(&m->d_exp_off, exp_off.data(), exp_off.size(), stream);
    if (rc == BPE_OK) rc = upload(&m->d_exp_bytes, exp_bytes.data(), exp_bytes.size(), stream);
    if (rc == BPE_OK) {
      std::vector<uint4> e16((size_t)V), e16b((size_t)V);
      std::vector<int32_t> elen((size_t)V);
      for (int64_t v = 0; v < V; ++v) {
        uint8_t w[32] = {};
        std::memcpy(w, &exp_bytes[(size_t)exp_off[(size_t)v]],
                    (size_t)std::min<int64_t>(32, len[(size_t)v]));
        std::memcpy(&e16[(size_t)v], w, 16);
        std::memcpy(&e16b[(size_t)v], w + 16, 16);
        elen[(size_t)v] = (int32_t)len[(size_t)v];
      }
      rc = upload(&m->d_exp16, e16.data(), e16.size(), stream);
      if (rc == BPE_OK) rc = upload(&m->d_exp16b, e16b.data(), e16b.size(), stream);
      if (rc == BPE_OK) rc = upload(&m->d_exp_len, elen.data(), elen.size(), stream);
    }
    if (rc == BPE_OK && id_map) {
      inv.assign((size_t)max_id + 1, -1);
      for (int64_t v = 0; v < V; ++v) inv[(size_t)id_map[v]] = (int32_t)v;
      m->inv_size = max_id + 1;
      rc = upload(&m->d_inv_map, inv.data(), inv.size(), stream);
    }
    m->decode_ok = rc == BPE_OK;
    if (rc == BPE_OK) rc = build_word_table(m, exp_off, exp_bytes, stream);
  }
  if (rc == BPE_OK && hipStreamSynchronize(stream) != hipSuccess) rc = BPE_EHIP;
  if (rc != BPE_OK) {
    (void)hipStreamSynchronize(stream);
    free_model(m);
    return rc;
  }
  *out = m;
  return BPE_OK;
}

void bpe_free(bpe_model *model) { free_model(model); }

int64_t bpe_vocab_size(const bpe_model *model) { return model ? model->V : -1; }

int64_t bpe_max_token_bytes(const bpe_model *model) {
  return (model && model->decode_ok) ? model->max_token : -1;
}

size_t bpe_encode_workspace_bytes(const bpe_model *model, int64_t n_bytes, int64_t n_docs) {
  (void)model;
  return n_bytes > 0 ? enc_layout(n_bytes, n_docs).total : 0;
}

int bpe_encode_batch(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                     const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids,
                     int64_t ids_capacity, int64_t *d_id_off, void *d_workspace,
                     size_t workspace_bytes, int32_t *d_status, void *hip_stream) {
  return bpe::encode_checked(model, d_bytes, n_bytes, d_doc_off, n_docs, d_ids, ids_capacity,
                             d_id_off, d_workspace, workspace_bytes, d_status, hip_stream, true);
}

namespace {

// Whether id is the output ID of some symbol (so that encoding text can
// produce it).
bool symbol_id(const bpe_model *m, int64_t id) {
  if (m->used.empty()) return id >= 0 && id < m->V;
  return id >= 0 && (size_t)(id >> 6) < m->used.size() && ((m->used[(size_t)(id >> 6)] >> (id & 63)) & 1u);
}

// A reserved ID argument: -1 (none), or in [0, BPE_MAX_ID] and no symbol's ID.
bool reserved_ok(const bpe_model *m, int32_t id) {
  return id == -1 || (id >= 0 && id <= BPE_MAX_ID && !symbol_id(m, id));
}

}  // namespace

size_t bpe_encode_special_workspace_bytes(const bpe_model *model, int64_t n_bytes,
                                          int64_t n_docs) {
  return bpe_encode_workspace_bytes(model, n_bytes, n_docs);
}

int bpe_encode_batch_special(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                             const int64_t *d_doc_off, int64_t n_docs, int32_t bos_id,
                             int32_t eos_id, int32_t *d_ids, int64_t ids_capacity,
                             int64_t *d_id_off, void *d_workspace, size_t workspace_bytes,
                             int32_t *d_status, void *hip_stream) {
  if (!model || n_bytes < 0 || n_docs < 0 || ids_capacity < 0 || !d_doc_off || !d_id_off ||
      !d_status || (ids_capacity > 0 && !d_ids) || (n_bytes > 0 && (!d_bytes || !d_workspace)))
    return BPE_EINVAL;
  if (!reserved_ok(model, bos_id) || !reserved_ok(model, eos_id)) return BPE_EINVAL;
  if (enc_chunks(n_bytes) * kEncThreads > (int64_t)UINT32_MAX) return BPE_EINVAL;
  if ((n_docs + 1 + 255) / 256 > (int64_t)UINT32_MAX) return BPE_EINVAL;
  if (!on_model_device(model)) return BPE_EINVAL;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (n_bytes > 0 && workspace_bytes < enc_layout(n_bytes, n_docs).total) return BPE_EWORKSPACE;
  if (n_bytes > 0 || (bos_id < 0 && eos_id < 0))
    return enqueue_encode(model, d_bytes, n_bytes, d_doc_off, n_docs, d_ids, ids_capacity,
                          d_id_off, d_workspace, d_status, true, model->d_id_map, stream, bos_id,
                          eos_id);
  // an empty input: the offsets checked (and zeroed), then the reserved IDs
  if (launch_empty(d_doc_off, n_docs, BPE_STATUS_BAD_DOC_OFFSETS, d_id_off, d_status, stream) !=
      hipSuccess)
    return BPE_EHIP;
  SpecialArgs a;
  a.n_docs = n_docs;
  a.bos = bos_id;
  a.eos = eos_id;
  a.ids = d_ids;
  a.ids_cap = ids_capacity;
  a.id_off = d_id_off;
  a.status = d_status;
  return launch_special(a, stream) == hipSuccess ? BPE_OK : BPE_EHIP;
}

size_t bpe_decode_workspace_bytes(const bpe_model *model, int64_t n_ids, int64_t n_docs) {
  (void)model;
  (void)n_docs;
  return n_ids > 0 ? dec_layout(n_ids).total : 0;
}

int bpe_decode_batch(const bpe_model *model, const int32_t *d_ids, int64_t n_ids,
                     const int64_t *d_id_off, int64_t n_docs, uint8_t *d_bytes,
                     int64_t bytes_capacity, int64_t *d_byte_off, void *d_workspace,
                     size_t workspace_bytes, int32_t *d_status, void *hip_stream) {
  return bpe_decode_batch_special(model, d_ids, n_ids, d_id_off, n_docs, -1, -1, d_bytes,
                                  bytes_capacity, d_byte_off, d_workspace, workspace_bytes,
                                  d_status, hip_stream);
}

int bpe_decode_batch_special(const bpe_model *model, const int32_t *d_ids, int64_t n_ids,
                             const int64_t *d_id_off, int64_t n_docs, int32_t skip_a,
                             int32_t skip_b, uint8_t *d_bytes, int64_t bytes_capacity,
                             int64_t *d_byte_off, void *d_workspace, size_t workspace_bytes,
                             int32_t *d_status, void *hip_stream) {
  if (model && (!reserved_ok(model, skip_a) || !reserved_ok(model, skip_b))) return BPE_EINVAL;
  if (!model || n_ids < 0 || n_docs < 0 || bytes_capacity < 0 || !d_id_off || !d_byte_off ||
      !d_status || (bytes_capacity > 0 && !d_bytes) || (n_ids > 0 && (!d_ids || !d_workspace)))
    return BPE_EINVAL;
  if (!model->decode_ok) return BPE_ENOTSUP;
  if (dec_chunks(n_ids) * kDecThreads > (int64_t)UINT32_MAX) return BPE_EINVAL;
  if (!on_model_device(model)) return BPE_EINVAL;
  hipStream_t stream = (hipStream_t)hip_stream;
  if (n_ids == 0)
    return launch_empty(d_id_off, n_docs, BPE_STATUS_BAD_ID_OFFSETS, d_byte_off, d_status,
                        stream) == hipSuccess
               ? BPE_OK
               : BPE_EHIP;
  const DecLayout L = dec_layout(n_ids);
  if (workspace_bytes < L.total) return BPE_EWORKSPACE;
  uint8_t *ws = (uint8_t *)d_workspace;
  DecodeArgs a;
  a.ids = d_ids;
  a.n_ids = n_ids;
  a.id_off = d_id_off;
  a.n_docs = n_docs;
  a.out = d_bytes;
  a.out_cap = bytes_capacity;
  a.byte_off = d_byte_off;
  a.exp_off = model->d_exp_off;
  a.exp_bytes = model->d_exp_bytes;
  a.exp16 = model->d_exp16;
  a.exp16b = model->d_exp16b;
  a.exp_len = model->d_exp_len;
  a.inv_map = model->d_inv_map;
  a.inv_size = model->inv_size;
  a.vocab = model->V;
  a.tot = (int64_t *)(ws + L.tot);
  a.off = (int64_t *)(ws + L.off);
  a.bsum = (int64_t *)(ws + L.bsum);
  a.boff = (int64_t *)(ws + L.boff);
  a.dlo = (int64_t *)(ws + L.dlo);
  a.status = d_status;
  a.n_chunks = dec_chunks(n_ids);
  a.doc_per = (n_docs + 1 + a.n_chunks - 1) / a.n_chunks;
  a.skip0 = skip_a;
  a.skip1 = skip_b;
  if (launch_decode(a, stream, call_events(model, BPE_OP_DECODE)) != hipSuccess) return BPE_EHIP;
  return BPE_OK;
}

int bpe_stage_timing(bpe_model *model, int enable) {
  if (!model) return BPE_EINVAL;
  drop_events(model);
  model->timing = enable != 0;
  return BPE_OK;
}

int bpe_stage_count(int op) { return (op == BPE_OP_ENCODE || op == BPE_OP_DECODE) ? kStages[op] : -1; }

const char *bpe_stage_name(int op, int stage) {
  if (op == BPE_OP_ENCODE && stage >= 0 && stage < kEncStages) return kEncStageNames[stage];
  if (op == BPE_OP_DECODE && stage >= 0 && stage < kDecStages) return kDecStageNames[stage];
  return nullptr;
}

int bpe_stage_times(bpe_model *model, int op, double *ms, int max_stages, int64_t *n_calls) {
  if (!model || (op != BPE_OP_ENCODE && op != BPE_OP_DECODE) || !ms || !n_calls ||
      max_stages < kStages[op])
    return BPE_EINVAL;
  const int n = kStages[op] + 1;
  std::vector<hipEvent_t> &r = model->rec[op];
  for (int k = 0; k < kStages[op]; ++k) ms[k] = 0.0;
  int rc = BPE_OK;
  for (size_t c = 0; c + n <= r.size(); c += n) {
    if (hipEventSynchronize(r[c + n - 1]) != hipSuccess) rc = BPE_EHIP;
    for (int k = 0; k < kStages[op] && rc == BPE_OK; ++k) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, r[c + k], r[c + k + 1]) != hipSuccess) rc = BPE_EHIP;
      ms[k] += t;
    }
  }
  *n_calls = (int64_t)(r.size() / n);
  model->spare.insert(model->spare.end(), r.begin(), r.end());
  r.clear();
  return rc;
}

}  // extern "C"

namespace {

// Byte classes of the pre-token start rule, as the encode kernels apply it
// (readings R1-R3): a document start, or a class change unless a single space
// that opens the document or follows a non-whitespace byte leads a letter.
int host_class(uint8_t b) {
  if ((b >= 'A' && b <= 'Z') || (b >= 'a' && b <= 'z') || b >= 0x80) return 0;  // letter
  if (b >= '0' && b <= '9') return 1;                                          // digit
  if ((b >= 0x09 && b <= 0x0D) || b == 0x20) return 2;                         // whitespace
  return 3;                                                                    // punctuation
}

// The distinct pre-tokens of the documents with their frequencies (words in
// order of first appearance): each pre-token's bytes as symbols in sym from
// word_off[w], word_len[w] of them, and the pre-token of each position.  An
// open-addressing table of byte spans (a multiplicative hash of 8-byte
// words, compared with memcmp) finds a pre-token seen before.
void collect_pretokens(const uint8_t *bytes, const int64_t *doc_off, int64_t n_docs,
                       std::vector<int32_t> &sym, std::vector<int32_t> &pos_word,
                       std::vector<int64_t> &word_off, std::vector<int32_t> &word_len,
                       std::vector<int64_t> &word_freq) {
  uint8_t cls[256];
  for (int b = 0; b < 256; ++b) cls[b] = (uint8_t)host_class((uint8_t)b);
  std::vector<const uint8_t *> first;  // each word's bytes (its first occurrence)
  std::vector<uint64_t> hashes;
  std::vector<int32_t> table(1 << 16, -1);
  uint64_t mask = table.size() - 1;
  auto hash_of = [](const uint8_t *p, int64_t n) {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)n;
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
      uint64_t x;
      std::memcpy(&x, p + i, 8);
      h = (h ^ x) * 0xFF51AFD7ED558CCDull;
      h ^= h >> 32;
    }
    uint64_t x = 0;
    for (int64_t k = 0; i + k < n; ++k) x |= (uint64_t)p[i + k] << (8 * k);
    h = (h ^ x) * 0xC4CEB9FE1A85EC53ull;
    return h ^ (h >> 29);
  };
  auto insert = [&](const uint8_t *p, int64_t n, uint64_t h) {
    uint64_t s = h & mask;
    for (;;) {
      const int32_t w = table[s];
      if (w < 0) {
        table[s] = (int32_t)first.size();
        first.push_back(p);
        hashes.push_back(h);
        word_len.push_back((int32_t)n);
        word_freq.push_back(1);
        return;
      }
      if (hashes[(size_t)w] == h && word_len[(size_t)w] == n &&
          std::memcmp(first[(size_t)w], p, (size_t)n) == 0) {
        ++word_freq[(size_t)w];
        return;
      }
      s = (s + 1) & mask;
    }
  };
  for (int64_t d = 0; d < n_docs; ++d) {
    const uint8_t *doc = bytes + doc_off[d];
    const int64_t n = doc_off[d + 1] - doc_off[d];
    for (int64_t i = 0; i < n;) {
      int64_t e = i + 1;
      // the next start: a class change, unless a single space after a
      // non-whitespace byte (or at the document start) leads a letter
      while (e < n) {
        const int c0 = cls[doc[e]], c1 = cls[doc[e - 1]];
        if (c0 != c1 && !(c0 == 0 && doc[e - 1] == 0x20 && (e == 1 || cls[doc[e - 2]] != 2))) break;
        ++e;
      }
      insert(doc + i, e - i, hash_of(doc + i, e - i));
      i = e;
      if (2 * first.size() > table.size()) {
        // grow: twice the slots, every word placed again
        std::vector<int32_t> bigger(2 * table.size(), -1);
        mask = bigger.size() - 1;
        for (size_t w = 0; w < first.size(); ++w) {
          uint64_t s2 = hashes[w] & mask;
          while (bigger[s2] >= 0) s2 = (s2 + 1) & mask;
          bigger[s2] = (int32_t)w;
        }
        table.swap(bigger);
      }
    }
  }
  word_off.resize(first.size());
  int64_t total = 0;
  for (size_t w = 0; w < first.size(); ++w) {
    word_off[w] = total;
    total += word_len[w];
  }
  sym.resize((size_t)total);
  pos_word.resize((size_t)total);
  for (size_t w = 0; w < first.size(); ++w) {
    for (int32_t k = 0; k < word_len[w]; ++k) {
      sym[(size_t)(word_off[w] + k)] = first[w][k];
      pos_word[(size_t)(word_off[w] + k)] = (int32_t)w;
    }
  }
}

// Device copies for training, made before any kernel runs (blocking copies:
// the host vectors may go away as soon as they return).
template <class T>
T *dev_copy(const std::vector<T> &v, std::vector<void *> &owned) {
  void *p = nullptr;
  if (hipMalloc(&p, sizeof(T) * std::max<size_t>(v.size(), 1)) != hipSuccess) return nullptr;
  owned.push_back(p);
  if (!v.empty() && hipMemcpy(p, v.data(), sizeof(T) * v.size(), hipMemcpyHostToDevice) != hipSuccess)
    return nullptr;
  return (T *)p;
}

template <class T>
T *dev_zeros(size_t n, std::vector<void *> &owned) {
  void *p = nullptr;
  if (hipMalloc(&p, sizeof(T) * std::max<size_t>(n, 1)) != hipSuccess) return nullptr;
  owned.push_back(p);
  if (hipMemset(p, 0, sizeof(T) * std::max<size_t>(n, 1)) != hipSuccess) return nullptr;
  return (T *)p;
}

// The merges, kTrainGraph at a time: the three kernels of a merge take no
// argument that changes from merge to merge (the merge index is in device
// memory), so kTrainGraph merges are captured once as a HIP graph and the
// graph is launched until n merges are made or training stops (a step past
// either does nothing); the stop flag is read back every kTrainCheck
// launches.
constexpr int kTrainGraph = 64;
constexpr int kTrainCheck = 16;

int run_train_steps(const TrainArgs &a, int64_t n, hipStream_t stream) {
  const int64_t launches = (n + kTrainGraph - 1) / kTrainGraph;
  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int rc = BPE_OK;
  // the capture runs on a stream of its own, ordered after the caller's work
  if (hipStreamCreate(&cs) != hipSuccess) return BPE_EHIP;
  hipEvent_t ready = nullptr;
  if (hipEventCreateWithFlags(&ready, hipEventDisableTiming) != hipSuccess ||
      hipEventRecord(ready, stream) != hipSuccess || hipStreamWaitEvent(cs, ready, 0) != hipSuccess)
    rc = BPE_EHIP;
  if (rc == BPE_OK && hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) == hipSuccess) {
    bool ok = true;
    for (int k = 0; k < kTrainGraph && ok; ++k) ok = launch_train_step(a, cs) == hipSuccess;
    if (hipStreamEndCapture(cs, &graph) != hipSuccess || !ok) rc = BPE_EHIP;
  } else {
    rc = BPE_EHIP;
  }
  if (rc == BPE_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
    rc = BPE_EHIP;
  for (int64_t l = 0; rc == BPE_OK && l < launches; ++l) {
    if (hipGraphLaunch(exec, cs) != hipSuccess) {
      rc = BPE_EHIP;
      break;
    }
    if ((l + 1) % kTrainCheck == 0 && l + 1 < launches) {
      int32_t stop = 0;
      if (hipMemcpyAsync(&stop, a.stop, sizeof(stop), hipMemcpyDeviceToHost, cs) != hipSuccess ||
          hipStreamSynchronize(cs) != hipSuccess)
        rc = BPE_EHIP;
      else if (stop)
        break;
    }
  }
  if (hipStreamSynchronize(cs) != hipSuccess && rc == BPE_OK) rc = BPE_EHIP;
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (ready) (void)hipEventDestroy(ready);
  (void)hipStreamDestroy(cs);
  return rc;
}

}  // namespace

extern "C" {

int bpe_train(const uint8_t *bytes, int64_t n_bytes, const int64_t *doc_off, int64_t n_docs,
              int64_t n_merges, int32_t *merges_out, int64_t *counts_out, int64_t *n_made,
              void *hip_stream) {
  if (n_bytes < 0 || n_docs < 0 || !doc_off || (n_bytes > 0 && !bytes) || n_merges < 0 ||
      n_merges > BPE_MAX_MERGES || (n_merges > 0 && !merges_out) || !n_made)
    return BPE_EINVAL;
  if (doc_off[0] != 0 || doc_off[n_docs] != n_bytes) return BPE_EINVAL;
  if ((uint64_t)n_bytes >= ((uint64_t)1 << 32)) return BPE_EINVAL;  // pair counts are 32-bit
  for (int64_t d = 0; d < n_docs; ++d)
    if (doc_off[d + 1] < doc_off[d]) return BPE_EINVAL;
  *n_made = 0;
  // the distinct pre-tokens and their frequencies
  std::vector<int32_t> sym, pos_word, word_len;
  std::vector<int64_t> word_off, word_freq;
  collect_pretokens(bytes, doc_off, n_docs, sym, pos_word, word_off, word_len, word_freq);
  if (n_merges == 0 || sym.empty()) return BPE_OK;
  // the pre-tokens' symbols and the occurrence lists are indexed by 32 bits
  if (sym.size() >= ((size_t)1 << 30)) return BPE_EINVAL;
  hipStream_t stream = (hipStream_t)hip_stream;
  std::vector<void *> owned;
  int rc = BPE_OK;
  TrainArgs a;
  a.n_words = (int64_t)word_off.size();
  a.n_pos = (int64_t)sym.size();
  // keys are never removed: at most the initial pairs plus two per merged
  // occurrence (at most one occurrence per position), so 4 n_pos slots keep
  // the table at most three quarters full
  uint64_t slots = kTrainBlock;
  while (slots < 4 * (uint64_t)a.n_pos) slots *= 2;
  a.mask = slots - 1;
  a.nblocks = (int64_t)std::min<uint64_t>(slots / kTrainBlock, kTrainLoopBlocks);
  a.bsize = slots / (uint64_t)a.nblocks;
  a.n_target = n_merges;
  a.n_grid = std::min<int64_t>(n_merges, kTrainGridMerges);
  a.sym = dev_copy(sym, owned);
  {
    std::vector<uint4> wrec(word_off.size());
    for (size_t w = 0; w < word_off.size(); ++w)
      wrec[w] = uint4{(uint32_t)word_off[w], (uint32_t)word_len[w], (uint32_t)word_freq[w],
                      (uint32_t)((uint64_t)word_freq[w] >> 32)};
    a.wrec = dev_copy(wrec, owned);
  }
  a.pos_word = dev_copy(pos_word, owned);
  a.keys = dev_zeros<uint64_t>((size_t)slots, owned);
  a.counts = dev_zeros<uint32_t>((size_t)slots, owned);
  a.bmax = dev_zeros<uint32_t>((size_t)a.nblocks, owned);
  a.bkey = dev_zeros<unsigned long long>((size_t)a.nblocks, owned);
  a.dirty = dev_zeros<uint32_t>((size_t)a.nblocks, owned);
  a.dlist = dev_zeros<uint32_t>((size_t)a.nblocks, owned);
  a.ndirty = dev_zeros<uint32_t>(1, owned);
  {
    // occurrence lists of the bytes: each pre-token once per distinct byte;
    // the pool also holds one entry per pre-token a merge changes (at most
    // one per position in all)
    std::vector<int64_t> cnt(256, 0), off(256 + (size_t)n_merges, 0);
    std::vector<int32_t> len(256 + (size_t)n_merges, 0);
    std::vector<uint8_t> seen(256, 0);
    for (size_t w = 0; w < word_off.size(); ++w) {
      for (int32_t k = 0; k < word_len[w]; ++k) {
        const int b = sym[(size_t)(word_off[w] + k)];
        if (!seen[b]) {
          seen[b] = 1;
          ++cnt[b];
        }
      }
      for (int32_t k = 0; k < word_len[w]; ++k) seen[sym[(size_t)(word_off[w] + k)]] = 0;
    }
    int64_t total = 0;
    for (int b = 0; b < 256; ++b) {
      off[b] = total;
      len[b] = (int32_t)cnt[b];
      total += cnt[b];
    }
    std::vector<int32_t> pool((size_t)(total + a.n_pos));
    std::vector<int64_t> at(off.begin(), off.begin() + 256);
    for (size_t w = 0; w < word_off.size(); ++w) {
      for (int32_t k = 0; k < word_len[w]; ++k) {
        const int b = sym[(size_t)(word_off[w] + k)];
        if (!seen[b]) {
          seen[b] = 1;
          pool[(size_t)at[b]++] = (int32_t)w;
        }
      }
      for (int32_t k = 0; k < word_len[w]; ++k) seen[sym[(size_t)(word_off[w] + k)]] = 0;
    }
    a.pool = dev_copy(pool, owned);
    std::vector<uint2> lrec(off.size());
    for (size_t x = 0; x < off.size(); ++x) lrec[x] = uint2{(uint32_t)off[x], (uint32_t)len[x]};
    a.lrec = dev_copy(lrec, owned);
    std::vector<unsigned long long> top(1, (unsigned long long)total);
    a.pool_top = dev_copy(top, owned);
    a.zcount = dev_zeros<uint32_t>(1, owned);
  }
  a.best = dev_zeros<uint64_t>(3, owned);
  a.stop = dev_zeros<int32_t>(1, owned);
  a.merges = dev_zeros<int32_t>((size_t)(2 * n_merges), owned);
  a.out_counts = dev_zeros<int64_t>((size_t)n_merges, owned);
  a.made = dev_zeros<int64_t>(1, owned);
  if (!a.sym || !a.wrec || !a.pos_word || !a.keys ||
      !a.counts || !a.bmax || !a.bkey || !a.dirty || !a.dlist || !a.ndirty || !a.best ||
      !a.pool || !a.lrec || !a.pool_top || !a.zcount ||
      !a.stop || !a.merges || !a.out_counts || !a.made)
    rc = BPE_ENOMEM;
  if (rc == BPE_OK && launch_train_init(a, stream) != hipSuccess) rc = BPE_EHIP;
  if (rc == BPE_OK) rc = run_train_steps(a, a.n_grid, stream);
  if (rc == BPE_OK && n_merges > kTrainGridMerges && launch_train_loop(a, stream) != hipSuccess)
    rc = BPE_EHIP;
  int64_t made = 0;
  if (rc == BPE_OK &&
      (hipMemcpyAsync(&made, a.made, sizeof(int64_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
       hipMemcpyAsync(merges_out, a.merges, sizeof(int32_t) * 2 * (size_t)n_merges,
                      hipMemcpyDeviceToHost, stream) != hipSuccess ||
       (counts_out && hipMemcpyAsync(counts_out, a.out_counts, sizeof(int64_t) * (size_t)n_merges,
                                     hipMemcpyDeviceToHost, stream) != hipSuccess)))
    rc = BPE_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess && rc == BPE_OK) rc = BPE_EHIP;
  for (void *p : owned) (void)hipFree(p);
  if (rc == BPE_OK) *n_made = made;
  return rc;
}

const char *bpe_strerror(int code) {
  switch (code) {
    case BPE_OK: return "success";
    case BPE_EINVAL: return "invalid argument";
    case BPE_EMERGES: return "merge table rejected (repeated pair, operand out of range, or cycle)";
    case BPE_EIDMAP: return "id_map rejected (negative, repeated or too large ID)";
    case BPE_EWORKSPACE: return "workspace too small";
    case BPE_EHIP: return "HIP runtime error";
    case BPE_ENOMEM: return "out of memory";
    case BPE_ENOTSUP: return "decode unsupported: byte expansions of this table are too large";
    case BPE_EFORMAT: return "text form rejected (malformed line, JSON or UTF-8, or an unmapped character)";
    case BPE_ESCRATCH: return "input too large for the library's static scratch (BPE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

}  // extern "C"
