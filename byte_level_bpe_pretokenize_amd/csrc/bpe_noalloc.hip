// bpe_noalloc.hip -- bpe_encode_batch_noalloc: the encode pipeline on a
// static device array instead of a caller workspace, for callers that cannot
// allocate device memory (HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// gets its own copy at its own address when the code object is loaded there.
// In host code the name is only a host-side stand-in, so the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is handed to the kernels.
#include <mutex>

#include "../../include/bpe.h"
#include "bpe_internal.h"

namespace {

constexpr size_t kScratchBytes = BPE_NOALLOC_SCRATCH_BYTES;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, nullptr until looked up

// The address of `scratch` on device dev (the current device).
int scratch_on(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return BPE_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BPE_EHIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return BPE_OK;
}

}  // namespace

extern "C" int bpe_encode_batch_noalloc(const bpe_model *model, const uint8_t *d_bytes,
                                        int64_t n_bytes, const int64_t *d_doc_off, int64_t n_docs,
                                        int32_t *d_ids, int64_t ids_capacity, int64_t *d_id_off,
                                        int32_t *d_status, void *hip_stream) {
  if (!model || n_bytes < 0 || n_docs < 0) return BPE_EINVAL;
  if (bpe_encode_workspace_bytes(model, n_bytes, n_docs) > kScratchBytes) return BPE_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BPE_EHIP;
  if (dev != bpe::model_device(model)) return BPE_EINVAL;
  void *ws = nullptr;
  const int rc = scratch_on(dev, &ws);
  if (rc != BPE_OK) return rc;
  return bpe::encode_checked(model, d_bytes, n_bytes, d_doc_off, n_docs, d_ids, ids_capacity,
                             d_id_off, ws, kScratchBytes, d_status, hip_stream, false);
}
