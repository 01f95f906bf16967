// kvc_decode_static: kvc_decode without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The decode's scratch (chunk
// table, decode groups, row sums, header flags, per-stream payload offsets)
// lives in a fixed array in the library's device memory instead, one copy
// per GPU, held until the process ends.  Nothing here allocates.
#include <mutex>

#include "kvc_internal.h"

namespace {

// The array itself.  In host code its name is only a stand-in for the
// symbol: kernels get the device address looked up below, never the name.
static __device__ __align__(256) uint8_t scratch[KVC_DECODE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// The current device's copy of the array: its address is looked up once per
// device, with that device current, and kept.
void *device_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" kvc_status kvc_decode_static(const kvc_codec_desc *d, const void *tables,
                                        const kvc_chunk_ref *chunks, uint32_t n_chunks,
                                        uint16_t *kv_out, uint32_t T_total, int32_t *dev_status,
                                        hipStream_t stream) {
  if (kvc_validate_desc(d) != KVC_OK) return KVC_ERR_INVALID_ARG;
  if (n_chunks > 65535) return KVC_ERR_SHAPE;
  // the same scratch kvc_decode would take from a workspace must fit
  const uint64_t need = kvc_decode_ws_bytes(d, n_chunks);
  if (need > KVC_DECODE_STATIC_SCRATCH_BYTES) return KVC_ERR_CAPACITY;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_ERR_HIP;
  void *ws = device_scratch(dev);
  if (ws == nullptr) return KVC_ERR_HIP;
  return kvc_decode(d, tables, chunks, n_chunks, kv_out, T_total, ws,
                    KVC_DECODE_STATIC_SCRATCH_BYTES, dev_status, stream);
}
