// cb_rerope_k_noalloc: cb_rerope_k with its rotation table in a static device
// array instead of a caller workspace, for callers that cannot allocate.
//
// The array below is a per-GPU device symbol.  In host code its name denotes a
// host-side stand-in, not a device address, so the address on the current
// device is looked up once with hipGetSymbolAddress and kept per device; every
// kernel argument uses that address.
#include <mutex>

#include "cb_internal.h"

namespace {

constexpr size_t kScratchBytes = CB_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on first use).
cb_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return cb::record_failure(CB_ERR_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return cb::record_failure(CB_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return cb::record_failure(CB_ERR_DEVICE, "hipGetSymbolAddress of the static scratch array failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CB_OK;
}

}  // namespace

extern "C" cb_status cb_rerope_k_noalloc(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks,
                                         const cb_paged_kv* dst, uint32_t flags, cb_stream_t stream) {
  cb_status st = cb::rerope_check(cfg, chunks, n_chunks, dst, flags);
  if (st != CB_OK) return st;
  if (cb::rerope_table_bytes(*cfg, n_chunks) > kScratchBytes)
    return cb::record_failure(CB_ERR_WORKSPACE, "the rotation table exceeds the static scratch array "
                                                "(CB_NOALLOC_SCRATCH_BYTES)");
  void* table = nullptr;
  if ((st = scratch_address(&table)) != CB_OK) return st;
  return cb::rerope_enqueue(*cfg, chunks, n_chunks, *dst, flags, static_cast<float2*>(table),
                            reinterpret_cast<hipStream_t>(stream));
}
