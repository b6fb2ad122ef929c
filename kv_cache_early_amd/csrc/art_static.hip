// art_decode_static: art_decode on a device buffer the library owns, for
// callers that cannot allocate (see include/art.h).
//
// The buffer is a file-scope device array.  In host code its name is only a
// host-side stand-in, so its device address is looked up once per device
// (with that device current) through hipGetSymbolAddress and kept; every
// use goes through that address.  The decode path needs no cleared
// workspace (each launch rewrites what it reads), so nothing is cleared here.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "art.h"
#include "art_internal.h"

namespace {

constexpr size_t kStaticScratchBytes = ART_STATIC_SCRATCH_BYTES;  // per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// The device address of this device's copy of the array (nullptr on failure).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

art_status art_decode_static(const art_shape* shape, const art_params* params, const void* q, const void* k,
                             const void* v, const int32_t* context_lens, const int32_t* block_table,
                             const int32_t* kept_blocks, const int32_t* kept_count, float* out,
                             int32_t* stop_idx, int32_t* blocks_issued, void* stream) {
  const size_t need = art_workspace_size(shape, params);
  if (need == 0)  // invalid shape or params: art_decode names the reason
    return art::decode_impl(shape, params, q, k, v, context_lens, block_table, kept_blocks, kept_count, out,
                            stop_idx, blocks_issued, nullptr, 0, stream);
  if (need > kStaticScratchBytes) return ART_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return ART_ERR_HIP;
  return art::decode_impl(shape, params, q, k, v, context_lens, block_table, kept_blocks, kept_count, out,
                          stop_idx, blocks_issued, ws, kStaticScratchBytes, stream);
}

}  // extern "C"
