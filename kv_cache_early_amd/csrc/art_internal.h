// Internal structures shared by the C-ABI front end (art_api.cpp) and the
// gfx950 kernels (art_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace art {

// Workspace header, written by work item 0 of every decode launch.  Every
// work item also writes its own ItemState on every launch, so a workspace
// needs no initialisation and a call enqueues no memset.
constexpr uint32_t kWsMagic = 0x31545241u;  // "ART1"
struct alignas(256) WsHeader {
  uint32_t magic;      // kWsMagic once a launch has written the header
  int32_t n_items;     // work items of that launch (ItemState entries)
  int32_t pad[62];
};

// Per work item (grid index), written unconditionally at its end.
struct ItemState {
  int32_t status;      // art_status seen by the item (ART_OK or a device error)
  int32_t issued;      // blocks whose loads the item issued
};

// Look-back carry published by a chunk for its successor (split ART mode):
// the prefix state of the probe dims after the chunk's last block.
template <int G, int NP>
struct alignas(16) Carry {
  int32_t flag;        // 0 not ready, 1 ready (running), 2 ready (stopped)
  int32_t counter;     // consecutive stable checks at the end of the chunk
  int32_t stop_idx;    // when stopped
  int32_t pad;
  float m[G];          // running max (log2 domain) per head
  double l[G];         // running denominator per head
  double pacc[G][NP];  // running numerators on the probe dims
};

struct KernelArgs {
  // shape
  int32_t batch, hq, hkv, dtype, page_size, max_ctx, max_pages, num_pages, max_kept;
  // params
  float eps_scale, eps_dir;
  int32_t patience, order, mode;
  // squared forms of the thresholds (see the stability tests in the kernel)
  double crit_hi, crit_lo, crit_c2;  // (1+eps_scale)^2, (1-eps_scale)^2, (1-eps_dir)^2
  int32_t crit_tau_lt1, crit_phi_le1; // eps_scale < 1, eps_dir <= 1
  int32_t chunk_blocks;  // traversal blocks per work item
  int32_t max_chunks;    // work items per unit
  int32_t waves;         // waves per workgroup (one work item per workgroup)
  // inputs
  const void* q;
  const void* k;
  const void* v;
  const int32_t* context_lens;
  const int32_t* block_table;
  const int32_t* kept_blocks;
  const int32_t* kept_count;
  // outputs
  float* out;
  int32_t* stop_idx;
  int32_t* blocks_issued;
  // workspace
  WsHeader* ws;
  ItemState* items;    // [max_chunks][units], grid order
  float* partials;     // [units][max_chunks][G][d + 2]  (m, l, acc[d])
  void* carries;       // [units][max_chunks] Carry<G, d/4>
  uint32_t spin_limit; // look-back polls before ART_ERR_TIMEOUT
};

// Workspace layout for a given shape (bytes, 256-aligned pieces).
struct WsLayout {
  size_t header, items, partials, carries, total;
};

hipError_t launch(const KernelArgs& a, hipStream_t stream);

}  // namespace art
