// Internal structures shared by the C-ABI front end (art_api.cpp) and the
// gfx950 kernels (art_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "art.h"

namespace art {

// Workspace header, written by work item 0 of every decode launch.  Every
// work item also writes its own ItemState on every launch, so a workspace
// needs no initialisation and a call enqueues no memset.
constexpr uint32_t kWsMagic = 0x31545241u;  // "ART1"
struct alignas(256) WsHeader {
  uint32_t magic;      // kWsMagic once a launch has written the header
  int32_t n_items;     // work items of that launch (ItemState entries)
  uint32_t ticket;     // split ART: next work item to hand out (zeroed per call)
  int32_t pad[61];
};

// Per work item (grid index), written unconditionally at its end.
struct ItemState {
  int32_t status;      // art_status seen by the item (ART_OK or a device error)
  int32_t issued;      // blocks whose loads the item issued (-1: kept list rejected)
};

// Summary of one ART block on the probe dims (probe dim 4p of query vector g
// at ps[p][g]), relative to the block's own score maximum m (log2 domain).
// GS query vectors (4 for up to four per unit).
template <int D, int GS = 4>
struct alignas(16) Summary {
  float m[GS];          // reference max per query vector
  float l[GS];          // softmax mass per query vector relative to m
  float ps[D / 4][GS];  // sums on the probe dims relative to m
};

// Split ART: what one chunk of a unit publishes for the chunks after it.
// Each part is written once and none waits for a later chunk, so a chunk
// finds its carry and its patience state by looking back over its
// predecessors' parts instead of waiting for a chain of hand-offs
// (decoupled look-back).  One state word, written whole by the chunk's
// thread 0 once the part it announces is acknowledged, says what is there:
//   bits 0-1   prefix: 0 nothing yet; 1 the aggregate is written; 2 the
//              inclusive prefix is written too; 3 the unit stopped before
//              this chunk (nothing else is written)
//   bit 2      the patience descriptor below is written
//   bits 3-7   descriptor: checks in the chunk (its positions but the unit's first)
//   bits 8-12  descriptor: leading stable checks
//   bits 13-17 descriptor: trailing stable checks
//   bits 18-22 descriptor: 1 + the blocks of the chunk up to the stop that a
//              run of `patience` stable checks after its first unstable one
//              makes (0: none)
//   bits 32-63 the stop rule's state at the chunk's end: 0 not yet; 1 |
//              counter << 2 no stop so far; 2 the unit stopped at or before
//              this chunk's end; 3 | counter << 2 detect-only, a stop
//              detected at or before this chunk's end
template <int D>
struct alignas(16) ChunkRec {
  uint64_t state;
  uint64_t pad;
  // aggregate: the chunk's own blocks, relative to their max (log2 domain)
  float am[4];
  double al[4];        // mass per query vector
  double ap[D / 4][4]; // numerators on the probe dims
  // inclusive prefix: every block of the unit up to the chunk's last
  float im[4];
  double il[4];
  double ip[D / 4][4];
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
  int32_t detect_only;   // record the stop, never terminate
  int32_t rows;          // query rows per sequence (q and out are [B][rows][Hq][d])
  int32_t gh;            // query heads per kv head (Hq / Hkv); a unit has rows * gh query vectors
  int32_t split_art;     // ART mode with several chunks per unit (look-back)
  int32_t chunk_blocks;  // traversal blocks per work item
  int32_t max_chunks;    // work items per unit
  int32_t waves;         // waves per workgroup, 4 or 8 (one work item per workgroup)
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
  int32_t* unit_stop;  // split ART: [units] traversal count at the stop, 0 while none
  float* partials;     // [units][max_chunks][G][d + 2]  (m, l, acc[d])
  void* carries;       // split ART: [units][max_chunks] ChunkRec<d>
  uint32_t spin_limit; // look-back polls before ART_ERR_TIMEOUT
  int32_t spec_depth;  // split ART: chunk k starts once chunk k - spec_depth has resolved the stop rule
};

// Workspace layout for a given shape (bytes, 256-aligned pieces).
struct WsLayout {
  size_t header, items, partials, unit_stop, carries, total;
};

hipError_t launch(const KernelArgs& a, hipStream_t stream);

// art_decode's work on a caller-chosen workspace (art_api.cpp): shared by
// art_decode and art_decode_static.
art_status decode_impl(const art_shape* shape, const art_params* params, const void* q, const void* k,
                       const void* v, const int32_t* context_lens, const int32_t* block_table,
                       const int32_t* kept_blocks, const int32_t* kept_count, float* out, int32_t* stop_idx,
                       int32_t* blocks_issued, void* workspace, size_t workspace_bytes, void* stream);

// Key-based block selection (block-mean keys, kept lists).
struct SelectArgs {
  int32_t batch, hq, hkv, dtype, page_size, max_ctx, max_pages, num_pages, max_kept;
  int32_t max_blocks;     // row stride (blocks) of `means`
  int32_t t_max;          // ceil(capacity / 64)
  int32_t groups;         // block-means launch: workgroups per unit (4 blocks each)
  float keep_frac;
  int32_t sink, recent, order;
  const void* q;
  const void* k;
  const int32_t* context_lens;
  const int32_t* block_table;
  float* means;           // [B][Hkv][max_blocks][d]
  int32_t* kept_blocks;   // [B][Hkv][max_kept]
  int32_t* kept_count;    // [B][Hkv]
  WsHeader* ws;
  ItemState* items;       // one per work item (workgroup) of the launch
};
hipError_t launch_block_means(const SelectArgs& a, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

}  // namespace art
