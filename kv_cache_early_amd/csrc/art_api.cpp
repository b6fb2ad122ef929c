// libart C-ABI front end: argument validation, work decomposition,
// workspace layout and kernel launches.  The operations themselves are
// described in include/art.h; the kernels live in art_kernels.hip.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>
#include <algorithm>

#include "art.h"
#include "art_internal.h"

namespace {

constexpr int kBlockTokens = 64;
constexpr int kProbeStride = 4;

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool finite_nonneg(float x) { return std::isfinite(x) && x >= 0.f; }

// Upper bound on T' (traversal blocks per unit) implied by the shape.
int64_t max_traversal(const art_shape& s) {
  if (s.max_kept > 0) return s.max_kept;
  int64_t tokens = s.page_size == 0 ? (int64_t)s.max_ctx : (int64_t)s.max_pages * s.page_size;
  return (tokens + kBlockTokens - 1) / kBlockTokens;
}

// Blocks a sequence can hold: ceil(capacity / 64), capacity = max_ctx or
// max_pages * page_size (the kept list does not matter for this bound).
int64_t capacity_blocks(const art_shape& s) {
  const int64_t tokens = s.page_size == 0 ? (int64_t)s.max_ctx : (int64_t)s.max_pages * s.page_size;
  return (tokens + kBlockTokens - 1) / kBlockTokens;
}
// Longest sequence (in blocks) whose GIVEN-order kept list the kernel can
// check for repeats: one bit per block in the 64 KiB of V slabs.
constexpr int64_t kGivenMaxBlocks = 65536LL * 8;

// Query rows per sequence (0 is read as 1).
int rows_of(const art_shape& s) { return s.q_rows > 0 ? s.q_rows : 1; }
// Query vectors per unit: G query heads times the query rows.
int64_t query_vectors(const art_shape& s) {
  return s.num_kv_heads > 0 ? (int64_t)(s.num_q_heads / s.num_kv_heads) * rows_of(s) : 1;
}

// Shape rules shared by every entry point.
art_status validate_shape(const art_shape* sp) {
  if (!sp || sp->struct_size != (int32_t)sizeof(art_shape)) return ART_ERR_INVALID_ARG;
  const art_shape& s = *sp;
  if (s.batch < 0 || s.num_q_heads <= 0 || s.num_kv_heads <= 0 || s.head_dim <= 0) return ART_ERR_INVALID_ARG;
  if (s.num_q_heads % s.num_kv_heads != 0) return ART_ERR_INVALID_ARG;
  if (s.dtype != ART_DT_F32 && s.dtype != ART_DT_BF16) return ART_ERR_INVALID_ARG;
  if (s.page_size < 0 || s.max_ctx < 0 || s.max_pages < 0 || s.num_pages < 0 || s.max_kept < 0)
    return ART_ERR_INVALID_ARG;
  if (s.page_size > 0 && s.page_size % 16 != 0) return ART_ERR_INVALID_ARG;
  if (s.q_rows < 0) return ART_ERR_INVALID_ARG;
  const int64_t GQ = (int64_t)(s.num_q_heads / s.num_kv_heads) * rows_of(s);  // query vectors per unit
  if (!((s.dtype == ART_DT_BF16 && s.head_dim == 128) || (s.dtype == ART_DT_F32 && s.head_dim == 64)))
    return ART_ERR_UNSUPPORTED;
  if (GQ != 1 && GQ != 2 && GQ != 4 && GQ != 8 && GQ != 16) return ART_ERR_UNSUPPORTED;
  if (s.page_size > 0 && (s.page_size & (s.page_size - 1)) != 0) return ART_ERR_UNSUPPORTED;  // powers of two
  // index ranges the kernels compute in 32-bit
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  if (units > (1 << 26) || max_traversal(s) > (1 << 24)) return ART_ERR_UNSUPPORTED;
  // paged pool rows (page * Hkv + h) * page_size + slot are 32-bit in the kernels
  if (s.page_size > 0 && (int64_t)s.num_pages * s.num_kv_heads * s.page_size > (int64_t)UINT32_MAX)
    return ART_ERR_UNSUPPORTED;
  return ART_OK;
}

art_status validate(const art_shape* sp, const art_params* pp) {
  if (!sp || !pp || pp->struct_size != (int32_t)sizeof(art_params)) return ART_ERR_INVALID_ARG;
  const art_shape& s = *sp;
  const art_params& p = *pp;
  if (p.block_size <= 0 || p.patience < 1 || p.split_blocks < 0) return ART_ERR_INVALID_ARG;
  if (!finite_nonneg(p.eps_scale) || !finite_nonneg(p.eps_dir)) return ART_ERR_INVALID_ARG;
  if (p.order < ART_ORDER_NATURAL || p.order > ART_ORDER_GIVEN) return ART_ERR_INVALID_ARG;
  if (p.mode != ART_MODE_FULL && p.mode != ART_MODE_ART) return ART_ERR_INVALID_ARG;
  constexpr int32_t kAllFlags = ART_FLAG_NO_SCALE | ART_FLAG_NO_DIR | ART_FLAG_DETECT_ONLY;
  if ((p.flags & ~kAllFlags) != 0 || (p.mode == ART_MODE_FULL && p.flags != 0)) return ART_ERR_INVALID_ARG;
  if (p.waves != 0 && p.waves != 4 && p.waves != 8) return ART_ERR_INVALID_ARG;
  if (p.order == ART_ORDER_GIVEN && s.max_kept == 0) return ART_ERR_INVALID_ARG;
  const art_status st = validate_shape(sp);
  if (st != ART_OK) return st;
  if (p.block_size != kBlockTokens) return ART_ERR_UNSUPPORTED;
  // ordered split ART keeps at most 4 query vectors per unit
  const int GQ = (s.num_q_heads / s.num_kv_heads) * rows_of(s);
  if (GQ > 4 && p.mode == ART_MODE_ART && p.split_blocks > 0 && p.split_blocks < max_traversal(s))
    return ART_ERR_UNSUPPORTED;
  // eight waves per workgroup: ART mode, one work item per unit, at most 4 query vectors
  if (p.waves == 8 && (p.mode != ART_MODE_ART || GQ > 4)) return ART_ERR_UNSUPPORTED;
  // GIVEN order: the kernel checks the kept list for repeated blocks with one
  // bit per block of the sequence in a 64 KiB LDS buffer
  if (p.order == ART_ORDER_GIVEN && capacity_blocks(s) > kGivenMaxBlocks) return ART_ERR_UNSUPPORTED;
  return ART_OK;
}

// Traversal blocks per work item.
//   full mode, at least one unit per compute unit: chunks sized so that
//     about kTargetItems workgroups balance uneven context lengths across
//     the compute units;
//   full mode, fewer units than compute units: about two work items per
//     compute unit (two workgroups fit on one), but no shorter than 32
//     blocks unless that leaves compute units without an item, and never
//     shorter than 8.  A work item's first block costs more than the steady
//     state, so short items lose more than they balance, while a call that
//     occupies few compute units is held to what each streams alone.
//     Measured on MI355X (full mode, chunk length: time): 128 units of 512
//     blocks 256: 0.368, 128: 0.360, 64: 0.365 ms; 32 units of 1024 kept
//     blocks 128: 0.198, 64: 0.198, 32: 0.205 ms; 16 units of 512 blocks
//     32: 0.059, 16: 0.063 ms; 4 units of 512 blocks 32: 0.041, 16: 0.030,
//     8: 0.028 ms; one unit of 512 blocks 32: 0.039, 16: 0.027, 8: 0.023 ms;
//   from kComputeUnits units on, at least 32 blocks (measured: 512 units of
//     128-512 blocks 64: 0.900, 32: 0.912 ms; 1024 units of 256 blocks 64:
//     1.448, 32: 1.481 ms);
//   either way a multiple of the wave count;
//   ART mode: one work item per unit (the stop rule's chain over the
//     positions) when there are enough units to fill the chip; otherwise
//     chunks of kSplitArtDefault blocks with look-back (ordered split ART).
//     A caller's split_blocks is honoured, rounded up to the wave count and
//     capped at kSplitArtBlocks (the look-back handles at most that many).
constexpr int64_t kTargetItems = 4096;
constexpr int64_t kComputeUnits = 256;  // MI355X
constexpr int kWavesPerItem = 4;
// Fewer units than this (the 256 CUs): split ART by default.  With fewer
// units than compute units, one work item per unit leaves CUs idle and a
// unit's walk is held to what one CU can stream (about 64 GB/s measured on
// MI355X); split ART spreads a unit over several CUs, its chunks' passes
// run in parallel and the stop rule is resolved by a decoupled look-back.
// Measured on MI355X (one work item per unit / split ART in 16-block
// chunks): 128 units of 512 blocks 0.394 / 0.242 ms where the criterion
// fires and 0.448 / 0.438 ms where it never does; 32 units of 1024 kept
// blocks 0.129 ms split (full mode 0.20 ms); one unit of 512 blocks 0.147
// / 0.048 ms.  At 512 units of 128-512 blocks one item per unit wins (0.40
// against 0.57 ms): every CU is busy and the chunks' look-backs only add.
constexpr int64_t kSplitArtUnits = 256;
// Chunk length: a chunk's look-back costs about the same whatever its
// length, so longer chunks spend less of the time in it where nothing
// stops, and load more blocks past the stop where the criterion fires.
// Measured on MI355X, 16 / 20 / 24-block chunks, criterion firing (share of
// the kept blocks loaded past the stop) and never firing: 32 units of 1024
// kept blocks 0.129 / 0.137 / 0.146 ms (12 / 18 / 23%) and 0.263 / 0.253 /
// 0.256 ms; 128 units of 512 blocks 0.242 / 0.244 / 0.248 ms (14 / 16 / 18%)
// and 0.438 / 0.423 / 0.416 ms; one unit of 512 blocks 0.048 / 0.055 /
// 0.054 ms.  The default favours the calls where the criterion fires.
constexpr int kSplitArtBlocks = 24;   // longest chunk the look-back handles
constexpr int kSplitArtDefault = 16;  // the library's chunk length for split ART
// Split ART: a chunk starts its speculative pass only once the chunk this
// many places before it (same unit) has resolved the stop rule.  Measured
// on MI355X with 16-block chunks, criterion firing / never firing (share of
// the kept blocks loaded past the stop): 32 units of 1024 kept blocks, 12
// places 0.136 / 0.275 ms (13.0%), 16 places 0.130 / 0.265 ms (12.1%), 24
// places 0.131 / 0.264 ms (13.2%); one unit of 512 blocks 0.063 / 0.085 ms
// (37.5%), 0.048 / 0.065 ms (24.2%), 0.049 / 0.063 ms (46.1%); 128 units of
// 512 blocks 0.245 / 0.439 ms at 12 and 0.241 / 0.440 ms at 16.  Fewer
// places serialize the chunks: 8 places 0.167 ms at 32 units, 4 places
// 0.245 ms (5.1%).
constexpr int kSplitArtDepth = 16;
int chunk_blocks(const art_shape& s, const art_params& p) {
  const int64_t tmax = std::max<int64_t>(1, max_traversal(s));
  if (p.mode == ART_MODE_ART) {
    const int64_t units = (int64_t)s.batch * s.num_kv_heads;
    int64_t c;
    if (p.split_blocks > 0)
      c = p.split_blocks >= tmax ? tmax : std::min<int64_t>((p.split_blocks + 3) / 4 * 4, kSplitArtBlocks);
    else  // split ART handles at most 4 query vectors per unit
      c = (units >= kSplitArtUnits || query_vectors(s) > 4) ? tmax : kSplitArtDefault;
    return (int)std::min<int64_t>(c, tmax);
  }
  if (p.split_blocks > 0) return (int)std::min<int64_t>(p.split_blocks, tmax);
  const int64_t units = std::max<int64_t>(1, (int64_t)s.batch * s.num_kv_heads);
  const int64_t total = tmax * units;
  int64_t c;
  if (units < kComputeUnits) {
    const int64_t two_per_cu = (total + 2 * kComputeUnits - 1) / (2 * kComputeUnits);
    const int64_t one_per_cu = (total + kComputeUnits - 1) / kComputeUnits;
    c = std::max<int64_t>(std::max<int64_t>(two_per_cu, std::min<int64_t>(32, one_per_cu)), 8);
  } else {
    c = std::max<int64_t>((total + kTargetItems - 1) / kTargetItems, 32);
  }
  c = (c + kWavesPerItem - 1) / kWavesPerItem * kWavesPerItem;
  return (int)std::min<int64_t>(c, tmax);
}

// Selection workspace: the header and one ItemState per workgroup of the
// larger of the two launches (block means: four blocks per workgroup).
size_t select_ws_bytes(const art_shape& s) {
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  const int64_t groups = std::max<int64_t>(1, (capacity_blocks(s) + 3) / 4);
  return round256(sizeof(art::WsHeader)) +
         round256(sizeof(art::ItemState) * (size_t)std::max<int64_t>(1, units * groups));
}

constexpr int64_t kSelectSortMax = 4096;  // blocks per unit the selection kernel sorts

// Waves per workgroup: 4 (two workgroups per CU) unless the caller asks
// for 8 (ART mode, one work item per unit, at most 4 query vectors per
// unit; one workgroup per CU, eight positions of a unit in flight).  Eight
// measured slower on MI355X wherever tried: 128 units of 512 blocks 0.447 vs
// 0.421 ms, 32 units of 1024 kept blocks 0.38 vs 0.34 ms, 512 units of
// 128-512 blocks 0.42 vs 0.40 ms (the stop rule's chain, not the waves'
// compute, sets a lone unit's pace).
int waves_per_item(const art_shape& s, const art_params& p, int max_chunks) {
  if (p.mode != ART_MODE_ART || max_chunks != 1 || query_vectors(s) > 4) return kWavesPerItem;
  return p.waves == 8 ? 8 : kWavesPerItem;
}

art::WsLayout layout(const art_shape& s, const art_params& p, int chunk, int max_chunks) {
  art::WsLayout L{};
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  const int G = (s.num_q_heads / s.num_kv_heads) * rows_of(s);  // query vectors per unit
  const int d = s.head_dim;
  L.header = round256(sizeof(art::WsHeader));
  L.items = round256(sizeof(art::ItemState) * (size_t)std::max<int64_t>(units * max_chunks, 1));
  L.partials = max_chunks > 1 ? round256((size_t)units * max_chunks * G * (d + 2) * sizeof(float)) : 0;
  const bool split_art = max_chunks > 1 && p.mode == ART_MODE_ART;
  const size_t carry_bytes = d == 128 ? sizeof(art::ChunkRec<128>) : sizeof(art::ChunkRec<64>);
  L.unit_stop = split_art ? round256((size_t)units * sizeof(int32_t)) : 0;
  L.carries = split_art ? round256((size_t)units * max_chunks * carry_bytes) : 0;
  (void)chunk;
  L.total = L.header + L.items + L.partials + L.unit_stop + L.carries;
  return L;
}

}  // namespace

namespace art {

// art_decode's work on a given workspace (also the body of the entry point
// that uses the library's own device buffer).
art_status decode_impl(const art_shape* shape, const art_params* params, const void* q, const void* k,
                       const void* v, const int32_t* context_lens, const int32_t* block_table,
                       const int32_t* kept_blocks, const int32_t* kept_count, float* out, int32_t* stop_idx,
                       int32_t* blocks_issued, void* workspace, size_t workspace_bytes, void* stream) {
  art_status st = validate(shape, params);
  if (st != ART_OK) return st;
  const art_shape& s = *shape;
  const art_params& p = *params;
  if ((kept_blocks == nullptr) != (kept_count == nullptr)) return ART_ERR_INVALID_ARG;
  if ((kept_blocks != nullptr) != (s.max_kept > 0)) return ART_ERR_INVALID_ARG;
  if (s.batch == 0) return ART_OK;
  if (!q || !k || !v || !context_lens || !out || !stop_idx) return ART_ERR_INVALID_ARG;
  if (s.page_size > 0 && (!block_table || s.max_pages <= 0 || s.num_pages <= 0)) return ART_ERR_INVALID_ARG;
  if (s.page_size == 0 && block_table) return ART_ERR_INVALID_ARG;

  const int chunk = chunk_blocks(s, p);
  const int64_t tmax = std::max<int64_t>(1, max_traversal(s));
  const int max_chunks = (int)((tmax + chunk - 1) / chunk);
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  if (units * max_chunks > INT32_MAX) return ART_ERR_UNSUPPORTED;
  const art::WsLayout L = layout(s, p, chunk, max_chunks);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return ART_ERR_WORKSPACE;

  art::KernelArgs a{};
  a.batch = s.batch;
  a.hq = s.num_q_heads;
  a.hkv = s.num_kv_heads;
  a.dtype = s.dtype;
  a.page_size = s.page_size;
  a.max_ctx = s.max_ctx;
  a.max_pages = s.max_pages;
  a.num_pages = s.num_pages;
  a.max_kept = s.max_kept;
  a.eps_scale = p.eps_scale;
  a.eps_dir = p.eps_dir;
  a.patience = p.patience;
  {
    const double tau = p.eps_scale, phi = p.eps_dir;
    a.crit_hi = (1.0 + tau) * (1.0 + tau);
    a.crit_lo = (1.0 - tau) * (1.0 - tau);
    a.crit_c2 = (1.0 - phi) * (1.0 - phi);
    a.crit_tau_lt1 = tau < 1.0;
    a.crit_phi_le1 = phi <= 1.0;
    // A test taken out always passes for a non-zero probe: an infinite upper
    // bound on |x_t|^2 / |x_{t-1}|^2, and for the direction the (1 - eps_dir)
    // > 0 branch off with an infinite bound on the negative side.
    if (p.flags & ART_FLAG_NO_SCALE) {
      a.crit_hi = INFINITY;
      a.crit_tau_lt1 = 0;
    }
    if (p.flags & ART_FLAG_NO_DIR) {
      a.crit_c2 = INFINITY;
      a.crit_phi_le1 = 0;
    }
  }
  a.detect_only = (p.flags & ART_FLAG_DETECT_ONLY) ? 1 : 0;
  a.rows = rows_of(s);
  a.gh = s.num_q_heads / s.num_kv_heads;
  a.order = p.order;
  a.mode = p.mode;
  a.chunk_blocks = chunk;
  a.max_chunks = max_chunks;
  a.split_art = (p.mode == ART_MODE_ART && max_chunks > 1) ? 1 : 0;
  a.waves = waves_per_item(s, p, max_chunks);
  a.q = q;
  a.k = k;
  a.v = v;
  a.context_lens = context_lens;
  a.block_table = block_table;
  a.kept_blocks = kept_blocks;
  a.kept_count = kept_count;
  a.out = out;
  a.stop_idx = stop_idx;
  a.blocks_issued = blocks_issued;
  char* w = static_cast<char*>(workspace);
  a.ws = reinterpret_cast<art::WsHeader*>(w);
  size_t off = L.header;
  a.items = reinterpret_cast<art::ItemState*>(w + off);
  off += L.items;
  a.partials = L.partials ? reinterpret_cast<float*>(w + off) : nullptr;
  off += L.partials;
  a.unit_stop = L.unit_stop ? reinterpret_cast<int32_t*>(w + off) : nullptr;
  off += L.unit_stop;
  a.carries = L.carries ? static_cast<void*>(w + off) : nullptr;
  a.spin_limit = 1u << 20;  // about a second of polling before ART_ERR_TIMEOUT
  a.spec_depth = kSplitArtDepth;

  hipError_t e = art::launch(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ART_OK : ART_ERR_HIP;
}

}  // namespace art

extern "C" {

size_t art_workspace_size(const art_shape* shape, const art_params* params) {
  if (validate(shape, params) != ART_OK) return 0;
  const int chunk = chunk_blocks(*shape, *params);
  const int64_t tmax = std::max<int64_t>(1, max_traversal(*shape));
  const int max_chunks = (int)((tmax + chunk - 1) / chunk);
  return layout(*shape, *params, chunk, max_chunks).total;
}

art_status art_decode(const art_shape* shape, const art_params* params, const void* q, const void* k,
                      const void* v, const int32_t* context_lens, const int32_t* block_table,
                      const int32_t* kept_blocks, const int32_t* kept_count, float* out, int32_t* stop_idx,
                      int32_t* blocks_issued, void* workspace, size_t workspace_bytes, void* stream) {
  return art::decode_impl(shape, params, q, k, v, context_lens, block_table, kept_blocks, kept_count, out,
                          stop_idx, blocks_issued, workspace, workspace_bytes, stream);
}

size_t art_select_workspace_size(const art_shape* shape) {
  if (validate_shape(shape) != ART_OK) return 0;
  return select_ws_bytes(*shape);
}

art_status art_block_means(const art_shape* shape, const void* k, const int32_t* context_lens,
                           const int32_t* block_table, float* means, int32_t max_blocks, void* workspace,
                           size_t workspace_bytes, void* stream) {
  art_status st = validate_shape(shape);
  if (st != ART_OK) return st;
  const art_shape& s = *shape;
  if (s.batch == 0) return ART_OK;
  if (!k || !context_lens || !means) return ART_ERR_INVALID_ARG;
  if (s.page_size > 0 && (!block_table || s.max_pages <= 0 || s.num_pages <= 0)) return ART_ERR_INVALID_ARG;
  if (s.page_size == 0 && block_table) return ART_ERR_INVALID_ARG;
  const int64_t tmax = capacity_blocks(s);
  if (max_blocks < tmax || max_blocks <= 0) return ART_ERR_INVALID_ARG;
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  const int64_t groups = std::max<int64_t>(1, (tmax + 3) / 4);
  if (units * groups > INT32_MAX) return ART_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < select_ws_bytes(s) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return ART_ERR_WORKSPACE;
  art::SelectArgs a{};
  a.batch = s.batch;
  a.hq = s.num_q_heads;
  a.hkv = s.num_kv_heads;
  a.dtype = s.dtype;
  a.page_size = s.page_size;
  a.max_ctx = s.max_ctx;
  a.max_pages = s.max_pages;
  a.num_pages = s.num_pages;
  a.max_blocks = max_blocks;
  a.t_max = (int)tmax;
  a.groups = (int)groups;
  a.k = k;
  a.context_lens = context_lens;
  a.block_table = block_table;
  a.means = means;
  char* w = static_cast<char*>(workspace);
  a.ws = reinterpret_cast<art::WsHeader*>(w);
  a.items = reinterpret_cast<art::ItemState*>(w + round256(sizeof(art::WsHeader)));
  return art::launch_block_means(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ART_OK : ART_ERR_HIP;
}

art_status art_select_blocks(const art_shape* shape, const art_select_params* params, const void* q,
                             const float* means, int32_t max_blocks, const int32_t* context_lens,
                             int32_t* kept_blocks, int32_t* kept_count, void* workspace, size_t workspace_bytes,
                             void* stream) {
  art_status st = validate_shape(shape);
  if (st != ART_OK) return st;
  if (!params) return ART_ERR_INVALID_ARG;
  const art_shape& s = *shape;
  const art_select_params& p = *params;
  if (!(p.keep_frac > 0.f && p.keep_frac <= 1.f) || p.sink < 0 || p.recent < 0) return ART_ERR_INVALID_ARG;
  if (p.order != ART_SELECT_ASCENDING && p.order != ART_SELECT_IMPORTANCE) return ART_ERR_INVALID_ARG;
  if (rows_of(s) != 1) return ART_ERR_INVALID_ARG;  // q is [B][Hq][d] here
  if (s.batch == 0) return ART_OK;
  if (!q || !means || !context_lens || !kept_blocks || !kept_count) return ART_ERR_INVALID_ARG;
  const int64_t tmax = capacity_blocks(s);
  if (max_blocks < tmax || max_blocks <= 0) return ART_ERR_INVALID_ARG;
  if (tmax > kSelectSortMax) return ART_ERR_UNSUPPORTED;
  const int64_t need = std::min<int64_t>(tmax, (int64_t)std::ceil((double)p.keep_frac * (double)tmax));
  if (s.max_kept < need) return ART_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < select_ws_bytes(s) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return ART_ERR_WORKSPACE;
  art::SelectArgs a{};
  a.batch = s.batch;
  a.hq = s.num_q_heads;
  a.hkv = s.num_kv_heads;
  a.dtype = s.dtype;
  a.page_size = s.page_size;
  a.max_ctx = s.max_ctx;
  a.max_pages = s.max_pages;
  a.num_pages = s.num_pages;
  a.max_kept = s.max_kept;
  a.max_blocks = max_blocks;
  a.t_max = (int)tmax;
  a.keep_frac = p.keep_frac;
  a.sink = p.sink;
  a.recent = p.recent;
  a.order = p.order;
  a.q = q;
  a.context_lens = context_lens;
  a.means = const_cast<float*>(means);
  a.kept_blocks = kept_blocks;
  a.kept_count = kept_count;
  char* w = static_cast<char*>(workspace);
  a.ws = reinterpret_cast<art::WsHeader*>(w);
  a.items = reinterpret_cast<art::ItemState*>(w + round256(sizeof(art::WsHeader)));
  return art::launch_select(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ART_OK : ART_ERR_HIP;
}

art_status art_last_error(const void* workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < sizeof(art::WsHeader)) return ART_ERR_INVALID_ARG;
  art::WsHeader h;
  if (hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return ART_ERR_HIP;
  if (h.magic != art::kWsMagic) return ART_OK;  // no launch has used this workspace
  const size_t off = round256(sizeof(art::WsHeader));
  if (h.n_items < 0 || off + (size_t)h.n_items * sizeof(art::ItemState) > workspace_bytes) return ART_ERR_WORKSPACE;
  std::vector<art::ItemState> items((size_t)h.n_items);
  if (h.n_items > 0 && hipMemcpy(items.data(), static_cast<const char*>(workspace) + off,
                                 items.size() * sizeof(art::ItemState), hipMemcpyDeviceToHost) != hipSuccess)
    return ART_ERR_HIP;
  int32_t worst = ART_OK;
  for (const art::ItemState& it : items) worst = std::max(worst, it.status);
  return static_cast<art_status>(worst);
}

const char* art_status_string(art_status status) {
  switch (status) {
    case ART_OK: return "ok";
    case ART_ERR_INVALID_ARG: return "invalid argument";
    case ART_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case ART_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ART_ERR_HIP: return "HIP runtime or launch failure";
    case ART_ERR_TIMEOUT: return "split look-back wait timed out on the device";
    case ART_ERR_DEVICE_INPUT: return "device-side input out of range (context length, page id or kept list)";
  }
  return "unknown status";
}

int32_t art_probe_stride(void) { return kProbeStride; }

int32_t art_abi_version(void) { return ART_ABI_VERSION; }

}  // extern "C"
