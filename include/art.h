/*
 * libart -- ART (Attention Run-time Termination) decode attention for AMD
 * Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * For every unit (batch b, kv head h) with G = num_q_heads / num_kv_heads
 * query heads (query head h*G + g uses kv head h):
 *
 *   * the KV cache of sequence b is split into blocks of `block_size` tokens
 *     (the last block may be partial) and walked in a traversal order pi
 *     (ART paper, section 3.1: blockwise FlashAttention-style execution over
 *     tiles {(K_t, V_t)}; gist.science explainer of the paper, section 2.4:
 *     recency-first / other orders, block 0 always evaluated first);
 *   * after t blocks the partial output O^(t) = softmax(q K_S^T / sqrt(d)) V_S
 *     over the tokens S of the first t blocks (ART paper, section 3.1,
 *     Eq. (1) restricted to the processed blocks);
 *   * a probe x^(t) = head dims 0, 4, 8, ..., d-4 of O^(t) for each of the G
 *     query heads, concatenated (ART paper, section 3.2: a fixed scattered
 *     subsample of the head dims);
 *   * for t >= 2 two metrics (gist.science explainer, section 2.2):
 *       d_scale = | |x^(t)| - |x^(t-1)| | / |x^(t-1)|
 *       d_dir   = 1 - cos(x^(t), x^(t-1))
 *     a check is stable when d_scale < eps_scale and d_dir < eps_dir (strict;
 *     a zero-norm probe is never stable);
 *   * with patience p (gist.science explainer, section 2.3) the unit stops
 *     after block t once the last p checks were all stable; no further KV
 *     block of that unit is loaded or computed.
 *
 * Outputs: out[b][h*G+g][:] = O^(stop_idx) in fp32, stop_idx[b][h] = number
 * of traversal blocks processed (1..T'), optional blocks_issued[b][h] =
 * number of blocks whose K/V loads were issued (processed + discarded
 * prefetch + speculative split work + recomputation).  In ART_MODE_FULL no
 * criterion is evaluated and stop_idx = T' (plain blockwise attention).
 * A unit with no tokens (context length 0, or kept_count 0) gets out = 0
 * and stop_idx = 0.
 *
 * Conventions (all entry points)
 * ------------------------------
 *   * Every data pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains memory.  Shape and parameter
 *     structs are HOST pointers, read during the call only.
 *   * art_decode is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  Argument errors are detected on the host
 *     and returned before anything is enqueued.  Errors only visible on the
 *     device (a malformed kept list, a look-back timeout) are recorded in the
 *     workspace; read them with art_last_error after synchronizing `stream`.
 *   * Nothing prints, throws or exits.  Calls that share one workspace must
 *     not overlap in time.
 *
 * Supported set (anything else returns ART_ERR_UNSUPPORTED):
 *   dtype ART_DT_BF16 with head_dim 128, or ART_DT_F32 with head_dim 64;
 *   G = num_q_heads / num_kv_heads in {1, 2, 4}; block_size 64;
 *   page_size 0 (contiguous) or a power of two >= 16.
 */
#ifndef LIBART_ART_H
#define LIBART_ART_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of this interface: the layout of art_params and art_shape and the
 * meaning of their fields.  A caller checks art_abi_version() against the
 * ART_ABI_VERSION it was built with, and sets every struct's struct_size to
 * sizeof(the struct); a mismatch makes every call return
 * ART_ERR_INVALID_ARG. */
#define ART_ABI_VERSION 2

typedef enum {
  ART_OK = 0,
  ART_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad parameter       */
  ART_ERR_UNSUPPORTED = 2,   /* valid but outside the supported set         */
  ART_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required  */
  ART_ERR_HIP = 4,           /* a HIP runtime call or launch failed         */
  ART_ERR_TIMEOUT = 5,       /* device: a bounded wait between waves or work
                                items of a call timed out                   */
  ART_ERR_DEVICE_INPUT = 6   /* device: a context length, page id or kept list
                                was out of range, a kept list not strictly
                                ascending where required, or a GIVEN-order
                                list held a block twice                     */
} art_status;

typedef enum { ART_DT_F32 = 0, ART_DT_BF16 = 1 } art_dtype;

/* Traversal order pi over the candidate blocks (all blocks, or the kept
 * list).  Block 0, when it is a candidate, is always first (gist.science
 * explainer, section 2.4).  NATURAL: ascending block index.  RECENT_FIRST:
 * descending (most recent first).  GIVEN: the kept list's own order; needs a
 * kept list. */
typedef enum { ART_ORDER_NATURAL = 0, ART_ORDER_RECENT_FIRST = 1, ART_ORDER_GIVEN = 2 } art_order;

typedef enum { ART_MODE_FULL = 0, ART_MODE_ART = 1 } art_mode;

/* Switches of the stop rule (art_params.flags, ART mode only), for the
 * detector-overhead and ablation measurements of the gist.science
 * explainer's experiments section:
 *  - NO_SCALE, NO_DIR take the magnitude test or the direction test out of
 *    the stability check (a zero-norm probe is still never stable);
 *    patience 1 is the no-patience ablation.
 *  - DETECT_ONLY runs the detector but never terminates: every block is
 *    read and attended to (out is full decode), stop_idx reports where the
 *    rule would have stopped (T' if nowhere), blocks_issued counts every
 *    block read. */
typedef enum { ART_FLAG_NO_SCALE = 1, ART_FLAG_NO_DIR = 2, ART_FLAG_DETECT_ONLY = 4 } art_flag;

typedef struct {
  int32_t struct_size;   /* sizeof(art_params)                               */
  int32_t block_size;    /* tokens per ART block (64)                        */
  float eps_scale;       /* tau: threshold on d_scale, >= 0, finite          */
  float eps_dir;         /* phi: threshold on d_dir (1 - cos), >= 0, finite  */
  int32_t patience;      /* p >= 1 consecutive stable checks                 */
  int32_t order;         /* art_order                                        */
  int32_t mode;          /* art_mode                                         */
  int32_t split_blocks;  /* blocks per split-KV chunk; 0 = library's choice,
                            a value >= T' means one chunk per unit.  In ART
                            mode, a value below T' selects ordered split ART
                            (chunks of min(round4(split_blocks), 24) blocks:
                            a speculative pass per chunk, the stop rule
                            resolved by a look-back over the earlier chunks'
                            published prefixes and patience descriptors, and
                            a recompute of the chunk holding the stop);
                            blocks_issued then counts the speculative and
                            re-read blocks, which vary from call to call.
                            A chunk starts loading only once the chunk 16
                            places before it has resolved the stop rule, and
                            stops loading once the unit's stop is published,
                            so a unit loads at most 15 chunks past its stop
                            chunk plus that chunk's recompute.
                            The library's choice in ART mode: split ART in
                            16-block chunks when the call has fewer than 256
                            units and at most 4 query vectors per unit, one
                            chunk per unit otherwise.  In full mode, with
                            at least 256 units (one per compute unit):
                            chunks of at least 32 blocks, sized so that about
                            4096 work items balance uneven lengths; with
                            fewer: about 512 work items (two per compute
                            unit), at least 32 blocks each unless that
                            leaves compute units without one, never fewer
                            than 8.
                            Either way
                            stop_idx and out do not depend on the choice
                            beyond floating-point rounding.                 */
  int32_t flags;         /* OR of art_flag; must be 0 in full mode           */
  int32_t waves;         /* ART mode with one work item per unit and at most
                            4 query vectors per unit: waves per workgroup,
                            0 = library's choice (4: two workgroups per
                            compute unit), 4 or 8 (one workgroup per compute
                            unit).  With W waves, W consecutive traversal
                            positions of a unit are in flight at once: a
                            unit loads at most 2 W - 1 blocks past its stop
                            (blocks_issued <= stop_idx + 2 W - 1).  Ignored
                            (4) in every other case; 8 where it does not
                            apply is ART_ERR_UNSUPPORTED.  out and stop_idx
                            do not depend on it beyond floating-point
                            rounding.                                        */
} art_params;

typedef struct {
  int32_t struct_size;    /* sizeof(art_shape)                               */
  int32_t batch;          /* B                                               */
  int32_t num_q_heads;    /* Hq                                              */
  int32_t num_kv_heads;   /* Hkv (Hq % Hkv == 0)                             */
  int32_t head_dim;       /* d                                               */
  int32_t dtype;          /* art_dtype of q, K and V                         */
  int32_t page_size;      /* 0: contiguous K/V [B][Hkv][max_ctx][d];
                             else paged K/V [num_pages][Hkv][page_size][d]   */
  int32_t max_ctx;        /* contiguous: row stride in tokens; every
                             context_lens[b] <= max_ctx                      */
  int32_t max_pages;      /* paged: row stride of block_table; every
                             context_lens[b] <= max_pages * page_size        */
  int32_t num_pages;      /* paged: pages in the pool (bounds check only)    */
  int32_t max_kept;       /* row stride of kept_blocks; 0 = no kept list     */
  int32_t q_rows;         /* M query rows per sequence (0 is read as 1): q
                             and out are [B][M][Hq][d].  The M * G query
                             vectors of a unit (G = Hq / Hkv) share its
                             traversal and its one stop, their probes
                             concatenated row by row (ART paper section 3.1
                             writes Q with any number of rows; per-row or
                             per-block stopping is not fixed by the pages).
                             M * G must be 1, 2, 4, 8 or 16; above 4, split
                             ART and 8 waves are not available.              */
} art_shape;

/* Bytes of device workspace art_decode needs for this shape and params
 * (never 0).  Returns 0 if the shape or params are invalid. */
size_t art_workspace_size(const art_shape* shape, const art_params* params);

/* Blockwise ART decode attention (see the top of this file).
 *
 *   q             [B][M][Hq][d] in `dtype` (M = q_rows; [B][Hq][d] when 1)
 *   k, v          contiguous [B][Hkv][max_ctx][d] or paged
 *                 [num_pages][Hkv][page_size][d], in `dtype`
 *   context_lens  int32 [B], 0 <= len (bounded as described in art_shape)
 *   block_table   int32 [B][max_pages] page ids (paged only, else NULL);
 *                 entries past ceil(len/page_size) are never read
 *   kept_blocks   int32 [B][Hkv][max_kept] candidate block indices, or NULL;
 *                 strictly ascending for NATURAL/RECENT_FIRST, distinct and
 *                 in [0, ceil(len/block_size)) for all orders; a list that
 *                 breaks this is reported as ART_ERR_DEVICE_INPUT (its unit
 *                 gets out = 0, stop_idx = -1).  GIVEN order needs
 *                 ceil(capacity / 64) <= 524288 blocks (capacity = max_ctx
 *                 or max_pages * page_size), ART_ERR_UNSUPPORTED otherwise
 *   kept_count    int32 [B][Hkv] entries used per unit (NULL iff kept_blocks)
 *   out           fp32 [B][M][Hq][d]               (written)
 *   stop_idx      int32 [B][Hkv]                   (written)
 *   blocks_issued int32 [B][Hkv] or NULL           (written)
 *   workspace     device buffer of >= art_workspace_size() bytes, 256-byte
 *                 aligned; its contents on entry do not matter (every call
 *                 rewrites what it reads, so no initialisation or per-call
 *                 clearing is needed and the call enqueues no memset)
 *
 * ART_MODE_ART with one work item per unit enqueues one kernel; ordered
 * split ART enqueues an init kernel, the decode kernel and an LSE-combine
 * kernel; ART_MODE_FULL with more than one chunk per unit enqueues the
 * decode kernel and the combine kernel.
 */
art_status art_decode(const art_shape* shape, const art_params* params,
                      const void* q, const void* k, const void* v,
                      const int32_t* context_lens, const int32_t* block_table,
                      const int32_t* kept_blocks, const int32_t* kept_count,
                      float* out, int32_t* stop_idx, int32_t* blocks_issued,
                      void* workspace, size_t workspace_bytes, void* stream);

/* art_decode without a caller-provided workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments and outputs as for
 * art_decode; the workspace is a device buffer of ART_STATIC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends
 * (one per device, found on the device current at the call).
 *   * Returns ART_ERR_WORKSPACE, before anything is enqueued, when
 *     art_workspace_size(shape, params) exceeds ART_STATIC_SCRATCH_BYTES;
 *     other argument errors as art_decode.  Allocates nothing.
 *   * All calls on one GPU share its buffer: calls that overlap in time on
 *     one GPU (other streams, other host threads) race and give undefined
 *     results.  Sequential calls need no clearing between them.
 *   * Device-side errors are recorded in that buffer and cannot be read
 *     back with art_last_error; a unit whose kept list is rejected still
 *     shows stop_idx = -1 and out = 0. */
#define ART_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
art_status art_decode_static(const art_shape* shape, const art_params* params,
                             const void* q, const void* k, const void* v,
                             const int32_t* context_lens, const int32_t* block_table,
                             const int32_t* kept_blocks, const int32_t* kept_count,
                             float* out, int32_t* stop_idx, int32_t* blocks_issued,
                             void* stream);

/* Device-side error recorded by the last call (art_decode, art_block_means
 * or art_select_blocks) that enqueued work on `workspace` (ART_OK,
 * ART_ERR_TIMEOUT or ART_ERR_DEVICE_INPUT; the most severe over its work
 * items).  ART_OK if no launch has used the workspace.
 * Synchronous (device-to-host copies of the workspace's status words); call
 * after synchronizing the decode's stream.  `workspace_bytes` bounds what is
 * read: ART_ERR_WORKSPACE if the recorded work does not fit in it. */
art_status art_last_error(const void* workspace, size_t workspace_bytes);

/* ---- key-based block selection and importance-first traversal ----------
 *
 * The gist.science explainer (section 2.4) composes ART with KV-cache
 * managers through the traversal sequence, naming importance-first as one
 * order.  The importance of block j of unit (b, h) is taken as
 *   s_j = qbar . kbar_j,
 * qbar = the mean of the unit's G query rows, kbar_j = the mean of the
 * block's valid key rows (64-token blocks).  A kept list keeps the first
 * `sink` blocks, the `recent` most recent blocks, and fills up to
 * n = min(T, ceil(keep_frac * T)) blocks with the highest s_j, ties to the
 * lower block index (T = ceil(len / 64)).  ART_SELECT_ASCENDING writes the
 * list in ascending block order (for ART_ORDER_NATURAL / RECENT_FIRST);
 * ART_SELECT_IMPORTANCE writes it by decreasing s_j, ties to the lower
 * index (for ART_ORDER_GIVEN: an importance-first traversal; with
 * keep_frac = 1 it orders every block). */
typedef enum { ART_SELECT_ASCENDING = 0, ART_SELECT_IMPORTANCE = 1 } art_select_order;

typedef struct {
  float keep_frac;  /* (0, 1]                                               */
  int32_t sink;     /* leading blocks always kept, >= 0                     */
  int32_t recent;   /* most recent blocks always kept, >= 0                 */
  int32_t order;    /* art_select_order of the written list                 */
} art_select_params;

/* Workspace bytes for art_block_means and art_select_blocks on `shape`
 * (0 on an invalid shape).  Same rules as art_decode's workspace: device
 * memory, 256-byte aligned, no initialisation needed; art_last_error reads
 * the status they record. */
size_t art_select_workspace_size(const art_shape* shape);

/* Block-mean keys.  For every unit (b, h) and block j < ceil(len_b / 64):
 *   means[((b * Hkv + h) * max_blocks + j) * d + i] = mean over the block's
 *   valid tokens of K[token][i]            (fp32, written)
 * Entries for j >= ceil(len_b / 64) are not written.  K, context_lens and
 * block_table as for art_decode (shape.max_kept is ignored); max_blocks >=
 * ceil(capacity / 64), capacity = max_ctx (contiguous) or max_pages *
 * page_size (paged).  Reads every key once; meant to run when blocks are
 * written, not per decode step.  Lengths outside [0, capacity] are clamped
 * and page ids outside the pool read page 0; both are reported as
 * ART_ERR_DEVICE_INPUT by art_last_error. */
art_status art_block_means(const art_shape* shape, const void* k, const int32_t* context_lens,
                           const int32_t* block_table, float* means, int32_t max_blocks,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Kept lists from block-mean keys (see above): for every unit writes
 * kept_blocks[(b * Hkv + h) * shape.max_kept + i] for i < n, and
 * kept_count[b * Hkv + h] = n.  q as for art_decode; means as written by
 * art_block_means with the same max_blocks; shape.q_rows 0 or 1.  Requires shape.max_kept >=
 * min(T_max, ceil(keep_frac * T_max)) for T_max = ceil(capacity / 64), and
 * T_max <= 4096 (ART_ERR_UNSUPPORTED otherwise). */
art_status art_select_blocks(const art_shape* shape, const art_select_params* params, const void* q,
                             const float* means, int32_t max_blocks, const int32_t* context_lens,
                             int32_t* kept_blocks, int32_t* kept_count,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Static English description of a status code. */
const char* art_status_string(art_status status);

/* Probe-stride constant used for x^(t) (4), for callers that report it. */
int32_t art_probe_stride(void);

/* ART_ABI_VERSION of the built library. */
int32_t art_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBART_ART_H */
