// ART decode attention kernels for gfx950 (MI355X).
//
// Work decomposition.  One workgroup of W waves (W = blockDim.x / 64) owns
// one work item = (unit, chunk): unit = (batch b, kv head h) with its query
// vectors (G query heads times the query rows), chunk = a range of
// positions of the unit's traversal order.  Wave w walks positions
// t0 + w, t0 + w + W, ... of the item.
//
// Per 64-token ART block a wave
//   1. has K in MFMA A-operand registers (16-byte loads straight from HBM)
//      and V in a private 16 KB LDS slab (direct global->LDS loads), both
//      issued one block ahead;
//   2. computes the transposed scores S^T = K q^T, 64 tokens x G heads, with
//      v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x4_f32 for fp32 inputs); the
//      B operand holds the G query rows replicated over the 16 MFMA columns;
//   3. runs the online softmax (running max in the log2 domain) per head;
//      a lane holds the weights of four consecutive tokens of one head,
//      which is exactly the A-operand layout of the P V product;
//   4. computes P V with MFMA: B operands come from the V slab through the
//      transposing LDS read ds_read_b64_tr_b16 (fp32: plain LDS reads), and
//      bf16 P is split into a high and a low bf16 part (two MFMAs), which
//      keeps P to about 16 significant bits;
//   5. (ART mode) folds the block into the stop rule, in one of two ways:
//      - one work item per unit: a chain over the positions through LDS.
//        The wave of position t merges its block's summary (per query
//        vector its max, mass and sums on the probe dims) onto the prefix
//        state the wave of t - 1 left, runs the two stability tests and the
//        patience counter of position t, and hands the state on.  A wave
//        commits its block only once the state of t - 1 shows no stop
//        before it, so the stop is the one a strictly sequential walk finds.
//      - split ART (a unit cut into chunks, one workgroup each): a chunk
//        walks all its blocks speculatively, keeping their summaries in
//        LDS, then resolves the stop rule by a decoupled look-back over the
//        earlier chunks' published prefixes and patience descriptors, and
//        recomputes its output up to the stop if the stop falls inside it.
// The waves' states are merged in LDS at the end (log-sum-exp); with several
// chunks per unit a combine kernel merges the chunks' partial outputs.
//
// Method sources: ART paper section 3.1 Eq. (1) (blockwise attention and the
// partial outputs O^(t)), section 3.2 (probe of scattered head dims);
// gist.science explainer sections 2.2 (scale and direction metrics, dual
// threshold), 2.3 (patience), 2.4 (traversal order, block 0 first).
//
// Lane geometry (both supported element types have 256-byte rows cut into
// 16 chunks of 16 bytes): lane l = 16*lg + c with lg = l / 16, c = l % 16.
//   K (A operand)  : load j of tile nt -> token 16*nt + c, chunk 4*j + lg.
//   q (B operand)  : k-step j           -> head c % G,     chunk 4*j + lg.
//   S^T, O (D)     : lane l holds column c and rows 4*lg + r (r = 0..3); for
//                    S^T the rows are tokens 16*nt + 4*lg + r of head c % G,
//                    for O the rows are heads (4*lg + r) % G of dim 16*dt + c.
//   V (LDS slab)   : DMA n (0..15) carries tokens 4n..4n+3 as four 256-byte
//                    rows; chunk x of token row y (y = token % 4) is stored
//                    at position x ^ 2y ^ 8(n & 1), which spreads the 16
//                    lanes of a transposed read over distinct LDS banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "art.h"
#include "art_internal.h"

namespace art {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxWaves = 8;      // waves per workgroup (4 or 8)
constexpr int kBlk = 64;          // tokens per ART block
constexpr int kTiles = kBlk / 16; // 16-token MFMA tiles per block
constexpr int kRowChunks = 16;    // 16-byte chunks per K/V row
constexpr int kLoads = kBlk * kRowChunks / kWave;   // 16 loads per lane per block (K), 16 DMAs (V)
constexpr int kVSlab = kBlk * kRowChunks * 16;      // 16 KB: V of one block

template <int DT>
struct Geo;
template <>
struct Geo<ART_DT_BF16> {
  static constexpr int D = 128, ES = 2, PPC = 2;  // PPC: probe dims per 16-byte chunk
};
template <>
struct Geo<ART_DT_F32> {
  static constexpr int D = 64, ES = 4, PPC = 1;
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
#define ART_DPP_I(x, ctrl, rmask) __builtin_amdgcn_update_dpp(0, (x), (ctrl), (rmask), 0xF, false)
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
constexpr int kQx1 = 0xB1, kQx2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

template <int CTRL, int RMASK = 0xF>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = ART_DPP_I((int)(uint32_t)u, CTRL, RMASK);
  const int hi = ART_DPP_I((int)(uint32_t)(u >> 32), CTRL, RMASK);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}
// All-reduce of an fp64 value over the 16 lanes of each row.
__device__ __forceinline__ double row_sum_d(double x) {
  x += dpp<kQx1>(x);
  x += dpp<kQx2>(x);
  x += dpp<kHalfMirror>(x);
  return x + dpp<kMirror>(x);
}

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }
// All-reduce over the four 16-lane rows: every lane gets the result over the
// lanes with its own column (lanes l, l ^ 16, l ^ 32, l ^ 48).  The row swap
// exchanges odd rows of its first operand with even rows of its second, the
// half swap the upper half of the first with the lower half of the second.
__device__ __forceinline__ float col_max(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  x = fmaxf(u2f(s[0]), u2f(s[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(t[0]), u2f(t[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  x = u2f(s[0]) + u2f(s[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(t[0]) + u2f(t[1]);
}
// The same all-reduce over the four rows for an fp64 value (both halves swapped).
__device__ __forceinline__ double col_sum_d(double x) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
  const auto sl = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto sh = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  x = __builtin_bit_cast(double, ((uint64_t)sh[0] << 32) | sl[0]) +
      __builtin_bit_cast(double, ((uint64_t)sh[1] << 32) | sl[1]);
  u = __builtin_bit_cast(uint64_t, x);
  const auto tl = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto th = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  return __builtin_bit_cast(double, ((uint64_t)th[0] << 32) | tl[0]) +
         __builtin_bit_cast(double, ((uint64_t)th[1] << 32) | tl[1]);
}
// All-reduce of three fp64 values over the 64 lanes, in lockstep: three
// independent chains, so each stage's latency is paid once.  The row stages
// are DPP moves with bound_ctrl (every lane reads a lane of its own row, so
// no old value is needed), the column stages the row and half swaps.
template <int CTRL>
__device__ __forceinline__ double dpp_b(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <bool H32>
__device__ __forceinline__ double swap_add(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  if constexpr (H32) {
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]) +
           __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
  } else {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    return __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]) +
           __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
  }
}
__device__ __forceinline__ void allsum3_d(double& x, double& y, double& z) {
  x += dpp_b<kQx1>(x);
  y += dpp_b<kQx1>(y);
  z += dpp_b<kQx1>(z);
  x += dpp_b<kQx2>(x);
  y += dpp_b<kQx2>(y);
  z += dpp_b<kQx2>(z);
  x += dpp_b<kHalfMirror>(x);
  y += dpp_b<kHalfMirror>(y);
  z += dpp_b<kHalfMirror>(z);
  x += dpp_b<kMirror>(x);
  y += dpp_b<kMirror>(y);
  z += dpp_b<kMirror>(z);
  x = swap_add<false>(x);
  y = swap_add<false>(y);
  z = swap_add<false>(z);
  x = swap_add<true>(x);
  y = swap_add<true>(y);
  z = swap_add<true>(z);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
// The lane index, produced by an instruction the compiler cannot move or
// reuse: LDS addresses derived from it are computed where they are used
// instead of being kept (and spilled) from the kernel's start.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ float lane_f(float x, int l) { return u2f(__builtin_amdgcn_readlane(f2u(x), l)); }
// A uniform value the compiler must treat as new at each use: the LDS
// addresses derived from it are then formed where they are used (one scalar
// add each) instead of being hoisted out of the walk and kept in spilled
// scalar registers (a lane read back for every DMA).
__device__ __forceinline__ uint32_t fresh_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// fp64 reciprocal: fp32 estimate plus one Newton step (relative error ~1e-14).
__device__ __forceinline__ double recip_d(double x) {
  const double r0 = (double)__builtin_amdgcn_rcpf((float)x);
  return fma(r0, fma(-x, r0, 1.0), r0);
}

// The two stability tests on squared quantities, a = |x^(t-1)|, b = |x^(t)|,
// p = x^(t).x^(t-1) (a, b > 0):
//   |b - a| / a < tau   <=>  (1-tau)^2 a^2 < b^2 < (1+tau)^2 a^2   (tau < 1;
//                            only the upper bound for tau >= 1)
//   1 - p/(ab)  < phi   <=>  p > (1-phi) a b, i.e. for phi <= 1: p > 0 and
//                            p^2 > (1-phi)^2 a^2 b^2; for phi > 1: p >= 0 or
//                            p^2 < (phi-1)^2 a^2 b^2.
// Squaring keeps the comparisons strict and avoids fp64 square roots and
// divisions on the stop rule's critical path.
struct Criterion {
  double hi, lo, c2;   // (1+tau)^2, (1-tau)^2, (1-phi)^2, computed on the host
  bool tau_lt1, phi_le1;
  // Non-short-circuit forms (bitwise on the comparison results): no
  // branches on the stop rule's critical path.
  __device__ bool scale_ok(double a2, double b2) const {
    return (b2 < hi * a2) & ((!tau_lt1) | (b2 > lo * a2));
  }
  __device__ bool dir_ok(double a2, double b2, double p) const {
    const double r = c2 * a2 * b2;
    const double pp = p * p;
    return (phi_le1 & (p > 0.0) & (pp > r)) | ((!phi_le1) & ((p >= 0.0) | (pp < r)));
  }
};

// Two fp32 values rounded to nearest-even bf16, packed (first value in the
// low half), and the two halves of a packed pair widened back to fp32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// Uniform load through the scalar data cache (read-only metadata: context
// lengths, block tables, kept lists).  Keeps metadata off the vector-load
// counter, so waiting for it never waits for in-flight K/V loads.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Direct global -> LDS load of 16 bytes per lane: lane l writes
// lds + 16*l (lds uniform, passed in M0).  Issued as inline assembly so the
// compiler, which cannot track LDS-DMA completion per LDS object, does not
// put a full vmcnt(0) in front of every later LDS access; all waits for it
// are explicit (wait_vm).  M0 has no other use in these kernels (LDS
// instructions on this target do not read it, and no indirect register
// indexing is generated), so setting it here cannot disturb compiler state.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
// The same with a uniform 64-bit base in SGPRs plus a per-lane 32-bit offset.
__device__ __forceinline__ void lds_dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Wait until at most N vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte global load issued as inline assembly, so the compiler does not
// place its own (over-conservative) vmcnt waits for it; users wait with
// wait_v_tied.  The variant with `dep` takes a register operand it does not
// use: the load is then issued only after the instruction that produced it.
template <int OFF = 0>
__device__ __forceinline__ u32x4 gload16(const void* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(r) : "v"(p), "n"(OFF) : "memory");
  return r;
}
template <int OFF = 0>
__device__ __forceinline__ u32x4 gload16_after(const void* p, float dep) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2 ; after %3" : "=v"(r) : "v"(p), "n"(OFF), "v"(dep) : "memory");
  return r;
}
// Uniform 64-bit base in SGPRs plus a per-lane 32-bit offset.
template <int OFF = 0>
__device__ __forceinline__ u32x4 gload16s(uint32_t voff, const void* sbase) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3" : "=v"(r) : "v"(voff), "s"(sbase), "n"(OFF) : "memory");
  return r;
}
template <int OFF = 0>
__device__ __forceinline__ u32x4 gload16s_after(uint32_t voff, const void* sbase, float dep) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 ; after %4"
               : "=v"(r)
               : "v"(voff), "s"(sbase), "n"(OFF), "v"(dep)
               : "memory");
  return r;
}
// Wait until at most N vector-memory operations are outstanding, tying the
// 16 K registers to the wait so no use of them is scheduled ahead of it.
template <int N>
__device__ __forceinline__ void wait_v_tied(u32x4 (&v)[16]) {
  asm volatile("s_waitcnt vmcnt(%16)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                 "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                 "+v"(v[15])
               : "n"(N)
               : "memory");
}

// The same wait, also tying one more register (a dword loaded by gload_sys).
template <int N>
__device__ __forceinline__ void wait_v_tied_s(u32x4 (&v)[16], int& w) {
  asm volatile("s_waitcnt vmcnt(%17)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                 "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                 "+v"(v[15]), "+v"(w)
               : "n"(N)
               : "memory");
}
// A dword read at the point of coherence (like ld_sys), issued as inline
// assembly so that it joins the hand-counted vector-memory waits.
__device__ __forceinline__ int gload_sys(const int* p) {
  int r;
  asm volatile("global_load_dword %0, %1, off sc0 sc1" : "=v"(r) : "v"(p) : "memory");
  return r;
}

// Transposing 8-byte LDS read (gfx950): within each 16-lane row, element e of
// lane i is element i % 4 of what lane 4e + i / 4 of that row addresses.
__device__ __forceinline__ s16x4 lds_read_tr(const __attribute__((address_space(3))) uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Coherent single accesses between workgroups on different XCDs (each XCD
// has its own L2): relaxed system-scope atomics reach the point of coherence
// one by one, so no cache-wide write-back or invalidation is needed.  A
// writer waits for its stores to be acknowledged before it raises a flag.
template <typename T>
__device__ __forceinline__ T ld_sys(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename T>
__device__ __forceinline__ void st_sys(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Single LDS words shared between the waves of a workgroup, read and written
// as volatile LDS accesses.  The explicit address space matters: a volatile
// access through a generic pointer (which is what a lambda's captured
// reference to a __shared__ object is) stays a flat access, and a flat load
// waits on the vector-memory counter too, i.e. for every K/V load in flight.
__device__ __forceinline__ int lds_get(const int& x) {
  return *(const volatile __attribute__((address_space(3))) int*)(&x);
}
__device__ __forceinline__ void lds_put(int& x, int v) { *(volatile __attribute__((address_space(3))) int*)(&x) = v; }
__device__ __forceinline__ double lds_get(const double& x) {
  return *(const volatile __attribute__((address_space(3))) double*)(&x);
}
__device__ __forceinline__ float lds_get(const float& x) {
  return *(const volatile __attribute__((address_space(3))) float*)(&x);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic
// and meets the other waves, without waiting for in-flight global loads (a
// full __syncthreads() would drain the K/V prefetch).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// per-unit view of the inputs (all fields uniform)
// ---------------------------------------------------------------------------
struct UnitView {
  const char* k;         // contiguous: row 0 of (b, h); paged: pool base
  const char* v;
  const int32_t* bt;     // block-table row of b (paged)
  const int32_t* kept;   // kept list of (b, h) or null
  int n_ctx;             // tokens in the sequence
  int n_blocks;          // ceil(n_ctx / 64)
  int n_pages;           // ceil(n_ctx / page) (paged)
  int n_trav;            // T'
  int zero_pos;          // GIVEN order: position of block 0 in the list, or -1
  int log2_page;         // paged: log2(page size)
  int row_pages;         // paged: entries per block-table row (max_pages)
  int hkv, h;
  int num_pages;
};

// Block index at traversal position t.  Block 0, when a candidate, comes
// first; NATURAL ascending, RECENT_FIRST descending, GIVEN list order.
__device__ __forceinline__ int block_at(const UnitView& u, int order, int t) {
  if (!u.kept) {
    if (order == ART_ORDER_NATURAL) return t;
    return t == 0 ? 0 : u.n_blocks - t;  // RECENT_FIRST: [0, T-1, ..., 1]
  }
  const int n = u.n_trav;
  if (order == ART_ORDER_NATURAL) return sload(u.kept + t);
  if (order == ART_ORDER_RECENT_FIRST) {
    if (sload(u.kept) == 0) return t == 0 ? 0 : sload(u.kept + (n - t));
    return sload(u.kept + (n - 1 - t));
  }
  if (u.zero_pos < 0) return sload(u.kept + t);
  if (t == 0) return 0;
  return sload(u.kept + (t <= u.zero_pos ? t - 1 : t));
}

// Uniform addressing of one 64-token block.
//   contiguous: rows past the context are clamped per lane to the last token
//               at load time (read in bounds, then masked);
//   paged:      one base per 16-token group (page sizes are powers of two
//               >= 16), page ids read through the scalar cache; page indices
//               past the sequence are clamped to its last page, page ids
//               outside the pool are replaced by page 0 and recorded.
struct BlockAddr {
  uint32_t row[4];     // row of token 16*g of the block: paged, in the pool
                       // ((page * Hkv + h) * page + slot); contiguous, in the unit
  int j;               // block index
  int nvalid;          // valid tokens in the block
};

template <int ROW, bool PAGED>
__device__ __forceinline__ BlockAddr block_addr(const UnitView& u, int j, int& bad) {
  BlockAddr ba;
  ba.j = j;
  ba.nvalid = min(kBlk, u.n_ctx - j * kBlk);
  if constexpr (PAGED) {
    const int pmask = (1 << u.log2_page) - 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tok = j * kBlk + 16 * g;
      const int pi = min(tok >> u.log2_page, u.n_pages - 1);
      int pg = sload(u.bt + pi);
      const bool oob = (unsigned)pg >= (unsigned)u.num_pages;
      bad |= oob;
      pg = oob ? 0 : pg;
      ba.row[g] = (((uint32_t)pg * (uint32_t)u.hkv + (uint32_t)u.h) << u.log2_page) + (uint32_t)(tok & pmask);
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) ba.row[g] = (uint32_t)(j * kBlk + 16 * g);
  }
  return ba;
}

// Paged rows of block j from one 16-byte scalar load instead of four
// dependent ones.  The four block-table entries starting at
// min((64 j) >> log2(page), max_pages - 4) hold the pages of all four
// 16-token groups of block j, also those clamped to the sequence's last
// page: the groups' pages are consecutive from (64 j) >> log2(page), and the
// window only moves back from the row's end when it would pass it.  Rows of
// fewer than 4 entries take the per-group path.
template <int ROW, bool PAGED>
__device__ __forceinline__ BlockAddr block_addr4(const UnitView& u, int j, int& bad) {
  if constexpr (PAGED) {
    if (u.row_pages >= 4) {
      const int base = min((j * kBlk) >> u.log2_page, u.row_pages - 4);
      const int32_t* w = u.bt + base;
      const int e[4] = {sload(w), sload(w + 1), sload(w + 2), sload(w + 3)};  // merged into one load
      BlockAddr ba;
      ba.j = j;
      ba.nvalid = min(kBlk, u.n_ctx - j * kBlk);
      const int pmask = (1 << u.log2_page) - 1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tok = j * kBlk + 16 * g;
        const int idx = min(tok >> u.log2_page, u.n_pages - 1) - base;  // in [0, 3]
        int pg = idx == 0 ? e[0] : (idx == 1 ? e[1] : (idx == 2 ? e[2] : e[3]));
        const bool oob = (unsigned)pg >= (unsigned)u.num_pages;
        bad |= oob;
        pg = oob ? 0 : pg;
        ba.row[g] = (((uint32_t)pg * (uint32_t)u.hkv + (uint32_t)u.h) << u.log2_page) + (uint32_t)(tok & pmask);
      }
      return ba;
    }
  }
  return block_addr<ROW, PAGED>(u, j, bad);
}

// ---------------------------------------------------------------------------
// LDS layout (one workgroup)
// ---------------------------------------------------------------------------
// The stop rule runs as two chains over the traversal positions (ART mode
// with one work item per unit): the wave holding position t merges its
// block onto the prefix state after position t - 1 and publishes the
// prefix state after t (first chain), then runs the checks of position t
// and hands the patience counter on (second chain).  A prefix record holds
// one lane's share of that state (lane (lg, c): query vectors lg + 4 hh for
// hh < NH, or lg alone with up to four; probe dims c * PPC .. c * PPC +
// PPC - 1).
template <int NPL, int NH>
struct alignas(16) LaneLink {
  double p[NPL];  // prefix numerators on the probe dims, relative to m
  double l[NH];   // prefix mass per query vector, relative to m
  float m[NH];    // reference max per query vector (log2 domain)
};
struct alignas(16) LinkHead {
  int seq;        // position + 1 once the prefix record of that position is complete
  int seqc;       // position + 1 once counter and detected of that position are written
  int counter;    // consecutive stable checks after the position
  int detected;   // detect-only: the first stop the rule reached, 0 if none
};
template <int NPL, int NH, int NL>
struct alignas(16) RoundLds {
  LaneLink<NPL, NH> link[2][NL];       // by position parity (NL lanes; 1 where no chain runs)
  LinkHead head[2];
  int stop_at;                         // blocks processed at the stop, 0 while none
  int detected;                        // detect-only: the first stop, 0 while none
  int timeout;                         // a wave's wait for its predecessor's record timed out
  int bad;
  int zero_pos;
  int ticket;                          // split ART: this workgroup's work item
  int flag;                            // split ART: the unit's stop, then the bounding chunk's outcome
};
// Split ART: the block summaries of the chunk being walked (pass 0), in
// the look-back's layout [block][query vector][probe dim]; LDS of their own,
// written during the walk.
constexpr int kSplitMax = 24;  // chunk length the look-back handles
template <int D, int N>
struct alignas(16) SplitSum {
  float m[N][4];        // reference max per query vector
  float l[N][4];        // softmax mass per query vector relative to m
  float ps[N][4][D / 4];  // sums on the probe dims relative to m
};
// Split ART look-back state (reuses the V slabs, below the waves' stash).
template <int D>
struct alignas(16) LookbackLds {
  // the chunk's prefix numerators after each block, on its own maximum; rows
  // padded by one element, so that the 64 lanes of the per-position reads
  // (eight positions x four query vectors x two halves) spread over the banks
  double Q[kSplitMax][4][D / 4 + 1];
  double lam[kSplitMax][4];       // the chunk's prefix mass after each block, on the same maximum
  double pc[4][D / 4];            // the carry's numerators
  double lc[4];                   // the carry's mass
  float mc[4];                    // the carry's maximum
  float ml[4];                    // the chunk's own maximum
  double stt[kSplitMax + 1];      // stt[j + 1] = |x|^2 at position j; stt[0] from the carry
  int bits[kSplitMax];
  int stop_local;                 // blocks of the chunk up to and including the stop, -1 if none
  int lb;                         // look-back: the chunk whose inclusive prefix the carry starts from
  int found;                      // the stop (or detect-only: the first stop) this chunk found, -1 if none
  int outcome;                    // 0 the chunk counts; 1 a wait timed out; 2 the unit stopped before it
};
template <int G, int D, int W>
struct alignas(16) EpilogueLds {     // per-wave final state (reuses the V slabs)
  static constexpr int GS = G > 4 ? G : 4;
  float m[W][GS];
  float l[W][GS];
  int issued[W];
  int bad[W];
  float acc[W][D][GS];               // [wave][dim][query vector]
};

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------
// SPLIT: the ordered split-ART instantiation (ticket order, look-back,
// recompute); the other instantiation serves full mode and single-chunk ART.
// W waves per workgroup: 4 (two workgroups per CU), or 8 on request (one
// per CU; single-chunk ART with up to 4 query vectors per unit: eight
// positions of a unit in flight).
template <int DT, int G, bool PAGED, bool SPLIT, int W>
__global__ __launch_bounds__(kWave * W, W == 4 ? 2 : 1) void art_decode_kernel(KernelArgs a) {
  static_assert(W == 4 || (W == 8 && !SPLIT && G <= 4), "waves per workgroup");
  // G is the number of query vectors of a unit: rows * (Hq / Hkv).  Up to 4
  // they fill the 16 MFMA columns by repetition; 8 or 16 (multi-row queries)
  // take the columns and output rows one for one (no split ART).
  static_assert(G == 1 || G == 2 || G == 4 || ((G == 8 || G == 16) && !SPLIT), "query vectors per unit");
  using GE = Geo<DT>;
  constexpr int D = GE::D, ES = GE::ES, PPC = GE::PPC;
  constexpr int NDT = D / 16;  // 16-dim output tiles
  constexpr int ROW = D * ES;
  constexpr int NT = kWave * W;  // threads per workgroup
  constexpr int NH = G > 4 ? G / 4 : 1;  // query vectors per lane row in the stop rule's layout
  constexpr int NPL = NH * PPC;          // probe values per lane there
  static_assert(ROW == kRowChunks * 16, "rows must be 16 chunks of 16 bytes");
  // the chain's records are not used by split ART, whose block summaries
  // take LDS of their own instead
  __shared__ RoundLds<SPLIT ? 1 : NPL, SPLIT ? 1 : NH, SPLIT ? 1 : kWave> R;
  __shared__ SplitSum<D, SPLIT ? kSplitMax : 1> SS;
  __shared__ alignas(16) uint8_t vbuf[W][kVSlab];
  // the waves' final state is stashed above the look-back state, so a split
  // chunk can keep its pass-0 result in LDS while the look-back runs
  constexpr int kEpiOff = SPLIT ? 32768 : 0;
  static_assert(!SPLIT || sizeof(LookbackLds<D>) <= kEpiOff, "look-back state must fit below the stash");
  static_assert(kEpiOff + sizeof(EpilogueLds<G, D, W>) <= sizeof(vbuf), "stash must fit the V slabs");

  const int tid = threadIdx.x;
  const int wid = uni(tid >> 6);
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int c = lane & 15;

  // ---- work item --------------------------------------------------------
  const int n_units = a.batch * a.hkv;
  const int n_items = n_units * a.max_chunks;
  // Split ART hands out work items in ticket order, chunk-major: an item's
  // predecessor chunk always holds a smaller ticket, so it is running or done
  // when the item waits for its carry.
  int item = blockIdx.x;
  if constexpr (SPLIT) {
    if (tid == 0) R.ticket = (int)atomicAdd(&a.ws->ticket, 1u);
    __syncthreads();
    item = uni(R.ticket);
  }
  if (item == 0 && tid == 0) {
    a.ws->magic = kWsMagic;
    a.ws->n_items = n_items;
  }
  int unit = item % n_units;
  // One work item per unit: pair long and short sequences on a CU.  With
  // more units than CUs, workgroups i and i + n/2 share a CU (the
  // dispatcher places them round-robin over the XCDs and then over each
  // XCD's CUs), and a CU's two units share its bandwidth.  Batch slot k takes
  // the sequence of length rank k (longest first) in the first half of the
  // batch and of rank B-1-(k-B/2) in the second, so a CU's load is about
  // even where work follows length.  Outputs are indexed by unit, so the
  // results do not change.  Measured on MI355X, 512 units of 128-512 blocks:
  // criterion never firing 1.115 -> 0.93 ms, full mode in one item per
  // unit 1.011 -> 0.869 ms; criterion firing (work independent of length)
  // 0.92-1.05x over six seeds, about 1.0 on average.  Ranking all lengths in
  // every workgroup costs B^2/64 compares per lane, hence the bound on B.
  if (!SPLIT && W == 4 && a.max_chunks == 1 && a.batch >= 2 && a.batch <= 256) {
    const int B = a.batch, half = B / 2;
    const int k = unit / a.hkv, hh = unit % a.hkv;
    const int r = k < half ? k : B - 1 - (k - half);
    int found = -1;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int cand = c0 + lane;
      const int lc = cand < B ? a.context_lens[cand] : -1;
      int rank = 0;
      for (int j0 = 0; j0 < B; j0 += kWave) {
        const int lj_own = j0 + lane < B ? a.context_lens[j0 + lane] : -1;
        const int n = min(kWave, B - j0);
        for (int jj = 0; jj < n; ++jj) {
          const int lj = __builtin_amdgcn_readlane(lj_own, jj);
          const int j = j0 + jj;
          rank += (lj > lc || (lj == lc && j < cand)) ? 1 : 0;
        }
      }
      const unsigned long long hit = __ballot(cand < B && rank == r);
      if (found < 0 && hit) found = c0 + __builtin_ctzll(hit);
    }
    found = uni(found);
    if (found >= 0) unit = found * a.hkv + hh;
    item = unit;  // one chunk per unit: the item state follows the unit
  }
  const int chunk = item / n_units;
  const int b = unit / a.hkv;
  const int h = unit % a.hkv;

  UnitView u;
  u.hkv = a.hkv;
  u.h = h;
  u.num_pages = a.num_pages;
  int bad_input = 0;
  {
    const int len = sload(a.context_lens + b);
    const long long cap = PAGED ? (long long)a.max_pages * a.page_size : (long long)a.max_ctx;
    bad_input = (len < 0) || ((long long)len > cap);
    u.n_ctx = len < 0 ? 0 : ((long long)len > cap ? (int)cap : len);
  }
  u.n_blocks = (u.n_ctx + kBlk - 1) / kBlk;
  if constexpr (PAGED) {
    u.log2_page = 31 - __builtin_clz(a.page_size);
    u.row_pages = a.max_pages;
    u.n_pages = (u.n_ctx + a.page_size - 1) >> u.log2_page;
    u.bt = a.block_table + (size_t)b * a.max_pages;
    u.k = (const char*)a.k;
    u.v = (const char*)a.v;
  } else {
    u.log2_page = 0;
    u.row_pages = 0;
    u.n_pages = 0;
    u.bt = nullptr;
    const size_t base = ((size_t)b * a.hkv + h) * (size_t)a.max_ctx * ROW;
    u.k = (const char*)a.k + base;
    u.v = (const char*)a.v + base;
  }
  u.kept = nullptr;
  u.zero_pos = -1;
  u.n_trav = u.n_blocks;
  if (a.kept_blocks) {
    u.kept = a.kept_blocks + ((size_t)b * a.hkv + h) * a.max_kept;
    u.n_trav = sload(a.kept_count + unit);
  }
  const int t_begin = chunk * a.chunk_blocks;
  const int t_end = min(u.n_trav, t_begin + a.chunk_blocks);
  const bool single = a.chunk_blocks >= u.n_trav;  // whole traversal in this work item
  // query vector g of the unit: row g / gh, head h * gh + g % gh
  auto q_index = [&](int g) -> size_t {
    return ((size_t)b * a.rows + g / a.gh) * a.hq + (size_t)h * a.gh + g % a.gh;
  };
  auto out_at = [&](int i) -> float& { return a.out[q_index(i / D) * D + i % D]; };  // i = g * D + dim

  // ---- kept list: validate (device input) and find block 0 --------------
  if (u.kept) {
    if (tid == 0) {
      R.bad = (u.n_trav < 0 || u.n_trav > a.max_kept) ? 1 : 0;
      R.zero_pos = 0x7fffffff;
    }
    __syncthreads();
    if (u.n_trav >= 0 && u.n_trav <= a.max_kept) {
      // GIVEN order: the entries must be distinct.  One bit per block of the
      // sequence, in the V slabs (unused until the first loads), marks the
      // entries seen; the host bounds the sequences' block count by the bits
      // the slabs hold.
      const bool given = a.order == ART_ORDER_GIVEN;
      uint32_t* seen = reinterpret_cast<uint32_t*>(&vbuf[0][0]);
      const int nwords = (u.n_blocks + 31) >> 5;
      const bool fits = nwords <= (int)(sizeof(vbuf) / sizeof(uint32_t));
      if (given && fits) {
        for (int i = tid; i < nwords; i += NT) seen[i] = 0u;
        __syncthreads();
      }
      if (given && !fits && tid == 0) R.bad = 1;
      for (int i = tid; i < u.n_trav; i += NT) {
        const int e = u.kept[i];
        bool lb = e < 0 || e >= u.n_blocks;
        if (!given && i > 0) lb |= e <= u.kept[i - 1];
        if (given && fits && !lb) lb = ((atomicOr(&seen[e >> 5], 1u << (e & 31)) >> (e & 31)) & 1u) != 0;
        if (lb) atomicOr(&R.bad, 1);
        if (e == 0) atomicMin(&R.zero_pos, i);
      }
    }
    __syncthreads();
    const int bad = uni(R.bad);
    const int zp = uni(R.zero_pos);
    __syncthreads();
    if (bad) {
      if (tid == 0) a.items[item] = ItemState{ART_ERR_DEVICE_INPUT, -1};
      if (chunk == 0) {
        for (int i = tid; i < G * D; i += NT) out_at(i) = 0.f;
        if (tid == 0) {
          a.stop_idx[unit] = -1;
          if (a.blocks_issued) a.blocks_issued[unit] = 0;
        }
      }
      return;
    }
    u.zero_pos = zp == 0x7fffffff ? -1 : zp;
  }
  const int item_status = bad_input ? ART_ERR_DEVICE_INPUT : ART_OK;
  if (u.n_trav <= 0 || t_begin >= u.n_trav) {  // nothing (left) to attend to
    if (tid == 0) a.items[item] = ItemState{item_status, 0};
  }
  if (u.n_trav <= 0) {  // out = 0, stop = 0
    if (chunk == 0) {
      for (int i = tid; i < G * D; i += NT) out_at(i) = 0.f;
      if (tid == 0) {
        a.stop_idx[unit] = 0;
        if (a.blocks_issued) a.blocks_issued[unit] = 0;
      }
    }
    return;
  }
  if (t_begin >= t_end) return;  // chunk past this unit's traversal

  // ---- query operand (B of S^T = K q^T): k-step j, lane (lg, c) holds the
  // 16 bytes of chunk 4j + lg of head c % G (heads replicated over columns)
  u32x4 qv[4];
  {
    const char* qrow = (const char*)a.q + q_index(c % G) * D * ES;
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[j] = *(const u32x4*)(qrow + (4 * j + lg) * 16);
  }
  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // ---- per-wave running softmax state -------------------------------------
  // m_c, l_c: running max and mass of head c % G (this lane's S^T column);
  // acc: running output in the O layout (rows = heads, columns = dims)
  float m_c = -INFINITY, l_c = 0.f;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool art_mode = a.mode == ART_MODE_ART;
  const bool detect_only = art_mode && a.detect_only != 0;  // record the stop, read every block
  const Criterion crit{a.crit_hi, a.crit_lo, a.crit_c2, a.crit_tau_lt1 != 0, a.crit_phi_le1 != 0};

  // ---- loads ---------------------------------------------------------------
  u32x4 kr[kLoads];  // K of the current block: [tile][k-step]
  const __attribute__((address_space(3))) uint8_t* vb =
      (const __attribute__((address_space(3))) uint8_t*)&vbuf[wid][0];
  const uint32_t slab = (uint32_t)(uintptr_t)vb;
  // K: load j of tile nt -> token 16 nt + c, chunk 4j + lg.  The first load
  // of a block waits for `dep` (the score maximum), so it overwrites the K
  // registers only after the MFMAs that read them have completed.
  // The four loads of tile nt; tile 0's first load waits for `dep`.
  // Before a walk (no MFMA reads the K registers) the first load needs no
  // dependency: `first` drops it.
  // The lane's offsets are formed at each call from a fresh lane index, so
  // they are not held in registers across the walk.  Contiguous KV takes one
  // path for every block: rows clamped to the sequence's last token, which
  // changes nothing for a full block.
  auto load_k_tile = [&](const BlockAddr& ba, auto ntc, float dep, auto first) {
    constexpr int nt = decltype(ntc)::value;
    constexpr bool kDep = nt == 0 && !decltype(first)::value;
    const int fl = fresh_lane(), flg = fl >> 4, fc = fl & 15;
    const char* base;
    uint32_t off;
    if constexpr (PAGED) {
      base = u.k + (size_t)ba.row[nt] * ROW;
      off = (uint32_t)(fc * ROW + flg * 16);
    } else {
      base = u.k + (size_t)ba.row[0] * ROW;
      off = (uint32_t)(min(16 * nt + fc, uni(ba.nvalid) - 1) * ROW + flg * 16);
    }
    if constexpr (kDep)
      kr[0] = gload16s_after<0>(off, base, dep);
    else
      kr[4 * nt] = gload16s<0>(off, base);
    kr[4 * nt + 1] = gload16s<64>(off, base);
    kr[4 * nt + 2] = gload16s<128>(off, base);
    kr[4 * nt + 3] = gload16s<192>(off, base);
  };
  auto load_k_first = [&](const BlockAddr& ba) {
    static_for<0, kTiles>([&](auto ntc) { load_k_tile(ba, ntc, 0.f, std::true_type{}); });
  };
  // V: the 16 DMAs of a block into this wave's slab (DMA n -> bytes 1024 n);
  // group g is DMAs 4g .. 4g + 3 (16-token group g).  The caller has waited
  // for the LDS reads of the previous block (load_v does).
  // V DMA n = 4g + q (tile g, quad q of its 16 tokens): lane (lg, c) carries
  // token 4n + lg, global chunk c ^ 2lg ^ 8(q & 1).  Paged: byte offsets
  // within the 16-token group of rows, one per q; contiguous: rows clamped
  // to the sequence's last token, from the block's first row.
  auto load_v = [&](const BlockAddr& ba) {
    wait_lgkm0();  // LDS reads of the previous block have landed
    const int fl = fresh_lane(), flg = fl >> 4, fc = fl & 15;
    const uint32_t sl = fresh_s(slab);
    if constexpr (PAGED) {
      const uint32_t e = (uint32_t)(flg * ROW + ((fc ^ (2 * flg)) * 16));
      const uint32_t voff[4] = {e, (e ^ 128u) + 4 * ROW, e + 8 * ROW, (e ^ 128u) + 12 * ROW};
      static_for<0, kTiles>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const char* base = u.v + (size_t)ba.row[g] * ROW;
        static_for<0, 4>([&](auto qc) {
          constexpr int q = decltype(qc)::value;
          lds_dma16s(voff[q], base, sl + (4 * g + q) * 1024);
        });
      });
    } else {
      const char* base = u.v + (size_t)ba.row[0] * ROW;
      const int last = uni(ba.nvalid) - 1;
      static_for<0, 4 * kTiles>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        const uint32_t off = (uint32_t)(min(4 * n + flg, last) * ROW + ((fc ^ (2 * flg) ^ (8 * (n & 1))) * 16));
        lds_dma16s(off, base, sl + n * 1024);
      });
    }
    compiler_fence();
  };
  // Transposed V reads (bf16): lane (lg, c) addresses token 4lg + c/4 of a
  // tile, dims 16dt + 4(c%4)..+3, i.e. chunk 2dt + (c%4)/2, half c%2, stored
  // at position (2dt + (c%4)/2) ^ 2(c/4) ^ 8(lg&1) of row c/4 of DMA 4tt + lg.

  int bad_page = 0;
  int issued = 0;
  int stop = -1;  // traversal blocks processed at the stop (ART mode)
  // Split ART: pass 0 walks the whole chunk speculatively, storing block
  // summaries; the look-back then decides the stop; if it lies inside the
  // chunk, pass 1 recomputes the chunk's output up to the stop.  In a split
  // launch a unit whose traversal fits one chunk takes the same path (its
  // look-back finds nothing before it), so the split instantiation carries
  // no code of the chain below.
  const bool split = SPLIT && art_mode;
  bool discard = false;  // the unit stopped before this chunk
  int t_stop = t_end;
  // ART mode in one work item per unit: the stop rule runs as a chain over
  // the positions (below)
  const bool chain = !SPLIT && art_mode;
  if (chain) __builtin_amdgcn_s_setprio(1);  // see link_wait
  if (chain) {
    if (tid == 0) {
      R.stop_at = 0;
      R.detected = 0;
      R.timeout = 0;
      R.head[0].seq = 0;
      R.head[1].seq = 0;
      R.head[0].seqc = 0;
      R.head[1].seqc = 0;
    }
    __syncthreads();
  }

  // ---- split ART: the stop rule over this chunk, by decoupled look-back -------
  // After pass 0 the chunk's block summaries are in LDS.  A scan (one thread
  // per query vector and probe dim) forms the chunk's own prefix numerators
  // Q_j after each of its blocks j, on the chunk's own maximum Ml, and the
  // masses; the chunk's aggregate (Ml, its mass, Q after its last block) is
  // published at once.  The carry (the prefix state P_c, m_c, l_c after the
  // predecessor's last block) is then the inclusive prefix of the nearest
  // predecessor that has published one, merged with the aggregates of the
  // chunks after it, so no chunk waits for its predecessor's own look-back.
  // On the common maximum M = max(m_c, Ml) the prefix numerators are
  // P_j = a P_c + b Q_j with a = 2^(m_c - M), b = 2^(Ml - M), so
  //   |P_j|^2       = a^2 |P_c|^2 + 2ab P_c.Q_j + b^2 |Q_j|^2,
  //   P_j.P_{j-1}   = a^2 |P_c|^2 + ab (P_c.Q_j + P_c.Q_{j-1}) + b^2 Q_j.Q_{j-1}.
  // Eight lanes per position (four query vectors, two halves of the probe
  // dims) form these dot products, hence |x^(t)|^2 and x^(t).x^(t-1) and
  // every check of the chunk at once.
  // The patience counter's passage through a chunk depends on the counter
  // it enters with only through the chunk's leading and trailing stable
  // checks and the first run of `patience` stable checks after its first
  // unstable one; the chunk publishes that descriptor, and the counter
  // entering it is the state of the nearest resolved predecessor carried
  // through the descriptors of the chunks after it.
  // Returns the chunk's blocks up to and including the stop, or -1; sets
  // `discard` when the unit stopped before the chunk.
  // The waves' running state (m, l, output) goes to LDS, where the
  // epilogue merges it; pass-0 results of a split chunk wait there during
  // the look-back.
  auto& E = *reinterpret_cast<EpilogueLds<G, D, W>*>(reinterpret_cast<uint8_t*>(vbuf) + kEpiOff);
  auto stash_waves = [&]() {
    // speculative loads may still be landing in the V slabs and in the K
    // registers (a walk that stopped leaves its prefetch in flight): the K
    // registers are tied to the wait, so none is reused before it
    wait_v_tied<0>(kr);
    __syncthreads();
    if (lane < 16) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *(f32x4*)&E.acc[wid][16 * dt + c][0] = acc[dt];
    }
    if (G > 4 && lane >= 16 && lg < G / 4) {  // rows 4 lg .. 4 lg + 3 hold query vectors of their own
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *(f32x4*)&E.acc[wid][16 * dt + c][4 * lg] = acc[dt];
    }
    if (lane < G) {
      E.m[wid][lane] = m_c;
      E.l[wid][lane] = l_c;
    }
    if (lane == 0) {
      E.issued[wid] = issued;
      E.bad[wid] = bad_page;
    }
    __syncthreads();
  };
  int dev_status = item_status;
  ChunkRec<D>* const recs = SPLIT ? reinterpret_cast<ChunkRec<D>*>(a.carries) + (size_t)unit * a.max_chunks : nullptr;
  // A chunk that will not count (the unit stopped before it) says so in its
  // state word, so that chunks looking back past it stop there too.
  constexpr uint64_t kDiscardWord = 3ull | 4ull | (2ull << 32);
  auto publish_discard = [&]() {
    if (tid == 0) st_sys(&recs[chunk].state, kDiscardWord);
  };
  // The stop (blocks of a chunk up to and including it) that a chunk starting
  // at traversal position tb makes when the patience counter enters it at c,
  // from its descriptor; -1 if none.  A counter that reaches `patience` within
  // the leading stable checks stops at the (patience - c)-th check (the
  // unit's first position has no check).
  auto chunk_stop = [&](int tb, int lead, int run_stop, int cin) -> int {
    if (cin < a.patience && cin + lead >= a.patience) return (tb == 0 ? 1 : 0) + (a.patience - cin);
    return run_stop;
  };
  auto split_lookback = [&]() -> int {
    LookbackLds<D>& RL = *reinterpret_cast<LookbackLds<D>*>(&vbuf[0][0]);
    ChunkRec<D>& co = recs[chunk];
    const int Cn = t_end - t_begin;
    constexpr int NP = D / 4;  // probe dims
    constexpr int NQ = D / 8;  // probe dims per thread in the per-position layout (half of them)
    uint64_t word = 0;         // this chunk's state word (thread 0 writes it)
    wait_vm<0>();     // speculative loads have landed (the V slabs are reused below)
    __syncthreads();  // the block summaries (LDS, written by every wave) are complete
    // ---- the chunk's own prefix: a scan over its blocks per (query vector,
    // probe dim), on the chunk's own maximum; published as its aggregate at
    // once (it needs no other chunk)
    if (tid < 4 * NP + 4) {
      const int g = tid < 4 * NP ? tid / NP : tid - 4 * NP;
      const int gg = g < G ? g : 0;
      float Ml = -INFINITY;
      for (int i = 0; i < Cn; ++i) Ml = fmaxf(Ml, SS.m[i][gg]);
      double acc = 0.0;
      if (tid < 4 * NP) {
        const int q = tid % NP;
        for (int i = 0; i < Cn; ++i) {
          acc = fma((double)SS.ps[i][g][q], (double)__builtin_amdgcn_exp2f(SS.m[i][gg] - Ml), acc);
          RL.Q[i][g][q] = acc;
        }
        if (q == 0) RL.ml[g] = Ml;
      } else {
        for (int i = 0; i < Cn; ++i) {
          acc = fma((double)SS.l[i][gg], (double)__builtin_amdgcn_exp2f(SS.m[i][gg] - Ml), acc);
          RL.lam[i][g] = acc;
        }
      }
    }
    __syncthreads();
    // ---- the carry: look back to the nearest inclusive prefix ---------------------
    // Wave 0 publishes the aggregate (its stores alone, so that its own
    // wait covers them) and raises its flag once the first poll has
    // returned, without holding the other waves.  Lane i of wave 0 watches
    // chunk - 1 - i; before chunk 0 is the unit's start (an empty prefix).
    // The wait ends once some predecessor has its inclusive prefix written
    // and every chunk after it its aggregate; a predecessor that knows the
    // unit stopped before it ends it at once.
    if (wid == 0) {
      for (int e = lane; e < 4 * NP; e += kWave) st_sys(&co.ap[e % NP][e / NP], RL.Q[Cn - 1][e / NP][e % NP]);
      if (lane < 4) {
        st_sys(&co.am[lane], RL.ml[lane]);
        st_sys(&co.al[lane], RL.lam[Cn - 1][lane]);
      }
      int lo;
      for (uint32_t polls = 0;; ++polls) {
        const int jc = chunk - 1 - lane;
        const int s = jc >= 0 ? (int)(ld_sys(&recs[jc].state) & 3ull) : 2;
        if (polls == 0) {
          wait_vm<0>();  // the aggregate's stores are acknowledged
          word = 1;
          if (lane == 0) st_sys(&co.state, word);
        }
        // the unit's stop, once some chunk has published it, lies before this
        // chunk (only the chunk holding it writes it)
        const int us = (lane == 0 && !detect_only) ? ld_sys(&a.unit_stop[unit]) : 0;
        const uint64_t inc = __ballot(s == 2), agg = __ballot(s >= 1), gone = __ballot(s == 3 || us > 0);
        if (gone) {
          lo = -3;
          break;
        }
        const int i0 = inc ? __builtin_ctzll(inc) : 64;
        const uint64_t below = i0 >= 64 ? ~0ull : ((1ull << i0) - 1);
        if (i0 < 64 && (agg & below) == below) {
          lo = chunk - 1 - i0;
          break;
        }
        if (polls >= a.spin_limit) {
          lo = -4;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      if (lane == 0) RL.lb = lo;
    }
    __syncthreads();
    const int lb = uni(RL.lb);
    if (lb < -1) {  // the unit stopped before this chunk (or the wait timed out)
      if (lb == -4) dev_status = ART_ERR_TIMEOUT;
      discard = true;
      publish_discard();
      return -1;
    }
    {  // from here on, indices (and the LDS addresses built on them) are recomputed
    const int tid = wid * kWave + fresh_lane();
    const int lane = tid & (kWave - 1);
    // The records to merge, in order: the inclusive prefix of chunk lb (none
    // for lb = -1), then the aggregates of chunks lb + 1 .. chunk - 1.
    // Thread (query vector, probe dim) folds its element of every record
    // into a running (maximum, sum), and four threads do the same for the
    // mass; the loads of successive records do not wait for one another.
    {
      const int n_rec = (lb >= 0 ? 1 : 0) + (chunk - 1 - lb);
      if (tid < 4 * NP + 4) {
        const bool mass = tid >= 4 * NP;
        const int g = mass ? tid - 4 * NP : tid / NP, q = mass ? 0 : tid % NP, gg = g < G ? g : 0;
        float Mr = -INFINITY;
        double Sr = 0.0;
#pragma unroll 4
        for (int r = 0; r < n_rec; ++r) {
          const bool inc = lb >= 0 && r == 0;
          const ChunkRec<D>& rc = recs[inc ? lb : lb + r + (lb >= 0 ? 0 : 1)];
          const float m2 = ld_sys(inc ? &rc.im[gg] : &rc.am[gg]);
          const double v2 = mass ? ld_sys(inc ? &rc.il[gg] : &rc.al[gg]) : ld_sys(inc ? &rc.ip[q][gg] : &rc.ap[q][gg]);
          const float Mn = fmaxf(Mr, m2);
          Sr = fma((double)__builtin_amdgcn_exp2f(Mr - Mn), Sr, (double)__builtin_amdgcn_exp2f(m2 - Mn) * v2);
          Mr = Mn;
        }
        if (mass) {
          RL.mc[g] = Mr;
          RL.lc[g] = Sr;
        } else {
          RL.pc[g][q] = Sr;
        }
      }
      __syncthreads();
    }
    // ---- every check of the chunk at once ------------------------------------------
    const bool has_carry = chunk > 0;
    const int j = tid >> 3, g = (tid >> 1) & 3, hh = tid & 1;
    const bool on = j < Cn && g < G;
    const int jj = j < Cn ? j : 0, gg = g < G ? g : 0;
    const float Mc = RL.mc[gg], Ml = RL.ml[gg];
    const double Lc = RL.lc[gg];
    const float Ms = fmaxf(Mc, Ml);
    const double ca = has_carry ? (double)__builtin_amdgcn_exp2f(Mc - Ms) : 0.0;
    const double cb = (double)__builtin_amdgcn_exp2f(Ml - Ms);
    const double Lam = RL.lam[jj][gg], Lamp = jj == 0 ? 0.0 : RL.lam[jj - 1][gg];
    const double L = fma(ca, Lc, cb * Lam), Lp = fma(ca, Lc, cb * Lamp);
    double S1 = 0.0, S2 = 0.0, cpc = 0.0, Dj = 0.0, Dp = 0.0;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const double qj = RL.Q[jj][gg][hh * NQ + qq];
      const double qp = jj == 0 ? 0.0 : RL.Q[jj - 1][gg][hh * NQ + qq];
      const double pc = RL.pc[gg][hh * NQ + qq];
      S1 = fma(qj, qj, S1);
      S2 = fma(qj, qp, S2);
      cpc = fma(pc, pc, cpc);
      Dj = fma(pc, qj, Dj);
      Dp = fma(pc, qp, Dp);
    }
    S1 += dpp<kQx1>(S1);  // the two halves of the probe dims
    S2 += dpp<kQx1>(S2);
    cpc += dpp<kQx1>(cpc);
    Dj += dpp<kQx1>(Dj);
    Dp += dpp<kQx1>(Dp);
    // |x|^2 at the predecessor's last position, from the carry
    const double iLc = Lc > 0.0 ? recip_d(Lc) : 0.0;
    double s0 = g < G ? cpc * (iLc * iLc) : 0.0;
    s0 += dpp<kQx2>(s0);  // heads g and g ^ 1
    s0 += dpp<kHalfMirror>(s0);  // heads {0, 1} and {2, 3}
    if (tid == 0) RL.stt[0] = has_carry ? s0 : 0.0;
    const double A = ca * ca * cpc + 2.0 * ca * cb * Dj + cb * cb * S1;
    const double X = ca * ca * cpc + ca * cb * (Dj + Dp) + cb * cb * S2;
    const double iL = recip_d(L), iLp = Lp > 0.0 ? recip_d(Lp) : 0.0;
    double stt = on ? A * (iL * iL) : 0.0, stp = on ? X * (iL * iLp) : 0.0;
    stt += dpp<kQx2>(stt);  // heads g and g ^ 1
    stp += dpp<kQx2>(stp);
    stt += dpp<kHalfMirror>(stt);  // heads {0, 1} and {2, 3}
    stp += dpp<kHalfMirror>(stp);
    if (on && (tid & 7) == 0) RL.stt[j + 1] = stt;
    __syncthreads();
    if (on && (tid & 7) == 0) {
      const double spr = RL.stt[j];
      const bool exists = t_begin + j >= 1;  // a check exists from the second traversal block on
      const bool stable = (spr > 0.0) & (stt > 0.0) & crit.scale_ok(spr, stt) & crit.dir_ok(spr, stt, stp);
      RL.bits[j] = (exists ? 2 : 0) | (stable ? 1 : 0);
    }
    __syncthreads();
    if (wid == 0) {
      // ---- this chunk's inclusive prefix: P after its last block on the
      // common maximum, and the mass there; stored by this wave alone, and
      // announced with the stop rule's state below (after the wait there)
      for (int e = lane; e < 4 * NP; e += kWave) {
        const int g2 = e / NP, q = e % NP, g3 = g2 < G ? g2 : 0;
        const float Mc2 = RL.mc[g3], Ml2 = RL.ml[g3], Ms2 = fmaxf(Mc2, Ml2);
        const double ca2 = has_carry ? (double)__builtin_amdgcn_exp2f(Mc2 - Ms2) : 0.0;
        const double cb2 = (double)__builtin_amdgcn_exp2f(Ml2 - Ms2);
        st_sys(&co.ip[q][g2], fma(ca2, RL.pc[g3][q], cb2 * RL.Q[Cn - 1][g3][q]));
      }
      if (lane < 4) {
        const int g3 = lane < G ? lane : 0;
        const float Mc2 = RL.mc[g3], Ml2 = RL.ml[g3], Ms2 = fmaxf(Mc2, Ml2);
        const double ca2 = has_carry ? (double)__builtin_amdgcn_exp2f(Mc2 - Ms2) : 0.0;
        const double cb2 = (double)__builtin_amdgcn_exp2f(Ml2 - Ms2);
        st_sys(&co.im[lane], Ms2);
        st_sys(&co.il[lane], fma(ca2, RL.lc[g3], cb2 * RL.lam[Cn - 1][g3]));
      }
      // ---- the chunk's patience descriptor (needs no other chunk's stop rule) ------
      const int bt = lane < Cn ? RL.bits[lane] : 0;
      const uint64_t ex = __ballot((bt & 2) != 0), sb = __ballot(bt == 3);
      const uint64_t fail = ex & ~sb;
      const int n_chk = __popcll(ex);
      int lead = n_chk, trail = n_chk, run_stop = -1;
      if (fail) {
        const int f0 = __builtin_ctzll(fail), f1 = 63 - __builtin_clzll(fail);
        lead = __popcll(ex & ((1ull << f0) - 1));
        trail = __popcll(ex & ~((2ull << f1) - 1));
        int cnt = 0;  // a run after the first unstable check
        for (int i = f0 + 1; i < Cn; ++i) {
          if (!((ex >> i) & 1)) continue;
          cnt = ((sb >> i) & 1) ? cnt + 1 : 0;
          if (cnt >= a.patience) {
            run_stop = i + 1;
            break;
          }
        }
      }
      word = 1ull | 4ull | ((uint64_t)n_chk << 3) | ((uint64_t)lead << 8) | ((uint64_t)trail << 13) |
             ((uint64_t)(run_stop + 1) << 18);
      if (lane == 0) st_sys(&co.state, word);  // the descriptor lives in the word itself
      // ---- the stop rule's state entering the chunk ------------------------------------
      // The nearest predecessor whose state is resolved, carried through the
      // descriptors of the chunks after it (each of them must be written).
      // One word per chunk holds both.
      if (lane == 0) RL.found = -1;
      int lo = -1;
      uint64_t wv = 0;
      for (uint32_t polls = 0;; ++polls) {
        const int jc = chunk - 1 - lane;
        wv = jc >= 0 ? ld_sys(&recs[jc].state) : ((1ull << 32) | 4ull);  // before chunk 0: no stop, counter 0
        const uint64_t rb = __ballot((wv >> 32) != 0), db = __ballot(((wv >> 2) & 1) != 0);
        const int i0 = rb ? __builtin_ctzll(rb) : 64;
        const uint64_t below = i0 >= 64 ? ~0ull : ((1ull << i0) - 1);
        if (i0 < 64 && (db & below) == below) {
          lo = i0;
          break;
        }
        if (polls >= a.spin_limit) {
          lo = -4;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      int state;  // as the state word's high half, for this chunk's end
      int own = -1;
      int outcome = 0;  // 0 this chunk counts; 1 the wait timed out; 2 the unit stopped before this chunk
      if (lo < 0) {
        state = 2;  // timed out: end here, and every chunk after
        outcome = 1;
      } else {
        const int base = __builtin_amdgcn_readlane((int)(wv >> 32), lo);
        const int dw = (int)(wv & 0xffffffffu);
        bool stopped = (base & 3) == 2, det = (base & 3) == 3;
        int cnt = base >> 2;
        for (int i = lo - 1; i >= 0 && !stopped; --i) {  // oldest first
          const int d = __builtin_amdgcn_readlane(dw, i);
          const int n = (d >> 3) & 31, ld = (d >> 8) & 31, tr = (d >> 13) & 31, rs = ((d >> 18) & 31) - 1;
          if (!det && chunk_stop((chunk - 1 - i) * a.chunk_blocks, ld, rs, cnt) >= 0) {
            if (detect_only)
              det = true;
            else
              stopped = true;
          }
          cnt = ld == n ? cnt + n : tr;
        }
        if (stopped) {
          state = 2;
          outcome = 2;
        } else {
          own = det ? -1 : chunk_stop(t_begin, lead, run_stop, cnt);
          const int cout = lead == n_chk ? cnt + n_chk : trail;
          if (own >= 0 && !detect_only) {
            state = 2;
          } else {
            state = ((det || own >= 0) ? 3 : 1) | (cout << 2);
          }
          if (own >= 0 && lane == 0) {
            st_sys(&a.unit_stop[unit], t_begin + own);
            RL.found = t_begin + own;  // a unit in one chunk reports it itself
          }
          if (detect_only) own = -1;
        }
      }
      if (lane == 0) {
        RL.stop_local = own;
        RL.outcome = outcome;
      }
      wait_vm<0>();  // the inclusive prefix's and the stop's stores are acknowledged before the state
      word = outcome != 0 ? kDiscardWord : (((word & 0xffffffffull) & ~3ull) | 2ull | ((uint64_t)(uint32_t)state << 32));
      if (lane == 0) st_sys(&co.state, word);
    }
    __syncthreads();
    const int st = uni(RL.stop_local);
    const int outcome = uni(RL.outcome);
    const int found = uni(RL.found);
    if (found >= 0) stop = found;
    __syncthreads();  // the V slabs are free again
    if (outcome == 1) dev_status = ART_ERR_TIMEOUT;
    if (outcome != 0) {  // the unit stopped before this chunk
      discard = true;
      return -1;
    }
    return st;
    }
  };

  // Before its walk a chunk k > 0 learns, in one round trip, whether the
  // unit has stopped before it (a published stop at or before its first
  // block), and, for k >= spec_depth, whether the chunk spec_depth places
  // before it has resolved the stop rule.  The second is the bound on
  // speculation: a chunk walks only once that chunk has resolved (or the
  // unit's stop is seen).  That chunk holds a smaller ticket, so it is
  // running or done, and the wait ends.  Without the bound every chunk
  // handed out walks at once, and with few units nearly all of them lie past
  // the stop.  f takes the resolved state's low bits (2: the unit stopped at
  // or before that chunk's end), 2 for a stop seen published, -1 on timeout.
  if (split && chunk > 0) {
    const bool bound = a.spec_depth > 0 && chunk >= a.spec_depth;
    if (tid == 0) {
      int f;
      uint32_t polls = 0;
      for (;;) {
        const int us = detect_only ? 0 : ld_sys(&a.unit_stop[unit]);
        f = bound ? (int)(ld_sys(&recs[chunk - a.spec_depth].state) >> 32) : 1;
        if (us > 0 && us <= t_begin) {
          f = 2;
          break;
        }
        if (f != 0) break;
        if (++polls >= a.spin_limit) {
          f = -1;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      R.flag = f;
    }
    __syncthreads();
    const int f = uni(R.flag);
    if (f < 0) dev_status = ART_ERR_TIMEOUT;
    if ((f < 0 || (f & 3) == 2) && !detect_only) {  // the unit stopped before this chunk or at the bound
      discard = true;
      publish_discard();
    }
  }
  bool stashed = false;
  // The stop rule as two chains over the positions.  The wave holding
  // position t (t = t_begin + wid, then every W positions)
  //   1. reads the prefix record of position t - 1 (the prefix state on the
  //      probe dims after t - 1), merges its block's summary onto it and
  //      publishes the prefix record of t at once: elementwise work per
  //      lane, no reduction on this chain;
  //   2. forms |x^(t)|^2, x^(t).x^(t-1) and |x^(t-1)|^2 from the two prefix
  //      states (64-lane reductions, off both chains) and the stability of
  //      check t;
  //   3. reads the patience counter after t - 1 (second chain), applies
  //      check t and publishes the counter after t, and the stop if the
  //      counter reaches `patience`.
  // Records alternate by position parity: the record of t - 1 is read (by
  // the wave of t) before the record of t + 1 can be written, since that
  // one needs the record of t; the same holds for each chain on its own.
  // The wave commits its block once the counter after t - 1 is there and
  // shows no stop before t, so no block after the stop is ever committed,
  // and the decision is the one a strictly sequential walk makes.  No
  // workgroup barrier sits in the walk: a wave waits only for its
  // predecessor's records.  A stop, once found, is also published in
  // R.stop_at, which every wave reads before it computes or prefetches a
  // block.
  // Waits until sequence word `seq` (the head's seq or seqc) of position
  // t - 1 reads t; false when the unit stopped after at most t blocks
  // (position t does not count).  A poll reads the sequence number, then the
  // stop word; once the sequence number matches, the record is read.  These
  // are ordered LDS reads (LDS serves a wave's accesses in order), and a
  // writer completes the record (and, on a stop, the stop word) before its
  // sequence number, so a matching sequence number vouches for what is read
  // after it.  The poll does not sleep between reads: measured on MI355X,
  // s_sleep 1 there slowed a lone unit's walk by a quarter.  While it polls
  // the wave drops to issue priority 0 (the walking waves run at 1), so
  // that on a SIMD shared with the other workgroup's wave the poll yields
  // to work: measured on MI355X, 1-2% off every chain workload (a lone unit
  // 0.098 -> 0.0965 ms, 512 units 0.401 -> 0.399 ms).  The wait is
  // bounded: past a.spin_limit * 4 polls (far beyond any legitimate wait)
  // the wave records a timeout and publishes a stop after the first block,
  // which ends every wave's walk.
  auto link_wait = [&](int t, const int& seq) -> bool {
    __builtin_amdgcn_s_setprio(0);
    for (uint32_t polls = 0;; ++polls) {
      const int q = uni(lds_get(seq));
      const int st = uni(lds_get(R.stop_at));
      if (st > 0 && st <= t) { __builtin_amdgcn_s_setprio(1); return false; }
      if (q == t) { __builtin_amdgcn_s_setprio(1); return true; }
      if (polls >= 4u * a.spin_limit) {
        if (lane == 0) {
          lds_put(R.timeout, 1);
          lds_put(R.stop_at, 1);
        }
        __builtin_amdgcn_s_setprio(1);
        return false;
      }
    }
  };
  // The walk over positions t_begin + wid, then every W, up to t_stop.
  // Split ART walks a chunk twice when its stop lies inside it: pass 0
  // speculatively over the whole chunk (publishing block summaries), pass 1
  // up to the stop.  The two passes are separate inlined copies.
  auto walk = [&](auto passc) __attribute__((always_inline)) {
    constexpr int pass = decltype(passc)::value;
    int t = t_begin + wid;
    // split ART, pass 0: the unit's stop as read with the block's K (see below)
    int us_seen = 0;
    BlockAddr cur;
    if (t < t_stop) {
      cur = block_addr4<ROW, PAGED>(u, uni(block_at(u, a.order, t)), bad_page);
      load_k_first(cur);
      if constexpr (SPLIT && pass == 0) us_seen = gload_sys(split ? a.unit_stop + unit : a.context_lens);
      load_v(cur);
      ++issued;
    }
    for (; t < t_stop; t += W) {
      const int tn = t + W;
      bool has_next = tn < t_stop;
      if (chain) {  // a stop already found: drop this block, or the next one's loads
        const int sa = uni(lds_get(R.stop_at));
        if (sa > 0 && t >= sa) break;
        if (sa > 0 && tn >= sa) has_next = false;
      }
      BlockAddr nxt = cur;
      if (has_next) nxt = block_addr4<ROW, PAGED>(u, uni(block_at(u, a.order, tn)), bad_page);

      const int nvalid = cur.nvalid;
      // ---- scores S^T[token][head] = k_token . q_head --------------------------
      if constexpr (SPLIT && pass == 0) {
        // this block's K, and the unit's stop read with it (issued between
        // the block's K loads and its V DMAs, so it has landed with this K)
        wait_v_tied_s<kLoads>(kr, us_seen);
        // a published stop lies in an earlier chunk (only the chunk holding
        // the stop writes it, once every chunk before it has walked): the
        // rest of this chunk is past the stop.  The waves may leave at
        // different blocks; the look-back then finds the stop published and
        // discards the chunk for all of them alike.
        if (!detect_only && uni(us_seen) > 0) break;
      } else {
        wait_v_tied<kLoads>(kr);  // this block's K (its 16 V DMAs were issued after it)
      }
      f32x4 S[kTiles];
      static_for<0, kTiles>([&](auto ntc) {
        constexpr int nt = decltype(ntc)::value;
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DT == ART_DT_BF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[4 * nt + j]),
                                                           __builtin_bit_cast(bf16x8, qv[j]), sacc, 0, 0, 0);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(u2f(kr[4 * nt + j][e]), u2f(qv[j][e]), sacc, 0, 0, 0);
        }
        S[nt] = sacc;
      });
      // ---- online softmax of head c % G against its running max ---------------
      const int tb = 4 * lg;  // token of register 0 within each tile
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sv = (16 * nt + tb + r < nvalid) ? S[nt][r] * c2 : -INFINITY;
          S[nt][r] = sv;
          mx = fmaxf(mx, sv);
        }
      mx = col_max(mx);
      const float m_new = fmaxf(m_c, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_c - m_new);
      float ls = 0.f;
      // the next block's K, one tile at a time between the tiles'
      // exponentials: the wave computes while the address unit drains.  With
      // no next block the loads still go out, to this block's own addresses
      // (read a moment ago, so mostly from L2): every iteration then issues
      // the same 16 K loads and 16 V loads whatever the path, which keeps
      // the explicit vmcnt waits path independent.
      static_for<0, kTiles>([&](auto ntc) {
        constexpr int nt = decltype(ntc)::value;
        load_k_tile(nxt, ntc, mx, std::false_type{});
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(S[nt][r] - m_new);
          S[nt][r] = p;
          ls += p;
        }
      });
      if (has_next) ++issued;
      const float lblk = col_sum(ls);
      // ---- P V on MFMA ---------------------------------------------------------
      f32x4 bacc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) bacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // V of this block: the 16 K loads of the next block were issued after it
      wait_vm<kLoads>();
      const bool partial = nvalid < kBlk;  // weights of the tail tokens are 0; their V may be garbage
      if constexpr (DT == ART_DT_BF16) {
        // A operand of tile pair jp: element e < 4 is token 16(2jp) + 4lg + e,
        // element e >= 4 is token 16(2jp+1) + 4lg + e - 4, split as P = hi + lo
        u32x4 ph[2], pl[2];
#pragma unroll
        for (int jp = 0; jp < 2; ++jp)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int nt = 2 * jp + hh;
            const uint32_t w0 = pk_bf16(S[nt][0], S[nt][1]);
            const uint32_t w1 = pk_bf16(S[nt][2], S[nt][3]);
            ph[jp][2 * hh] = w0;
            ph[jp][2 * hh + 1] = w1;
            pl[jp][2 * hh] = pk_bf16(S[nt][0] - bf16_lo(w0), S[nt][1] - bf16_hi(w0));
            pl[jp][2 * hh + 1] = pk_bf16(S[nt][2] - bf16_lo(w1), S[nt][3] - bf16_hi(w1));
          }
        // B operand of (tile pair jp, dim tile dt): two transposed reads,
        // tokens of tile 2jp then tile 2jp+1, dims 16dt + c.  The lane's
        // offsets are formed here from a fresh lane index, so their eight
        // variants are not held in registers across the walk.
        const int fl = fresh_lane(), flg = fl >> 4, fc = fl & 15;
        const uint32_t trl = (uint32_t)(flg * 1024 + (fc >> 2) * 256 + 8 * (fc & 1));
        const uint32_t trx = (uint32_t)(16 * (((fc & 3) >> 1) | (2 * (fc >> 2)) | (8 * (flg & 1))));
        auto read_b = [&](int jp, int dt, bool mask) -> bf16x8 {
          const auto* pv = vb + trl + (((uint32_t)(32 * dt)) ^ trx);
          s16x4 v0 = lds_read_tr(pv + (2 * jp) * 4096);
          s16x4 v1 = lds_read_tr(pv + (2 * jp + 1) * 4096);
          if (mask) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (32 * jp + tb + e >= nvalid) v0[e] = 0;
              if (32 * jp + 16 + tb + e >= nvalid) v1[e] = 0;
            }
          }
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // per tile pair and group of four dim tiles: the reads first, then the
        // hi MFMAs, then the lo MFMAs (four independent accumulator chains)
        auto pv_pass = [&](int jp, bool mask) {
#pragma unroll
          for (int d0 = 0; d0 < NDT; d0 += 4) {
            bf16x8 bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = read_b(jp, d0 + i, mask);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              bacc[d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph[jp]), bv[i],
                                                                     bacc[d0 + i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              bacc[d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl[jp]), bv[i],
                                                                     bacc[d0 + i], 0, 0, 0);
          }
        };
        if (!partial) {
          pv_pass(0, false);
          pv_pass(1, false);
        } else {  // the last block of a sequence: zero the tail tokens' values
          pv_pass(0, true);
          pv_pass(1, true);
        }
      } else {
        // fp32: k = lg of step (nt, r) is token 16nt + 4lg + r; B element
        // (token, dim 16dt + c) read directly from the slab
        const auto* vf = (const __attribute__((address_space(3))) float*)vb;
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * nt + tb + r;
            const int zsw = (2 * r) ^ (8 * (lg & 1));
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int pos = (4 * dt + (c >> 2)) ^ zsw;
              float v = vf[((4 * nt + lg) * 1024 + r * 256 + pos * 16 + 4 * (c & 3)) >> 2];
              if (tok >= nvalid) v = 0.f;
              bacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(S[nt][r], v, bacc[dt], 0, 0, 0);
            }
          }
      }

      if constexpr (SPLIT) {
        if (split && pass == 0) {
          // split ART: the block summary goes to LDS for the look-back; probe
          // dim 4 dt + c / 4 of query vector r is register r of bacc[dt] in
          // lane c (c % 4 == 0, c < 16)
          const int jl = t - t_begin;
          if (lane < 16 && (c & 3) == 0) {
            float* sp = &SS.ps[jl][0][c >> 2];  // fixed offsets from here on
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
              for (int r = 0; r < 4; ++r) sp[r * (D / 4) + 4 * dt] = bacc[dt][r];
          }
          if (lane < G) {
            SS.m[jl][lane] = m_new;
            SS.l[jl][lane] = lblk;
          }
        }
      }
      // ---- (ART mode) the block's summary, read back in the stop rule's layout ----
      // It goes through the wave's own V slab, free between this block's P V
      // reads and the next block's V loads.  Probe dim 4p of query vector r
      // (G <= 4: rows r % G) is register r of lane c = 4 (p % 4), tile p / 4,
      // in the O layout's row 0 (more than 4 query vectors: rows 4 lg .. 4 lg
      // + 3 are vectors of their own).
      float mt[NH];
      double lt[NH], ps[NPL];
      if (chain) {
        wait_lgkm0();  // this block's transposed V reads have landed
        auto& sw = *reinterpret_cast<Summary<D, (G > 4 ? G : 4)>*>(&vbuf[wid][0]);
        if constexpr (G <= 4) {
          if (lane < 16 && (c & 3) == 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *(f32x4*)&sw.ps[4 * dt + (c >> 2)][0] = bacc[dt];
          }
        } else {
          if ((c & 3) == 0 && lg < G / 4) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *(f32x4*)&sw.ps[4 * dt + (c >> 2)][4 * lg] = bacc[dt];
          }
        }
        if (lane < G) {
          sw.m[lane] = m_new;
          sw.l[lane] = lblk;
        }
        // this wave's own writes, read back by this wave (LDS keeps a wave's order)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const int g = G <= 4 ? (lg < G ? lg : 0) : lg + 4 * hh;
          mt[hh] = sw.m[g];
          lt[hh] = (double)sw.l[g];
#pragma unroll
          for (int i = 0; i < PPC; ++i) ps[hh * PPC + i] = (double)sw.ps[c * PPC + i][g];
        }
      }
      // V of the next block: after this block's LDS reads (load_v waits for
      // them, and in ART mode for the summary's round trip)
      if constexpr (SPLIT && pass == 0)  // every iteration, whatever the path: the waits count it
        us_seen = gload_sys(split ? a.unit_stop + unit : a.context_lens);
      load_v(nxt);

      bool commit = true, last = false;
      if constexpr (!SPLIT) if (chain) {  // (split ART has no chain)
        // ---- first chain: the prefix state after position t - 1 ---------------
        float Mp[NH];
        double Lp[NH], P[NPL];
        bool go = true;
        if (t > t_begin) {
          const int par = (t - 1) & 1;
          go = uni(link_wait(t, R.head[par].seq) ? 1 : 0) != 0;
          const LaneLink<NPL, NH>& lk = R.link[par][lane];
#pragma unroll
          for (int i = 0; i < NPL; ++i) P[i] = lds_get(lk.p[i]);
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            Lp[hh] = lds_get(lk.l[hh]);
            Mp[hh] = lds_get(lk.m[hh]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < NPL; ++i) P[i] = 0.0;
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            Lp[hh] = 0.0;
            Mp[hh] = -INFINITY;
          }
        }
        if (!go) {  // the unit stopped before this position: the block does not count
          commit = false;
          last = true;
        } else {
          // ---- merge, and publish the state after position t ------------------
          // x = P / L per query vector (scale free): both on the common maximum
          float Mn[NH];
          double Ln[NH], Pn[NPL];
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            Mn[hh] = fmaxf(Mp[hh], mt[hh]);
            const double fa = (double)__builtin_amdgcn_exp2f(Mp[hh] - Mn[hh]);  // 0 before the first block
            const double fb = (double)__builtin_amdgcn_exp2f(mt[hh] - Mn[hh]);
            Ln[hh] = fma(Lp[hh], fa, lt[hh] * fb);
#pragma unroll
            for (int i = 0; i < PPC; ++i) Pn[hh * PPC + i] = fma(P[hh * PPC + i], fa, ps[hh * PPC + i] * fb);
          }
          LaneLink<NPL, NH>& lo = R.link[t & 1][lane];
#pragma unroll
          for (int i = 0; i < NPL; ++i) lo.p[i] = Pn[i];
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            lo.l[hh] = Ln[hh];
            lo.m[hh] = Mn[hh];
          }
          wait_lgkm0();  // the record is in LDS before its sequence number
          if (lane == 0) lds_put(R.head[t & 1].seq, t + 1);
          // ---- |x^(t)|^2, x^(t).x^(t-1), |x^(t-1)|^2 ------------------------------
          double sa = 0.0, sc = 0.0, sb = 0.0;
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            double pa = 0.0, pc = 0.0, pb = 0.0;
#pragma unroll
            for (int i = 0; i < PPC; ++i) {
              const double pn = Pn[hh * PPC + i], pp = P[hh * PPC + i];
              pa = fma(pn, pn, pa);
              pc = fma(pn, pp, pc);
              pb = fma(pp, pp, pb);
            }
            const double in = recip_d(Ln[hh]);
            const double ip = Lp[hh] > 0.0 ? recip_d(Lp[hh]) : 0.0;
            sa = fma(pa, in * in, sa);
            sc = fma(pc, in * ip, sc);
            sb = fma(pb, ip * ip, sb);
          }
          const double keep = (G >= 4 || lg < G) ? 1.0 : 0.0;  // rows past G repeat query vector 0
          double stt = sa * keep, stp = sc * keep, spr = sb * keep;
          allsum3_d(stt, stp, spr);
          // a check exists from the second traversal block on
          const bool exists = t >= 1;
          const bool stable =
              exists & (spr > 0.0) & (stt > 0.0) & crit.scale_ok(spr, stt) & crit.dir_ok(spr, stt, stp);
          // ---- second chain: the patience counter after position t - 1 ----------
          int counter = 0, det = 0;
          if (t > t_begin) {
            const int par = (t - 1) & 1;
            go = uni(link_wait(t, R.head[par].seqc) ? 1 : 0) != 0;
            counter = uni(lds_get(R.head[par].counter));
            det = uni(lds_get(R.head[par].detected));
          }
          if (!go) {
            commit = false;
            last = true;
          } else {
            counter = exists ? (stable ? counter + 1 : 0) : 0;
            int st = (exists && counter >= a.patience) ? t + 1 : 0;
            if (detect_only) {  // keep the first stop, terminate nothing
              if (st > 0 && det == 0) det = st;
              st = 0;
            }
            st = uni(st);
            if (lane == 0) {
              LinkHead& ho = R.head[t & 1];
              ho.counter = counter;
              ho.detected = det;
              if (st > 0) R.stop_at = st;
              if (detect_only && det > 0 && det == t + 1) R.detected = det;
            }
            wait_lgkm0();  // counter and stop are in LDS before the sequence number
            if (lane == 0) lds_put(R.head[t & 1].seqc, t + 1);
            if (st > 0) {
              stop = st;
              last = true;
            }
          }
        }
      }
      // ---- commit this wave's block ----------------------------------------------
      if (commit) {
        // row r of the O layout holds head r % G, whose column values sit in lane r % G
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (G <= 4)
            al[r] = lane_f(alpha, r % G);
          else  // row 4 lg + r is query vector (4 lg + r) % G
            al[r] = __shfl(alpha, (4 * lg + r) % G);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[dt][r] = fmaf(acc[dt][r], al[r], bacc[dt][r]);
        m_c = m_new;
        l_c = fmaf(l_c, alpha, lblk);
      }
      if (last) break;
      cur = nxt;
    }
  };
  if (!discard) {
    walk(std::integral_constant<int, 0>{});
    if (split) {
      stash_waves();
      stashed = true;
      const int stop_local = split_lookback();
      if (!discard && stop_local >= 0 && stop_local < t_end - t_begin) {
        t_stop = t_begin + stop_local;  // recompute the blocks up to the stop
        stashed = false;
        m_c = -INFINITY;
        l_c = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        walk(std::integral_constant<int, 1>{});
      }
    }
  }
  // Every load of the walk has landed before anything below reuses its
  // registers, on every path out of the loop (stash_waves waits as well, but
  // only where it runs).
  wait_v_tied<0>(kr);
  if (!stashed) stash_waves();
  if (chain) {  // every wave has left the walk (stash_waves ends on a barrier)
    const int sa = uni(R.stop_at), dd = uni(R.detected);
    stop = sa > 0 ? sa : (dd > 0 ? dd : t_end);
    if (R.timeout) dev_status = ART_ERR_TIMEOUT;
  }
  if (stop < 0) stop = t_end;

  // ---- epilogue: merge the stashed waves, normalize -----------------------------
  for (int o = tid; o < G * D; o += NT) {
    const int g = o / D, dim = o % D;
    float M = -INFINITY;
    for (int w2 = 0; w2 < W; ++w2)
      if (E.l[w2][g] > 0.f) M = fmaxf(M, E.m[w2][g]);
    float L = 0.f, num = 0.f;
    for (int w2 = 0; w2 < W; ++w2) {
      if (!(E.l[w2][g] > 0.f)) continue;  // a wave with no committed block
      const float s = __builtin_amdgcn_exp2f(E.m[w2][g] - M);
      L = fmaf(E.l[w2][g], s, L);
      num = fmaf(E.acc[w2][dim][g], s, num);
    }
    if (discard) L = 0.f;  // nothing of this chunk counts
    if (single) {
      out_at(o) = num / L;
    } else {
      float* part = a.partials + ((size_t)unit * a.max_chunks + chunk) * G * (D + 2) + g * (D + 2);
      part[2 + dim] = num;
      if (dim == 0) {
        part[0] = M;
        part[1] = L;
      }
    }
  }
  if (tid == 0) {
    int tot = 0, bad = 0;
    for (int w2 = 0; w2 < W; ++w2) {
      tot += E.issued[w2];
      bad |= E.bad[w2];
    }
    a.items[item] = ItemState{bad ? (int)ART_ERR_DEVICE_INPUT : dev_status, tot};
    if (single) {
      a.stop_idx[unit] = stop;
      if (a.blocks_issued) a.blocks_issued[unit] = tot;
    }
  }
}

// ---------------------------------------------------------------------------
// LSE combine of split partials (full mode)
// ---------------------------------------------------------------------------
// One workgroup per unit, one wave per query vector.  Lane k of a wave
// holds chunk k's reference max and mass (64 chunks per pass), so the
// common max and the total mass are wave reductions; the output loop then
// walks the chunks in order with the loads of sixteen chunks in flight.
template <int D, int G>
__global__ __launch_bounds__(kWave * 16) void art_combine_kernel(KernelArgs a) {
  const int unit = blockIdx.x;
  const int b = unit / a.hkv, h = unit % a.hkv;
  int n_ctx = sload(a.context_lens + b);
  const long long cap = a.page_size ? (long long)a.max_pages * a.page_size : (long long)a.max_ctx;
  n_ctx = n_ctx < 0 ? 0 : ((long long)n_ctx > cap ? (int)cap : n_ctx);
  int n_trav = (n_ctx + kBlk - 1) / kBlk;
  if (a.kept_blocks) {
    n_trav = sload(a.kept_count + unit);
    if (n_trav > a.max_kept) return;  // rejected by the decode kernel
  }
  if (n_trav <= 0) return;
  const int n_chunks = (n_trav + a.chunk_blocks - 1) / a.chunk_blocks;
  if (n_chunks <= 1) return;  // written directly by the decode kernel
  if (a.items[unit].issued == -1) return;  // kept list rejected: already reported
  const int lane = threadIdx.x & (kWave - 1);
  const int g = uni((int)(threadIdx.x / kWave));
  const float* part = a.partials + (size_t)unit * a.max_chunks * G * (D + 2);
  constexpr int S = G * (D + 2);  // floats between consecutive chunks of one query vector
  const float* pg = part + g * (D + 2);

  // common reference max over the chunks that hold mass
  float M = -INFINITY;
  for (int k = lane; k < n_chunks; k += kWave) {
    const float l = pg[(size_t)k * S + 1];
    if (l > 0.f) M = fmaxf(M, pg[(size_t)k * S]);
  }
  for (int o = kWave / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
  // total mass
  float L = 0.f;
  for (int k = lane; k < n_chunks; k += kWave) {
    const float l = pg[(size_t)k * S + 1];
    if (l > 0.f) L = fmaf(l, __builtin_amdgcn_exp2f(pg[(size_t)k * S] - M), L);
  }
  for (int o = kWave / 2; o > 0; o >>= 1) L += __shfl_xor(L, o, kWave);

  // numerators, chunk by chunk in order; a chunk without mass weighs 0
  float o0 = 0.f, o1 = 0.f;
  for (int k0 = 0; k0 < n_chunks; k0 += kWave) {
    const int k = k0 + lane;
    float wl = 0.f;
    if (k < n_chunks) {
      const float l = pg[(size_t)k * S + 1];
      wl = l > 0.f ? __builtin_amdgcn_exp2f(pg[(size_t)k * S] - M) : 0.f;
    }
    const int n = min(kWave, n_chunks - k0);
    int j = 0;
    // sixteen chunks' loads in flight at a time, then four, then one; the
    // sums still run over the chunks in order
    for (; j + 16 <= n; j += 16) {
      float x0[16], x1[16], w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* pk = pg + (size_t)(k0 + j + i) * S + 2;
        x0[i] = pk[lane];
        x1[i] = D > kWave ? pk[kWave + lane] : 0.f;
        w[i] = __shfl(wl, j + i, kWave);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o0 = fmaf(x0[i], w[i], o0);
        if (D > kWave) o1 = fmaf(x1[i], w[i], o1);
      }
    }
    for (; j + 4 <= n; j += 4) {
      float x0[4], x1[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* pk = pg + (size_t)(k0 + j + i) * S + 2;
        x0[i] = pk[lane];
        x1[i] = D > kWave ? pk[kWave + lane] : 0.f;
        w[i] = __shfl(wl, j + i, kWave);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0 = fmaf(x0[i], w[i], o0);
        if (D > kWave) o1 = fmaf(x1[i], w[i], o1);
      }
    }
    for (; j < n; ++j) {
      const float* pk = pg + (size_t)(k0 + j) * S + 2;
      const float w = __shfl(wl, j, kWave);
      o0 = fmaf(pk[lane], w, o0);
      if (D > kWave) o1 = fmaf(pk[kWave + lane], w, o1);
    }
  }
  float* dst = a.out + (((size_t)b * a.rows + g / a.gh) * a.hq + (size_t)h * a.gh + g % a.gh) * D;
  dst[lane] = o0 / L;
  if (D > kWave) dst[kWave + lane] = o1 / L;

  if (g == 0) {
    int tot = 0;
    if (a.blocks_issued)
      for (int k = lane; k < n_chunks; k += kWave) tot += a.items[(size_t)k * a.batch * a.hkv + unit].issued;
    for (int o = kWave / 2; o > 0; o >>= 1) tot += __shfl_xor(tot, o, kWave);
    if (lane == 0) {
      int stop = n_trav;
      if (a.split_art) {
        const int us = a.unit_stop[unit];
        if (us > 0) stop = us;
      }
      a.stop_idx[unit] = stop;
      if (a.blocks_issued) a.blocks_issued[unit] = tot;
    }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int DT, int G, bool PAGED>
static hipError_t launch_t(const KernelArgs& a, int grid, int waves, hipStream_t s) {
  if constexpr (G <= 4) {
    if (a.split_art) {
      if (waves != 4) return hipErrorInvalidValue;
      hipLaunchKernelGGL((art_decode_kernel<DT, G, PAGED, true, 4>), dim3(grid), dim3(kWave * 4), 0, s, a);
    } else if (waves == 8) {
      if (a.max_chunks != 1 || a.mode != ART_MODE_ART) return hipErrorInvalidValue;
      hipLaunchKernelGGL((art_decode_kernel<DT, G, PAGED, false, 8>), dim3(grid), dim3(kWave * 8), 0, s, a);
    } else {
      hipLaunchKernelGGL((art_decode_kernel<DT, G, PAGED, false, 4>), dim3(grid), dim3(kWave * 4), 0, s, a);
    }
  } else {  // more than 4 query vectors per unit: no split ART, 4 waves
    if (a.split_art || waves != 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((art_decode_kernel<DT, G, PAGED, false, 4>), dim3(grid), dim3(kWave * 4), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_chunks > 1) {
    hipLaunchKernelGGL((art_combine_kernel<Geo<DT>::D, G>), dim3(a.batch * a.hkv), dim3(kWave * G), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

template <int DT, int G>
static hipError_t launch_g(const KernelArgs& a, int grid, int waves, hipStream_t s) {
  return a.page_size ? launch_t<DT, G, true>(a, grid, waves, s) : launch_t<DT, G, false>(a, grid, waves, s);
}

// Split ART: zero the ticket, the per-unit stops and the chunks' state words (a
// kernel rather than a memset, so the call stays safe to capture in a graph).
template <int D>
__global__ void art_split_init_kernel(KernelArgs a) {
  const int n_units = a.batch * a.hkv;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) a.ws->ticket = 0;
  if (i < n_units) a.unit_stop[i] = 0;
  if (i < n_units * a.max_chunks) {
    reinterpret_cast<ChunkRec<D>*>(a.carries)[i].state = 0;
  }
}

hipError_t launch(const KernelArgs& a, hipStream_t s) {
  const int n_units = a.batch * a.hkv;
  if (a.split_art) {
    const int n = n_units * a.max_chunks;
    if (a.dtype == ART_DT_BF16)
      hipLaunchKernelGGL(art_split_init_kernel<128>, dim3((n + 255) / 256), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(art_split_init_kernel<64>, dim3((n + 255) / 256), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int grid = n_units * a.max_chunks;
  const int waves = a.waves;
  if (waves != 4 && waves != 8) return hipErrorInvalidValue;
  const int G = a.rows * a.gh;  // query vectors per unit
  if (a.dtype == ART_DT_BF16) {
    switch (G) {
      case 1: return launch_g<ART_DT_BF16, 1>(a, grid, waves, s);
      case 2: return launch_g<ART_DT_BF16, 2>(a, grid, waves, s);
      case 4: return launch_g<ART_DT_BF16, 4>(a, grid, waves, s);
      case 8: return launch_g<ART_DT_BF16, 8>(a, grid, waves, s);
      case 16: return launch_g<ART_DT_BF16, 16>(a, grid, waves, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (G) {
    case 1: return launch_g<ART_DT_F32, 1>(a, grid, waves, s);
    case 2: return launch_g<ART_DT_F32, 2>(a, grid, waves, s);
    case 4: return launch_g<ART_DT_F32, 4>(a, grid, waves, s);
    case 8: return launch_g<ART_DT_F32, 8>(a, grid, waves, s);
    case 16: return launch_g<ART_DT_F32, 16>(a, grid, waves, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace art
