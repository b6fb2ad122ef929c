// ART decode attention kernels for gfx950 (MI355X).
//
// Work decomposition.  One workgroup of W waves (W = blockDim.x / 64) owns
// one work item = (unit, chunk): unit = (batch b, kv head h) with its G
// query heads, chunk = a range of positions of the unit's traversal order
// (the whole traversal in ART mode).  The work item is walked in rounds of W
// consecutive traversal positions; wave w takes position t0 + w of round t0.
//
// Per 64-token ART block a wave
//   1. has K in MFMA B-operand registers and V in row order (16-byte loads,
//      issued one round ahead);
//   2. computes the G x 64 scores with v_mfma_f32_16x16x32_bf16
//      (v_mfma_f32_16x16x4_f32 for fp32 inputs); the A operand holds the
//      G query rows replicated over the 16 MFMA rows, so every lane receives
//      the scores of "its" token for all G heads;
//   3. runs the online softmax (running max in the log2 domain) against the
//      wave's running maximum;
//   4. accumulates P V on the VALU in fp32 (P stays fp32);
//   5. (ART mode) publishes a block summary: per head its reference max,
//      its softmax mass and its sums on the probe dims.
// (ART mode) After a barrier every wave merges the summaries of positions up
// to its own onto the carried prefix state (fp64 on the probe dims), so wave
// w holds the probe x^(t) at its position t and x^(t-1); it evaluates the two
// stability metrics there.  After a second barrier every wave runs the
// patience counter over the round's checks in order: the first position
// where `patience` consecutive checks were stable is the stop, blocks after
// it are discarded and no further loads are issued.  The decision is the
// one a strictly sequential walk makes.
//
// Method sources: ART paper section 3.1 Eq. (1) (blockwise attention and the
// partial outputs O^(t)), section 3.2 (probe of scattered head dims);
// gist.science explainer sections 2.2 (scale and direction metrics, dual
// threshold), 2.3 (patience), 2.4 (traversal order, block 0 first).
//
// Lane geometry (both supported element types have 256-byte rows cut into
// 16 chunks of 16 bytes): lane l = 16*lg + c with lg = l / 16, c = l % 16.
//   K (MFMA B operand): load i of tile nt -> token 16*nt + c, chunk 4*i + lg.
//   V (row order)     : load i            -> token 16*lg + i,  chunk c.
// The score of token 16*lg + i sits in lane i of row lg (MFMA tile lg), so
// PV fetches it with a row broadcast instead of an LDS exchange.  PV
// accumulators are partial over the four token groups lg and are summed
// through LDS for the probe and for the output.  For the probe, lane
// (lg, c) owns head lg (when lg < G) and the probe dims inside chunk c.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "art.h"
#include "art_internal.h"

namespace art {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxWaves = 4;      // waves per workgroup (launch bound)
constexpr int kBlk = 64;          // tokens per ART block
constexpr int kTiles = kBlk / 16; // 16-token MFMA tiles per block
constexpr int kRowChunks = 16;    // 16-byte chunks per K/V row
constexpr int kVLoads = kBlk * kRowChunks / kWave;  // 16 row-order loads per block
constexpr int kKLoads = kRowChunks / 4;             // 4 loads per tile per lane

template <int DT>
struct Geo;
template <>
struct Geo<ART_DT_BF16> {
  static constexpr int D = 128, ES = 2, EPC = 8, PPC = 2;  // elements / probe dims per chunk
};
template <>
struct Geo<ART_DT_F32> {
  static constexpr int D = 64, ES = 4, EPC = 4, PPC = 1;
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
#define ART_DPP_I(x, ctrl, rmask) __builtin_amdgcn_update_dpp(0, (x), (ctrl), (rmask), 0xF, false)
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror, row_bcast:15, row_bcast:31
constexpr int kQx1 = 0xB1, kQx2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140, kBcast15 = 0x142, kBcast31 = 0x143;

template <int CTRL, int RMASK = 0xF>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, ART_DPP_I(__builtin_bit_cast(int, x), CTRL, RMASK));
}
template <int CTRL, int RMASK = 0xF>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = ART_DPP_I((int)(uint32_t)u, CTRL, RMASK);
  const int hi = ART_DPP_I((int)(uint32_t)(u >> 32), CTRL, RMASK);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// All-reduce over the 16 lanes of each row (every lane gets its row's result).
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<kQx1>(x));
  x = fmaxf(x, dpp<kQx2>(x));
  x = fmaxf(x, dpp<kHalfMirror>(x));
  return fmaxf(x, dpp<kMirror>(x));
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kQx1>(x);
  x += dpp<kQx2>(x);
  x += dpp<kHalfMirror>(x);
  return x + dpp<kMirror>(x);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ double lane_d(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// All-reduce of an fp64 value over the 16 lanes of each row.
__device__ __forceinline__ double row_sum_d(double x) {
  x += dpp<kQx1>(x);
  x += dpp<kQx2>(x);
  x += dpp<kHalfMirror>(x);
  return x + dpp<kMirror>(x);
}
// Sum over all 64 lanes in fp64, returned uniform.  Rows are reduced with
// mirrors, then row totals are chained with row broadcasts; lane 63 ends
// with the total.
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp<kQx1>(x);
  x += dpp<kQx2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kMirror>(x);
  x += dpp<kBcast15, 0xA>(x);
  x += dpp<kBcast31, 0xC>(x);
  return lane_d(x, 63);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
// acc += bcast_N(p) * v where bcast_N = row_newbcast:N (gfx90a and later):
// every lane of a 16-lane row reads p from lane N of that row.  One fused
// instruction, so the broadcast value never occupies a register.  The
// caller guarantees two wait states between the last VALU write of p and
// the first use (see pv_sources_ready).
template <int N>
__device__ __forceinline__ float fma_bcast(float acc, float p, float v) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
               : "+v"(acc)
               : "v"(p), "v"(v), "n"(N));
  return acc;
}
// Two wait states after the VALU writes of the broadcast sources.
__device__ __forceinline__ void pv_sources_ready(float a, float b, float c, float d) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b), "v"(c), "v"(d));
}

// Sums of 2 x 4 fp64 values at once (one DPP chain shared by all): first
// over the 16 lanes of each row (every lane gets its row's sum), then over
// the four rows (result uniform).
#define ART_STEP8(CTRL, RM)                                \
  _Pragma("unroll") for (int i = 0; i < 4; ++i) {          \
    a[i] += dpp<CTRL, RM>(a[i]);                           \
    b[i] += dpp<CTRL, RM>(b[i]);                           \
  }
__device__ __forceinline__ void row_sum_d8(double (&a)[4], double (&b)[4]) {
  ART_STEP8(kQx1, 0xF)
  ART_STEP8(kQx2, 0xF)
  ART_STEP8(kHalfMirror, 0xF)
  ART_STEP8(kMirror, 0xF)
}
__device__ __forceinline__ void cross_row_sum_d8(double (&a)[4], double (&b)[4]) {
  ART_STEP8(kBcast15, 0xA)
  ART_STEP8(kBcast31, 0xC)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = lane_d(a[i], 63);
    b[i] = lane_d(b[i], 63);
  }
}
#undef ART_STEP8

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
// divisions on the round's critical path.
struct Criterion {
  double hi, lo, c2;   // (1+tau)^2, (1-tau)^2, (1-phi)^2, computed on the host
  bool tau_lt1, phi_le1;
  __device__ bool scale_ok(double a2, double b2) const {
    return b2 < hi * a2 && (!tau_lt1 || b2 > lo * a2);
  }
  __device__ bool dir_ok(double a2, double b2, double p) const {
    const double r = c2 * a2 * b2;
    if (phi_le1) return p > 0.0 && p * p > r;
    return p >= 0.0 || p * p < r;
  }
};

// Reinterpret a 32-bit word as fp32.  Takes the word by value: bit-casting a
// vector-element expression directly reads element 0 with this compiler.
__device__ __forceinline__ float as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

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
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Wait until at most N vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte LDS read issued as inline assembly.  The compiler, which cannot
// count LDS-DMA completions precisely, would otherwise put a full vmcnt(0)
// in front of any read of a DMA-written buffer and so also wait for the
// unrelated V loads in flight.  The caller orders the DMA with wait_vm and
// the result with wait_lgkm_tied.
__device__ __forceinline__ u32x4 lds_read16(const void* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
  return r;
}
// 16-byte global load issued as inline assembly, so the compiler does not
// place its own (over-conservative) vmcnt waits for it; users wait with
// wait_v_tied.
template <int OFF = 0>
__device__ __forceinline__ u32x4 gload16(const void* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(r) : "v"(p), "n"(OFF) : "memory");
  return r;
}
// Wait until at most N vector-memory operations are outstanding, tying the
// 16 V registers to the wait so no use of them is scheduled ahead of it.
template <int N>
__device__ __forceinline__ void wait_v_tied(u32x4 (&v)[16]) {
  asm volatile("s_waitcnt vmcnt(%16)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                 "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                 "+v"(v[15])
               : "n"(N)
               : "memory");
}
// Wait until at most N LDS/scalar operations are outstanding, tying four
// operand registers to the wait so no use of them is scheduled ahead of it.
// LDS operations complete in order, so after issuing reads A then B,
// lgkmcnt(|B|) guarantees A (other outstanding scalar loads only make the
// wait stricter).
template <int N>
__device__ __forceinline__ void wait_lgkm_tied(u32x4 (&k)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]) : "n"(N));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic
// and meets the other waves, without waiting for in-flight global loads (a
// full __syncthreads() would drain the K/V prefetch).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Order LDS traffic between the lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// ---------------------------------------------------------------------------
// LDS layout (one workgroup)
// ---------------------------------------------------------------------------
template <int G, int D>
struct Summary {             // one block, published for the round
  float m[4];                // reference max per head (log2 domain)
  float l[4];                // softmax mass per head relative to m
  float ps[G][D / 4];        // sums on the probe dims relative to m
};
template <int G>
struct alignas(16) WaveLds {
  float probe[4][16][G][2];       // per-token-group sums on probe dims
};
// K of each wave's current block: 16 slabs, one per DMA load n, holding the
// tokens 16*g + n (g = 0..3) as 4 rows of 256 B.  Slabs are 1040 B apart (256
// B rows plus 16 B), so the 16 tokens one MFMA operand read touches (same g,
// n = 0..15) fall into 16 different 16-byte bank groups.  A separate LDS
// object from everything else, so the compiler can tell the DMA target apart
// from the round's bookkeeping.
constexpr int kKSlab = 4 * kRowChunks * 16 + 16;
typedef uint8_t KBuf[kMaxWaves][kVLoads * kKSlab];
template <int G, int D>
struct alignas(16) RoundLds {
  uint8_t q[G][kRowChunks * 16];    // the unit's G query rows (256 B each)
  WaveLds<G> wave[kMaxWaves];
  Summary<G, D> sum[2][kMaxWaves];  // by round parity
  double crit[2][kMaxWaves][4][2];   // by round parity: per position, per head (a, c)
  int bad;
  int zero_pos;
};
template <int G, int EPC>
struct alignas(16) EpilogueLds {   // per-wave final state (reuses the K buffers)
  float m[kMaxWaves][4];
  float l[kMaxWaves][4];
  int issued[kMaxWaves];
  float acc[kMaxWaves][4][16][G][EPC];
};

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------
template <int DT, int G, bool PAGED>
__global__ __launch_bounds__(kWave * kMaxWaves, 2) void art_decode_kernel(KernelArgs a) {
  using GE = Geo<DT>;
  constexpr int D = GE::D, ES = GE::ES, EPC = GE::EPC, PPC = GE::PPC;
  constexpr int ROW = D * ES;
  static_assert(ROW == kRowChunks * 16, "rows must be 16 chunks of 16 bytes");
  __shared__ RoundLds<G, D> R;
  __shared__ alignas(16) KBuf kbuf;
  static_assert(sizeof(EpilogueLds<G, EPC>) <= sizeof(KBuf), "epilogue state must fit the K buffers");

  const int W = blockDim.x >> 6;
  const int wid = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int c = lane & 15;
  WaveLds<G>& wl = R.wave[wid];

  // ---- work item --------------------------------------------------------
  const int n_units = a.batch * a.hkv;
  const int unit = blockIdx.x % n_units;
  const int chunk = blockIdx.x / n_units;
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
    u.n_pages = (u.n_ctx + a.page_size - 1) >> u.log2_page;
    u.bt = a.block_table + (size_t)b * a.max_pages;
    u.k = (const char*)a.k;
    u.v = (const char*)a.v;
  } else {
    u.log2_page = 0;
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
  float* out_rows = a.out + ((size_t)b * a.hq + h * G) * D;

  // ---- kept list: validate (device input) and find block 0 --------------
  if (u.kept) {
    if (threadIdx.x == 0) {
      R.bad = (u.n_trav < 0 || u.n_trav > a.max_kept) ? 1 : 0;
      R.zero_pos = 0x7fffffff;
    }
    __syncthreads();
    if (u.n_trav >= 0 && u.n_trav <= a.max_kept) {
      for (int i = threadIdx.x; i < u.n_trav; i += blockDim.x) {
        const int e = u.kept[i];
        bool lb = e < 0 || e >= u.n_blocks;
        if (a.order != ART_ORDER_GIVEN && i > 0) lb |= e <= u.kept[i - 1];
        if (lb) atomicOr(&R.bad, 1);
        if (e == 0) atomicMin(&R.zero_pos, i);
      }
    }
    __syncthreads();
    const int bad = uni(R.bad);
    const int zp = uni(R.zero_pos);
    __syncthreads();
    if (bad) {
      if (threadIdx.x == 0) atomicMax(&a.ws->error, (int)ART_ERR_DEVICE_INPUT);
      if (chunk == 0) {
        for (int i = threadIdx.x; i < G * D; i += blockDim.x) out_rows[i] = 0.f;
        if (threadIdx.x == 0) {
          a.stop_idx[unit] = -1;
          if (a.blocks_issued) a.blocks_issued[unit] = 0;
        }
      }
      return;
    }
    u.zero_pos = zp == 0x7fffffff ? -1 : zp;
  }
  if (bad_input && chunk == 0 && threadIdx.x == 0) atomicMax(&a.ws->error, (int)ART_ERR_DEVICE_INPUT);

  if (u.n_trav <= 0) {  // nothing to attend to: out = 0, stop = 0
    if (chunk == 0) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) out_rows[i] = 0.f;
      if (threadIdx.x == 0) {
        a.stop_idx[unit] = 0;
        if (a.blocks_issued) a.blocks_issued[unit] = 0;
      }
    }
    return;
  }
  if (t_begin >= t_end) return;  // chunk past this unit's traversal

  // ---- query rows in LDS; per block each lane reads its MFMA A operand
  // (rows replicated: MFMA row r -> head r % G) instead of pinning 16 VGPRs
  {
    const char* qsrc = (const char*)a.q + (((size_t)b * a.hq + h * G) * D) * ES;
    for (int i = threadIdx.x; i < G * kRowChunks; i += blockDim.x)
      *(u32x4*)&R.q[i / kRowChunks][(i % kRowChunks) * 16] = *(const u32x4*)(qsrc + i * 16);
  }
  __syncthreads();
  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // ---- per-wave running softmax state -------------------------------------
  float m_w[G], l_w[G], acc[G][EPC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_w[g] = -INFINITY;
    l_w[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }
  const bool art_mode = a.mode == ART_MODE_ART;
  // prefix state on the probe dims (same in every wave): running max, mass and
  // numerators for head hg = lg (lanes with lg >= G carry head 0 unused),
  // the previous probe, its squared norm, and the patience counter
  const int hg = lg < G ? lg : 0;
  float mP = -INFINITY;
  double lP = 0.0, pP[PPC];
#pragma unroll
  for (int k = 0; k < PPC; ++k) pP[k] = 0.0;
  double stt_last = 0.0;
  int counter = 0;
  const Criterion crit{a.crit_hi, a.crit_lo, a.crit_c2, a.crit_tau_lt1 != 0, a.crit_phi_le1 != 0};

  // ---- loads ---------------------------------------------------------------
  u32x4 vr[kVLoads];
  // Row of token 16*lg of a block (this lane's 16-token group), picked with a
  // select tree (an indexed pick is lowered to a private-memory array).
  auto lane_row = [&](const BlockAddr& ba) -> uint32_t {
    const uint32_t r01 = (lg & 1) ? ba.row[1] : ba.row[0];
    const uint32_t r23 = (lg & 1) ? ba.row[3] : ba.row[2];
    return (lg & 2) ? r23 : r01;
  };
  // K: DMA load n carries token 16*lg + n, chunk c, into slab n.  Rows past a
  // contiguous context are clamped to its last token (read in bounds, masked).
  auto load_k = [&](const BlockAddr& ba) {
    wait_lgkm0();  // operand reads of the previous block have landed
    uint8_t* dst = &kbuf[wid][0];
    if (PAGED || ba.nvalid == kBlk) {
      const char* base = u.k + (size_t)lane_row(ba) * ROW + c * 16;
      static_for<0, kVLoads>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        lds_dma16(base + n * ROW, dst + n * kKSlab);
      });
    } else {
      static_for<0, kVLoads>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        const int tok = min(ba.j * kBlk + 16 * lg + n, u.n_ctx - 1);
        lds_dma16(u.k + (size_t)tok * ROW + c * 16, dst + n * kKSlab);
      });
    }
    compiler_fence();
  };
  // V load i -> token 16*lg + i, chunk c (four 256-byte rows, one per tile).
  auto load_v = [&](const BlockAddr& ba) {
    if (PAGED || ba.nvalid == kBlk) {
      const char* base = u.v + (size_t)lane_row(ba) * ROW + c * 16;
      static_for<0, kVLoads>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        vr[i] = gload16<i * ROW>(base);
      });
    } else {
      static_for<0, kVLoads>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int tok = min(ba.j * kBlk + 16 * lg + i, u.n_ctx - 1);
        vr[i] = gload16(u.v + (size_t)tok * ROW + c * 16);
      });
    }
  };

  int bad_page = 0;
  int issued = 0;
  int stop = -1;  // traversal blocks processed at the stop (ART mode)
  BlockAddr cur;
  if (t_begin + wid < t_end) {
    cur = block_addr<ROW, PAGED>(u, uni(block_at(u, a.order, t_begin + wid)), bad_page);
    load_k(cur);
    load_v(cur);
    ++issued;
  }
  int parity = 0;

  for (int t0 = t_begin; t0 < t_end; t0 += W) {
    const int t = t0 + wid;
    const bool active = t < t_end;
    const int n_act = min(W, t_end - t0);
    const int tn = t + W;
    const bool has_next = tn < t_end;
    BlockAddr nxt = cur;
    if (has_next) nxt = block_addr<ROW, PAGED>(u, uni(block_at(u, a.order, tn)), bad_page);

    float alpha[G], m_new[G], lblk[G];
    float bacc[G][EPC];
    if (active) {
      const int nvalid = cur.nvalid;
      // ---- scores: S[nt][r] = q_{r%G} . k_{16 nt + c} ----------------------
      wait_vm<kVLoads>();  // this block's K (its 16 V loads were issued after it)
      // operand reads run two tiles ahead of the MFMAs
      u32x4 qa[kKLoads];
      u32x4 kb[kTiles][kKLoads];
      auto read_tile = [&](int nt) {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          kb[nt][i] = lds_read16(&kbuf[wid][c * kKSlab + nt * 256 + (4 * i + lg) * 16]);
      };
      f32x4 S[kTiles];
      auto mfma_tile = [&](int nt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DT == ART_DT_BF16) {
#pragma unroll
          for (int i = 0; i < kKLoads; ++i)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[i]),
                                                        __builtin_bit_cast(bf16x8, kb[nt][i]), s, 0, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < kKLoads; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(qa[i][e]), as_f32(kb[nt][i][e]), s, 0, 0, 0);
        }
        S[nt] = s;
      };
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) qa[i] = lds_read16(&R.q[c % G][(4 * i + lg) * 16]);
      read_tile(0);
      read_tile(1);
      wait_lgkm_tied<8>(qa);
      wait_lgkm_tied<4>(kb[0]);
      mfma_tile(0);
      read_tile(2);
      wait_lgkm_tied<4>(kb[1]);
      mfma_tile(1);
      read_tile(3);
      wait_lgkm_tied<4>(kb[2]);
      mfma_tile(2);
      wait_lgkm_tied<0>(kb[3]);
      mfma_tile(3);
      if (has_next) {
        load_k(nxt);
        ++issued;
      }
      // ---- online softmax against the wave's running max --------------------
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) {
          const float sv = (nt * 16 + c < nvalid) ? S[nt][g] * c2 : -INFINITY;
          S[nt][g] = sv;
          mx = fmaxf(mx, sv);
        }
        mx = uni_f(row_max(mx));
        m_new[g] = fmaxf(m_w[g], mx);
        alpha[g] = __builtin_amdgcn_exp2f(m_w[g] - m_new[g]);
        float ls = 0.f;
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) {
          const float pv = __builtin_amdgcn_exp2f(S[nt][g] - m_new[g]);
          S[nt][g] = pv;
          ls += pv;
        }
        lblk[g] = uni_f(row_sum(ls));
      }
      // weights of tile lg (tokens 16*lg + 0..15, one per lane of the row),
      // picked with a select tree
      f32x4 mine;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float s01 = (lg & 1) ? S[1][g] : S[0][g];
        const float s23 = (lg & 1) ? S[3][g] : S[2][g];
        mine[g] = (lg & 2) ? s23 : s01;
      }
      // ---- P V ---------------------------------------------------------------
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPC; ++e) bacc[g][e] = 0.f;
      // V of this block: the 16 K loads of the next block (if any) were issued after it
      if (!has_next) wait_vm<0>();  // no K loads follow this block's V
      wait_v_tied<kVLoads>(vr);
      const float mg[4] = {mine[0], G > 1 ? mine[1] : 0.f, G > 2 ? mine[2] : 0.f, G > 3 ? mine[3] : 0.f};
      pv_sources_ready(mg[0], mg[1], mg[2], mg[3]);
      static_for<0, kVLoads>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int tok = 16 * lg + i;
        u32x4 w = vr[i];
        if (tok >= nvalid) w = u32x4{0u, 0u, 0u, 0u};
        float ve[EPC];
        if constexpr (DT == ART_DT_BF16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ve[2 * k] = bf16_lo(w[k]);
            ve[2 * k + 1] = bf16_hi(w[k]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) ve[k] = as_f32(w[k]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPC; ++e) bacc[g][e] = fma_bcast<i>(bacc[g][e], mg[g], ve[e]);
      });
      if (has_next) {
        compiler_fence();
        load_v(nxt);
      }
    }

    int stop_round = -1;  // this round's stop, as a traversal count
    if (art_mode) {
      // ---- publish the block summary ------------------------------------------
      Summary<G, D>& sw = R.sum[parity][wid];
      if (active) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          wl.probe[lg][c][g][0] = bacc[g][0];
          if (PPC > 1) wl.probe[lg][c][g][1] = bacc[g][PPC > 1 ? 4 : 0];
        }
        wave_lds_sync();
        if (lg < G) {
#pragma unroll
          for (int k = 0; k < PPC; ++k)
            sw.ps[lg][c * PPC + k] = (wl.probe[0][c][lg][k] + wl.probe[1][c][lg][k]) +
                                     (wl.probe[2][c][lg][k] + wl.probe[3][c][lg][k]);
        }
        if (lane < G) {
          float mv = m_new[0], lv = lblk[0];
#pragma unroll
          for (int g = 1; g < G; ++g)
            if (lane == g) mv = m_new[g], lv = lblk[g];
          sw.m[lane] = mv;
          sw.l[lane] = lv;
        }
      }
      lds_barrier();
      // ---- the round's positions, in order ------------------------------------
      // Every wave merges all block summaries of the round onto the prefix
      // state on the probe dims (lane (lg, c): head lg if lg < G, probe dims
      // of chunk c), which keeps that state identical in all waves.  With
      // P^(t) the prefix numerators and l^(t) the prefix mass of a head,
      // x^(t) = P^(t) / l^(t).  At its own position a wave also forms, per
      // head, A = P^(t).P^(t) and C = P^(t).P^(t-1) (row sums), scales them
      // to a = A / l^(t)^2 and c = C / (l^(t) l^(t-1)) and publishes them; the
      // ratio P/l is scale free, so P^(t-1), l^(t-1) keep their own running-
      // max scale.  After a second barrier every wave sums the heads in a
      // fixed order, so all reach the same |x^(t)|^2, x^(t).x^(t-1) and the
      // same decision.
      double own_a = 0.0, own_c = 0.0, l_before = 0.0, l_after = 1.0;
#pragma unroll
      for (int w2 = 0; w2 < kMaxWaves; ++w2) {
        if (w2 < n_act) {
          const Summary<G, D>& s2 = R.sum[parity][w2];
          const float mb = s2.m[hg];
          const float M = fmaxf(mP, mb);
          const double sP = (double)__builtin_amdgcn_exp2f(mP - M);
          const double sB = (double)__builtin_amdgcn_exp2f(mb - M);
          const bool mine = w2 == wid;
          if (mine) l_before = lP;
          lP = fma(lP, sP, (double)s2.l[hg] * sB);
          if (mine) l_after = lP;
          mP = M;
#pragma unroll
          for (int k = 0; k < PPC; ++k) {
            const double p = fma(pP[k], sP, (double)s2.ps[hg][c * PPC + k] * sB);
            if (mine && lg < G) {
              own_a = fma(p, p, own_a);
              own_c = fma(p, pP[k], own_c);
            }
            pP[k] = p;
          }
        }
      }
      if (active) {
        own_a = row_sum_d(own_a);
        own_c = row_sum_d(own_c);
        const double it = recip_d(l_after);
        const double ip = l_before > 0.0 ? recip_d(l_before) : 0.0;
        if (c == 0 && lg < G) {
          R.crit[parity][wid][lg][0] = own_a * (it * it);
          R.crit[parity][wid][lg][1] = own_c * (it * ip);
        }
      }
      lds_barrier();
      // ---- stability checks and patience counter, in traversal order -----------
      double stt_prev = stt_last;
#pragma unroll
      for (int w2 = 0; w2 < kMaxWaves; ++w2) {
        if (w2 < n_act) {
          double stt = 0.0, stp = 0.0;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            stt += R.crit[parity][w2][g][0];
            stp += R.crit[parity][w2][g][1];
          }
          const int cnt = t0 + w2 + 1;
          if (cnt >= 2 && stop_round < 0) {  // a check exists from the second block on
            const bool stable =
                stt_prev > 0.0 && stt > 0.0 && crit.scale_ok(stt_prev, stt) && crit.dir_ok(stt_prev, stt, stp);
            counter = stable ? counter + 1 : 0;
            if (counter >= a.patience) stop_round = cnt;
          }
          stt_prev = stt;
        }
      }
      stt_last = stt_prev;
      stop_round = uni(stop_round);
      parity ^= 1;
    }

    // ---- commit this wave's block (unless it lies after the stop) -------------
    if (active && (stop_round < 0 || t + 1 <= stop_round)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m_w[g] = m_new[g];
        l_w[g] = l_w[g] * alpha[g] + lblk[g];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = fmaf(acc[g][e], alpha[g], bacc[g][e]);
      }
    }
    if (stop_round >= 0) {
      stop = stop_round;
      break;
    }
    cur = nxt;
  }
  if (stop < 0) stop = t_end;

  // ---- epilogue: merge waves, reduce token groups, normalize ---------------
  wait_vm<0>();  // speculative K loads may still be landing in the K buffers
  __syncthreads();
  auto& E = *reinterpret_cast<EpilogueLds<G, EPC>*>(&kbuf[0][0]);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPC; ++e) E.acc[wid][lg][c][g][e] = acc[g][e];
  if (lane < G) {
    float mv = m_w[0], lv = l_w[0];
#pragma unroll
    for (int g = 1; g < G; ++g)
      if (lane == g) mv = m_w[g], lv = l_w[g];
    E.m[wid][lane] = mv;
    E.l[wid][lane] = lv;
  }
  if (lane == 0) E.issued[wid] = issued;
  __syncthreads();
  for (int o = threadIdx.x; o < G * D; o += blockDim.x) {
    const int g = o / D, dim = o % D;
    const int cc = dim / EPC, e = dim % EPC;
    float M = -INFINITY;
    for (int w2 = 0; w2 < W; ++w2)
      if (E.l[w2][g] > 0.f) M = fmaxf(M, E.m[w2][g]);
    float L = 0.f, num = 0.f;
    for (int w2 = 0; w2 < W; ++w2) {
      if (!(E.l[w2][g] > 0.f)) continue;  // a wave with no committed block
      const float s = __builtin_amdgcn_exp2f(E.m[w2][g] - M);
      L = fmaf(E.l[w2][g], s, L);
      const float v = (E.acc[w2][0][cc][g][e] + E.acc[w2][1][cc][g][e]) +
                      (E.acc[w2][2][cc][g][e] + E.acc[w2][3][cc][g][e]);
      num = fmaf(v, s, num);
    }
    if (single) {
      out_rows[o] = num / L;
    } else {
      float* part = a.partials + ((size_t)unit * a.max_chunks + chunk) * G * (D + 2) + g * (D + 2);
      part[2 + dim] = num;
      if (dim == 0) {
        part[0] = M;
        part[1] = L;
      }
    }
  }
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w2 = 0; w2 < W; ++w2) tot += E.issued[w2];
    if (single) {
      a.stop_idx[unit] = stop;
      if (a.blocks_issued) a.blocks_issued[unit] = tot;
    } else {
      atomicAdd(&a.unit_state[unit].issued, tot);
    }
  }
  if (bad_page && lane == 0) atomicMax(&a.ws->error, (int)ART_ERR_DEVICE_INPUT);
}

// ---------------------------------------------------------------------------
// LSE combine of split partials (full mode)
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kWave) void art_combine_kernel(KernelArgs a) {
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
  if (a.kept_blocks && a.stop_idx[unit] == -1) return;  // bad kept list: already reported
  const float* part = a.partials + (size_t)unit * a.max_chunks * G * (D + 2);
  for (int g = 0; g < G; ++g) {
    float M = -INFINITY;
    for (int k = 0; k < n_chunks; ++k)
      if (part[(k * G + g) * (D + 2) + 1] > 0.f) M = fmaxf(M, part[(k * G + g) * (D + 2)]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int k = 0; k < n_chunks; ++k) {
      const float* pk = part + (k * G + g) * (D + 2);
      if (!(pk[1] > 0.f)) continue;
      const float w = __builtin_amdgcn_exp2f(pk[0] - M);
      L = fmaf(pk[1], w, L);
      o0 = fmaf(pk[2 + threadIdx.x], w, o0);
      if (D > kWave) o1 = fmaf(pk[2 + kWave + threadIdx.x], w, o1);
    }
    float* dst = a.out + ((size_t)b * a.hq + h * G + g) * D;
    dst[threadIdx.x] = o0 / L;
    if (D > kWave) dst[kWave + threadIdx.x] = o1 / L;
  }
  if (threadIdx.x == 0) {
    a.stop_idx[unit] = n_trav;
    if (a.blocks_issued) a.blocks_issued[unit] = a.unit_state[unit].issued;
  }
}

// ---------------------------------------------------------------------------
// workspace initialisation (a kernel, not a memset, so the call stays safe
// to capture into a graph)
// ---------------------------------------------------------------------------
__global__ void art_init_kernel(WsHeader* ws, UnitState* st, int n_units) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    ws->error = 0;
    ws->ticket = 0;
  }
  if (i < n_units) {
    st[i].status = 0;
    st[i].stop_chunk = -1;
    st[i].stop_idx = 0;
    st[i].issued = 0;
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int DT, int G, bool PAGED>
static hipError_t launch_t(const KernelArgs& a, int grid, int waves, hipStream_t s) {
  hipLaunchKernelGGL((art_decode_kernel<DT, G, PAGED>), dim3(grid), dim3(kWave * waves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_chunks > 1) {
    hipLaunchKernelGGL((art_combine_kernel<Geo<DT>::D, G>), dim3(a.batch * a.hkv), dim3(kWave), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

template <int DT, int G>
static hipError_t launch_g(const KernelArgs& a, int grid, int waves, hipStream_t s) {
  return a.page_size ? launch_t<DT, G, true>(a, grid, waves, s) : launch_t<DT, G, false>(a, grid, waves, s);
}

hipError_t launch(const KernelArgs& a, hipStream_t s) {
  const int n_units = a.batch * a.hkv;
  hipLaunchKernelGGL(art_init_kernel, dim3((n_units + 255) / 256), dim3(256), 0, s, a.ws, a.unit_state, n_units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = n_units * a.max_chunks;
  const int waves = a.waves < 1 ? 1 : (a.waves > kMaxWaves ? kMaxWaves : a.waves);
  const int G = a.hq / a.hkv;
  if (a.dtype == ART_DT_BF16) {
    if (G == 1) return launch_g<ART_DT_BF16, 1>(a, grid, waves, s);
    if (G == 2) return launch_g<ART_DT_BF16, 2>(a, grid, waves, s);
    return launch_g<ART_DT_BF16, 4>(a, grid, waves, s);
  }
  if (G == 1) return launch_g<ART_DT_F32, 1>(a, grid, waves, s);
  if (G == 2) return launch_g<ART_DT_F32, 2>(a, grid, waves, s);
  return launch_g<ART_DT_F32, 4>(a, grid, waves, s);
}

}  // namespace art
