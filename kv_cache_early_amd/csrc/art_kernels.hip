// ART decode attention kernels for gfx950 (MI355X).
//
// One 64-lane wave owns one work item = (unit, chunk): unit = (batch b, kv
// head h) with its G query heads, chunk = a contiguous range of positions of
// the unit's traversal order.  Per 64-token ART block the wave
//   1. loads K straight into MFMA B-operand registers and V in row order,
//      16-byte loads, one block ahead (software pipeline);
//   2. computes the G x 64 scores with v_mfma_f32_16x16x32_bf16
//      (v_mfma_f32_16x16x4_f32 for fp32 inputs); the A operand holds the
//      G query rows replicated over the 16 MFMA rows, so every lane receives
//      the scores of "its" token for all G heads;
//   3. runs the online softmax (running max in the log2 domain);
//   4. accumulates P V on the VALU in fp32 (P stays fp32);
//   5. builds the probe (dims 0,4,8,... of every head) from fp64 running sums
//      of the per-block contributions and evaluates the two stability
//      metrics and the patience counter; the decision is wave-uniform, and a
//      stopped unit issues no further loads.
//
// Method sources: ART paper section 3.1 Eq. (1) (blockwise attention and
// the partial outputs O^(t)), section 3.2 (probe of scattered head dims);
// gist.science explainer sections 2.2 (scale and direction metrics, dual
// threshold), 2.3 (patience), 2.4 (traversal order, block 0 first).
//
// Lane geometry (both supported element types have 256-byte rows cut into
// 16 chunks of 16 bytes): lane l = 16*lg + c with lg = l / 16, c = l % 16.
//   K (MFMA B operand): load i of tile nt -> token 16*nt + c, chunk 4*i + lg.
//   V (row order)     : load i            -> token 4*i + lg,   chunk c.
// PV accumulators are therefore partial over the four token groups lg and
// are summed through LDS for the probe and for the output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "art.h"
#include "art_internal.h"

namespace art {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlk = 64;          // tokens per ART block
constexpr int kTiles = kBlk / 16; // 16-token MFMA tiles per block
constexpr int kRowChunks = 16;    // 16-byte chunks per K/V row
constexpr int kVLoads = kBlk * kRowChunks / kWave;  // 16 row-order loads per block
constexpr int kKLoads = kRowChunks / 4;             // 4 loads per tile per lane

// ---------------------------------------------------------------------------
// element-type geometry
// ---------------------------------------------------------------------------
template <int DT>
struct Geo;
template <>
struct Geo<ART_DT_BF16> {
  static constexpr int D = 128, ES = 2, EPC = 8, PPC = 2;  // elements / probes per chunk
};
template <>
struct Geo<ART_DT_F32> {
  static constexpr int D = 64, ES = 4, EPC = 4, PPC = 1;
};

// ---------------------------------------------------------------------------
// cross-lane helpers (gfx9 DPP; all 64 lanes active)
// ---------------------------------------------------------------------------
#define ART_DPP(x, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctrl), 0xF, 0xF, false))
#define ART_DPP_I(x, ctrl) __builtin_amdgcn_update_dpp(0, (x), (ctrl), 0xF, 0xF, false)

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kQx1 = 0xB1, kQx2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, ART_DPP(x, kQx1));
  x = fmaxf(x, ART_DPP(x, kQx2));
  x = fmaxf(x, ART_DPP(x, kHalfMirror));
  x = fmaxf(x, ART_DPP(x, kMirror));
  return x;
}
__device__ __forceinline__ float row_sum(float x) {
  x += ART_DPP(x, kQx1);
  x += ART_DPP(x, kQx2);
  x += ART_DPP(x, kHalfMirror);
  x += ART_DPP(x, kMirror);
  return x;
}
#define ART_DPP_D(x, ctrl)                                                              \
  ({                                                                                    \
    uint64_t _u = __builtin_bit_cast(uint64_t, (x));                                    \
    int _lo = ART_DPP_I((int)(uint32_t)_u, ctrl);                                       \
    int _hi = ART_DPP_I((int)(uint32_t)(_u >> 32), ctrl);                               \
    __builtin_bit_cast(double, ((uint64_t)(uint32_t)_hi << 32) | (uint64_t)(uint32_t)_lo); \
  })
__device__ __forceinline__ double row_sum_d(double x) {
  x += ART_DPP_D(x, kQx1);
  x += ART_DPP_D(x, kQx2);
  x += ART_DPP_D(x, kHalfMirror);
  x += ART_DPP_D(x, kMirror);
  return x;
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ double uni_d(double x) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
  uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Reinterpret a 32-bit word as fp32.  Takes the word by value: bit-casting a
// vector-element expression directly reads element 0 with this compiler.
__device__ __forceinline__ float as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// per-unit view of the inputs
// ---------------------------------------------------------------------------
struct UnitView {
  const char* k;         // contiguous: row 0 of (b, h); paged: pool base
  const char* v;
  const int32_t* bt;     // block-table row of b (paged) or null
  const int32_t* kept;   // kept list of (b, h) or null
  int n_ctx;             // tokens in the sequence
  int n_blocks;          // ceil(n_ctx / 64)
  int n_pages;           // ceil(n_ctx / page) (paged)
  int n_trav;            // T'
  int zero_pos;          // GIVEN order: position of block 0 in the list, or -1
  int page;              // page size (0 = contiguous)
  int hkv;               // kv heads
  int h;                 // kv head of this unit
  int num_pages;         // pages in the pool (page ids are checked against it)
  WsHeader* ws;
};

// Context length of sequence b, clamped to what the shape can hold; an
// out-of-range value is recorded as a device input error.
__device__ __forceinline__ int clamped_len(const KernelArgs& a, int b, bool report) {
  const int len = a.context_lens[b];
  const long long cap = a.page_size ? (long long)a.max_pages * a.page_size : (long long)a.max_ctx;
  if (len < 0 || (long long)len > cap) {
    if (report && threadIdx.x == 0) atomicMax(&a.ws->error, (int)ART_ERR_DEVICE_INPUT);
    return len < 0 ? 0 : (int)cap;
  }
  return len;
}

// Block index at traversal position t (uniform).  Block 0, when a candidate,
// comes first; NATURAL ascending, RECENT_FIRST descending, GIVEN list order.
__device__ __forceinline__ int block_at(const UnitView& u, int order, int t) {
  if (!u.kept) {
    if (order == ART_ORDER_NATURAL) return t;
    return t == 0 ? 0 : u.n_blocks - t;  // RECENT_FIRST: [0, T-1, ..., 1]
  }
  const int n = u.n_trav;
  if (order == ART_ORDER_NATURAL) return u.kept[t];
  if (order == ART_ORDER_RECENT_FIRST) {
    const bool has0 = u.kept[0] == 0;
    if (has0) return t == 0 ? 0 : u.kept[n - t];
    return u.kept[n - 1 - t];
  }
  // GIVEN
  if (u.zero_pos < 0) return u.kept[t];
  if (t == 0) return 0;
  return t <= u.zero_pos ? u.kept[t - 1] : u.kept[t];
}

// Page ids covering one 64-token block (uniform).  Page sizes are multiples
// of 16, so a 16-token MFMA tile and a 4-token row-order load never straddle
// a page.  Indices past the sequence's last page are clamped to it: those
// rows are read (in bounds) and then masked.
struct BlockPages {
  int pg[4];
};
__device__ __forceinline__ BlockPages block_pages(const UnitView& u, int j) {
  BlockPages bp;
  if (u.page == 0) return bp;
  const int first = (j * kBlk) / u.page;
  const int npb = u.page >= kBlk ? 1 : kBlk / u.page;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int pg = i < npb ? uni(u.bt[min(first + i, u.n_pages - 1)]) : 0;
    if (pg < 0 || pg >= u.num_pages) {  // never address outside the pool
      if (threadIdx.x == 0) atomicMax(&u.ws->error, (int)ART_ERR_DEVICE_INPUT);
      pg = 0;
    }
    bp.pg[i] = pg;
  }
  return bp;
}
// Uniform base pointer of the row of token j*64 + tb (tb a multiple of 4
// within one page); lanes add their own row / chunk offsets.
template <int ROW>
__device__ __forceinline__ const char* row_base(const UnitView& u, const char* base, const BlockPages& bp,
                                                int j, int tb) {
  if (u.page == 0) return base + (size_t)(j * kBlk + tb) * ROW;
  const int idx = u.page >= kBlk ? 0 : tb / u.page;
  int pg = bp.pg[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) pg = idx == i ? bp.pg[i] : pg;
  return base + (((size_t)pg * u.hkv + u.h) * u.page + (j * kBlk + tb) % u.page) * ROW;
}

// ---------------------------------------------------------------------------
// LDS scratch of one wave
// ---------------------------------------------------------------------------
template <int G, int EPC>
struct alignas(16) Lds {
  union {
    float p[kBlk][4];                 // softmax weights of the block, by token
    float acc[4][16][G][EPC];         // epilogue: per-token-group partial outputs
  };
  float probe[4][16][G][2];           // per-token-group block sums on probe dims
  double red[4][2];                   // per-row partial (|x|^2, x.x_prev)
};

// ---------------------------------------------------------------------------
// the decode kernel
// ---------------------------------------------------------------------------
template <int DT, int G>
__global__ __launch_bounds__(kWave) void art_decode_kernel(KernelArgs a) {
  using GE = Geo<DT>;
  constexpr int D = GE::D, ES = GE::ES, EPC = GE::EPC, PPC = GE::PPC;
  constexpr int ROW = D * ES;
  static_assert(ROW == kRowChunks * 16, "rows must be 16 chunks of 16 bytes");
  __shared__ Lds<G, EPC> lds;

  const int lane = threadIdx.x;
  const int lg = lane >> 4;   // token group / MFMA k-slot group
  const int c = lane & 15;    // chunk / MFMA row-column index

  // ---- work item -------------------------------------------------------
  const int n_units = a.batch * a.hkv;
  const int item = blockIdx.x;
  const int unit = item % n_units;
  const int chunk = item / n_units;
  const int b = unit / a.hkv;
  const int h = unit % a.hkv;

  UnitView u;
  u.ws = a.ws;
  u.num_pages = a.num_pages;
  u.n_ctx = clamped_len(a, b, chunk == 0);
  u.n_blocks = (u.n_ctx + kBlk - 1) / kBlk;
  u.page = a.page_size;
  u.hkv = a.hkv;
  u.h = h;
  if (a.page_size) {
    u.n_pages = (u.n_ctx + a.page_size - 1) / a.page_size;
    u.bt = a.block_table + (size_t)b * a.max_pages;
    u.k = (const char*)a.k;
    u.v = (const char*)a.v;
  } else {
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
    u.n_trav = a.kept_count[(size_t)b * a.hkv + h];
  }

  const int t_begin = chunk * a.chunk_blocks;
  const int t_end = min(u.n_trav, t_begin + a.chunk_blocks);
  if (t_begin >= u.n_trav && !(chunk == 0)) return;

  // ---- validate the kept list (device-side input) ----------------------
  if (u.kept) {
    bool bad = u.n_trav < 0 || u.n_trav > a.max_kept;
    int zp = -1;
    if (!bad) {
      for (int base = 0; base < u.n_trav; base += kWave) {
        const int i = base + lane;
        bool lane_bad = false;
        bool is0 = false;
        if (i < u.n_trav) {
          const int e = u.kept[i];
          lane_bad = e < 0 || e >= u.n_blocks;
          if (a.order != ART_ORDER_GIVEN && i > 0) lane_bad |= e <= u.kept[i - 1];
          is0 = e == 0;
        }
        if (__builtin_amdgcn_ballot_w64(lane_bad)) bad = true;
        const uint64_t z = __builtin_amdgcn_ballot_w64(is0);
        if (z && zp < 0) zp = base + __builtin_ctzll(z);
      }
    }
    if (bad) {
      if (lane == 0) atomicMax(&a.ws->error, (int)ART_ERR_DEVICE_INPUT);
      if (chunk == 0) {
        for (int i = lane; i < G * D; i += kWave) a.out[((size_t)b * a.hq + h * G) * D + i] = 0.f;
        if (lane == 0) {
          a.stop_idx[unit] = -1;
          if (a.blocks_issued) a.blocks_issued[unit] = 0;
        }
      }
      return;
    }
    u.zero_pos = zp;
  }

  if (u.n_trav == 0) {  // nothing to attend to: out = 0, stop = 0
    if (chunk == 0) {
      for (int i = lane; i < G * D; i += kWave) a.out[((size_t)b * a.hq + h * G) * D + i] = 0.f;
      if (lane == 0) {
        a.stop_idx[unit] = 0;
        if (a.blocks_issued) a.blocks_issued[unit] = 0;
      }
    }
    return;
  }

  // ---- query operand (rows replicated: MFMA row r -> head r % G) --------
  const int qhead = c % G;
  const char* qrow = (const char*)a.q + (((size_t)b * a.hq + h * G + qhead) * D) * ES;
  u32x4 qa[kKLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) qa[i] = *(const u32x4*)(qrow + (4 * i + lg) * 16);

  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // ---- state -------------------------------------------------------------
  float m_run[G], l_run[G];
  float acc[G][EPC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[g][e] = 0.f;
  }
  // fp64 probe state of this lane: head lg (if lg < G), probe dims of chunk c
  double pacc[PPC], xprev[PPC];
#pragma unroll
  for (int k = 0; k < PPC; ++k) pacc[k] = 0.0, xprev[k] = 0.0;
  double l64 = 0.0;        // running denominator of head lg (uniform per row)
  double spp = 0.0;        // |x^(t-1)|^2
  int counter = 0;
  int processed = 0;       // traversal blocks folded into the state
  int issued = 0;
  const bool art_mode = a.mode == ART_MODE_ART;
  const double tau = (double)a.eps_scale, phi = (double)a.eps_dir;

  // ---- loads -------------------------------------------------------------
  u32x4 kr[kTiles][kKLoads];
  u32x4 vr[kVLoads];

  // K of tile nt -> token 16*nt + c, chunk 4*i + lg.  Contiguous rows past
  // the context are clamped to the last token (masked later); paged rows stay
  // inside the (clamped) page.
  auto load_k = [&](int jb, const BlockPages& bp) {
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
      const char* row;
      if (u.page == 0) {
        row = u.k + (size_t)min(jb * kBlk + nt * 16 + c, u.n_ctx - 1) * ROW;
      } else {
        row = row_base<ROW>(u, u.k, bp, jb, nt * 16) + c * ROW;
      }
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) kr[nt][i] = *(const u32x4*)(row + (4 * i + lg) * 16);
    }
  };
  // V load i -> token 4*i + lg, chunk c.
  auto load_v = [&](int jb, const BlockPages& bp) {
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const char* row;
      if (u.page == 0) {
        row = u.v + (size_t)min(jb * kBlk + 4 * i + lg, u.n_ctx - 1) * ROW;
      } else {
        row = row_base<ROW>(u, u.v, bp, jb, 4 * i) + lg * ROW;
      }
      vr[i] = *(const u32x4*)(row + c * 16);
    }
  };

  int t = t_begin;
  int j = uni(block_at(u, a.order, t));
  {
    const BlockPages bp0 = block_pages(u, j);
    load_k(j, bp0);
    load_v(j, bp0);
  }
  issued = 1;
  int jn = (t + 1 < t_end) ? uni(block_at(u, a.order, t + 1)) : j;
  BlockPages bpn = block_pages(u, jn);
  int stop = -1;

  for (; t < t_end; ++t) {
    const int nvalid = min(kBlk, u.n_ctx - j * kBlk);

    // ---- scores: S[nt][r] = q_{r%G} . k_{16 nt + c} ------------------------
    f32x4 S[kTiles];
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DT == ART_DT_BF16) {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[i]),
                                                      __builtin_bit_cast(bf16x8, kr[nt][i]), s, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(qa[i][e]), as_f32(kr[nt][i][e]), s, 0, 0, 0);
      }
      S[nt] = s;
    }
    if (t + 1 < t_end) {
      load_k(jn, bpn);
      ++issued;
    }

    // ---- online softmax (log2 domain) -------------------------------------
    float alpha[G], lblk[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
        const bool ok = nt * 16 + c < nvalid;
        const float sv = ok ? S[nt][g] * c2 : -INFINITY;
        S[nt][g] = sv;
        mx = fmaxf(mx, sv);
      }
      mx = uni_f(row_max(mx));
      const float mnew = fmaxf(m_run[g], mx);
      alpha[g] = __builtin_amdgcn_exp2f(m_run[g] - mnew);
      m_run[g] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
        const float pv = __builtin_amdgcn_exp2f(S[nt][g] - mnew);
        S[nt][g] = pv;
        ls += pv;
      }
      lblk[g] = uni_f(row_sum(ls));
      l_run[g] = l_run[g] * alpha[g] + lblk[g];
    }
    // publish this lane's token (16*lg + c) weights; tile lg selected by lane
    {
      f32x4 mine = S[0];
#pragma unroll
      for (int nt = 1; nt < kTiles; ++nt) mine = (lg == nt) ? S[nt] : mine;
      float4 w;
      w.x = mine[0];
      w.y = G > 1 ? mine[1] : 0.f;
      w.z = G > 2 ? mine[2] : 0.f;
      w.w = G > 3 ? mine[3] : 0.f;
      *(float4*)&lds.p[16 * lg + c][0] = w;
    }
    __syncthreads();

    // ---- P V --------------------------------------------------------------
    float bacc[G][EPC];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPC; ++e) bacc[g][e] = 0.f;
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int tok = 4 * i + lg;
      const float4 pw = *(const float4*)&lds.p[tok][0];
      const float pg[4] = {pw.x, pw.y, pw.z, pw.w};
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
        for (int e = 0; e < EPC; ++e) bacc[g][e] = fmaf(pg[g], ve[e], bacc[g][e]);
    }
    if (t + 1 < t_end) load_v(jn, bpn);
    // next-next block: index and pages, consumed by the next iteration's loads
    const int jnn = (t + 2 < t_end) ? uni(block_at(u, a.order, t + 2)) : jn;
    const BlockPages bpnn = (t + 2 < t_end) ? block_pages(u, jnn) : bpn;

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[g][e] = fmaf(acc[g][e], alpha[g], bacc[g][e]);
    ++processed;

    // ---- probe + criterion -------------------------------------------------
    if (art_mode) {
      // block sums on probe dims (elements 0 and 4 of the chunk), per token group
#pragma unroll
      for (int g = 0; g < G; ++g) {
        lds.probe[lg][c][g][0] = bacc[g][0];
        if (PPC > 1) lds.probe[lg][c][g][1] = bacc[g][PPC > 1 ? 4 : 0];
      }
      __syncthreads();
      double sxx = 0.0, sxp = 0.0;
      if (lg < G) {
        double alpha_g = 0.0, lb = 0.0;
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (g == lg) alpha_g = (double)alpha[g], lb = (double)lblk[g];
        l64 = l64 * alpha_g + lb;
        const double inv_l = 1.0 / l64;
#pragma unroll
        for (int k = 0; k < PPC; ++k) {
          const float s = (lds.probe[0][c][lg][k] + lds.probe[1][c][lg][k]) +
                          (lds.probe[2][c][lg][k] + lds.probe[3][c][lg][k]);
          pacc[k] = pacc[k] * alpha_g + (double)s;
          const double x = pacc[k] * inv_l;
          sxx = fma(x, x, sxx);
          sxp = fma(x, xprev[k], sxp);
          xprev[k] = x;
        }
      }
      sxx = row_sum_d(sxx);
      sxp = row_sum_d(sxp);
      if (c == 0) {
        lds.red[lg][0] = sxx;
        lds.red[lg][1] = sxp;
      }
      __syncthreads();
      const double stt = uni_d((lds.red[0][0] + lds.red[1][0]) + (lds.red[2][0] + lds.red[3][0]));
      const double stp = uni_d((lds.red[0][1] + lds.red[1][1]) + (lds.red[2][1] + lds.red[3][1]));
      const int count = t + 1;  // traversal blocks processed so far
      if (count >= 2) {
        const double pa = sqrt(spp), pb = sqrt(stt);
        bool stable = false;
        if (pa > 0.0 && pb > 0.0) {
          const double ds = fabs(pb - pa) / pa;
          const double dd = 1.0 - stp / (pa * pb);
          stable = (ds < tau) && (dd < phi);
        }
        counter = stable ? counter + 1 : 0;
        if (counter >= a.patience) {
          stop = count;
          break;
        }
      }
      spp = stt;
    }
    __syncthreads();
    j = jn;
    jn = jnn;
    bpn = bpnn;
  }
  if (stop < 0) stop = t_end;  // single-chunk: ran to the end

  // ---- epilogue: reduce token groups, normalize, write ----------------------
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPC; ++e) lds.acc[lg][c][g][e] = acc[g][e];
  __syncthreads();
  if (a.chunk_blocks >= u.n_trav) {
    // whole traversal in this work item: write the output directly
    if (lg < G) {
      float l_g = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (g == lg) l_g = l_run[g];
      const float inv = 1.0f / l_g;
      float o[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        o[e] = ((lds.acc[0][c][lg][e] + lds.acc[1][c][lg][e]) + (lds.acc[2][c][lg][e] + lds.acc[3][c][lg][e])) * inv;
      float* dst = a.out + ((size_t)b * a.hq + h * G + lg) * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) *(float4*)(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    }
    if (lane == 0) {
      a.stop_idx[unit] = stop;
      if (a.blocks_issued) a.blocks_issued[unit] = issued;
    }
  } else {
    // split (full mode): write this chunk's partial (m, l, unnormalized acc)
    float* part = a.partials + ((size_t)unit * a.max_chunks + chunk) * G * (D + 2);
    if (lg < G) {
      float o[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        o[e] = (lds.acc[0][c][lg][e] + lds.acc[1][c][lg][e]) + (lds.acc[2][c][lg][e] + lds.acc[3][c][lg][e]);
      float* dst = part + lg * (D + 2) + 2 + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = o[e];
      if (c == 0) {
        float m_g = 0.f, l_g = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (g == lg) m_g = m_run[g], l_g = l_run[g];
        part[lg * (D + 2) + 0] = m_g;
        part[lg * (D + 2) + 1] = l_g;
      }
    }
    if (lane == 0) atomicAdd(&a.unit_state[unit].issued, issued);
  }
}

// ---------------------------------------------------------------------------
// LSE combine of split partials (full mode)
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kWave) void art_combine_kernel(KernelArgs a) {
  const int unit = blockIdx.x;
  const int b = unit / a.hkv, h = unit % a.hkv;
  const int n_ctx = clamped_len(a, b, false);
  const int n_trav = a.kept_blocks ? a.kept_count[unit] : (n_ctx + kBlk - 1) / kBlk;
  if (n_trav <= 0 || n_trav > (a.kept_blocks ? a.max_kept : (1 << 30))) return;  // handled by the decode kernel
  const int n_chunks = (n_trav + a.chunk_blocks - 1) / a.chunk_blocks;
  if (n_chunks <= 1) return;
  if (__builtin_amdgcn_readfirstlane(a.ws->error) != 0) {
    // a kept-list error was recorded; the decode kernel already wrote this unit if bad
  }
  const float* part = a.partials + (size_t)unit * a.max_chunks * G * (D + 2);
  for (int g = 0; g < G; ++g) {
    float M = -INFINITY;
    for (int k = 0; k < n_chunks; ++k) M = fmaxf(M, part[(k * G + g) * (D + 2)]);
    float L = 0.f;
    float o0 = 0.f, o1 = 0.f;
    for (int k = 0; k < n_chunks; ++k) {
      const float* pk = part + (k * G + g) * (D + 2);
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
template <int DT, int G>
static hipError_t launch_t(const KernelArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((art_decode_kernel<DT, G>), dim3(grid), dim3(kWave), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_chunks > 1) {
    hipLaunchKernelGGL((art_combine_kernel<Geo<DT>::D, G>), dim3(a.batch * a.hkv), dim3(kWave), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch(const KernelArgs& a, hipStream_t s) {
  const int n_units = a.batch * a.hkv;
  hipLaunchKernelGGL(art_init_kernel, dim3((n_units + 255) / 256), dim3(256), 0, s, a.ws, a.unit_state, n_units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = n_units * a.max_chunks;
  const int G = a.hq / a.hkv;
  if (a.dtype == ART_DT_BF16) {
    if (G == 1) return launch_t<ART_DT_BF16, 1>(a, grid, s);
    if (G == 2) return launch_t<ART_DT_BF16, 2>(a, grid, s);
    return launch_t<ART_DT_BF16, 4>(a, grid, s);
  }
  if (G == 1) return launch_t<ART_DT_F32, 1>(a, grid, s);
  if (G == 2) return launch_t<ART_DT_F32, 2>(a, grid, s);
  return launch_t<ART_DT_F32, 4>(a, grid, s);
}

}  // namespace art
