// Key-based block selection on gfx950: block-mean keys and per-unit kept
// lists, for importance-first traversal and for moving a key-based KV
// selection onto the device.
//
// The gist.science explainer of the ART paper (section 2.4) composes ART
// with KV-cache managers through the traversal sequence of the KV blocks and
// names importance-first as one order; the importance used here (mean query
// . block-mean key) and the kept-list rule are stated in include/art.h.
//
// block_means_kernel: one wave per 64-token block.  Lane (r0, c) reads
// 16-byte chunk c of rows r0, r0 + 4, ..., r0 + 60 (each 256-byte row is 16
// chunks, so four rows per load instruction are contiguous 1 KiB), sums them
// in fp32, and the four r0 lanes of each chunk are summed with two
// cross-lane exchanges.  The kernel is bandwidth-bound (it reads every key
// once, 16 KiB per bf16 block) and meant to run when blocks are written.
//
// select_kernel: one workgroup per unit.  Scores in fp32 (the mean query
// in LDS, one block per thread), then one bitonic sort in LDS of 64-bit keys
// (forced blocks first, then decreasing score, then increasing index) whose
// first n entries are the kept set, and a second sort of those n entries
// into the requested order.  Up to 4096 blocks per unit (48.5 KiB of LDS).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "art.h"
#include "art_internal.h"

namespace art {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelBlk = 64;     // tokens per block
constexpr int kSortMax = 4096;  // blocks per unit the selection sorts
constexpr int kRowBytes = 256;  // one key row (bf16 d = 128 or fp32 d = 64)

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Context length of sequence b clamped to the capacity; `bad` is set when
// clamping was needed.
__device__ __forceinline__ int clamped_len(const SelectArgs& a, int b, int& bad) {
  const int len = a.context_lens[b];
  const long long cap = a.page_size ? (long long)a.max_pages * a.page_size : (long long)a.max_ctx;
  bad |= (len < 0) || ((long long)len > cap);
  return len < 0 ? 0 : ((long long)len > cap ? (int)cap : len);
}

template <int DT, bool PAGED>
__global__ __launch_bounds__(kSelThreads) void block_means_kernel(SelectArgs a) {
  constexpr int D = DT == ART_DT_BF16 ? 128 : 64;
  constexpr int PER = DT == ART_DT_BF16 ? 8 : 4;  // values per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: page ids by scalar loads
  const int item = blockIdx.x;
  const int unit = item / a.groups;
  const int j = (item % a.groups) * 4 + wid;
  const int b = unit / a.hkv, h = unit % a.hkv;
  int bad = 0;
  const int n = clamped_len(a, b, bad);
  const int T = (n + kSelBlk - 1) / kSelBlk;
  const int c = lane & 15, r0 = lane >> 4;
  if (j < T) {
    // all 16 row addresses first (rows past the sequence's end re-read its
    // last row and are masked below), then all 16 loads back to back.  Rows
    // r0 + 4i (r0 < 4) of one i share a page (pages hold a multiple of 16
    // tokens), so the page ids are wave-uniform.
    const int last = n - 1;
    const int32_t* bt = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
    const int log2p = PAGED ? 31 - __builtin_clz(a.page_size) : 0;
    const char* src[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = min(j * kSelBlk + r0 + 4 * i, last);
      size_t row;
      if constexpr (PAGED) {
        int pg = bt[min(j * kSelBlk + 4 * i, last) >> log2p];
        if ((unsigned)pg >= (unsigned)a.num_pages) {
          bad = 1;
          pg = 0;
        }
        row = ((size_t)pg * a.hkv + h) * a.page_size + (tok & (a.page_size - 1));
      } else {
        row = ((size_t)b * a.hkv + h) * a.max_ctx + tok;
      }
      src[i] = (const char*)a.k + row * kRowBytes + c * 16;
    }
    u32x4v v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load((const u32x4v*)src[i]);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool in = j * kSelBlk + r0 + 4 * i <= last;
      if constexpr (DT == ART_DT_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += in ? __uint_as_float(v[i][e] << 16) : 0.f;
          acc[2 * e + 1] += in ? __uint_as_float(v[i][e] & 0xffff0000u) : 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += in ? __uint_as_float(v[i][e]) : 0.f;
      }
    }
    // the four row groups of each chunk: lanes c, c + 16, c + 32, c + 48
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    if (r0 == 0) {
      const float cnt = (float)min(kSelBlk, n - j * kSelBlk);
      float* dst = a.means + ((size_t)unit * a.max_blocks + j) * D + c * PER;
#pragma unroll
      for (int e = 0; e < PER; e += 4)
        *(f32x4v*)(dst + e) = f32x4v{acc[e] / cnt, acc[e + 1] / cnt, acc[e + 2] / cnt, acc[e + 3] / cnt};
    }
  }
  // one status per workgroup: a bad page id may be seen by any of its waves
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    const int done = max(0, min(4, T - (item % a.groups) * 4));
    a.items[item] = ItemState{bad ? (int)ART_ERR_DEVICE_INPUT : (int)ART_OK, done};
    if (item == 0) {
      a.ws->magic = kWsMagic;
      a.ws->n_items = (int)gridDim.x;
    }
  }
}

// Order-preserving map of a score to 32 bits, reversed so that a higher
// score gives a smaller key; never 0 (0 marks a forced block).  -0 is folded
// into +0 first, so equal scores always tie.
__device__ __forceinline__ uint32_t desc_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return max(~ord, 1u);
}

// Ascending bitonic sort of key[0, P) (P a power of two), whole workgroup.
__device__ __forceinline__ void bitonic_sort(uint64_t* key, int P, int tid) {
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += kSelThreads) {
        const int l = i ^ jj;
        if (l > i) {
          const uint64_t x = key[i], y = key[l];
          if ((x > y) == ((i & k) == 0)) {
            key[i] = y;
            key[l] = x;
          }
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <int DT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  constexpr int D = DT == ART_DT_BF16 ? 128 : 64;
  __shared__ float qbar[D];
  __shared__ float score[kSortMax];
  __shared__ uint64_t key[kSortMax];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int b = unit / a.hkv, h = unit % a.hkv;
  const int G = a.hq / a.hkv;
  int bad = 0;
  const int n = clamped_len(a, b, bad);
  const int T = (n + kSelBlk - 1) / kSelBlk;  // <= t_max <= kSortMax (host check)

  // ---- mean query of the unit's G heads ------------------------------------
  for (int d = tid; d < D; d += kSelThreads) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) {
      const size_t idx = ((size_t)b * a.hq + h * G + g) * D + d;
      s += DT == ART_DT_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)a.q)[idx] << 16)
                             : ((const float*)a.q)[idx];
    }
    qbar[d] = s / (float)G;
  }
  __syncthreads();
  // ---- scores: mean query . block-mean key ---------------------------------
  for (int j = tid; j < T; j += kSelThreads) {
    const float* m = a.means + ((size_t)unit * a.max_blocks + j) * D;
    float s = 0.f;
    for (int d = 0; d < D; d += 4) {
      const f32x4v v = *(const f32x4v*)(m + d);
      s = fmaf(v[0], qbar[d], s);
      s = fmaf(v[1], qbar[d + 1], s);
      s = fmaf(v[2], qbar[d + 2], s);
      s = fmaf(v[3], qbar[d + 3], s);
    }
    score[j] = s;
  }
  // ---- kept set: forced blocks, then decreasing score, then index ----------
  const int n_keep = T == 0 ? 0 : min(T, (int)ceil((double)a.keep_frac * (double)T));
  const int n_sink = min(a.sink, n_keep);
  const int n_recent = max(0, min(a.recent, n_keep - n_sink));
  const int P = pow2_ceil(max(T, 1));
  __syncthreads();
  for (int i = tid; i < P; i += kSelThreads) {
    uint64_t k = ~0ull;
    if (i < T) {
      const bool forced = i < n_sink || i >= T - n_recent;
      k = ((uint64_t)(forced ? 0u : desc_key(score[i])) << 32) | (uint32_t)i;
    }
    key[i] = k;
  }
  __syncthreads();
  bitonic_sort(key, P, tid);
  // ---- the kept entries in the requested order ------------------------------
  const int P2 = pow2_ceil(max(n_keep, 1));
  for (int i = tid; i < P2; i += kSelThreads) {
    uint64_t k = ~0ull;
    if (i < n_keep) {
      const uint32_t j = (uint32_t)key[i];
      k = a.order == ART_SELECT_IMPORTANCE ? (((uint64_t)desc_key(score[j]) << 32) | j) : (uint64_t)j;
    }
    key[i] = k;  // each thread rewrites only the entries it read
  }
  __syncthreads();
  bitonic_sort(key, P2, tid);
  for (int i = tid; i < n_keep; i += kSelThreads) a.kept_blocks[(size_t)unit * a.max_kept + i] = (int)(uint32_t)key[i];
  if (tid == 0) {
    a.kept_count[unit] = n_keep;
    a.items[unit] = ItemState{bad ? (int)ART_ERR_DEVICE_INPUT : (int)ART_OK, n_keep};
    if (unit == 0) {
      a.ws->magic = kWsMagic;
      a.ws->n_items = (int)gridDim.x;
    }
  }
}

}  // namespace

hipError_t launch_block_means(const SelectArgs& a, hipStream_t s) {
  const int grid = a.batch * a.hkv * a.groups;
  if (a.dtype == ART_DT_BF16) {
    if (a.page_size)
      hipLaunchKernelGGL((block_means_kernel<ART_DT_BF16, true>), dim3(grid), dim3(kSelThreads), 0, s, a);
    else
      hipLaunchKernelGGL((block_means_kernel<ART_DT_BF16, false>), dim3(grid), dim3(kSelThreads), 0, s, a);
  } else {
    if (a.page_size)
      hipLaunchKernelGGL((block_means_kernel<ART_DT_F32, true>), dim3(grid), dim3(kSelThreads), 0, s, a);
    else
      hipLaunchKernelGGL((block_means_kernel<ART_DT_F32, false>), dim3(grid), dim3(kSelThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int grid = a.batch * a.hkv;
  if (a.dtype == ART_DT_BF16)
    hipLaunchKernelGGL((select_kernel<ART_DT_BF16>), dim3(grid), dim3(kSelThreads), 0, s, a);
  else
    hipLaunchKernelGGL((select_kernel<ART_DT_F32>), dim3(grid), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace art
