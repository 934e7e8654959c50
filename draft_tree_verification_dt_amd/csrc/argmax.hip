// Row-wise arg-max of fp32 target logits: the target's greedy prediction at
// every tree node (DARTree paper, Preliminaries > Speculative Sampling, T = 0),
// and the same scan over Gumbel-perturbed logits: the target's sample at every
// node for exact target-sample matching at T > 0 (same passage, the DFlash
// rule; Experimental Setup > Evaluation Details, T = 1).
//
// Pure streaming work, bound by HBM bandwidth. With at least one row per CU
// every row is one workgroup; fewer rows are cut into chunks so that the
// launch has enough workgroups (a 16-node chain has 16 rows of 152K entries; a
// 2048-node batch has 2048). A workgroup scans its chunk with 16-byte loads,
// several in flight per thread, keeping the first (lowest-index) maximum per
// thread; waves reduce with cross-lane shuffles and the waves through LDS.
// With one chunk per row the result is written directly; otherwise per-chunk
// (value, index) pairs go to the workspace and a second kernel merges them.
// Ties go to the lowest index.
//
// Sampling (Gumbel-max): argmax_j (l_j / T - ln(-ln U_j)) is an exact draw from
// softmax(l / T). The uniforms come from Philox4x32-10 (Salmon et al., "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011) with counter
// (row, j / 4, offset_lo, offset_hi) and key (seed_lo, seed_hi); word j % 4 of
// the output block gives U_j = (2 * (word >> 9) + 1) * 2^-24. One Philox call
// covers the four entries of a 16-byte load. The kernel compares, in fp32,
//   s_j = l_j * (log2(e) / T) - log2(-log2 U_j),
// which is the natural-log score times log2(e) minus a constant, so it ranks
// the vocabulary exactly as the definition does (up to fp32 rounding). Three of
// the four counter words (all but the block index) and the key are uniform
// across a workgroup, so much of the first three rounds is computed once per
// thread (see RowPhilox). The 32x32->64-bit
// multiplies (sixteen lane-varying ones per four entries) put this variant's
// ALU time close to its HBM time.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cfloat>
#include <cmath>
#include <cstdint>

#include "internal.h"

namespace dt {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kChunkQuantum = 4 * kThreads * kUnroll;  // elements; keeps chunks 16-byte aligned

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sampling parameters passed by value; unused by the greedy variant.
struct Gumbel {
  float c;         // log2(e) / T
  uint32_t k0, k1; // Philox key: seed low and high words
  uint32_t o0, o1; // counter words 2 and 3: offset low and high words
};

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;  // round multipliers
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;  // key increments

// Philox4x32-10 of counter (c0, c1, c2, c3) and key (k0, k1), in place.
__device__ inline void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                     uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    // three-input XOR in one VALU op (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
}

// The four Philox words of vocabulary block j (entries 4j .. 4j+3) of a row.
__device__ inline void gumbel_block(const Gumbel& g, uint32_t row, uint32_t j, uint32_t w[4]) {
  uint32_t c0 = row, c1 = j, c2 = g.o0, c3 = g.o1;
  philox4x32_10(c0, c1, c2, c3, g.k0, g.k1);
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

// The same generator for the blocks of one row, restructured: in counter
// (row, j, o0, o1) only word 1, the block index j, differs between the row's
// blocks, so most of the first three rounds is the same for all of them. With
// c0 = j ^ a after round 1 (a, and the other three words, uniform), round 2
// multiplies one lane-varying word (the other product is uniform) and round 3
// likewise; the uniform words are computed once per thread (row_philox) and
// rounds 4-10 run as usual. Sixteen lane-varying products per block instead of
// twenty; the output words are identical.
struct RowPhilox {
  uint32_t a;   // round 1: c0 = j ^ a
  uint32_t d1;  // round 2: c2 = hi(M0 c0) ^ d1
  uint32_t jx;  // round 3: c0 = hi(M1 c2) ^ jx
  uint32_t h;   // round 3: c2 = c3 ^ h
  uint32_t i;   // round 3: c3 = i
  uint32_t k0, k1;
};

__device__ inline RowPhilox row_philox(const Gumbel& g, uint32_t row) {
  RowPhilox r;
  const uint64_t p0 = (uint64_t)kPhiloxM0 * row, p1 = (uint64_t)kPhiloxM1 * g.o0;  // round 1
  r.a = (uint32_t)(p1 >> 32) ^ g.k0;
  const uint32_t b = (uint32_t)p1, c = (uint32_t)(p0 >> 32) ^ g.o1 ^ g.k1, d = (uint32_t)p0;
  const uint64_t q1 = (uint64_t)kPhiloxM1 * c;  // round 2, uniform half
  const uint32_t e = (uint32_t)(q1 >> 32) ^ b ^ (g.k0 + kPhiloxW0), f = (uint32_t)q1;
  r.d1 = d ^ (g.k1 + kPhiloxW1);
  r.jx = f ^ (g.k0 + 2 * kPhiloxW0);
  const uint64_t q0 = (uint64_t)kPhiloxM0 * e;  // round 3, uniform half
  r.h = (uint32_t)(q0 >> 32) ^ (g.k1 + 2 * kPhiloxW1);
  r.i = (uint32_t)q0;
  r.k0 = g.k0;
  r.k1 = g.k1;
  return r;
}

// The four Philox words of block j of the row that rp describes.
__device__ inline void gumbel_block_row(const RowPhilox& rp, uint32_t j, uint32_t w[4]) {
  const uint64_t p0 = (uint64_t)kPhiloxM0 * (j ^ rp.a);  // round 2
  uint32_t c2 = (uint32_t)(p0 >> 32) ^ rp.d1, c3 = (uint32_t)p0;
  const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;  // round 3
  uint32_t c0 = (uint32_t)(p1 >> 32) ^ rp.jx, c1 = (uint32_t)p1;
  c2 = c3 ^ rp.h;
  c3 = rp.i;
  uint32_t k0 = rp.k0 + 3 * kPhiloxW0, k1 = rp.k1 + 3 * kPhiloxW1;
#pragma unroll
  for (int r = 3; r < 10; ++r) {
    if (r > 3) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t q0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t q1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(q1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(q0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)q1;
    c3 = (uint32_t)q0;
    c0 = n0;
    c2 = n2;
  }
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

// s = l * log2(e)/T - log2(-log2 U), U = (2 * (w >> 9) + 1) * 2^-24. The
// subtraction is exact: 1 + k 2^-23 minus (1 - 2^-24) is (2k + 1) 2^-24. Both
// logarithms see normal inputs (U >= 2^-24, -log2 U >= 8.5e-8).
__device__ inline float gumbel_score(float l, uint32_t w, float c) {
  const float u = __uint_as_float(0x3F800000u | (w >> 9)) - __uint_as_float(0x3F7FFFFFu);
  const float e = -__builtin_amdgcn_logf(u);
  return fmaf(l, c, -__builtin_amdgcn_logf(e));
}

// A thread visits its entries in increasing index order, so within a thread a
// strictly larger value is the only way to improve (the lowest index of a tie
// is already held). Across threads and chunks the index breaks ties.
#define TAKE_IF_LARGER(val, idx) \
  if ((val) > bv) {              \
    bv = (val);                  \
    bi = (idx);                  \
  }

// Is (v, i) a better arg-max candidate than (bv, bi)? Larger value, then lower index.
__device__ inline bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

__device__ inline void wave_reduce(float& bv, int& bi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

template <int THREADS>
__device__ inline void block_reduce(float& bv, int& bi) {
  __shared__ float sv[THREADS / 64];
  __shared__ int si[THREADS / 64];
  wave_reduce(bv, bi);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < THREADS / 64; ++k)
      if (better(sv[k], si[k], bv, bi)) {
        bv = sv[k];
        bi = si[k];
      }
  }
}

// Value compared for entry t of a row: the logit, or its Gumbel score.
template <bool SAMPLE>
__device__ inline float entry_value(float l, int64_t t, uint32_t row, const Gumbel& g) {
  if (!SAMPLE) return l;
  uint32_t w[4];
  gumbel_block(g, row, (uint32_t)(t >> 2), w);
  const int k = (int)(t & 3);
  const uint32_t wk = k == 0 ? w[0] : k == 1 ? w[1] : k == 2 ? w[2] : w[3];
  return gumbel_score(l, wk, g.c);
}

// Gumbel scores of the four entries of vocabulary block j.
__device__ inline f32x4 gumbel4(f32x4 v, const RowPhilox& rp, uint32_t j, float c) {
  uint32_t w[4];
  gumbel_block_row(rp, j, w);
  v.x = gumbel_score(v.x, w[0], c);
  v.y = gumbel_score(v.y, w[1], c);
  v.z = gumbel_score(v.z, w[2], c);
  v.w = gumbel_score(v.w, w[3], c);
  return v;
}

// grid: (chunks, rows). VEC: row starts are 16-byte aligned. SAMPLE: compare
// Gumbel scores instead of logits. THREADS x UNROLL 16-byte loads in flight.
template <bool VEC, bool SAMPLE, int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void argmax_chunks(const float* __restrict__ x, int64_t vocab, int64_t stride,
                                                          int64_t chunk_len, int chunks, int32_t* __restrict__ out_idx,
                                                          float2* __restrict__ part, const Gumbel g) {
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const float* xr = x + row * stride;
  const int64_t beg = (int64_t)c * chunk_len;
  const int64_t end = std::min<int64_t>(vocab, beg + chunk_len);
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (VEC) {
    const RowPhilox rp = SAMPLE ? row_philox(g, (uint32_t)row) : RowPhilox{};
    const int64_t beg4 = beg >> 2, end4 = end >> 2;  // full float4s; beg is a multiple of 4
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    int64_t j = beg4 + threadIdx.x;
    constexpr int64_t kGroup = (int64_t)UNROLL * THREADS;  // entries (float4s) of one group of loads
    auto scan_group = [&](f32x4* v, int64_t jj) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int base = (int)((jj + u * THREADS) << 2);
        if (SAMPLE) v[u] = gumbel4(v[u], rp, (uint32_t)(jj + u * THREADS), g.c);
        TAKE_IF_LARGER(v[u].x, base);
        TAKE_IF_LARGER(v[u].y, base + 1);
        TAKE_IF_LARGER(v[u].z, base + 2);
        TAKE_IF_LARGER(v[u].w, base + 3);
      }
    };
    if (!SAMPLE) {
      // Greedy: UNROLL loads per thread, then their compares (measured faster
      // here than keeping the next group in flight during the compares).
      for (; j + (UNROLL - 1) * THREADS < end4; j += kGroup) {
        f32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(x4 + j + u * THREADS);
        scan_group(v, j);
      }
    } else {
      // Sampling: the Philox arithmetic is long, so the next group's loads
      // are in flight while this one is scored (double-buffered). Pairs of
      // groups per iteration, with no exit between a group's loads and its
      // compares, so that neither the scheduler (the barrier) nor the
      // optimiser moves the loads below the previous group's work; the last
      // prefetch of an even count re-reads the current group (in range, unused).
      const int64_t groups =
          end4 > j + (UNROLL - 1) * THREADS ? (end4 - j - (UNROLL - 1) * THREADS - 1) / kGroup + 1 : 0;
      auto load_group = [&](f32x4* v, int64_t jj) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(x4 + jj + u * THREADS);
        __builtin_amdgcn_sched_barrier(0);
      };
      if (groups > 0) {
        f32x4 va[UNROLL], vb[UNROLL];
        load_group(va, j);
        int64_t gq = 0;
        for (; gq + 2 <= groups; gq += 2) {
          load_group(vb, j + kGroup);
          scan_group(va, j);
          load_group(va, gq + 2 < groups ? j + 2 * kGroup : j);
          scan_group(vb, j + kGroup);
          j += 2 * kGroup;
        }
        if (gq < groups) {
          scan_group(va, j);
          j += kGroup;
        }
      }
    }
    for (; j < end4; j += THREADS) {
      f32x4 v = __builtin_nontemporal_load(x4 + j);
      const int base = (int)(j << 2);
      if (SAMPLE) v = gumbel4(v, rp, (uint32_t)j, g.c);
      TAKE_IF_LARGER(v.x, base);
      TAKE_IF_LARGER(v.y, base + 1);
      TAKE_IF_LARGER(v.z, base + 2);
      TAKE_IF_LARGER(v.w, base + 3);
    }
    for (int64_t t = (end4 << 2) + threadIdx.x; t < end; t += THREADS) {
      const float v = entry_value<SAMPLE>(xr[t], t, (uint32_t)row, g);
      TAKE_IF_LARGER(v, (int)t);
    }
  } else {
    for (int64_t t = beg + threadIdx.x; t < end; t += THREADS) {
      const float v = entry_value<SAMPLE>(xr[t], t, (uint32_t)row, g);
      TAKE_IF_LARGER(v, (int)t);
    }
  }
  block_reduce<THREADS>(bv, bi);
  if (threadIdx.x == 0) {
    if (chunks == 1) {
      out_idx[row] = (bi >= 0 && bi < vocab) ? bi : 0;  // bi stays unset only when no entry exceeds -inf (all -inf, or NaN): index 0
    } else {
      float2 r;
      r.x = bv;
      r.y = __int_as_float(bi);
      part[row * chunks + c] = r;
    }
  }
}

// One wave per row: merge the per-chunk winners (chunks are in index order).
__global__ __launch_bounds__(256) void argmax_merge(int64_t rows, int64_t vocab, int chunks,
                                                    const float2* __restrict__ part, int32_t* __restrict__ out_idx) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int c = lane; c < chunks; c += 64) {
    const float2 r = part[row * chunks + c];
    const int i = __float_as_int(r.y);
    if (better(r.x, i, bv, bi)) { bv = r.x; bi = i; }
  }
  wave_reduce(bv, bi);
  if (lane == 0) out_idx[row] = (bi >= 0 && bi < vocab) ? bi : 0;
}

// Scans of at least one row per CU take one workgroup per row, so no merge
// kernel runs. Greedy: 1024 threads with 4 loads in flight each (64 KB per
// workgroup: with a workgroup on every CU that is about what HBM needs in
// flight; four waves per SIMD measured 1-2 % faster than 512 threads with 8
// loads each). Sampling, below eight rows per CU: 512 threads with 2 loads
// each, double-buffered (the Philox arithmetic dominates; fewer registers per
// wave let more rows share a CU and some waves' arithmetic overlap others'
// loads: 4 % faster than 1024 x 4 at 256 rows, 8 % at 1024). From eight rows
// per CU on, 256-thread workgroups. Fewer rows than CUs are cut into chunks of
// 256-thread workgroups and merged.
constexpr int kWideThreads = 1024;
constexpr int kWideUnroll = 4;
constexpr int kSampleWideThreads = 512;
constexpr int kSampleWideUnroll = 2;

int plan_chunks(int64_t rows, int64_t vocab, int cus, int64_t* chunk_len, int* chunks) {
  if (rows >= cus) {
    *chunk_len = vocab;
    *chunks = 1;
    return DT_OK;
  }
  // enough workgroups to cover the CUs several times over, chunks >= 8K entries
  const int64_t target_wg = 8LL * cus;
  int64_t c = ceil_div(target_wg, std::max<int64_t>(rows, 1));
  c = std::min<int64_t>(c, std::max<int64_t>(1, vocab / 8192));
  int64_t len = ceil_div(ceil_div(vocab, c), kChunkQuantum) * kChunkQuantum;
  c = ceil_div(vocab, len);
  if (c > 65535) return DT_ERR_UNSUPPORTED;
  *chunk_len = len;
  *chunks = (int)c;
  return DT_OK;
}

}  // namespace
}  // namespace dt

namespace dt {
namespace {

int scan_workspace_size(int64_t rows, int64_t vocab, size_t* bytes) {
  if (!bytes) return DT_ERR_NULL;
  if (rows < 0 || vocab < 1 || vocab > INT_MAX) return DT_ERR_SHAPE;
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != DT_OK) return st;
  int64_t len;
  int chunks;
  st = plan_chunks(rows, vocab, cus, &len, &chunks);
  if (st != DT_OK) return st;
  *bytes = chunks > 1 ? round_up((size_t)rows * chunks * sizeof(float2), 256) : 0;
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_argmax_rows_workspace_size(int64_t rows, int64_t vocab, size_t* bytes) {
  return dt::scan_workspace_size(rows, vocab, bytes);
}

namespace dt {
namespace {

int launch_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t* out_idx,
                void* workspace, size_t workspace_bytes, void* stream, bool sample, const Gumbel& g) {
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != DT_OK) return st;
  int64_t len;
  int chunks;
  st = plan_chunks(rows, vocab, cus, &len, &chunks);
  if (st != DT_OK) return st;
  float2* part = nullptr;
  if (chunks > 1) {
    const size_t need = round_up((size_t)rows * chunks * sizeof(float2), 256);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return DT_ERR_WORKSPACE;
    part = static_cast<float2*>(workspace);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = aligned(logits, 16) && (row_stride % 4 == 0);
  dim3 grid((unsigned)chunks, (unsigned)rows);
  const bool wide = !sample && rows >= cus;
  const bool sample_wide = sample && rows >= cus && rows < 8LL * cus;
#define DT_LAUNCH_SCAN(V, S)                                                                                         \
  do {                                                                                                              \
    if (sample_wide)                                                                                                \
      hipLaunchKernelGGL((argmax_chunks<V, S, kSampleWideThreads, kSampleWideUnroll>), grid, dim3(kSampleWideThreads), \
                         0, s, logits, vocab, row_stride, len, chunks, out_idx, part, g);                           \
    else if (wide)                                                                                                  \
      hipLaunchKernelGGL((argmax_chunks<V, S, kWideThreads, kWideUnroll>), grid, dim3(kWideThreads), 0, s, logits,  \
                         vocab, row_stride, len, chunks, out_idx, part, g);                                         \
    else                                                                                                            \
      hipLaunchKernelGGL((argmax_chunks<V, S, kThreads, kUnroll>), grid, dim3(kThreads), 0, s, logits, vocab,       \
                         row_stride, len, chunks, out_idx, part, g);                                                \
  } while (0)
  if (sample) {
    if (vec) DT_LAUNCH_SCAN(true, true);
    else DT_LAUNCH_SCAN(false, true);
  } else {
    if (vec) DT_LAUNCH_SCAN(true, false);
    else DT_LAUNCH_SCAN(false, false);
  }
#undef DT_LAUNCH_SCAN
  if (chunks > 1)
    hipLaunchKernelGGL(argmax_merge, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, rows, vocab, chunks, part, out_idx);
  return launch_status();
}

int check_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, const int32_t* out_idx) {
  if (rows < 0 || vocab < 1 || vocab > INT_MAX || row_stride < vocab) return DT_ERR_SHAPE;
  if (rows > 65535) return DT_ERR_UNSUPPORTED;
  if (rows == 0) return DT_OK;
  if (!logits || !out_idx) return DT_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(out_idx, 4)) return DT_ERR_SHAPE;
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_argmax_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t* out_idx,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const int st = dt::check_rows(logits, rows, vocab, row_stride, out_idx);
  if (st != DT_OK || rows == 0) return st;
  return dt::launch_rows(logits, rows, vocab, row_stride, out_idx, workspace, workspace_bytes, stream, false,
                         dt::Gumbel{});
}

extern "C" int dt_sample_rows_workspace_size(int64_t rows, int64_t vocab, size_t* bytes) {
  return dt::scan_workspace_size(rows, vocab, bytes);
}

extern "C" int dt_sample_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, float temperature,
                              uint64_t seed, uint64_t offset, int32_t* out_idx, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int st = dt::check_rows(logits, rows, vocab, row_stride, out_idx);
  if (st != DT_OK) return st;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return DT_ERR_VALUE;
  const double c = 1.4426950408889634 / (double)temperature;  // log2(e) / T
  if (!(c <= (double)FLT_MAX)) return DT_ERR_VALUE;
  if (rows == 0) return DT_OK;
  dt::Gumbel g;
  g.c = (float)c;
  g.k0 = (uint32_t)seed;
  g.k1 = (uint32_t)(seed >> 32);
  g.o0 = (uint32_t)offset;
  g.o1 = (uint32_t)(offset >> 32);
  return dt::launch_rows(logits, rows, vocab, row_stride, out_idx, workspace, workspace_bytes, stream, true, g);
}
