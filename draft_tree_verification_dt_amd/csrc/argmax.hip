// Row-wise arg-max of fp32 target logits: the target's greedy prediction at
// every tree node (DARTree paper, Preliminaries > Speculative Sampling, T = 0).
//
// Pure streaming work, bound by HBM bandwidth. Each row is cut into chunks so
// that the launch has enough workgroups whatever the row count (a 16-node
// chain has 16 rows of 152K entries; a 2048-node batch has 2048). A workgroup
// scans its chunk with 16-byte loads, four in flight per thread, keeping the
// first (lowest-index) maximum per thread; waves reduce with cross-lane
// shuffles and the four waves through LDS. With one chunk per row the result
// is written directly; otherwise per-chunk (value, index) pairs go to the
// workspace and a second kernel merges them. Ties go to the lowest index.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "internal.h"

namespace dt {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kChunkQuantum = 4 * kThreads * kUnroll;  // elements; keeps chunks 16-byte aligned

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

__device__ inline void block_reduce(float& bv, int& bi) {
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  wave_reduce(bv, bi);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k)
      if (better(sv[k], si[k], bv, bi)) {
        bv = sv[k];
        bi = si[k];
      }
  }
}

// grid: (chunks, rows). VEC: row starts are 16-byte aligned.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void argmax_chunks(const float* __restrict__ x, int64_t vocab, int64_t stride,
                                                          int64_t chunk_len, int chunks, int32_t* __restrict__ out_idx,
                                                          float2* __restrict__ part) {
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const float* xr = x + row * stride;
  const int64_t beg = (int64_t)c * chunk_len;
  const int64_t end = std::min<int64_t>(vocab, beg + chunk_len);
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (VEC) {
    const int64_t beg4 = beg >> 2, end4 = end >> 2;  // full float4s; beg is a multiple of 4
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    int64_t j = beg4 + threadIdx.x;
    for (; j + (kUnroll - 1) * kThreads < end4; j += kUnroll * kThreads) {
      f32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x4 + j + u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int base = (int)((j + u * kThreads) << 2);
        if (better(v[u].x, base, bv, bi)) { bv = v[u].x; bi = base; }
        if (better(v[u].y, base + 1, bv, bi)) { bv = v[u].y; bi = base + 1; }
        if (better(v[u].z, base + 2, bv, bi)) { bv = v[u].z; bi = base + 2; }
        if (better(v[u].w, base + 3, bv, bi)) { bv = v[u].w; bi = base + 3; }
      }
    }
    for (; j < end4; j += kThreads) {
      const f32x4 v = __builtin_nontemporal_load(x4 + j);
      const int base = (int)(j << 2);
      if (better(v.x, base, bv, bi)) { bv = v.x; bi = base; }
      if (better(v.y, base + 1, bv, bi)) { bv = v.y; bi = base + 1; }
      if (better(v.z, base + 2, bv, bi)) { bv = v.z; bi = base + 2; }
      if (better(v.w, base + 3, bv, bi)) { bv = v.w; bi = base + 3; }
    }
    for (int64_t t = (end4 << 2) + threadIdx.x; t < end; t += kThreads)
      if (better(xr[t], (int)t, bv, bi)) { bv = xr[t]; bi = (int)t; }
  } else {
    for (int64_t t = beg + threadIdx.x; t < end; t += kThreads)
      if (better(xr[t], (int)t, bv, bi)) { bv = xr[t]; bi = (int)t; }
  }
  block_reduce(bv, bi);
  if (threadIdx.x == 0) {
    if (chunks == 1) {
      out_idx[row] = (bi >= 0 && bi < vocab) ? bi : 0;  // only a NaN-filled row leaves bi unset
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

int plan_chunks(int64_t rows, int64_t vocab, int cus, int64_t* chunk_len, int* chunks) {
  // enough workgroups to cover the CUs several times over, chunks >= 8K entries
  const int64_t target_wg = 8LL * cus;
  int64_t c = rows >= target_wg ? 1 : ceil_div(target_wg, std::max<int64_t>(rows, 1));
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

extern "C" int dt_argmax_rows_workspace_size(int64_t rows, int64_t vocab, size_t* bytes) {
  if (!bytes) return DT_ERR_NULL;
  if (rows < 0 || vocab < 1 || vocab > INT_MAX) return DT_ERR_SHAPE;
  int cus = 0;
  int st = dt::current_device_cus(&cus);
  if (st != DT_OK) return st;
  int64_t len;
  int chunks;
  st = dt::plan_chunks(rows, vocab, cus, &len, &chunks);
  if (st != DT_OK) return st;
  *bytes = chunks > 1 ? dt::round_up((size_t)rows * chunks * sizeof(float2), 256) : 0;
  return DT_OK;
}

extern "C" int dt_argmax_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t* out_idx,
                              void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dt;
  if (rows < 0 || vocab < 1 || vocab > INT_MAX || row_stride < vocab) return DT_ERR_SHAPE;
  if (rows > 65535) return DT_ERR_UNSUPPORTED;
  if (rows == 0) return DT_OK;
  if (!logits || !out_idx) return DT_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(out_idx, 4)) return DT_ERR_SHAPE;
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
  if (vec)
    hipLaunchKernelGGL(argmax_chunks<true>, grid, dim3(kThreads), 0, s, logits, vocab, row_stride, len, chunks, out_idx, part);
  else
    hipLaunchKernelGGL(argmax_chunks<false>, grid, dim3(kThreads), 0, s, logits, vocab, row_stride, len, chunks, out_idx, part);
  if (chunks > 1)
    hipLaunchKernelGGL(argmax_merge, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, rows, vocab, chunks, part, out_idx);
  return launch_status();
}
