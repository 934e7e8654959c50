// Accepted-path KV commit: the keys and values the verification forward
// computed for the accepted tree nodes become the next cache rows.
//
// DARTree paper, Preliminaries > Speculative Sampling (every round commits the
// accepted draft prefix and one bonus token) and Figure 3 (tree verification
// hands the accepted tokens and their features to the next round). Node
// path[t] of sequence s sits at position P_s + t (its depth), where the forward
// already placed it, so its K/V rows are copied unchanged into cache row
// P_s + t, for t = 0 .. accept_len[s] and every layer.
//
// A pure gather/scatter of (L + 1) x Hkv x d bf16 per layer and sequence: a few
// MB for a whole model, far below anything bandwidth-relevant, so the point is
// one launch for all layers and sequences (grid: path position x sequence x
// layer; the blocks past a sequence's accepted length exit at once) with
// 16-byte accesses. Accepted lengths stay on the device: no host round trip.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "internal.h"

namespace dt {
namespace {

constexpr int kCommitThreads = 256;
constexpr int kCommitLayers = 40;  // layers per launch (pointer tables travel as kernel arguments)
constexpr int kCommitSeqs = 32;    // sequences per launch

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CommitSeq {
  int64_t dst_row;   // prefix_row_start + P: cache row of path position 0
  int32_t node_off;  // first packed node row of the sequence
  int32_t n;         // nodes of the sequence
};

struct CommitParams {
  const u32x4* kt[kCommitLayers];
  const u32x4* vt[kCommitLayers];
  u32x4* kc[kCommitLayers];
  u32x4* vc[kCommitLayers];
  const int32_t* path;
  const int32_t* accept_len;
  int64_t t_rs;      // tree row stride, 16-byte units
  int64_t c_rs;      // cache row stride, 16-byte units
  int64_t c_hs;      // cache head stride, 16-byte units
  int32_t vph;       // 16-byte vectors per head (d / 8)
  int32_t hkv;
  int32_t max_path;  // path positions covered by the grid
  int32_t seq0;      // batch index of this launch's first sequence (indexes accept_len)
  CommitSeq seq[kCommitSeqs];
};

// grid: (max_path, sequences, layers) of this launch.
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(const CommitParams p) {
  const int t = blockIdx.x;
  const CommitSeq sq = p.seq[blockIdx.y];
  const int l = blockIdx.z;
  const int len = p.accept_len[p.seq0 + blockIdx.y];  // accepted draft tokens; path positions 0 .. len
  if (t > len || t >= sq.n || t >= p.max_path) return;
  const int node = p.path[sq.node_off + t];
  if (node < 0 || node >= sq.n) return;  // violated device contract: nothing written
  const int64_t src = (int64_t)(sq.node_off + node) * p.t_rs;
  const int64_t dst = (sq.dst_row + t) * p.c_rs;
  const int per_row = p.hkv * p.vph;
  for (int v = threadIdx.x; v < per_row; v += kCommitThreads) {
    const int h = v / p.vph;
    const int e = v - h * p.vph;
    const u32x4 k = __builtin_nontemporal_load(p.kt[l] + src + v);
    const u32x4 x = __builtin_nontemporal_load(p.vt[l] + src + v);
    p.kc[l][dst + h * p.c_hs + e] = k;
    p.vc[l][dst + h * p.c_hs + e] = x;
  }
}

int check_commit(const dt_commit_desc* d, const void* const* k_tree, const void* const* v_tree,
                 void* const* k_cache, void* const* v_cache, const int32_t* path, const int32_t* accept_len,
                 int* grid_paths) {
  if (!d) return DT_ERR_NULL;
  if (d->num_seqs < 1 || d->num_layers < 1 || d->num_kv_heads < 1) return DT_ERR_SHAPE;
  if (d->head_dim < 8 || d->head_dim % 8 || d->max_path < 0) return DT_ERR_SHAPE;
  if (!d->node_offsets || !d->prefix_lens || !d->prefix_row_start || !d->cache_rows) return DT_ERR_NULL;
  if (!k_tree || !v_tree || !k_cache || !v_cache || !path || !accept_len) return DT_ERR_NULL;
  const int64_t D = d->head_dim;
  const int64_t trs = d->tree_row_stride ? d->tree_row_stride : d->num_kv_heads * D;
  if (trs < d->num_kv_heads * D || trs % 8) return DT_ERR_SHAPE;
  if (d->cache_row_stride < 8 || d->cache_row_stride % 8) return DT_ERR_SHAPE;
  if (d->cache_head_stride % 8 || (d->num_kv_heads > 1 && d->cache_head_stride < D)) return DT_ERR_SHAPE;
  if (d->cache_head_stride < 0) return DT_ERR_SHAPE;
  if (d->node_offsets[0] != 0) return DT_ERR_SHAPE;
  int widest = 1;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int64_t n = (int64_t)d->node_offsets[s + 1] - d->node_offsets[s];
    if (n < 1) return DT_ERR_SHAPE;
    if (d->prefix_lens[s] < 0 || d->prefix_row_start[s] < 0) return DT_ERR_SHAPE;
    const int64_t m = d->max_path ? std::min<int64_t>(d->max_path, n) : n;  // path rows that may be written
    if ((int64_t)d->prefix_lens[s] + m > d->cache_rows[s]) return DT_ERR_SHAPE;
    widest = (int)std::max<int64_t>(widest, m);
  }
  if (widest > 65535) return DT_ERR_UNSUPPORTED;
  // device buffers last
  for (int l = 0; l < d->num_layers; ++l) {
    if (!k_tree[l] || !v_tree[l] || !k_cache[l] || !v_cache[l]) return DT_ERR_NULL;
    if (!aligned(k_tree[l], 16) || !aligned(v_tree[l], 16) || !aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
      return DT_ERR_SHAPE;
  }
  if (!aligned(path, 4) || !aligned(accept_len, 4)) return DT_ERR_SHAPE;
  *grid_paths = widest;
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_commit_kv(const dt_commit_desc* desc, const void* const* k_tree, const void* const* v_tree,
                            void* const* k_cache, void* const* v_cache, const int32_t* path,
                            const int32_t* accept_len, void* stream) {
  using namespace dt;
  int widest = 0;
  const int st = check_commit(desc, k_tree, v_tree, k_cache, v_cache, path, accept_len, &widest);
  if (st != DT_OK) return st;
  const dt_commit_desc* d = desc;
  const int64_t trs = d->tree_row_stride ? d->tree_row_stride : (int64_t)d->num_kv_heads * d->head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CommitParams p = {};
  p.path = path;
  p.accept_len = accept_len;
  p.t_rs = trs / 8;
  p.c_rs = d->cache_row_stride / 8;
  p.c_hs = d->cache_head_stride / 8;
  p.vph = d->head_dim / 8;
  p.hkv = d->num_kv_heads;
  p.max_path = widest;
  for (int s0 = 0; s0 < d->num_seqs; s0 += kCommitSeqs) {
    const int ns = std::min(kCommitSeqs, d->num_seqs - s0);
    p.seq0 = s0;
    for (int i = 0; i < ns; ++i) {
      const int sq = s0 + i;
      p.seq[i].dst_row = d->prefix_row_start[sq] + d->prefix_lens[sq];
      p.seq[i].node_off = d->node_offsets[sq];
      p.seq[i].n = d->node_offsets[sq + 1] - d->node_offsets[sq];
    }
    for (int l0 = 0; l0 < d->num_layers; l0 += kCommitLayers) {
      const int nl = std::min(kCommitLayers, d->num_layers - l0);
      for (int i = 0; i < nl; ++i) {
        p.kt[i] = static_cast<const u32x4*>(k_tree[l0 + i]);
        p.vt[i] = static_cast<const u32x4*>(v_tree[l0 + i]);
        p.kc[i] = static_cast<u32x4*>(k_cache[l0 + i]);
        p.vc[i] = static_cast<u32x4*>(v_cache[l0 + i]);
      }
      hipLaunchKernelGGL(commit_kv_kernel, dim3((unsigned)widest, (unsigned)ns, (unsigned)nl), dim3(kCommitThreads),
                         0, s, p);
    }
  }
  return launch_status();
}
