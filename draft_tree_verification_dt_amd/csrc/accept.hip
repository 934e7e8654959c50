// Greedy acceptance walk (DARTree paper, Preliminaries > Speculative Sampling,
// T = 0, and Tree Verification and DDTree): from the root, keep moving to the
// child whose draft token equals the target's greedy prediction at the current
// node; stop at the first node with no such child. The accepted path, its
// length L and the bonus token (the prediction at the last accepted node) are
// written out.
//
// One workgroup per tree. The walk itself is a chain of dependent steps, so
// the work that can be parallel is done first: every node checks its own edge
// (token[c] == argmax[parent[c]]) and the lowest matching child of each node
// is recorded in LDS with an atomic min. The walk is then a handful of LDS
// reads by one lane instead of a scan over the tree per step.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "internal.h"

namespace dt {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSeqs = 64;       // sequences per launch (host loops over larger batches)
constexpr int kMaxWalkNodes = 16384;

struct AcceptParams {
  const int32_t* parent;
  const int32_t* token;
  const int32_t* argmax;
  int32_t* path;
  int32_t* accept_len;
  int32_t* bonus;
  int32_t seq0;  // index of the first sequence of this launch
  int32_t offs[kMaxSeqs + 1];
};

__global__ __launch_bounds__(kThreads) void accept_walk(const AcceptParams p) {
  extern __shared__ int32_t best_child[];  // [n]: lowest matching child of each node
  __shared__ int32_t s_len;
  const int s = blockIdx.x;
  const int off = p.offs[s];
  const int n = p.offs[s + 1] - off;
  for (int i = threadIdx.x; i < n; i += kThreads) best_child[i] = INT_MAX;
  __syncthreads();
  for (int c = 1 + threadIdx.x; c < n; c += kThreads) {
    const int u = p.parent[off + c];
    if (u >= 0 && u < c && p.token[off + c] == p.argmax[off + u]) atomicMin(&best_child[u], c);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int cur = 0, L = 0;
    p.path[off] = 0;
    for (;;) {
      const int nxt = best_child[cur];
      if (nxt == INT_MAX) break;  // children always have larger indices, so the walk ends
      cur = nxt;
      ++L;
      p.path[off + L] = cur;
    }
    p.accept_len[p.seq0 + s] = L;
    p.bonus[p.seq0 + s] = p.argmax[off + cur];
    s_len = L;
  }
  __syncthreads();
  for (int t = s_len + 1 + threadIdx.x; t < n; t += kThreads) p.path[off + t] = -1;
}

}  // namespace
}  // namespace dt

extern "C" int dt_accept_path(int32_t num_seqs, const int32_t* node_offsets, const int32_t* parent,
                              const int32_t* token, const int32_t* argmax_idx, int32_t* path, int32_t* accept_len,
                              int32_t* bonus, void* stream) {
  using namespace dt;
  if (num_seqs < 1) return DT_ERR_SHAPE;
  if (!node_offsets || !parent || !token || !argmax_idx || !path || !accept_len || !bonus) return DT_ERR_NULL;
  if (node_offsets[0] != 0) return DT_ERR_SHAPE;
  int max_n = 1;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = node_offsets[s + 1] - node_offsets[s];
    if (n < 1) return DT_ERR_SHAPE;
    if (n > kMaxWalkNodes) return DT_ERR_UNSUPPORTED;
    max_n = std::max(max_n, n);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int s0 = 0; s0 < num_seqs; s0 += kMaxSeqs) {
    AcceptParams a;
    const int cnt = std::min(kMaxSeqs, num_seqs - s0);
    a.parent = parent;
    a.token = token;
    a.argmax = argmax_idx;
    a.path = path;
    a.accept_len = accept_len;
    a.bonus = bonus;
    a.seq0 = s0;
    int local_max = 1;
    for (int i = 0; i <= cnt; ++i) a.offs[i] = node_offsets[s0 + i];
    for (int i = 0; i < cnt; ++i) local_max = std::max(local_max, a.offs[i + 1] - a.offs[i]);
    hipLaunchKernelGGL(accept_walk, dim3(cnt), dim3(kThreads), sizeof(int32_t) * local_max, st, a);
    int rc = launch_status();
    if (rc != DT_OK) return rc;
  }
  return DT_OK;
}
