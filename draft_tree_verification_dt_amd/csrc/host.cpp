// Host-side entry points: status strings, tree validation, and the best-first
// (DDTree) draft-tree builder.
//
// The builder follows the DARTree paper, Figure 3 caption: a max-heap over
// frontier prefixes, where each pop turns the highest-mass prefix into a tree
// node and pushes that prefix's next sibling and its first child. The mass of
// a prefix is the product of its per-position draft probabilities (Tree
// Verification and DDTree, eq. 4 and the decomposition after it); it is kept
// as a log-mass, the float64 sum of the candidates' log-probabilities added
// from the root down.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "internal.h"

extern "C" const char* dt_status_string(int status) {
  switch (status) {
    case DT_OK: return "ok";
    case DT_ERR_NULL: return "a required pointer is NULL";
    case DT_ERR_SHAPE: return "a count, size, stride or offset is out of range or misaligned";
    case DT_ERR_TREE: return "parent array is not a topologically numbered tree (parent[0] = -1, 0 <= parent[i] < i)";
    case DT_ERR_VALUE: return "candidate table violates its contract (finite, <= 0, rows non-increasing, distinct tokens)";
    case DT_ERR_UNSUPPORTED: return "request not supported by this library";
    case DT_ERR_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case DT_ERR_HIP: return "a HIP runtime call failed";
    case DT_ERR_NOMEM: return "temporary host memory could not be obtained";
    default: return "unknown status";
  }
}

extern "C" int dt_abi_version(void) { return (2 << 16) | 0; }

extern "C" int dt_validate_tree(const int32_t* parent, int32_t n) {
  if (n < 1) return DT_ERR_SHAPE;
  if (!parent) return DT_ERR_NULL;
  if (parent[0] != -1) return DT_ERR_TREE;
  for (int32_t i = 1; i < n; ++i)
    if (parent[i] < 0 || parent[i] >= i) return DT_ERR_TREE;
  return DT_OK;
}

namespace dt {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];
hipError_t g_cu_err[kMaxDevices];

// A frontier prefix: the `rank`-th candidate at position `depth` appended to
// tree node `parent_node`.
struct Frontier {
  double score;
  int32_t depth;
  int32_t parent_node;
  int32_t rank;
};

class Builder {
 public:
  Builder(int32_t depths, int32_t k, const float* lp, int32_t n_nodes)
      : depths_(depths), k_(k), lp_(lp) {
    ranks_.assign(static_cast<size_t>(n_nodes) * depths, 0);
    node_depth_.assign(n_nodes, 0);
    node_score_.assign(n_nodes, 0.0);
    heap_.reserve(static_cast<size_t>(n_nodes) + 2);
  }

  // Lexicographic comparison of the rank tuples of two same-depth frontier
  // entries: the parents' tuples first, then the entries' own ranks.
  bool ranks_less(const Frontier& a, const Frontier& b) const {
    if (a.parent_node != b.parent_node) {
      const uint16_t* ra = &ranks_[static_cast<size_t>(a.parent_node) * depths_];
      const uint16_t* rb = &ranks_[static_cast<size_t>(b.parent_node) * depths_];
      for (int32_t i = 0; i < a.depth - 1; ++i)
        if (ra[i] != rb[i]) return ra[i] < rb[i];
    }
    return a.rank < b.rank;
  }

  // True when a must be popped before b: higher score, then shallower, then
  // lexicographically smaller rank tuple. A child never precedes its parent
  // and a next sibling never precedes its elder sibling under this order.
  bool before(const Frontier& a, const Frontier& b) const {
    if (a.score != b.score) return a.score > b.score;
    if (a.depth != b.depth) return a.depth < b.depth;
    return ranks_less(a, b);
  }

  void push(const Frontier& f) {
    heap_.push_back(f);
    size_t i = heap_.size() - 1;
    while (i > 0) {
      size_t p = (i - 1) / 2;
      if (!before(heap_[i], heap_[p])) break;
      std::swap(heap_[i], heap_[p]);
      i = p;
    }
  }

  Frontier pop() {
    Frontier top = heap_[0];
    heap_[0] = heap_.back();
    heap_.pop_back();
    size_t i = 0, n = heap_.size();
    for (;;) {
      size_t l = 2 * i + 1, r = l + 1, m = i;
      if (l < n && before(heap_[l], heap_[m])) m = l;
      if (r < n && before(heap_[r], heap_[m])) m = r;
      if (m == i) break;
      std::swap(heap_[i], heap_[m]);
      i = m;
    }
    return top;
  }

  bool empty() const { return heap_.empty(); }

  float lp(int32_t depth, int32_t rank) const { return lp_[static_cast<size_t>(depth - 1) * k_ + rank]; }

  // Record node `node` made from frontier entry f.
  void place(int32_t node, const Frontier& f) {
    node_depth_[node] = f.depth;
    node_score_[node] = f.score;
    uint16_t* dst = &ranks_[static_cast<size_t>(node) * depths_];
    if (f.depth > 1) std::memcpy(dst, &ranks_[static_cast<size_t>(f.parent_node) * depths_], sizeof(uint16_t) * (f.depth - 1));
    dst[f.depth - 1] = static_cast<uint16_t>(f.rank);
  }

  double node_score(int32_t node) const { return node_score_[node]; }

 private:
  int32_t depths_, k_;
  const float* lp_;
  std::vector<uint16_t> ranks_;  // [node][depth] rank tuple of each node
  std::vector<int32_t> node_depth_;
  std::vector<double> node_score_;
  std::vector<Frontier> heap_;
};

int check_table(int32_t depths, int32_t k, const float* lp, const int32_t* tok) {
  std::vector<int32_t> row(static_cast<size_t>(k));
  for (int32_t d = 0; d < depths; ++d) {
    const float* l = lp + static_cast<size_t>(d) * k;
    const int32_t* t = tok + static_cast<size_t>(d) * k;
    for (int32_t r = 0; r < k; ++r) {
      if (!std::isfinite(l[r]) || l[r] > 0.0f) return DT_ERR_VALUE;
      if (r > 0 && l[r] > l[r - 1]) return DT_ERR_VALUE;
      if (t[r] < 0) return DT_ERR_VALUE;
    }
    std::memcpy(row.data(), t, sizeof(int32_t) * k);
    std::sort(row.begin(), row.end());
    for (int32_t r = 1; r < k; ++r)
      if (row[r] == row[r - 1]) return DT_ERR_VALUE;
  }
  return DT_OK;
}

}  // namespace

int current_device_cus(int* cus) {
  int dev = 0;
  DT_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DT_ERR_UNSUPPORTED;
  std::call_once(g_cu_once[dev], [dev]() {
    g_cu_err[dev] = hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  if (g_cu_err[dev] != hipSuccess) return DT_ERR_HIP;
  *cus = g_cus[dev];
  return DT_OK;
}

}  // namespace dt

extern "C" int dt_build_tree(int32_t depths, int32_t k, const float* cand_logprob, const int32_t* cand_token,
                             int32_t root_token, int32_t n_nodes, int32_t* parent, int32_t* token, int32_t* depth,
                             double* score, int32_t* n_out) {
  if (!cand_logprob || !cand_token || !parent || !token || !depth || !n_out) return DT_ERR_NULL;
  if (depths < 1 || depths > 64 || k < 1 || k > 65535 || n_nodes < 1 || root_token < 0) return DT_ERR_SHAPE;
  try {
    int st = dt::check_table(depths, k, cand_logprob, cand_token);
    if (st != DT_OK) return st;

    dt::Builder b(depths, k, cand_logprob, n_nodes);
    parent[0] = -1;
    token[0] = root_token;
    depth[0] = 0;
    if (score) score[0] = 0.0;
    int32_t n = 1;
    if (n_nodes > 1) b.push({0.0 + static_cast<double>(b.lp(1, 0)), 1, 0, 0});
    while (n < n_nodes && !b.empty()) {
      dt::Frontier f = b.pop();
      const int32_t node = n++;
      b.place(node, f);
      parent[node] = f.parent_node;
      token[node] = cand_token[static_cast<size_t>(f.depth - 1) * k + f.rank];
      depth[node] = f.depth;
      if (score) score[node] = f.score;
      if (f.rank + 1 < k)  // next sibling: same parent, next-ranked candidate
        b.push({b.node_score(f.parent_node) + static_cast<double>(b.lp(f.depth, f.rank + 1)), f.depth,
                f.parent_node, f.rank + 1});
      if (f.depth < depths)  // first child: best candidate one position deeper
        b.push({f.score + static_cast<double>(b.lp(f.depth + 1, 0)), f.depth + 1, node, 0});
    }
    *n_out = n;
    return DT_OK;
  } catch (const std::bad_alloc&) {
    return DT_ERR_NOMEM;
  } catch (...) {
    return DT_ERR_NOMEM;
  }
}
