// Drives the library's host-side C ABI (include/dtree.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer: the best-first tree builder
// on random candidate tables (sorted rows with ties, distinct tokens, every
// size from a single candidate to budgets larger than the table holds), its
// contract errors, the tree validator and the status strings. Each built tree
// is checked for the properties its header states: parent[0] = -1 and
// parent[i] < i, depth(i) = depth(parent) + 1, the node's token is a candidate
// of its draft position, scores are the running sums of the candidates'
// log-probabilities, emitted in non-increasing order, and n_out is the budget
// unless the table runs out of prefixes. Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <vector>

#include "dtree.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}
int uniform(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

int g_failures = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "check failed: %s: ", #cond); \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      ++g_failures;                                       \
    }                                                     \
  } while (0)

struct Table {
  int depths, k;
  std::vector<float> lp;
  std::vector<int32_t> tok;
};

Table random_table(int depths, int k, bool ties) {
  Table t{depths, k, std::vector<float>((size_t)depths * k), std::vector<int32_t>((size_t)depths * k)};
  for (int d = 0; d < depths; ++d) {
    std::vector<float> row(k);
    for (int j = 0; j < k; ++j) {
      float v = -(float)(next_u64() % 20000) / 1000.f;
      if (ties) v = std::round(v * 2.f) / 2.f;  // many equal log-probs
      row[j] = v;
    }
    std::sort(row.begin(), row.end(), [](float a, float b) { return a > b; });
    const int32_t base = uniform(0, 1000), stride = uniform(1, 7);
    for (int j = 0; j < k; ++j) {
      t.lp[(size_t)d * k + j] = row[j];
      t.tok[(size_t)d * k + j] = base + j * stride;
    }
  }
  return t;
}

// number of prefixes of length 1..depths over k candidates, capped at cap
int64_t prefixes(int depths, int k, int64_t cap) {
  int64_t total = 0, level = 1;
  for (int d = 0; d < depths && total < cap; ++d) {
    level = std::min<int64_t>(level * k, cap);
    total += level;
  }
  return std::min(total, cap);
}

void check_tree(const Table& t, int n, int root, const std::vector<int32_t>& parent, const std::vector<int32_t>& token,
                const std::vector<int32_t>& depth, const std::vector<double>& score, bool with_score, int n_out) {
  const int64_t avail = prefixes(t.depths, t.k, n);
  CHECK(n_out == std::min<int64_t>(n, 1 + avail), "n_out %d for budget %d (%lld prefixes)", n_out, n, (long long)avail);
  CHECK(dt_validate_tree(parent.data(), n_out) == DT_OK, "built tree does not validate");
  CHECK(parent[0] == -1 && token[0] == root && depth[0] == 0, "root entry");
  for (int i = 1; i < n_out; ++i) {
    const int p = parent[i];
    CHECK(p >= 0 && p < i, "parent[%d] = %d", i, p);
    if (p < 0 || p >= i) continue;
    CHECK(depth[i] == depth[p] + 1 && depth[i] <= t.depths, "depth[%d] = %d", i, depth[i]);
    const int d = depth[i] - 1;
    int rank = -1;
    for (int j = 0; j < t.k; ++j)
      if (t.tok[(size_t)d * t.k + j] == token[i]) rank = j;
    CHECK(rank >= 0, "token[%d] = %d is not a candidate of position %d", i, token[i], d + 1);
    if (with_score && rank >= 0) {
      const double expect = score[p] + (double)t.lp[(size_t)d * t.k + rank];
      CHECK(score[i] == expect, "score[%d] = %.17g, expected %.17g", i, score[i], expect);
      CHECK(i == 1 || score[i] <= score[i - 1], "scores rise at node %d", i);
    }
  }
  for (int i = 1; i < n_out; ++i)
    for (int j = 1; j < i; ++j)  // siblings carry distinct tokens
      if (parent[i] == parent[j]) CHECK(token[i] != token[j], "siblings %d and %d share a token", i, j);
}

void random_builds() {
  for (int trial = 0; trial < 2000; ++trial) {
    const int depths = uniform(1, 16), k = uniform(1, 40), n = uniform(1, 300), root = uniform(0, 5000);
    const bool ties = trial % 3 == 0, with_score = trial % 2 == 0;
    const Table t = random_table(depths, k, ties);
    std::vector<int32_t> parent(n, 12345), token(n, 12345), depth(n, 12345);
    std::vector<double> score(n, 0.0);
    int32_t n_out = -1;
    const int st = dt_build_tree(depths, k, t.lp.data(), t.tok.data(), root, n, parent.data(), token.data(),
                                 depth.data(), with_score ? score.data() : nullptr, &n_out);
    CHECK(st == DT_OK, "trial %d: status %d", trial, st);
    if (st == DT_OK) check_tree(t, n, root, parent, token, depth, score, with_score, n_out);
  }
}

void contract_errors() {
  Table t = random_table(4, 5, false);
  std::vector<int32_t> parent(8), token(8), depth(8);
  int32_t n_out = 0;
  auto build = [&](const Table& tb, int n) {
    return dt_build_tree(tb.depths, tb.k, tb.lp.data(), tb.tok.data(), 3, n, parent.data(), token.data(),
                         depth.data(), nullptr, &n_out);
  };
  CHECK(build(t, 8) == DT_OK, "valid table");
  CHECK(dt_build_tree(4, 5, nullptr, t.tok.data(), 3, 8, parent.data(), token.data(), depth.data(), nullptr, &n_out) ==
            DT_ERR_NULL, "null log-probs");
  CHECK(dt_build_tree(4, 5, t.lp.data(), t.tok.data(), 3, 8, parent.data(), token.data(), depth.data(), nullptr,
                      nullptr) == DT_ERR_NULL, "null n_out");
  CHECK(build(t, 0) == DT_ERR_SHAPE, "zero budget");
  CHECK(dt_build_tree(0, 5, t.lp.data(), t.tok.data(), 3, 8, parent.data(), token.data(), depth.data(), nullptr,
                      &n_out) == DT_ERR_SHAPE, "zero depths");
  CHECK(dt_build_tree(4, 5, t.lp.data(), t.tok.data(), -1, 8, parent.data(), token.data(), depth.data(), nullptr,
                      &n_out) == DT_ERR_SHAPE, "negative root token");
  Table u = t;
  std::swap(u.lp[0], u.lp[4]);  // row 0 no longer non-increasing (its values are distinct)
  CHECK(u.lp[0] == u.lp[4] || build(u, 8) == DT_ERR_VALUE, "unsorted row");
  u = t;
  u.lp[7] = 0.5f;
  CHECK(build(u, 8) == DT_ERR_VALUE, "positive log-prob");
  u = t;
  u.lp[9] = std::nanf("");
  CHECK(build(u, 8) == DT_ERR_VALUE, "NaN log-prob");
  u = t;
  u.tok[6] = u.tok[5];
  CHECK(build(u, 8) == DT_ERR_VALUE, "repeated token");
  u = t;
  u.tok[2] = -4;
  CHECK(build(u, 8) == DT_ERR_VALUE, "negative token");
}

void validator() {
  const int32_t ok[] = {-1, 0, 0, 1, 3, 2};
  CHECK(dt_validate_tree(ok, 6) == DT_OK, "valid tree");
  const int32_t self[] = {-1, 1};
  CHECK(dt_validate_tree(self, 2) == DT_ERR_TREE, "self parent");
  const int32_t fwd[] = {-1, 2, 0};
  CHECK(dt_validate_tree(fwd, 3) == DT_ERR_TREE, "forward parent");
  const int32_t two_roots[] = {-1, -1};
  CHECK(dt_validate_tree(two_roots, 2) == DT_ERR_TREE, "second root");
  const int32_t bad_root[] = {0};
  CHECK(dt_validate_tree(bad_root, 1) == DT_ERR_TREE, "root with a parent");
  CHECK(dt_validate_tree(nullptr, 3) == DT_ERR_NULL, "null parent array");
  CHECK(dt_validate_tree(ok, 0) == DT_ERR_SHAPE, "empty tree");
}

void status_strings() {
  for (int s = -12; s <= 2; ++s) {
    const char* m = dt_status_string(s);
    CHECK(m != nullptr && std::strlen(m) > 0, "status %d has no message", s);
  }
  CHECK(dt_abi_version() > 0, "ABI version");
}

}  // namespace

int main() {
  status_strings();
  validator();
  contract_errors();
  random_builds();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
