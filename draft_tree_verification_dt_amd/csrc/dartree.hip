// DARTree tree construction on the GPU: per-depth top-K candidates, depth-wise
// fixed-width expansion and deferred top-B pruning (DARTree paper, Methodology:
// Depth-Wise Parallel Supertree Construction, Algorithm 1, and Deferred
// Best-First Pruning, eq. 5-6 with Lemma 1).
//
// All three are selections "the best m of M candidates" under a total order
// (value descending, then a candidate index ascending). Two block-wide routines
// do them. select_ordered first filters: a threshold that provably admits the
// best m (from the waves' per-thread bests, or a caller's hint) leaves a
// few candidates, each ranked against the others, which yields them in order.
// When more than 256 pass, a most-significant-digit radix select (four 8-bit
// passes with an LDS histogram) finds the m-th best value, a
// second radix select over the candidate indices of the elements equal to it
// resolves ties by lowest index, and the selected elements are gathered and
// sorted with a bitonic network in LDS. Exact ties are handled either way, so
// the result is the definition's.
//
//   topk_chunks + topk_merge   C_d = TopK(L_d, K) over the vocabulary, with the
//                              log-softmax value of every kept token (the row's
//                              log-sum-exp is merged from per-chunk (max, sum));
//                              each chunk's K best are written in order, so the
//                              merge takes its filter threshold from the lists'
//                              heads
//   expand_kernel              one depth: scores (s_parent + log q~) + beta of all
//                              W_prev x K children, the best W kept in order
//   prune_kernel               the best B supertree nodes by (score, depth,
//                              slot), flattened into a verification tree

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace dt {
namespace {

constexpr int kSelThreads = 256;    // threads of the expansion workgroup
constexpr int kPruneThreads = 512;  // threads of the pruning workgroup (its ranking: two lanes per candidate)
constexpr int kChunkThreads = 512;  // two waves per SIMD while a chunk is selected
constexpr int kMergeThreads = 512;  // ... and while a row's chunk lists are merged
constexpr int kSelCand = 256;       // candidates select_ordered ranks (more: the radix select)
constexpr int kSelMaxCand = 16384;  // candidates one block selects from (64 per thread)
constexpr int kSelPerThread = kSelMaxCand / kSelThreads;
constexpr int kTopkChunkSmall = 4096;   // vocabulary entries per chunk workgroup (8 per thread)
constexpr int kTopkChunkLarge = 10240;  // ... from 16 rows on (20 per thread: about one workgroup per CU)
constexpr int kMaxSortedK = 1024;   // largest selection that is returned in order

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Order-preserving map of a float to an unsigned key (larger float, larger
// key); -0 is first made +0 so that the two compare equal, as floats do.
__device__ inline uint32_t float_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum and sum over a wave: DPP moves within each 16-lane row (quad
// swaps, then the row's halves, then its two halves of eight), then the four
// rows' values read as scalars.
template <int CTRL>
__device__ inline float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));   // quad_perm 1,0,3,2
  v = fmaxf(v, dpp_move<0x4E>(v));   // quad_perm 2,3,0,1
  v = fmaxf(v, dpp_move<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ inline float wave_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
  auto mv = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  v = mv(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mv(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mv(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mv(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return mv(mv((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
            mv((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

struct SelShared {
  uint32_t hist[256];  // digit histogram; the threads' best keys in select_ordered
  uint32_t red[16];  // one per wave (up to 1024 threads)
  uint32_t bin, remaining, in_bin, total;
  uint32_t count;
  uint32_t thr;  // select_ordered's candidate threshold
};

// Keys are never 0 for a candidate (float_key of a finite value, or the bitwise
// complement of a non-negative index); 0 marks an empty slot.

// Histogram of digit (key >> shift) & 255 over the keys whose bits above the
// digit equal `prefix` (mask selects them); then wave 0 finds, counting from the
// top bin down, the bin holding the `remaining`-th key, and publishes it with
// the count of keys above it, its own count and the total.
template <int E, int NT>
__device__ void digit_pass(const uint32_t (&key)[E], uint32_t prefix, uint32_t mask, int shift, uint32_t remaining,
                           SelShared& sh) {
  static_assert(NT >= 256, "one thread per bin");
  if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] != 0u && (key[e] & mask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & 255u], 1u);
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint32_t c0 = sh.hist[4 * lane], c1 = sh.hist[4 * lane + 1], c2 = sh.hist[4 * lane + 2],
                   c3 = sh.hist[4 * lane + 3];
    const uint32_t s = c0 + c1 + c2 + c3;
    uint32_t incl = s;  // keys in this lane's bins and above
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(incl, off);
      if (lane + off < 64) incl += o;
    }
    if (lane == 0) sh.total = incl;
    uint32_t cum = incl - s;  // keys in higher bins
    const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (cum < remaining && cum + cs[j] >= remaining) {
        sh.bin = 4 * lane + j;
        sh.remaining = remaining - cum;
        sh.in_bin = cs[j];
      }
      cum += cs[j];
    }
  }
  __syncthreads();
}

// The m-th largest key (1 <= m <= number of non-zero keys) and how many keys
// equal to it belong to the best m (used for index tie-breaks only).
template <int E, int NT>
__device__ void radix_select(const uint32_t (&key)[E], uint32_t m, SelShared& sh, uint32_t& thr, uint32_t& need_eq) {
  uint32_t prefix = 0, mask = 0, remaining = m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    digit_pass<E, NT>(key, prefix, mask, shift, remaining, sh);
    prefix |= sh.bin << shift;
    mask |= 0xFFu << shift;
    remaining = sh.remaining;
    __syncthreads();
  }
  thr = prefix;
  need_eq = remaining;
}

// Select the best m candidates (non-zero keys) by (key desc, idx asc) and
// append them with their two payload words, unordered, to the LDS arrays
// through sh.count. Returns the number selected: min(m, candidates), uniform
// across the block. Candidate indices are unique and non-negative.
//
// The first digit pass also counts the candidates. A pass whose chosen bin is
// taken whole (its count equals what is still needed) ends the search: every
// key at or above that bin's lowest value is in. Only when the last digit
// leaves a tie does a second radix select over the tied indices run.
template <int E, bool PAY, int NT>
__device__ uint32_t select_best(const uint32_t (&key)[E], const int32_t (&idx)[E], const int32_t (&p0)[E],
                                const int32_t (&p1)[E], uint32_t m, SelShared& sh, uint32_t* out_key, int32_t* out_idx,
                                int32_t* out_p0, int32_t* out_p1) {
  if (m == 0) return 0;
  uint32_t prefix = 0, mask = 0, remaining = m;
  uint32_t lo = 1;                                      // mode A: take every key >= lo
  bool tie = false;                                     // mode B: key > prefix, or == prefix and idx <= idx_thr
  uint32_t idx_thr = 0xFFFFFFFFu, take = m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    digit_pass<E, NT>(key, prefix, mask, shift, remaining, sh);
    const uint32_t total = sh.total, bin = sh.bin, rem = sh.remaining, in_bin = sh.in_bin;
    __syncthreads();
    if (shift == 24 && total <= m) {  // everything is taken
      take = total;
      break;
    }
    prefix |= bin << shift;
    mask |= 0xFFu << shift;
    if (in_bin == rem) {  // the whole bin is in
      lo = prefix;
      break;
    }
    remaining = rem;
    if (shift == 0) {  // a tie at one key value: the lowest indices among it
      tie = true;
      uint32_t ikey[E];
#pragma unroll
      for (int e = 0; e < E; ++e) ikey[e] = key[e] == prefix ? ~(uint32_t)idx[e] : 0u;  // largest ~idx first
      uint32_t t2, unused;
      radix_select<E, NT>(ikey, remaining, sh, t2, unused);
      idx_thr = ~t2;
    }
  }
  if (take == 0) return 0;
  if (threadIdx.x == 0) sh.count = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = key[e] != 0u &&
                    (tie ? (key[e] > prefix || (key[e] == prefix && (uint32_t)idx[e] <= idx_thr)) : key[e] >= lo);
    if (in) {
      const uint32_t pos = atomicAdd(&sh.count, 1u);
      out_key[pos] = key[e];
      out_idx[pos] = idx[e];
      if (PAY) {
        out_p0[pos] = p0[e];
        out_p1[pos] = p1[e];
      }
    }
  }
  __syncthreads();
  return take;
}

// Is (ka, ia) ahead of (kb, ib)? Larger key, then smaller index.
__device__ inline bool ahead(uint32_t ka, int32_t ia, uint32_t kb, int32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Order of the n (<= kMaxSortedK) selected entries: ord[r] = the LDS position of
// the r-th best; sk and si are left as they are. Up to 256 entries every thread
// ranks one entry against all of them (no barriers inside the loop); more are
// sorted by a bitonic network over copies (tk, ti) that carries the positions.
template <int NT>
__device__ void order_selected(const uint32_t* sk, const int32_t* si, int n, int32_t* ord, uint32_t* tk,
                               int32_t* ti) {
  static_assert(NT >= 256, "one thread per entry up to 256");
  if (n <= 256) {
    const int j = threadIdx.x;
    if (j < n) {
      const uint32_t kj = sk[j];
      const int32_t ij = si[j];
      int r = 0;
      for (int t = 0; t < n; ++t) r += ahead(sk[t], si[t], kj, ij) ? 1 : 0;
      ord[r] = j;
    }
    __syncthreads();
    return;
  }
  const int np = pow2_at_least(n);  // padding sorts behind every real entry
  for (int j = threadIdx.x; j < np; j += NT) {
    tk[j] = j < n ? sk[j] : 0u;
    ti[j] = j < n ? si[j] : INT_MAX;
    ord[j] = j;
  }
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < np / 2; i += NT) {
        const int a = 2 * i - (i & (stride - 1));
        const int b = a + stride;
        const bool best_first = (a & size) == 0;
        if (ahead(tk[b], ti[b], tk[a], ti[a]) == best_first) {
          const uint32_t x = tk[a];
          tk[a] = tk[b];
          tk[b] = x;
          const int32_t y = ti[a];
          ti[a] = ti[b];
          ti[b] = y;
          const int32_t z = ord[a];
          ord[a] = ord[b];
          ord[b] = z;
        }
      }
      __syncthreads();
    }
  }
}

// LDS of the selecting kernels: the selected entries, their order and scratch.
struct SelLds {
  uint32_t key[kMaxSortedK];
  int32_t idx[kMaxSortedK];
  int32_t p0[kMaxSortedK];
  int32_t p1[kMaxSortedK];
  int32_t ord[kMaxSortedK];
  uint32_t tk[kMaxSortedK];
  int32_t ti[kMaxSortedK];
  uint64_t cand[kSelCand];  // select_ordered's candidates (rank words; 0: empty) and payloads
  int32_t cp0[kSelCand];
  int32_t cp1[kSelCand];
};

// The value held by lane (this lane ^ J) of the wave, J a power of two below
// 64: DPP quad permutations for 1 and 2, the swizzle crossbar for 4 to 16,
// a permute for 32.
template <int J>
__device__ inline uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (J < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (J << 10));
  else return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) << 2), (int)v);
}

// Inclusive prefix sum over the wave's 64 lanes: shifts by 1, 2, 4 and 8
// within each 16-lane row (lanes shifted in from outside the row add 0), then
// the row totals carried forward by the row broadcasts of lanes 15 and 31.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_add(uint32_t v) {
  return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ inline uint32_t wave_incl_sum(uint32_t v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Bitonic sort of the wave's 64 values (one per lane), largest in lane 0.
__device__ inline uint32_t wave_sort_desc(uint32_t v) {
  const int lane = threadIdx.x & 63;
  auto step = [&](auto JJ, int k) __attribute__((always_inline)) {
    constexpr int J = decltype(JJ)::value;
    const uint32_t o = lane_xor<J>(v);
    // within a block of k lanes sorted descending when (lane & k) == 0: the
    // lower lane of a pair keeps the larger value
    const bool lower = (lane & J) == 0;
    const bool desc = (lane & k) == 0;
    v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  using I32 = std::integral_constant<int, 32>;
  step(I1{}, 2);
  step(I2{}, 4), step(I1{}, 4);
  step(I4{}, 8), step(I2{}, 8), step(I1{}, 8);
  step(I8{}, 16), step(I4{}, 16), step(I2{}, 16), step(I1{}, 16);
  step(I16{}, 32), step(I8{}, 32), step(I4{}, 32), step(I2{}, 32), step(I1{}, 32);
  step(I32{}, 64), step(I16{}, 64), step(I8{}, 64), step(I4{}, 64), step(I2{}, 64), step(I1{}, 64);
  return v;
}

// (key, index) as one 64-bit word that orders as (key desc, index asc) does;
// 0 is below every candidate's word (keys of candidates are non-zero).
__device__ inline uint64_t rank_word(uint32_t key, int32_t idx) { return ((uint64_t)key << 32) | (uint32_t)~idx; }
__device__ inline uint32_t word_key(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ inline int32_t word_idx(uint64_t w) { return (int32_t)~(uint32_t)w; }

// Ranks of the first n words of w (n <= 256; the slots from n up to the next
// multiple of 8 * lpc hold 0), NT threads: lane `part` of the lpc adjacent
// lanes given word `ci` counts the words above it among every lpc-th slot from
// `part` on, eight reads in flight per step, and the group's counts are summed.
// lpc is NT / 64 (n <= 64), NT / 128 (n <= 128) or NT / 256, at most 16; ci =
// threadIdx.x / lpc may be >= n (its word is then a padding 0 or past the
// words; the caller ignores it).
template <int NT>
__device__ inline uint32_t rank_in_lds(const uint64_t* w, uint32_t n, uint64_t& mine, uint32_t& ci, uint32_t& part) {
  static_assert(NT == 256 || NT == 512 || NT == 1024, "whole groups of lanes per wave");
  const uint32_t lpc = n <= 64 ? NT / 64 : (n <= 128 ? NT / 128 : NT / 256);
  ci = threadIdx.x / lpc;
  part = threadIdx.x % lpc;
  mine = w[ci];
  const uint32_t step = 8u * lpc;
  const uint32_t end = (n + step - 1) / step * step;
  uint32_t r = 0;
  for (uint32_t jb = part; jb < end; jb += step) {
    uint64_t o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = w[jb + u * lpc];
#pragma unroll
    for (int u = 0; u < 8; ++u) r += o[u] > mine ? 1u : 0u;
  }
  // the lpc lanes of a group are adjacent, within sixteen
  if (lpc >= 2) r += lane_xor<1>(r);
  if (lpc >= 4) r += lane_xor<2>(r);
  if (lpc >= 8) r += lane_xor<4>(r);
  if (lpc >= 16) r += lane_xor<8>(r);
  return r;
}

// Select the best m candidates (non-zero keys) by (key desc, idx asc), in
// order: on return L.key/idx/p0/p1[r] hold the r-th best for r < the returned
// count (min(m, candidates), uniform across the block) and L.ord[r] = r.
//
// Most selections have few contenders near the top, so a filter comes first.
// With NT threads, i.e. W = NT / 64 waves, every wave sorts its 64 threads' own
// best keys. With q = ceil(m / W), let t be the smallest q-th largest among the
// F waves that have q non-empty threads: their q best thread keys are F q
// distinct candidates with keys >= t, so when F q >= m the m-th best key is
// >= t and every one of the best m passes the filter key >= t (otherwise t =
// 1: every candidate passes). Any one wave's m-th largest (m <= 64) is also a
// valid threshold, since that wave alone has m candidates at or above it; the
// filter takes the larger of the two. When at most 256
// candidates pass, each is ranked against all the others (its rank is its
// position in the order; indices are unique, so ranks are distinct);
// otherwise the radix select and the sort below run as usual.
//
// A caller that knows a valid threshold (one with at least m candidates at
// or above it) passes it as `hint` (0: none), and the waves' sort is skipped.
// Passing candidates get their slots from a prefix sum over each wave and one
// LDS atomic per wave; the slots past the last candidate stay 0, so the
// ranking (rank_in_lds) reads whole groups of eight with no bounds checks.
template <int E, bool PAY, int NT>
__device__ int select_ordered(const uint32_t (&key)[E], const int32_t (&idx)[E], const int32_t (&p0)[E],
                              const int32_t (&p1)[E], uint32_t m, SelShared& sh, SelLds& L, uint32_t hint = 0) {
  if (m == 0) return 0;
  static_assert(E <= 64, "one bit per slot");
  if (threadIdx.x == 0) sh.count = 0u;
  if (threadIdx.x < kSelCand) L.cand[threadIdx.x] = 0ull;  // published by the barrier below, before any slot is written
  uint32_t thr = 1u;
  if (hint) {
    thr = hint;
    __syncthreads();
  } else if (m <= (uint32_t)kSelCand) {
    constexpr int kWaves = NT / 64;
    const uint32_t q = (m + kWaves - 1) / kWaves;
    uint32_t best = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) best = key[e] > best ? key[e] : best;
    // tw: the wave's q-th best thread key; tm: its m-th best (m <= 64), which
    // alone has m candidates at or above it (0 when it does not exist)
    const uint32_t sorted = wave_sort_desc(best);
    const uint32_t tw = (uint32_t)__builtin_amdgcn_readlane((int)sorted, (int)(q - 1));
    const uint32_t tm = m <= 64 ? (uint32_t)__builtin_amdgcn_readlane((int)sorted, (int)(m - 1)) : 0u;
    if ((threadIdx.x & 63) == 0) {
      sh.red[threadIdx.x >> 6] = tw;
      sh.hist[threadIdx.x >> 6] = tm;
    }
    __syncthreads();
    uint32_t t = 0xFFFFFFFFu, full = 0, t_one = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t tv = sh.red[w];
      full += tv ? 1u : 0u;
      t = (tv && tv < t) ? tv : t;
      t_one = sh.hist[w] > t_one ? sh.hist[w] : t_one;
    }
    const uint32_t t_all = full * q >= m ? t : 1u;
    thr = t_one > t_all ? t_one : t_all;
  } else {
    __syncthreads();
  }
  // this thread's candidates as bits (kept opaque, so that the compiler does
  // not carry E compare masks in scalar registers to the writes below)
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t in = key[e] >= thr ? 1u : 0u;  // thr >= 1: no empty slot passes
    if (e < 32) lo |= in << e;
    else hi |= in << (e - 32);
  }
  asm volatile("" : "+v"(lo), "+v"(hi));
  const uint32_t mine = __builtin_popcount(lo) + __builtin_popcount(hi);
  const uint32_t incl = wave_incl_sum(mine);
  const uint32_t wave_total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if (wave_total) {  // uniform over the wave
    uint32_t wbase = 0;
    if ((threadIdx.x & 63) == 63) wbase = atomicAdd(&sh.count, wave_total);
    uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63) + incl - mine;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t in = ((e < 32 ? lo : hi) >> (e & 31)) & 1u;
      if (in && pos < (uint32_t)kSelCand) {
        L.cand[pos] = rank_word(key[e], idx[e]);
        if (PAY) {
          L.cp0[pos] = p0[e];
          L.cp1[pos] = p1[e];
        }
      }
      pos += in;
    }
  }
  __syncthreads();
  const uint32_t n = sh.count;
  if (n > (uint32_t)kSelCand) {
    const int got = (int)select_best<E, PAY, NT>(key, idx, p0, p1, m, sh, L.key, L.idx, L.p0, L.p1);
    order_selected<NT>(L.key, L.idx, got, L.ord, L.tk, L.ti);
    return got;
  }
  uint64_t wc;
  uint32_t ci, part;
  const uint32_t r = rank_in_lds<NT>(L.cand, n, wc, ci, part);
  if (part == 0 && ci < n && r < m) {
    L.key[r] = word_key(wc);
    L.idx[r] = word_idx(wc);
    if (PAY) {
      L.p0[r] = L.cp0[ci];
      L.p1[r] = L.cp1[ci];
    }
    L.ord[r] = (int32_t)r;
  }
  __syncthreads();
  return (int)(n < m ? n : m);
}

// ---------------------------------------------------------------- top-K of rows

struct TopkParams {
  const float* x;
  int64_t vocab, stride;
  int32_t k, chunks;
  uint32_t* part_key;   // [rows][chunks][k]
  int32_t* part_idx;    // [rows][chunks][k]
  float2* part_stat;    // [rows][chunks]: (chunk max, sum of exp(x - max))
  int32_t* out_token;   // [rows][k]
  float* out_logprob;   // [rows][k]
};

// grid (chunks, rows), kChunkThreads threads: the chunk's best k entries, in
// order, and its (max, sum exp) pair. A chunk is E entries per thread.
template <bool VEC, int E>
__global__ __launch_bounds__(kChunkThreads) void topk_chunks(const TopkParams p) {
  constexpr int NT = kChunkThreads;
  __shared__ SelShared sh;
  __shared__ SelLds L;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const float* xr = p.x + row * p.stride;
  const int64_t beg = (int64_t)c * (NT * E);
  static_assert(E % 4 == 0, "16-byte loads");
  float v[E];
  uint32_t key[E];
  int32_t idx[E];
  // Entries past the vocabulary (only in a row's last chunk) read as -inf,
  // which changes neither the maximum nor the sum below, and get key 0 (an
  // empty slot) at the end; a chunk wholly inside the row has no such checks.
  const bool full = VEC && beg + (int64_t)NT * E <= p.vocab;  // uniform
  // entry e of thread t: 4 * (t + NT * (e / 4)) + e % 4 within the chunk (16-byte loads, coalesced)
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const int64_t i0 = beg + 4 * ((int64_t)threadIdx.x + NT * q);
    if (full || (VEC && i0 + 3 < p.vocab)) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr + i0));
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * q + j] = i0 + j < p.vocab ? xr[i0 + j] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) idx[4 * q + j] = (int32_t)(i0 + j);
  }
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, v[e]);
  m = wave_max(m);
  constexpr int kWaves = NT / 64;
  __shared__ float wm[kWaves], ws[kWaves];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wm[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, wm[w]);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) s += __expf(v[e] - m);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (full || idx[e] < p.vocab) ? float_key(v[e]) : 0u;
  // (select_ordered's first barrier also publishes ws)
  const int got = select_ordered<E, false, NT>(key, idx, idx, idx, (uint32_t)p.k, sh, L);
  const size_t base = ((size_t)row * p.chunks + c) * p.k;
  if (threadIdx.x == 0) {
    float s_all = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_all += ws[w];
    p.part_stat[(size_t)row * p.chunks + c] = make_float2(m, s_all);
  }
  // the chunk's best k in order; a short last chunk pads with empty slots
  for (int r = threadIdx.x; r < p.k; r += NT) {
    const bool ok = r < got;
    p.part_key[base + r] = ok ? L.key[L.ord[r]] : 0u;
    p.part_idx[base + r] = ok ? L.idx[L.ord[r]] : -1;
  }
}

// grid (rows), kMergeThreads threads: merge the chunks' candidates and
// statistics; k best in order. E candidate slots per thread (E * kMergeThreads
// >= chunks * k).
template <int E>
__global__ __launch_bounds__(kMergeThreads) void topk_merge(const TopkParams p) {
  constexpr int NT = kMergeThreads, kWaves = NT / 64;
  __shared__ SelShared sh;
  __shared__ SelLds L;
  __shared__ float red[kWaves];
  const int64_t row = blockIdx.x;
  const int M = p.chunks * p.k;
  const size_t base = (size_t)row * M;
  // the chunks' candidates (keys and indices requested together; padding of a
  // short chunk has key 0, an empty slot) and their (max, sum) pairs
  // Each thread takes a contiguous run of slots (the chunks' lists are sorted,
  // so a run mixes ranks, which keeps select_ordered's filter tight).
  const int per = (M + NT - 1) / NT;  // <= E
  uint32_t key[E];
  int32_t idx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = threadIdx.x * per + e;
    const bool in = e < per && j < M;
    key[e] = in ? p.part_key[base + j] : 0u;
    idx[e] = in ? p.part_idx[base + j] : -1;
  }
  const float2* ps = p.part_stat + (size_t)row * p.chunks;
  const float2 st = threadIdx.x < p.chunks ? ps[threadIdx.x] : make_float2(-INFINITY, 0.f);
  // log-sum-exp of the row from the chunk pairs
  float m = st.x;
  for (int c = threadIdx.x + NT; c < p.chunks; c += NT) m = fmaxf(m, ps[c].x);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  float s = threadIdx.x < p.chunks ? st.y * __expf(st.x - m) : 0.f;
  for (int c = threadIdx.x + NT; c < p.chunks; c += NT) s += ps[c].y * __expf(ps[c].x - m);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  float s_all = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s_all += red[w];
  const float lse = m + __logf(s_all);
  // Each chunk's list is sorted, so with r0 = ceil(k / chunks) the first r0
  // entries of every list are |S| = chunks * r0 >= k distinct candidates; the
  // k-th best of S is a valid threshold for select_ordered (at least k
  // candidates reach it), and a tight one: besides S only list entries past
  // the r0-th that beat it pass. It is found by ranking S's members against
  // each other (|S| <= 256); no hint (0) when S is larger or a short list has
  // an empty slot in it (then no member has rank k - 1 among the non-empty).
  const int r0 = (p.k + p.chunks - 1) / p.chunks;
  const int ns = p.chunks * r0;
  uint32_t tmin = 0u;
  if (ns <= kSelCand) {
    const int j = threadIdx.x;
    uint64_t w = 0;
    if (j < ns) {
      const size_t slot = base + (size_t)(j / r0) * p.k + (j % r0);
      const uint32_t sk = p.part_key[slot];
      w = sk ? rank_word(sk, p.part_idx[slot]) : 0ull;
    }
    if (j < kSelCand) L.cand[j] = w;  // zero past |S|, as rank_in_lds needs
    if (j == 0) sh.thr = 0u;
    __syncthreads();
    uint64_t ws;
    uint32_t ci, part;
    const uint32_t r = rank_in_lds<NT>(L.cand, (uint32_t)ns, ws, ci, part);
    if (part == 0 && ci < (uint32_t)ns && ws != 0ull && r == (uint32_t)p.k - 1) sh.thr = word_key(ws);
    __syncthreads();  // also: every read of L.cand is done before select_ordered clears it
    tmin = sh.thr;
  }
  const int got = select_ordered<E, false, NT>(key, idx, idx, idx, (uint32_t)p.k, sh, L, tmin);
  for (int r = threadIdx.x; r < p.k; r += NT) {
    const bool ok = r < got;
    const int j = ok ? L.ord[r] : 0;
    p.out_token[row * p.k + r] = ok ? L.idx[j] : -1;
    p.out_logprob[row * p.k + r] = ok ? key_float(L.key[j]) - lse : -INFINITY;
  }
}

// ---------------------------------------------------------------- one depth of expansion

struct ExpandParams {
  const float* parent_score;  // [S] rows of w_prev, stride ps_stride
  const float* child_logq;    // [S][w_prev][k] rows, stride lq_stride
  const int32_t* cand_token;  // [S] rows of k, stride ct_stride
  int32_t* sel_parent;        // [S] rows of w, stride out_stride (same for the four outputs)
  int32_t* sel_cand;
  int32_t* sel_token;
  float* sel_score;
  int64_t ps_stride, lq_stride, ct_stride, out_stride;
  int32_t w_prev, k, w;
  float beta;
};

// grid (S): scores of every (parent slot p, candidate c) child, index p * k + c,
// and the w best by (score desc, index asc), written in that order. E slots
// per thread (E * kSelThreads >= w_prev * k).
template <int E>
__global__ __launch_bounds__(kSelThreads) void expand_kernel(const ExpandParams p) {
  constexpr int NT = kSelThreads;
  __shared__ SelShared sh;
  __shared__ SelLds L;
  const int64_t s = blockIdx.x;
  const float* ps = p.parent_score + s * p.ps_stride;
  const float* lq = p.child_logq + s * p.lq_stride;
  const int32_t* ct = p.cand_token + s * p.ct_stride;
  const int M = p.w_prev * p.k;
  // a contiguous run of children per thread (each parent's candidates come
  // sorted, so a run mixes ranks, which keeps select_ordered's filter tight)
  const int per = (M + NT - 1) / NT;  // <= E
  uint32_t key[E];
  int32_t idx[E], tok[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = threadIdx.x * per + e;
    const bool in = e < per && j < M;
    float sc = -INFINITY;
    tok[e] = -1;
    if (in) {
      const int par = j / p.k;
      const float a = ps[par] + lq[j];  // Algorithm 1's score update (eq. 5), in this order
      sc = a + p.beta;
      tok[e] = ct[j - par * p.k];
    }
    key[e] = (in && isfinite(sc)) ? float_key(sc) : 0u;
    idx[e] = in ? j : -1;
  }
  const int got = select_ordered<E, true, NT>(key, idx, tok, tok, (uint32_t)p.w, sh, L);
  const int64_t o = s * p.out_stride;
  for (int r = threadIdx.x; r < p.w; r += NT) {
    const bool ok = r < got;
    const int j = ok ? L.ord[r] : 0;
    const int child = ok ? L.idx[j] : 0;
    p.sel_parent[o + r] = ok ? child / p.k : -1;
    p.sel_cand[o + r] = ok ? child % p.k : -1;
    p.sel_token[o + r] = ok ? L.p0[j] : -1;
    p.sel_score[o + r] = ok ? key_float(L.key[j]) : -INFINITY;
  }
}

// ---------------------------------------------------------------- deferred top-B

struct PruneParams {
  const int32_t* sel_parent;  // [S][depths][w]
  const int32_t* sel_token;
  const float* sel_score;
  const int32_t* root_token;  // [S]
  int32_t* parent;            // [S][budget + 1]
  int32_t* token;
  int32_t* depth;
  float* score;
  int32_t* n_out;             // [S]
  int32_t depths, w, budget;
};

// grid (S): the best `budget` supertree nodes by (score desc, depth asc, slot
// asc) -- node index (d - 1) * w + slot orders depth, then slot -- flattened
// after the root in that order. E slots per thread (E * kPruneThreads >= depths * w).
template <int E>
__global__ __launch_bounds__(kPruneThreads) void prune_kernel(const PruneParams p) {
  constexpr int NT = kPruneThreads;
  __shared__ SelShared sh;
  __shared__ SelLds L;
  __shared__ int16_t newpos[kSelMaxCand];  // supertree node -> row in the output (-1: not kept)
  __shared__ int bad;
  const int64_t s = blockIdx.x;
  const int M = p.depths * p.w;
  const int32_t* spar = p.sel_parent + s * M;
  const int32_t* stok = p.sel_token + s * M;
  const float* ssc = p.sel_score + s * M;
  uint32_t key[E];
  int32_t idx[E], tok[E], par[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = threadIdx.x + NT * e;
    const bool in = j < M;
    const float sc = in ? ssc[j] : -INFINITY;
    par[e] = in ? spar[j] : -1;
    tok[e] = in ? stok[j] : -1;
    key[e] = (in && par[e] >= 0 && par[e] < p.w && isfinite(sc)) ? float_key(sc) : 0u;
    idx[e] = j;
  }
  for (int j = threadIdx.x; j < M; j += NT) newpos[j] = -1;
  if (threadIdx.x == 0) bad = 0;
  const int got = select_ordered<E, true, NT>(key, idx, tok, par, (uint32_t)p.budget, sh, L);
  for (int r = threadIdx.x; r < got; r += NT) newpos[L.idx[L.ord[r]]] = (int16_t)(r + 1);
  __syncthreads();
  // With beta <= 0 and log-probabilities <= 0 a child never precedes its parent
  // (Lemma 1); check it, and if the data break it keep only nodes whose parent
  // is kept before them.
  for (int r = threadIdx.x; r < got; r += NT) {
    const int j = L.ord[r];
    const int node = L.idx[j];
    if (node >= p.w) {  // depth > 1
      const int pp = newpos[node - p.w - node % p.w + L.p1[j]];
      if (pp < 1 || pp > r) bad = 1;
    }
  }
  __syncthreads();
  int kept = got;
  if (bad) {  // violated device contract: a sequential, prefix-closed subset
    if (threadIdx.x == 0) {
      for (int j = 0; j < M; ++j) newpos[j] = -1;
      int cnt = 0;
      for (int r = 0; r < got; ++r) {
        const int j = L.ord[r];
        const int node = L.idx[j];
        const int pp = node >= p.w ? newpos[node - p.w - node % p.w + L.p1[j]] : 0;
        if (pp >= 0) {
          L.ord[cnt] = j;
          newpos[node] = (int16_t)(cnt + 1);
          ++cnt;
        }
      }
      sh.count = (uint32_t)cnt;
    }
    __syncthreads();
    kept = (int)sh.count;
  }
  const int64_t o = s * (int64_t)(p.budget + 1);
  if (threadIdx.x == 0) {
    p.parent[o] = -1;
    p.token[o] = p.root_token[s];
    p.depth[o] = 0;
    p.score[o] = 0.f;
    p.n_out[s] = kept + 1;
  }
  for (int r = threadIdx.x; r < p.budget; r += NT) {
    const int64_t row = o + 1 + r;
    if (r < kept) {
      const int j = L.ord[r];
      const int node = L.idx[j];
      p.parent[row] = node >= p.w ? newpos[node - p.w - node % p.w + L.p1[j]] : 0;
      p.token[row] = L.p0[j];
      p.depth[row] = node / p.w + 1;
      p.score[row] = key_float(L.key[j]);
    } else {
      p.parent[row] = -1;
      p.token[row] = -1;
      p.depth[row] = -1;
      p.score[row] = -INFINITY;
    }
  }
}

// Chunk size: 10240 entries from 16 rows on (about one workgroup per CU for
// a 16-row, 152K-entry table, and fewer lists to merge), 4096 below.
int topk_chunk_len(int64_t rows) { return rows >= 16 ? kTopkChunkLarge : kTopkChunkSmall; }

int topk_plan(int64_t rows, int64_t vocab, int32_t k, int* chunks) {
  if (rows < 0 || vocab < 1 || vocab > INT_MAX) return DT_ERR_SHAPE;
  if (k < 1 || k > vocab) return DT_ERR_SHAPE;
  if (k > kMaxSortedK || rows > 65535) return DT_ERR_UNSUPPORTED;
  const int64_t c = ceil_div(vocab, topk_chunk_len(rows));
  if (c * k > kSelMaxCand || c > 65535) return DT_ERR_UNSUPPORTED;
  *chunks = (int)c;
  return DT_OK;
}

size_t topk_ws_bytes(int64_t rows, int chunks, int32_t k) {
  const size_t cand = (size_t)rows * chunks * k;
  return round_up(cand * 4, 256) + round_up(cand * 4, 256) + round_up((size_t)rows * chunks * sizeof(float2), 256);
}

}  // namespace
}  // namespace dt

extern "C" int dt_topk_rows_workspace_size(int64_t rows, int64_t vocab, int32_t k, size_t* bytes) {
  if (!bytes) return DT_ERR_NULL;
  int chunks = 0;
  const int st = dt::topk_plan(rows, vocab, k, &chunks);
  if (st != DT_OK) return st;
  *bytes = dt::topk_ws_bytes(rows, chunks, k);
  return DT_OK;
}

extern "C" int dt_topk_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t k,
                            int32_t* out_token, float* out_logprob, void* workspace, size_t workspace_bytes,
                            void* stream) {
  using namespace dt;
  int chunks = 0;
  int st = topk_plan(rows, vocab, k, &chunks);
  if (st != DT_OK) return st;
  if (row_stride < vocab) return DT_ERR_SHAPE;
  if (rows == 0) return DT_OK;
  if (!logits || !out_token || !out_logprob) return DT_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(out_token, 4) || !aligned(out_logprob, 4)) return DT_ERR_SHAPE;
  const size_t need = topk_ws_bytes(rows, chunks, k);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return DT_ERR_WORKSPACE;
  const size_t cand = (size_t)rows * chunks * k;
  char* ws = static_cast<char*>(workspace);
  TopkParams p;
  p.x = logits;
  p.vocab = vocab;
  p.stride = row_stride;
  p.k = k;
  p.chunks = chunks;
  p.part_key = reinterpret_cast<uint32_t*>(ws);
  p.part_idx = reinterpret_cast<int32_t*>(ws + round_up(cand * 4, 256));
  p.part_stat = reinterpret_cast<float2*>(ws + 2 * round_up(cand * 4, 256));
  p.out_token = out_token;
  p.out_logprob = out_logprob;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = aligned(logits, 16) && row_stride % 4 == 0;
  const dim3 cgrid((unsigned)chunks, (unsigned)rows);
  constexpr int kEL = kTopkChunkLarge / kChunkThreads, kES = kTopkChunkSmall / kChunkThreads;
  if (topk_chunk_len(rows) == kTopkChunkLarge) {
    if (vec) hipLaunchKernelGGL((topk_chunks<true, kEL>), cgrid, dim3(kChunkThreads), 0, s, p);
    else hipLaunchKernelGGL((topk_chunks<false, kEL>), cgrid, dim3(kChunkThreads), 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((topk_chunks<true, kES>), cgrid, dim3(kChunkThreads), 0, s, p);
    else hipLaunchKernelGGL((topk_chunks<false, kES>), cgrid, dim3(kChunkThreads), 0, s, p);
  }
  const int64_t M = (int64_t)chunks * k;
  constexpr int kM0 = 1024 / kMergeThreads, kM1 = 4096 / kMergeThreads, kM2 = kSelMaxCand / kMergeThreads;
  if (M <= kM0 * kMergeThreads)
    hipLaunchKernelGGL(topk_merge<kM0>, dim3((unsigned)rows), dim3(kMergeThreads), 0, s, p);
  else if (M <= kM1 * kMergeThreads)
    hipLaunchKernelGGL(topk_merge<kM1>, dim3((unsigned)rows), dim3(kMergeThreads), 0, s, p);
  else
    hipLaunchKernelGGL(topk_merge<kM2>, dim3((unsigned)rows), dim3(kMergeThreads), 0, s, p);
  return launch_status();
}

extern "C" int dt_expand_depth(int32_t num_seqs, int32_t w_prev, int32_t k, int32_t w, float beta,
                               const float* parent_score, int64_t parent_score_stride, const float* child_logq,
                               int64_t child_logq_stride, const int32_t* cand_token, int64_t cand_token_stride,
                               int32_t* sel_parent, int32_t* sel_cand, int32_t* sel_token, float* sel_score,
                               int64_t out_stride, void* stream) {
  using namespace dt;
  if (num_seqs < 0 || w_prev < 1 || k < 1 || w < 1) return DT_ERR_SHAPE;
  if ((int64_t)w_prev * k > kSelMaxCand || w > kMaxSortedK || num_seqs > 65535) return DT_ERR_UNSUPPORTED;
  if (!(beta <= 0.f) || !std::isfinite(beta)) return DT_ERR_VALUE;
  if (parent_score_stride < w_prev || child_logq_stride < (int64_t)w_prev * k || cand_token_stride < k ||
      out_stride < w)
    return DT_ERR_SHAPE;
  if (num_seqs == 0) return DT_OK;
  if (!parent_score || !child_logq || !cand_token || !sel_parent || !sel_cand || !sel_token || !sel_score)
    return DT_ERR_NULL;
  if (!aligned(parent_score, 4) || !aligned(child_logq, 4) || !aligned(cand_token, 4) || !aligned(sel_parent, 4) ||
      !aligned(sel_cand, 4) || !aligned(sel_token, 4) || !aligned(sel_score, 4))
    return DT_ERR_SHAPE;
  ExpandParams p;
  p.parent_score = parent_score;
  p.child_logq = child_logq;
  p.cand_token = cand_token;
  p.sel_parent = sel_parent;
  p.sel_cand = sel_cand;
  p.sel_token = sel_token;
  p.sel_score = sel_score;
  p.ps_stride = parent_score_stride;
  p.lq_stride = child_logq_stride;
  p.ct_stride = cand_token_stride;
  p.out_stride = out_stride;
  p.w_prev = w_prev;
  p.k = k;
  p.w = w;
  p.beta = beta;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = (int64_t)w_prev * k;
  if (M <= 4 * kSelThreads)
    hipLaunchKernelGGL(expand_kernel<4>, dim3((unsigned)num_seqs), dim3(kSelThreads), 0, st, p);
  else if (M <= 16 * kSelThreads)
    hipLaunchKernelGGL(expand_kernel<16>, dim3((unsigned)num_seqs), dim3(kSelThreads), 0, st, p);
  else
    hipLaunchKernelGGL(expand_kernel<kSelPerThread>, dim3((unsigned)num_seqs), dim3(kSelThreads), 0, st, p);
  return launch_status();
}

extern "C" int dt_prune_topb(int32_t num_seqs, int32_t depths, int32_t w, int32_t budget, const int32_t* sel_parent,
                             const int32_t* sel_token, const float* sel_score, const int32_t* root_token,
                             int32_t* parent, int32_t* token, int32_t* depth, float* score, int32_t* n_out,
                             void* stream) {
  using namespace dt;
  if (num_seqs < 0 || depths < 1 || w < 1 || budget < 0) return DT_ERR_SHAPE;
  if ((int64_t)depths * w > kSelMaxCand || budget + 1 > DT_MAX_TREE_NODES || num_seqs > 65535)
    return DT_ERR_UNSUPPORTED;
  if (num_seqs == 0) return DT_OK;
  if (!sel_parent || !sel_token || !sel_score || !root_token || !parent || !token || !depth || !score || !n_out)
    return DT_ERR_NULL;
  if (!aligned(sel_parent, 4) || !aligned(sel_token, 4) || !aligned(sel_score, 4) || !aligned(root_token, 4) ||
      !aligned(parent, 4) || !aligned(token, 4) || !aligned(depth, 4) || !aligned(score, 4) || !aligned(n_out, 4))
    return DT_ERR_SHAPE;
  PruneParams p;
  p.sel_parent = sel_parent;
  p.sel_token = sel_token;
  p.sel_score = sel_score;
  p.root_token = root_token;
  p.parent = parent;
  p.token = token;
  p.depth = depth;
  p.score = score;
  p.n_out = n_out;
  p.depths = depths;
  p.w = w;
  p.budget = budget;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = (int64_t)depths * w;
  constexpr int kP0 = 1024 / kPruneThreads, kP1 = 4096 / kPruneThreads, kP2 = kSelMaxCand / kPruneThreads;
  if (M <= kP0 * kPruneThreads)
    hipLaunchKernelGGL(prune_kernel<kP0>, dim3((unsigned)num_seqs), dim3(kPruneThreads), 0, st, p);
  else if (M <= kP1 * kPruneThreads)
    hipLaunchKernelGGL(prune_kernel<kP1>, dim3((unsigned)num_seqs), dim3(kPruneThreads), 0, st, p);
  else
    hipLaunchKernelGGL(prune_kernel<kP2>, dim3((unsigned)num_seqs), dim3(kPruneThreads), 0, st, p);
  return launch_status();
}
