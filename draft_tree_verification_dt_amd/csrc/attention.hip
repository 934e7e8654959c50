// Ancestor-only tree attention on gfx950.
//
// Operation (DARTree paper, Preliminaries > Tree Verification and DDTree; DDTree
// abstract): every node of a flattened draft tree attends to the whole verified
// prefix (already in the KV cache) and to the tree nodes on its own
// root-to-node path, in one pass for all nodes.
//
// Design
//  * Grouped-query packing: the g = Hq/Hkv query heads that share a KV head are
//    packed with the tree's nodes into n*g query rows, so one KV head's keys
//    meet a dense (n*g) x keys score block -- a real contraction for the
//    matrix cores even though n is a few hundred at most.
//  * A workgroup (4 waves) owns 128 query rows of one (sequence, KV head) and
//    one chunk of that sequence's keys. Keys are visited in tiles of 64; each
//    tile of K and V is staged in LDS once and read by all four waves. Two
//    workgroups share a CU, so one's tile loads overlap the other's math.
//  * Each wave holds 32 query rows. Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so that every lane ends up
//    holding the scores of ONE query row: the softmax needs no cross-lane
//    traffic except one exchange between the two half-waves, and the
//    probabilities are already laid out as the B operand of O^T = V^T P^T.
//    V is therefore staged transposed (V^T, d-major) in LDS.
//  * Online softmax in the exp2 domain, fp32 statistics and accumulators;
//    probabilities are rounded to bf16 (nearest-even) for the PV product.
//  * Prefix keys need no mask. For tree keys the ancestor bitmask of each of
//    the workgroup's nodes is built in LDS by walking parent pointers.
//    Because parent[i] < i, a node's ancestors never exceed it, so tree keys
//    beyond the workgroup's last node are skipped outright.
//  * Sequences with too few row tiles to fill the GPU split their keys into
//    chunks; partial (O, m, l) go to a workspace and a second kernel merges
//    them with log-sum-exp weights.
//  * Work items are remapped so that the row tiles sharing one KV chunk are
//    dispatched to the same XCD (workgroups go round-robin over the 8 XCDs),
//    which keeps that chunk's K/V in one L2.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.h"

namespace dt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_bits;

constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kMaxSeqs = 32;    // sequences per launch (host loops over larger batches)
constexpr int kXcds = 8;
constexpr int kMinTiles = 4;   // key tiles per work item at least (automatic split sizing)
constexpr float kLog2e = 1.4426950408889634f;

struct SeqGeom {
  int64_t prefix_row0;  // first prefix row of this sequence
  int32_t node_off;     // first node row
  int32_t n;            // nodes
  int32_t P;            // prefix length
  int32_t splits;       // key chunks
  int32_t row_tiles;    // ceil(n*g / kBM)
  int32_t item_start;   // first work item
  int32_t part_base;    // first partial row (split sequences), else -1
  int32_t comb_start;   // first combine row (split sequences)
};

struct AttnParams {
  const bf16_bits* q;
  const bf16_bits* kt;
  const bf16_bits* vt;
  const bf16_bits* kp;
  const bf16_bits* vp;
  const int32_t* parent;
  bf16_bits* out;
  float* part_o;   // [part rows][D] unnormalised partial outputs
  float2* part_ml; // [part rows] (running max in log2 units, sum)
  int64_t q_rs, out_rs, t_rs, p_rs, p_hs;
  float scale_log2;
  int32_t Hq, Hkv, g;
  int32_t chunk;        // keys per split
  int32_t nseq;
  int32_t total_items;
  int32_t per_xcd;
  int32_t mask_words;   // words per ancestor-mask row (>= ceil(max n / 32) + 2)
  int32_t mask_rows;    // rows of the ancestor-mask table (max nodes per row tile)
  int32_t max_n;
  int32_t comb_rows;
  SeqGeom seq[kMaxSeqs];
};

__device__ inline int find_seq(const AttnParams& p, int item) {
  int s = 0;
  for (int i = 1; i < p.nseq; ++i)
    if (p.seq[i].item_start <= item) s = i;
  return s;
}

// 16-byte (8 x bf16) global load.
__device__ inline uint4 ld16(const bf16_bits* ptr) { return *reinterpret_cast<const uint4*>(ptr); }

// LDS tiles (D = head dim, rows of D*2 bytes, no padding). A tile of 64 keys
// of K and one of V per buffer, double-buffered. Rows are XOR-swizzled at
// 16-byte-chunk granularity so that the MFMA operand reads are free of bank
// conflicts while every lane's swizzle stays constant across the tile:
//   K: logical chunk c of row r sits at chunk c ^ k_swz(r)
//   V: logical chunk c of row r sits at chunk c ^ v_swz(r)
// Tiles are filled straight from global memory with global_load_lds_dwordx4
// (each wave instruction writes 1 KB of consecutive LDS; the lane picks the
// global chunk that belongs at its swizzled slot), so no registers stage them.
template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;  // rows one wave instruction fills
  static constexpr int kInstrPerWave = kBN / kRowsPerInstr / 4;
  static constexpr int kBytes = kBN * kRowBytes;          // one K (or V) tile
};

// The LDS has 64 four-byte banks, i.e. a bank row of 256 bytes (one row of a
// d = 128 tile, two rows of a d = 64 tile). The swizzles spread the 16 rows
// read by one quarter-wave (K, 16-byte reads) and the 4 rows x 4 chunks read by
// one half-wave (V, 8-byte transposing reads) over all 64 banks.
template <int D>
__device__ inline int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// Issue the loads of one K tile and one V tile (keys kb .. kb+63) into LDS,
// general form: each row may come from the prefix cache or from the tree's own
// K/V. Keys at or beyond key_end are read from row key_end-1 instead (always
// valid; those keys are masked out, so their values only need to be finite).
template <int D>
__device__ inline void issue_tile(const AttnParams& p, const SeqGeom& sg, int head, int kb, int key_end,
                                  char* kbuf, char* vbuf, int wave, int lane) {
  using T = Tile<D>;
  // The four base pointers as uniform values: selecting between them per lane
  // must not turn into a per-lane load of the pointer (which would also wait
  // for every load in flight).
  const char* kp = reinterpret_cast<const char*>(p.kp);
  const char* vp = reinterpret_cast<const char*>(p.vp);
  const char* kt = reinterpret_cast<const char*>(p.kt);
  const char* vt = reinterpret_cast<const char*>(p.vt);
  const int rsub = lane / T::kChunks;  // row within the instruction's rows
  const int pc = lane % T::kChunks;    // physical chunk this lane fills
#pragma unroll
  for (int i = 0; i < T::kInstrPerWave; ++i) {
    const int instr = wave * T::kInstrPerWave + i;
    const int row = instr * T::kRowsPerInstr + rsub;
    int key = kb + row;
    key = key < key_end ? key : key_end - 1;
    const bool pre = key < sg.P;
    const int64_t off = pre ? ((sg.prefix_row0 + key) * p.p_rs + (int64_t)head * p.p_hs) * 2
                            : ((int64_t)(sg.node_off + key - sg.P) * p.t_rs + (int64_t)head * D) * 2;
    const char* ksrc = (pre ? kp : kt) + off + ((pc ^ k_swz<D>(row)) << 4);
    const char* vsrc = (pre ? vp : vt) + off + ((pc ^ v_swz<D>(row)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)ksrc, (lds_void_ptr)(kbuf + instr * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)vsrc, (lds_void_ptr)(vbuf + instr * 1024), 16, 0, 0);
  }
}

// A wave-uniform pointer, kept in scalar registers.
__device__ inline const char* uniform_ptr(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Fast form for tiles that lie wholly inside the prefix: one wave-uniform base
// address per tile plus per-lane 32-bit byte offsets fixed for the whole loop.
template <int D>
struct PrefixLoads {
  using T = Tile<D>;
  uint32_t koff[T::kInstrPerWave];
  uint32_t voff[T::kInstrPerWave];

  __device__ inline void init(int64_t row_stride, int wave, int lane) {
    const int rsub = lane / T::kChunks, pc = lane % T::kChunks;
#pragma unroll
    for (int i = 0; i < T::kInstrPerWave; ++i) {
      const int row = (wave * T::kInstrPerWave + i) * T::kRowsPerInstr + rsub;
      const uint32_t roff = (uint32_t)(row * row_stride * 2);
      koff[i] = roff + ((pc ^ k_swz<D>(row)) << 4);
      voff[i] = roff + ((pc ^ v_swz<D>(row)) << 4);
    }
  }

  __device__ inline void issue(const AttnParams& p, const SeqGeom& sg, int head, int kb, char* kbuf, char* vbuf,
                               int wave) const {
    const int64_t first = ((sg.prefix_row0 + kb) * p.p_rs + (int64_t)head * p.p_hs) * 2;
    const char* kbase = uniform_ptr(reinterpret_cast<const char*>(p.kp) + first);
    const char* vbase = uniform_ptr(reinterpret_cast<const char*>(p.vp) + first);
#pragma unroll
    for (int i = 0; i < T::kInstrPerWave; ++i) {
      const int instr = wave * T::kInstrPerWave + i;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + koff[i]), (lds_void_ptr)(kbuf + instr * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + voff[i]), (lds_void_ptr)(vbuf + instr * 1024), 16, 0, 0);
    }
  }
};

// Bits [j0, j0 + cnt) of an ancestor-mask row, cnt <= 64, j0 >= 0.
__device__ inline uint64_t mask_bits(const uint32_t* row, int j0, int cnt) {
  const int w = j0 >> 5, off = j0 & 31;
  uint64_t lo = (uint64_t)row[w] | ((uint64_t)row[w + 1] << 32);
  uint64_t x = off ? ((lo >> off) | ((uint64_t)row[w + 2] << (64 - off))) : lo;
  return cnt >= 64 ? x : (x & ((1ull << cnt) - 1));
}

// Combine a value of lane l with that of lane l ^ 32 (the other half-wave),
// with one v_permlane32_swap (a VALU op; no LDS round trip).
__device__ inline float2 halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_halves(float v) {
  const float2 h = halves(v);
  return fmaxf(h.x, h.y);
}
__device__ inline float sum_halves(float v) {
  const float2 h = halves(v);
  return h.x + h.y;
}

constexpr float kRescaleSlack = 8.f;  // log2 units a stale running max may lag the true one
constexpr float kInitMax = -1.0e30f;  // finite "minus infinity" for the running max

template <int D>
__global__ __launch_bounds__(kThreads, 2) void tree_attn_fwd(const AttnParams p) {
  using T = Tile<D>;
  constexpr int KS = D / 16;  // k-steps of the QK^T product
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim
  // Double-buffered K and V tiles, four separate LDS objects: every access
  // names its buffer statically (the tile loop is unrolled by two), so the
  // compiler can tell that reading one buffer does not depend on the
  // asynchronous global->LDS loads still filling the other.
  __shared__ __attribute__((aligned(1024))) char k0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char k1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char v1[T::kBytes];
  extern __shared__ uint32_t dyn[];  // [max_n] parents, then [mask_rows][mask_words] ancestor masks

  // ---- work item (XCD-aware remap: consecutive items share an XCD) ----
  const int b = blockIdx.x;
  const int item = (b % kXcds) * p.per_xcd + b / kXcds;
  if (item >= p.total_items) return;
  const int s = find_seq(p, item);
  const SeqGeom& sg = p.seq[s];
  int local = item - sg.item_start;
  const int tile = local % sg.row_tiles;
  local /= sg.row_tiles;
  const int split = local % sg.splits;
  const int head = local / sg.splits;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const int lr = lane & 31;   // query row within the wave
  const int hh = lane >> 5;   // half-wave
  const int g = p.g;
  const int nrows = sg.n * g;

  const int row0 = tile * kBM;
  const int my_row = row0 + wave * 32 + lr;
  const bool row_ok = my_row < nrows;
  const int my_node = row_ok ? my_row / g : 0;
  const int my_qh = head * g + (row_ok ? my_row % g : 0);
  const int node_lo = row0 / g;
  const int node_hi = min(sg.n - 1, (min(row0 + kBM, nrows) - 1) / g);

  // ---- key range of this work item ----
  const int key_lo = split * p.chunk;
  int key_hi = min(key_lo + p.chunk, sg.P + sg.n);
  key_hi = min(key_hi, sg.P + node_hi + 1);  // later tree keys are no one's ancestor here
  const int ntiles = __builtin_amdgcn_readfirstlane(key_hi > key_lo ? (key_hi - key_lo + kBN - 1) / kBN : 0);

  // tiles below this key are wholly prefix and take the fast load path
  const int fast_end = min(sg.P, key_hi);
  PrefixLoads<D> pl;
  pl.init(p.p_rs, wave, lane);
  if (ntiles > 0) {
    if (key_lo + kBN <= fast_end)
      pl.issue(p, sg, head, key_lo, k0, v0, wave);
    else
      issue_tile<D>(p, sg, head, key_lo, key_hi, k0, v0, wave, lane);
  }

  uint32_t* par_s = dyn;
  uint32_t* masks = dyn + p.max_n;

  // ---- ancestor bitmasks of this tile's nodes (only if tree keys are visited) ----
  if (key_hi > sg.P) {
    for (int i = tid; i <= node_hi; i += kThreads) par_s[i] = (uint32_t)p.parent[sg.node_off + i];
    const int nmask = (node_hi - node_lo + 1) * p.mask_words;
    for (int i = tid; i < nmask; i += kThreads) masks[i] = 0u;
    __syncthreads();
    if (tid <= node_hi - node_lo) {
      uint32_t* row = masks + tid * p.mask_words;
      int j = node_lo + tid;
      // Walk to the root; parent[j] < j bounds the walk even for a malformed array.
      for (;;) {
        row[j >> 5] |= 1u << (j & 31);
        const int pj = (int)par_s[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
      }
    }
  }

  // ---- Q rows as the B operand of S^T = K Q^T: lane holds row lr, dims 16k + 8hh .. +7 ----
  bf16x8 qreg[KS];
  {
    const bf16_bits* qrow = p.q + (int64_t)(sg.node_off + my_node) * p.q_rs + (int64_t)my_qh * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint4 v = row_ok ? ld16(qrow + k * 16 + hh * 8) : make_uint4(0, 0, 0, 0);
      qreg[k] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  float m_run = kInitMax;  // running max (log2 units; may lag the true max by < kRescaleSlack)
  float l_run = 0.f;       // running sum over this half-wave's keys
  const float c = p.scale_log2;
  const int prefix_end = min(sg.P, key_hi);  // keys below this are visible to every row
  const uint32_t* my_mask = masks + (my_node - node_lo) * p.mask_words;

  // per-lane LDS byte offsets of the operand reads
  const int k_off = lr * T::kRowBytes;                       // + chunk, see below
  const int s16 = lane & 15, grp = lane >> 4;
  const int v_row = hh * 4 + (s16 >> 2);                     // + 32bb + 16sub + 8hi
  const int v_chunk_lo = (grp & 1) * 2 + ((s16 & 3) >> 1);    // + 4db, then swizzled
  const int v_in = (s16 & 1) * 8;

  // One tile: keys kb .. kb+63 from (kt, vt); the next tile is prefetched into (nk, nv).
  auto step = [&](const int t, const char* kt, const char* vt, char* nk, char* nv) __attribute__((always_inline)) {
    const int kb = key_lo + t * kBN;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads of tile t have landed (vmcnt = 0)
    __syncthreads();                     // everyone's have; everyone is done with tile t-1
    if (t + 1 < ntiles) {
      if (kb + 2 * kBN <= fast_end)
        pl.issue(p, sg, head, kb + kBN, nk, nv, wave);
      else
        issue_tile<D>(p, sg, head, kb + kBN, key_hi, nk, nv, wave, lane);
    }

    // S^T block bb (keys kb + 32bb ..): lane (lr, hh) gets keys 32bb + 8(j/4) + 4hh + (j%4), j = 0..15.
    // Operand reads are phased so that at most one K block and half of the V
    // operands are in registers at a time (the kernel runs two waves per SIMD,
    // 256 registers each); scheduling barriers keep the compiler from hoisting
    // later reads into earlier phases.
    auto load_k = [&](bf16x8* ka, int bb) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int chunk = (2 * k + hh) ^ k_swz<D>(lr);
        ka[k] = *reinterpret_cast<const bf16x8*>(kt + bb * 32 * T::kRowBytes + k_off + chunk * 16);
      }
    };
    // V^T operand (i, bb, sub): d = 32i .., keys 32bb + 16sub ..
    auto load_v = [&](bf16x8* va, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const int vch = ((i * 4 + v_chunk_lo) ^ v_swz<D>(v_row)) * 16 + v_in;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const char* vp0 = vt + (bb * 32 + sub * 16 + v_row) * T::kRowBytes + vch;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)vp0);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vp0 + 8 * T::kRowBytes));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            va[((i - i0) * 2 + bb) * 2 + sub] = *reinterpret_cast<const bf16x8*>(&a8);
          }
      }
    };
    constexpr int kVHalf = DB / 2 > 0 ? DB / 2 : 1;  // d-blocks whose V operands are read before the softmax
    f32x16 sc[2];
    bf16x8 va[kVHalf * 4];
    {
      bf16x8 ka[KS];
      load_k(ka, 0);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k], qreg[k], k ? sc[0] : f32x16{}, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_k(ka, 1);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k], qreg[k], k ? sc[1] : f32x16{}, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_v(va, 0, kVHalf);
    }

    // ---- mask (tiles touching tree keys or the range end), then the running max ----
    if (kb + kBN > prefix_end) {
      uint64_t vis = 0;
      const int npre = prefix_end - kb;
      if (npre > 0) vis = npre >= 64 ? ~0ull : ((1ull << npre) - 1);
      const int tlo = max(sg.P, kb), thi = min(key_hi, kb + kBN);
      if (row_ok && thi > tlo) vis |= mask_bits(my_mask, tlo - sg.P, thi - tlo) << (tlo - kb);
      // this half-wave's keys sit at bits 32bb + 8(j/4) + 4hh + (j%4); after the
      // per-lane shift by 4hh every bit position below is a constant
      const uint64_t vh = vis >> (hh * 4);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kk = bb * 32 + (j >> 2) * 8 + (j & 3);
          if (!((vh >> kk) & 1ull)) sc[bb][j] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) mx = fmaxf(mx, fmaxf(sc[bb][j], sc[bb][j + 1]));
    mx = max_halves(mx);
    const float mt = mx * c;
    // Rescale only when a row's max jumps by more than the slack (rare after
    // the first tiles). The decision is per row, so a row's arithmetic depends
    // on its own visible keys only; the branch is taken if any row needs it.
    const bool need = mt > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] *= alpha;
    }
    const float neg_m = -m_run;
    bf16x8 pb[2][2];
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        bf16x2 pr;
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][j], c, neg_m));
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][j + 1], c, neg_m));
        pb[bb][j >> 3][j & 7] = pr[0];
        pb[bb][j >> 3][(j & 7) + 1] = pr[1];
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);  // sums the rounded probabilities
      }

    // ---- O^T += V^T P^T, first the d-blocks whose operands are in registers ----
#pragma unroll
    for (int i = 0; i < kVHalf; ++i)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[(i * 2 + bb) * 2 + sub], pb[bb][sub], acc[i], 0, 0, 0);
    if constexpr (DB > kVHalf) {
      load_v(va, kVHalf, DB);
#pragma unroll
      for (int i = kVHalf; i < DB; ++i)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[((i - kVHalf) * 2 + bb) * 2 + sub], pb[bb][sub],
                                                               acc[i], 0, 0, 0);
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, k0, v0, k1, v1);
    if (t + 1 < ntiles) step(t + 1, k1, v1, k0, v0);
  }

  // ---- epilogue: lane (lr, hh) holds O^T[d][row lr] for d = 32i + 8(j/4) + 4hh + (j%4) ----
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  if (sg.splits == 1) {
    const float inv = 1.f / l_tot;
    bf16_bits* orow = p.out + (int64_t)(sg.node_off + my_node) * p.out_rs + (int64_t)my_qh * D;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        __bf16 o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[i][j4 * 4 + e] * inv);
        *reinterpret_cast<uint2*>(orow + i * 32 + j4 * 8 + hh * 4) = *reinterpret_cast<uint2*>(o4);
      }
  } else {
    const int64_t prow = (int64_t)sg.part_base + ((int64_t)split * sg.n + my_node) * p.Hq + my_qh;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *reinterpret_cast<float4*>(po + i * 32 + j4 * 8 + hh * 4) =
            make_float4(acc[i][j4 * 4], acc[i][j4 * 4 + 1], acc[i][j4 * 4 + 2], acc[i][j4 * 4 + 3]);
    if (hh == 0) p.part_ml[prow] = make_float2(m_run, l_tot);
  }
}

// Merge the per-chunk partials of split sequences. A thread owns four
// consecutive dims of one (node, query head) row, so the threads of a row read
// each chunk's partial as one contiguous 512-byte (d = 128) line.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine(const AttnParams p) {
  constexpr int kTpr = D / 4;          // threads per row
  constexpr int kRpb = 256 / kTpr;     // rows per block
  const int row = blockIdx.x * kRpb + threadIdx.x / kTpr;
  const int c4 = threadIdx.x % kTpr;
  if (row >= p.comb_rows) return;
  int s = -1;
  for (int i = 0; i < p.nseq; ++i)
    if (p.seq[i].splits > 1 && p.seq[i].comb_start <= row) s = i;
  if (s < 0) return;
  const SeqGeom& sg = p.seq[s];
  const int r = row - sg.comb_start;  // = node * Hq + qh
  if (r >= sg.n * p.Hq) return;
  const int node = r / p.Hq, qh = r % p.Hq;
  // partial row of chunk k: part_base + (k * n + node) * Hq + qh = part_base + r + k * n * Hq
  const int64_t prow0 = (int64_t)sg.part_base + r;
  const int64_t kstride = (int64_t)sg.n * p.Hq;
  const float4* po = reinterpret_cast<const float4*>(p.part_o);
  // One pass with a running maximum; chunks are loaded eight at a time so
  // that their loads are in flight together.
  constexpr int kBatch = 8;
  float m = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < sg.splits; k0 += kBatch) {
    float2 ml[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = min(k0 + u, sg.splits - 1);
      const int64_t prow = prow0 + k * kstride;
      ml[u] = p.part_ml[prow];
      v[u] = po[prow * kTpr + c4];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // a chunk that saw no visible key for this row (l = 0) contributes nothing
      if (k0 + u < sg.splits && ml[u].y > 0.f) {
        const float mn = fmaxf(m, ml[u].x);
        const float a = __builtin_amdgcn_exp2f(m - mn);
        const float w = __builtin_amdgcn_exp2f(ml[u].x - mn);
        l = l * a + w * ml[u].y;
        o.x = o.x * a + w * v[u].x;
        o.y = o.y * a + w * v[u].y;
        o.z = o.z * a + w * v[u].z;
        o.w = o.w * a + w * v[u].w;
        m = mn;
      }
    }
  }
  const float inv = 1.f / l;
  __bf16 o4[4] = {(__bf16)(o.x * inv), (__bf16)(o.y * inv), (__bf16)(o.z * inv), (__bf16)(o.w * inv)};
  bf16_bits* orow = p.out + (int64_t)(sg.node_off + node) * p.out_rs + (int64_t)qh * D + c4 * 4;
  *reinterpret_cast<uint2*>(orow) = *reinterpret_cast<uint2*>(o4);
}

// ---------------------------------------------------------------- host side

struct Plan {
  std::vector<AttnParams> launches;  // one per group of <= kMaxSeqs sequences
  std::vector<int> grid;             // workgroups per launch
  std::vector<int> comb_grid;        // combine blocks per launch (0 = none)
  std::vector<size_t> lds;           // dynamic LDS bytes per launch
  size_t ws_bytes = 0;
};

int check_desc(const dt_attn_desc* d) {
  if (!d) return DT_ERR_NULL;
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return DT_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads) return DT_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return DT_ERR_UNSUPPORTED;
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale)) return DT_ERR_SHAPE;
  if (d->split_keys < 0 || d->split_keys % kBN) return DT_ERR_SHAPE;
  if (!d->node_offsets || !d->prefix_lens || !d->prefix_row_start) return DT_ERR_NULL;
  if (d->node_offsets[0] != 0) return DT_ERR_SHAPE;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int n = d->node_offsets[s + 1] - d->node_offsets[s];
    if (n < 1 || n > DT_MAX_TREE_NODES) return n < 1 ? DT_ERR_SHAPE : DT_ERR_UNSUPPORTED;
    if (d->prefix_lens[s] < 0 || d->prefix_row_start[s] < 0) return DT_ERR_SHAPE;
  }
  const int64_t D = d->head_dim;
  const int64_t qrs = d->q_row_stride ? d->q_row_stride : d->num_q_heads * D;
  const int64_t ors = d->out_row_stride ? d->out_row_stride : d->num_q_heads * D;
  const int64_t trs = d->tree_row_stride ? d->tree_row_stride : d->num_kv_heads * D;
  if (qrs < d->num_q_heads * D || ors < d->num_q_heads * D || trs < d->num_kv_heads * D) return DT_ERR_SHAPE;
  if (qrs % 8 || ors % 8 || trs % 8 || d->prefix_row_stride % 8 || d->prefix_head_stride % 8) return DT_ERR_SHAPE;
  if (d->prefix_row_stride < 0 || d->prefix_head_stride < 0) return DT_ERR_SHAPE;
  // the kernel addresses 64 cache rows of a tile with 32-bit byte offsets
  if (d->prefix_row_stride >= ((int64_t)1 << 24)) return DT_ERR_UNSUPPORTED;
  return DT_OK;
}

int make_plan(const dt_attn_desc* d, Plan* plan) {
  int st = check_desc(d);
  if (st != DT_OK) return st;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != DT_OK) return st;
  const int g = d->num_q_heads / d->num_kv_heads;
  const int D = d->head_dim;

  // Keys per split. Every work item streams at most `chunk` keys; `chunk` is
  // uniform, so items cost about the same and the per-XCD item ranges balance.
  // It is sized so that the items fill the GPU's workgroup slots (two per CU)
  // about once, with at least kMinTiles key tiles per item to amortise the
  // prologue (Q rows, ancestor masks) and keep the tile pipeline busy.
  int64_t chunk = d->split_keys;
  if (chunk == 0) {
    int64_t total_tiles = 0, max_keys = 0;
    for (int s = 0; s < d->num_seqs; ++s) {
      const int n = d->node_offsets[s + 1] - d->node_offsets[s];
      const int64_t keys = (int64_t)d->prefix_lens[s] + n;
      const int64_t units = ceil_div((int64_t)n * g, kBM) * d->num_kv_heads;
      total_tiles += units * ceil_div(keys, kBN);
      max_keys = std::max(max_keys, keys);
    }
    const int64_t slots = 2LL * cus;
    const int64_t tiles = std::max<int64_t>(kMinTiles, ceil_div(total_tiles, slots));
    chunk = std::min(tiles * kBN, ceil_div(max_keys, kBN) * kBN);
  }
  if (chunk > (int64_t)1 << 30) chunk = (int64_t)1 << 30;

  size_t part_rows = 0;
  for (int s0 = 0; s0 < d->num_seqs; s0 += kMaxSeqs) {
    AttnParams a;
    std::memset(&a, 0, sizeof(a));
    a.nseq = std::min(kMaxSeqs, d->num_seqs - s0);
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.g = g;
    a.chunk = (int32_t)chunk;
    a.scale_log2 = d->softmax_scale * kLog2e;
    int items = 0, comb = 0, max_n = 1;
    for (int i = 0; i < a.nseq; ++i) {
      const int s = s0 + i;
      SeqGeom& sg = a.seq[i];
      sg.node_off = d->node_offsets[s];
      sg.n = d->node_offsets[s + 1] - d->node_offsets[s];
      sg.P = d->prefix_lens[s];
      sg.prefix_row0 = d->prefix_row_start[s];
      sg.row_tiles = (int32_t)ceil_div((int64_t)sg.n * g, kBM);
      sg.splits = (int32_t)std::max<int64_t>(1, ceil_div((int64_t)sg.P + sg.n, chunk));
      sg.item_start = items;
      items += sg.row_tiles * sg.splits * d->num_kv_heads;
      if (sg.splits > 1) {
        sg.part_base = (int32_t)part_rows;
        part_rows += (size_t)sg.splits * sg.n * d->num_q_heads;
        sg.comb_start = comb;
        comb += sg.n * d->num_q_heads;
      } else {
        sg.part_base = -1;
        sg.comb_start = -1;
      }
      max_n = std::max(max_n, sg.n);
    }
    if (part_rows > (size_t)INT32_MAX) return DT_ERR_UNSUPPORTED;
    a.total_items = items;
    a.per_xcd = (int32_t)ceil_div(items, kXcds);
    a.max_n = max_n;
    a.mask_words = (max_n + 31) / 32 + 2;
    a.mask_rows = (kBM - 1) / g + 2;
    a.comb_rows = comb;
    plan->launches.push_back(a);
    plan->grid.push_back(a.per_xcd * kXcds);
    plan->comb_grid.push_back(comb ? (int)ceil_div(comb, 256 / (d->head_dim / 4)) : 0);
    plan->lds.push_back(sizeof(uint32_t) * ((size_t)a.max_n + (size_t)a.mask_rows * a.mask_words));
  }
  (void)D;
  plan->ws_bytes = part_rows ? round_up(part_rows * (size_t)d->head_dim * sizeof(float), 256) +
                                   round_up(part_rows * sizeof(float2), 256)
                             : 0;
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_tree_attention_workspace_size(const dt_attn_desc* desc, size_t* bytes) {
  if (!bytes) return DT_ERR_NULL;
  dt::Plan plan;
  int st = dt::make_plan(desc, &plan);
  if (st != DT_OK) return st;
  *bytes = plan.ws_bytes;
  return DT_OK;
}

extern "C" int dt_tree_attention(const dt_attn_desc* desc, const void* q, const void* k_tree, const void* v_tree,
                                 const void* k_prefix, const void* v_prefix, const int32_t* parent, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dt;
  if (!q || !k_tree || !v_tree || !parent || !out) return DT_ERR_NULL;
  Plan plan;
  int st = make_plan(desc, &plan);
  if (st != DT_OK) return st;
  bool any_prefix = false;
  for (int s = 0; s < desc->num_seqs; ++s) any_prefix |= desc->prefix_lens[s] > 0;
  if (any_prefix && (!k_prefix || !v_prefix)) return DT_ERR_NULL;
  for (const void* ptr : {q, k_tree, v_tree, (const void*)out})
    if (!aligned(ptr, 16)) return DT_ERR_SHAPE;
  if (any_prefix && (!aligned(k_prefix, 16) || !aligned(v_prefix, 16))) return DT_ERR_SHAPE;
  if (!aligned(parent, 4)) return DT_ERR_SHAPE;
  if (plan.ws_bytes) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return DT_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DT_ERR_WORKSPACE;
  }

  const int64_t D = desc->head_dim;
  const int64_t qrs = desc->q_row_stride ? desc->q_row_stride : desc->num_q_heads * D;
  const int64_t ors = desc->out_row_stride ? desc->out_row_stride : desc->num_q_heads * D;
  const int64_t trs = desc->tree_row_stride ? desc->tree_row_stride : desc->num_kv_heads * D;
  size_t part_rows_bytes = 0;
  for (auto& a : plan.launches)
    for (int i = 0; i < a.nseq; ++i)
      if (a.seq[i].splits > 1)
        part_rows_bytes = std::max(part_rows_bytes,
                                   (size_t)(a.seq[i].part_base + (size_t)a.seq[i].splits * a.seq[i].n * a.Hq));
  float* part_o = static_cast<float*>(workspace);
  float2* part_ml = plan.ws_bytes
                        ? reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                                    round_up(part_rows_bytes * D * sizeof(float), 256))
                        : nullptr;

  hipStream_t st_ = static_cast<hipStream_t>(stream);
  for (size_t li = 0; li < plan.launches.size(); ++li) {
    AttnParams a = plan.launches[li];
    a.q = static_cast<const bf16_bits*>(q);
    a.kt = static_cast<const bf16_bits*>(k_tree);
    a.vt = static_cast<const bf16_bits*>(v_tree);
    a.kp = static_cast<const bf16_bits*>(k_prefix);
    a.vp = static_cast<const bf16_bits*>(v_prefix);
    a.parent = parent;
    a.out = static_cast<bf16_bits*>(out);
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.q_rs = qrs;
    a.out_rs = ors;
    a.t_rs = trs;
    a.p_rs = desc->prefix_row_stride;
    a.p_hs = desc->prefix_head_stride;
    if (a.total_items == 0) continue;
    if (D == 128) {
      hipLaunchKernelGGL(tree_attn_fwd<128>, dim3(plan.grid[li]), dim3(kThreads), plan.lds[li], st_, a);
      if (plan.comb_grid[li]) hipLaunchKernelGGL(tree_attn_combine<128>, dim3(plan.comb_grid[li]), dim3(256), 0, st_, a);
    } else {
      hipLaunchKernelGGL(tree_attn_fwd<64>, dim3(plan.grid[li]), dim3(kThreads), plan.lds[li], st_, a);
      if (plan.comb_grid[li]) hipLaunchKernelGGL(tree_attn_combine<64>, dim3(plan.comb_grid[li]), dim3(256), 0, st_, a);
    }
    st = launch_status();
    if (st != DT_OK) return st;
  }
  return DT_OK;
}
