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
//  * A workgroup of eight waves (two per SIMD, one workgroup per CU); each
//    wave owns 32 query rows. The workgroup is WM row groups x WN key slices
//    (WM * WN = 8): 256 rows x 64 keys per step for large trees, 128 x 128 or
//    64 x 256 for small ones (tiny trees over a long prefix take 128 x 128 even
//    with half its rows empty, for a deeper K/V ring). Every K/V tile staged in LDS serves all the
//    workgroup's rows, and the key slices of one row group are merged through
//    LDS at the end.
//  * Scores are computed transposed, S^T = K Q^T, so every lane holds the
//    scores of one query row: the softmax needs no cross-lane traffic except
//    one v_permlane32_swap between half-waves, and the probabilities are
//    already the B operand of O^T = V^T P^T. V stays row-major in LDS; its
//    transposed operand comes from ds_read_b64_tr_b16.
//  * K/V tiles go from global memory straight to LDS (global_load_lds_dwordx4)
//    through a ring of up to four stages, so that up to three tiles are in
//    flight while one is consumed: the load latency (one to three
//    microseconds under load) times the bytes one step consumes is what the
//    ring must cover. Each stage is its own LDS object so the compiler can see
//    that reading one stage does not wait on the loads filling the others.
//  * Online softmax in the exp2 domain with fp32 statistics and accumulators;
//    the running max is rescaled lazily; probabilities are rounded to bf16
//    (nearest-even) for the PV product and the row sums add those rounded
//    values.
//  * Prefix keys need no mask. For tree keys the ancestor bitmask of each of
//    the workgroup's nodes is built in LDS by walking parent pointers; because
//    parent[i] < i, tree keys beyond the workgroup's last node are skipped.
//  * When there are too few (sequence, KV head, row tile) units to occupy the
//    GPU, each unit's keys are split into chunks; partial (O, m, l) go to the
//    workspace (O as fp16 after an exact power-of-two scaling per row), each
//    workgroup's rows as one contiguous block, and a second kernel merges them
//    with log-sum-exp weights.
//  * Work items are ordered so that the row tiles sharing one key chunk are
//    dispatched to the same XCD (workgroups go round-robin over the 8 XCDs),
//    which keeps that chunk's K/V in one L2.
//  * Both kernels have a second instantiation for profiling that records the
//    GPU's real-time counter at fixed points of every workgroup (the
//    descriptor's phase stamps); the default instantiation has none of it.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>
#include <mutex>

#include "internal.h"

namespace dt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_bits;
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

constexpr int kWaveRows = 32;    // query rows per wave (one 32-row MFMA block)
constexpr int kBN = 64;          // keys per wave per step
constexpr int kWaves = 8;        // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSeqs = 32;     // sequences per launch (host loops over larger batches)
constexpr int kXcds = 8;
constexpr int kStageBudget = 128 * 1024;  // LDS bytes for the K/V pipeline
constexpr int kLdsBytes = 160 * 1024;     // LDS per workgroup on gfx950
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // log2 units a stale running max may lag the true one
constexpr int kStampSlots = 8;          // phase-stamp slots per workgroup (slot 7: 1 forward, 2 merge)
constexpr float kInitMax = -1.0e30f;  // finite "minus infinity" for the running max

struct SeqGeom {
  int64_t prefix_row0;  // first prefix row of this sequence
  int32_t node_off;     // first node row
  int32_t n;            // nodes
  int32_t P;            // prefix length
  int32_t splits;       // key chunks
  int32_t row_tiles;    // ceil(n*g / rows per workgroup)
  int32_t item_start;   // first work item
  int32_t part_base;    // first partial row (split sequences), else -1; the sequence's
                        // partial rows go (key chunk, KV head, packed row node * g + j)
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
  _Float16* part_o;  // [part rows][D] unnormalised partial outputs times 2^-e (|values| < 1)
  float4* part_ml;   // [part rows] (running max in log2 units, sum, 2^e, unused)
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
  uint64_t* stamps;     // optional phase stamps, kStampSlots per row: the forward kernel's
  int32_t stamp_wg0;    // workgroup b writes row stamp_wg0 + b, the merge kernel's block b
  int32_t stamp_cb0;    // row stamp_cb0 + b; rows from stamp_rows on are not written
  int32_t stamp_rows;
  SeqGeom seq[kMaxSeqs];
};

__device__ inline int find_seq(const AttnParams& p, int item) {
  int s = 0;
  for (int i = 1; i < p.nseq; ++i)
    if (p.seq[i].item_start <= item) s = i;
  return s;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// ---------------------------------------------------------------- tiles in LDS
//
// A tile is 64 keys x D dims of K or V, rows of 2D bytes without padding. The
// rows are XOR-swizzled at 16-byte-chunk granularity:
//   K: logical chunk c of row r sits at chunk c ^ k_swz(r)
//   V: logical chunk c of row r sits at chunk c ^ v_swz(r)
// The LDS has 64 four-byte banks, i.e. a bank row of 256 bytes (one row of a
// d = 128 tile, two rows of a d = 64 tile); the swizzles spread the 16 rows
// read by one quarter-wave (K, 16-byte reads) and the 4 rows x 4 chunks read
// by one half-wave (V, 8-byte transposing reads) over all 64 banks. Each
// global_load_lds_dwordx4 instruction of a wave writes 1 KB of consecutive LDS;
// every lane fetches the global chunk that belongs at its swizzled slot.
template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;  // rows one wave instruction fills
  static constexpr int kBytes = kBN * kRowBytes;          // one 64-key tile
  static constexpr int kSwzPeriod = D == 128 ? 4 : 2;     // instructions after which the lane swizzles repeat
};

template <int D>
__device__ inline int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Workgroup shape: WM row groups of 32 rows x WN key slices of 64 keys.
template <int D, int WM>
struct Shape {
  static constexpr int WN = kWaves / WM;
  static constexpr int RM = kWaveRows * WM;          // query rows per workgroup
  static constexpr int KN = kBN * WN;                // keys per step
  static constexpr int kPartBytes = KN * D * 2;      // the K (or V) part of a stage
  static constexpr int kStageBytes = 2 * kPartBytes;
  static constexpr int NST = kStageBudget / kStageBytes >= 4 ? 4 : (kStageBudget / kStageBytes >= 2 ? 2 : 1);
  static constexpr int kInstr = kPartBytes / 1024 / kWaves;  // per wave, per tensor, per stage
  static constexpr int kRegionBytes = 64 * (D / 32) * 16 * 4;  // one wave's accumulators
  static constexpr int kMergeRegions = (WN - 1) * WM;           // key-slice merge buffer (stage 0's K and V parts)
  static_assert(kInstr >= 1, "at least one load instruction per wave");
  static_assert(kPartBytes % kRegionBytes == 0, "merge regions tile a stage part");
  static_assert(kMergeRegions * kRegionBytes <= kStageBytes, "merge buffer fits in stage 0");
};

// Workgroup barrier for the K/V pipeline: this wave's LDS reads are complete
// (lgkmcnt = 0) and every wave has arrived. Unlike __syncthreads() it does not
// wait for this wave's outstanding global->LDS loads, which belong to later
// stages (each wave waits for the loads of the stage it is about to read
// before arriving); the memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ inline void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// A wave-uniform pointer, kept in scalar registers.
__device__ inline const char* uniform_ptr(const char* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

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

template <int D, int WM, bool STAMPS>
__global__ __launch_bounds__(kThreads, 2) void tree_attn_fwd(const AttnParams p) {
  using T = Tile<D>;
  using SH = Shape<D, WM>;
  constexpr int WN = SH::WN, RM = SH::RM, KN = SH::KN, NST = SH::NST;
  constexpr int KS = D / 16;  // k-steps of the QK^T product
  constexpr int DB = D / 32;  // 32-wide blocks of the head dim
  constexpr int kPer = 2 * SH::kInstr;  // vector-memory operations per wave per stage

  // K/V pipeline stages; the K and V tiles of every stage are separate LDS objects.
  __shared__ __attribute__((aligned(1024))) char k0[SH::kPartBytes];
  __shared__ __attribute__((aligned(1024))) char v0[SH::kPartBytes];
  __shared__ __attribute__((aligned(1024))) char k1[NST > 1 ? SH::kPartBytes : 1024];
  __shared__ __attribute__((aligned(1024))) char v1[NST > 1 ? SH::kPartBytes : 1024];
  __shared__ __attribute__((aligned(1024))) char k2[NST > 2 ? SH::kPartBytes : 1024];
  __shared__ __attribute__((aligned(1024))) char v2[NST > 2 ? SH::kPartBytes : 1024];
  __shared__ __attribute__((aligned(1024))) char k3[NST > 3 ? SH::kPartBytes : 1024];
  __shared__ __attribute__((aligned(1024))) char v3[NST > 3 ? SH::kPartBytes : 1024];
  struct Stage {
    char* k;
    char* v;
  };
  extern __shared__ uint32_t dyn[];  // parents, ancestor masks, key-slice merge statistics

  // Phase stamps (the STAMPS instantiation, for profiling only): lane 0 of
  // wave 0 records the 100 MHz real-time counter at fixed points of the
  // workgroup's life. The default instantiation has none of this code.
  auto stamp = [&](int k) __attribute__((always_inline)) {
    if constexpr (STAMPS) {
      const int row = p.stamp_wg0 + (int)blockIdx.x;
      if (threadIdx.x == 0 && row < p.stamp_rows) {
        p.stamps[(int64_t)row * kStampSlots + k] = __builtin_amdgcn_s_memrealtime();
        if (k == 0) p.stamps[(int64_t)row * kStampSlots + 7] = 1;
      }
    }
  };
  stamp(0);

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
  // Row group and key slice of this wave. Waves go round-robin over the four
  // SIMDs, so with this order the two waves of a SIMD hold different row
  // groups whenever WN > 1: a tile whose last row groups are empty (a small
  // tree) leaves one working wave on every SIMD instead of two on half of them.
  const int wm = wave / WN;  // row group
  const int wn = wave % WN;  // key slice
  const int lr = lane & 31;  // query row within a 32-row block
  const int hh = lane >> 5;  // half-wave
  const int g = p.g;
  const int nrows = sg.n * g;

  const int row0 = tile * RM;
  const int my_row = row0 + wm * kWaveRows + lr;
  const bool row_ok = my_row < nrows;
  const int my_node = row_ok ? my_row / g : 0;
  const int my_qh = head * g + (row_ok ? my_row % g : 0);
  const int node_lo = row0 / g;
  const int node_hi = min(sg.n - 1, (min(row0 + RM, nrows) - 1) / g);
  // a wave whose 32 rows are all past the tree's last row only loads and
  // synchronises; it computes nothing
  const bool wave_active = row0 + wm * kWaveRows < nrows;

  // ---- key range of this work item ----
  const int key_lo = split * p.chunk;
  int key_hi = min(key_lo + p.chunk, sg.P + sg.n);
  key_hi = min(key_hi, sg.P + node_hi + 1);  // later tree keys are no one's ancestor here
  const int nsteps = __builtin_amdgcn_readfirstlane(key_hi > key_lo ? (key_hi - key_lo + KN - 1) / KN : 0);
  const int fast_end = min(sg.P, key_hi);    // keys below this are prefix keys
  const int prefix_end = fast_end;           // ... and visible to every row

  uint32_t* par_s = dyn;
  uint32_t* masks = dyn + p.max_n;
  float* merge_ml = reinterpret_cast<float*>(masks + p.mask_rows * p.mask_words);

  // ---- K/V stage loads ----
  const char* kp_base = reinterpret_cast<const char*>(p.kp);
  const char* vp_base = reinterpret_cast<const char*>(p.vp);
  const char* kt_base = reinterpret_cast<const char*>(p.kt);
  const char* vt_base = reinterpret_cast<const char*>(p.vt);
  const int rsub = lane / T::kChunks;  // row within an instruction's rows
  const int pc = lane % T::kChunks;    // physical chunk this lane fills
  // Per-lane byte offsets of the prefix fast path, one per load instruction of this wave.
  uint32_t lane_k[SH::kInstr], lane_v[SH::kInstr];
#pragma unroll
  for (int i = 0; i < SH::kInstr; ++i) {
    const int row = (wave * SH::kInstr + i) * T::kRowsPerInstr + rsub;
    lane_k[i] = (uint32_t)(rsub * p.p_rs * 2) + ((pc ^ k_swz<D>(row)) << 4);
    lane_v[i] = (uint32_t)(rsub * p.p_rs * 2) + ((pc ^ v_swz<D>(row)) << 4);
  }
  // Issue the loads of the stage that holds keys kb .. kb + KN - 1.
  auto issue = [&](int kb, Stage stage) __attribute__((always_inline)) {
    if (kb + KN <= fast_end) {
      // wholly inside the prefix: uniform base per instruction plus the lane offsets
      // (uniform 64-bit base in scalar registers + a 32-bit lane offset)
      const int64_t first = ((sg.prefix_row0 + kb) * p.p_rs + (int64_t)head * p.p_hs) * 2;
#pragma unroll
      for (int i = 0; i < SH::kInstr; ++i) {
        const int instr = wave * SH::kInstr + i;
        const int64_t roff = first + (int64_t)instr * T::kRowsPerInstr * p.p_rs * 2;
        const char* kb_i = uniform_ptr(kp_base + roff);
        const char* vb_i = uniform_ptr(vp_base + roff);
        __builtin_amdgcn_global_load_lds((const void*)(kb_i + lane_k[i]), (lds_void_ptr)(stage.k + instr * 1024), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb_i + lane_v[i]), (lds_void_ptr)(stage.v + instr * 1024), 16,
                                         0, 0);
      }
    } else {
      // general form: rows from the prefix cache or from the tree's own K/V;
      // keys at or beyond key_hi re-read row key_hi - 1 (finite; masked out)
#pragma unroll
      for (int i = 0; i < SH::kInstr; ++i) {
        const int instr = wave * SH::kInstr + i;
        const int row = instr * T::kRowsPerInstr + rsub;
        int key = kb + row;
        key = key < key_hi ? key : key_hi - 1;
        const bool pre = key < sg.P;
        const int64_t off = pre ? ((sg.prefix_row0 + key) * p.p_rs + (int64_t)head * p.p_hs) * 2
                                : ((int64_t)(sg.node_off + key - sg.P) * p.t_rs + (int64_t)head * D) * 2;
        const char* ksrc = (pre ? kp_base : kt_base) + off + ((pc ^ k_swz<D>(row)) << 4);
        const char* vsrc = (pre ? vp_base : vt_base) + off + ((pc ^ v_swz<D>(row)) << 4);
        __builtin_amdgcn_global_load_lds((const void*)ksrc, (lds_void_ptr)(stage.k + instr * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)vsrc, (lds_void_ptr)(stage.v + instr * 1024), 16, 0, 0);
      }
    }
  };

  // The first stage is requested before anything else (Q, the masks), so
  // that its latency overlaps the rest of the set-up; the tree's parents go
  // first when this item needs them, so that waiting for them does not wait
  // for the stage.
  const bool need_mask = key_hi > sg.P;
  uint32_t par0 = 0;
  if (need_mask && tid <= node_hi) par0 = (uint32_t)p.parent[sg.node_off + tid];
  if (nsteps > 0) issue(key_lo, Stage{k0, v0});
  stamp(1);

  // ---- Q rows (B operand of S^T = K Q^T): lane holds row lr, dims 16k + 8hh .. +7 ----
  bf16x8 qreg[KS];
  {
    const bf16_bits* qrow = p.q + (int64_t)(sg.node_off + my_node) * p.q_rs + (int64_t)my_qh * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qrow + k * 16 + hh * 8) : make_uint4(0, 0, 0, 0);
      qreg[k] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  // ---- ancestor bitmasks of this tile's nodes (only if tree keys are visited) ----
  // Its barriers wait for LDS traffic only (the first stage's loads stay in
  // flight), and the first pass of parents was read before that stage.
  if (need_mask) {
    if (tid <= node_hi) par_s[tid] = par0;
    for (int i = tid + kThreads; i <= node_hi; i += kThreads) par_s[i] = (uint32_t)p.parent[sg.node_off + i];
    const int nmask = (node_hi - node_lo + 1) * p.mask_words;
    for (int i = tid; i < nmask; i += kThreads) masks[i] = 0u;
    stage_barrier();
    for (int t = tid; t <= node_hi - node_lo; t += kThreads) {
      uint32_t* row = masks + t * p.mask_words;
      int j = node_lo + t;
      // Walk to the root; parent[j] < j bounds the walk even for a malformed array.
      for (;;) {
        row[j >> 5] |= 1u << (j & 31);
        const int pj = (int)par_s[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
      }
    }
    stage_barrier();
  }

  // ---- running state ----
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  float m_run = kInitMax;  // running max (log2 units; may lag the true max by < kRescaleSlack)
  float l_run = 0.f;       // running sum over this half-wave's keys
  const float c = p.scale_log2;
  const uint32_t* my_mask = masks + (my_node - node_lo) * p.mask_words;

  // per-lane LDS byte offsets of the operand reads (within the wave's 64-key slice)
  const int k_off = lr * T::kRowBytes;
  const int s16 = lane & 15, grp = lane >> 4;
  const int v_row = hh * 4 + (s16 >> 2);                    // + 32bb + 16sub + 8hi
  const int v_chunk_lo = (grp & 1) * 2 + ((s16 & 3) >> 1);  // + 4i, then swizzled
  const int v_in = (s16 & 1) * 8;

  // Per-step pieces. S(step) = K Q^T of this wave's 64 keys of the step
  // (registers sc), P(step) = its probabilities (registers pb, after the online
  // softmax), and O^T += V^T P^T with the same step's V.
  f32x16 sc[2];     // S^T blocks bb: lane (lr, hh) holds keys 32bb + 8(j/4) + 4hh + (j%4), j = 0..15
  bf16x8 pb[2][2];  // P^T: B operand of the PV product, [bb][sub]

  auto load_k = [&](const char* kt, bf16x8* ka, int bb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int chunk = (2 * k + hh) ^ k_swz<D>(lr);
      ka[k] = *reinterpret_cast<const bf16x8*>(kt + bb * 32 * T::kRowBytes + k_off + chunk * 16);
    }
  };
  // V^T operands of d-blocks i0 .. i0+1, (i, bb, sub): d = 32i .., keys 32bb + 16sub ..
  // The sixteen transposing reads and the wait for them are one inline-assembly
  // statement, so no instruction can see the registers before the data has
  // arrived. Every read targets a stage whose global->LDS loads this wave has
  // already waited for. (With the compiler's transposing-read builtin instead,
  // it issues these reads four at a time, each group followed by a full wait,
  // which measured slower.)
  auto load_v = [&](const char* vt, uint2* vr, int i0) __attribute__((always_inline)) {
    uint32_t a[2];
#pragma unroll
    for (int il = 0; il < 2; ++il) {
      const int vch = (((i0 + il) * 4 + v_chunk_lo) ^ v_swz<D>(v_row)) * 16 + v_in;
      a[il] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(vt + v_row * T::kRowBytes + vch);
    }
    // vr[8 il + m] <- rows 8m .. of d-block i0 + il, i.e. [il][bb][sub][lo, hi]
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%18\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:%19\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:%23\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %8, %17 offset:%18\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%19\n\t"
        "ds_read_b64_tr_b16 %10, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:%21\n\t"
        "ds_read_b64_tr_b16 %12, %17 offset:%22\n\t"
        "ds_read_b64_tr_b16 %13, %17 offset:%23\n\t"
        "ds_read_b64_tr_b16 %14, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %15, %17 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15])
        : "v"(a[0]), "v"(a[1]), "i"(0 * T::kRowBytes), "i"(8 * T::kRowBytes), "i"(16 * T::kRowBytes),
          "i"(24 * T::kRowBytes), "i"(32 * T::kRowBytes), "i"(40 * T::kRowBytes), "i"(48 * T::kRowBytes),
          "i"(56 * T::kRowBytes));
  };
  // operand (il, bb, sub) of the d-block pair held in vr
  auto v_operand = [&](const uint2* vr, int il, int bb, int sub) __attribute__((always_inline)) -> bf16x8 {
    const uint2 lo = vr[il * 8 + (bb * 2 + sub) * 2], hi = vr[il * 8 + (bb * 2 + sub) * 2 + 1];
    const uint4 q = make_uint4(lo.x, lo.y, hi.x, hi.y);
    return *reinterpret_cast<const bf16x8*>(&q);
  };
  static_assert(DB % 2 == 0, "d-blocks come in pairs");

  // S(step): both 32-key blocks; one K block in registers at a time. Each
  // operand of the second block is read into the register of the first
  // block's operand that the product just issued has consumed, so those reads
  // overlap the first block's products.
  auto s_product = [&](const char* kt) __attribute__((always_inline)) {
    bf16x8 ka[KS];
    load_k(kt, ka, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k], qreg[k], k ? sc[0] : f32x16{}, 0, 0, 0);
      const int chunk = (2 * k + hh) ^ k_swz<D>(lr);
      ka[k] = *reinterpret_cast<const bf16x8*>(kt + 32 * T::kRowBytes + k_off + chunk * 16);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product,
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // then one LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k], qreg[k], k ? sc[1] : f32x16{}, 0, 0, 0);
  };
  // O^T += V^T P^T, two d-blocks at a time
  auto pv_product = [&](const char* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int i0 = 0; i0 < DB; i0 += 2) {
      uint2 vr[16];
      load_v(vt, vr, i0);
#pragma unroll
      for (int il = 0; il < 2; ++il)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
            acc[i0 + il] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(vr, il, bb, sub), pb[bb][sub],
                                                                   acc[i0 + il], 0, 0, 0);
    }
  };
  // Mask and online softmax of S(step) into P(step).
  auto softmax = [&](int step) __attribute__((always_inline)) {
    const int kbw = key_lo + step * KN + wn * kBN;
    if (kbw + kBN > prefix_end) {
      const int npre = prefix_end - kbw;
      uint64_t vis = npre <= 0 ? 0ull : (npre >= 64 ? ~0ull : ((1ull << npre) - 1));
      const int tlo = max(sg.P, kbw), thi = min(key_hi, kbw + kBN);
      if (row_ok && thi > tlo) vis |= mask_bits(my_mask, tlo - sg.P, thi - tlo) << (tlo - kbw);
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
    // row max as a tree (independent operations at every level, no serial chain)
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = fmaxf(sc[i >> 3][(i & 7) * 2], sc[i >> 3][(i & 7) * 2 + 1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = fmaxf(t[i], t[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = fmaxf(t[i], t[i + 4]);
    float mx = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
    mx = max_halves(mx);
    const float mt = mx * c;
    // Rescale only when a row's max jumps by more than the slack (rare after
    // the first steps). The decision is per row, so a row's arithmetic depends
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
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial row sums
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        bf16x2 pr;
        pr[0] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][j], c, neg_m));
        pr[1] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][j + 1], c, neg_m));
        pb[bb][j >> 3][j & 7] = pr[0];
        pb[bb][j >> 3][(j & 7) + 1] = pr[1];
        const int q = (j >> 1) & 3;
        ls[q] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls[q], false);  // sums the rounded probabilities
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // The whole step for one wave (the schedule without ping-pong).
  auto compute = [&](int step, Stage stage) __attribute__((always_inline)) {
    if (!wave_active) return;
    s_product(stage.k + wn * T::kBytes);
    softmax(step);
    pv_product(stage.v + wn * T::kBytes);
  };

  // ---- the pipeline: stage u of every group of NST steps lives in st<u> ----
  auto stage_ptr = [&](auto U) __attribute__((always_inline)) -> Stage {
    constexpr int u = decltype(U)::value;
    if constexpr (u == 0) return Stage{k0, v0};
    else if constexpr (u == 1) return Stage{k1, v1};
    else if constexpr (u == 2) return Stage{k2, v2};
    else return Stage{k3, v3};
  };
  // Wait until this wave's loads for `step` have landed: the loads of the
  // later steps already issued may stay in flight.
  auto wait_step = [&](int step) __attribute__((always_inline)) {
    const int later = min(NST - 2, nsteps - 1 - step);
    if (NST >= 4 && later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPer));
    else if (NST >= 3 && later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };
  auto run_step = [&](int step, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    wait_step(step);
    stage_barrier();  // every wave's loads of this step have landed; everyone is done with step - 1
    if (step == 0) stamp(3);
    if constexpr (NST > 1) {
      if (step + NST - 1 < nsteps)
        issue(key_lo + (step + NST - 1) * KN, stage_ptr(std::integral_constant<int, (u + NST - 1) % NST>{}));
    }
    compute(step, stage_ptr(U));
    if constexpr (NST == 1) {
      stage_barrier();  // everyone is done with the only stage
      if (step + 1 < nsteps) issue(key_lo + (step + 1) * KN, Stage{k0, v0});
    }
  };

  stamp(2);
  if constexpr (NST == 4 && WN == 1) {
    // Ping-pong: waves 0-3 (group A, one per SIMD) and waves 4-7 (group B) take
    // turns. Every step has two phases, each closed by a workgroup barrier; in
    // one a group runs its MFMA block -- O += V P of the previous step, then S
    // of this one -- while the other group runs the softmax of its step, so each
    // SIMD's matrix core is fed by one of its two waves while the other works
    // on the VALU. Group B trails group A by one phase. Tile s is read from
    // phase 2s (A's S) to phase 2s + 3 (B's PV); its stage is refilled with
    // tile s + 4 from phase 2s + 4 on, and each tile is loaded two steps ahead.
    // Each group requests its share of a tile at the start of its own softmax
    // phase (B in phase 2s, A in phase 2s + 1), so only four waves contend for
    // the address unit at a time and the MFMA blocks start without it.
    const bool grp_b = wave >= 4;
    auto x_block = [&](int s, Stage cur, Stage prev) __attribute__((always_inline)) {
      if (!wave_active) return;
      if (s > 0) pv_product(prev.v);
      s_product(cur.k);
    };
    // even phase of step s: tile s must have landed (tile s + 1 may still be
    // in flight); after the barrier, group B requests its share of tile s + 2
    auto even_barrier = [&](int s, auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      if (s + 1 < nsteps) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPer));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      stage_barrier();
      if (grp_b && s + 2 < nsteps) issue(key_lo + (s + 2) * KN, stage_ptr(std::integral_constant<int, (u + 2) % 4>{}));
    };
    // The two groups run separate copies of the loop (so that S and P are
    // never both live across a barrier) with the same sequence of barriers.
    auto group_a = [&](int s, auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      even_barrier(s, U);
      if (s == 0) stamp(3);
      x_block(s, stage_ptr(U), stage_ptr(std::integral_constant<int, (u + 3) % 4>{}));
      stage_barrier();
      if (s + 2 < nsteps) issue(key_lo + (s + 2) * KN, stage_ptr(std::integral_constant<int, (u + 2) % 4>{}));
      if (wave_active) softmax(s);
    };
    auto group_b = [&](int s, auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      even_barrier(s, U);
      if (s > 0 && wave_active) softmax(s - 1);
      stage_barrier();
      x_block(s, stage_ptr(U), stage_ptr(std::integral_constant<int, (u + 3) % 4>{}));
    };
    if (nsteps > 1) issue(key_lo + KN, Stage{k1, v1});
    if (!grp_b) {
      for (int s0 = 0; s0 < nsteps; s0 += 4) {
        group_a(s0, std::integral_constant<int, 0>{});
        if (s0 + 1 < nsteps) group_a(s0 + 1, std::integral_constant<int, 1>{});
        if (s0 + 2 < nsteps) group_a(s0 + 2, std::integral_constant<int, 2>{});
        if (s0 + 3 < nsteps) group_a(s0 + 3, std::integral_constant<int, 3>{});
      }
    } else {
      for (int s0 = 0; s0 < nsteps; s0 += 4) {
        group_b(s0, std::integral_constant<int, 0>{});
        if (s0 + 1 < nsteps) group_b(s0 + 1, std::integral_constant<int, 1>{});
        if (s0 + 2 < nsteps) group_b(s0 + 2, std::integral_constant<int, 2>{});
        if (s0 + 3 < nsteps) group_b(s0 + 3, std::integral_constant<int, 3>{});
      }
    }
    // drain: A finishes the last PV; B its last softmax, then its last PV
    if (nsteps > 0) {
      const int last = nsteps - 1;
      const Stage tail = (last & 3) == 0 ? Stage{k0, v0} : (last & 3) == 1 ? Stage{k1, v1}
                       : (last & 3) == 2 ? Stage{k2, v2} : Stage{k3, v3};
      stage_barrier();
      if (wave_active && !grp_b) pv_product(tail.v);
      else if (wave_active) softmax(last);
      stage_barrier();
      if (wave_active && grp_b) pv_product(tail.v);
    }
  } else {
  // prologue: the first NST - 1 stages (one if NST == 1); the first is in flight already
  if constexpr (NST > 2) {
    if (nsteps > 1) issue(key_lo + KN, Stage{k1, v1});
    if (nsteps > 2) issue(key_lo + 2 * KN, Stage{k2, v2});
  }
  for (int s0 = 0; s0 < nsteps; s0 += NST) {
    run_step(s0, std::integral_constant<int, 0>{});
    if constexpr (NST > 1) if (s0 + 1 < nsteps) run_step(s0 + 1, std::integral_constant<int, 1>{});
    if constexpr (NST > 2) if (s0 + 2 < nsteps) run_step(s0 + 2, std::integral_constant<int, 2>{});
    if constexpr (NST > 3) if (s0 + 3 < nsteps) run_step(s0 + 3, std::integral_constant<int, 3>{});
  }
  }

  stamp(4);

  // ---- epilogue: lane (lr, hh) holds O^T[d][row lr] for d = 32i + 8(j/4) + 4hh + (j%4) ----
  float l_tot = sum_halves(l_run);
  const int wrow0 = row0 + wm * kWaveRows;  // the wave's first query row

  if constexpr (WN > 1) {
    // merge the key slices of each row group through LDS (stage 0 is free now)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // region r (one wave's accumulators) lives in k0, then continues in v0
    auto region = [&](int r) __attribute__((always_inline)) -> float* {
      constexpr int kPerPart = SH::kPartBytes / SH::kRegionBytes;
      return reinterpret_cast<float*>(r < kPerPart ? k0 + r * SH::kRegionBytes : v0 + (r - kPerPart) * SH::kRegionBytes);
    };
    if (wn > 0) {
      const int r = (wn - 1) * WM + wm;
      float* dst = region(r);
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[(i * 16 + j) * 64 + lane] = acc[i][j];
      float* ml = merge_ml + (r * 64 + lane) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    __syncthreads();
    if (wn == 0) {
      for (int w2 = 1; w2 < WN; ++w2) {
        const int r = (w2 - 1) * WM + wm;
        const float* src = region(r);
        const float* ml = merge_ml + (r * 64 + lane) * 2;
        const float m2 = ml[0], l2 = ml[1];
        const float mn = fmaxf(m_run, m2);
        const float a1 = __builtin_amdgcn_exp2f(m_run - mn);
        const float a2 = __builtin_amdgcn_exp2f(m2 - mn);
        m_run = mn;
        l_tot = l_tot * a1 + l2 * a2;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[i][j] = acc[i][j] * a1 + src[(i * 16 + j) * 64 + lane] * a2;
      }
    }
    if (wn != 0 || !row_ok) return;
  } else {
    if (wrow0 >= nrows) return;
  }

  // An unsplit row is final: O / l in bf16. A split row is a partial for the
  // merge: the unnormalised output scaled by a power of two 2^-e so that every
  // |value| < 1, in fp16 (an exact scaling, so the stored values keep 11
  // significant bits relative to the row's largest entry whatever the
  // magnitude of V), with (m, l, 2^e) beside it.
  const bool part = sg.splits > 1;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(acc[i][j]));
  amax = max_halves(amax);
  const int e = min(((int)((__float_as_uint(amax) >> 23) & 255)) - 126, 127);  // amax < 2^e (or e = 127)
  const float mul = part ? __builtin_amdgcn_ldexpf(1.f, -e) : 1.f / l_tot;
  // the four-value groups (d = 32i + 8j4 + 4hh ..) of this lane's row, in the output's 16-bit format
  auto pack = [&](int i, int j4) __attribute__((always_inline)) -> uint2 {
    if (part) {
      _Float16 h4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h4[q] = (_Float16)(acc[i][j4 * 4 + q] * mul);
      return *reinterpret_cast<uint2*>(h4);
    }
    __bf16 b4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b4[q] = (__bf16)(acc[i][j4 * 4 + q] * mul);
    return *reinterpret_cast<uint2*>(b4);
  };
  // first element of a row's output (bf16 O, or the fp16 partial of this split)
  const int64_t part_row0 = (int64_t)sg.part_base + (int64_t)split * sg.n * p.Hq + (int64_t)head * nrows;
  auto row_dst = [&](int row) __attribute__((always_inline)) -> uint16_t* {
    return part ? reinterpret_cast<uint16_t*>(p.part_o) + (part_row0 + row) * D
                : p.out + (int64_t)(sg.node_off + row / g) * p.out_rs + (int64_t)(head * g + row % g) * D;
  };
  if (part && row_ok && hh == 0) {
    const int64_t prow = part_row0 + my_row;
    p.part_ml[prow] = make_float4(m_run, l_tot, __builtin_amdgcn_ldexpf(1.f, e), 0.f);
  }

  if constexpr (WN > 1) {
    // few rows per workgroup: every lane stores its own row, 16 bytes at a time.
    // For each pair of four-value groups (j4, j4 + 1) the half-waves swap one
    // group through v_permlane32_swap, so that lane (lr, 0) holds dims
    // 32i + 8 j4 .. + 7 and lane (lr, 1) dims 32i + 8 (j4 + 1) .. + 7.
    uint16_t* orow = row_dst(my_row);
    typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j4 = 0; j4 < 4; j4 += 2) {
        const uint2 a = pack(i, j4), b = pack(i, j4 + 1);
        const auto sx = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
        *reinterpret_cast<u32x4s*>(orow + i * 32 + j4 * 8 + hh * 8) = u32x4s{sx[0], sy[0], sx[1], sy[1]};
      }
  } else {
    // 256 rows per workgroup, all of them finishing together across the chip:
    // the wave's 32 rows leave through a wave-private LDS buffer (32 rows of
    // 2D bytes, 16-byte chunks XOR-swizzled by row) so that every store
    // instruction writes whole rows -- D/8 adjacent lanes store one row's
    // chunks, 512/D rows per instruction, and the rows of one node's query
    // heads are adjacent in memory -- instead of 16-byte pieces of 32 rows.
    // The buffer is a stage that no wave reads any more: not the last one
    // (the other group may still be reading it); the group of waves 0-3
    // takes the stage after it, the other group the stage after that, each
    // wave a quarter of that stage.
    static_assert(NST == 4, "one key slice only in the ping-pong schedule");
    const int st = (max(nsteps - 1, 0) + 1 + (wave >> 2)) & 3;
    const int wq = wave & 3;
    char* ob = ((wq < 2) ? (st == 0 ? k0 : st == 1 ? k1 : st == 2 ? k2 : k3)
                         : (st == 0 ? v0 : st == 1 ? v1 : st == 2 ? v2 : v3)) +
               (wq & 1) * (kWaveRows * D * 2);
    constexpr int kCh = D / 8;               // 16-byte chunks per row
    constexpr int kRowsPerStore = 64 / kCh;  // rows one store instruction covers
    auto swz = [](int r) __attribute__((always_inline)) { return (D == 128 ? r : (r >> 1)) & (kCh - 1); };
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *reinterpret_cast<uint2*>(ob + lr * (2 * D) + (((i * 4 + j4) ^ swz(lr)) << 4) + hh * 8) = pack(i, j4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's buffer writes are complete
    const int sr = lane / kCh, sc16 = lane % kCh;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kStores = kWaveRows / kRowsPerStore;
    u32x4 v[kStores];  // all reads in flight together, then the stores
#pragma unroll
    for (int k = 0; k < kStores; ++k) {
      const int r = k * kRowsPerStore + sr;
      v[k] = *reinterpret_cast<const u32x4*>(ob + r * (2 * D) + ((sc16 ^ swz(r)) << 4));
    }
#pragma unroll
    for (int k = 0; k < kStores; ++k) {
      const int row = wrow0 + k * kRowsPerStore + sr;
      if (row < nrows) *reinterpret_cast<u32x4*>(row_dst(row) + sc16 * 8) = v[k];
    }
  }
  stamp(5);
}

// Merge the per-chunk partials of split sequences. A thread owns eight
// consecutive dims of one (node, query head) row (one 16-byte load per chunk),
// so the threads of a row read each chunk's partial as one contiguous line.
// One partial row per (row, eight-dim slice) thread, or, with G > 1, G threads
// per (row, slice) that take every G-th chunk and merge their running (m, l, O)
// through cross-lane shuffles at the end (for many chunks and few rows, so that
// more threads carry the loads). The G * D/8 threads of a row are adjacent lanes
// of one wave. Rows go in the partials' order, (KV head, node, query head within
// the group), so a block's rows are contiguous in every chunk, and contiguous
// ranges of blocks go to one XCD, as the forward kernel's work items do.
template <int D, int G, bool STAMPS>
__global__ __launch_bounds__(256) void tree_attn_combine(const AttnParams p) {
  // phase stamps (the STAMPS instantiation only): entry (slot 0) and output
  // stored (slot 5) of lane 0 of the block
  auto stamp = [&](int k) __attribute__((always_inline)) {
    if constexpr (STAMPS) {
      const int row = p.stamp_cb0 + (int)blockIdx.x;
      if (threadIdx.x == 0 && row < p.stamp_rows) {
        p.stamps[(int64_t)row * kStampSlots + k] = __builtin_amdgcn_s_memrealtime();
        if (k == 0) p.stamps[(int64_t)row * kStampSlots + 7] = 2;
      }
    }
  };
  stamp(0);
  constexpr int kTpr = D / 8;          // threads per row and chunk group
  constexpr int kRpb = 256 / (kTpr * G);  // rows per block
  const int nbx = gridDim.x / kXcds;
  const int cb = (blockIdx.x % kXcds) * nbx + blockIdx.x / kXcds;
  const int row = cb * kRpb + threadIdx.x / (kTpr * G);
  const int gi = (threadIdx.x / kTpr) % G;
  const int c8 = threadIdx.x % kTpr;
  if (row >= p.comb_rows) return;  // the row's G * kTpr lanes leave together
  int s = -1;
  for (int i = 0; i < p.nseq; ++i)
    if (p.seq[i].splits > 1 && p.seq[i].comb_start <= row) s = i;
  if (s < 0) return;
  const SeqGeom& sg = p.seq[s];
  const int r = row - sg.comb_start;  // = (KV head * n + node) * g + j, for query head KV head * g + j
  if (r >= sg.n * p.Hq) return;
  const int ng = sg.n * p.g;
  const int hkv = r / ng, rem = r - hkv * ng;
  const int node = rem / p.g, qh = hkv * p.g + rem % p.g;
  // partial row of chunk k: part_base + k * n * Hq + r (the order the forward kernel writes them in)
  const int64_t prow0 = (int64_t)sg.part_base + r;
  const int64_t kstride = (int64_t)sg.n * p.Hq;
  const uint4* po = reinterpret_cast<const uint4*>(p.part_o);  // eight fp16 values per thread
  // Chunks gi, gi + G, ... are merged eight at a time (their loads in flight
  // together): the batch's maximum first, then every chunk with one weight.
  constexpr int kBatch = 8;
  float m = -INFINITY, l = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = gi; k0 < sg.splits; k0 += G * kBatch) {
    float4 ml[kBatch];
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = min(k0 + u * G, sg.splits - 1);
      const int64_t prow = prow0 + k * kstride;
      ml[u] = p.part_ml[prow];
      v[u] = po[prow * kTpr + c8];
    }
    // a chunk that saw no visible key for this row (l = 0) contributes nothing
    bool ok[kBatch];
    float mb = m;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      ok[u] = k0 + u * G < sg.splits && ml[u].y > 0.f;
      if (ok[u]) mb = fmaxf(mb, ml[u].x);
    }
    if (mb == -INFINITY) continue;  // nothing visible yet
    const float a = __builtin_amdgcn_exp2f(m - mb);  // 0 on the first visible batch
    l *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= a;
    m = mb;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!ok[u]) continue;
      const float w = __builtin_amdgcn_exp2f(ml[u].x - m);
      const float ws = w * ml[u].z;  // undoes the stored 2^-e
      const _Float16* h = reinterpret_cast<const _Float16*>(&v[u]);
      l += w * ml[u].y;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += ws * (float)h[e];
    }
  }
  if constexpr (G > 1) {
#pragma unroll
    for (int off = kTpr; off < kTpr * G; off <<= 1) {
      const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[e], off);
      const float mn = fmaxf(m, m2);
      if (mn == -INFINITY) continue;  // neither side has seen a visible key
      const float a1 = __builtin_amdgcn_exp2f(m - mn), a2 = __builtin_amdgcn_exp2f(m2 - mn);
      l = l * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = o[e] * a1 + o2[e] * a2;
      m = mn;
    }
    if (gi != 0) return;
  }
  const float inv = 1.f / l;
  __bf16 o8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o8[e] = (__bf16)(o[e] * inv);
  bf16_bits* orow = p.out + (int64_t)(sg.node_off + node) * p.out_rs + (int64_t)qh * D + c8 * 8;
  *reinterpret_cast<uint4*>(orow) = *reinterpret_cast<uint4*>(o8);
  stamp(5);
}

// ---------------------------------------------------------------- host side

// The call-wide choices; each launch (a group of at most kMaxSeqs sequences)
// is derived from them when it is enqueued, so planning touches no heap.
struct Plan {
  int wm = 8;            // row groups per workgroup (64, 128 or 256 rows)
  int64_t chunk = 0;     // keys per split
  size_t part_rows = 0;  // split-partial rows over the whole call
  size_t ws_bytes = 0;
};

struct Launch {
  AttnParams a;
  int grid = 0;         // workgroups
  int comb_grid = 0;    // combine blocks (0 = none)
  int comb_groups = 1;  // chunk groups per combine row (1 or 4)
  size_t lds = 0;       // dynamic LDS bytes
};

int check_desc(const dt_attn_desc* d) {
  if (!d) return DT_ERR_NULL;
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return DT_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads) return DT_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return DT_ERR_UNSUPPORTED;
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale)) return DT_ERR_SHAPE;
  if (d->phase_stamp_rows < 0 || (d->phase_stamps && !aligned(d->phase_stamps, 8))) return DT_ERR_SHAPE;
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
  // per-lane offsets within one load instruction's rows are 32-bit
  if (d->prefix_row_stride >= ((int64_t)1 << 24)) return DT_ERR_UNSUPPORTED;
  return DT_OK;
}

template <int D, int WM>
size_t static_lds() {
  using SH = Shape<D, WM>;
  return (size_t)SH::kStageBytes * SH::NST + 1024 * (4 - SH::NST);
}

size_t static_lds_for(int D, int wm) {
  if (D == 128) return wm == 8 ? static_lds<128, 8>() : wm == 4 ? static_lds<128, 4>() : static_lds<128, 2>();
  return wm == 8 ? static_lds<64, 8>() : wm == 4 ? static_lds<64, 4>() : static_lds<64, 2>();
}

// Dynamic LDS of one launch: parents, ancestor masks and the key-slice merge statistics.
size_t dynamic_lds(int max_n, int g, int wm) {
  const int rm = kWaveRows * wm;
  const size_t mask_rows = (size_t)((rm - 1) / g + 2);
  const size_t mask_words = (size_t)((max_n + 31) / 32 + 2);
  const size_t merge = (size_t)(kWaves / wm - 1) * wm * 64 * 2;
  return sizeof(uint32_t) * ((size_t)max_n + mask_rows * mask_words + merge);
}

// Workgroup shape: WM row groups of 32 rows, WM in {2, 4, 8}. A workgroup
// needs enough rows for every wave to do useful work; with fewer rows the
// eight waves split the keys of each step instead.
int choose_wm(const dt_attn_desc* d, int g) {
  int max_rows = 0;
  int64_t max_keys = 0;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int n = d->node_offsets[s + 1] - d->node_offsets[s];
    max_rows = std::max(max_rows, n * g);
    max_keys = std::max<int64_t>(max_keys, (int64_t)d->prefix_lens[s] + n);
  }
  // At most 64 rows over a long prefix the call streams K/V from HBM: 128-row
  // tiles (half the row groups idle) keep two 64 KB stages in flight where the
  // 64 x 256 shape has room for one 128 KB stage only.
  if (max_rows <= 64) return max_keys > 16 * kBN ? 4 : 2;
  if (max_rows <= 128) return 4;
  return 8;
}

// Keys per split for a given workgroup shape. Every work item streams at
// most `chunk` keys; `chunk` is uniform, so items cost about the same and the
// per-XCD item ranges balance. It is sized so that the items fill the CUs (one
// workgroup each) about once.
int64_t choose_chunk(const dt_attn_desc* d, int g, int rm, int cus) {
  if (d->split_keys) return d->split_keys;
  int64_t total_tiles = 0, max_keys = 0;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int n = d->node_offsets[s + 1] - d->node_offsets[s];
    const int64_t keys = (int64_t)d->prefix_lens[s] + n;
    const int64_t units = ceil_div((int64_t)n * g, rm) * d->num_kv_heads;
    total_tiles += units * ceil_div(keys, kBN);
    max_keys = std::max(max_keys, keys);
  }
  const int64_t tiles = std::max<int64_t>(1, ceil_div(total_tiles, cus));
  return std::min(tiles * kBN, ceil_div(max_keys, kBN) * kBN);
}

// Sequences whose key counts differ widely (a ragged batch: the longest has
// more than 1.5 times the keys of the shortest) make units of unequal length:
// sized for one workgroup per CU, the chunks would leave the CUs that drew
// short units idle while long ones finish. There the chunks are sized for
// about three workgroups per CU (at least 16 tiles), which the dispatcher
// balances as workgroups finish. Nearly equal lengths keep the one-wave plan.
bool ragged_keys(const dt_attn_desc* d) {
  int64_t lo = INT64_MAX, hi = 0;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int64_t keys = (int64_t)d->prefix_lens[s] + (d->node_offsets[s + 1] - d->node_offsets[s]);
    lo = std::min(lo, keys);
    hi = std::max(hi, keys);
  }
  return 2 * hi > 3 * lo;
}

int64_t choose_chunk_ragged(const dt_attn_desc* d, int g, int rm, int cus) {
  int64_t total_tiles = 0, max_keys = 0;
  for (int s = 0; s < d->num_seqs; ++s) {
    const int n = d->node_offsets[s + 1] - d->node_offsets[s];
    const int64_t keys = (int64_t)d->prefix_lens[s] + n;
    total_tiles += ceil_div((int64_t)n * g, rm) * d->num_kv_heads * ceil_div(keys, kBN);
    max_keys = std::max(max_keys, keys);
  }
  const int64_t tiles = std::max<int64_t>(16, ceil_div(total_tiles, 3 * (int64_t)cus));
  return std::min(tiles * kBN, ceil_div(max_keys, kBN) * kBN);
}

bool needs_split(const dt_attn_desc* d, int64_t chunk) {
  for (int s = 0; s < d->num_seqs; ++s)
    if ((int64_t)d->prefix_lens[s] + (d->node_offsets[s + 1] - d->node_offsets[s]) > chunk) return true;
  return false;
}

bool lds_fits(int D, int wm, int max_n, int g) {
  return static_lds_for(D, wm) + dynamic_lds(max_n, g, wm) <= (size_t)kLdsBytes;
}

// The launch of sequences [s0, s0 + kMaxSeqs) under a call-wide plan (wm and
// chunk chosen). *part_rows carries the split-partial rows of the earlier
// launches in and this launch's end out.
void plan_launch(const dt_attn_desc* d, const Plan& plan, int s0, size_t* part_rows, Launch* L) {
  const int g = d->num_q_heads / d->num_kv_heads;
  const int rm = kWaveRows * plan.wm;
  AttnParams& a = L->a;
  std::memset(&a, 0, sizeof(a));
  a.nseq = std::min(kMaxSeqs, d->num_seqs - s0);
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.g = g;
  a.chunk = (int32_t)plan.chunk;
  a.scale_log2 = d->softmax_scale * kLog2e;
  int items = 0, comb = 0, launch_max_n = 1, max_splits = 1;
  for (int i = 0; i < a.nseq; ++i) {
    const int s = s0 + i;
    SeqGeom& sg = a.seq[i];
    sg.node_off = d->node_offsets[s];
    sg.n = d->node_offsets[s + 1] - d->node_offsets[s];
    sg.P = d->prefix_lens[s];
    sg.prefix_row0 = d->prefix_row_start[s];
    sg.row_tiles = (int32_t)ceil_div((int64_t)sg.n * g, rm);
    sg.splits = (int32_t)std::max<int64_t>(1, ceil_div((int64_t)sg.P + sg.n, plan.chunk));
    sg.item_start = items;
    items += sg.row_tiles * sg.splits * d->num_kv_heads;
    if (sg.splits > 1) {
      sg.part_base = (int32_t)*part_rows;
      *part_rows += (size_t)sg.splits * sg.n * d->num_q_heads;
      sg.comb_start = comb;
      comb += sg.n * d->num_q_heads;
    } else {
      sg.part_base = -1;
      sg.comb_start = -1;
    }
    launch_max_n = std::max(launch_max_n, sg.n);
    max_splits = std::max(max_splits, sg.splits);
  }
  a.total_items = items;
  a.per_xcd = (int32_t)ceil_div(items, kXcds);
  a.max_n = launch_max_n;
  a.mask_words = (launch_max_n + 31) / 32 + 2;
  a.mask_rows = (rm - 1) / g + 2;
  a.comb_rows = comb;
  L->grid = a.per_xcd * kXcds;
  // many chunks per row: four threads share each (row, slice), more threads carry the loads
  L->comb_groups = max_splits > 8 ? 4 : 1;
  L->comb_grid = comb ? (int)ceil_div(ceil_div(comb, 256 / (d->head_dim / 8 * L->comb_groups)), kXcds) * kXcds : 0;
  L->lds = dynamic_lds(launch_max_n, g, plan.wm);
}

int make_plan(const dt_attn_desc* d, Plan* plan) {
  int st = check_desc(d);
  if (st != DT_OK) return st;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != DT_OK) return st;
  const int g = d->num_q_heads / d->num_kv_heads;
  const int D = d->head_dim;
  int max_n = 1;
  for (int s = 0; s < d->num_seqs; ++s) max_n = std::max(max_n, d->node_offsets[s + 1] - d->node_offsets[s]);

  // 256 rows per workgroup (the ping-pong schedule) unless, in a batch of
  // (nearly) equal lengths, 128 rows avoid splitting the keys where 256 would
  // need it; fewer rows when the trees are small or the ancestor masks do not
  // fit the LDS. A ragged batch keeps 256-row tiles and balances through
  // smaller key chunks.
  int wm = choose_wm(d, g);
  const bool ragged = !d->split_keys && ragged_keys(d);
  // 128-row tiles instead of 256-row ones when that avoids the key split, or
  // when the split would leave each workgroup at most eight steps: there the
  // split partials' round trip (written by every chunk, read back by the
  // merge) costs more than the shorter tiles, and 128-row tiles halve it.
  if (wm == 8 && !d->split_keys && !ragged && lds_fits(D, 4, max_n, g)) {
    const int64_t chunk8 = choose_chunk(d, g, kWaveRows * 8, cus);
    if (needs_split(d, chunk8) &&
        (!needs_split(d, choose_chunk(d, g, kWaveRows * 4, cus)) || chunk8 <= 8 * kBN))
      wm = 4;
  }
  while (!lds_fits(D, wm, max_n, g) && wm > 2) wm /= 2;
  if (!lds_fits(D, wm, max_n, g)) return DT_ERR_UNSUPPORTED;
  plan->wm = wm;
  const int rm = kWaveRows * wm;
  int64_t chunk = ragged && wm == 8 ? choose_chunk_ragged(d, g, rm, cus) : choose_chunk(d, g, rm, cus);
  if (chunk > (int64_t)1 << 30) chunk = (int64_t)1 << 30;
  plan->chunk = chunk;

  size_t part_rows = 0;
  Launch L;
  for (int s0 = 0; s0 < d->num_seqs; s0 += kMaxSeqs) {
    plan_launch(d, *plan, s0, &part_rows, &L);
    if (part_rows > (size_t)INT32_MAX) return DT_ERR_UNSUPPORTED;
  }
  plan->part_rows = part_rows;
  plan->ws_bytes = part_rows ? round_up(part_rows * (size_t)d->head_dim * sizeof(_Float16), 256) +
                                   round_up(part_rows * sizeof(float4), 256)
                             : 0;
  return DT_OK;
}

template <int D, bool STAMPS>
void launch_fwd_as(int wm, int grid, size_t lds, hipStream_t st, const AttnParams& a) {
  if (wm == 8)
    hipLaunchKernelGGL((tree_attn_fwd<D, 8, STAMPS>), dim3(grid), dim3(kThreads), lds, st, a);
  else if (wm == 4)
    hipLaunchKernelGGL((tree_attn_fwd<D, 4, STAMPS>), dim3(grid), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((tree_attn_fwd<D, 2, STAMPS>), dim3(grid), dim3(kThreads), lds, st, a);
}

template <int D, bool STAMPS>
void launch_kernels(const Launch& L, int wm, hipStream_t st) {
  launch_fwd_as<D, STAMPS>(wm, L.grid, L.lds, st, L.a);
  if (L.comb_grid) {
    if (L.comb_groups > 1)
      hipLaunchKernelGGL((tree_attn_combine<D, 4, STAMPS>), dim3(L.comb_grid), dim3(256), 0, st, L.a);
    else
      hipLaunchKernelGGL((tree_attn_combine<D, 1, STAMPS>), dim3(L.comb_grid), dim3(256), 0, st, L.a);
  }
}

// One launch's kernels: the forward kernel, then the merge of split rows.
template <int D>
void launch_call(const Launch& L, int wm, hipStream_t st) {
  if (L.a.stamps)
    launch_kernels<D, true>(L, wm, st);
  else
    launch_kernels<D, false>(L, wm, st);
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

namespace dt {
namespace {

// Enqueue a planned call (arguments checked by the caller).
int run_attention(const dt_attn_desc* desc, const Plan& plan, const void* q, const void* k_tree, const void* v_tree,
                  const void* k_prefix, const void* v_prefix, const int32_t* parent, void* out, void* workspace,
                  void* stream) {
  const int64_t D = desc->head_dim;
  const int64_t qrs = desc->q_row_stride ? desc->q_row_stride : desc->num_q_heads * D;
  const int64_t ors = desc->out_row_stride ? desc->out_row_stride : desc->num_q_heads * D;
  const int64_t trs = desc->tree_row_stride ? desc->tree_row_stride : desc->num_kv_heads * D;
  _Float16* part_o = static_cast<_Float16*>(workspace);
  float4* part_ml = plan.ws_bytes
                        ? reinterpret_cast<float4*>(static_cast<char*>(workspace) +
                                                    round_up(plan.part_rows * D * sizeof(_Float16), 256))
                        : nullptr;

  hipStream_t st_ = static_cast<hipStream_t>(stream);
  size_t part_rows = 0;
  int32_t stamp_wg0 = 0;
  Launch L;
  for (int s0 = 0; s0 < desc->num_seqs; s0 += kMaxSeqs) {
    plan_launch(desc, plan, s0, &part_rows, &L);
    AttnParams& a = L.a;
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
    a.stamps = desc->phase_stamps;
    a.stamp_rows = (int32_t)std::min<int64_t>(desc->phase_stamp_rows, INT32_MAX);
    if (a.total_items == 0) continue;
    a.stamp_wg0 = stamp_wg0;
    a.stamp_cb0 = stamp_wg0 + L.grid;
    stamp_wg0 += L.grid + L.comb_grid;
    if (D == 128)
      launch_call<128>(L, plan.wm, st_);
    else
      launch_call<64>(L, plan.wm, st_);
    const int st = launch_status();
    if (st != DT_OK) return st;
  }
  return DT_OK;
}

// Checks of the buffers shared by both entry points.
int check_buffers(const dt_attn_desc* desc, const void* q, const void* k_tree, const void* v_tree,
                  const void* k_prefix, const void* v_prefix, const int32_t* parent, const void* out) {
  if (!q || !k_tree || !v_tree || !parent || !out) return DT_ERR_NULL;
  bool any_prefix = false;
  for (int s = 0; s < desc->num_seqs; ++s) any_prefix |= desc->prefix_lens[s] > 0;
  if (any_prefix && (!k_prefix || !v_prefix)) return DT_ERR_NULL;
  for (const void* ptr : {q, k_tree, v_tree, out})
    if (!aligned(ptr, 16)) return DT_ERR_SHAPE;
  if (any_prefix && (!aligned(k_prefix, 16) || !aligned(v_prefix, 16))) return DT_ERR_SHAPE;
  if (!aligned(parent, 4)) return DT_ERR_SHAPE;
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_tree_attention(const dt_attn_desc* desc, const void* q, const void* k_tree, const void* v_tree,
                                 const void* k_prefix, const void* v_prefix, const int32_t* parent, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dt;
  if (!q || !k_tree || !v_tree || !parent || !out) return DT_ERR_NULL;
  Plan plan;
  int st = make_plan(desc, &plan);
  if (st != DT_OK) return st;
  st = check_buffers(desc, q, k_tree, v_tree, k_prefix, v_prefix, parent, out);
  if (st != DT_OK) return st;
  if (plan.ws_bytes) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return DT_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DT_ERR_WORKSPACE;
  }
  return run_attention(desc, plan, q, k_tree, v_tree, k_prefix, v_prefix, parent, out, workspace, stream);
}

// ---------------------------------------------------------------- no-allocation entry point
//
// dt_tree_attention_noalloc keeps the split partials in this array instead of
// a caller workspace. Its host-side name is not a device address: the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is ever passed to
// kernels. The kernels write every partial before reading it, so the array
// needs no clearing between calls; calls that overlap on one GPU (other
// streams, other threads) share it and race.
static __device__ __align__(256) unsigned char scratch[DT_NOALLOC_SCRATCH_BYTES];

namespace dt {
namespace {

constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];

int scratch_address(void** ptr) {
  int dev = 0;
  DT_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kScratchDevices) return DT_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return DT_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return DT_OK;
}

// The default plan, or, when its partials exceed the scratch array, the same
// call with key chunks doubled until they fit (fewer splits; none at all at
// worst). A caller-forced chunk is kept, and one too large is an error.
int plan_within_scratch(const dt_attn_desc* desc, Plan* plan) {
  int st = make_plan(desc, plan);
  if (st != DT_OK) return st;
  if (plan->ws_bytes <= (size_t)DT_NOALLOC_SCRATCH_BYTES) return DT_OK;
  if (desc->split_keys) return DT_ERR_WORKSPACE;
  dt_attn_desc d2 = *desc;
  int64_t chunk = plan->chunk;
  while (plan->ws_bytes > (size_t)DT_NOALLOC_SCRATCH_BYTES) {
    chunk *= 2;
    if (chunk > ((int64_t)1 << 30)) return DT_ERR_WORKSPACE;
    d2.split_keys = (int32_t)chunk;
    *plan = Plan();
    st = make_plan(&d2, plan);
    if (st != DT_OK) return st;
  }
  return DT_OK;
}

}  // namespace
}  // namespace dt

extern "C" int dt_tree_attention_noalloc(const dt_attn_desc* desc, const void* q, const void* k_tree,
                                         const void* v_tree, const void* k_prefix, const void* v_prefix,
                                         const int32_t* parent, void* out, void* stream) {
  using namespace dt;
  if (!q || !k_tree || !v_tree || !parent || !out) return DT_ERR_NULL;
  Plan plan;
  int st = plan_within_scratch(desc, &plan);
  if (st != DT_OK) return st;
  st = check_buffers(desc, q, k_tree, v_tree, k_prefix, v_prefix, parent, out);
  if (st != DT_OK) return st;
  void* ws = nullptr;
  if (plan.ws_bytes) {
    st = scratch_address(&ws);
    if (st != DT_OK) return st;
  }
  return run_attention(desc, plan, q, k_tree, v_tree, k_prefix, v_prefix, parent, out, ws, stream);
}
