/*
 * dtree.h -- C ABI of libdtree: verifying a draft tree in one target forward
 * on AMD Instinct MI355X (gfx950).
 *
 * Speculative decoding with draft trees (DARTree: "Speculative Diffusion
 * Decoding with Autoregressive Draft Trees", Preliminaries > Tree Verification
 * and DDTree; DDTree: "Accelerating Speculative Decoding with Block Diffusion
 * Draft Trees", abstract) verifies a whole prefix tree of draft tokens in a
 * single target forward: the tree's nodes are flattened, each node attends to
 * the verified context plus the nodes on its own root-to-node path (an
 * ancestor-only mask), the target's greedy prediction is taken at every node,
 * and the longest root-to-leaf path whose tokens match those predictions is
 * accepted, followed by one bonus token.
 *
 * This library provides that path:
 *   dt_build_tree       host: best-first (DDTree) tree construction
 *   dt_tree_attention   GPU:  ancestor-only tree attention over a KV-cached prefix
 *   dt_tree_attention_noalloc  the same without a workspace (a static device buffer)
 *   dt_argmax_rows      GPU:  per-node greedy prediction (row arg-max)
 *   dt_sample_rows      GPU:  per-node target sample at temperature T > 0 (Gumbel-max)
 *   dt_accept_path      GPU:  longest accepted path and bonus token
 *   dt_commit_kv        GPU:  accepted path's K/V into the KV cache, all layers
 *   dt_topk_rows        GPU:  per-depth top-K draft candidates with log-softmax values
 *   dt_expand_depth     GPU:  one depth of DARTree's fixed-width supertree
 *   dt_prune_topb       GPU:  deferred top-B pruning into the verification tree
 *
 * Conventions shared by every entry point
 *  - Every function returns an int status: DT_OK (0) or a negative DT_ERR_*.
 *    Nothing throws across this boundary, aborts or prints.
 *  - Ownership: the caller owns every buffer, host and device. The library
 *    allocates no device memory (scratch comes from a caller-provided
 *    workspace), uses host memory only for temporaries freed before the call
 *    returns, and keeps no pointer after a call returns. The one exception is
 *    dt_tree_attention_noalloc, whose scratch is a static device buffer of
 *    fixed size that the library holds per GPU (see there).
 *  - Device work is enqueued on the caller's HIP stream, passed as `void*`
 *    (a hipStream_t; NULL means the default stream). Outputs are valid once
 *    the stream reaches that point. No call synchronises the stream.
 *  - Arguments are validated before anything is enqueued; an invalid call
 *    leaves every output untouched. Device data that cannot be read on the
 *    host (device parent/token arrays, logits) is the caller's contract, as
 *    stated per call; a violated device-side contract gives unspecified
 *    results but never an out-of-bounds access.
 *  - DT_ERR_HIP reports a failed HIP runtime call (e.g. a launch error); an
 *    asynchronous device fault surfaces at the caller's next synchronisation.
 *  - The library keeps no mutable global state (device properties are cached
 *    once per device), so calls from several host threads are safe, except
 *    overlapping dt_tree_attention_noalloc calls on one GPU (they share its
 *    static buffer).
 *
 * Tree representation (all calls): a tree of n nodes is an int32 array
 * parent[n] with parent[0] == -1 (node 0 is the root: the last committed
 * token, whose logits predict draft position 1) and 0 <= parent[i] < i for
 * i > 0, i.e. nodes are numbered in a topological order. Several trees are
 * packed back to back; node_offsets[s] .. node_offsets[s+1]-1 are the rows
 * of tree s and its parent entries are local to the tree.
 */
#ifndef DTREE_H
#define DTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dt_status {
  DT_OK = 0,
  DT_ERR_NULL = -1,        /* a required pointer is NULL */
  DT_ERR_SHAPE = -2,       /* a count, size, stride or offset is out of range or misaligned */
  DT_ERR_TREE = -3,        /* a (host) parent array is not a topologically numbered tree */
  DT_ERR_VALUE = -4,       /* candidate table: unsorted row, non-finite or positive log-prob, repeated token */
  DT_ERR_UNSUPPORTED = -5, /* a valid request the library does not implement (e.g. head_dim not 64/128) */
  DT_ERR_WORKSPACE = -6,   /* workspace NULL, too small or not 256-byte aligned */
  DT_ERR_HIP = -7,         /* a HIP runtime call failed */
  DT_ERR_NOMEM = -8        /* temporary host memory could not be obtained (dt_build_tree) */
};

/* Largest tree (nodes per sequence, root included) dt_tree_attention accepts. */
#define DT_MAX_TREE_NODES 1024

/* Static, NUL-terminated description of a status code (never NULL). */
const char* dt_status_string(int status);

/* ABI version of this header: (major << 16) | minor; 2.0 (dt_attn_desc gained phase_stamps). */
int dt_abi_version(void);

/*
 * dt_build_tree -- DDTree best-first construction of a draft tree (host).
 *
 * Defined by: DARTree paper, Figure 3 caption (a max-heap over frontier
 * prefixes: each pop takes the prefix of highest mass, which becomes a node,
 * and pushes its next sibling and its first, highest-probability child); the
 * objective it maximises is eq. 4 with the mass decomposition that follows it
 * (Tree Verification and DDTree): the sum over tree prefixes of the product
 * of their per-position draft probabilities. Lemma 1 (Deferred Best-First
 * Pruning, eq. 6) shows the result equals global top-B selection when every
 * step adds a non-positive log-probability and ancestors win ties.
 *
 * Inputs (host):
 *   depths       number of draft positions (the drafting block, e.g. 16); 1..64
 *   k            candidates per position; 1..65535
 *   cand_logprob [depths][k] row-major float: log-probability of the r-th
 *                candidate at each position. Every entry finite and <= 0;
 *                each row non-increasing (ties in any token order).
 *   cand_token   [depths][k] row-major int32 token ids, >= 0, distinct within a row.
 *   root_token   token of the root (the last committed token), >= 0.
 *   n_nodes      node budget counting the root (>= 1): the tree gets the root
 *                plus up to n_nodes - 1 draft prefixes.
 * Outputs (host, caller-allocated, n_nodes entries each; entries past n_out
 * are left untouched):
 *   parent       parent[0] = -1; parent[i] < i (pop order is topological)
 *   token        token[0] = root_token; token[i] = the candidate's token id
 *   depth        depth[0] = 0; depth[i] = draft position of node i (1-based)
 *   score        nullable; log-mass of each node (sum of its candidates'
 *                log-probs added root-first in double; score[0] = 0)
 *   n_out        number of nodes written: n_nodes, or fewer if the table has
 *                fewer prefixes.
 * Order: nodes are emitted in pop order, i.e. by (score descending, depth
 * ascending, rank tuple ascending lexicographically), which every parent
 * precedes its children in.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE (sizes), DT_ERR_VALUE (table contract).
 */
int dt_build_tree(int32_t depths, int32_t k, const float* cand_logprob, const int32_t* cand_token,
                  int32_t root_token, int32_t n_nodes, int32_t* parent, int32_t* token, int32_t* depth,
                  double* score, int32_t* n_out);

/*
 * dt_validate_tree -- check a host parent array against the tree
 * representation above. Returns DT_OK, DT_ERR_NULL (parent NULL with n > 0),
 * DT_ERR_SHAPE (n < 1) or DT_ERR_TREE.
 */
int dt_validate_tree(const int32_t* parent, int32_t n);

/*
 * Description of one tree-attention call. Counts and strides in elements.
 *
 * Sequences: S trees, tree s has n_s = node_offsets[s+1] - node_offsets[s]
 * nodes (1..DT_MAX_TREE_NODES) and a verified prefix of P_s = prefix_lens[s]
 * tokens (>= 0) already in the KV cache at rows
 * prefix_row_start[s] .. prefix_row_start[s] + P_s - 1 of k_prefix/v_prefix.
 * The host arrays are read during the call only (they fix the launch
 * geometry and are passed to the kernels by value).
 */
typedef struct dt_attn_desc {
  int32_t num_seqs;              /* S >= 1 */
  int32_t num_q_heads;           /* Hq >= 1 */
  int32_t num_kv_heads;          /* Hkv >= 1, Hq % Hkv == 0; query head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;              /* d: 64 or 128 */
  float softmax_scale;           /* > 0 and finite; conventionally 1 / sqrt(d) */
  int32_t split_keys;            /* 0: automatic. > 0: process each sequence's keys in chunks of
                                    this many keys (a multiple of 64) and merge; for testing/tuning */
  const int32_t* node_offsets;   /* host [S+1]; node_offsets[0] = 0, increasing */
  const int32_t* prefix_lens;    /* host [S] */
  const int64_t* prefix_row_start; /* host [S] */
  int64_t q_row_stride;          /* elements between consecutive nodes in q; 0 means Hq*d */
  int64_t out_row_stride;        /* ... in out; 0 means Hq*d */
  int64_t tree_row_stride;       /* ... in k_tree and v_tree; 0 means Hkv*d */
  int64_t prefix_row_stride;     /* elements between consecutive cache rows of k_prefix/v_prefix */
  int64_t prefix_head_stride;    /* elements between consecutive KV heads within a cache row */
  uint64_t* phase_stamps;        /* optional, for profiling (NULL: nothing is recorded): device
                                    buffer, 8-byte aligned, of phase_stamp_rows rows of 8 uint64.
                                    Row w belongs to the call's w-th workgroup, counting, launch
                                    by launch, the forward kernel's workgroups and then the merge
                                    kernel's (split rows only). Lane 0 of a workgroup writes the
                                    GPU's 100 MHz real-time counter into its row's slots: forward
                                    kernel 0 entry, 1 first K/V stage requested, 2 set-up done (Q in
                                    registers, ancestor masks built), 3 first stage landed, 4 main
                                    loop done, 5 outputs stored; merge kernel 0 entry, 5 outputs
                                    stored; and slot 7 = 1 (forward) or 2 (merge) at entry. Other
                                    slots, and those of phases a workgroup does not reach, are left
                                    as they were; rows from phase_stamp_rows on are not written.
                                    Recording uses separate kernel builds: with NULL the call runs
                                    the same kernels as without this field. */
  int64_t phase_stamp_rows;      /* rows of phase_stamps (>= 0) */
} dt_attn_desc;

/*
 * dt_tree_attention_workspace_size -- bytes of device workspace that
 * dt_tree_attention needs for this description on the current device (0 when
 * no sequence is split). Errors as dt_tree_attention's host checks.
 */
int dt_tree_attention_workspace_size(const dt_attn_desc* desc, size_t* bytes);

/*
 * dt_tree_attention -- ancestor-only tree attention (GPU).
 *
 * Defined by: DARTree paper, Preliminaries > Tree Verification and DDTree
 * (flattened nodes; each node attends only to the verified context and the
 * tokens on its root-to-node path, so one target forward scores every
 * branch); DDTree abstract (ancestor-only attention mask). For tree s, node i
 * and query head h, with g = Hq / Hkv and kv = h / g:
 *   keys    = prefix rows 0..P_s-1, then tree nodes j of tree s with j on the
 *             path root..i (i included); every other tree node is invisible
 *   out[i,h] = sum_j softmax_j(scale * <q[i,h], k_j>) * v_j
 * The mask is derived in-kernel from `parent`; no dense mask is formed.
 * Q and K are expected post-rotary (the caller places node i at position
 * P_s + depth(i)).
 *
 * Device buffers (bf16 = IEEE bfloat16, 16-byte aligned; strides multiples of 8):
 *   q        [N][Hq][d] with row stride q_row_stride; N = node_offsets[S]
 *   k_tree   [N][Hkv][d], v_tree likewise, row stride tree_row_stride
 *   k_prefix row r, head h at k_prefix + r*prefix_row_stride + h*prefix_head_stride
 *            (d contiguous elements); v_prefix likewise with the same strides
 *   parent   int32 [N], tree-local parents (contract: the tree representation
 *            above; violating it gives unspecified values, never a fault)
 *   out      [N][Hq][d] bf16, row stride out_row_stride; must not alias inputs
 *   workspace  device scratch of at least dt_tree_attention_workspace_size
 *            bytes, 256-byte aligned (may be NULL when that size is 0). The
 *            library neither needs it zeroed nor preserves its contents.
 * Arithmetic: bf16 operands, fp32 scores/softmax/accumulation, probabilities
 * rounded to bf16 (nearest-even) for the value product, output rounded to bf16.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_UNSUPPORTED, DT_ERR_WORKSPACE, DT_ERR_HIP.
 */
int dt_tree_attention(const dt_attn_desc* desc, const void* q, const void* k_tree, const void* v_tree,
                      const void* k_prefix, const void* v_prefix, const int32_t* parent, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device buffer behind dt_tree_attention_noalloc (per GPU). */
#define DT_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * dt_tree_attention_noalloc -- dt_tree_attention for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same operation, arguments and errors as
 * dt_tree_attention, without a workspace: the split partials live in a static
 * device buffer of DT_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on
 * every GPU it runs on until the process ends. The call allocates nothing.
 *   - When the partials of the default plan would exceed the buffer, the keys
 *     are processed in larger chunks (fewer splits, possibly none), so every
 *     valid description runs; results then equal dt_tree_attention's within
 *     rounding rather than bit for bit.
 *   - A caller-forced desc->split_keys whose partials exceed the buffer is
 *     rejected with DT_ERR_WORKSPACE.
 *   - The buffer keeps the last call's contents. Calls on one stream are
 *     ordered; calls that overlap on one GPU (other streams or threads) share
 *     the buffer and race, so the caller serializes them.
 * Errors: as dt_tree_attention (DT_ERR_WORKSPACE as above; DT_ERR_HIP also
 * when the buffer's device address cannot be obtained).
 */
int dt_tree_attention_noalloc(const dt_attn_desc* desc, const void* q, const void* k_tree, const void* v_tree,
                              const void* k_prefix, const void* v_prefix, const int32_t* parent, void* out,
                              void* stream);

/*
 * dt_argmax_rows_workspace_size -- bytes of device workspace dt_argmax_rows
 * needs for `rows` rows of `vocab` entries on the current device.
 */
int dt_argmax_rows_workspace_size(int64_t rows, int64_t vocab, size_t* bytes);

/*
 * dt_argmax_rows -- the target's greedy prediction at every node (GPU).
 *
 * Defined by: DARTree paper, Preliminaries > Speculative Sampling: at T = 0
 * a draft token is accepted when it equals the target model's greedy
 * prediction. out_idx[r] = the lowest j in [0, vocab) with
 * logits[r*row_stride + j] == max over the row (IEEE compare: -0 == +0).
 *   logits     device float32, rows x vocab, row stride row_stride >= vocab;
 *              4-byte aligned. Contract: finite values (a NaN gives an
 *              unspecified index in [0, vocab)).
 *   rows >= 0 (0 is a no-op; at most 65535), 1 <= vocab < 2^31
 *   out_idx    device int32 [rows]
 *   workspace  device scratch, >= dt_argmax_rows_workspace_size bytes,
 *              256-byte aligned; may be NULL when that size is 0.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_UNSUPPORTED (rows > 65535),
 * DT_ERR_WORKSPACE, DT_ERR_HIP.
 */
int dt_argmax_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t* out_idx,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * dt_sample_rows_workspace_size -- bytes of device workspace dt_sample_rows
 * needs for `rows` rows of `vocab` entries on the current device.
 */
int dt_sample_rows_workspace_size(int64_t rows, int64_t vocab, size_t* bytes);

/*
 * dt_sample_rows -- the target's sample at every node, T > 0 (GPU).
 *
 * Defined by: DARTree paper, Preliminaries > Speculative Sampling (exact
 * target-sample matching, the DFlash rule: accept draft tokens while they
 * equal the target's samples, emit the target's sample at the first mismatch;
 * the target distribution at temperature T is p_T = softmax(logits / T)) and
 * Experimental Setup > Evaluation Details (at T = 1 verification accepts the
 * longest sampled prefix in the tree). Feeding out_idx to dt_accept_path in
 * place of dt_argmax_rows' output gives that rule on a tree.
 *
 * The draw is Gumbel-max: out_idx[r] = the lowest j maximising
 *   logits[r*row_stride + j] / T - ln(-ln U[r][j]),
 * which is an exact sample of p_T. U comes from Philox4x32-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011):
 *   w = Philox4x32-10(counter = (r, j / 4, offset & 0xffffffff, offset >> 32),
 *                     key = (seed & 0xffffffff, seed >> 32))[j % 4]
 *   U = (2 * (w >> 9) + 1) * 2^-24          (in (0, 1), exact in fp32)
 * so every (seed, offset, row, j) has one fixed draw; use a new offset (or
 * seed) per verification round. The comparison runs in fp32 as
 * logits * (log2(e) / T) - log2(-log2 U), an order-preserving rescaling of the
 * definition; candidates whose exact scores differ by less than fp32 rounding
 * (a relative 1e-6 or so) may resolve either way.
 *   logits, rows, vocab, row_stride, out_idx, workspace: as dt_argmax_rows.
 *   temperature  > 0 and finite, with log2(e) / T representable in fp32
 *                (T = 0, greedy decoding, is dt_argmax_rows); contract:
 *                logits / T finite.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_VALUE (temperature),
 * DT_ERR_UNSUPPORTED (rows > 65535), DT_ERR_WORKSPACE, DT_ERR_HIP.
 */
int dt_sample_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, float temperature,
                   uint64_t seed, uint64_t offset, int32_t* out_idx, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * dt_accept_path -- longest accepted root-to-leaf path and bonus token (GPU).
 *
 * Defined by: DARTree paper, Preliminaries > Speculative Sampling (T = 0:
 * accept consecutive draft tokens equal to the target's greedy predictions;
 * at the first mismatch emit the target prediction; each round commits the
 * accepted prefix plus that bonus token) and Tree Verification and DDTree
 * (the accepted root-to-leaf prefix is selected according to the target).
 * Per tree s: start at the root; while some child c of the current node has
 * token[c] == argmax_idx[current], move to the lowest-index such child.
 * L_s = number of moves; bonus_s = argmax_idx[last node]; tau = L_s + 1.
 *   node_offsets host int32 [S+1] (as in dt_attn_desc), read during the call
 *   parent, token, argmax_idx  device int32 [N] (parent and path tree-local;
 *              argmax_idx typically dt_argmax_rows' output)
 *   path       device int32 [N]: path[node_offsets[s] + t], t = 0..L_s, is the
 *              t-th accepted node (t = 0 is the root); the tree's other
 *              entries are set to -1
 *   accept_len device int32 [S] (L_s); bonus device int32 [S]
 * Contract: parent as in the tree representation (a cycle-free walk is
 * guaranteed regardless: the walk only moves to higher indices).
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_HIP.
 */
int dt_accept_path(int32_t num_seqs, const int32_t* node_offsets, const int32_t* parent, const int32_t* token,
                   const int32_t* argmax_idx, int32_t* path, int32_t* accept_len, int32_t* bonus, void* stream);

/*
 * Description of one KV commit. Counts and strides in elements (bf16).
 *
 * Sequence s has n_s = node_offsets[s+1] - node_offsets[s] tree nodes (>= 1),
 * a verified prefix of P_s = prefix_lens[s] rows starting at cache row
 * prefix_row_start[s], and cache_rows[s] rows of room from that start (the
 * verified rows included). Host arrays are read during the call only.
 */
typedef struct dt_commit_desc {
  int32_t num_seqs;                /* S >= 1 */
  int32_t num_layers;              /* >= 1: one (tree K/V, cache K/V) quadruple per layer */
  int32_t num_kv_heads;            /* Hkv >= 1 */
  int32_t head_dim;                /* d >= 8, a multiple of 8 */
  int32_t max_path;                /* 0, or a bound on accept_len[s] + 1 for every s (e.g. the
                                      trees' depth + 1): fewer positions to launch and to reserve */
  const int32_t* node_offsets;     /* host [S+1]; node_offsets[0] = 0, increasing */
  const int32_t* prefix_lens;      /* host [S] */
  const int64_t* prefix_row_start; /* host [S] */
  const int64_t* cache_rows;       /* host [S]: must be >= P_s + min(n_s, max_path or n_s) */
  int64_t tree_row_stride;         /* between node rows of k_tree/v_tree; 0 means Hkv*d */
  int64_t cache_row_stride;        /* between cache rows (>= 8) */
  int64_t cache_head_stride;       /* between KV heads within a cache row (>= d when Hkv > 1) */
} dt_commit_desc;

/*
 * dt_commit_kv -- write the accepted path's keys and values into the KV cache (GPU).
 *
 * Defined by: DARTree paper, Preliminaries > Speculative Sampling (every round
 * commits the accepted draft prefix followed by one bonus token) and Figure 3
 * (tree verification passes the accepted tokens and their features on). The
 * verification forward computed K/V for every tree node at position
 * P_s + depth; for the accepted path path[0] = root, ..., path[L_s], where the
 * node at path position t has depth t, the call copies, for every layer,
 *   cache row prefix_row_start[s] + P_s + t  <-  tree row node_offsets[s] + path[t]
 * for t = 0 .. L_s (K and V, all KV heads). Afterwards the sequence's verified
 * prefix is P_s + L_s + 1 rows; the bonus token has no K/V yet (it is the next
 * round's root). Only those rows are written.
 *   k_tree, v_tree    host arrays [num_layers] of device pointers: [N][Hkv][d] bf16,
 *                     row stride tree_row_stride (the same buffers dt_tree_attention read)
 *   k_cache, v_cache  host arrays [num_layers] of device pointers: row r, head h
 *                     at base + r*cache_row_stride + h*cache_head_stride
 *   path, accept_len  device int32, as written by dt_accept_path ([N] tree-local
 *                     nodes and [S] accepted lengths); read on the device, so
 *                     the call needs no host synchronisation.
 * Every buffer 16-byte aligned (path, accept_len: 4). Cache buffers must not
 * alias tree buffers. Contract: path and accept_len as dt_accept_path leaves
 * them; a path entry outside [0, n_s), or positions at or past max_path, are
 * skipped, never written out of bounds.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE (counts, strides, alignment, room),
 * DT_ERR_UNSUPPORTED (more than 65535 path positions), DT_ERR_HIP.
 */
int dt_commit_kv(const dt_commit_desc* desc, const void* const* k_tree, const void* const* v_tree,
                 void* const* k_cache, void* const* v_cache, const int32_t* path, const int32_t* accept_len,
                 void* stream);

/*
 * DARTree tree construction (GPU): the drafter's per-depth candidates, the
 * depth-wise fixed-width expansion and the deferred top-B pruning of DARTree
 * paper, Methodology (Depth-Wise Parallel Supertree Construction, Algorithm 1;
 * Deferred Best-First Pruning, eq. 5-6 and Lemma 1). The correction head that
 * scores candidates under each prefix (Algorithm 1's correction step) is a trained
 * network and stays with the caller: it turns the retained prefixes of depth
 * d-1 into log q~ values for every (prefix, candidate) pair, which
 * dt_expand_depth consumes.
 */

/*
 * dt_topk_rows_workspace_size -- device workspace of dt_topk_rows.
 */
int dt_topk_rows_workspace_size(int64_t rows, int64_t vocab, int32_t k, size_t* bytes);

/*
 * dt_topk_rows -- C_d = TopK(L_d, K): the k best entries of every row, in
 * order, with their log-softmax values (GPU).
 *
 * Defined by: DARTree paper, Depth-Wise Parallel Supertree Construction (only
 * the drafter's top-K token predictions at each position are candidate
 * extensions) and Algorithm 1's candidate step. Per row r: out_token[r][0..k-1] are the
 * indices of the k largest logits ordered by (logit descending, index
 * ascending; -0 == +0), and out_logprob[r][j] = logits[r][out_token[r][j]] -
 * log(sum_v exp(logits[r][v])) in fp32. The same table, one row per draft
 * position, is the candidate input of dt_build_tree.
 *   logits     device float32, rows x vocab, row stride >= vocab (4-byte
 *              aligned; 16-byte rows read faster). Contract: finite values.
 *   rows       0 .. 65535 (0 is a no-op); 1 <= k <= min(vocab, 1024), and
 *              ceil(vocab / 4096) * k <= 16384 (DT_ERR_UNSUPPORTED otherwise)
 *   out_token  device int32 [rows][k]; out_logprob device float32 [rows][k]
 *   workspace  >= dt_topk_rows_workspace_size bytes, 256-byte aligned.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_UNSUPPORTED, DT_ERR_WORKSPACE, DT_ERR_HIP.
 */
int dt_topk_rows(const float* logits, int64_t rows, int64_t vocab, int64_t row_stride, int32_t k,
                 int32_t* out_token, float* out_logprob, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dt_expand_depth -- one depth of DARTree's fixed-width supertree (GPU).
 *
 * Defined by: DARTree paper, Algorithm 1's expansion step with eq. 5's score. For
 * every sequence s, every retained prefix (slot p < w_prev of depth d-1, score
 * parent_score[p]) and every candidate c < k of depth d, the child scores
 *   score(p, c) = (parent_score[p] + child_logq[p][c]) + beta      (fp32, in this order)
 * and the w children with the highest scores are kept, ordered by (score
 * descending, p ascending, c ascending). Children whose score is not finite
 * (e.g. an absent parent slot with score -inf) are never kept; when fewer than
 * w remain, the extra output slots get parent = cand = token = -1 and score -inf.
 *   parent_score  device float [S] rows of w_prev, row stride parent_score_stride
 *                 (depth 1: the root alone, w_prev = 1, score 0)
 *   child_logq    device float [S] rows of w_prev * k (row-major [p][c]), row
 *                 stride child_logq_stride: the correction head's log q~
 *   cand_token    device int32 [S] rows of k (stride cand_token_stride): the
 *                 candidates' tokens, e.g. dt_topk_rows' output for this depth
 *   sel_parent, sel_cand, sel_token, sel_score  device [S] rows of w, row
 *                 stride out_stride: the kept children (their scores are the
 *                 next depth's parent_score)
 *   beta          depth bonus, <= 0 and finite (Algorithm 1 requires beta <= 0)
 * Limits: w_prev * k <= 16384, w <= 1024, S <= 65535 (DT_ERR_UNSUPPORTED).
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_VALUE (beta), DT_ERR_UNSUPPORTED, DT_ERR_HIP.
 */
int dt_expand_depth(int32_t num_seqs, int32_t w_prev, int32_t k, int32_t w, float beta, const float* parent_score,
                    int64_t parent_score_stride, const float* child_logq, int64_t child_logq_stride,
                    const int32_t* cand_token, int64_t cand_token_stride, int32_t* sel_parent, int32_t* sel_cand,
                    int32_t* sel_token, float* sel_score, int64_t out_stride, void* stream);

/*
 * dt_prune_topb -- deferred top-B pruning of the supertree into the
 * verification tree (GPU).
 *
 * Defined by: DARTree paper, Deferred Best-First Pruning, eq. 6 and Lemma 1
 * (with beta <= 0 and ancestors preferred on ties, the best-first heap over the
 * supertree equals its global top-B by s_beta), and Algorithm 1's final pruning.
 * The supertree of sequence s is depths layers of w slots (dt_expand_depth's
 * outputs, layer d-1 at offset (d-1)*w): slot j of depth d is the child of slot
 * sel_parent of depth d-1 (depth 1: of the root), carries sel_token and
 * sel_score; slots with sel_parent < 0 or a non-finite score are empty. The
 * call keeps the budget best nodes by (score descending, depth ascending, slot
 * ascending) and writes the tree root first, then those nodes in that order,
 * which lists every parent before its children:
 *   parent[s][i] (tree-local, parent[s][0] = -1), token[s][i] (token[s][0] =
 *   root_token[s]), depth[s][i], score[s][i] (score[s][0] = 0) for
 *   i < n_out[s] = 1 + min(budget, non-empty slots); rows past n_out[s] get
 *   parent = token = depth = -1, score -inf.
 *   sel_parent, sel_token, sel_score  device [S][depths][w]
 *   root_token  device int32 [S]
 *   parent, token, depth, score  device [S][budget + 1]; n_out device int32 [S]
 * Contract: the log q~ behind the scores are <= 0 and beta <= 0 (then every
 * child scores at most its parent, Lemma 1). If the device data break it, the
 * output is still a tree: a kept node whose parent is not kept before it is
 * dropped.
 * Limits: depths * w <= 16384, budget + 1 <= DT_MAX_TREE_NODES, S <= 65535.
 * Errors: DT_ERR_NULL, DT_ERR_SHAPE, DT_ERR_UNSUPPORTED, DT_ERR_HIP.
 */
int dt_prune_topb(int32_t num_seqs, int32_t depths, int32_t w, int32_t budget, const int32_t* sel_parent,
                  const int32_t* sel_token, const float* sel_score, const int32_t* root_token, int32_t* parent,
                  int32_t* token, int32_t* depth, float* score, int32_t* n_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DTREE_H */
