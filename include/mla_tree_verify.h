/*
 * mla_tree_verify.h -- C ABI of the MI355X (gfx950) absorbed-MLA tree-verify
 * attention library (libmla_tree_verify.so).
 *
 * The operation. In the speculative tree-verify decode step, every node of a
 * small draft tree (about nine of them, "The Moment of Certainty", section
 * Message 12190) queries, for each head, a long compressed-latent KV cache kept
 * in a pool with one token per page and reached through a per-token page table
 * ("The 130x Slowdown", The Reasoning, step 4; "The Moment of Certainty", The
 * User Provides the Final Piece, for why the page size is 1). The long prefix is
 * visible to every node; the tree block that follows it is filtered by a
 * per-node visibility bitmask ("The Moment of Certainty", The Path Forward;
 * "The GPU That Wasn't There", The Native Engine Thesis). In absorbed form the
 * 576-wide latent row is the key and its first 512 elements are the value
 * ("The 130x Slowdown", The Technical Depth). For sequence b, node i, head h:
 *
 *   V(b,i)  = { p < S_b - N }  u  { S_b - N + j : bit j of tree_mask[b][i] }
 *   s_p     = scale * < q[b][i][h][0:576], kv_pool[page_table[b][p]][0:576] >
 *   lse     = ln sum_{p in V} exp(s_p)                          (natural log)
 *   out     = sum_{p in V} exp(s_p - lse) * kv_pool[page_table[b][p]][0:512]
 *
 * An empty visible set yields out = 0 and lse = -inf.
 *
 * How it runs: a split-KV kernel (each workgroup takes one slice of one
 * sequence's key positions for up to 64 query rows, stages the slice's page
 * indices and the gathered 1152-byte rows in LDS, and runs Q.K^T and P.V on
 * bf16 MFMA with an online softmax in fp32), then a log-sum-exp combine kernel
 * that merges the slices and writes out and lse. Both are enqueued on `stream`.
 * Slices are balanced over the whole batch from seq_lens on the device: every
 * sequence is cut into slices of the same number of 32-key tiles, sized from
 * the batch's total, so a long sequence gets many slices and a short one few
 * (a batch of one sequence is sliced for max_kv keys).
 */
#ifndef MLA_TREE_VERIFY_H
#define MLA_TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ limits */
#define MTV_D_LATENT 512      /* value / latent width                        */
#define MTV_D_ROPE 64         /* RoPE key width                              */
#define MTV_D_QK 576          /* key and absorbed-query width (512 + 64)     */
#define MTV_MAX_NODES 64      /* tree nodes per sequence (two mask words)    */
#define MTV_MAX_BATCH 65535
#define MTV_MAX_KV (1 << 26)  /* key positions per sequence                  */

/* ------------------------------------------------------------ status codes */
#define MTV_OK 0
#define MTV_ERR_NULL -1       /* a required pointer is NULL                  */
#define MTV_ERR_SHAPE -2      /* shape outside the limits above              */
#define MTV_ERR_ALIGN -3      /* q, kv_pool or out not 16-byte aligned, or a
                                 4-byte array or the workspace misaligned     */
#define MTV_ERR_WORKSPACE -4  /* workspace_bytes below the required size     */
#define MTV_ERR_HIP -5        /* the HIP runtime refused a query or a launch */
#define MTV_ERR_SCRATCH -6    /* mla_tree_verify_noalloc: the call needs more
                                 than MTV_NOALLOC_SCRATCH_BYTES of workspace  */

/* Size of the fixed device scratch that mla_tree_verify_noalloc uses in
 * place of a caller workspace (one copy per GPU, held until the process
 * ends). */
#define MTV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * Problem shape. All fields are host values.
 *   batch      B >= 1 sequences
 *   num_nodes  N in [1, 64] tree nodes per sequence
 *   num_heads  H >= 1 query heads (N * H <= 65536 query rows per sequence)
 *   max_kv     row length of page_table; every S_b must lie in [N, max_kv]
 *   num_slots  rows in kv_pool, in [1, 2^31)
 */
typedef struct {
    int32_t batch;
    int32_t num_nodes;
    int32_t num_heads;
    int32_t max_kv;
    int64_t num_slots;
} mtv_shape;

/*
 * Bytes of device workspace mla_tree_verify needs for `shape` on the current
 * device (the split plan depends on the device's compute-unit count); the same
 * size serves mla_tree_verify_paged and the splitkv/combine pair. Returns 0
 * if the shape is invalid. Host-only; never synchronises.
 */
size_t mla_tree_verify_workspace_size(const mtv_shape* shape);

/*
 * Enqueue the verify attention on `stream` (NULL: the null stream).
 *
 * Device pointers (all caller-owned; the library never allocates, frees or
 * synchronises, so the call may be captured into a HIP graph):
 *   q          bf16 [B][N][H][576]  absorbed query, q_latent[512] | q_rope[64]
 *                                   (RoPE already applied); 16-byte aligned
 *   kv_pool    bf16 [num_slots][576] latent[512] | rope_k[64], 1152 B per row;
 *                                   16-byte aligned
 *   page_table int32 [B][max_kv]    pool slot of key position p of sequence b.
 *                                   Positions [0, S_b - N) are the prefix;
 *                                   positions [S_b - N, S_b) are tree nodes
 *                                   0..N-1 in node order. Entries at p >= S_b
 *                                   are never used.
 *   seq_lens   int32 [B]            S_b = prefix length + N
 *   tree_mask  uint32 [B][N][W], W = ceil(N/32): node i may attend tree node j
 *                                   iff bit (j & 31) of word (j >> 5) is set.
 *                                   Bits for j >= N are ignored.
 *   scale      softmax scale applied to the full 576-wide dot (e.g. 1/sqrt(192))
 *   out        bf16 [B][N][H][512]  written in full (round to nearest even)
 *   lse        fp32 [B][N][H]       natural-log sum of exp(scaled scores)
 *   workspace  >= mla_tree_verify_workspace_size(shape) bytes, 256-byte aligned;
 *              scratch for per-slice partial results and each sequence's
 *              slice range. Its contents need no initialisation and are
 *              meaningless after the call.
 *
 * Outputs must not alias inputs or the workspace. Calls that share a workspace
 * must be ordered on one stream.
 *
 * Errors: returns MTV_OK or a negative MTV_ERR_* code. Only host-visible
 * arguments are validated (no device memory is read on the host). Device
 * contents are clamped inside the kernels so that no access leaves its buffer:
 * S_b is clamped to [N, max_kv] and page indices to [0, num_slots); such
 * out-of-range values give unspecified results but never a fault. Rows
 * referenced at positions < S_b should hold finite values: a non-finite tree
 * row can reach nodes that mask it out (it is multiplied by a zero weight).
 */
int mla_tree_verify(const mtv_shape* shape,
                    const void* q,
                    const void* kv_pool,
                    const int32_t* page_table,
                    const int32_t* seq_lens,
                    const uint32_t* tree_mask,
                    float scale,
                    void* out,
                    float* lse,
                    void* workspace,
                    size_t workspace_bytes,
                    hipStream_t stream);

/*
 * mla_tree_verify with hybrid paging of the key positions: the prefix goes
 * through pages of page_size slots, the tree block through a per-token list.
 * The pages propose larger pages for the prefix while the draft tree stays
 * fine-grained ("The 130x Slowdown: Diagnosing Latency-Bound Decode in
 * Speculative Decoding on Blackwell GPUs", The Broader Implications: What
 * This Diagnosis Means), i.e. the contiguous prefix read in page-sized runs and only the
 * tree block addressed per token ("The Moment of Certainty", The Path Forward:
 * From Diagnosis to Solution).
 *
 * Key position p of sequence b (S_b = seq_lens[b], t0 = S_b - N) lives at
 *   p <  t0:  prefix_pages[b][p / page_size] * page_size + p % page_size
 *   p >= t0:  tree_slots[b][p - t0]           (tree node p - t0)
 * and everything else is exactly mla_tree_verify: the result equals an
 * mla_tree_verify call whose page_table holds those slots, bit for bit, when
 * that call also runs one 64-row group per split workgroup. This call always
 * does; mla_tree_verify runs two on many rows over long slices (see
 * mtv_plan_query), and then its slices, and so its rounding, differ.
 *   page_size    in [1, MTV_MAX_KV] (64 is the pages' figure)
 *   max_pages    row length of prefix_pages, >= ceil((max_kv - N) / page_size)
 *                for every position to have a page; a page number beyond the
 *                row reads its last entry
 *   prefix_pages int32 [B][max_pages], tree_slots int32 [B][N] (device,
 *                4-byte aligned)
 * Slots are clamped to [0, num_slots) like page indices. Workspace, other
 * arguments and errors are those of mla_tree_verify (page_table is not used).
 */
int mla_tree_verify_paged(const mtv_shape* shape,
                          int32_t page_size,
                          int32_t max_pages,
                          const void* q,
                          const void* kv_pool,
                          const int32_t* prefix_pages,
                          const int32_t* tree_slots,
                          const int32_t* seq_lens,
                          const uint32_t* tree_mask,
                          float scale,
                          void* out,
                          float* lse,
                          void* workspace,
                          size_t workspace_bytes,
                          hipStream_t stream);

/*
 * The two phases of mla_tree_verify, for callers that time them apart or that
 * merge slice partials themselves (for instance slices computed on several
 * devices, each holding part of a sequence's key positions).
 *
 * mla_tree_verify_splitkv enqueues only the split-KV kernel: it takes the same
 * inputs as mla_tree_verify and leaves, in `workspace`, one partial per
 * (64-row group, key slice of the batch): the unnormalised weighted latent sum
 * (stored as bf16, 1024 B per row), the running max of the scaled scores in
 * log2 units and the sum of 2^(score*log2(e) - max) (fp32, 8 B per row),
 * and, per sequence, its first batch slice and slice count (two int32).
 * mla_tree_verify_combine merges those partials by
 * log-sum-exp and writes out and lse. The combine must run on a workspace
 * filled by a splitkv call with the same shape, seq_lens and device, ordered
 * after it on a stream (both derive the slicing from seq_lens). Arguments, alignment
 * and error codes are those of mla_tree_verify; mla_tree_verify is exactly
 * the splitkv call followed by the combine call on the same stream.
 */
int mla_tree_verify_splitkv(const mtv_shape* shape,
                            const void* q,
                            const void* kv_pool,
                            const int32_t* page_table,
                            const int32_t* seq_lens,
                            const uint32_t* tree_mask,
                            float scale,
                            void* workspace,
                            size_t workspace_bytes,
                            hipStream_t stream);

int mla_tree_verify_combine(const mtv_shape* shape,
                            const int32_t* seq_lens,
                            void* out,
                            float* lse,
                            void* workspace,
                            size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Enqueue, on `stream`, the build of tree_mask from the draft tree's parent
 * array: node i may attend tree node j iff j == i or j is an ancestor of i.
 * This is the visibility the verify attention applies to the tree block ("The
 * GPU That Wasn't There", The Native Engine Thesis; "The Moment of Certainty",
 * The Path Forward: From Diagnosis to Solution), built on the device instead
 * of the host ("The GPU That Wasn't There", Assumptions and Their Validity,
 * which times the host build).
 *
 * Device pointers (caller-owned, 4-byte aligned):
 *   parents    int32 [B][N]   parent of node i, in [-1, i): -1 marks a root
 *                             (forests are allowed). Any other value is read as
 *                             -1, so a malformed tree still yields a valid mask.
 *   tree_mask  uint32 [B][N][W], W = ceil(N/32), the layout mla_tree_verify
 *                             reads; written in full (bits j >= N are zero).
 * batch in [1, MTV_MAX_BATCH], num_nodes in [1, MTV_MAX_NODES].
 * Returns MTV_OK or MTV_ERR_NULL / MTV_ERR_SHAPE / MTV_ERR_ALIGN / MTV_ERR_HIP.
 * Never allocates or synchronises; the call may be captured into a HIP graph.
 */
int mla_tree_mask_build(int32_t batch,
                        int32_t num_nodes,
                        const int32_t* parents,
                        uint32_t* tree_mask,
                        hipStream_t stream);

/*
 * Tier-0 commit of an accepted tree path, enqueued on `stream`: the accepted
 * nodes' latent rows move from their scattered tree-block slots into the
 * request's contiguous run of slots, and the page table follows them. The
 * pages keep per-request KV contiguous in the pool this way ("The Moment of
 * Reckoning: A User's Challenge That Reshaped a Long-Context Inference
 * Investigation", Output Knowledge Created by This Message); the tree block is
 * what is scattered ("The Moment of Certainty", The User Provides the Final
 * Piece).
 *
 * For each sequence b, with S_b = seq_lens[b] clamped to [N, max_kv],
 * t0 = S_b - N (the first tree position), L = accept_len[b] clamped to [0, N]
 * and k < L:
 *   node n_k = accept_path[b][k] (clamped to [0, N)),
 *   source slot = page_table[b][t0 + n_k], destination = region_base[b] + t0 + k;
 *   the source row is copied to the destination and page_table[b][t0 + k] is
 *   set to the destination. Every source row of a sequence is read before any
 *   of its destinations is written, so the destinations may overlap that
 *   sequence's own tree-block slots.
 * Device pointers (caller-owned): kv_pool bf16 [num_slots][576] (16-byte
 * aligned; rows are moved in place), page_table int32 [B][max_kv] (updated),
 * seq_lens int32 [B], accept_len int32 [B], accept_path int32 [B][N] (the path
 * in commit order, e.g. root first), region_base int32 [B] (slot of position
 * 0 of the request's run); all 4-byte aligned. Different sequences' reads and
 * writes must not overlap one another. Slots are clamped to the pool on read;
 * a destination outside the pool is skipped and its table entry kept. The
 * caller advances seq_lens to t0 + L for the next step.
 * Returns MTV_OK or MTV_ERR_NULL / MTV_ERR_SHAPE / MTV_ERR_ALIGN / MTV_ERR_HIP.
 */
int mla_kv_commit(int32_t batch,
                  int32_t num_nodes,
                  int32_t max_kv,
                  int64_t num_slots,
                  void* kv_pool,
                  int32_t* page_table,
                  const int32_t* seq_lens,
                  const int32_t* accept_len,
                  const int32_t* accept_path,
                  const int32_t* region_base,
                  hipStream_t stream);

/*
 * Tier-0 defragmentation of whole sequences (same pages as mla_kv_commit),
 * enqueued on `stream`: the rows of positions [0, S_b) of sequence b, S_b =
 * seq_lens[b] clamped to [0, max_kv], are copied from their page-table slots to
 * region_base[b] + p, and page_table[b][p] is set to region_base[b] + p. The
 * destination runs must not overlap any source row or each other (for
 * instance, a freshly allocated region); otherwise the result is unspecified
 * (never out of bounds: reads are clamped to the pool, destinations outside it
 * skipped). Pointers as for mla_kv_commit. One launch: the copy, with each
 * workgroup rewriting the table entries of the rows it moved once all of them
 * have been read.
 * Returns MTV_OK or MTV_ERR_NULL / MTV_ERR_SHAPE / MTV_ERR_ALIGN / MTV_ERR_HIP.
 */
int mla_kv_defrag(int32_t batch,
                  int32_t max_kv,
                  int64_t num_slots,
                  void* kv_pool,
                  int32_t* page_table,
                  const int32_t* seq_lens,
                  const int32_t* region_base,
                  hipStream_t stream);

/*
 * Count, on `stream`, the device-resident inputs of mla_tree_verify that lie
 * outside their ranges. The attention itself only clamps them (checking them
 * on the host would cost a copy and a synchronisation per call). The inputs
 * are the ones the operation above defines: the per-token page table ("The
 * 130x Slowdown", The Reasoning, step 4), S_b = prefix length + N and the
 * per-node tree bitmask ("The Moment of Certainty", The Path Forward).
 *
 * counts (uint64 [3], device memory, 8-byte aligned) is overwritten with:
 *   counts[0]  sequences b with seq_lens[b] outside [N, max_kv];
 *   counts[1]  table entries page_table[b][p] outside [0, num_slots), over
 *              the positions p < S_b that the attention reads, S_b =
 *              seq_lens[b] clamped to [N, max_kv];
 *   counts[2]  mask rows (b, i) with a bit set for a node j >= N (in the last
 *              word of the row; the attention ignores such bits).
 * All zero means every index the attention reads is in range. The other
 * device pointers (page_table int32 [B][max_kv], seq_lens int32 [B],
 * tree_mask uint32 [B][N][W]) are as for mla_tree_verify, read only, 4-byte
 * aligned. shape->num_heads is not used. Nothing is allocated or
 * synchronised, and the counters are cleared by a kernel (no memset), so the
 * call may be captured into a HIP graph; the caller reads counts after the
 * stream reaches it.
 * Returns MTV_OK or MTV_ERR_NULL / MTV_ERR_SHAPE / MTV_ERR_ALIGN / MTV_ERR_HIP.
 */
int mtv_check_inputs(const mtv_shape* shape,
                     const int32_t* page_table,
                     const int32_t* seq_lens,
                     const uint32_t* tree_mask,
                     uint64_t* counts,
                     hipStream_t stream);

/*
 * mla_tree_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, semantics, validation and errors as mla_tree_verify, minus
 * the workspace: the per-slice partials live in a fixed array of
 * MTV_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, whose device
 * address is looked up on the first call on each device. The call never
 * allocates, frees or synchronises.
 *
 * Limit: a call whose mla_tree_verify_workspace_size(shape) exceeds
 * MTV_NOALLOC_SCRATCH_BYTES returns MTV_ERR_SCRATCH and enqueues nothing
 * (compare the two beforehand to know). On a 256-CU MI355X one sequence of
 * up to 32,768 query rows (N * H) fits at any context (at most about 34 MB),
 * as do batches of up to 759 sequences of 8 nodes x 8 heads, or up to 380 of
 * 16 x 8.
 *
 * Sharing: every call on one GPU uses that GPU's one array, which keeps the
 * last call's contents (nothing in it needs clearing: a call writes every word
 * it reads). Calls that may overlap on one GPU race on it -- calls on
 * different streams, or from different threads, must be ordered by the caller
 * (events or one stream). Calls on different GPUs do not interact.
 */
int mla_tree_verify_noalloc(const mtv_shape* shape,
                            const void* q,
                            const void* kv_pool,
                            const int32_t* page_table,
                            const int32_t* seq_lens,
                            const uint32_t* tree_mask,
                            float scale,
                            void* out,
                            float* lse,
                            hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* mtv_status_string(int status);

/*
 * Introspection of the split plan the library uses for `shape` on a device with
 * `num_cus` compute units, for a batch whose sequences all hold max_kv keys:
 * key slices per sequence (*splits), keys per slice (*chunk, a multiple of 32)
 * and 64-row groups per sequence (*row_groups). Batches of other lengths are
 * sliced on the device from seq_lens with the same rule (slices of one size
 * for the whole batch, sized from its total key count). This is the plan of
 * the per-token-table calls: from 16 row groups and 48 tiles (1536 keys) per
 * slice, or from 8 row groups and 64 tiles, two row groups share a split
 * workgroup and the slots per row group double; mla_tree_verify_paged always runs one row group per workgroup, so
 * its slicing can differ. Host-only arithmetic.
 * Returns MTV_OK, MTV_ERR_NULL or MTV_ERR_SHAPE.
 */
int mtv_plan_query(const mtv_shape* shape, int num_cus, int* splits, int* chunk, int* row_groups);

#ifdef __cplusplus
}
#endif
#endif /* MLA_TREE_VERIFY_H */
