// gfx950 kernels that move latent KV rows inside the page_size=1 pool after a
// verify step: the commit of an accepted tree path into the request's
// contiguous run of slots, and the move of a whole sequence into such a run
// (Tier-0 defragmentation: "The Moment of Reckoning: A User's Challenge That
// Reshaped a Long-Context Inference Investigation", Output Knowledge Created by
// This Message). Accepted tree nodes sit at scattered slots because the tree
// block is not contiguous ("The Moment of Certainty", The User Provides the
// Final Piece); both kernels gather rows through the per-token page table with
// the same 16-byte chunking as the attention's gather and rewrite the table.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mtv_internal.h"

namespace mtv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowChunks = kRowBytes / 16;  // 72 x 16 B per 1152-byte row
constexpr int kMaxPath = 64;                // accepted nodes per sequence (N <= 64)
constexpr int kCommitThreads = 256;

// One workgroup per sequence. Positions S-N .. S-1 of the page-table row hold
// tree nodes 0..N-1. For k < L (the accepted count, clamped to [0, N]):
// node n_k = path[k] (clamped to [0, N)), source slot = table[S-N+n_k],
// destination slot = base + S-N+k. All L source rows are read into LDS before
// any destination row is written, so a destination that is also some other
// accepted node's source is still read first; then each row is written and
// table[S-N+k] is set to its destination. Slots are clamped to the pool on
// read; a destination outside the pool is not written (its table entry is
// left as it was).
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(
    int nodes, int max_kv, int64_t num_slots, u32x4* __restrict__ kv, int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ path, const int32_t* __restrict__ base)
{
    __shared__ u32x4 s_rows[kMaxPath * kRowChunks];  // 72 KB
    __shared__ int s_src[kMaxPath];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int S = min(max(seq_lens[b], nodes), max_kv);
    const int L = min(max(accept_len[b], 0), nodes);
    const int t0 = S - nodes;  // first tree position
    int32_t* trow = table + (int64_t)b * max_kv;
    const int64_t maxslot = num_slots - 1;
    if (tid < L) {
        const int n = min(max(path[(int64_t)b * nodes + tid], 0), nodes - 1);
        const int64_t s = trow[t0 + n];
        s_src[tid] = (int)(s < 0 ? 0 : (s > maxslot ? maxslot : s));
    }
    __syncthreads();
    for (int c = tid; c < L * kRowChunks; c += kCommitThreads) {
        const int k = c / kRowChunks;
        s_rows[c] = kv[(int64_t)s_src[k] * kRowChunks + (c - k * kRowChunks)];
    }
    __syncthreads();  // every source row is in LDS before any destination is written
    const int64_t d0 = (int64_t)base[b] + t0;
    for (int c = tid; c < L * kRowChunks; c += kCommitThreads) {
        const int k = c / kRowChunks;
        const int64_t d = d0 + k;
        if (d >= 0 && d <= maxslot)
            kv[d * kRowChunks + (c - k * kRowChunks)] = s_rows[c];
    }
    if (tid < L) {
        const int64_t d = d0 + tid;
        if (d >= 0 && d <= maxslot)
            trow[t0 + tid] = (int32_t)d;
    }
}

constexpr int kMoveThreads = 256;
constexpr int kMoveRows = 32;                              // rows per workgroup pass
constexpr int kMoveLoads = kMoveRows * kRowChunks / kMoveThreads;  // 9 chunks per lane
static_assert(kMoveRows * kRowChunks % kMoveThreads == 0, "whole chunks per lane");

// Whole-sequence move, copy phase: rows of positions [0, S_b) of each sequence
// go from their table slots to base_b + p. A workgroup copies 32 rows per pass
// (2304 chunks, 9 per lane, all loads issued before any store), striding over
// the batch's rows. Destination runs must not overlap any source row (the host
// documents this), so passes need no ordering among themselves. Rows are read
// and written once: non-temporal loads and stores keep them out of the caches.
// Reads are clamped to the pool; destinations outside it are skipped.
__global__ __launch_bounds__(kMoveThreads) void kv_move_kernel(
    int batch, int max_kv, int64_t num_slots, u32x4* __restrict__ kv,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ base, int64_t rows_per_seq_stride)
{
    const int tid = threadIdx.x;
    const int64_t maxslot = num_slots - 1;
    // pass q covers rows 32q .. 32q+31 of the flattened (sequence, position)
    // space [0, batch * rows_per_seq_stride)
    const int64_t passes = ((int64_t)batch * rows_per_seq_stride + kMoveRows - 1) / kMoveRows;
    for (int64_t q = blockIdx.x; q < passes; q += gridDim.x) {
        // (sequence, position) of the pass's first row; one division per pass
        const int64_t f0 = q * kMoveRows;
        const int64_t b0 = f0 / rows_per_seq_stride;
        const int64_t p0 = f0 - b0 * rows_per_seq_stride;
        u32x4 v[kMoveLoads];
        int32_t drow[kMoveLoads];  // destination slot, or -1
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int c = j * kMoveThreads + tid;        // chunk within the pass
            const int r = c / kRowChunks;                 // row within the pass
            int64_t pp = p0 + r;
            int64_t bb = b0;
            while (pp >= rows_per_seq_stride) {  // at most 32 / stride steps
                pp -= rows_per_seq_stride;
                ++bb;
            }
            const int b = (int)(bb < batch ? bb : batch);
            const int p = (int)pp;
            drow[j] = -1;
            v[j] = u32x4{0u, 0u, 0u, 0u};
            if (b < batch) {
                const int S = min(max(seq_lens[b], 0), max_kv);
                if (p < S) {
                    int64_t s = table[(int64_t)b * max_kv + p];
                    s = s < 0 ? 0 : (s > maxslot ? maxslot : s);
                    v[j] = __builtin_nontemporal_load(&kv[s * kRowChunks + (c - r * kRowChunks)]);
                    const int64_t d = (int64_t)base[b] + p;
                    if (d >= 0 && d <= maxslot)
                        drow[j] = (int32_t)d;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int c = j * kMoveThreads + tid;
            const int r = c / kRowChunks;
            if (drow[j] >= 0)
                __builtin_nontemporal_store(v[j], &kv[(int64_t)drow[j] * kRowChunks + (c - r * kRowChunks)]);
        }
    }
}

// Whole-sequence move, table phase (after the copy phase on the same stream):
// table[b][p] = base_b + p for p < S_b whose destination lies in the pool.
__global__ __launch_bounds__(kMoveThreads) void kv_move_table_kernel(
    int batch, int max_kv, int64_t num_slots, int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ base)
{
    const int b = blockIdx.y;
    const int S = min(max(seq_lens[b], 0), max_kv);
    for (int p = blockIdx.x * kMoveThreads + threadIdx.x; p < S; p += gridDim.x * kMoveThreads) {
        const int64_t d = (int64_t)base[b] + p;
        if (d >= 0 && d < num_slots)
            table[(int64_t)b * max_kv + p] = (int32_t)d;
    }
}

}  // namespace

hipError_t launch_kv_commit(const KvArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_commit_kernel, dim3(a.batch), dim3(kCommitThreads), 0, stream, a.nodes,
                       a.max_kv, a.num_slots, (u32x4*)a.kv, a.page_table, a.seq_lens, a.accept_len,
                       a.path, a.base);
    return hipGetLastError();
}

hipError_t launch_kv_move(const KvArgs& a, int cus, hipStream_t stream)
{
    // rows per sequence slot in the flattened space: the longest possible S
    const int64_t stride = a.max_kv;
    const int64_t passes = ((int64_t)a.batch * stride + kMoveRows - 1) / kMoveRows;
    const int64_t grid = passes < (int64_t)cus * 8 ? passes : (int64_t)cus * 8;
    hipLaunchKernelGGL(kv_move_kernel, dim3((unsigned)grid), dim3(kMoveThreads), 0, stream, a.batch,
                       a.max_kv, a.num_slots, (u32x4*)a.kv, a.page_table, a.seq_lens, a.base, stride);
    if (hipGetLastError() != hipSuccess)
        return hipErrorLaunchFailure;
    const int xb = (a.max_kv + kMoveThreads - 1) / kMoveThreads;
    hipLaunchKernelGGL(kv_move_table_kernel, dim3(xb < 1024 ? xb : 1024, a.batch), dim3(kMoveThreads), 0,
                       stream, a.batch, a.max_kv, a.num_slots, a.page_table, a.seq_lens, a.base);
    return hipGetLastError();
}

}  // namespace mtv
