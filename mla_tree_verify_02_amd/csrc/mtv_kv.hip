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
// (2304 chunks, 9 per lane), striding over the batch's rows. The passes of a
// workgroup are software-pipelined: the table words of pass q+1 are loaded
// before the rows of pass q are stored, and its rows are loaded right after
// those stores are issued, so a pass's load latency overlaps the previous
// pass's stores (vmcnt retires in order: waiting for a load never waits for
// stores issued after it). Destination runs must not overlap any source row
// (the host documents this), so passes need no ordering among themselves.
// Rows are read and written once: non-temporal loads and stores keep them out
// of the caches. Reads are clamped to the pool; destinations outside it are
// skipped.
// The table phase follows in the same kernel: every table word belongs to one
// pass and every pass to one workgroup, so once all of a workgroup's waves are
// past its last pass (one barrier), it sets table[b][p] = base_b + p for the
// rows of its own passes whose destination lies in the pool. No other
// workgroup reads those words.
__global__ __launch_bounds__(kMoveThreads) void kv_move_kernel(
    int batch, int max_kv, int64_t num_slots, u32x4* __restrict__ kv,
    int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ base, int64_t rows_per_seq_stride)
{
    const int tid = threadIdx.x;
    const int64_t maxslot = num_slots - 1;
    // pass q covers rows 32q .. 32q+31 of the flattened (sequence, position)
    // space [0, batch * rows_per_seq_stride)
    const int64_t passes = ((int64_t)batch * rows_per_seq_stride + kMoveRows - 1) / kMoveRows;
    int64_t q = blockIdx.x;
    if (q >= passes)
        return;

    // Table words of pass qq for this lane's chunks: src = the source slot
    // (clamped to the pool) or -1 (no row: past the batch or the sequence),
    // dst = the destination slot or -1 (no row, or outside the pool). The
    // table word, the length and the base are loaded independently; the
    // length only decides afterwards whether the row exists.
    auto fetch = [&](int64_t qq, int32_t* src, int32_t* dst) {
        const int64_t f0 = qq * kMoveRows;
        const int64_t b0 = f0 / rows_per_seq_stride;  // one division per pass
        const int64_t p0 = f0 - b0 * rows_per_seq_stride;
        int32_t tv[kMoveLoads], sl[kMoveLoads], bs[kMoveLoads], pos[kMoveLoads];
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int r = (j * kMoveThreads + tid) / kRowChunks;  // row within the pass
            int64_t pp = p0 + r;
            int64_t bb = b0;
            while (pp >= rows_per_seq_stride) {  // at most 32 / stride steps
                pp -= rows_per_seq_stride;
                ++bb;
            }
            pos[j] = -1;
            tv[j] = 0, sl[j] = 0, bs[j] = 0;
            if (bb < batch) {
                pos[j] = (int)pp;  // < max_kv: inside the table row
                tv[j] = table[bb * max_kv + pp];
                sl[j] = seq_lens[bb];
                bs[j] = base[bb];
            }
        }
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int S = min(max(sl[j], 0), max_kv);
            src[j] = -1;
            dst[j] = -1;
            if (pos[j] >= 0 && pos[j] < S) {
                const int64_t sv = tv[j];
                src[j] = (int32_t)(sv < 0 ? 0 : (sv > maxslot ? maxslot : sv));
                const int64_t d = (int64_t)bs[j] + pos[j];
                if (d >= 0 && d <= maxslot)
                    dst[j] = (int32_t)d;
            }
        }
    };
    auto load_rows = [&](const int32_t* src, u32x4* v) {
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int c = j * kMoveThreads + tid;
            const int r = c / kRowChunks;
            v[j] = src[j] >= 0 ? __builtin_nontemporal_load(&kv[(int64_t)src[j] * kRowChunks + (c - r * kRowChunks)])
                               : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_rows = [&](const int32_t* dst, const u32x4* v) {
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j) {
            const int c = j * kMoveThreads + tid;
            const int r = c / kRowChunks;
            if (dst[j] >= 0)
                __builtin_nontemporal_store(v[j], &kv[(int64_t)dst[j] * kRowChunks + (c - r * kRowChunks)]);
        }
    };

    int32_t src[kMoveLoads], dst[kMoveLoads];
    u32x4 v[kMoveLoads];
    fetch(q, src, dst);
    load_rows(src, v);
    for (;;) {
        const int64_t qn = q + gridDim.x;
        const bool more = qn < passes;  // uniform
        int32_t srcn[kMoveLoads], dstn[kMoveLoads];
        if (more)
            fetch(qn, srcn, dstn);
        store_rows(dst, v);
        if (!more)
            break;
        load_rows(srcn, v);
#pragma unroll
        for (int j = 0; j < kMoveLoads; ++j)
            dst[j] = dstn[j];
        q = qn;
    }

    // Table phase for this workgroup's passes: one thread per row.
    __syncthreads();  // every wave has read its table words
    if (tid < kMoveRows) {
        for (int64_t qq = blockIdx.x; qq < passes; qq += gridDim.x) {
            const int64_t f = qq * kMoveRows + tid;
            const int64_t bb = f / rows_per_seq_stride;
            const int64_t pp = f - bb * rows_per_seq_stride;
            if (bb < batch && pp < min(max(seq_lens[bb], 0), max_kv)) {
                const int64_t d = (int64_t)base[bb] + pp;
                if (d >= 0 && d <= maxslot)
                    table[bb * max_kv + pp] = (int32_t)d;
            }
        }
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
    // A resident grid: the copy kernel's registers allow three workgroups per
    // compute unit, and each workgroup loops over passes (pipelined).
    const int64_t grid = passes < (int64_t)cus * 3 ? passes : (int64_t)cus * 3;
    hipLaunchKernelGGL(kv_move_kernel, dim3((unsigned)grid), dim3(kMoveThreads), 0, stream, a.batch,
                       a.max_kv, a.num_slots, (u32x4*)a.kv, a.page_table, a.seq_lens, a.base, stride);
    return hipGetLastError();
}

}  // namespace mtv
