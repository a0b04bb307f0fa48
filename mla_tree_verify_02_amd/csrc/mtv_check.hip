// gfx950 kernels that count out-of-range device inputs of the verify attention.
//
// The attention reads three caller-owned index inputs that live in device
// memory: the per-token page table ("The 130x Slowdown", The Reasoning, step
// 4), the sequence lengths (prefix plus tree block) and the per-node tree
// bitmask ("The Moment of Certainty", The Path Forward). Checking them on the
// host would need a copy and a synchronisation on every call, so the
// attention only clamps them. These kernels count what the clamps would hide,
// on the stream, for callers that want to know.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mtv_internal.h"

namespace mtv {
namespace {

constexpr int kCheckThreads = 256;

__global__ void check_zero_kernel(unsigned long long* counts)
{
    if (threadIdx.x < kCheckCounts)
        counts[threadIdx.x] = 0ull;
}

__device__ __forceinline__ unsigned long long wave_total(unsigned long long v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Workgroups (x, y) take sequences y, y + gridDim.y, ... and, in each, the
// table positions x * 256 + tid, stepping by gridDim.x * 256, below the
// sequence's key count. Workgroup x = 0 of a sequence also checks its length
// and its N mask rows. Each wave adds its totals with one atomic per counter.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(int batch, int nodes, int max_kv,
                                                              int64_t num_slots,
                                                              const int32_t* __restrict__ page_table,
                                                              const int32_t* __restrict__ seq_lens,
                                                              const uint32_t* __restrict__ mask,
                                                              unsigned long long* counts)
{
    const int tid = threadIdx.x;
    const int W = (nodes + 31) >> 5;
    const int used = nodes - 32 * (W - 1);  // bits of the last word that name nodes: 1..32
    const uint32_t spare = used == 32 ? 0u : ~((1u << used) - 1u);
    unsigned long long bad_len = 0, bad_slot = 0, bad_mask = 0;
    for (int b = blockIdx.y; b < batch; b += gridDim.y) {
        const int raw = seq_lens[b];
        // the key count the attention uses: S_b clamped to [N, max_kv]
        const int S = min(max(raw, nodes), max_kv);
        const int32_t* row = page_table + (int64_t)b * max_kv;
        for (int p = blockIdx.x * kCheckThreads + tid; p < S; p += gridDim.x * kCheckThreads) {
            const int v = row[p];
            bad_slot += (v < 0 || (int64_t)v >= num_slots) ? 1ull : 0ull;
        }
        if (blockIdx.x == 0) {
            if (tid == 0)
                bad_len += (raw < nodes || raw > max_kv) ? 1ull : 0ull;
            for (int i = tid; i < nodes; i += kCheckThreads)
                bad_mask += (mask[((int64_t)b * nodes + i) * W + (W - 1)] & spare) ? 1ull : 0ull;
        }
    }
    bad_len = wave_total(bad_len);
    bad_slot = wave_total(bad_slot);
    bad_mask = wave_total(bad_mask);
    if ((tid & 63) == 0) {
        if (bad_len)
            atomicAdd(&counts[0], bad_len);
        if (bad_slot)
            atomicAdd(&counts[1], bad_slot);
        if (bad_mask)
            atomicAdd(&counts[2], bad_mask);
    }
}

}  // namespace

hipError_t launch_check_inputs(int batch, int nodes, int max_kv, int64_t num_slots,
                               const int32_t* page_table, const int32_t* seq_lens,
                               const uint32_t* mask, unsigned long long* counts, int cus,
                               hipStream_t stream)
{
    // a fill kernel rather than a memset, so that the call can be captured
    hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(64), 0, stream, counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // about four workgroups per CU in all: positions over x, sequences over y
    const int total = 4 * (cus > 0 ? cus : 256);
    const int gy = batch < total ? batch : total;
    int gx = (max_kv + kCheckThreads - 1) / kCheckThreads;
    const int room = (total + gy - 1) / gy;
    if (gx > room)
        gx = room;
    if (gx < 1)
        gx = 1;
    hipLaunchKernelGGL(check_kernel, dim3(gx, gy), dim3(kCheckThreads), 0, stream, batch, nodes,
                       max_kv, num_slots, page_table, seq_lens, mask, counts);
    return hipGetLastError();
}

}  // namespace mtv
