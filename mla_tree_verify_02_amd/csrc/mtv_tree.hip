// gfx950 kernel that builds the tree-verify visibility bitmask from the draft
// tree's parent array on the device.
//
// The verify attention lets tree node i see tree node j exactly when j is i or
// one of i's ancestors; the pages carry that visibility as a per-node bitmask
// next to the per-token page table ("The GPU That Wasn't There", The Native
// Engine Thesis) and build it on the CPU today, measured at 0.18 ms per step
// ("The GPU That Wasn't There", Assumptions and Their Validity). Here it is
// built where the attention consumes it, so no host round trip sits between
// the drafter's tree and the verify step.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mtv_internal.h"

namespace mtv {
namespace {

constexpr int kTreeThreads = 256;  // four sequences per workgroup, one per wave

// One wave per sequence, lane i = tree node i (N <= 64). Each lane walks its
// parent chain, reading the next parent from the lane that holds it, and sets
// one bit per node visited (itself first). A parent outside [-1, i) ends the
// walk as a root would, so every walk ends within i + 1 steps and reads only
// lanes below its own; the loop runs until no lane of the wave is still
// walking.
__global__ __launch_bounds__(kTreeThreads) void tree_mask_kernel(int batch, int nodes,
                                                                 const int32_t* __restrict__ parents,
                                                                 uint32_t* __restrict__ mask)
{
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (kTreeThreads / 64) + (threadIdx.x >> 6);
    if (b >= batch)
        return;  // whole waves: b is uniform within a wave
    const bool node = lane < nodes;
    int par = -1;
    if (node) {
        const int p = parents[(int64_t)b * nodes + lane];
        par = (p >= -1 && p < lane) ? p : -1;
    }
    uint32_t lo = 0u, hi = 0u;
    int j = node ? lane : -1;  // the node this lane visits next
    while (__builtin_amdgcn_ballot_w64(j >= 0) != 0) {
        if (j >= 0) {
            if (j < 32)
                lo |= 1u << j;
            else
                hi |= 1u << (j - 32);
        }
        const int pj = __shfl(par, j >= 0 ? j : 0);  // parent of node j
        j = (j >= 0) ? pj : -1;
    }
    if (node) {
        const int W = (nodes + 31) >> 5;
        uint32_t* out = mask + ((int64_t)b * nodes + lane) * W;
        out[0] = lo;
        if (W > 1)
            out[1] = hi;
    }
}

}  // namespace

hipError_t launch_tree_mask(int batch, int nodes, const int32_t* parents, uint32_t* mask,
                            hipStream_t stream)
{
    const int per = kTreeThreads / 64;
    hipLaunchKernelGGL(tree_mask_kernel, dim3((batch + per - 1) / per), dim3(kTreeThreads), 0, stream,
                       batch, nodes, parents, mask);
    return hipGetLastError();
}

}  // namespace mtv
