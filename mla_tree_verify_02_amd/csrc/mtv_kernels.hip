// gfx950 kernels for absorbed-MLA tree-verify attention over a page_size=1 pool.
//
// split_kernel: one workgroup = one key slice of one sequence x up to 64 query
//   rows (4 waves x 16 rows), or x 128 (4 waves x 32 rows) for calls with many
//   rows and long slices. Per slice it stages the page indices in LDS (by
//   direct global->LDS word loads), then streams 32-key tiles through a
//   3-buffer LDS ring filled by direct
//   global->LDS 16-byte loads (each 1152-byte latent row is nine full 128-byte
//   lines), computes S^T = K.Q^T and O^T += V^T.P^T on 16x16x32 bf16 MFMA, and
//   keeps an online softmax (running max in log2 units, running sum) in fp32.
//   The pages locate the time of this step in the per-token gather through the
//   page table ("The 130x Slowdown", The Reasoning, steps 2-5) and ask for a
//   kernel that reads the prefix without a mask and applies the tree bitmask
//   only to the tree block ("The Moment of Certainty", The Path Forward; "The
//   GPU That Wasn't There", The Native Engine Thesis): here the mask test runs
//   only in tiles that reach the tree block or the end of the sequence.
//   Slices have one length for the whole batch, derived on the device from
//   seq_lens (slicing()), so a long sequence gets many and a short one few.
//   Partial results go out with device-scope stores (through the XCD's L2).
//   The 64-row form runs for hybrid paging; per-token calls with one row
//   group per workgroup run split_ws_kernel instead, the same computation
//   with 8 waves: 4 compute the scores and weights, 4 the weighted values,
//   two waves per SIMD.
// combine_kernel: merges the slices of each row by log-sum-exp and writes the
//   bf16 output and the natural-log lse; one workgroup per work item, or, for
//   batches of 2..64 sequences, a fixed grid that walks the items the batch
//   needs.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mtv_internal.h"

namespace mtv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStages = 3;                                      // LDS tile buffers
constexpr int kWinTiles = 128;                                  // tiles per staged index window
constexpr int kWinKeys = kWinTiles * kTileKeys;                 // 4096 page indices per window
constexpr int kChunks = kRowBytes / 16;                          // 72 x 16 B per row
constexpr int kTileBytes = kTileKeys * kRowBytes;                // 36864
constexpr int kKeysPerWave = kTileKeys / kWaves;                 // 8 rows loaded per wave
constexpr int kLoadsPerWave = kKeysPerWave * kChunks / 64;       // 9 loads per wave per tile
constexpr int kKSteps = kDqk / 32;                               // 18 MFMA k-steps for Q.K^T
constexpr int kColBlocks = kDv / 16;                             // 32 output column blocks
constexpr int kPartRowElems = kDv;                               // bf16 elements per row of partial O
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kCombineWaves = 8;                                 // waves per combine workgroup
constexpr int kCombineThreads = kCombineWaves * 64;

static_assert(kKeysPerWave * kChunks % 64 == 0, "tile rows must fill whole wave loads");
static_assert(kTileKeys == 32, "the P.V k-step covers exactly one tile");

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same with every LDS operation of the wave completed as well. Used before
// a barrier that publishes this wave's LDS writes (ds_write) to other waves
// while its direct-to-LDS gathers are in flight: __syncthreads() alone emits
// no LDS wait here, and a wave that wrote a tile's rescale flag just before
// the barrier was measured to leave it unseen by the reader after it (wrong
// output in about 1 of 9 calls made right after the GPU had been idle).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Gathers straight into LDS are issued as inline assembly so that the
// compiler's wait insertion does not treat every later LDS read as dependent
// on them; their completion is tracked by the explicit vmcnt waits in the tile
// loop, and the "memory" clobber keeps LDS accesses in program order. The LDS
// destination is M0 plus the instruction offset (which moves the global
// address alike) plus the lane's index times the load size; nothing else in
// these kernels reads M0 (gfx9 LDS instructions do not).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Gather j (0..8) of a tile's row plan into the tile slot at slot_lds (wave
// uniform): lane i's 16 bytes land at slot_lds + 1024 j + 16 i. The gathers of
// a group of four share one M0 value, slot_lds + 4096 (j / 4), and take
// instruction offsets 1024 (j % 4); src is therefore the row address minus
// 1024 (j % 4), which the row plan folds into its byte offsets. M0 is an input
// operand, so the compiler writes it only when its value changes (one write
// per group instead of one per gather); the s_nop is the wait state an M0
// write needs before a load to LDS.
template <int kSub>
__device__ __forceinline__ void gather16_off(uint64_t src, uint32_t m0v)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
                 :
                 : "v"(src), "{m0}"(m0v), "i"(kSub * 1024)
                 : "memory");
}
__device__ __forceinline__ void gather16_slot(uint64_t src_minus_sub, uint32_t slot_lds, int j)
{
    // readfirstlane keeps the value in a scalar register even where the
    // compiler cannot prove it uniform
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(slot_lds + (uint32_t)(j >> 2) * 4096u);
    switch (j & 3) {  // j is a constant after unrolling
    case 0: gather16_off<0>(src_minus_sub, m0v); break;
    case 1: gather16_off<1>(src_minus_sub, m0v); break;
    case 2: gather16_off<2>(src_minus_sub, m0v); break;
    default: gather16_off<3>(src_minus_sub, m0v); break;
    }
}

// clamp(x, 0, hi) for hi >= 0, in one instruction
__device__ __forceinline__ int clamp_slot(int x, int hi)
{
    int r;
    asm("v_med3_i32 %0, %1, 0, %2" : "=v"(r) : "v"(x), "v"(hi));
    return r;
}

// One 4-byte word per lane: lane i's word lands at lds_addr + 4 * i (lds_addr
// wave uniform). It sets M0 itself and declares the clobber, so a later
// gather16_slot has the compiler write M0 again.
__device__ __forceinline__ void gather4_to_lds(const void* src, uint32_t lds_addr)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(m0v)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Chunk permutation of tile row `key`: physical 16-byte slot of logical chunk c
// is c ^ swz(key) (an involution inside each 128-byte band). It spreads both the
// K-operand reads (16 rows, one chunk) and the transposed V-operand reads (4 rows,
// two adjacent chunks) over distinct banks.
__device__ __forceinline__ int swz(int key)
{
    return key & 7;
}

// Items per XCD block: an eighth of the items, rounded up to whole slices when
// a slice has at most 8 row groups.
__host__ __device__ inline int xcd_block(int items, int row_groups)
{
    int per = (items + 7) / 8;
    if (row_groups <= 8)
        per = (per + row_groups - 1) / row_groups * row_groups;
    return per;
}

// Length-balanced slicing, derived on the device from seq_lens by every
// workgroup of both kernels (so they agree without any host round trip):
// every sequence's key positions are cut into slices of c whole tiles, in
// sequence order; slice k of sequence b is global slice start_b + k. With T
// tiles in the batch and G slice slots per row group, c = ceil(T / G') where
// G' = G - (B - 1) when that leaves more than half of G, else G' = G.
// Rounding each sequence up to whole slices adds fewer than B slices, so the
// total stays within G in the first case (one workgroup per slot; for one
// sequence ceil(T / ceil(T / G)) <= G) and within G + B in the second.

// Keys of sequence b: S_b clamped to [N, max_kv].
__device__ __forceinline__ int seq_keys(const Args& a, int b)
{
    return min(max(a.seq_lens[b], a.nodes), a.max_kv);
}

// Tiles of sequence b: its keys in 32-key tiles.
__device__ __forceinline__ int64_t seq_tiles(const Args& a, int b)
{
    return (seq_keys(a, b) + kTileKeys - 1) / kTileKeys;
}

// Sum of v over the workgroup's NT threads; every thread gets it. red holds
// NT/64 words of LDS; the first barrier lets a previous call's readers finish.
template <int NT>
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* red)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    int64_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i)
        t += red[i];
    return t;
}

// Exclusive prefix sum of v over the workgroup's threads in thread order;
// total receives the sum over all of them.
template <int NT>
__device__ __forceinline__ int64_t block_excl_scan(int64_t v, int64_t* red, int64_t& total)
{
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o);
        if (lane >= o)
            x += y;
    }
    __syncthreads();
    if (lane == 63)
        red[w] = x;
    __syncthreads();
    int64_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        if (i < w)
            before += red[i];
        tot += red[i];
    }
    total = tot;
    return before + x - v;
}

// Sum over the 64 lanes of a wave; every lane gets it.
__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o)
            v += y;
    }
    return v;
}

// Batches of at most this many sequences are sliced by every wave on its own
// (one sequence per lane, shuffles only: no LDS, no barrier).
constexpr int kWaveBatch = 64;

// Tiles per slice c and the number of slices of all sequences together.
// sk and tb receive the keys and tiles of one sequence: of the batch's only
// sequence when B = 1 (every thread); of sequence (lane) when B <= 64 (0
// past the batch); of sequence threadIdx.x when B <= NT (0 past the batch);
// else 0. A single sequence takes c from the host (sized for max_kv, so that
// the grid holds exactly its slices) and needs no reduction and no barrier;
// up to 64 sequences need one load per lane and no barrier; up to NT one
// load per thread.
template <int NT>
__device__ __forceinline__ void slicing(const Args& a, int slots, int single_c, int64_t* red,
                                        int64_t& c, int64_t& nslices, int& sk, int64_t& tb)
{
    const int B = a.batch;
    const int target = (slots > 2 * (B - 1)) ? slots - (B - 1) : slots;
    if (__builtin_expect(B == 1, 1)) {  // laid out as the straight-line path
        sk = seq_keys(a, 0);
        const int t1 = (sk + kTileKeys - 1) / kTileKeys;  // < 2^21: 32-bit arithmetic
        tb = t1;
        c = single_c;
        nslices = (t1 + single_c - 1) / single_c;
        return;
    }
    if (B <= kWaveBatch) {
        const int lane = threadIdx.x & 63;
        sk = lane < B ? seq_keys(a, lane) : 0;
        const int t1 = (sk + kTileKeys - 1) / kTileKeys;  // totals < 2^27: 32-bit
        tb = t1;
        const int T = wave_sum(t1);
        const int cc = max(1, (T + target - 1) / target);
        c = cc;
        nslices = wave_sum((t1 + cc - 1) / cc);
        return;
    }
    int64_t t = 0;
    sk = 0;
    tb = 0;
    if (B <= NT) {
        if ((int)threadIdx.x < B) {
            sk = seq_keys(a, threadIdx.x);
            tb = (sk + kTileKeys - 1) / kTileKeys;
        }
        t = tb;
    } else {
        for (int b = threadIdx.x; b < B; b += NT)
            t += seq_tiles(a, b);
    }
    const int64_t T = block_sum<NT>(t, red);
    c = (T + target - 1) / target;
    if (c < 1)
        c = 1;
    int64_t n = 0;
    if (B <= NT) {
        n = (tb + c - 1) / c;
    } else {
        for (int b = threadIdx.x; b < B; b += NT)
            n += (seq_tiles(a, b) + c - 1) / c;
    }
    nslices = block_sum<NT>(n, red);
}

// kPaged selects how a key position finds its pool slot: false, through the
// per-token page table (slot = page_table[b][p]); true, the hybrid layout, in
// which prefix positions go through pages of page_size slots
// (slot = prefix_pages[b][p / page_size] * page_size + p % page_size) and the
// N tree positions through a per-token list (slot = tree_slots[b][p - (S - N)]).
// The two differ only in the index staging below.
//
// kRB is the number of 16-row blocks per wave: 1 (64 rows per workgroup) or 2
// (128 rows: every K and V^T operand read from LDS feeds two MFMAs, and each
// gathered tile serves twice the rows; for MFMA-bound calls with many rows).
// Workgroup group g covers the 64-row groups kRB*g .. kRB*g + kRB - 1, and row
// block rb of wave w holds rows 64 (kRB g + rb) + 16 w .. + 15, so partial
// results keep the one-row-group layout the combine reads.
template <bool kPaged, int kRB>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(Args a, int slots, int single_c,
                                                            int max_slices, int row_groups,
                                                            float scale_log2)
{
    static_assert(kRB == 1 || kRB == 2, "one or two row blocks per wave");
    __shared__ __attribute__((aligned(16))) char s_kv[kStages * kTileBytes];
    __shared__ int s_idx[2][kWinKeys];  // page indices, two windows of 128 tiles

    __shared__ int64_t s_red[kWaves];
    __shared__ int s_hit[3];

    // This batch's slicing (see slicing()): c tiles per slice, nslices in all.
    int64_t c, nslices, tb;
    int sk;
    slicing<kThreads>(a, slots, single_c, s_red, c, nslices, sk, tb);

    // XCD-aware order: workgroups are dealt to the eight XCDs round-robin by
    // id, so ids x, x + 8, x + 16, ... run on XCD x (and share its L2). The
    // (slice, row group) items, slice-major, are cut into eight contiguous
    // blocks, block x on XCD x, so the row groups of one slice run side by
    // side on one XCD and all but the first read the slice's rows from its L2
    // (with at most 8 row groups, blocks hold whole slices). The grid is sized
    // for max_slices; workgroups past this batch's blocks exit here. One
    // sequence is laid out by the host bound (its exact slice count for
    // max_kv keys), so the mapping does not wait for seq_lens.
    const int L = blockIdx.x;
    const int wg_groups = (row_groups + kRB - 1) / kRB;
    const int items = (a.batch == 1 ? max_slices : (int)nslices) * wg_groups;
    const int per_xcd = xcd_block(items, wg_groups);
    const int item = (L & 7) * per_xcd + (L >> 3);
    if ((L >> 3) >= per_xcd || item >= items)
        return;  // the whole workgroup (every value above is uniform)
    const int gslice = item / wg_groups;
    const int grp = item - gslice * wg_groups;  // workgroup group: row groups kRB*grp ..
    const int tid = threadIdx.x;

    // The sequence b holding global slice gslice, its slice index there and
    // its keys S (clamped to [N, max_kv]).
    int b = 0;
    int split = gslice;
    int S = sk;
    if (a.batch == 1 && gslice >= nslices) {
        // A sequence shorter than max_kv: this slice holds none of its keys.
        // Its slots get the empty partial, (max, sum) = (-inf, 0) and O = 0,
        // so that the combine can merge every slice the host planned for
        // max_kv without waiting for seq_lens (stale slots would hold another
        // call's values).
        for (int rg = grp * kRB; rg < min(grp * kRB + kRB, row_groups); ++rg) {
            const size_t pz = (size_t)rg * max_slices + gslice;
            if (tid < kRowsPerGroup) {
                float2* pm = (float2*)a.part_ml + pz * kRowsPerGroup + tid;
                *pm = make_float2(-INFINITY, 0.f);
            }
            uint4* po = (uint4*)((__bf16*)a.part_o + pz * (size_t)(kRowsPerGroup * kPartRowElems));
            for (int i = tid; i < kRowsPerGroup * kPartRowElems * 2 / 16; i += kThreads)
                po[i] = uint4{0u, 0u, 0u, 0u};
        }
        return;  // the whole workgroup
    }
    if (__builtin_expect(a.batch > 1 && a.batch <= kWaveBatch, 0)) {
        // one sequence per lane: the lane whose slice range holds gslice
        const int nl = (int)((tb + c - 1) / c);
        const int incl = wave_incl_scan(nl);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(nl > 0 && gslice >= incl - nl && gslice < incl);
        const int bl = __builtin_ctzll(hit);  // exactly one lane: slices are disjoint
        b = bl;
        split = gslice - (__shfl(incl, bl) - __shfl(nl, bl));
        S = __shfl(sk, bl);
    } else if (__builtin_expect(a.batch > kWaveBatch, 0)) {
        if (tid == 0)
            s_hit[0] = 0, s_hit[1] = 0, s_hit[2] = 0;
        int64_t base = 0;
        for (int b0 = 0; b0 < a.batch; b0 += kThreads) {
            const int bb = b0 + tid;
            int64_t n = 0;
            if (a.batch <= kThreads)
                n = (tb + c - 1) / c;
            else if (bb < a.batch)
                n = (seq_tiles(a, bb) + c - 1) / c;
            int64_t tot;
            const int64_t st = base + block_excl_scan<kThreads>(n, s_red, tot);
            if (n > 0 && gslice >= st && gslice < st + n) {
                s_hit[0] = bb;
                s_hit[1] = (int)(gslice - st);
                s_hit[2] = a.batch <= kThreads ? sk : seq_keys(a, bb);
            }
            base += tot;
        }
        __syncthreads();
        b = s_hit[0];
        split = s_hit[1];
        S = s_hit[2];
    }
    // the same values in every lane (one sequence's length, or LDS words every
    // lane reads): keep them in scalar registers
    b = __builtin_amdgcn_readfirstlane(b);
    split = __builtin_amdgcn_readfirstlane(split);
    S = __builtin_amdgcn_readfirstlane(S);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rl = lane & 15;   // row (and key) within a 16-block
    const int lg = lane >> 4;   // lane group 0..3
    const int N = a.nodes;
    const int H = a.heads;
    const int R = N * H;

    // The workgroup of a sequence's first slice (row group 0) records where the
    // sequence's slices start and how many there are, for the combine.
    if (split == 0 && grp == 0 && tid == 0) {
        const int tiles_b = (S + kTileKeys - 1) / kTileKeys;
        a.seq_slices[2 * b] = gslice;
        a.seq_slices[2 * b + 1] = (int)((tiles_b + c - 1) / c);
    }
    // k0 < S (split < ceil(tiles_b / c)); both uniform, kept in scalar registers
    const int k0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * c * kTileKeys));
    const int nkeys = __builtin_amdgcn_readfirstlane((int)min((int64_t)S - k0, c * kTileKeys));
    const int ntiles = (nkeys + kTileKeys - 1) / kTileKeys;

    // Stage the slice's pool slots in windows of 128 tiles: window w (tiles
    // 128w .. 128w+127) into s_idx[w % 2]. Positions past the end reuse the
    // last valid position's row (finite data, weight zero); slots (and page
    // numbers) are clamped so that no read leaves its buffer. Window 0 is
    // staged here; a slice longer than one window stages window w+1 halfway
    // through window w.
    const int32_t* pt = a.page_table + (int64_t)b * a.max_kv;
    const int maxslot = (int)(a.num_slots - 1);
    const int nwin = (ntiles + kWinTiles - 1) / kWinTiles;
    // Hybrid layout: a prefix position p takes page p / page_size of its row
    // (a page number past the row reads the last entry) plus p % page_size; a
    // tree position takes its tree_slots entry (a shift for a power-of-two
    // page size).
    auto win_len = [&](int w) { return min(ntiles * kTileKeys - w * kWinKeys, kWinKeys); };
    // Window 0 with pages of at least 16 slots: the page entries it spans (at
    // most 258) go straight to LDS, into the index ring's other half (idle
    // until window 1, halfway through window 0), and so do the tree slots
    // when the window reaches the tree block; no registers, so their round
    // trip overlaps Q's loads. expand0 then forms the window's slots from LDS
    // while Q's loads are still in flight: a few positions per thread,
    // against the page arithmetic of sixteen.
    constexpr int kTreeOff = kWinKeys - 64;  // tree slots' place in that half
    auto stage_pages0 = [&]() {
        if constexpr (kPaged) {
            const int n = win_len(0);
            const int ps = a.page_size;
            const int t0 = S - N;
            const int pg0 = k0 / ps;
            const int count = k0 < t0 ? min(k0 + n - 1, t0 - 1) / ps - pg0 + 1 : 0;  // uniform
            const int32_t* prow = a.prefix_pages + (int64_t)b * a.max_pages;
            const uint32_t base = (uint32_t)(uintptr_t)(LDS_AS int*)s_idx[1];
            for (int e = 0; e < count; e += kThreads)
                gather4_to_lds(prow + min(pg0 + min(e + tid, count - 1), a.max_pages - 1),
                               base + (e + wave * 64) * 4);
            if (k0 + n > t0 && wave == 0)  // uniform: the window reaches the tree block
                gather4_to_lds(a.tree_slots + (int64_t)b * N + min(lane, N - 1), base + kTreeOff * 4);
        }
    };
    auto expand0 = [&]() {
        if constexpr (kPaged) {
            const int n = win_len(0);
            const int ps = a.page_size;
            const bool pow2 = (ps & (ps - 1)) == 0;
            const int sh = __builtin_ctz((unsigned)ps);
            const int t0 = S - N;
            const int pg0 = k0 / ps;
            for (int i = tid; i < n; i += kThreads) {
                const int p = min(k0 + i, S - 1);
                int64_t v;
                if (p < t0) {
                    const int pg = pow2 ? (p >> sh) : p / ps;
                    v = (int64_t)s_idx[1][pg - pg0] * ps + (p - pg * ps);
                } else {
                    v = s_idx[1][kTreeOff + (p - t0)];
                }
                s_idx[0][i] = (int)(v < 0 ? 0 : (v > maxslot ? maxslot : v));  // clamped to the pool
            }
        }
    };
    auto stage = [&](int w) {
        const int n = min(ntiles * kTileKeys - w * kWinKeys, kWinKeys);
        if constexpr (kPaged) {
            // Windows after the first, and window 0 with pages under 16 slots:
            // every entry of this thread's positions is loaded first, so the
            // window costs one round trip.
            constexpr int kPer = kWinKeys / kThreads;
            const int ps = a.page_size;
            const bool pow2 = (ps & (ps - 1)) == 0;
            const int sh = __builtin_ctz((unsigned)ps);
            const int t0 = S - N;
            const int32_t* prow = a.prefix_pages + (int64_t)b * a.max_pages;
            const int32_t* trow = a.tree_slots + (int64_t)b * N;
            int32_t e[kPer];
            int off[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                e[j] = 0;
                off[j] = -1;  // -1: a tree position (no page arithmetic)
                if (j * kThreads < n) {  // uniform
                    const int p = min(k0 + w * kWinKeys + min(tid + j * kThreads, n - 1), S - 1);
                    const int32_t* src = trow + (p - t0);
                    if (p < t0) {
                        const int pg = pow2 ? (p >> sh) : p / ps;
                        off[j] = p - pg * ps;
                        src = prow + min(pg, a.max_pages - 1);
                    }
                    e[j] = *src;
                }
            }
            int* dst = s_idx[w & 1];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = tid + j * kThreads;
                if (i < n) {
                    const int64_t v = off[j] >= 0 ? (int64_t)e[j] * ps + off[j] : (int64_t)e[j];
                    dst[i] = (int)(v < 0 ? 0 : (v > maxslot ? maxslot : v));  // clamped to the pool
                }
            }
        } else {
            // Table words go straight to LDS (direct loads, no registers and
            // no wait here): the vmcnt waits of the tile loop, which only
            // follow later loads, cover them, and the barriers publish them.
            // The position is clamped in the address; the slot value when a
            // lane reads it (load_idx).
            const uint32_t dst = (uint32_t)(uintptr_t)(LDS_AS int*)s_idx[w & 1] + wave * 256;
            for (int i = 0; i < n; i += kThreads)
                gather4_to_lds(pt + min(k0 + w * kWinKeys + i + tid, S - 1), dst + i * 4);
        }
    };
    const bool pages0 = kPaged && a.page_size >= 16;  // uniform
    if (pages0)
        stage_pages0();
    else
        stage(0);

    // This lane's query row in each row block: fragments of Q as the B operand
    // of S^T = K.Q^T, and the tree-mask words of the row's node.
    const int W = (N + 31) >> 5;
    bf16x8 qf[kRB][kKSteps];
    uint32_t mw0[kRB], mw1[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int row = (grp * kRB + rb) * kRowsPerGroup + wave * 16 + rl;
        const bool row_ok = row < R;
        const __bf16* qrow = (const __bf16*)a.q + ((int64_t)b * R + (row_ok ? row : 0)) * kDqk;
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            bf16x8 v = *(const bf16x8*)(qrow + (4 * s + lg) * 8);
            if (!row_ok)
                v = bf16x8{};
            qf[rb][s] = v;
        }
        const int node = (row_ok ? row : 0) / H;
        const uint32_t* mrow = a.tree_mask + ((int64_t)b * N + node) * W;
        mw0[rb] = mrow[0];
        mw1[rb] = W > 1 ? mrow[1] : 0u;
    }
    const int tree0 = S - N;  // first key position holding a tree node
    if (pages0) {
        // The page entries are older than Q's 18 loads and the mask words (at
        // least 19 operations, in order), so this waits for the entries only;
        // the expansion then runs while Q's loads are in flight, and the
        // barrier below publishes its slots.
        static_assert(kKSteps == 18, "Q's loads per row block");
        wait_vmcnt<19>();
        __syncthreads();
        expand0();
    }

    const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)s_kv;
    const char* kv = (const char*)a.kv;

    // Gather plan of this lane: wave w fills tile rows 8w..8w+7 with nine
    // wave-wide 1024-byte loads; load j puts lane l's 16 bytes at row
    // kl = (64j + l) / 72, slot (64j + l) % 72, which holds logical chunk
    // slot ^ swz(kl). Every aligned 8-lane group covers one full 128-byte band.
    // With two row blocks the pair is packed in one register (byte offset in
    // the low 16 bits) and passed through an empty asm statement once per tile
    // (opaque_plan), so that the unpacking and the row addresses derived from
    // it are formed in the loop rather than kept live across it: that leaves
    // room for the second block's Q and O.
    // gcs[j]: the byte offset less 1024 (j % 4) (see gather16_slot); packed
    // with the row as (gcs + 3072) | row << 16, the low half non-negative.
    int gkl[kLoadsPerWave];
    int gcs[kLoadsPerWave];
    int gpk[kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
        const int z = j * 64 + lane;
        gkl[j] = z / kChunks;
        gcs[j] = ((z - gkl[j] * kChunks) ^ swz(gkl[j])) * 16 - (j & 3) * 1024;
        gpk[j] = (gcs[j] + 3072) | (gkl[j] << 16);
    }
    auto g_kl = [&](int j) { return kRB == 1 ? gkl[j] : gpk[j] >> 16; };
    // The gather's address less 1024 (j % 4), as an integer: it can lie below
    // the pool's start and is only formed, never read, before the instruction
    // offset is added back.
    const uint64_t kv_addr = (uint64_t)(uintptr_t)kv;
    auto g_src = [&](int j, int slot) {
        return kRB == 1 ? kv_addr + (uint64_t)((int64_t)slot * kRowBytes + gcs[j])
                        : kv_addr - 3072u + (uint64_t)((int64_t)slot * kRowBytes + (gpk[j] & 0xffff));
    };
    auto opaque_plan = [&]() {
        if constexpr (kRB > 1)
            asm volatile(""
                         : "+v"(gpk[0]), "+v"(gpk[1]), "+v"(gpk[2]), "+v"(gpk[3]), "+v"(gpk[4]),
                           "+v"(gpk[5]), "+v"(gpk[6]), "+v"(gpk[7]), "+v"(gpk[8]));
    };
    static_assert(kLoadsPerWave == 9, "opaque_plan names every load of the plan");
    // Page indices of the rows this lane gathers for a tile, read from the ring
    // one tile ahead of the gathers that use them (nothing consumes them before
    // then, so the LDS latency stays off the tile's path). A wave's words were
    // loaded (or, with hybrid paging, written) by other waves' lanes, so what
    // orders them is each loader's vmcnt wait followed by a barrier: the one
    // before the first gathers for window 0, the tile barriers for later ones.
    auto load_idx = [&](int t, int* out) {
        const int* tidx = &s_idx[(t / kWinTiles) & 1][(t % kWinTiles) * kTileKeys + wave * kKeysPerWave];
#pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j)
            out[j] = clamp_slot(tidx[g_kl(j)], maxslot);  // slots clamped to the pool
    };
    auto issue = [&](int t, const int* idx) {
        const uint32_t dst = lds0 + (uint32_t)((t % kStages) * kTileBytes +
                                               wave * (kKeysPerWave * kRowBytes));
#pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j)
            gather16_slot(g_src(j, idx[j]), dst, j);
    };

    // Per-lane LDS byte offsets inside a tile buffer; everything else is an
    // instruction immediate.
    //  K operand (row rl of key block kb, chunk 4s+lg): (s odd ? koff1 : koff0)
    //    + kb*16 rows + 128*(s/2)
    const int fk = swz(rl);
    const int koff0 = rl * kRowBytes + 16 * (lg ^ fk);
    const int koff1 = rl * kRowBytes + 16 * ((4 + lg) ^ fk);
    //  V^T operand (transposed 8-byte reads): lane (lg, rl) reads tile row
    //  4lg + rl/4 (and +16), columns 16cb + 4(rl%4) .. +3, i.e. chunk
    //  2cb + (rl%4)/2, half rl%2: voff[cb%4] + 128*(cb/4) (+16 rows)
    const int vkey = 4 * lg + (rl >> 2);
    const int fv = swz(vkey);
    const int vsel = (rl & 3) >> 1;
    int voff[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        voff[qd] = vkey * kRowBytes + 16 * ((2 * qd + vsel) ^ fv) + (rl & 1) * 8;

    f32x4 o[kRB][kColBlocks];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
            o[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Reference max m_ref (log2 units, shared by the row's four lanes) and this
    // lane's share of the running sum. Weights are 2^(x - m_ref); the reference
    // is raised only when a tile's max exceeds it by more than kSlack, so weights
    // stay below 2^kSlack. Raising it rescales O, which happens outside the
    // steady-state loop (at the first tile and whenever scores jump by more than
    // kSlack), so the hot loop touches O only through MFMA accumulation.
    constexpr float kSlack = 16.0f;
    float m_ref[kRB], l_run[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        m_ref[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }

    // Q fragments and mask words must be in registers, and the first index
    // window in LDS, before the gathers start: past this point the only
    // outstanding vector-memory operations are this wave's gathers (and, on
    // slices longer than a window, the reads of the next window, which the
    // waits below only make stricter).
    wait_vmcnt_lds<0>();  // and the slots expanded in LDS are written
    __syncthreads();      // index window 0 staged
    int idx_n[kLoadsPerWave];  // page indices of the next tile to gather
    load_idx(0, idx_n);
    issue(0, idx_n);
    if (ntiles > 1) {
        load_idx(1, idx_n);
        issue(1, idx_n);
    }

    // K-operand reads per group (double-buffered): groups of 4 give 9 groups,
    // one per row gather of tile t+2 (measured against groups of 6 with the
    // last three gathers in the P.V: 2 % faster on 128 rows, 3-5 % on the
    // MFMA-bound 64 x 64 heads, same elsewhere, bit-identical). With two row
    // blocks, groups of 4 K reads and 4 V column blocks were measured against
    // 1, 2 and 4 of each on the 64 x 64 heads: 2-3 % ahead of (2, 2), 25 %
    // ahead of single K reads.
    constexpr int kKGroup = 4;
    constexpr int kKReads = 2 * kKSteps;  // 36 per tile (two key blocks)
    constexpr int kVGroup = 4;            // column blocks per V-operand group
    constexpr int kKGroups = kKReads / kKGroup;

    // Tile t's rows are in LDS once at most the rows of tile t+1 remain
    // outstanding and every wave has passed the barrier; the barrier also
    // frees the buffer of tile t-1 for the gathers of tile t+2. Halfway
    // through window w (step 128w + 64) the next window is staged into the
    // other half of s_idx, whose last reader (tile 128w - 1) ran at step
    // 128w - 4; later barriers publish it before its first reader (tile
    // 128(w+1), at step 128(w+1) - 3).
    auto next_tile = [&](int t) {
        if (t + 1 < ntiles)
            wait_vmcnt<kLoadsPerWave>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (t % kWinTiles == kWinTiles / 2 && t / kWinTiles + 1 < nwin)
            stage(t / kWinTiles + 1);
        if (t + 2 < ntiles)
            load_idx(t + 2, idx_n);
    };

    // Scores of a tile that reaches the tree block or the end of the sequence
    // get the tree bitmask and the end of the sequence (-inf where hidden).
    auto mask_tail = [&](int base, float (&x)[kRB][8]) {
        if (base + kTileKeys > tree0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int p = base + (k >> 2) * 16 + 4 * lg + (k & 3);
                const int j = p - tree0;
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb) {
                    bool vis = p < tree0;
                    if (p >= tree0 && p < S)
                        vis = (((j < 32) ? mw0[rb] : mw1[rb]) >> (j & 31)) & 1u;
                    if (!vis)
                        x[rb][k] = -INFINITY;
                }
            }
        }
    };

    int t = 0;
    // byte offsets of tile t's buffer and of the one tile t+2 gathers into,
    // (t % 3) and ((t + 2) % 3) buffers, advanced with t
    int cur_off = 0, gat_off = 2 * kTileBytes;
    next_tile(0);
    if constexpr (kRB > 1) {
        // Every row's first reference comes from tile 0's scores, computed
        // once here: leaving the loop to raise a reference makes the compiler
        // move O and much else through memory, and at tile 0 every wave would.
        // The result is that of the raise path (O and the sum are still zero).
        const char LDS_AS* kb0 = (const char LDS_AS*)s_kv + koff0;  // tile 0: buffer 0
        const char LDS_AS* kb1 = (const char LDS_AS*)s_kv + koff1;
        f32x4 sacc[kRB][2];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
            sacc[rb][0] = sacc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < kKReads; ++n) {
            const int s = n >> 1;
            const bf16x8 kfv =
                *(const bf16x8 LDS_AS*)(((s & 1) ? kb1 : kb0) + (n & 1) * 16 * kRowBytes + 128 * (s >> 1));
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
                sacc[rb][n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfv, qf[rb][s], sacc[rb][n & 1], 0, 0, 0);
        }
        float x0[kRB][8];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int k = 0; k < 8; ++k)
                x0[rb][k] = sacc[rb][k >> 2][k & 3] * scale_log2;
        mask_tail(k0, x0);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float m = x0[rb][0];
#pragma unroll
            for (int k = 1; k < 8; ++k)
                m = fmaxf(m, x0[rb][k]);
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            m_ref[rb] = m;
        }
    }
    while (true) {
        float x[kRB][8];
        float mt[kRB];
        // The two-row-block form reloads part of O from scratch here (on entry
        // and after a raise). Waiting for those loads before the tile loop
        // keeps the compiler's own waits for them out of the loop body: there
        // they would run on every tile and, since vector-memory operations
        // retire in order, also drain the row gathers in flight.
        if constexpr (kRB > 1)
            wait_vmcnt<0>();
        for (;;) {
            opaque_plan();
            static_assert(kStages == 3, "the ring offsets rotate over three buffers");
            const char LDS_AS* buf = (const char LDS_AS*)s_kv + cur_off;
            const char LDS_AS* kb0 = buf + koff0;
            const char LDS_AS* kb1 = buf + koff1;
            const int base = k0 + t * kTileKeys;
            // Tile t+2's rows go into the buffer tile t-1 used, spread over
            // this tile's Q.K^T (one per K-operand group; any left over go
            // between V^T groups of the P.V) so that the address unit works
            // while the MFMAs issue. Past the last tile (and when a raised
            // reference makes this tile run again) the same loads go out again
            // from the last staged indices into that free buffer: identical or
            // never-read bytes, rows already in L2, and waits that only get
            // stricter.
            const uint32_t gdst = lds0 + (uint32_t)(gat_off + wave * (kKeysPerWave * kRowBytes));

            // S^T = K.Q^T for key blocks 0 and 1 (keys kb*16 + 4*lg + i against
            // row rl), two interleaved MFMA chains fed by double-buffered groups
            // of LDS reads. Read n covers k-step n/2 of key block n%2.
            auto kptr = [&](int n) {
                const int s = n >> 1;
                return ((s & 1) ? kb1 : kb0) + (n & 1) * 16 * kRowBytes + 128 * (s >> 1);
            };
            bf16x8 kf[2][kKGroup];
#pragma unroll
            for (int j = 0; j < kKGroup; ++j)
                kf[0][j] = *(const bf16x8 LDS_AS*)kptr(j);
            f32x4 sacc[kRB][2];
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
                sacc[rb][0] = sacc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < kKReads / kKGroup; ++g) {
                if (g + 1 < kKReads / kKGroup) {
#pragma unroll
                    for (int j = 0; j < kKGroup; ++j)
                        kf[(g + 1) & 1][j] =
                            *(const bf16x8 LDS_AS*)kptr((g + 1) * kKGroup + j);
                }
                if (g < kLoadsPerWave)
                    gather16_slot(g_src(g, idx_n[g]), gdst, g);
#pragma unroll
                for (int j = 0; j < kKGroup; ++j) {
                    const int n = g * kKGroup + j;
#pragma unroll
                    for (int rb = 0; rb < kRB; ++rb)
                        sacc[rb][n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kf[g & 1][j], qf[rb][n >> 1], sacc[rb][n & 1], 0, 0, 0);
                }
            }

            // first V^T group in flight while the softmax runs
            auto vptr = [&](int cb) { return buf + voff[cb & 3] + 128 * (cb >> 2); };
            bf16x4 vt[2][2 * kVGroup];
#pragma unroll
            for (int c = 0; c < kVGroup; ++c) {
                vt[0][2 * c] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)vptr(c));
                vt[0][2 * c + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (bf16x4 LDS_AS*)(vptr(c) + 16 * kRowBytes));
            }

#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    x[rb][k] = sacc[rb][k >> 2][k & 3] * scale_log2;

            // keep one group of K-operand reads in flight ahead of the Q.K^T MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, kKGroup, 0);
#pragma unroll
            for (int i = 0; i < kKReads - kKGroup; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, kRB, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kKGroup * kRB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVGroup, 0);
            mask_tail(base, x);

            // This lane's largest score per row; whether any exceeds its
            // reference by more than kSlack decides the (rare) rescale. A row's
            // exact max over its four lanes is only formed on that path.
            bool raise = false;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                mt[rb] = x[rb][0];
#pragma unroll
                for (int k = 1; k < 8; ++k)
                    mt[rb] = fmaxf(mt[rb], x[rb][k]);
                raise = raise || mt[rb] > m_ref[rb] + kSlack;
            }
            if (__builtin_amdgcn_ballot_w64(raise) != 0)
                break;  // raise the reference first (outside this loop)

            bf16x8 pb[kRB];
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const float mr = (m_ref[rb] == -INFINITY) ? 0.f : m_ref[rb];
                float psum = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    // hardware 2^x (v_exp_f32): the argument lies in [-inf,
                    // kSlack]; results below the smallest normal float (weights
                    // under 2^-126 of the reference) flush to zero
                    const float pk = __builtin_amdgcn_exp2f(x[rb][k] - mr);
                    psum += pk;
                    pb[rb][k] = (__bf16)pk;
                }
                l_run[rb] += psum;
            }

            // O^T[col][row] += V^T[col][key] . P^T[key][row]; the k order of the
            // MFMA is keys (4lg..4lg+3, 16+4lg..16+4lg+3), matching pb.
#pragma unroll
            for (int g = 0; g < kColBlocks / kVGroup; ++g) {
                if (g + 1 < kColBlocks / kVGroup) {
#pragma unroll
                    for (int c = 0; c < kVGroup; ++c) {
                        const int cb = (g + 1) * kVGroup + c;
                        vt[(g + 1) & 1][2 * c] =
                            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)vptr(cb));
                        vt[(g + 1) & 1][2 * c + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (bf16x4 LDS_AS*)(vptr(cb) + 16 * kRowBytes));
                    }
                }
                {
                    // the gathers the Q.K^T groups did not issue, spread evenly
                    // over the P.V groups
                    constexpr int kRest = kLoadsPerWave > kKGroups ? kLoadsPerWave - kKGroups : 0;
                    constexpr int kVGs = kColBlocks / kVGroup;
#pragma unroll
                    for (int j = kKGroups + g * kRest / kVGs; j < kKGroups + (g + 1) * kRest / kVGs; ++j)
                        gather16_slot(g_src(j, idx_n[j]), gdst, j);
                }
#pragma unroll
                for (int c = 0; c < kVGroup; ++c) {
                    const int cb = g * kVGroup + c;
                    const bf16x8 va = __builtin_shufflevector(
                        vt[g & 1][2 * c], vt[g & 1][2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int rb = 0; rb < kRB; ++rb)
                        o[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rb], o[rb][cb], 0, 0, 0);
                }
            }

            // two transposed V reads per column block's MFMAs, one group ahead
#pragma unroll
            for (int i = 0; i < kColBlocks - kVGroup; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, kRB, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kVGroup * kRB, 1);
            gat_off = cur_off;
            cur_off = cur_off == 2 * kTileBytes ? 0 : cur_off + kTileBytes;
            if (++t >= ntiles) {
                // The two-row-block form leaves straight for the stores: a
                // shared exit with the raise path below would run that path's
                // spill code at the end of every slice.
                if constexpr (kRB > 1)
                    goto slice_done;
                else
                    break;
            }
            next_tile(t);
        }
        if (t >= ntiles)
            break;
        // Some row of this wave outgrew its reference on tile t: raise every
        // row's reference to its running max, rescale, and redo tile t.
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float m = fmaxf(mt[rb], __shfl_xor(mt[rb], 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            const float m_new = fmaxf(m_ref[rb], m);
            const float alpha = (m_ref[rb] == -INFINITY) ? 0.f : exp2f(m_ref[rb] - m_new);
            m_ref[rb] = m_new;
            l_run[rb] *= alpha;
            if constexpr (kRB == 1) {
#pragma unroll
                for (int cb = 0; cb < kColBlocks; ++cb)
                    o[rb][cb] *= alpha;
            } else {
                // O fills every accumulation register here, and a plain
                // multiply makes the compiler move it through memory on every
                // tile; so each value is scaled in place, one accumulation
                // register at a time. No MFMA is in flight on O: the MFMA pipe
                // retires in order and the last Q.K^T result was read before
                // this point, and the next MFMA that reads O follows a whole
                // Q.K^T of the redone tile.
#pragma unroll
                for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float e = o[rb][cb][i];
                        float tmp;
                        asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                                     "v_mul_f32 %1, %1, %2\n\t"
                                     "v_accvgpr_write_b32 %0, %1"
                                     : "+a"(e), "=&v"(tmp)
                                     : "v"(alpha));
                        o[rb][cb][i] = e;
                    }
            }
        }
    }

slice_done:
    // Partial results of this slice, in the register-fragment order.
    // O is stored rounded to bf16 (round to nearest even, relative error at
    // most 2^-8 per element); the combine scales each slice's O by a factor of
    // at most 1, so the merged output carries at most that relative error per
    // slice term. It halves the partial traffic; the running max and sum stay
    // fp32, so the lse is unaffected. The stores are device-scope: written
    // through this XCD's L2 (the combine runs on every XCD and reads past it),
    // so the end of the kernel has no dirty lines to write back. They go out
    // before the wait for the last prefetch gathers, so that the two latencies
    // overlap.
    if constexpr (kRB == 1) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const int rg = grp * kRB + rb;
            float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 16);
            l_tot += __shfl_xor(l_tot, 32);
            const size_t pidx = (size_t)rg * max_slices + gslice;
            __bf16* po = (__bf16*)a.part_o + pidx * (size_t)(kRowsPerGroup * kPartRowElems) +
                         (size_t)wave * (kColBlocks * 64 * 4);
#pragma unroll
            for (int cb = 0; cb < kColBlocks; ++cb) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (__bf16)o[rb][cb][i];
                __hip_atomic_store((uint64_t*)(po + (cb * 64 + lane) * 4), __builtin_bit_cast(uint64_t, v),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (lg == 0) {
                float2* pm = (float2*)a.part_ml + pidx * kRowsPerGroup + wave * 16 + rl;
                __hip_atomic_store((uint64_t*)pm, __builtin_bit_cast(uint64_t, make_float2(m_ref[rb], l_tot)),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // The last prefetch gathers write LDS, so they must land before the
        // workgroup ends. The 32 stores of O are younger than every gather,
        // and vmcnt retires in order: at most 32 outstanding operations means
        // every gather has landed, without waiting for the stores.
        wait_vmcnt<kColBlocks>();
    } else {
        // Every address and (max, sum) pair is formed first and passed through
        // an empty asm, so that whatever the compiler reloads from scratch for
        // them lands before the first store: a reload between stores makes it
        // wait for every store issued before.
        const int g0 = __builtin_amdgcn_readfirstlane(grp * kRB);  // uniform
        uint64_t ml[kRB], pm[kRB], po[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 16);
            l_tot += __shfl_xor(l_tot, 32);
            const size_t pidx = (size_t)(g0 + rb) * max_slices + gslice;
            ml[rb] = __builtin_bit_cast(uint64_t, make_float2(m_ref[rb], l_tot));
            pm[rb] = (uint64_t)((float2*)a.part_ml + pidx * kRowsPerGroup + wave * 16 + rl);
            po[rb] = (uint64_t)((__bf16*)a.part_o + pidx * (size_t)(kRowsPerGroup * kPartRowElems) +
                                (size_t)wave * (kColBlocks * 64 * 4) + lane * 4);
        }
        static_assert(kRB == 2, "the asm below names two row blocks");
        asm volatile("" : "+v"(ml[0]), "+v"(ml[1]), "+v"(pm[0]), "+v"(pm[1]), "+v"(po[0]), "+v"(po[1]));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
            if (g0 + rb < row_groups && lg == 0)  // a last workgroup group may hold one row group
                __hip_atomic_store((uint64_t GLOBAL_AS*)pm[rb], ml[rb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            if (g0 + rb >= row_groups)
                break;  // uniform
#pragma unroll
            for (int cb = 0; cb < kColBlocks; ++cb) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (__bf16)o[rb][cb][i];
                __hip_atomic_store((uint64_t GLOBAL_AS*)po[rb] + cb * 64, __builtin_bit_cast(uint64_t, v),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // As for one row block, the 32 stores of O of the first row block are
        // younger than every gather; with a second one 64 are, and 63 (the
        // counter's limit) leaves the first block's stores in flight too.
        if (g0 + kRB - 1 < row_groups)
            wait_vmcnt<63>();
        else
            wait_vmcnt<kColBlocks>();
    }
}

// Split kernel with the work of one 64-row group divided between two kinds of
// wave, two waves per SIMD (per-token table, one 16-row block per wave):
// - score waves (0..3) hold Q for their 16 rows, stage the index windows,
//   read K from LDS, compute S^T = K.Q^T, mask, keep the running max and sum,
//   and publish the bf16 weights P of a tile in LDS;
// - value waves (4..7) each hold O for all 64 rows and 128 of the 512
//   columns and accumulate O^T += V^T.P^T one tile behind the score waves.
//   Split by
//   columns, each value wave reads a quarter of the tile's V^T and the four
//   row blocks' weights, and each V^T operand feeds four MFMAs: the tile's LDS
//   reads of V fall to a quarter, and LDS bandwidth is what bounds the tile.
// With one wave per SIMD the split kernel issues one instruction every few
// clocks and cannot keep the matrix pipe busy; two waves per SIMD issue side
// by side. After the index staging the arithmetic is that of
// split_kernel<true, 1> (hybrid paging) in the same order, so a per-token call
// and a paged call over the same rows give the same bits.
//
// Wave w of each kind gathers its share of tile rows 8w .. 8w+7: the score
// wave five of the nine 1 KB loads, the value wave four (measured against all
// nine on either kind: the tile is 1-2 % shorter, same bits).
//
// Iteration i (0..ntiles) of both kinds starts at one barrier. Before it, each
// wave has waited for its gathers of tile i (only tile i+1's may still be in
// flight) and the score waves have published P(i-1). After it, the score waves
// work on tile i (ring slot i % 4), the value waves on tile i-1 (slot
// (i-1) % 4), and both gather tile i+2 into slot (i+2) % 4, whose last readers
// (tile i-2) finished before the barrier. P and the rescale flag of tile i use
// buffer i % 2, read by the value waves in iteration i+1.
constexpr int kWsThreads = 512;
constexpr int kWsStages = 4;
constexpr int kWsWinTiles = 16;                       // tiles per staged index window
constexpr int kWsWinKeys = kWsWinTiles * kTileKeys;   // 512 page indices per window
constexpr int kWsScoreLoads = 5;  // of a wave's nine row loads per tile; the value waves issue the rest

// Gather plan of loads J0 .. J1-1 of a wave (wave w fills rows 8w .. 8w+7 of a
// tile): load j puts lane l's 16 bytes at row kl = (64j + l) / 72, chunk
// (64j + l) % 72 (stored at chunk ^ swz(kl)); gcs holds the byte offset less
// 1024 (j % 4), as gather16_slot takes it.
template <int J0, int J1>
__device__ __forceinline__ void ws_plan(int lane, int* gcs, int* gkl)
{
#pragma unroll
    for (int j = J0; j < J1; ++j) {
        const int z = j * 64 + lane;
        gkl[j] = z / kChunks;
        gcs[j] = ((z - gkl[j] * kChunks) ^ swz(gkl[j])) * 16 - (j & 3) * 1024;
    }
}

// Slots of loads J0 .. J1-1 from a tile's 8 staged page indices (clamped to the pool).
template <int J0, int J1>
__device__ __forceinline__ void ws_load_idx(const int* tidx, const int* gkl, int maxslot, int* out)
{
#pragma unroll
    for (int j = J0; j < J1; ++j)
        out[j] = clamp_slot(tidx[gkl[j]], maxslot);
}

__global__ __launch_bounds__(kWsThreads, 1) void split_ws_kernel(Args a, int slots, int single_c,
                                                                 int max_slices, int row_groups,
                                                                 float scale_log2)
{
    __shared__ __attribute__((aligned(16))) char s_kv[kWsStages * kTileBytes];
    __shared__ __attribute__((aligned(16))) int s_idx[2][kWsWinKeys];
    __shared__ __attribute__((aligned(16))) bf16x8 s_p[2][kWaves][64];  // weights of a tile
    __shared__ float s_alpha[2][kWaves][16];  // O rescale factors of a tile's rows
    __shared__ int s_raise[2][kWaves];        // whether a tile rescales O
    __shared__ int64_t s_red[kWsThreads / 64];
    __shared__ int s_hit[3];

    int64_t c, nslices, tb;
    int sk;
    slicing<kWsThreads>(a, slots, single_c, s_red, c, nslices, sk, tb);

    // XCD-aware order, as in split_kernel (one row group per workgroup)
    const int L = blockIdx.x;
    const int items = (a.batch == 1 ? max_slices : (int)nslices) * row_groups;
    const int per_xcd = xcd_block(items, row_groups);
    const int item = (L & 7) * per_xcd + (L >> 3);
    if ((L >> 3) >= per_xcd || item >= items)
        return;  // the whole workgroup (every value above is uniform)
    const int gslice = item / row_groups;
    const int grp = item - gslice * row_groups;
    const int tid = threadIdx.x;

    int b = 0;
    int split = gslice;
    int S = sk;
    if (a.batch == 1 && gslice >= nslices) {
        // past a shorter sequence: the empty partial, (max, sum) = (-inf, 0), O = 0
        const size_t pz = (size_t)grp * max_slices + gslice;
        if (tid < kRowsPerGroup) {
            float2* pm = (float2*)a.part_ml + pz * kRowsPerGroup + tid;
            *pm = make_float2(-INFINITY, 0.f);
        }
        uint4* po = (uint4*)((__bf16*)a.part_o + pz * (size_t)(kRowsPerGroup * kPartRowElems));
        for (int i = tid; i < kRowsPerGroup * kPartRowElems * 2 / 16; i += kWsThreads)
            po[i] = uint4{0u, 0u, 0u, 0u};
        return;  // the whole workgroup
    }
    if (__builtin_expect(a.batch > 1 && a.batch <= kWaveBatch, 0)) {
        const int nl = (int)((tb + c - 1) / c);
        const int incl = wave_incl_scan(nl);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(nl > 0 && gslice >= incl - nl && gslice < incl);
        const int bl = __builtin_ctzll(hit);
        b = bl;
        split = gslice - (__shfl(incl, bl) - __shfl(nl, bl));
        S = __shfl(sk, bl);
    } else if (__builtin_expect(a.batch > kWaveBatch, 0)) {
        if (tid == 0)
            s_hit[0] = 0, s_hit[1] = 0, s_hit[2] = 0;
        int64_t base = 0;
        for (int b0 = 0; b0 < a.batch; b0 += kWsThreads) {
            const int bb = b0 + tid;
            int64_t n = 0;
            if (a.batch <= kWsThreads)
                n = (tb + c - 1) / c;
            else if (bb < a.batch)
                n = (seq_tiles(a, bb) + c - 1) / c;
            int64_t tot;
            const int64_t st = base + block_excl_scan<kWsThreads>(n, s_red, tot);
            if (n > 0 && gslice >= st && gslice < st + n) {
                s_hit[0] = bb;
                s_hit[1] = (int)(gslice - st);
                s_hit[2] = a.batch <= kWsThreads ? sk : seq_keys(a, bb);
            }
            base += tot;
        }
        __syncthreads();
        b = s_hit[0];
        split = s_hit[1];
        S = s_hit[2];
    }
    b = __builtin_amdgcn_readfirstlane(b);
    split = __builtin_amdgcn_readfirstlane(split);
    S = __builtin_amdgcn_readfirstlane(S);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool score = wave < kWaves;  // uniform
    const int rw = wave & (kWaves - 1);  // 16-row block of this wave
    const int rl = lane & 15;
    const int lg = lane >> 4;
    const int N = a.nodes;
    const int H = a.heads;
    const int R = N * H;

    if (split == 0 && grp == 0 && tid == 0) {
        const int tiles_b = (S + kTileKeys - 1) / kTileKeys;
        a.seq_slices[2 * b] = gslice;
        a.seq_slices[2 * b + 1] = (int)((tiles_b + c - 1) / c);
    }
    const int k0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * c * kTileKeys));
    const int nkeys = __builtin_amdgcn_readfirstlane((int)min((int64_t)S - k0, c * kTileKeys));
    const int ntiles = (nkeys + kTileKeys - 1) / kTileKeys;

    // Index windows of 16 tiles: window w into s_idx[w % 2], staged by the score
    // waves: window 0 before the first barrier, window w+1 at iteration 16w + 4,
    // when the last reader of that half (tile 16w - 1, read at iteration
    // 16w - 4) is past, and well before its first reader (iteration 16w + 13).
    const int32_t* pt = a.page_table + (int64_t)b * a.max_kv;
    const int maxslot = (int)(a.num_slots - 1);
    const int nwin = (ntiles + kWsWinTiles - 1) / kWsWinTiles;
    auto stage_win = [&](int w) {  // score waves only
        const int n = min(ntiles * kTileKeys - w * kWsWinKeys, kWsWinKeys);
        const uint32_t dst = (uint32_t)(uintptr_t)(LDS_AS int*)s_idx[w & 1] + rw * 256;
        for (int i = 0; i < n; i += kWaves * 64)
            gather4_to_lds(pt + min(k0 + w * kWsWinKeys + i + rw * 64 + lane, S - 1), dst + i * 4);
    };

    const int tree0 = S - N;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)s_kv;
    const uint64_t kv_addr = (uint64_t)(uintptr_t)a.kv;
    auto slot_lds = [&](int t) {  // this wave's rows of ring slot t % 4
        return lds0 + (uint32_t)((t % kWsStages) * kTileBytes + rw * (kKeysPerWave * kRowBytes));
    };

    if (score) {
        // ------------------------------------------------ score waves
        // Q fragments and tree-mask words of this lane's row; index window 0
        // (this kind stages the windows, gathers the rows and waits for them)
        const int W = (N + 31) >> 5;
        const int row = grp * kRowsPerGroup + rw * 16 + rl;
        bf16x8 qf[kKSteps];
        uint32_t mw0, mw1;
        stage_win(0);
        {
            const bool row_ok = row < R;
            const __bf16* qrow = (const __bf16*)a.q + ((int64_t)b * R + (row_ok ? row : 0)) * kDqk;
#pragma unroll
            for (int s = 0; s < kKSteps; ++s) {
                bf16x8 v = *(const bf16x8*)(qrow + (4 * s + lg) * 8);
                if (!row_ok)
                    v = bf16x8{};
                qf[s] = v;
            }
            const int node = (row_ok ? row : 0) / H;
            const uint32_t* mrow = a.tree_mask + ((int64_t)b * N + node) * W;
            mw0 = mrow[0];
            mw1 = W > 1 ? mrow[1] : 0u;
        }
        wait_vmcnt<0>();
        __syncthreads();  // index window 0 staged

        // This kind's row loads: 0 .. kWsScoreLoads-1 of the wave's nine.
        // Gathers go out for every iteration; past the last tile they repeat the
        // last staged indices into a free slot (rows already fetched, never
        // read), which keeps one wait count for every iteration.
        constexpr int kJ1 = kWsScoreLoads;
        int gcs[kLoadsPerWave], gkl[kLoadsPerWave], idx_n[kLoadsPerWave];
        ws_plan<0, kJ1>(lane, gcs, gkl);
        auto g_src = [&](int j, int slot) { return kv_addr + (uint64_t)((int64_t)slot * kRowBytes + gcs[j]); };
        auto load_idx = [&](int t) {
            ws_load_idx<0, kJ1>(&s_idx[(t / kWsWinTiles) & 1][(t % kWsWinTiles) * kTileKeys + rw * kKeysPerWave],
                                gkl, maxslot, idx_n);
        };
        load_idx(0);
#pragma unroll
        for (int j = 0; j < kJ1; ++j)
            gather16_slot(g_src(j, idx_n[j]), slot_lds(0), j);
        if (ntiles > 1)
            load_idx(1);
#pragma unroll
        for (int j = 0; j < kJ1; ++j)
            gather16_slot(g_src(j, idx_n[j]), slot_lds(1), j);
        if (ntiles > 2)
            load_idx(2);

        const int fk = swz(rl);
        const int koff0 = rl * kRowBytes + 16 * (lg ^ fk);
        const int koff1 = rl * kRowBytes + 16 * ((4 + lg) ^ fk);
        constexpr float kSlack = 16.0f;
        float m_ref = -INFINITY, l_run = 0.f;
        constexpr int kKGroup = 4;
        constexpr int kKReads = 2 * kKSteps;
        static_assert(kKReads / kKGroup >= kJ1, "at most one gather per K-operand group");
        int cur_off = 0;
        for (int i = 0; i <= ntiles; ++i) {
            // this kind's rows of tile i landed (only tile i+1's gathers may
            // be in flight) and P(i-1) with its rescale flag and factors is
            // written; the value waves are past P(i-2)
            wait_vmcnt_lds<kJ1>();
            __syncthreads();
            if (i == ntiles)
                break;
            if (i % kWsWinTiles == 4 && i / kWsWinTiles + 1 < nwin)
                stage_win(i / kWsWinTiles + 1);
            const uint32_t gdst = slot_lds(i + 2);
            const char LDS_AS* buf = (const char LDS_AS*)s_kv + cur_off;
            const char LDS_AS* kb0 = buf + koff0;
            const char LDS_AS* kb1 = buf + koff1;
            const int base = k0 + i * kTileKeys;
            auto kptr = [&](int n) {
                const int s = n >> 1;
                return ((s & 1) ? kb1 : kb0) + (n & 1) * 16 * kRowBytes + 128 * (s >> 1);
            };
            bf16x8 kf[2][kKGroup];
#pragma unroll
            for (int j = 0; j < kKGroup; ++j)
                kf[0][j] = *(const bf16x8 LDS_AS*)kptr(j);
            f32x4 sacc[2];
            sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < kKReads / kKGroup; ++g) {
                if (g + 1 < kKReads / kKGroup) {
#pragma unroll
                    for (int j = 0; j < kKGroup; ++j)
                        kf[(g + 1) & 1][j] = *(const bf16x8 LDS_AS*)kptr((g + 1) * kKGroup + j);
                }
                // gather g of tile i+2 (into the slot tile i-2 used)
                if (g < kJ1)
                    gather16_slot(g_src(g, idx_n[g]), gdst, g);
#pragma unroll
                for (int j = 0; j < kKGroup; ++j) {
                    const int n = g * kKGroup + j;
                    sacc[n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[g & 1][j], qf[n >> 1], sacc[n & 1], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, kKGroup, 0);
#pragma unroll
            for (int q = 0; q < kKReads - kKGroup; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kKGroup, 0);
            float x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                x[k] = sacc[k >> 2][k & 3] * scale_log2;
            if (base + kTileKeys > tree0) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int p = base + (k >> 2) * 16 + 4 * lg + (k & 3);
                    const int j = p - tree0;
                    bool vis = p < tree0;
                    if (p >= tree0 && p < S)
                        vis = (((j < 32) ? mw0 : mw1) >> (j & 31)) & 1u;
                    if (!vis)
                        x[k] = -INFINITY;
                }
            }
            float mt = x[0];
#pragma unroll
            for (int k = 1; k < 8; ++k)
                mt = fmaxf(mt, x[k]);
            const int pb_i = i & 1;
            int raised = 0;
            if (__builtin_amdgcn_ballot_w64(mt > m_ref + kSlack) != 0) {
                // raise every row's reference to its running max; O is
                // rescaled by the value waves before they add this tile
                float m = fmaxf(mt, __shfl_xor(mt, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                const float m_new = fmaxf(m_ref, m);
                const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - m_new);
                m_ref = m_new;
                l_run *= alpha;
                if (lg == 0)
                    s_alpha[pb_i][rw][rl] = alpha;
                raised = 1;
            }
            if (lane == 0)
                s_raise[pb_i][rw] = raised;
            bf16x8 pb;
            {
                const float mr = (m_ref == -INFINITY) ? 0.f : m_ref;
                float psum = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float pk = __builtin_amdgcn_exp2f(x[k] - mr);
                    psum += pk;
                    pb[k] = (__bf16)pk;
                }
                l_run += psum;
            }
            s_p[pb_i][rw][lane] = pb;
            if (i + 3 < ntiles)
                load_idx(i + 3);
            cur_off = cur_off == (kWsStages - 1) * kTileBytes ? 0 : cur_off + kTileBytes;
        }
        // this slice's (max, sum) per row; the last (repeated) gathers land
        // first, so that no LDS write outlives the workgroup
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        wait_vmcnt<0>();
        if (lg == 0) {
            const size_t pidx = (size_t)grp * max_slices + gslice;
            float2* pm = (float2*)a.part_ml + pidx * kRowsPerGroup + rw * 16 + rl;
            __hip_atomic_store((uint64_t*)pm, __builtin_bit_cast(uint64_t, make_float2(m_ref, l_tot)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }

    // ---------------------------------------------------- value waves
    __syncthreads();  // index window 0 staged
    // This kind's row loads: kWsScoreLoads .. 8 of the wave's nine, two tiles
    // ahead like the score waves' (and repeated past the last tile alike).
    constexpr int kJ0 = kWsScoreLoads;
    constexpr int kVLoads = kLoadsPerWave - kJ0;
    int gcs[kLoadsPerWave], gkl[kLoadsPerWave], idx_n[kLoadsPerWave];
    ws_plan<kJ0, kLoadsPerWave>(lane, gcs, gkl);
    auto g_src = [&](int j, int slot) { return kv_addr + (uint64_t)((int64_t)slot * kRowBytes + gcs[j]); };
    auto load_idx = [&](int t) {
        ws_load_idx<kJ0, kLoadsPerWave>(
            &s_idx[(t / kWsWinTiles) & 1][(t % kWsWinTiles) * kTileKeys + rw * kKeysPerWave], gkl, maxslot, idx_n);
    };
    load_idx(0);
#pragma unroll
    for (int j = kJ0; j < kLoadsPerWave; ++j)
        gather16_slot(g_src(j, idx_n[j]), slot_lds(0), j);
    if (ntiles > 1)
        load_idx(1);
#pragma unroll
    for (int j = kJ0; j < kLoadsPerWave; ++j)
        gather16_slot(g_src(j, idx_n[j]), slot_lds(1), j);
    if (ntiles > 2)
        load_idx(2);
    const int vkey = 4 * lg + (rl >> 2);
    const int fv = swz(vkey);
    const int vsel = (rl & 3) >> 1;
    int voff[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        voff[qd] = vkey * kRowBytes + 16 * ((2 * qd + vsel) ^ fv) + (rl & 1) * 8;
    // O^T of this wave's columns: column block cb0 + c (c = 0..7) for row block r
    constexpr int kWsCols = kColBlocks / kWaves;  // 8 column blocks per value wave
    const int cb0 = rw * kWsCols;
    f32x4 o[kWaves][kWsCols];
#pragma unroll
    for (int r = 0; r < kWaves; ++r)
#pragma unroll
        for (int c = 0; c < kWsCols; ++c)
            o[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // iteration 0: the score waves work on tile 0; this kind gathers tile 2
    wait_vmcnt<kVLoads>();
    __syncthreads();
#pragma unroll
    for (int j = kJ0; j < kLoadsPerWave; ++j)
        gather16_slot(g_src(j, idx_n[j]), slot_lds(2), j);
    if (3 < ntiles)
        load_idx(3);
    for (int i = 1; i <= ntiles; ++i) {
        // this kind's rows of tile i landed (only tile i+1's may be in flight)
        wait_vmcnt<kVLoads>();
        __syncthreads();  // P(i-1) published
        const uint32_t gdst = slot_lds(i + 2);
        // P.V of tile i-1, after the rescales its scores asked for (rare);
        // each value is multiplied in place, so that O keeps its registers.
        const int pb_i = (i - 1) & 1;
#pragma unroll
        for (int r = 0; r < kWaves; ++r) {
            if (__builtin_amdgcn_readfirstlane(s_raise[pb_i][r]) != 0) {
                const float alpha = s_alpha[pb_i][r][rl];
#pragma unroll
                for (int c = 0; c < kWsCols; ++c)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float e = o[r][c][k];
                        asm volatile("v_mul_f32 %0, %0, %1" : "+v"(e) : "v"(alpha));
                        o[r][c][k] = e;
                    }
            }
        }
        bf16x8 pb[kWaves];
#pragma unroll
        for (int r = 0; r < kWaves; ++r)
            pb[r] = s_p[pb_i][r][lane];
        const char LDS_AS* buf = (const char LDS_AS*)s_kv + ((i - 1) % kWsStages) * kTileBytes;
        auto vptr = [&](int cb) { return buf + voff[cb & 3] + 128 * (cb >> 2); };
        // V^T operands two column blocks ahead of their MFMAs
        bf16x4 vt[3][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            vt[c][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)vptr(cb0 + c));
            vt[c][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)(vptr(cb0 + c) + 16 * kRowBytes));
        }
#pragma unroll
        for (int c = 0; c < kWsCols; ++c) {
            if (c + 2 < kWsCols) {
                vt[(c + 2) % 3][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)vptr(cb0 + c + 2));
                vt[(c + 2) % 3][1] =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)(vptr(cb0 + c + 2) + 16 * kRowBytes));
            }
            const bf16x8 va = __builtin_shufflevector(vt[c % 3][0], vt[c % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
            // this kind's gathers of tile i+2 (into the slot tile i-2 used),
            // spread over the column blocks
#pragma unroll
            for (int j = kJ0 + c * kVLoads / kWsCols; j < kJ0 + (c + 1) * kVLoads / kWsCols; ++j)
                gather16_slot(g_src(j, idx_n[j]), gdst, j);
#pragma unroll
            for (int r = 0; r < kWaves; ++r)
                o[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[r], o[r][c], 0, 0, 0);
        }
        if (i + 3 < ntiles)
            load_idx(i + 3);
    }
    // this slice's O, rounded to bf16, in the register-fragment order of the
    // row blocks
    const size_t pidx = (size_t)grp * max_slices + gslice;
#pragma unroll
    for (int r = 0; r < kWaves; ++r) {
        __bf16* po = (__bf16*)a.part_o + pidx * (size_t)(kRowsPerGroup * kPartRowElems) +
                     (size_t)r * (kColBlocks * 64 * 4);
#pragma unroll
        for (int c = 0; c < kWsCols; ++c) {
            bf16x4 v;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[k] = (__bf16)o[r][c][k];
            __hip_atomic_store((uint64_t*)(po + ((cb0 + c) * 64 + lane) * 4), __builtin_bit_cast(uint64_t, v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // The last (repeated) gathers write LDS, so they land before the
    // workgroup ends; the 32 stores are younger, and vmcnt retires in order.
    wait_vmcnt<kWaves * kWsCols>();
}

// Merge of one (sequence b, 16-row block rb, group xblk of column units) by
// the workgroup's 8 waves. A unit is a 16-column block (kVals = 4: a lane
// holds the 4 values of one fragment lane) or half of one (kVals = 2: 8
// columns, 2 values per lane, twice the waves for the same data; used for one
// sequence with many slices, where the slices rather than the rows are the
// work). `wpc` waves share each unit (1, 2, 4 or 8, from the sequence's slice
// count). A wave takes every wpc-th of the sequence's nvalid slices (from
// batch slice `start` on), loads kUnroll of them at once and folds them into
// its running (max, sum, weighted sum) with one exp per slice against the
// round's max. The waves of a unit then merge through LDS, and the first of
// them writes the bf16 output and, for column block 0, the lse. Every wave
// passes the one barrier inside.
template <int kVals>
struct CombineSmem {
    typedef float fvec __attribute__((ext_vector_type(kVals)));
    float m[kCombineWaves][64];
    float l[kCombineWaves][64];
    fvec o[kCombineWaves][64];
};

template <int kVals, bool kZeroEmpty>
__device__ __forceinline__ void combine_unit(const Args& a, CombineSmem<kVals>& sm, int b, int rb, int xblk,
                                             int64_t start, int nvalid, int wpc, int max_slices)
{
    constexpr int kUnroll = kVals == 2 ? 32 : 16;   // slices in flight per wave
    typedef float fvec __attribute__((ext_vector_type(kVals)));
    typedef __bf16 bvec __attribute__((ext_vector_type(kVals)));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = rb >> 2;
    const int w = rb & 3;
    const int R = a.nodes * a.heads;
    const int unit = xblk * (kCombineWaves / wpc) + wave / wpc;
    const int sub = wave % wpc;          // this wave's share of the slices
    // column block, fragment lane of the split kernel's O^T layout, and the
    // first of this lane's values in it
    const int cb = kVals == 4 ? unit : unit >> 1;
    const int fl = kVals == 4 ? lane : 32 * (unit & 1) + (lane >> 1);
    const int v0 = kVals == 4 ? 0 : 2 * (lane & 1);
    const int rl = fl & 15;
    const int row = grp * kRowsPerGroup + w * 16 + rl;

    const size_t pbase = (size_t)grp * max_slices + (size_t)start;
    const float2* pml = (const float2*)a.part_ml + pbase * kRowsPerGroup + w * 16 + rl;
    const __bf16* pob = (const __bf16*)a.part_o + pbase * (size_t)(kRowsPerGroup * kPartRowElems) +
                        (size_t)w * (kColBlocks * 64 * 4) + (cb * 64 + fl) * 4 + v0;

    float M = -INFINITY;
    float L = 0.f;
    fvec acc = fvec{};
    for (int s0 = sub; s0 < nvalid; s0 += wpc * kUnroll) {
        float2 ml[kUnroll];
        bvec ov[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int s = s0 + u * wpc;
            const size_t ss = s < nvalid ? (size_t)s : 0;
            ml[u] = pml[ss * kRowsPerGroup];
            ov[u] = *(const bvec*)(pob + ss * (kRowsPerGroup * kPartRowElems));
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (s0 + u * wpc >= nvalid)
                ml[u] = make_float2(-INFINITY, 0.f);  // past the sequence: weight 0
            // A slice with no visible key has O = 0 already. Selecting it
            // explicitly changes how the compiler orders the loads, which is
            // measured faster in the batch combine (11.3 -> 9.7 us, batch 8)
            // and not in the one-sequence grid.
            if (kZeroEmpty && ml[u].x == -INFINITY)
                ov[u] = bvec{};
            mx = fmaxf(mx, ml[u].x);
        }
        if (mx == -INFINITY)
            continue;  // nothing visible to this row so far
        const float ca = exp2f(M - mx);  // 0 while M is still -inf
        L *= ca;
        acc *= ca;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // a slice that saw nothing has (m, l, o) = (-inf, 0, 0): weight 0
            const float cs = exp2f(ml[u].x - mx);
            L += ml[u].y * cs;
#pragma unroll
            for (int i = 0; i < kVals; ++i)
                acc[i] += (float)ov[u][i] * cs;
        }
        M = mx;
    }
    sm.m[wave][lane] = M;
    sm.l[wave][lane] = L;
    sm.o[wave][lane] = acc;
    __syncthreads();
    if (sub != 0)
        return;
    float Mt = sm.m[wave][lane];
    for (int k = 1; k < wpc; ++k)
        Mt = fmaxf(Mt, sm.m[wave + k][lane]);
    const float mref = (Mt == -INFINITY) ? 0.f : Mt;
    float Lt = 0.f;
    fvec ot = fvec{};
    for (int k = 0; k < wpc; ++k) {
        const float c = exp2f(sm.m[wave + k][lane] - mref);  // 0 for waves that saw nothing
        Lt += sm.l[wave + k][lane] * c;
        ot += sm.o[wave + k][lane] * c;
    }
    if (row >= R)
        return;
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    bvec v;
#pragma unroll
    for (int i = 0; i < kVals; ++i)
        v[i] = (__bf16)(ot[i] * inv);
    __bf16* orow = (__bf16*)a.out + ((size_t)b * R + row) * kDv;
    *(bvec*)(orow + 16 * cb + 4 * (fl >> 4) + v0) = v;
    if (cb == 0 && fl < 16 && v0 == 0)
        a.lse[(size_t)b * R + row] = Lt > 0.f ? (Mt + log2f(Lt)) * kLn2 : -INFINITY;
}

// Waves per column unit for a sequence of nvalid slices: enough that a wave
// loads at most one round of slices.
template <int kVals>
__device__ __forceinline__ int combine_wpc(int nvalid)
{
    constexpr int kUnroll = kVals == 2 ? 32 : 16;
    int wpc = 1;
    while (wpc < kCombineWaves && wpc * kUnroll < nvalid)
        wpc *= 2;
    return wpc;
}

// kLoop = false: one workgroup per (sequence, 16-row block, group of column
// units); the grid is sized for the most waves per unit a sequence can need,
// and workgroups a sequence does not need exit at once.
// kLoop = true (batches of 2..64 sequences): a fixed grid whose workgroups
// walk the (sequence, 16-row block, group) items the batch actually needs,
// numbered sequence by sequence. Every workgroup derives the count of each
// sequence from the slice table the split kernel recorded (one sequence per
// lane of each wave, with a scan and a ballot), so no workgroup is launched
// only to exit; a grid sized for the worst case had spent most of the batch
// combine dispatching such workgroups.
template <int kVals, bool kLoop>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(Args a, int single_c, int max_slices,
                                                                   int row_groups)
{
    constexpr int kUnits = kColBlocks * 4 / kVals;  // units per 16-row block
    __shared__ CombineSmem<kVals> sm;
    if constexpr (!kLoop) {
        const int b = blockIdx.z;
        // This sequence's slices: nvalid of them, from batch slice start on.
        // One sequence has the host's slicing (for max_kv, known before any
        // load); in a batch, the split kernel recorded each sequence's range
        // in the workspace.
        int64_t start = 0;
        int nvalid;
        if (a.batch == 1) {
            // every slice the host planned for max_kv: those past a shorter
            // sequence hold (-inf, 0), written by the split kernel
            nvalid = max_slices;
        } else {
            start = a.seq_slices[2 * b];
            nvalid = a.seq_slices[2 * b + 1];
        }
        nvalid = __builtin_amdgcn_readfirstlane(nvalid);
        const int wpc = combine_wpc<kVals>(nvalid);
        if ((int)blockIdx.x >= kUnits * wpc / kCombineWaves)
            return;  // the whole workgroup (uniform)
        combine_unit<kVals, false>(a, sm, b, blockIdx.y, blockIdx.x, start, nvalid, wpc, max_slices);
    } else {
        const int lane = threadIdx.x & 63;
        const int rbs = row_groups * 4;  // 16-row blocks per sequence
        int st = 0, nv = 0, items = 0, wpc_l = 1;
        if (lane < a.batch) {
            st = a.seq_slices[2 * lane];
            nv = a.seq_slices[2 * lane + 1];
            wpc_l = combine_wpc<kVals>(nv);
            items = rbs * (kUnits * wpc_l / kCombineWaves);
        }
        const int incl = wave_incl_scan(items);
        const int total = __shfl(incl, 63);
        for (int item = blockIdx.x; item < total; item += gridDim.x) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(items > 0 && item >= incl - items && item < incl);
            const int b = __builtin_ctzll(hit);  // exactly one lane: the ranges are disjoint
            const int local = item - (__shfl(incl, b) - __shfl(items, b));
            const int wpc = __builtin_amdgcn_readfirstlane(__shfl(wpc_l, b));
            const int per = kUnits * wpc / kCombineWaves;  // workgroup items per 16-row block
            combine_unit<kVals, true>(a, sm, b, local / per, local % per, __shfl(st, b),
                                __builtin_amdgcn_readfirstlane(__shfl(nv, b)), wpc, max_slices);
            __syncthreads();  // the next item reuses the LDS
        }
    }
}

}  // namespace

hipError_t launch_split(const Plan& p, const Args& a, hipStream_t stream)
{
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int wg_groups = (p.row_groups + p.rb - 1) / p.rb;
    const int per_xcd = xcd_block(p.max_slices * wg_groups, wg_groups);
    // two row blocks per wave only with per-token tables (the plan never
    // pairs them with the hybrid layout)
    if (p.rb == 2 && a.prefix_pages)
        return hipErrorInvalidValue;
    // one row block per wave with a per-token table: score and value waves,
    // two per SIMD
    if (p.rb == 1 && !a.prefix_pages) {
        hipLaunchKernelGGL(split_ws_kernel, dim3(8 * per_xcd), dim3(kWsThreads), 0, stream, a, p.slots,
                           p.single_c, p.max_slices, p.row_groups, scale_log2);
        return hipGetLastError();
    }
    auto kernel = p.rb == 2 ? split_kernel<false, 2> : split_kernel<true, 1>;
    hipLaunchKernelGGL(kernel, dim3(8 * per_xcd),
                       dim3(kThreads), 0, stream, a, p.slots, p.single_c, p.max_slices, p.row_groups,
                       scale_log2);
    return hipGetLastError();
}

hipError_t launch_combine(const Plan& p, const Args& a, hipStream_t stream)
{
    // One sequence with many slices: half column blocks (twice the waves, 32
    // slices in flight each); otherwise whole column blocks (16 in flight).
    if (a.batch > 1 && a.batch <= 64) {
        // two resident workgroups per compute unit walk the batch's items
        hipLaunchKernelGGL((combine_kernel<4, true>), dim3(2 * p.cus), dim3(kCombineThreads), 0, stream, a,
                           p.single_c, p.max_slices, p.row_groups);
        return hipGetLastError();
    }
    // The grid is sized for the most waves per unit a sequence can need (it
    // has at most `slots` slices); each workgroup picks its sequence's count.
    const bool half = a.batch == 1 && p.splits > 32;
    const int unroll = half ? 32 : 16;
    const int units = half ? 2 * kColBlocks : kColBlocks;
    int wpc = 1;
    while (wpc < kCombineWaves && wpc * unroll < p.slots)
        wpc *= 2;
    hipLaunchKernelGGL((half ? combine_kernel<2, false> : combine_kernel<4, false>),
                       dim3(units * wpc / kCombineWaves, p.row_groups * 4, a.batch), dim3(kCombineThreads), 0,
                       stream, a, p.single_c, p.max_slices, p.row_groups);
    return hipGetLastError();
}

}  // namespace mtv
