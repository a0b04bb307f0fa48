// Internal interface between the host API (mtv_api.cpp) and the kernels
// (mtv_kernels.hip). Not installed; not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace mtv {

constexpr int kDqk = 576;          // key / absorbed query width
constexpr int kDv = 512;           // value width (the latent)
constexpr int kRowBytes = kDqk * 2;
constexpr int kTileKeys = 32;      // keys per LDS tile
constexpr int kRowsPerGroup = 64;  // query rows per row group (4 waves x 16)
// Two row groups per split workgroup from 16 row groups and 48 tiles per
// slice, or from 8 row groups and 64 tiles per slice.
constexpr int kRB2MinRowGroups = 8;
constexpr int kRB2MinTiles(int row_groups) { return row_groups >= 16 ? 48 : 64; }

// How one call is cut into workgroups. Depends only on host values.
struct Plan {
    int rows;          // R = N * H query rows per sequence
    int cus;           // compute units of the device the plan is for
    int row_groups;    // ceil(R / 64)
    int rb;            // row groups per split workgroup (16-row blocks per wave): 1 or 2
    int slots;         // G: target key slices per split workgroup group over the whole batch
    int max_slices;    // G + B: bound on the slices of all sequences together
    int single_c;      // tiles per slice of a batch of one sequence (from max_kv)
    int splits;        // slices per sequence when every sequence holds max_kv keys
    int chunk;         // keys per slice in that case, a multiple of kTileKeys
    size_t part_o_off, part_ml_off, seq_off, bytes;  // workspace layout
};

struct Args {
    const void* q;
    const void* kv;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const uint32_t* tree_mask;
    float scale;
    void* out;
    float* lse;
    uint16_t* part_o;  // bf16 [row group][batch slice][64 rows as 4 waves x 32 col-blocks x 64 lanes x 4]
    float* part_ml;    // [row group][batch slice][64 rows][2]  (running max in log2 units, sum)
    int32_t* seq_slices;  // [B][2]: first batch slice and slice count of each sequence
    int batch, nodes, heads, max_kv;
    int64_t num_slots;
    // hybrid paging (NULL prefix_pages: the per-token page_table is used)
    const int32_t* prefix_pages;  // [B][max_pages] pages of page_size slots
    const int32_t* tree_slots;    // [B][N] slot of each tree node
    int page_size, max_pages;
};

// Arguments of the KV-row moves (accepted-path commit, whole-sequence move).
struct KvArgs {
    int batch, nodes, max_kv;
    int64_t num_slots;
    void* kv;
    int32_t* page_table;
    const int32_t* seq_lens;
    const int32_t* accept_len;  // commit only
    const int32_t* path;        // commit only
    const int32_t* base;
};

hipError_t launch_split(const Plan& plan, const Args& a, hipStream_t stream);
hipError_t launch_combine(const Plan& plan, const Args& a, hipStream_t stream);
hipError_t launch_tree_mask(int batch, int nodes, const int32_t* parents, uint32_t* mask,
                            hipStream_t stream);
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t stream);
hipError_t launch_kv_move(const KvArgs& a, int cus, hipStream_t stream);

// Counters written by the input check: out-of-range sequence lengths, table
// entries, and mask rows with bits past the last node.
constexpr int kCheckCounts = 3;
hipError_t launch_check_inputs(int batch, int nodes, int max_kv, int64_t num_slots,
                               const int32_t* page_table, const int32_t* seq_lens,
                               const uint32_t* mask, unsigned long long* counts, int cus,
                               hipStream_t stream);

}  // namespace mtv
