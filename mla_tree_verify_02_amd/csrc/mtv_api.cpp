// Host side of the C ABI: argument validation, the split plan, workspace
// layout and the two launches. Never allocates, frees or synchronises.
#include <atomic>
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "mla_tree_verify.h"
#include "mtv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // zero-initialised: unknown

// Compute units of the current device, cached per device id.
int current_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return -1;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0)
        return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
        return -1;
    g_cu_count[dev].store(c, std::memory_order_relaxed);
    return c;
}

bool shape_ok(const mtv_shape& s)
{
    if (s.batch < 1 || s.batch > MTV_MAX_BATCH)
        return false;
    if (s.num_nodes < 1 || s.num_nodes > MTV_MAX_NODES)
        return false;
    if (s.num_heads < 1 || (int64_t)s.num_nodes * s.num_heads > 65536)
        return false;
    if (s.max_kv < s.num_nodes || s.max_kv > MTV_MAX_KV)
        return false;
    if (s.num_slots < 1 || s.num_slots > INT32_MAX)
        return false;
    return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The plan: enough slices per sequence that the batch's (sequence, row group)
// pairs give about one workgroup per compute unit, each slice a whole number of
// 32-key tiles.
// The batch's key positions are cut into slices of c whole tiles, one c for
// every sequence, sized from the total: G slice slots per row group (about
// one workgroup per compute unit), c = ceil(T / G') for T tiles in the batch
// with G' = G - (B - 1) when that is at least G / 2 (else G), so the slices of
// all sequences number at most G (at most G + B in the other case) and none
// is longer than the others. The kernels derive c and each slice's sequence
// from seq_lens on the device; the host only bounds the slice count for the
// grid and the workspace.
mtv::Plan make_plan_rb(const mtv_shape& s, int cus, int rb)
{
    mtv::Plan p{};
    p.rows = s.num_nodes * s.num_heads;
    p.cus = cus;
    p.row_groups = (p.rows + mtv::kRowsPerGroup - 1) / mtv::kRowsPerGroup;
    p.rb = rb;
    const int wg_groups = (p.row_groups + rb - 1) / rb;
    int64_t slots = ((int64_t)cus + wg_groups - 1) / wg_groups;
    if (slots < 1)
        slots = 1;
    p.slots = (int)slots;
    // slices of the whole batch: at most G when the target is reduced (always
    // for one sequence), at most G + B otherwise; the grid and the workspace
    // are sized by this bound, so a tight one keeps every workgroup resident
    const bool reduced = slots > 2 * ((int64_t)s.batch - 1);
    // the slicing of a batch whose sequences all hold max_kv keys
    const int64_t tiles = (s.max_kv + mtv::kTileKeys - 1) / mtv::kTileKeys;
    const int64_t target = reduced ? slots - (s.batch - 1) : slots;
    int64_t c = ((int64_t)s.batch * tiles + target - 1) / target;
    if (c > tiles)
        c = tiles;
    p.splits = (int)((tiles + c - 1) / c);
    p.chunk = (int)(c * mtv::kTileKeys);
    // One sequence keeps that slicing whatever its length (a shorter one uses
    // fewer of the slices), so the grid holds exactly the slices it can use.
    p.single_c = (int)c;
    p.max_slices = s.batch == 1 ? p.splits : (int)(reduced ? slots : slots + s.batch);
    const size_t parts = (size_t)p.row_groups * (size_t)p.max_slices;
    p.part_o_off = 0;
    p.part_ml_off = align_up(parts * mtv::kRowsPerGroup * mtv::kDv * sizeof(uint16_t), 256);
    p.seq_off = align_up(p.part_ml_off + parts * mtv::kRowsPerGroup * 2 * sizeof(float), 256);
    p.bytes = align_up(p.seq_off + (size_t)s.batch * 2 * sizeof(int32_t), 256);
    return p;
}

// Many rows over long slices make the call MFMA-bound: then two row groups
// share each split workgroup (two 16-row blocks per wave), which halves the
// LDS operand reads per MFMA and the tile gathers per row. That form costs
// about 12-17 us more per call (two blocks of Q to load, tile 0's Q.K^T ahead
// of the loop, twice the partials to store and, with the slots per row group
// doubled, to combine) and saves about 0.3-0.45 us per tile of a slice.
// Measured on 16, 32 and 64 row groups at 8192-65536 keys, it breaks even
// near 40 tiles per slice; on 8 row groups, whose slices are shared by fewer
// workgroups, near 50. So it is taken from 16 row groups and 48 tiles per
// slice, or from 8 row groups and 64. Per-token tables only: the hybrid
// layout's index staging leaves that form no registers to spare.
mtv::Plan make_plan(const mtv_shape& s, int cus, bool paged)
{
    const int row_groups = (s.num_nodes * s.num_heads + mtv::kRowsPerGroup - 1) / mtv::kRowsPerGroup;
    if (!paged && row_groups >= mtv::kRB2MinRowGroups) {
        const mtv::Plan p2 = make_plan_rb(s, cus, 2);
        if (p2.single_c >= mtv::kRB2MinTiles(row_groups))
            return p2;
    }
    return make_plan_rb(s, cus, 1);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

size_t mla_tree_verify_workspace_size(const mtv_shape* shape)
{
    if (!shape || !shape_ok(*shape))
        return 0;
    int cus = current_cu_count();
    if (cus <= 0)
        cus = 256;  // no device visible: size for a full MI355X
    // one workspace serves both layouts
    return std::max(make_plan(*shape, cus, false).bytes, make_plan(*shape, cus, true).bytes);
}

int mtv_plan_query(const mtv_shape* shape, int num_cus, int* splits, int* chunk, int* row_groups)
{
    if (!shape || !splits || !chunk || !row_groups)
        return MTV_ERR_NULL;
    if (!shape_ok(*shape) || num_cus < 1)
        return MTV_ERR_SHAPE;
    const mtv::Plan p = make_plan(*shape, num_cus, false);
    *splits = p.splits;
    *chunk = p.chunk;
    *row_groups = p.row_groups;
    return MTV_OK;
}

}  // extern "C"

namespace {

enum Phase { kSplit = 1, kCombine = 2 };

// Shared validation and dispatch of the three launching entry points. Pointers
// a phase does not use may be NULL for that phase.
// Hybrid paging of the split phase (prefix_pages == NULL: per-token table).
struct Paging {
    const int32_t* prefix_pages = nullptr;
    const int32_t* tree_slots = nullptr;
    int page_size = 0, max_pages = 0;
};

int run(int phases, const mtv_shape* shape, const void* q, const void* kv_pool,
        const int32_t* page_table, const int32_t* seq_lens, const uint32_t* tree_mask,
        float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
        hipStream_t stream, const Paging& pg = Paging())
{
    const bool split = phases & kSplit;
    const bool combine = phases & kCombine;
    const bool paged = pg.prefix_pages || pg.tree_slots;
    if (!shape || !seq_lens || !workspace)
        return MTV_ERR_NULL;
    if (split && (!q || !kv_pool || !tree_mask))
        return MTV_ERR_NULL;
    if (split && !paged && !page_table)
        return MTV_ERR_NULL;
    if (split && paged && (!pg.prefix_pages || !pg.tree_slots))
        return MTV_ERR_NULL;
    if (paged && (pg.page_size < 1 || pg.page_size > MTV_MAX_KV || pg.max_pages < 1 ||
                  pg.max_pages > MTV_MAX_KV))
        return MTV_ERR_SHAPE;
    if (paged && (!aligned(pg.prefix_pages, 4) || !aligned(pg.tree_slots, 4)))
        return MTV_ERR_ALIGN;
    if (combine && (!out || !lse))
        return MTV_ERR_NULL;
    if (!shape_ok(*shape) || (split && !std::isfinite(scale)))
        return MTV_ERR_SHAPE;
    if (!aligned(seq_lens, 4) || !aligned(workspace, 256))
        return MTV_ERR_ALIGN;
    if (split && (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(page_table, 4) ||
                  !aligned(tree_mask, 4)))  // page_table may be NULL when paged
        return MTV_ERR_ALIGN;
    if (combine && (!aligned(out, 16) || !aligned(lse, 4)))
        return MTV_ERR_ALIGN;
    const int cus = current_cu_count();
    if (cus <= 0)
        return MTV_ERR_HIP;
    const mtv::Plan plan = make_plan(*shape, cus, paged);
    if (workspace_bytes < plan.bytes)
        return MTV_ERR_WORKSPACE;

    mtv::Args a{};
    a.q = q;
    a.kv = kv_pool;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.tree_mask = tree_mask;
    a.scale = scale;
    a.out = out;
    a.lse = lse;
    a.part_o = (uint16_t*)((char*)workspace + plan.part_o_off);
    a.part_ml = (float*)((char*)workspace + plan.part_ml_off);
    a.seq_slices = (int32_t*)((char*)workspace + plan.seq_off);
    a.batch = shape->batch;
    a.nodes = shape->num_nodes;
    a.heads = shape->num_heads;
    a.max_kv = shape->max_kv;
    a.num_slots = shape->num_slots;
    a.prefix_pages = pg.prefix_pages;
    a.tree_slots = pg.tree_slots;
    a.page_size = pg.page_size;
    a.max_pages = pg.max_pages;
    if (split && mtv::launch_split(plan, a, stream) != hipSuccess)
        return MTV_ERR_HIP;
    if (combine && mtv::launch_combine(plan, a, stream) != hipSuccess)
        return MTV_ERR_HIP;
    return MTV_OK;
}

}  // namespace

extern "C" {

int mla_tree_verify(const mtv_shape* shape, const void* q, const void* kv_pool,
                    const int32_t* page_table, const int32_t* seq_lens, const uint32_t* tree_mask,
                    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                    hipStream_t stream)
{
    // every pointer is required here, including those of the combine phase
    if (!out || !lse || !q || !kv_pool || !page_table || !tree_mask)
        return MTV_ERR_NULL;
    return run(kSplit | kCombine, shape, q, kv_pool, page_table, seq_lens, tree_mask, scale, out,
               lse, workspace, workspace_bytes, stream);
}

int mla_tree_verify_paged(const mtv_shape* shape, int32_t page_size, int32_t max_pages,
                          const void* q, const void* kv_pool, const int32_t* prefix_pages,
                          const int32_t* tree_slots, const int32_t* seq_lens,
                          const uint32_t* tree_mask, float scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!out || !lse || !q || !kv_pool || !prefix_pages || !tree_slots || !tree_mask)
        return MTV_ERR_NULL;
    Paging pg;
    pg.prefix_pages = prefix_pages;
    pg.tree_slots = tree_slots;
    pg.page_size = page_size;
    pg.max_pages = max_pages;
    return run(kSplit | kCombine, shape, q, kv_pool, nullptr, seq_lens, tree_mask, scale, out, lse,
               workspace, workspace_bytes, stream, pg);
}

int mla_tree_verify_splitkv(const mtv_shape* shape, const void* q, const void* kv_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const uint32_t* tree_mask, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    return run(kSplit, shape, q, kv_pool, page_table, seq_lens, tree_mask, scale, nullptr, nullptr,
               workspace, workspace_bytes, stream);
}

int mla_tree_verify_combine(const mtv_shape* shape, const int32_t* seq_lens, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return run(kCombine, shape, nullptr, nullptr, nullptr, seq_lens, nullptr, 0.f, out, lse,
               workspace, workspace_bytes, stream);
}

int mla_tree_mask_build(int32_t batch, int32_t num_nodes, const int32_t* parents,
                        uint32_t* tree_mask, hipStream_t stream)
{
    if (!parents || !tree_mask)
        return MTV_ERR_NULL;
    if (batch < 1 || batch > MTV_MAX_BATCH || num_nodes < 1 || num_nodes > MTV_MAX_NODES)
        return MTV_ERR_SHAPE;
    if (!aligned(parents, 4) || !aligned(tree_mask, 4))
        return MTV_ERR_ALIGN;
    if (mtv::launch_tree_mask(batch, num_nodes, parents, tree_mask, stream) != hipSuccess)
        return MTV_ERR_HIP;
    return MTV_OK;
}

int mla_kv_commit(int32_t batch, int32_t num_nodes, int32_t max_kv, int64_t num_slots,
                  void* kv_pool, int32_t* page_table, const int32_t* seq_lens,
                  const int32_t* accept_len, const int32_t* accept_path,
                  const int32_t* region_base, hipStream_t stream)
{
    if (!kv_pool || !page_table || !seq_lens || !accept_len || !accept_path || !region_base)
        return MTV_ERR_NULL;
    if (batch < 1 || batch > MTV_MAX_BATCH || num_nodes < 1 || num_nodes > MTV_MAX_NODES ||
        max_kv < num_nodes || max_kv > MTV_MAX_KV || num_slots < 1 || num_slots > INT32_MAX)
        return MTV_ERR_SHAPE;
    if (!aligned(kv_pool, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
        !aligned(accept_len, 4) || !aligned(accept_path, 4) || !aligned(region_base, 4))
        return MTV_ERR_ALIGN;
    mtv::KvArgs a{batch, num_nodes, max_kv, num_slots, kv_pool, page_table, seq_lens,
                  accept_len, accept_path, region_base};
    if (mtv::launch_kv_commit(a, stream) != hipSuccess)
        return MTV_ERR_HIP;
    return MTV_OK;
}

int mla_kv_defrag(int32_t batch, int32_t max_kv, int64_t num_slots, void* kv_pool,
                  int32_t* page_table, const int32_t* seq_lens, const int32_t* region_base,
                  hipStream_t stream)
{
    if (!kv_pool || !page_table || !seq_lens || !region_base)
        return MTV_ERR_NULL;
    if (batch < 1 || batch > MTV_MAX_BATCH || max_kv < 1 || max_kv > MTV_MAX_KV || num_slots < 1 ||
        num_slots > INT32_MAX)
        return MTV_ERR_SHAPE;
    if (!aligned(kv_pool, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
        !aligned(region_base, 4))
        return MTV_ERR_ALIGN;
    const int cus = current_cu_count();
    if (cus <= 0)
        return MTV_ERR_HIP;
    mtv::KvArgs a{batch, 0, max_kv, num_slots, kv_pool, page_table, seq_lens, nullptr, nullptr,
                  region_base};
    if (mtv::launch_kv_move(a, cus, stream) != hipSuccess)
        return MTV_ERR_HIP;
    return MTV_OK;
}

int mtv_check_inputs(const mtv_shape* shape, const int32_t* page_table, const int32_t* seq_lens,
                     const uint32_t* tree_mask, uint64_t* counts, hipStream_t stream)
{
    if (!shape || !page_table || !seq_lens || !tree_mask || !counts)
        return MTV_ERR_NULL;
    const mtv_shape& s = *shape;
    if (s.batch < 1 || s.batch > MTV_MAX_BATCH || s.num_nodes < 1 || s.num_nodes > MTV_MAX_NODES ||
        s.max_kv < s.num_nodes || s.max_kv > MTV_MAX_KV || s.num_slots < 1 || s.num_slots > INT32_MAX)
        return MTV_ERR_SHAPE;
    if (!aligned(page_table, 4) || !aligned(seq_lens, 4) || !aligned(tree_mask, 4) ||
        !aligned(counts, 8))
        return MTV_ERR_ALIGN;
    const int cus = current_cu_count();
    if (cus <= 0)
        return MTV_ERR_HIP;
    if (mtv::launch_check_inputs(s.batch, s.num_nodes, s.max_kv, s.num_slots, page_table, seq_lens,
                                 tree_mask, (unsigned long long*)counts, cus, stream) != hipSuccess)
        return MTV_ERR_HIP;
    return MTV_OK;
}

const char* mtv_status_string(int status)
{
    switch (status) {
    case MTV_OK:
        return "success";
    case MTV_ERR_NULL:
        return "a required pointer is NULL";
    case MTV_ERR_SHAPE:
        return "shape or scalar argument out of range";
    case MTV_ERR_ALIGN:
        return "misaligned pointer (q, kv_pool, out need 16 B; workspace 256 B; arrays 4 B)";
    case MTV_ERR_WORKSPACE:
        return "workspace smaller than mla_tree_verify_workspace_size()";
    case MTV_ERR_HIP:
        return "HIP runtime error (no device, or a launch failed)";
    case MTV_ERR_SCRATCH:
        return "the call needs more workspace than the no-alloc scratch holds (MTV_NOALLOC_SCRATCH_BYTES)";
    default:
        return "unknown status";
    }
}

}  // extern "C"
