// mla_tree_verify_noalloc: mla_tree_verify with its workspace in a fixed
// device array of this library instead of a caller buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in for the symbol): the device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and that pointer is what
// the kernels receive as their workspace.
#include <hip/hip_runtime.h>

#include <atomic>

#include "mla_tree_verify.h"

namespace {

constexpr size_t kScratchBytes = MTV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the workspace contract wants 256-byte multiples");

// The scratch: per-slice partial results and per-sequence slice ranges of one
// call. Nothing in it needs clearing between calls: each call writes every
// word it later reads before reading it.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // zero-initialised: not looked up yet

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device; NULL if the runtime refuses.
void* scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    // Two threads racing here get the same address; either store is correct.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

int mla_tree_verify_noalloc(const mtv_shape* shape, const void* q, const void* kv_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const uint32_t* tree_mask, float scale, void* out, float* lse,
                            hipStream_t stream)
{
    if (!shape)
        return MTV_ERR_NULL;
    // the size test first, so that an oversized call fails the same way on
    // every device; 0 means an invalid shape
    const size_t need = mla_tree_verify_workspace_size(shape);
    if (need == 0)
        return MTV_ERR_SHAPE;
    if (need > kScratchBytes)
        return MTV_ERR_SCRATCH;
    void* ws = scratch_ptr();
    if (!ws)
        return MTV_ERR_HIP;
    // Everything else (validation, plan, the two launches) is mla_tree_verify's
    // own path, with the scratch as its workspace.
    return mla_tree_verify(shape, q, kv_pool, page_table, seq_lens, tree_mask, scale, out, lse, ws,
                           kScratchBytes, stream);
}

}  // extern "C"
