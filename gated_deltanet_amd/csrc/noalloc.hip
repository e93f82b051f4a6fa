// noalloc.hip -- ForkAttention for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// fork_attn_forward needs a caller-provided workspace for the round's derived
// metadata (segment starts, positions, ancestor chains, the tile list and its
// order, the status word).  fork_attn_forward_noalloc instead keeps that
// metadata in one file-scope device array of FK_NOALLOC_SCRATCH_BYTES per GPU,
// builds it (the same builder kernels as fk_tree_build) and runs the same
// K/V append and attention kernels on it, so its outputs have the bits of
// fk_tree_build + fork_attn_forward.  Nothing here calls hipMalloc, hipFree or
// an allocating library routine.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on each device comes from hipGetSymbolAddress, taken
// once per device on that device's first call (with that device current) and
// kept; kernels receive that address, never the name.  Every call on a GPU
// shares that GPU's array, which keeps the last call's contents: the builder
// writes every word it later reads (it clears the status and its counters
// first), and calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fk_common.h"

extern "C" int fk_tree_build(const fk_tree_meta *meta, void *ws, size_t ws_bytes, fk_stream_t stream);
extern "C" int fork_attn_forward(const fk_tree_meta *meta, const void *q, const void *k, const void *v, int dtype,
                                 int Hq, int Hkv, int d, float scale, void *k_pool, void *v_pool, void *out,
                                 void *ws, size_t ws_bytes, fk_stream_t stream);

namespace fk {
namespace noalloc {

constexpr size_t SCRATCH_BYTES = (size_t)FK_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void *g_ptr[MAX_DEVICES];   // the array's device address, per device

// the current device's address of `scratch`, looked up on its first use
int scratch_ptr(void **out)
{
    int dev = 0;
    FK_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return FK_E_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FK_E_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return FK_OK;
}

}  // namespace noalloc
}  // namespace fk

using namespace fk;

extern "C" int fork_attn_forward_noalloc(const fk_tree_meta *meta, const void *q, const void *k, const void *v,
                                         int dtype, int Hq, int Hkv, int d, float scale, void *k_pool,
                                         void *v_pool, void *out, int32_t *status, fk_stream_t stream)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (ws_layout(*meta, 0, 0, 0).total > noalloc::SCRATCH_BYTES) return FK_E_WORKSPACE;
    void *ws = nullptr;
    if ((rc = noalloc::scratch_ptr(&ws))) return rc;
    if ((rc = fk_tree_build(meta, ws, noalloc::SCRATCH_BYTES, stream))) return rc;
    if ((rc = fork_attn_forward(meta, q, k, v, dtype, Hq, Hkv, d, scale, k_pool, v_pool, out, ws,
                                noalloc::SCRATCH_BYTES, stream)))
        return rc;
    if (status)   // the round's status word (offset 0 of the metadata), device to device
        FK_HIP(hipMemcpyAsync(status, ws, sizeof(int32_t), hipMemcpyDeviceToDevice, (hipStream_t)stream));
    return FK_OK;
}
