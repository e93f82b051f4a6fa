// checkpoint.hip -- save and resume of float32 recurrent states (Flide
// section 3.4: a checkpoint stores the float32 Gated DeltaNet state at its
// position; the keys/values before it stay in their pages, retained by id).
// A plain HBM-bound copy with 16-byte accesses.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {

__global__ void __launch_bounds__(256) k_copy_f32(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                  size_t n4)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

int copy_state(const float *src, float *dst, size_t elems, hipStream_t st)
{
    if (((uintptr_t)src | (uintptr_t)dst) & 15 || elems % 4) return FK_E_INVALID_ARG;
    const size_t n4 = elems / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048);
    k_copy_f32<<<blocks > 0 ? blocks : 1, 256, 0, st>>>((const float4 *)src, (float4 *)dst, n4);
    return launch_status();
}

}  // namespace fk

using namespace fk;

static int check_ckpt(const float *a, const float *b, int32_t slot, int32_t count, int32_t n_slots, int32_t Hv,
                      int32_t dk, int32_t dv)
{
    if (!a || !b || slot < 0 || count < 1 || (int64_t)slot + count > n_slots || Hv < 1 || dk < 1 || dv < 1)
        return FK_E_INVALID_ARG;
    return FK_OK;
}

extern "C" int gdn_checkpoint_save(const float *state_out, int32_t slot, int32_t count, int32_t n_slots, int32_t Hv,
                                   int32_t dk, int32_t dv, float *ckpt, fk_stream_t stream)
{
    int rc = check_ckpt(state_out, ckpt, slot, count, n_slots, Hv, dk, dv);
    if (rc) return rc;
    const size_t elems = (size_t)Hv * dk * dv;
    return copy_state(state_out + (size_t)slot * elems, ckpt, elems * count, (hipStream_t)stream);
}

extern "C" int gdn_checkpoint_resume(const float *ckpt, float *state_in, int32_t slot, int32_t count, int32_t n_slots,
                                     int32_t Hv, int32_t dk, int32_t dv, fk_stream_t stream)
{
    int rc = check_ckpt(ckpt, state_in, slot, count, n_slots, Hv, dk, dv);
    if (rc) return rc;
    const size_t elems = (size_t)Hv * dk * dv;
    return copy_state(ckpt, state_in + (size_t)slot * elems, elems * count, (hipStream_t)stream);
}
