// peak.hip -- a measurement utility, not part of the method: the dense bf16
// MFMA rate this device sustains, for reporting next to the published peak.
// Each wave runs `iters` rounds of eight independent
// v_mfma_f32_32x32x16_bf16 accumulations on register operands (no memory
// traffic; eight chains keep the matrix pipe fed without waiting on a
// result), then folds its accumulators into one word per work-group.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {
namespace peak {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 8;

__global__ void __launch_bounds__(256) k_peak_mfma(float *__restrict__ sink, int iters)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.f / (1 + ((lane + e) & 7)));
        b[e] = (__bf16)(1.f / (1 + ((lane * 3 + e) & 7)));
    }
    f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (threadIdx.x == 0) sink[blockIdx.x] = s;   // keeps the products alive
}

}  // namespace peak
}  // namespace fk

using namespace fk;

extern "C" int fk_peak_mfma_bf16(float *sink, int32_t n_wg, int32_t iters, double *flops, fk_stream_t stream)
{
    if (!sink || n_wg < 1 || iters < 1 || !flops) return FK_E_INVALID_ARG;
    *flops = (double)n_wg * 4.0 * (double)iters * peak::CHAINS * (2.0 * 32 * 32 * 16);
    peak::k_peak_mfma<<<dim3((unsigned)n_wg), 256, 0, (hipStream_t)stream>>>(sink, iters);
    return launch_status();
}
