// gdn_bf16.hip -- placeholder until the chunked MFMA kernel lands.
#include <hip/hip_runtime.h>

#include "fk_common.h"

int fk_launch_gdn_bf16(const fk_tree_meta *, int, const void *, const void *, const void *, const float *,
                       const float *, int, int, const float *, float *, void *, const void *, float *, hipStream_t)
{
    return FK_E_UNSUPPORTED;
}
