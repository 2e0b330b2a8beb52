// fused_kernel.h -- the persistent fused kernel's __global__ entry (one template for every build: eight or
// four waves per workgroup, the SwiGLU epilogue, the half-width tile for a ragged last column block).
#pragma once

#include <hip/hip_runtime.h>

#include "fused_dev.h"

namespace mk {

template <class C, bool SW, bool HALF_N = false>
__global__ __launch_bounds__(C::THREADS, 1) void k_fused(FusedArgs a)
{
    __shared__ __attribute__((aligned(1024))) char stg[4 * C::STAGE];   // the four stage arrays, consecutive
    __shared__ int32_t off[1025], toff[1025], uoff[1025];
    __shared__ uint16_t basetab[kBaseTab];
    LdsStages ls;
    char *st[4];   // filled one by one: a constant initializer would become a static one
    for (int k = 0; k < 4; ++k) {
        st[k] = stg + k * C::STAGE;
        ls.p[k] = (lds_char_t *)st[k];
    }
    const uint32_t call = fused_call_epoch(a);
    fused_kernel_body<C, SW, HALF_N>(a, call, st, ls, off, toff, uoff, basetab);
    fused_exit(a, call);
}

}  // namespace mk
