// kernels_w4.hip -- the fused kernel with four waves per workgroup (one per SIMD, a 128 x 128 block of the
// 256 x 256 tile per wave), for batches where a uniform routing gives every expert at most 32 rows, so that
// every GEMM task is a short weight-streaming tile.  A code object of its own: the eight-wave builds in
// kernels.hip keep the code placement they have without it.
#include <hip/hip_runtime.h>

#include "fused_kernel.h"
#include "mk_launch.h"

namespace mk {

typedef Tiles<4>::M256 FusedTile4;

hipError_t launch_fused4(const FusedArgs &a, int grid, bool cooperative, hipStream_t s)
{
    const void *k = (const void *)k_fused<FusedTile4, false>;
    void *args[] = {(void *)&a};
    if (cooperative)
        return hipLaunchCooperativeKernel(k, dim3(grid), dim3(FusedTile4::THREADS), args, 0, s);
    return hipLaunchKernel(k, dim3(grid), dim3(FusedTile4::THREADS), args, 0, s);
}

int fused4_per_cu()
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_fused<FusedTile4, false>,
                                                     FusedTile4::THREADS, 0) != hipSuccess)
        return 0;
    return per_cu;
}

}  // namespace mk
