// kernels.hip -- __global__ entry points of libmk and their launch wrappers.
// The stage-by-stage kernels here run the same device code as the fused
// persistent kernel, one launch per step.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fused_dev.h"
#include "fused_kernel.h"
#include "gemm_dev.h"
#include "layout_dev.h"
#include "mk_launch.h"
#include "route_dev.h"

namespace mk {

// Router partial sums: one wave task per wave, four per workgroup.
__global__ __launch_bounds__(256) void k_router(RouterArgs a)
{
    __shared__ __attribute__((aligned(16))) char lds[4 * kRtLdsPerWave];
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int q = (int)blockIdx.x * 4 + wave;
    if (q < router_tasks(a.T, a.E)) router_task(a, q, (lds_byte_t *)(lds + wave * kRtLdsPerWave));
}

// Token-per-wave top-k, four tokens per workgroup.
__global__ __launch_bounds__(256) void k_topk_wave(TopkArgs ta) { topk_wave_loop(ta, blockIdx.x, gridDim.x); }

__global__ __launch_bounds__(256) void k_count_given(const int32_t *ids_in, int32_t *ids_ws, int32_t *ids_user,
                                                     CountArgs ca)
{
    __shared__ int32_t ids_lds[kTokBlock * kMaxK];
    __shared__ int32_t cnt_lds[1024];
    __shared__ uint64_t mask_lds[1024];
    const int base_t = blockIdx.x * kTokBlock;
    const int n_t = min(kTokBlock, ca.T - base_t);
    for (int i = threadIdx.x; i < n_t * ca.k; i += blockDim.x) {
        const size_t o = (size_t)base_t * ca.k + i;
        const int32_t id = ids_in[o];
        ids_lds[i] = id;
        ids_ws[o] = id;
        if (ids_user) ids_user[o] = id;
    }
    __syncthreads();
    count_block(ca, blockIdx.x, ids_lds, cnt_lds, mask_lds);
}

__global__ __launch_bounds__(1024) void k_scan(ScanArgs a)
{
    __shared__ int32_t s_cnt[1024], s_til[1024];
    scan_block(a, s_cnt, s_til);
}

__global__ __launch_bounds__(256) void k_slots(SlotArgs a)
{
    const int n = a.T * a.k;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) slot_one(a, i);
}

__global__ __launch_bounds__(256) void k_move(SrcRows src, const int32_t *row_token, uint16_t *x_perm, int d,
                                              const WsHeader *hdr)
{
    const int R = (int)hdr->R;
    const int waves = gridDim.x * (blockDim.x / kWave);
    const int wid = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    for (int r = wid; r < R; r += waves) move_row(src, row_token, x_perm, d, r, threadIdx.x % kWave);
}

template <class C, bool SW = false>
__global__ __launch_bounds__(C::THREADS, 1) void k_gemm(GemmArgs a)
{
    __shared__ __attribute__((aligned(1024))) char stg[4 * C::STAGE];   // the four stage arrays, consecutive
    LdsStages ls;
    for (int k = 0; k < 4; ++k) ls.p[k] = (lds_char_t *)(stg + k * C::STAGE);
    gemm_worker<C, SW>(a, blockIdx.x, gridDim.x, ls);
}

// Combine: wave task q = (token q / nc, 512-column chunk q % nc); the lane owns
// 8 consecutive columns (16 bytes).  The token's slots and gates are read by
// the first k lanes and taken one at a time with readlane (uniform), the rows
// of four choices are loaded before they are accumulated.
__global__ __launch_bounds__(256) void k_combine(const uint16_t *y, int32_t rows, const int32_t *slot_of,
                                                 const float *gate, int32_t T, int32_t k, int32_t N, uint16_t *out)
{
    const int lane = threadIdx.x % kWave;
    const int nc = (N + 8 * kWave - 1) / (8 * kWave);
    const int waves = (int)gridDim.x * (int)(blockDim.x / kWave);
    for (int q = (int)blockIdx.x * (int)(blockDim.x / kWave) + (int)threadIdx.x / kWave; q < T * nc; q += waves) {
        const int t = __builtin_amdgcn_readfirstlane(q / nc);
        const int col = (q - t * nc) * 8 * kWave + 8 * lane;
        const bool in = col < N;   // N % 8 == 0: a lane's 8 columns are all inside or all outside
        const int my_slot = lane < k ? slot_of[(size_t)t * k + lane] : -1;
        const float my_w = lane < k ? gate[(size_t)t * k + lane] : 0.0f;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 4) {
            u32x4_t v[4];
            float wj[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = min(j0 + u, k - 1);
                const int slot = __builtin_amdgcn_readlane(my_slot, j);
                wj[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
                ok[u] = j0 + u < k && slot >= 0 && slot < rows;
                v[u] = ok[u] && in ? *(const u32x4_t *)(y + (size_t)slot * N + col) : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!ok[u]) continue;   // uniform
                float f[8];
                unpack8(v[u], f);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj[u], f[i], acc[i]);
            }
        }
        if (in) {
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
            *(u32x4_t *)(out + (size_t)t * N + col) = o;
        }
    }
}

// SwiGLU over gate|up rows: item i = (row i / (F / 8), 8 columns); h = bf16(silu(g) * u), fp32.
__global__ __launch_bounds__(256) void k_swiglu(const uint16_t *gu, int32_t rows, int32_t F, uint16_t *h)
{
    const long items = (long)rows * (F / 8);
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += (long)gridDim.x * blockDim.x) {
        const long r = i / (F / 8);
        const int c = (int)(i - r * (F / 8)) * 8;
        float g[8], u[8];
        unpack8(*(const u32x4_t *)(gu + r * 2 * F + c), g);
        unpack8(*(const u32x4_t *)(gu + r * 2 * F + F + c), u);
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = g[2 * q] / (1.0f + expf(-g[2 * q])) * u[2 * q];
            const float b = g[2 * q + 1] / (1.0f + expf(-g[2 * q + 1])) * u[2 * q + 1];
            o[q] = pack_bf16x2(a, b);
        }
        *(u32x4_t *)(h + r * F + c) = o;
    }
}

// The row-tile table of a layout given by its expert offsets (one thread).
__global__ void k_tiles(const int32_t *offsets, int32_t E_local, int32_t bm, int32_t *tile_off, WsHeader *hdr)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int32_t t = 0;
    tile_off[0] = 0;
    for (int e = 0; e < E_local; ++e) {
        t += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
        tile_off[e + 1] = t;
    }
    hdr->n_tiles = (uint32_t)t;
    hdr->R = (uint32_t)offsets[E_local];
}

// The call status of a staged call into status[2] (error code, detail), then the workspace's error
// words cleared (one thread); and a zero fill of n16 16-byte words (a kernel, so that a caller's graph
// capture records no memset node).
__global__ void k_status(WsHeader *hdr, int32_t *status)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    status[0] = (int32_t)hdr->err;
    status[1] = (int32_t)hdr->err_detail;
    hdr->err = 0u;
    hdr->err_detail = 0u;
}

__global__ void k_zero(uint4 *p, size_t n16)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------- wrappers

hipError_t launch_status(WsHeader *hdr, int32_t *status, hipStream_t s)
{
    hipLaunchKernelGGL(k_status, dim3(1), dim3(64), 0, s, hdr, status);
    return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    const int grid = (int)std::min<size_t>((n16 + 255) / 256, 1024);
    hipLaunchKernelGGL(k_zero, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, (uint4 *)p, n16);
    return hipGetLastError();
}

hipError_t launch_router(const RouterArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_router, dim3((router_tasks(a.T, a.E) + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &ta, const CountArgs &ca, bool do_count, hipStream_t s)
{
    // token-parallel selection, then the per-block histogram from the ids it wrote
    hipLaunchKernelGGL(k_topk_wave, dim3(topk_wave_units(ta.T, 4)), dim3(256), 0, s, ta);
    if (!do_count) return hipGetLastError();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_count_given(ta.ids, ta.ids, nullptr, ca, s);
}

hipError_t launch_count_given(const int32_t *ids_in, int32_t *ids_ws, int32_t *ids_user, const CountArgs &ca,
                              hipStream_t s)
{
    const int nblk = (ca.T + kTokBlock - 1) / kTokBlock;
    hipLaunchKernelGGL(k_count_given, dim3(nblk), dim3(256), 0, s, ids_in, ids_ws, ids_user, ca);
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_slots(const SlotArgs &a, hipStream_t s)
{
    const long n = (long)a.T * a.k;
    int grid = (int)((n + 255) / 256);
    grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);
    hipLaunchKernelGGL(k_slots, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_move(const SrcRows &src, const int32_t *row_token, uint16_t *x_perm, int d, const WsHeader *hdr,
                       hipStream_t s)
{
    hipLaunchKernelGGL(k_move, dim3(1024), dim3(256), 0, s, src, row_token, x_perm, d, hdr);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t *y, int32_t rows, const int32_t *slot_of, const float *gate, int32_t T,
                          int32_t k, int32_t N, uint16_t *out, hipStream_t s)
{
    const long tasks = (long)T * ((N + 8 * kWave - 1) / (8 * kWave));
    const int grid = (int)std::min<long>((tasks + 3) / 4, 65536);
    hipLaunchKernelGGL(k_combine, dim3(grid), dim3(256), 0, s, y, rows, slot_of, gate, T, k, N, out);
    return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t *gu, int32_t rows, int32_t F, uint16_t *h, hipStream_t s)
{
    const long items = (long)rows * (F / 8);
    const int grid = (int)std::min<long>((items + 255) / 256, 65536);
    hipLaunchKernelGGL(k_swiglu, dim3(grid), dim3(256), 0, s, gu, rows, F, h);
    return hipGetLastError();
}

hipError_t launch_tiles(const int32_t *offsets, int32_t E_local, int32_t bm, int32_t *tile_off, WsHeader *hdr,
                        hipStream_t s)
{
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(64), 0, s, offsets, E_local, bm, tile_off, hdr);
    return hipGetLastError();
}

typedef Tiles<8>::M256 Tile256;       // the grouped GEMM launches: eight waves per workgroup
typedef Tiles<8>::M256 FusedTile;     // the fused kernel: eight waves per workgroup

hipError_t launch_gemm(const GemmArgs &a, int bm, int bn, int grid, hipStream_t s)
{
    if (bm == 256 && bn == 256) {
        hipLaunchKernelGGL((k_gemm<Tile256>), dim3(grid), dim3(Tile256::THREADS), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_swiglu(const GemmArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_gemm<Tile256, true>), dim3(grid), dim3(Tile256::THREADS), 0, s, a);
    return hipGetLastError();
}

int gemm_max_grid(int bm, int bn)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (bm == 256 && bn == 256) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_gemm<Tile256>, Tile256::THREADS,
                                                         0) != hipSuccess)
            return 0;
    }
    return cus * per_cu;
}

// An ordinary launch of at most as many workgroups as the device holds at
// once, or (cooperative) a cooperative launch, which costs ~15 us more per
// call.  The grid barriers need every workgroup resident together: with the
// device's CUs free of other work the dispatcher places them all; work of
// other streams only delays the late ones, and a wait that outlasts the bound
// ends the call with MK_ETIMEOUT.  A cooperative launch has the runtime
// guarantee co-residency instead.
hipError_t launch_fused(const FusedArgs &a, int grid, bool cooperative, bool four_waves, hipStream_t s)
{
    // four_waves, with neither of the builds below: the four-wave build (kernels_w4.hip)
    if (four_waves && a.ga.F == 0 && a.ga.N % 256 == 0) return launch_fused4(a, grid, cooperative, s);
    // a.ga.F > 0: the gate|up weights with the SwiGLU epilogue; a ragged N (N % 256 != 0): the build whose
    // last column block runs the half-width tile
    const void *k = a.ga.F > 0          ? (const void *)k_fused<FusedTile, true>
                    : a.ga.N % 256 != 0 ? (const void *)k_fused<FusedTile, false, true>
                                        : (const void *)k_fused<FusedTile, false>;
    void *args[] = {(void *)&a};
    if (cooperative)   // the runtime guarantees co-residency (or refuses the launch)
        return hipLaunchCooperativeKernel(k, dim3(grid), dim3(FusedTile::THREADS), args, 0, s);
    return hipLaunchKernel(k, dim3(grid), dim3(FusedTile::THREADS), args, 0, s);
}

int fused_max_grid()
{
    constexpr int kMaxDevices = 64;
    static int cached[kMaxDevices] = {};   // per device: computed once
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices && cached[dev] > 0) return cached[dev];
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    int per_cu_sw = 0, per_cu_half = 0;   // every build must fit (one workspace layout, one grid)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_fused<FusedTile, false>,
                                                     FusedTile::THREADS, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_sw, (const void *)k_fused<FusedTile, true>,
                                                     FusedTile::THREADS, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_half, (const void *)k_fused<FusedTile, false, true>,
                                                     FusedTile::THREADS, 0) != hipSuccess)
        return 0;
    const int per_cu_4 = fused4_per_cu();
    per_cu = std::min(std::min(per_cu, per_cu_4), std::min(per_cu_sw, per_cu_half));
    if (dev >= 0 && dev < kMaxDevices) cached[dev] = cus * per_cu;
    return cus * per_cu;
}

}  // namespace mk
