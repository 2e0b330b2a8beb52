// mk_launch.h -- host-side launch wrappers for the libmk kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "mk_args.h"

namespace mk {

struct RouterArgs;
struct TopkArgs;
struct CountArgs;
struct ScanArgs;
struct SlotArgs;
struct GemmArgs;
struct FusedArgs;
struct WsHeader;

// Router partial sums, one wave task per wave (router_tasks).
hipError_t launch_router(const RouterArgs &a, hipStream_t s);
// Top-k + gate for all tokens; with do_count also the per-block histogram and ranks.
hipError_t launch_topk(const TopkArgs &ta, const CountArgs &ca, bool do_count, hipStream_t s);
// Histogram and ranks of caller-given ids (copied into the workspace id array).
hipError_t launch_count_given(const int32_t *ids_in, int32_t *ids_ws, int32_t *ids_user, const CountArgs &ca,
                              hipStream_t s);
hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
// Expert FFN: h = bf16(silu(g) * u) over [g | u] rows; the row-tile table of a given layout.
hipError_t launch_swiglu(const uint16_t *gu, int32_t rows, int32_t F, uint16_t *h, hipStream_t s);
hipError_t launch_tiles(const int32_t *offsets, int32_t E_local, int32_t bm, int32_t *tile_off, WsHeader *hdr,
                        hipStream_t s);
// Combine: out[t] = bf16(sum over local choices of gate * y_perm[slot]).
hipError_t launch_combine(const uint16_t *y, int32_t rows, const int32_t *slot_of, const float *gate, int32_t T,
                          int32_t k, int32_t N, uint16_t *out, hipStream_t s);
hipError_t launch_slots(const SlotArgs &a, hipStream_t s);
hipError_t launch_move(const SrcRows &src, const int32_t *row_token, uint16_t *x_perm, int d, const WsHeader *hdr,
                       hipStream_t s);
// Grouped GEMM over the tile table; bm/bn select the tile shape.
hipError_t launch_gemm(const GemmArgs &a, int bm, int bn, int grid, hipStream_t s);
// The grouped gate|up GEMM with the SwiGLU epilogue (a.F features per expert, a.N == 2 a.F).
hipError_t launch_gemm_swiglu(const GemmArgs &a, int grid, hipStream_t s);
// Largest co-resident grid of the GEMM kernel for this tile shape.
int gemm_max_grid(int bm, int bn);
// The persistent fused kernel: one workgroup per resident slot of the device (its grid barriers need them all
// resident together).
hipError_t launch_fused(const FusedArgs &a, int grid, bool cooperative, bool four_waves, hipStream_t s);
int fused_max_grid();
// The four-wave build (kernels_w4.hip): its launch, and how many of its workgroups a CU holds.
hipError_t launch_fused4(const FusedArgs &a, int grid, bool cooperative, hipStream_t s);
int fused4_per_cu();
// A staged call's status into status[2], then the error words cleared; a zero fill of bytes (% 16 == 0).
hipError_t launch_status(WsHeader *hdr, int32_t *status, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

}  // namespace mk
