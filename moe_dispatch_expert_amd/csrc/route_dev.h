// route_dev.h -- router device code: fp32 logits in the fixed segmented order
// (per-segment partial sums, then an ordered sum), top-k selection, softmax
// gate, and the per-block expert histogram with in-block ranks from wave
// ballots.
//
// Token routing is the first half of the "MoE Dispatch+GEMM" kernel named in
// "mKernel UCCL fuses NVLink/RDMA/compute into one persistent CUDA kernel"
// (zubnet.ai), paragraph 2; "mKernel : une bibliotheque de noyaux fusionnes
// ..." (lefilia.fr), paragraph 3, notes that each token is routed dynamically.
// The pages fix neither the arithmetic nor the tie rule; this code implements
// the readings: fp32 logits l = x . Wr in a fixed order (8 contiguous K
// segments, ascending fused multiply-add chain in each, partials added left to
// right, bias last), top-k by (logit desc, expert id asc), softmax over all E.
#pragma once

#include "mk_args.h"
#include "mk_device.h"

namespace mk {

struct RouterArgs {
    SrcRows src;
    const float *wr;    // [d, E]
    float *part;        // [8, T, E] per-segment partial sums
    int32_t T, d, E;
};

// Row t of the token matrix.  The shard pointers are kernel arguments: when
// every lane of the wave reads from one shard (always for S == 1, and for
// whole blocks of rows otherwise) the pointer is a scalar load; a per-lane
// shard index would need a vector load of the pointer, whose wait would also
// drain every load the wave has in flight.
__device__ __forceinline__ const uint16_t *token_row(const SrcRows &s, int t, int d)
{
    if (s.S == 1) return s.p[0] + (size_t)t * d;
    const int sh = t / s.rows_per_src;
    const int sh0 = __builtin_amdgcn_readfirstlane(sh);
    const uint16_t *base;
    if (__builtin_amdgcn_ballot_w64(sh != sh0) == 0) base = s.p[sh0];
    else base = s.p[sh];
    return base + (size_t)(t - sh * s.rows_per_src) * d;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const u32x4_t v, float (&f)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f[2 * p] = __uint_as_float(w[p] << 16);
        f[2 * p + 1] = __uint_as_float(w[p] & 0xFFFF0000u);
    }
}

// ---------------------------------------------------------------- partial sums
// part[s][t][e] = fma chain over i in K segment s, ascending (fp32, one rounding
// per step).  The work is split into wave tasks (segment s, block of 64 tokens,
// group of TE experts); lane l owns token 64 b + l and the TE chains of that
// token.  Per K step a lane needs one x value (its own row: 16 K values in two
// 16-byte loads) and TE router weights that are the same for every lane.  The
// weights travel 16 to a VGPR (lane i of each 16-lane row holds weight i) and
// reach the FMAs by DPP row broadcast, so a weight costs 4 bytes of load
// return per row instead of 4 bytes per lane; broadcasting them through LDS or
// same-address loads would bound the loop by data return, and scalar loads
// (out-of-order returns, so every use waits for all of them) expose the L2
// latency once per batch.  All loads are vector loads, in order, several
// groups ahead; no LDS and no barrier.  Tasks are numbered expert group
// fastest, so consecutive tasks (the waves of one workgroup) read the same
// token rows and share them in L1/L2.

// Experts per lane: 8 when there are many tasks (fewer bf16 unpacks per FMA), else 4.
__host__ __device__ inline int router_te(int T, int E)
{
    return ((T + kTokBlock - 1) / kTokBlock) * ((E + 7) / 8) * kRouterSegments >= 2048 ? 8 : 4;
}
__host__ __device__ inline int router_tasks(int T, int E)
{
    const int te = router_te(T, E);
    return ((T + kTokBlock - 1) / kTokBlock) * ((E + te - 1) / te) * kRouterSegments;
}

constexpr int kRouterQK = 16;   // K steps per quarter: one FMA block per W float4 set
constexpr int kRouterGQ = 4;    // quarters per group: 64 K steps, one 128-byte line of x per lane
constexpr int kRouterGD = 3;    // groups in flight per wave

// The FMA blocks: acc[j] += W[step][j] * x[step] over the block's K steps in
// ascending order, with W from DPP row broadcasts of a float4 set (see the
// load layout in router_task_body).  The leading s_nop covers the DPP read
// hazards (a VALU or EXEC write of the broadcast registers just before).  DPP
// on the accumulating FMA is written out because the compiler does not fold a
// separate DPP move into it.
// TE = 4: 16 K steps; lane q of the set holds step q, component j expert j.
__device__ __forceinline__ void fma_block4(float (&acc)[4], const f32x4_t w, const float (&x)[16])
{
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %5, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %7, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]),
          "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]),
          "v"(x[14]), "v"(x[15]));
}
// TE = 8: 8 K steps; lane 2 r + j / 4 of the set holds step r, component j % 4 expert j.
__device__ __forceinline__ void fma_block8(float (&acc)[8], const f32x4_t w, const float *x)
{
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %8, %12 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %12 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %12 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %12 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %12 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %12 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %12 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %12 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %13 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %13 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %13 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %13 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %14 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %15 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %16 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %18 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %18 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %18 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %18 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %1, %9, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %10, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %3, %11, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %5, %9, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %10, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t" "v_fmac_f32_dpp %7, %11, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]),
          "+v"(acc[7])
        : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]),
          "v"(x[5]), "v"(x[6]), "v"(x[7]));
}

// W float4 sets per quarter: TE / 4.  Lane p (of each 16-lane row) loads, for
// set h of the quarter at K step k0, the four weights
//   TE = 4: row k0 + p,              columns e0 .. e0 + 3;
//   TE = 8: row k0 + 8 h + p / 2,    columns e0 + 4 (p % 2) .. + 3,
// so a set holds 64 weights in 4 VGPRs, and each weight costs 4 bytes of load
// return per 16 lanes.  FULL: the four columns exist and are 16-byte aligned
// (one dwordx4 load); otherwise one load per column, columns past E repeating
// the last (those chains are never stored).
template <int TE, bool FULL>
struct RouterW {
    const float *p;   // this lane's first weight of quarter 0, set 0
    int E, clast;     // row stride; last valid column offset from this lane's first column
    __device__ __forceinline__ f32x4_t load(int quarter, int h) const
    {
        const float *q = p + ((size_t)quarter * kRouterQK + (TE == 8 ? 8 * h : 0)) * E;
        if (FULL) return *(const f32x4_t *)q;
        f32x4_t v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = q[min(c, clast)];
        return v;
    }
};

template <int TE, bool FULL>
__device__ __forceinline__ void router_task_body(const RouterArgs &a, int s, int tb, int e0)
{
    constexpr int WQ = TE / 4;   // W sets per quarter
    const int lane = threadIdx.x % kWave;
    const int seg = a.d / kRouterSegments;   // a multiple of 16 (d % 128 == 0)
    const int t = tb * kTokBlock + lane;
    const uint16_t *xr = token_row(a.src, min(t, a.T - 1), a.d) + (size_t)s * seg;
    const int p = lane & 15;
    const int row = TE == 4 ? p : p / 2, col = TE == 4 ? 0 : 4 * (p % 2);
    const RouterW<TE, FULL> W{a.wr + ((size_t)s * seg + row) * a.E + e0 + min(col, a.E - 1 - e0), a.E,
                              a.E - 1 - e0 - min(col, a.E - 1 - e0)};
    float acc[TE];
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[j] = 0.0f;
    // One quarter (16 K steps) from its x words (16 bf16) and W sets.
    auto quarter = [&](const u32x4_t (&xw)[2], const f32x4_t *w) {
        float xf[16];
        unpack8(xw[0], *(float (*)[8])&xf[0]);
        unpack8(xw[1], *(float (*)[8])&xf[8]);
        if constexpr (TE == 4) {
            fma_block4(acc, w[0], xf);
        } else {
            fma_block8(acc, w[0], &xf[0]);
            fma_block8(acc, w[1], &xf[8]);
        }
    };
    const int ng = seg / (kRouterQK * kRouterGQ);
    if (ng > 0) {
        // A group: the lane's whole 128-byte x line (8 loads, back to back, so the line is fetched
        // once) and the W sets of its 4 quarters; GD groups in flight.
        struct Grp {
            u32x4_t x[2 * kRouterGQ];
            f32x4_t w[kRouterGQ * WQ];
        };
        auto fetch = [&](int g, Grp &r) {
#pragma unroll
            for (int i = 0; i < 2 * kRouterGQ; ++i) r.x[i] = *(const u32x4_t *)(xr + g * 64 + 8 * i);
#pragma unroll
            for (int i = 0; i < kRouterGQ * WQ; ++i) r.w[i] = W.load(g * kRouterGQ + i / WQ, i % WQ);
        };
        Grp gr[kRouterGD];
#pragma unroll
        for (int i = 0; i < kRouterGD; ++i) {   // the same load order as the refills in the loop
            fetch(min(i, ng - 1), gr[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Group g's quarters, then its registers refilled with group g + GD (past the end: the last
        // group again, so the number of loads in flight never changes); scheduling barriers keep the
        // refill after the FMAs and before the next group.
        auto group = [&](int g, Grp &r) {
#pragma unroll
            for (int qq = 0; qq < kRouterGQ; ++qq) {
                const u32x4_t xw[2] = {r.x[2 * qq], r.x[2 * qq + 1]};
                quarter(xw, &r.w[qq * WQ]);
            }
            __builtin_amdgcn_sched_barrier(0);
            fetch(min(g + kRouterGD, ng - 1), r);
            __builtin_amdgcn_sched_barrier(0);
        };
        // Whole rounds of GD groups without conditions (exact wait counts), then the rest.
        int g0 = 0;
        for (; g0 + kRouterGD <= ng; g0 += kRouterGD) {
#pragma unroll
            for (int i = 0; i < kRouterGD; ++i) group(g0 + i, gr[i]);
        }
#pragma unroll
        for (int i = 0; i < kRouterGD - 1; ++i)
            if (g0 + i < ng) group(g0 + i, gr[i]);
    }
    // Segment lengths that are not a multiple of 64: the remaining quarters one at a time.
    for (int qi = ng * kRouterGQ; qi < seg / kRouterQK; ++qi) {
        const u32x4_t xw[2] = {*(const u32x4_t *)(xr + qi * kRouterQK), *(const u32x4_t *)(xr + qi * kRouterQK + 8)};
        f32x4_t w[WQ];
#pragma unroll
        for (int h = 0; h < WQ; ++h) w[h] = W.load(qi, h);
        quarter(xw, w);
    }
    if (t < a.T) {
        float *dst = a.part + ((size_t)s * a.T + t) * a.E + e0;
#pragma unroll
        for (int j = 0; j < TE; ++j)
            if (e0 + j < a.E) dst[j] = acc[j];
    }
}

template <int TE>
__device__ __forceinline__ void router_task_te(const RouterArgs &a, int q)
{
    const int neg = (a.E + TE - 1) / TE;
    const int ntb = (a.T + kTokBlock - 1) / kTokBlock;
    const int eg = __builtin_amdgcn_readfirstlane(q % neg);
    const int tb = __builtin_amdgcn_readfirstlane((q / neg) % ntb);
    const int s = __builtin_amdgcn_readfirstlane(q / (neg * ntb));
    if (a.E % 4 == 0 && eg * TE + TE <= a.E) router_task_body<TE, true>(a, s, tb, eg * TE);
    else router_task_body<TE, false>(a, s, tb, eg * TE);
}

// Wave task q (< router_tasks(T, E)); q must be uniform over the wave.
__device__ __forceinline__ void router_task(const RouterArgs &a, int q)
{
    if (router_te(a.T, a.E) == 8) router_task_te<8>(a, q);
    else router_task_te<4>(a, q);
}

struct TopkArgs {
    const float *part;       // [8, T, E] partial sums
    const float *bias;       // [E] or nullptr
    int32_t *ids;            // [T, k]  (workspace or user)
    int32_t *ids_user;       // [T, k] or nullptr (second copy)
    float *w_user;           // [T, k] or nullptr
    uint64_t *blkmask;       // [nblk, E_local] token masks to OR into (token-per-wave path), or nullptr
    int32_t T, E, k, e_begin, E_local;
};

// Top-k and gate of token t with the lanes of one wave spanning the experts
// (e = lane + 64 v, v < NV, E <= 64 NV).  The 8 partial sums of
// each logit come straight from the workspace (a token's E partials of one
// segment are contiguous, so the loads coalesce), all 8 NV of them in flight;
// the logit is their ordered sum plus the bias.  Then k rounds of a wave-wide
// max over (logit, -id) keys; ids and gates go to global memory only.
template <int NV>
__device__ __forceinline__ void topk_token_wave(const TopkArgs &a, int t)
{
#pragma clang fp contract(off)
    const int l = threadIdx.x % kWave;
    const size_t sstride = (size_t)a.T * a.E;
    const float *row = a.part + (size_t)t * a.E;
    float p[NV][kRouterSegments];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int e = min(l + v * kWave, a.E - 1);
#pragma unroll
        for (int s = 0; s < kRouterSegments; ++s) p[v][s] = row[s * sstride + e];
    }
    float lv[NV];
    uint64_t key[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int e = l + v * kWave;
        float x = p[v][0];
#pragma unroll
        for (int s = 1; s < kRouterSegments; ++s) x = x + p[v][s];
        if (a.bias) x = x + a.bias[min(e, a.E - 1)];
        lv[v] = x;
        key[v] = e < a.E ? topk_key(x, e) : 0ull;
    }
    float top_logit = 0.0f, sel_logit = 0.0f;
    int sel_id = 0;
    for (int j = 0; j < a.k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) best = key[v] > best ? key[v] : best;
        best = wave_max_u64(best);
        const int e = topk_key_expert(best);
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (key[v] == best) key[v] = 0ull;
        const uint32_t ok = (uint32_t)(best >> 32);
        const float logit = __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
        if (j == 0) top_logit = logit;
        if (l == j) {
            sel_logit = logit;
            sel_id = e;
        }
    }
    float zsum = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (l + v * kWave < a.E) zsum += expf(lv[v] - top_logit);
    zsum = wave_sum_f32(zsum);
    if (l < a.k) {
        const size_t o = (size_t)t * a.k + l;
        a.ids[o] = sel_id;
        if (a.ids_user) a.ids_user[o] = sel_id;
        if (a.w_user) a.w_user[o] = expf(sel_logit - top_logit) / zsum;
        // the token's bit in its block's mask of every local expert it chose
        const int le = sel_id - a.e_begin;
        if (a.blkmask && le >= 0 && le < a.E_local)
            __hip_atomic_fetch_or(a.blkmask + (size_t)(t / kTokBlock) * a.E_local + le, 1ull << (t % kTokBlock),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Token-per-wave top-k: workgroup unit u covers tokens 4u .. 4u+3, one per wave.
__host__ __device__ inline int topk_wave_units(int T) { return (T + 3) / 4; }
__device__ __forceinline__ void topk_wave_unit(const TopkArgs &a, int u)
{
    const int t = u * 4 + (int)threadIdx.x / kWave;
    if (t >= a.T) return;
    if (a.E <= 128) topk_token_wave<2>(a, t);
    else if (a.E <= 256) topk_token_wave<4>(a, t);
    else if (a.E <= 512) topk_token_wave<8>(a, t);
    else topk_token_wave<16>(a, t);
}


struct CountArgs {
    const int32_t *ids;   // [T, k]
    int32_t *lrank;       // [T, k] rank of the token among the block's tokens of that expert
    int32_t *blkcnt;      // [nblk, E_local]
    uint64_t *blkmask;    // [nblk, E_local] bit l: token blk*64 + l chose the expert
    uint32_t *err;        // workspace error word (bad ids)
    int32_t T, E, k, e_begin, E_local;
};

// Histogram, token masks and in-block ranks for tokens [blk*64, +64) with
// lane = token: loop over the distinct local experts present, one ballot each.
// ids_lds: [64][k] ids of the block (filled by the caller); cnt_lds: E_local
// ints; mask_lds: E_local uint64.
__device__ __forceinline__ void count_block(const CountArgs &a, int blk, const int32_t *ids_lds,
                                            int32_t *cnt_lds, uint64_t *mask_lds)
{
    for (int e = threadIdx.x; e < a.E_local; e += blockDim.x) {
        cnt_lds[e] = 0;
        mask_lds[e] = 0;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int l = threadIdx.x;
        const int t = blk * kTokBlock + l;
        uint32_t pend = 0;
        bool bad = false;
        if (t < a.T) {
            for (int j = 0; j < a.k; ++j) {
                const int id = ids_lds[l * a.k + j];
                if (id < 0 || id >= a.E) bad = true;
                for (int j2 = 0; j2 < j; ++j2)
                    if (ids_lds[l * a.k + j2] == id) bad = true;
                const int le = id - a.e_begin;
                if (le >= 0 && le < a.E_local) pend |= 1u << j;
            }
        }
        if (bad) {   // report the token, give none of its choices a slot
            raise_error(a.err, kErrInval, (uint32_t)t);
            for (int j = 0; j < a.k; ++j) a.lrank[(size_t)t * a.k + j] = -1;
            pend = 0;
        }
        for (;;) {
            const uint64_t active = __ballot(pend != 0);
            if (active == 0) break;
            const int leader = __ffsll((unsigned long long)active) - 1;
            const int my_first = pend ? ids_lds[l * a.k + (__ffs(pend) - 1)] : -1;
            const int e = __shfl(my_first, leader, kWave);
            int jj = -1;
            for (int j = 0; j < a.k; ++j)
                if (((pend >> j) & 1u) && ids_lds[l * a.k + j] == e) jj = j;
            const uint64_t m = __ballot(jj >= 0);
            if (jj >= 0) {
                a.lrank[(size_t)t * a.k + jj] = __popcll(m & lanemask_lt());
                pend &= ~(1u << jj);
            }
            if (l == 0) {
                cnt_lds[e - a.e_begin] = __popcll(m);
                mask_lds[e - a.e_begin] = m;
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < a.E_local; e += blockDim.x) {
        a.blkcnt[(size_t)blk * a.E_local + e] = cnt_lds[e];
        a.blkmask[(size_t)blk * a.E_local + e] = mask_lds[e];
    }
    __syncthreads();
}

}  // namespace mk
