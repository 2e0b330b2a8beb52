// route_dev.h -- router device code: fp32 logits in the fixed segmented order,
// top-k selection with ordered keys, softmax gate, and the per-block expert
// histogram with in-block ranks from wave ballots.
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
    const float *bias;  // [E] or nullptr
    float *logits;      // [T, E]
    int32_t T, d, E;
};

__device__ __forceinline__ const uint16_t *token_row(const SrcRows &s, int t, int d)
{
    const int sh = t / s.rows_per_src;
    return s.p[sh] + (size_t)(t - sh * s.rows_per_src) * d;
}

// One block of 256 threads computes logits for TB = (64/EL)*TPL tokens x EL
// experts.  Wave w runs the chains of segments w and w+4; lane = (token group
// g, expert e).  Partials meet in LDS and are added in segment order.
// lds: 8 * TB * EL floats.
template <int TPL, int EL>
__device__ void router_logits_block(const RouterArgs &a, int tb, int eb, float *lds)
{
#pragma clang fp contract(off)
    constexpr int G = kWave / EL;
    constexpr int TB = G * TPL;
    const int w = threadIdx.x / kWave;
    const int l = threadIdx.x % kWave;
    const int el = l % EL;
    const int g = l / EL;
    const int e = eb * EL + el;
    const int ec = e < a.E ? e : a.E - 1;   // idle lanes compute a real column, then drop it
    const int seg = a.d / kRouterSegments;
    const int s0 = w, s1 = w + 4;

    const uint16_t *xr[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        int t = tb * TB + g * TPL + j;
        t = t < a.T ? t : a.T - 1;
        xr[j] = token_row(a.src, t, a.d);
    }
    float acc0[TPL], acc1[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) { acc0[j] = 0.0f; acc1[j] = 0.0f; }

    const float *w0 = a.wr + (size_t)(s0 * seg) * a.E + ec;
    const float *w1 = a.wr + (size_t)(s1 * seg) * a.E + ec;
    for (int c = 0; c < seg; c += 8) {
        float wa[8], wb[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            wa[q] = w0[(size_t)(c + q) * a.E];
            wb[q] = w1[(size_t)(c + q) * a.E];
        }
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const uint4 xa = *(const uint4 *)(xr[j] + s0 * seg + c);
            const uint4 xb = *(const uint4 *)(xr[j] + s1 * seg + c);
            const uint32_t va[4] = {xa.x, xa.y, xa.z, xa.w};
            const uint32_t vb[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                acc0[j] = __builtin_fmaf(__uint_as_float(va[p] << 16), wa[2 * p], acc0[j]);
                acc0[j] = __builtin_fmaf(__uint_as_float(va[p] & 0xFFFF0000u), wa[2 * p + 1], acc0[j]);
                acc1[j] = __builtin_fmaf(__uint_as_float(vb[p] << 16), wb[2 * p], acc1[j]);
                acc1[j] = __builtin_fmaf(__uint_as_float(vb[p] & 0xFFFF0000u), wb[2 * p + 1], acc1[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        lds[(s0 * TB + g * TPL + j) * EL + el] = acc0[j];
        lds[(s1 * TB + g * TPL + j) * EL + el] = acc1[j];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < TB * EL; idx += blockDim.x) {
        const int tt = idx / EL, ee = idx % EL;
        const int t = tb * TB + tt, e2 = eb * EL + ee;
        if (t < a.T && e2 < a.E) {
            float v = lds[tt * EL + ee];
#pragma unroll
            for (int s = 1; s < kRouterSegments; ++s)
                v = v + lds[(s * TB + tt) * EL + ee];
            if (a.bias) v = v + a.bias[e2];
            a.logits[(size_t)t * a.E + e2] = v;
        }
    }
    __syncthreads();
}

struct TopkArgs {
    const float *logits;     // [T, E]
    int32_t *ids;            // [T, k]  (workspace or user)
    int32_t *ids_user;       // [T, k] or nullptr (second copy)
    float *w_user;           // [T, k] or nullptr
    int32_t T, E, k;
};

// Top-k and gate for tokens [blk*64, blk*64 + 64): wave w handles 16 tokens,
// lanes span the experts.  Writes ids into ids_lds[64][k] too.
__device__ __forceinline__ void topk_block(const TopkArgs &a, int blk, int32_t *ids_lds)
{
    constexpr int kMaxV = 16;   // E <= 1024
    const int w = threadIdx.x / kWave;
    const int l = threadIdx.x % kWave;
    const int nv = (a.E + kWave - 1) / kWave;
    for (int tt = 0; tt < 16; ++tt) {
        const int tl = w * 16 + tt;
        const int t = blk * kTokBlock + tl;
        if (t >= a.T) break;
        const float *lrow = a.logits + (size_t)t * a.E;
        float lv[kMaxV];
        uint64_t key[kMaxV];
#pragma unroll
        for (int v = 0; v < kMaxV; ++v) {
            const int e = l + v * kWave;
            const bool ok = v < nv && e < a.E;
            lv[v] = ok ? lrow[e] : 0.0f;
            key[v] = ok ? topk_key(lv[v], e) : 0ull;
        }
        float top_logit = 0.0f;
        float zsum = 0.0f;
        float sel_logit = 0.0f;   // lane j (< k) keeps the logit of the j-th choice
        int sel_id = 0;
        for (int j = 0; j < a.k; ++j) {
            uint64_t best = 0;
#pragma unroll
            for (int v = 0; v < kMaxV; ++v) best = key[v] > best ? key[v] : best;
            best = wave_max_u64(best);
            const int e = topk_key_expert(best);
#pragma unroll
            for (int v = 0; v < kMaxV; ++v)
                if (key[v] == best) key[v] = 0ull;
            const uint32_t ok = (uint32_t)(best >> 32);
            const float logit = __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
            if (j == 0) top_logit = logit;
            if (l == j) { sel_logit = logit; sel_id = e; }
        }
#pragma unroll
        for (int v = 0; v < kMaxV; ++v) {
            const int e = l + v * kWave;
            if (v < nv && e < a.E) zsum += expf(lv[v] - top_logit);
        }
        zsum = wave_sum_f32(zsum);
        if (l < a.k) {
            const size_t o = (size_t)t * a.k + l;
            a.ids[o] = sel_id;
            if (a.ids_user) a.ids_user[o] = sel_id;
            if (a.w_user) a.w_user[o] = expf(sel_logit - top_logit) / zsum;
            if (ids_lds) ids_lds[tl * a.k + l] = sel_id;
        }
    }
}

struct CountArgs {
    const int32_t *ids;   // [T, k]
    int32_t *lrank;       // [T, k] rank of the token among the block's tokens of that expert
    int32_t *blkcnt;      // [nblk, E_local]
    uint32_t *err;        // workspace error word (bad ids)
    int32_t T, E, k, e_begin, E_local;
};

// Histogram and in-block ranks for tokens [blk*64, +64) with lane = token:
// loop over the distinct local experts present, one ballot each.
// ids_lds: [64][k] ids of the block (filled by the caller); cnt_lds: E_local ints.
__device__ __forceinline__ void count_block(const CountArgs &a, int blk, const int32_t *ids_lds,
                                            int32_t *cnt_lds)
{
    for (int e = threadIdx.x; e < a.E_local; e += blockDim.x) cnt_lds[e] = 0;
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
            if (l == 0) cnt_lds[e - a.e_begin] = __popcll(m);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < a.E_local; e += blockDim.x)
        a.blkcnt[(size_t)blk * a.E_local + e] = cnt_lds[e];
    __syncthreads();
}

}  // namespace mk
