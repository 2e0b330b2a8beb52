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
    float *part;        // [8, E, T] per-segment partial sums
    int32_t T, d, E;
};

__device__ __forceinline__ const uint16_t *token_row(const SrcRows &s, int t, int d)
{
    const int sh = t / s.rows_per_src;
    return s.p[sh] + (size_t)(t - sh * s.rows_per_src) * d;
}

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f[2 * p] = __uint_as_float(w[p] << 16);
        f[2 * p + 1] = __uint_as_float(w[p] & 0xFFFF0000u);
    }
}

// ---------------------------------------------------------------- partial sums
// part[s][e][t] = fma chain over i in K segment s, ascending (fp32, one rounding
// per step).  Each of the 8 segments is an independent small SIMT GEMM
// [T x seg] . [seg x E]; one workgroup unit = (segment, block of BT tokens,
// block of BE experts), staged through LDS in K chunks of KC with the next
// chunk prefetched into registers; thread (ty, tx) owns TT tokens x TE experts
// and walks k in ascending order, so every accumulator is one chain.
struct RouterCfg {
    int BE, TE, TT, BT;
};

__host__ __device__ inline RouterCfg router_cfg(int E)
{
    if (E <= 8) return RouterCfg{8, 8, 1, 256};
    if (E <= 16) return RouterCfg{16, 8, 1, 128};
    if (E <= 32) return RouterCfg{32, 8, 2, 128};
    if (E <= 64) return RouterCfg{64, 8, 4, 128};
    return RouterCfg{64, 4, 1, 16};
}

__host__ __device__ inline int router_units(int T, int E)
{
    const RouterCfg c = router_cfg(E);
    return ((T + c.BT - 1) / c.BT) * ((E + c.BE - 1) / c.BE) * kRouterSegments;
}

constexpr int kRouterKC = 64;   // K chunk per LDS stage (a smaller divisor of the segment if needed)

template <int BE, int TE, int TT>
__device__ void router_unit_tiled(const RouterArgs &a, int unit, char *x0, char *w0, char *x1, char *w1)
{
#pragma clang fp contract(off)
    constexpr int NX = BE / TE;            // threads along the experts
    constexpr int NY = 256 / NX;           // threads along the tokens
    constexpr int BT = NY * TT;
    constexpr int XCH = BT * kRouterKC / 8;              // 16-byte x chunks per stage (max)
    constexpr int XPT = (XCH + 255) / 256;               // per thread
    constexpr int WPT = (kRouterKC * BE + 255) / 256;    // W floats per thread per stage (max)
    const int seg = a.d / kRouterSegments;
    const int KC = seg % kRouterKC == 0 ? kRouterKC : (seg % 32 == 0 ? 32 : 16);
    const int ntb = (a.T + BT - 1) / BT;
    const int neb = (a.E + BE - 1) / BE;
    const int tb = unit % ntb;
    const int eb = (unit / ntb) % neb;
    const int s = unit / (ntb * neb);
    const int tid = threadIdx.x;
    const int tx = tid % NX, ty = tid / NX;
    const int k_base = s * seg;

    // a stage is an x tile [BT][kRouterKC] bf16 (<= 32 KiB) and a W tile [kRouterKC][BE] fp32 (<= 16 KiB)
    static_assert(BT * kRouterKC * 2 <= 32768 && kRouterKC * BE * 4 <= 16384, "router stage sizes");
    static_assert(BT * kRouterKC * 2 + kRouterKC * BE * 4 <= 34816, "router stage fits one 34 KiB array");
    const int cpr = KC / 8;
    uint4 xr[XPT];
    float wrg[WPT];
#define MK_ROUTER_FETCH(k0)                                                                       \
    do {                                                                                          \
        _Pragma("unroll") for (int j = 0; j < XPT; ++j) {                                         \
            const int c = min(tid + j * 256, BT * cpr - 1);                                       \
            const int row = c / cpr, cc = c - row * cpr;                                          \
            const int t = min(tb * BT + row, a.T - 1);                                            \
            xr[j] = *(const uint4 *)(token_row(a.src, t, a.d) + k_base + (k0) + cc * 8);          \
        }                                                                                         \
        _Pragma("unroll") for (int j = 0; j < WPT; ++j) {                                         \
            const int c = min(tid + j * 256, KC * BE - 1);                                        \
            const int kk = c / BE, e = c - kk * BE;                                               \
            wrg[j] = a.wr[(size_t)(k_base + (k0) + kk) * a.E + min(eb * BE + e, a.E - 1)];        \
        }                                                                                         \
    } while (0)
#define MK_ROUTER_STASH(xs, ws)                                                                       \
    do {                                                                                          \
        _Pragma("unroll") for (int j = 0; j < XPT; ++j) {                                         \
            const int c = tid + j * 256;                                                          \
            if (c < BT * cpr)                                                                     \
                *(uint4 *)((uint16_t *)(xs) + (c / cpr) * kRouterKC + (c % cpr) * 8) = xr[j];     \
        }                                                                                         \
        _Pragma("unroll") for (int j = 0; j < WPT; ++j) {                                         \
            const int c = tid + j * 256;                                                          \
            if (c < KC * BE) ((float *)(ws))[c] = wrg[j];                                        \
        }                                                                                         \
    } while (0)

    float acc[TT][TE];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

    MK_ROUTER_FETCH(0);
    MK_ROUTER_STASH(x0, w0);
    __syncthreads();
    const int nk = seg / KC;
    for (int kc = 0; kc < nk; ++kc) {
        if (kc + 1 < nk) MK_ROUTER_FETCH((kc + 1) * KC);
        const uint16_t *xt = (const uint16_t *)((kc & 1) ? x1 : x0);
        const float *wt = (const float *)((kc & 1) ? w1 : w0);
        for (int k8 = 0; k8 < KC; k8 += 8) {
            float xf[TT][8];
#pragma unroll
            for (int i = 0; i < TT; ++i) unpack8(*(const uint4 *)(xt + (ty * TT + i) * kRouterKC + k8), xf[i]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float wv[TE];
#pragma unroll
                for (int j = 0; j < TE; j += 4) {
                    const float4 w4 = *(const float4 *)(wt + (k8 + q) * BE + tx * TE + j);
                    wv[j] = w4.x;
                    wv[j + 1] = w4.y;
                    wv[j + 2] = w4.z;
                    wv[j + 3] = w4.w;
                }
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int j = 0; j < TE; ++j) acc[i][j] = __builtin_fmaf(xf[i][q], wv[j], acc[i][j]);
            }
        }
        if (kc + 1 < nk) {
            if (kc & 1) MK_ROUTER_STASH(x0, w0);
            else MK_ROUTER_STASH(x1, w1);
        }
        __syncthreads();
    }
#undef MK_ROUTER_FETCH
#undef MK_ROUTER_STASH
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int t = tb * BT + ty * TT + i;
        if (t >= a.T) continue;
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int e = eb * BE + tx * TE + j;
            if (e < a.E) a.part[((size_t)s * a.E + e) * a.T + t] = acc[i][j];
        }
    }
}

// One workgroup unit of the partial-sum phase; two LDS stages, each an x part
// (x0, x1: 32 KiB) and a W part (w0, w1: 16 KiB).
__device__ __forceinline__ void router_unit(const RouterArgs &a, int unit, char *x0, char *w0, char *x1, char *w1)
{
    if (a.E <= 8) router_unit_tiled<8, 8, 1>(a, unit, x0, w0, x1, w1);
    else if (a.E <= 16) router_unit_tiled<16, 8, 1>(a, unit, x0, w0, x1, w1);
    else if (a.E <= 32) router_unit_tiled<32, 8, 2>(a, unit, x0, w0, x1, w1);
    else if (a.E <= 64) router_unit_tiled<64, 8, 4>(a, unit, x0, w0, x1, w1);
    else router_unit_tiled<64, 4, 1>(a, unit, x0, w0, x1, w1);
}

struct TopkArgs {
    const float *part;       // [8, E, T] partial sums
    const float *bias;       // [E] or nullptr
    int32_t *ids;            // [T, k]  (workspace or user)
    int32_t *ids_user;       // [T, k] or nullptr (second copy)
    float *w_user;           // [T, k] or nullptr
    int32_t T, E, k;
};

// Row stride (floats) of one token's logits in LDS: padded by one for E <= 64,
// where one lane reads one token's row, so that the lanes' rows fall in
// different banks; unpadded above, where one wave reads one row.
__host__ __device__ inline int topk_lg_stride(int E) { return E <= 64 ? E + 1 : E; }

constexpr int kTopkLdsBytes = 32768;   // LDS for the logits of one top-k sub-block

// Tokens per LDS sub-block of the top-k step: SB rows of logits fit in kTopkLdsBytes.
__host__ __device__ inline int topk_subblock(int E)
{
    int sb = kTokBlock;
    while (sb > 1 && (long)sb * topk_lg_stride(E) * 4 > kTopkLdsBytes) sb >>= 1;
    return sb;
}

// Logits of tokens [t0, t0 + nt) into LDS: lg[tl * stride + e] = ((P0 + P1) + ... + P7) + bias.
// Each thread keeps the 8 partial loads of 4 logits in flight.
__device__ __forceinline__ void block_logits(const TopkArgs &a, int t0, int nt, float *lg)
{
#pragma clang fp contract(off)
    const int n = nt * a.E;
    const size_t sstride = (size_t)a.E * a.T;
    for (int base = 0; base < n; base += 4 * (int)blockDim.x) {
        float p[4][kRouterSegments];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = base + u * (int)blockDim.x + (int)threadIdx.x;
            const int i2 = idx < n ? idx : n - 1;
            const float *src = a.part + (size_t)(i2 / nt) * a.T + t0 + i2 % nt;
#pragma unroll
            for (int s = 0; s < kRouterSegments; ++s) p[u][s] = src[s * sstride];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = base + u * (int)blockDim.x + (int)threadIdx.x;
            if (idx >= n) break;
            const int tl = idx % nt, e = idx / nt;
            float v = p[u][0];
#pragma unroll
            for (int s = 1; s < kRouterSegments; ++s) v = v + p[u][s];
            if (a.bias) v = v + a.bias[e];
            lg[tl * topk_lg_stride(a.E) + e] = v;
        }
    }
}

// Top-k and gate for one token whose E logits are in `row` (LDS), lane = token
// (E <= 64): a sequential selection over ascending ids, where a strict '>'
// keeps the lower id on ties (and -0 ties with +0, as float compare does).
// The chosen ids go to ids_row (LDS, k entries).
__device__ __forceinline__ void topk_one_lane(const TopkArgs &a, const float *row, int t, int32_t *ids_row)
{
    float lv[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) lv[e] = e < a.E ? row[e] : 0.0f;
    uint64_t taken = 0;
    float top = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        int best = -1;
        float bl = 0.0f;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
            if (e < a.E && !((taken >> e) & 1ull) && (best < 0 || lv[e] > bl)) {
                best = e;
                bl = lv[e];
            }
        }
        taken |= 1ull << best;
        if (j == 0) top = bl;
        ids_row[j] = best;
        const size_t o = (size_t)t * a.k + j;
        a.ids[o] = best;
        if (a.ids_user) a.ids_user[o] = best;
    }
    if (a.w_user) {
        float zsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 64; ++e)
            if (e < a.E) zsum += expf(lv[e] - top);
        for (int j = 0; j < a.k; ++j) a.w_user[(size_t)t * a.k + j] = expf(row[ids_row[j]] - top) / zsum;
    }
}

// Top-k for one token with lanes spanning the experts (E > 64): k rounds of a
// wave-wide max over (logit, -id) keys.
__device__ __forceinline__ void topk_one_wave(const TopkArgs &a, const float *row, int t, int32_t *ids_row)
{
    constexpr int kMaxV = 16;   // E <= 1024
    const int l = threadIdx.x % kWave;
    const int nv = (a.E + kWave - 1) / kWave;
    float lv[kMaxV];
    uint64_t key[kMaxV];
#pragma unroll
    for (int v = 0; v < kMaxV; ++v) {
        const int e = l + v * kWave;
        const bool ok = v < nv && e < a.E;
        lv[v] = ok ? row[e] : 0.0f;
        key[v] = ok ? topk_key(lv[v], e) : 0ull;
    }
    float top_logit = 0.0f, zsum = 0.0f, sel_logit = 0.0f;
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
        ids_row[l] = sel_id;
    }
}

// Top-k and gate for tokens [blk*64, blk*64 + 64), in sub-blocks whose logits
// are first gathered into LDS (lg: kTopkLdsBytes).  ids_lds: [64][k] (LDS).
__device__ void topk_block(const TopkArgs &a, int blk, float *lg, int32_t *ids_lds)
{
    const int w = threadIdx.x / kWave;
    const int l = threadIdx.x % kWave;
    const int sb = topk_subblock(a.E);
    const int t_end = min(a.T, (blk + 1) * kTokBlock);
    for (int t0 = blk * kTokBlock; t0 < t_end; t0 += sb) {
        const int nt = min(sb, t_end - t0);
        block_logits(a, t0, nt, lg);
        __syncthreads();
        if (a.E <= 64) {
            if (w == 0 && l < nt)
                topk_one_lane(a, lg + l * topk_lg_stride(a.E), t0 + l, ids_lds + (t0 - blk * kTokBlock + l) * a.k);
        } else {
            for (int tl = w; tl < nt; tl += (int)blockDim.x / kWave)
                topk_one_wave(a, lg + tl * topk_lg_stride(a.E), t0 + tl, ids_lds + (t0 - blk * kTokBlock + tl) * a.k);
        }
        __syncthreads();
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
