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
// per step).  Each of the 8 segments is an independent small SIMT GEMM
// [T x seg] . [seg x E]; one workgroup unit = (segment, block of BT tokens,
// block of BE experts), staged through LDS in K chunks of KC with the chunks
// two ahead prefetched into registers; thread (ty, tx) owns TT tokens x TE experts
// and walks k in ascending order, so every accumulator is one chain.
struct RouterCfg {
    int BE, TE, TT, BT;
};

// The configurations, by index; router_cfg_index picks one from E.
__host__ __device__ __forceinline__ constexpr RouterCfg router_cfg_at(int ci)
{
    return ci == 0 ? RouterCfg{8, 4, 1, 128}
         : ci == 1 ? RouterCfg{16, 8, 1, 128}
         : ci == 2 ? RouterCfg{32, 8, 2, 128}
         : ci == 3 ? RouterCfg{64, 8, 4, 128}
                   : RouterCfg{32, 4, 1, 32};
}
__host__ __device__ __forceinline__ constexpr int router_cfg_index(int E)
{
    return E <= 8 ? 0 : E <= 16 ? 1 : E <= 32 ? 2 : E <= 64 ? 3 : 4;
}
__host__ __device__ __forceinline__ constexpr RouterCfg router_cfg(int E) { return router_cfg_at(router_cfg_index(E)); }

__host__ __device__ inline int router_units(int T, int E)
{
    const RouterCfg c = router_cfg(E);
    return ((T + c.BT - 1) / c.BT) * ((E + c.BE - 1) / c.BE) * kRouterSegments;
}

constexpr int kRouterKC = 64;   // K chunk per LDS stage (a smaller divisor of the segment if needed)
// LDS row stride of the x tile (bf16): 16 bytes of padding per row put the
// rows that the lanes of one read touch in different banks.
constexpr int kRouterXS = kRouterKC + 8;

template <int CI>
__device__ __forceinline__ void router_unit_tiled(const RouterArgs &a, int unit, char *x0, char *w0, char *x1, char *w1)
{
#pragma clang fp contract(off)
    constexpr int BE = router_cfg_at(CI).BE, TE = router_cfg_at(CI).TE, TT = router_cfg_at(CI).TT;
    constexpr int NX = BE / TE;            // threads along the experts
    constexpr int NY = 256 / NX;           // threads along the tokens
    constexpr int BT = NY * TT;
    static_assert(router_cfg_at(CI).BT == BT, "the thread layout covers the configured token block");
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

    // a stage is an x tile [BT][kRouterXS] bf16 (<= 32 KiB) and a W tile [kRouterKC][BE] fp32 (<= 16 KiB)
    static_assert(BT * kRouterXS * 2 <= 32768 && kRouterKC * BE * 4 <= 16384, "router stage sizes");
    static_assert(BT * kRouterXS * 2 + kRouterKC * BE * 4 <= 34816, "router stage fits one 34 KiB array");
    const int cpr = KC / 8;
    const int nk = seg / KC;
    // Two register sets of prefetched chunks (A, B): a chunk is fetched two
    // chunk-computations before it is written to LDS.  Fetches past the last
    // chunk re-read the last one (unconditional loads keep the compiler's
    // wait counts exact).
    u32x4_t xrA[XPT], xrB[XPT];
    float wrA[WPT], wrB[WPT];
    // The token rows this thread fetches from, fixed for the whole unit: computed once, so the
    // chunk loop has no pointer loads (whose waits would drain the prefetches in flight).
    const uint16_t *xrow[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int c = min(tid + j * 256, BT * cpr - 1);
        const int row = c / cpr, cc = c - row * cpr;
        const int t = min(tb * BT + row, a.T - 1);
        xrow[j] = token_row(a.src, t, a.d) + k_base + cc * 8;
    }
#define MK_ROUTER_FETCH(xr, wrg, chunk)                                                           \
    do {                                                                                          \
        const int k0_ = min((chunk), nk - 1) * KC;                                                \
        _Pragma("unroll") for (int j = 0; j < XPT; ++j) xr[j] = *(const u32x4_t *)(xrow[j] + k0_); \
        _Pragma("unroll") for (int j = 0; j < WPT; ++j) {                                         \
            const int c = min(tid + j * 256, KC * BE - 1);                                        \
            const int kk = c / BE, e = c - kk * BE;                                               \
            wrg[j] = a.wr[(size_t)(k_base + k0_ + kk) * a.E + min(eb * BE + e, a.E - 1)];         \
        }                                                                                         \
    } while (0)
#define MK_ROUTER_STASH(xr, wrg, xs, ws)                                                          \
    do {                                                                                          \
        _Pragma("unroll") for (int j = 0; j < XPT; ++j) {                                         \
            const int c = tid + j * 256;                                                          \
            if (c < BT * cpr)                                                                     \
                *(u32x4_t *)((uint16_t *)(xs) + (c / cpr) * kRouterXS + (c % cpr) * 8) = xr[j];  \
        }                                                                                         \
        _Pragma("unroll") for (int j = 0; j < WPT; ++j) {                                         \
            const int c = tid + j * 256;                                                          \
            if (c < KC * BE) ((float *)(ws))[c] = wrg[j];                                        \
        }                                                                                         \
    } while (0)
#define MK_ROUTER_COMPUTE(xs, ws)                                                                 \
    do {                                                                                          \
        const uint16_t *xt = (const uint16_t *)(xs);                                              \
        const float *wt = (const float *)(ws);                                                    \
        for (int k8 = 0; k8 < KC; k8 += 8) {                                                      \
            float xf[TT][8];                                                                      \
            _Pragma("unroll") for (int i = 0; i < TT; ++i)                                        \
                unpack8(*(const u32x4_t *)(xt + (ty * TT + i) * kRouterXS + k8), xf[i]);         \
            _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                       \
                float wv[TE];                                                                     \
                _Pragma("unroll") for (int j = 0; j < TE; j += 4) {                               \
                    const float4 w4 = *(const float4 *)(wt + (k8 + q) * BE + tx * TE + j);        \
                    wv[j] = w4.x;                                                                 \
                    wv[j + 1] = w4.y;                                                             \
                    wv[j + 2] = w4.z;                                                             \
                    wv[j + 3] = w4.w;                                                             \
                }                                                                                 \
                _Pragma("unroll") for (int i = 0; i < TT; ++i)                                    \
                    _Pragma("unroll") for (int j = 0; j < TE; ++j)                                \
                        acc[i][j] = __builtin_fmaf(xf[i][q], wv[j], acc[i][j]);                   \
            }                                                                                     \
        }                                                                                         \
    } while (0)

    float acc[TT][TE];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

    MK_ROUTER_FETCH(xrA, wrA, 0);
    MK_ROUTER_FETCH(xrB, wrB, 1);
    MK_ROUTER_STASH(xrA, wrA, x0, w0);
    MK_ROUTER_FETCH(xrA, wrA, 2);
    __syncthreads();
    for (int kc = 0; kc < nk; kc += 2) {
        // stage 0 holds chunk kc, B holds chunk kc + 1, A holds chunk kc + 2
        MK_ROUTER_COMPUTE(x0, w0);
        MK_ROUTER_STASH(xrB, wrB, x1, w1);
        MK_ROUTER_FETCH(xrB, wrB, kc + 3);
        __syncthreads();
        if (kc + 1 >= nk) break;
        MK_ROUTER_COMPUTE(x1, w1);
        MK_ROUTER_STASH(xrA, wrA, x0, w0);
        MK_ROUTER_FETCH(xrA, wrA, kc + 4);
        __syncthreads();
    }
#undef MK_ROUTER_FETCH
#undef MK_ROUTER_STASH
#undef MK_ROUTER_COMPUTE
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int t = tb * BT + ty * TT + i;
        if (t >= a.T) continue;
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int e = eb * BE + tx * TE + j;
            if (e < a.E) a.part[((size_t)s * a.T + t) * a.E + e] = acc[i][j];
        }
    }
}

// One workgroup unit of the partial-sum phase; two LDS stages, each an x part
// (x0, x1: 32 KiB) and a W part (w0, w1: 16 KiB).
__device__ __forceinline__ void router_unit(const RouterArgs &a, int unit, char *x0, char *w0, char *x1, char *w1)
{
    switch (router_cfg_index(a.E)) {
    case 0: router_unit_tiled<0>(a, unit, x0, w0, x1, w1); break;
    case 1: router_unit_tiled<1>(a, unit, x0, w0, x1, w1); break;
    case 2: router_unit_tiled<2>(a, unit, x0, w0, x1, w1); break;
    case 3: router_unit_tiled<3>(a, unit, x0, w0, x1, w1); break;
    default: router_unit_tiled<4>(a, unit, x0, w0, x1, w1); break;
    }
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
