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
// per step).  The chains run on the matrix cores: v_mfma_f32_4x4x1_16b_f32 is
// 16 independent 4x4 outer products with K = 1, i.e. for each of its 256
// outputs exactly one fused multiply-add, and a sequence of them over
// ascending i is the fma chain itself (bit-exact against fmaf chains on
// gfx950).  It retires 256 fmas in 8 cycles, twice the rate of scalar-lane
// fp32 FMAs, and needs each weight in only one lane per output column.
//
// A wave task is (segment s, block of 32 tokens, group of 8 experts).  MFMA
// operand layout (A: lanes 4b .. 4b + 3 of block b give its 4 rows; B: lane l
// gives column l % 4 of block l / 4; output lane l, register r is row
// 4 (l / 4) + r, column l of the blocks' B lanes):
//   A lane l = x of token 32 tb + (l % 32)  (lanes 32..63 repeat 0..31)
//   B lane l = W_r[i][e0 + 4 (l / 32) + l % 4]
// so output lane l, register r is token 32 tb + 4 ((l % 32) / 4) + r,
// expert e0 + 4 (l / 32) + l % 4.
// Both operands are staged per wave in LDS, a chunk of kRtKC steps at a time,
// double buffered, from coalesced loads one chunk ahead: x as 32 token rows
// (16 lanes per 256-byte row segment, so a load touches whole lines; a lane
// then reads its own row 8 steps at a time), the weights transposed to 8
// expert rows (padded so the rows sit on distinct banks; a lane reads 4 steps
// of its column at a time).
constexpr int kRtTok = 32;                    // tokens per wave task
constexpr int kRtExp = 8;                     // experts per wave task

// Staging geometry for KC K steps per chunk (128 in the router's own launch, 64 in the fused kernel,
// whose eight waves share the GEMM's 128 KiB of stage arrays).
template <int KC, int NG = 1>
struct RtStage {
    static constexpr int WS = KC + 4;                 // LDS row stride of the staged weights (floats)
    static constexpr int XS = KC + 8;                 // LDS row stride of the staged x rows (bf16)
    static constexpr int WBUF = kRtExp * WS * 4;      // bytes of one expert group's weight buffer
    static constexpr int XBUF = kRtTok * XS * 2;      // bytes of one x buffer
    static constexpr int LDS_PER_WAVE = 2 * (NG * WBUF + XBUF);
};
constexpr int kRtKC = 128;                    // K steps per staged chunk of the router launch
constexpr int kRtKCFused = 64;                // ... of the fused kernel
constexpr int kRtKCPair = 32;                 // ... of the fused kernel, two or four expert groups per task
constexpr int kRtLdsPerWave = RtStage<kRtKC>::LDS_PER_WAVE;

// NG expert groups per task: NG independent chains per lane (the matrix core issues the next
// group's op while the previous one's result is pending: one dependent 4x4x1 chain waits ~48 cycles
// per step, two interleaved chains ~22 per op, four ~13, measured on the part).
__host__ __device__ inline int router_tasks(int T, int E, int NG = 1)
{
    return ((T + kRtTok - 1) / kRtTok) * ((E + kRtExp * NG - 1) / (kRtExp * NG)) * kRouterSegments;
}

typedef __attribute__((address_space(3))) float lds_float_t;
typedef __attribute__((address_space(3))) char lds_byte_t;

// FULL: the 8 NG columns exist and E % 4 == 0 (16-byte weight loads); otherwise
// one load per column, columns past E repeating the last (never stored).
// lds: this wave's RtStage<KC, NG>::LDS_PER_WAVE bytes.
template <bool FULL, int KC, int NG>
__device__ __forceinline__ void router_task_body(const RouterArgs &a, int s, int tb, int e0, lds_byte_t *lds)
{
    constexpr int kRtKC = KC;
    constexpr int kRtWS = RtStage<KC, NG>::WS, kRtXS = RtStage<KC, NG>::XS;
    constexpr int kRtWBuf = RtStage<KC, NG>::WBUF, kRtXBuf = RtStage<KC, NG>::XBUF;
    typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
    typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
    const int lane = threadIdx.x % kWave;
    const int seg = a.d / kRouterSegments;   // a multiple of 16 (d % 128 == 0)
    const int nch = (seg + kRtKC - 1) / kRtKC;
    const int eb = 4 * (lane >> 5) + (lane & 3);   // this lane's B column in the group
    // x staging: a chunk row is KC / 8 pieces of 16 bytes; lane l loads rows XR i + l / XP (i < 32 / XR),
    // piece l % XP, with XP = KC / 8 pieces per row and XR = 64 / XP rows per load.
    constexpr int XP = kRtKC / 8, XR = kWave / XP, XI = kRtTok / XR;
    const uint16_t *xrow[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i)
        xrow[i] = token_row(a.src, min(tb * kRtTok + XR * i + lane / XP, a.T - 1), a.d) + (size_t)s * seg +
                  8 * (lane % XP);
    // Weight staging: lane l loads rows (l / 2) + 32 i (i < KC / 32) of a chunk, columns 8 g + 4 (l % 2)
    // .. + 3 of group g (columns past E: the last one again).
    const int cl = 4 * (lane & 1);
    const float *wseg = a.wr + (size_t)s * seg * a.E;
    constexpr int WI = kRtKC / 32;
    struct Regs {
        u32x4_t x[XI];
        f32x4_t w[NG][WI];
    };
    // Chunk c into registers (past the end: the last chunk again; steps past the segment: clamped).
    auto fetch = [&](int c, Regs &r) {
        const int cc = min(c, nch - 1);
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int row = min(cc * kRtKC + (lane >> 1) + 32 * i, seg - 1);
            const float *q = wseg + (size_t)row * a.E;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int col = e0 + 8 * g + cl;
                if (FULL) {
                    r.w[g][i] = *(const f32x4_t *)(q + col);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) r.w[g][i][j] = q[min(col + j, a.E - 1)];
                }
            }
        }
        const int k0 = min(cc * kRtKC + 8 * (lane % XP), seg - 8) - 8 * (lane % XP);
#pragma unroll
        for (int i = 0; i < XI; ++i) r.x[i] = *(const u32x4_t *)(xrow[i] + k0);
    };
    auto wbuf = [&](int c, int g) { return (lds_float_t *)(lds + ((c & 1) * NG + g) * kRtWBuf); };
    auto xbuf = [&](int c) { return lds + 2 * NG * kRtWBuf + (c & 1) * kRtXBuf; };
    auto stash = [&](const Regs &r, int c) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            lds_float_t *wb = wbuf(c, g);
#pragma unroll
            for (int i = 0; i < WI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) wb[(4 * (lane & 1) + j) * kRtWS + (lane >> 1) + 32 * i] = r.w[g][i][j];
        }
        lds_byte_t *xb = xbuf(c);
#pragma unroll
        for (int i = 0; i < XI; ++i)
            *(lds_u32x4_t *)(xb + ((XR * i + lane / XP) * kRtXS + 8 * (lane % XP)) * 2) = r.x[i];
    };
    Regs r;
    fetch(0, r);
    stash(r, 0);
    fetch(1, r);
    f32x4_t acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < nch; ++c) {
        const lds_byte_t *xb = xbuf(c) + (lane & 31) * kRtXS * 2;
        const int len = min(kRtKC, seg - c * kRtKC);   // a multiple of 16
#pragma unroll
        for (int b = 0; b < kRtKC / 16; ++b) {
            if (b * 16 < len) {
                const u32x4_t x0 = *(const lds_u32x4_t *)(xb + 32 * b);
                const u32x4_t x1 = *(const lds_u32x4_t *)(xb + 32 * b + 16);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    f32x4_t w4[NG];
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        w4[g] = *(const lds_f32x4_t *)(wbuf(c, g) + eb * kRtWS + 16 * b + 4 * h);
                    const u32x4_t xw = h < 2 ? x0 : x1;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t word = xw[2 * (h & 1) + j / 2];
                        const float xf = __uint_as_float((j & 1) ? (word & 0xFFFF0000u) : (word << 16));
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            acc[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(xf, w4[g][j], acc[g], 0, 0, 0);
                    }
                }
            }
        }
        // chunk c + 1 into the other buffers (last read as chunk c - 1, before this chunk's reads; a
        // wave's LDS accesses complete in order), then chunk c + 2 into the registers.  (Keeping more
        // chunks in flight measured slower on every workload shape.)
        stash(r, c + 1);
        fetch(c + 2, r);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int e = e0 + 8 * g + eb;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = tb * kRtTok + 4 * ((lane & 31) >> 2) + q;
            if (t < a.T && e < a.E) store_through(a.part + ((size_t)s * a.T + t) * a.E + e, acc[g][q]);
        }
    }
}

// Wave task q (< router_tasks(T, E)); q uniform over the wave.  Task numbers
// run expert group fastest, so the waves of a workgroup share token rows.
template <int KC = kRtKC, int NG = 1>
__device__ __forceinline__ void router_task(const RouterArgs &a, int q, lds_byte_t *lds)
{
    constexpr int GE = kRtExp * NG;   // experts per task
    const int neg = (a.E + GE - 1) / GE;
    const int ntb = (a.T + kRtTok - 1) / kRtTok;
    const int eg = __builtin_amdgcn_readfirstlane(q % neg);
    const int tb = __builtin_amdgcn_readfirstlane((q / neg) % ntb);
    const int s = __builtin_amdgcn_readfirstlane(q / (neg * ntb));
    if (a.E % 4 == 0 && eg * GE + GE <= a.E) router_task_body<true, KC, NG>(a, s, tb, eg * GE, lds);
    else router_task_body<false, KC, NG>(a, s, tb, eg * GE, lds);
}

struct TopkArgs {
    const float *part;       // [8, T, E] partial sums
    const float *bias;       // [E] or nullptr
    int32_t *ids;            // [T, k]  (workspace or user)
    int32_t *ids_user;       // [T, k] or nullptr (second copy)
    float *w_user;           // [T, k] or nullptr
    float *logits_user;      // [T, E] or nullptr: every logit (ordered partial sum plus bias)
    uint64_t *blkmask;       // [nblk, E_local] token masks to OR into (token-per-wave path), or nullptr
    int32_t T, E, k, e_begin, E_local;
};

// Top-k and gate of token t with the lanes of one wave spanning the experts
// (e = lane + 64 v, v < NV, E <= 64 NV).  The 8 partial sums of each logit
// come straight from the workspace (a token's E partials of one segment are
// contiguous, so the loads coalesce); the logit is their ordered sum plus the
// bias.  Then k rounds of a wave-wide max over (logit, -id) keys; ids and
// gates go to global memory only.  A wave that handles several tokens loads
// the next token's partials before it selects the current one.
template <int NV>
struct TopkPartials {
    float p[NV][kRouterSegments];
};

template <int NV>
__device__ __forceinline__ void topk_load(const TopkArgs &a, int t, TopkPartials<NV> &r)
{
    const int l = threadIdx.x % kWave;
    const size_t sstride = (size_t)a.T * a.E;
    const float *row = a.part + (size_t)t * a.E;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int e = min(l + v * kWave, a.E - 1);
#pragma unroll
        for (int s = 0; s < kRouterSegments; ++s) r.p[v][s] = row[s * sstride + e];
    }
}

template <int NV>
__device__ __forceinline__ void topk_select(const TopkArgs &a, int t, const TopkPartials<NV> &r)
{
#pragma clang fp contract(off)
    const int l = threadIdx.x % kWave;
    float lv[NV];
    uint64_t key[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int e = l + v * kWave;
        float x = r.p[v][0];
#pragma unroll
        for (int s = 1; s < kRouterSegments; ++s) x = x + r.p[v][s];
        if (a.bias) x = x + a.bias[min(e, a.E - 1)];
        lv[v] = x;
        key[v] = e < a.E ? topk_key(x, e) : 0ull;
        if (a.logits_user && e < a.E) a.logits_user[(size_t)t * a.E + e] = x;
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
        store_through(a.ids + o, sel_id);   // read by other workgroups after the next grid barrier
        if (a.ids_user) a.ids_user[o] = sel_id;
        if (a.w_user) a.w_user[o] = expf(sel_logit - top_logit) / zsum;
        // the token's bit in its block's mask of every local expert it chose
        const int le = sel_id - a.e_begin;
        if (a.blkmask && le >= 0 && le < a.E_local)
            __hip_atomic_fetch_or(a.blkmask + (size_t)(t / kTokBlock) * a.E_local + le, 1ull << (t % kTokBlock),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Token-per-wave top-k: workgroup unit u of W waves covers tokens W u .. W u + W - 1, one per wave.
__host__ __device__ inline int topk_wave_units(int T, int waves) { return (T + waves - 1) / waves; }

// Units u0, u0 + stride, ... (< topk_wave_units(T, W)) of one workgroup.  For E <= 256 the next
// token's partials are in flight while the current one is selected; larger E holds one token's
// partials only (their registers would not leave room for a second wave per SIMD in the fused kernel).
template <int NV>
__device__ __forceinline__ void topk_wave_units_nv(const TopkArgs &a, int u0, int stride)
{
    const int W = (int)blockDim.x / kWave;
    const int wave = (int)threadIdx.x / kWave;
    const int units = topk_wave_units(a.T, W);
    int t = u0 * W + wave;
    if (u0 >= units || t >= a.T) return;
    if constexpr (NV <= 4) {
        TopkPartials<NV> cur, nxt;
        topk_load<NV>(a, t, cur);
        for (int u = u0; u < units; u += stride) {
            const int tn = (u + stride) * W + wave;
            const bool more = u + stride < units && tn < a.T;
            if (more) topk_load<NV>(a, tn, nxt);
            topk_select<NV>(a, t, cur);
            if (!more) break;
            cur = nxt;
            t = tn;
        }
    } else {
        for (int u = u0; u < units; u += stride) {
            const int tt = u * W + wave;
            if (tt >= a.T) break;
            TopkPartials<NV> cur;
            topk_load<NV>(a, tt, cur);
            topk_select<NV>(a, tt, cur);
        }
    }
}

__device__ __forceinline__ void topk_wave_loop(const TopkArgs &a, int u0, int stride)
{
    if (a.E <= 64) topk_wave_units_nv<1>(a, u0, stride);
    else if (a.E <= 128) topk_wave_units_nv<2>(a, u0, stride);
    else if (a.E <= 256) topk_wave_units_nv<4>(a, u0, stride);
    else if (a.E <= 512) topk_wave_units_nv<8>(a, u0, stride);
    else topk_wave_units_nv<16>(a, u0, stride);
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
            for (int j = 0; j < a.k; ++j) store_through(a.lrank + (size_t)t * a.k + j, -1);
            pend = 0;
        }
        for (;;) {
            const uint64_t active = __ballot(pend != 0);
            if (active == 0) break;
            const int leader = __ffsll((unsigned long long)active) - 1;
            const int my_first = pend ? ids_lds[l * a.k + (__ffs(pend) - 1)] : -1;
            const int e = __builtin_amdgcn_readlane(my_first, __builtin_amdgcn_readfirstlane(leader));   // uniform
            int jj = -1;
            for (int j = 0; j < a.k; ++j)
                if (((pend >> j) & 1u) && ids_lds[l * a.k + j] == e) jj = j;
            const uint64_t m = __ballot(jj >= 0);
            if (jj >= 0) {
                store_through(a.lrank + (size_t)t * a.k + jj, (int32_t)__popcll(m & lanemask_lt()));
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
        store_through(a.blkcnt + (size_t)blk * a.E_local + e, cnt_lds[e]);
        store_through(a.blkmask + (size_t)blk * a.E_local + e, mask_lds[e]);
    }
    __syncthreads();
}

}  // namespace mk
