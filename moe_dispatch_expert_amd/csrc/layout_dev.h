// layout_dev.h -- expert offsets (exclusive prefix sum of the histogram),
// GEMM row-tile table, token->slot map and its inverse, and the tile-chunked
// row scatter into the expert-contiguous buffer.
//
// The dispatch half of the "MoE Dispatch+GEMM" kernel ("mKernel UCCL fuses
// NVLink/RDMA/compute into one persistent CUDA kernel", zubnet.ai, paragraph
// 2): rows of each token are moved to the experts that chose it, tile by tile,
// so the GEMM can start on a tile while the next one is still moving.  Slot
// order is the reading "ascending token id within an expert" (a stable
// counting sort), which makes the map unique.
#pragma once

#include "mk_args.h"
#include "mk_device.h"
#include "route_dev.h"

namespace mk {

struct ScanArgs {
    const int32_t *blkcnt;     // [nblk, E_local]
    int32_t *blkbase;          // [nblk, E_local] exclusive prefix over blocks
    int32_t *offsets_ws;       // [E_local + 1] expert offsets (workspace copy)
    int32_t *offsets_user;     // [E_local + 1] or nullptr
    int32_t *tile_off;         // [E_local + 1] exclusive prefix of ceil(count / bm)
    WsHeader *hdr;
    int32_t nblk, E_local, bm;
};

// One block of 1024 threads: column scan over the token blocks (thread = expert),
// then block-wide exclusive scans of counts and tile counts.  E_local <= 1024.
__device__ __forceinline__ void scan_block(const ScanArgs &a, int32_t *s_cnt, int32_t *s_til)
{
    const int e = threadIdx.x;
    int32_t cnt = 0;
    if (e < a.E_local) {
        constexpr int kB = 16;   // loads in flight before the stores (which might alias them)
        for (int b0 = 0; b0 < a.nblk; b0 += kB) {
            int32_t c[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) c[j] = b0 + j < a.nblk ? a.blkcnt[(size_t)(b0 + j) * a.E_local + e] : 0;
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (b0 + j < a.nblk) a.blkbase[(size_t)(b0 + j) * a.E_local + e] = cnt;
                cnt += c[j];
            }
        }
    }
    const int32_t til = e < a.E_local ? (cnt + a.bm - 1) / a.bm : 0;
    s_cnt[e] = cnt;
    s_til[e] = til;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
        const int32_t c2 = e >= off ? s_cnt[e - off] : 0;
        const int32_t t2 = e >= off ? s_til[e - off] : 0;
        __syncthreads();
        s_cnt[e] += c2;
        s_til[e] += t2;
        __syncthreads();
    }
    // s_* now hold inclusive sums
    if (e < a.E_local) {
        a.offsets_ws[e + 1] = s_cnt[e];
        a.tile_off[e + 1] = s_til[e];
        if (a.offsets_user) a.offsets_user[e + 1] = s_cnt[e];
    }
    if (e == 0) {
        a.offsets_ws[0] = 0;
        a.tile_off[0] = 0;
        if (a.offsets_user) a.offsets_user[0] = 0;
        a.hdr->R = (uint32_t)s_cnt[a.E_local - 1];
        a.hdr->n_tiles = (uint32_t)s_til[a.E_local - 1];
    }
    __syncthreads();
}

struct SlotArgs {
    const int32_t *ids;        // [T, k]
    const int32_t *lrank;      // [T, k]
    const int32_t *blkbase;    // [nblk, E_local]
    const int32_t *offsets;    // [E_local + 1]
    int32_t *slot_of;          // [T, k] (user)
    int32_t *row_token_ws;     // [R_cap]
    int32_t *row_token_user;   // [R_cap] or nullptr
    int32_t T, k, e_begin, E_local;
};

__device__ __forceinline__ void slot_one(const SlotArgs &a, int i)
{
    const int t = i / a.k;
    const int le = a.ids[i] - a.e_begin;
    int32_t slot = -1;
    const int32_t rank = a.lrank[i];
    if (le >= 0 && le < a.E_local && rank >= 0) {
        slot = a.offsets[le] + a.blkbase[(size_t)(t / kTokBlock) * a.E_local + le] + rank;
        if (slot < a.offsets[le + 1]) {
            a.row_token_ws[slot] = t;
            if (a.row_token_user) a.row_token_user[slot] = t;
        } else {
            slot = -1;   // only reachable for ids that were rejected
        }
    }
    a.slot_of[i] = slot;
}

typedef unsigned int cp_u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) cp_u32x4_t gcuint4_t;
typedef __attribute__((address_space(1))) cp_u32x4_t guint4_t;

// Copy one row of d bf16 (cpr = d / 8 chunks of 16 bytes) with one wave: every
// lane first loads all of its chunks (clamped indices, so the loads are
// unconditional and in flight together), then stores them.  CPL = chunks per
// lane, a compile-time bound (cpr <= 64 * CPL).
template <int CPL>
__device__ __forceinline__ void copy_row_wave(const uint16_t *src_row, uint16_t *dst_row, int cpr, int lane)
{
    gcuint4_t *s = (gcuint4_t *)src_row;
    guint4_t *d = (guint4_t *)dst_row;
    cp_u32x4_t v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i] = s[min(lane + kWave * i, cpr - 1)];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        if (lane + kWave * i < cpr) d[lane + kWave * i] = v[i];
}

__device__ __forceinline__ void copy_row(const uint16_t *src_row, uint16_t *dst_row, int d, int lane)
{
    const int cpr = d / 8;
    if (cpr <= 4 * kWave) copy_row_wave<4>(src_row, dst_row, cpr, lane);
    else if (cpr <= 8 * kWave) copy_row_wave<8>(src_row, dst_row, cpr, lane);
    else if (cpr <= 16 * kWave) copy_row_wave<16>(src_row, dst_row, cpr, lane);
    else
        for (int c0 = 0; c0 < cpr; c0 += 16 * kWave)
            copy_row_wave<16>(src_row + (size_t)c0 * 8, dst_row + (size_t)c0 * 8, min(cpr - c0, 16 * kWave),
                              lane);
}

// Copy NR rows of d bf16 with one wave, all NR * CPL loads of a lane in
// flight before the first store (cpr = d / 8 <= 64 * CPL chunks per row).
// src[i] / dst[i] may be null for a row that is skipped.
template <int CPL, int NR>
__device__ __forceinline__ void copy_rows_wave(const uint16_t *const (&src)[NR], uint16_t *const (&dst)[NR],
                                               int cpr, int lane)
{
    cp_u32x4_t v[NR][CPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        gcuint4_t *s = (gcuint4_t *)(src[r] ? src[r] : src[0]);
#pragma unroll
        for (int i = 0; i < CPL; ++i) v[r][i] = s[min(lane + kWave * i, cpr - 1)];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (!dst[r]) continue;
        guint4_t *d = (guint4_t *)dst[r];
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            if (lane + kWave * i < cpr) d[lane + kWave * i] = v[r][i];
    }
}

// Copy one expert-buffer row r: x_perm[r] = x[row_token[r]].
__device__ __forceinline__ void move_row(const SrcRows &src, const int32_t *row_token, uint16_t *x_perm,
                                         int d, int r, int lane)
{
    copy_row(token_row(src, row_token[r], d), x_perm + (size_t)r * d, d, lane);
}

}  // namespace mk
