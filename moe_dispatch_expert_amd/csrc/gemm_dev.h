// gemm_dev.h -- per-expert grouped GEMM on gfx950 matrix cores.
//
// y_perm[r, n] = bf16_rne(sum_i x_perm[r, i] * W[e, n, i]) for the rows r of
// expert e, fp32 accumulation: the dense-compute half of the "MoE
// Dispatch+GEMM" kernel ("mKernel UCCL fuses NVLink/RDMA/compute into one
// persistent CUDA kernel", zubnet.ai, paragraph 2).  The pages give no GEMM
// design; the one here is written for CDNA4:
//   - a workgroup of 4 waves owns a BN x BM tile of y^T (W rows x token rows);
//     each wave a (BN/2) x (BM/2) quadrant made of 32x32 v_mfma bf16 blocks
//     with K = 16 per instruction;
//   - both operands are K-contiguous in HBM, so tiles are copied straight from
//     global memory into LDS (global_load_lds, 16 bytes per lane, no register
//     staging), two stages deep, with the 16-byte chunk index of each 128-byte
//     LDS row XOR-swizzled by (row & 7) so fragment reads are conflict-free;
//   - W is the MFMA "A" operand, so each lane ends with 4 consecutive output
//     columns of one row and the epilogue stores 8 bytes per lane;
//   - ragged tails: tile rows past the expert's count read padding or the next
//     expert's rows and are never stored; W rows past N are clamped.
#pragma once

#include "mk_args.h"
#include "mk_device.h"

namespace mk {

typedef __attribute__((address_space(3))) void lds_void_t;

struct GemmArgs {
    const uint16_t *x_perm;      // [x_perm_rows, d]
    const uint16_t *w;           // [E_local, N, d]
    uint16_t *y;                 // [R_cap, N]
    const int32_t *offsets;      // [E_local + 1]
    const int32_t *tile_off;     // [E_local + 1] exclusive prefix of row tiles
    const uint32_t *tile_flag;   // [max_tiles]: tile ready iff == epoch; nullptr = no waits
    WsHeader *hdr;
    uint64_t spin_limit;         // wall-clock ticks a wait may take
    uint32_t epoch;
    int32_t d, N, E_local;
};

template <int BM_, int BN_>
struct BigTile {
    static constexpr int BM = BM_;         // token rows per tile
    static constexpr int BN = BN_;         // W rows (output columns) per tile
    static constexpr int BK = 64;          // K per stage: one 128-byte LDS row
    static constexpr int NI = BN / 64;     // 32-wide blocks per wave along N
    static constexpr int MI = BM / 64;     // 32-wide blocks per wave along M
    static constexpr int W_BYTES = BN * BK * 2;
    static constexpr int X_BYTES = BM * BK * 2;
    static constexpr int STAGE = W_BYTES + X_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static constexpr int THREADS = 256;
};

// Buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes)
{
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)n, 0x00020000);
}

// Issue the copy of ROWS rows x 64 bf16 (columns k0 .. k0+63) into an LDS
// tile, 8 rows per wave instruction (buffer_load ... lds, 16 bytes per lane).
// Lane l lands at LDS row rb*8 + l/8, position l%8, and fetches the global
// 16-byte chunk (l%8) ^ (l/8): position p of tile row r holds chunk p ^ (r & 7).
// lane_off = (l/8) * row_bytes + ((l%8) ^ (l/8)) * 16.
template <int ROWS>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t src, uint32_t lane_off, uint32_t row_bytes,
                                           uint32_t k0_bytes, char *lds_tile, int wave)
{
#pragma unroll
    for (int it = 0; it < ROWS / 32; ++it) {
        const int rb = it * 4 + wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t *)(lds_tile + rb * 1024), 16, lane_off,
                                                 (uint32_t)rb * 8u * row_bytes + k0_bytes, 0, 0);
    }
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <class C>
__device__ __forceinline__ void tile_mfma(const char *stage, int wn, int wm, const int (&frag_off)[4],
                                          f32x16_t (&acc)[C::NI][C::MI])
{
    const char *wt = stage + (wn * (C::BN / 2)) * 128;
    const char *xt = stage + C::W_BYTES + (wm * (C::BM / 2)) * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[C::NI], bf[C::MI];
#pragma unroll
        for (int i = 0; i < C::NI; ++i) af[i] = *(const bf16x8_t *)(wt + i * 32 * 128 + frag_off[kk]);
#pragma unroll
        for (int j = 0; j < C::MI; ++j) bf[j] = *(const bf16x8_t *)(xt + j * 32 * 128 + frag_off[kk]);
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int j = 0; j < C::MI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
}

// One BN x BM tile: token rows [row0, row0 + BM) of x_perm (rows_valid of them
// stored), W rows [n0, n0 + BN) of expert e.  Two LDS stages (s0, s1), the
// K loop unrolled by two so each stage is a distinct array: the copy into one
// stage runs while the other feeds the matrix cores.
template <class C>
__device__ void gemm_tile_big(const GemmArgs &a, int e, int row0, int rows_valid, int n0, char *s0, char *s1)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps M0/soffset scalar
    const int lane = threadIdx.x % kWave;
    const int wn = wave & 1, wm = wave >> 1;
    const size_t w_first = (size_t)e * a.N + n0;
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(a.w + w_first * a.d, ((size_t)a.E_local * a.N - w_first) * a.d * 2);
    // Only the tile's valid rows are readable: rows past a ragged end return 0 without a memory access
    // (they may belong to a tile that is not yet moved).
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(a.x_perm + (size_t)row0 * a.d, (size_t)rows_valid * a.d * 2);
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    const uint32_t lane_off = (uint32_t)(lane >> 3) * row_bytes + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
    const int KT = a.d / C::BK;

    int frag_off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        frag_off[kk] = (lane & 31) * 128 + (((2 * kk + (lane >> 5)) ^ (lane & 7)) << 4);

    f32x16_t acc[C::NI][C::MI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // K steps come in pairs (d % 128 == 0): stage s0 holds even steps, s1 odd ones.
    issue_tile<C::BN>(wsrc, lane_off, row_bytes, 0, s0, wave);
    issue_tile<C::BM>(xsrc, lane_off, row_bytes, 0, s0 + C::W_BYTES, wave);
    wait_vmem_all();
    __syncthreads();
    const uint32_t step_bytes = C::BK * 2;
    for (int kt = 0; kt < KT - 2; kt += 2) {
        const uint32_t k1 = (uint32_t)(kt + 1) * step_bytes;
        issue_tile<C::BN>(wsrc, lane_off, row_bytes, k1, s1, wave);
        issue_tile<C::BM>(xsrc, lane_off, row_bytes, k1, s1 + C::W_BYTES, wave);
        tile_mfma<C>(s0, wn, wm, frag_off, acc);
        wait_vmem_all();
        __syncthreads();
        const uint32_t k2 = k1 + step_bytes;
        issue_tile<C::BN>(wsrc, lane_off, row_bytes, k2, s0, wave);
        issue_tile<C::BM>(xsrc, lane_off, row_bytes, k2, s0 + C::W_BYTES, wave);
        tile_mfma<C>(s1, wn, wm, frag_off, acc);
        wait_vmem_all();
        __syncthreads();
    }
    {
        const uint32_t k1 = (uint32_t)(KT - 1) * step_bytes;
        issue_tile<C::BN>(wsrc, lane_off, row_bytes, k1, s1, wave);
        issue_tile<C::BM>(xsrc, lane_off, row_bytes, k1, s1 + C::W_BYTES, wave);
        tile_mfma<C>(s0, wn, wm, frag_off, acc);
        wait_vmem_all();
        __syncthreads();
        tile_mfma<C>(s1, wn, wm, frag_off, acc);
        __syncthreads();   // every wave is done with s1 before the next tile refills it
    }

    // epilogue: lane holds y^T[n][m] for n = base + 8*(v/4) + 4*(lane/32) + v%4, m = lane%32
    const int n_limit = a.N - n0;
#pragma unroll
    for (int j = 0; j < C::MI; ++j) {
        const int m = wm * (C::BM / 2) + j * 32 + (lane & 31);
        if (m >= rows_valid) continue;
        uint16_t *yrow = a.y + (size_t)(row0 + m) * a.N + n0;
#pragma unroll
        for (int i = 0; i < C::NI; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = wn * (C::BN / 2) + i * 32 + 8 * g + 4 * (lane >> 5);
                if (n < n_limit) {
                    const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][4 * g + 0]) |
                                        ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][4 * g + 2]) |
                                        ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 3]) << 16);
                    *(uint2 *)(yrow + n) = make_uint2(lo, hi);
                }
            }
        }
    }
}

// Task q -> (expert, row tile, column block), tasks ordered expert-major, then
// column block, then row tile, so consecutive tasks share one W tile.
struct TaskPos {
    int e, mt, nb;
};
__device__ __forceinline__ TaskPos decode_task(const int32_t *tile_off, int E_local, int NB, int q)
{
    int lo = 0, hi = E_local;   // find e: tile_off[e]*NB <= q < tile_off[e+1]*NB
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] * NB <= q) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int nt = tile_off[e + 1] - tile_off[e];
    const int rem = q - tile_off[e] * NB;
    TaskPos p;
    p.e = e;
    p.nb = rem / nt;
    p.mt = rem % nt;
    return p;
}

// Persistent workgroup loop over GEMM tasks.  Workgroup w (of G, G % 8 == 0)
// runs task round*G + slot(w); slot() gives the workgroups of one XCD
// (w % 8 == x, dispatched round-robin over the 8 XCDs) a contiguous run of
// tasks, so tasks sharing a W tile share that XCD's L2.
template <class C>
__device__ void gemm_worker(const GemmArgs &a, int w, int G, char *s0, char *s1)
{
    const int n_tiles = (int)a.hdr->n_tiles;
    const int NB = (a.N + C::BN - 1) / C::BN;
    const int n_tasks = n_tiles * NB;
    const int slot = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
    for (int base = 0; base < n_tasks; base += G) {
        const int q = base + slot;
        if (q >= n_tasks) continue;
        const TaskPos p = decode_task(a.tile_off, a.E_local, NB, q);
        const int cnt = a.offsets[p.e + 1] - a.offsets[p.e];
        const int rows_valid = min(C::BM, cnt - p.mt * C::BM);
        const int row0 = a.offsets[p.e] + p.mt * C::BM;
        if (a.tile_flag) {
            __shared__ int ok_sh;
            if (threadIdx.x == 0)
                ok_sh = wait_flag_eq(a.tile_flag + a.tile_off[p.e] + p.mt, a.epoch, &a.hdr->err,
                                     a.spin_limit, 0x10000000u | (uint32_t)(a.tile_off[p.e] + p.mt));
            __syncthreads();
            if (!ok_sh) return;
        }
        gemm_tile_big<C>(a, p.e, row0, rows_valid, p.nb * C::BN, s0, s1);
    }
}

}  // namespace mk
