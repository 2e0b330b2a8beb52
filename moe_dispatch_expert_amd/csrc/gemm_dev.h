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
//     global memory into LDS (buffer_load ... lds, 16 bytes per lane, no
//     register staging) through four 32-deep stages, with the 16-byte chunk
//     index of each 64-byte LDS row XOR-swizzled by (row >> 2) & 3 so fragment
//     reads are conflict-free on the 64-bank LDS;
//   - fragment reads of the next K = 16 sub-step are interleaved with the
//     MFMAs of the current one (sched_group_barrier);
//   - W is the MFMA "A" operand, so each lane ends with 4 consecutive output
//     columns of one row and the epilogue stores 8 bytes per lane;
//   - ragged tails: tile rows past the expert's count read padding or the next
//     expert's rows and are never stored; W rows past N are clamped.
#pragma once

#include "mk_args.h"
#include "mk_device.h"

namespace mk {

typedef __attribute__((address_space(3))) char lds_char_t;

// The four LDS stage arrays of a GEMM workgroup, as LDS-space pointers (their
// 32-bit LDS addresses are compile-time constants once the arrays are placed).
struct LdsStages {
    lds_char_t *p[4];
};

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
    static constexpr int BK = 32;          // K per stage: one 64-byte LDS row
    static constexpr int NSTAGE = 4;       // LDS stages (distinct arrays)
    static constexpr int NI = BN / 64;     // 32-wide blocks per wave along N
    static constexpr int MI = BM / 64;     // 32-wide blocks per wave along M
    static constexpr int W_BYTES = BN * BK * 2;
    static constexpr int X_BYTES = BM * BK * 2;
    static constexpr int STAGE = W_BYTES + X_BYTES;
    static constexpr int DMA_PER_WAVE = (BN + BM) / 16 / 4;   // 1 KiB copies per wave per stage
    static constexpr int THREADS = 256;
};
static_assert(BigTile<256, 256>::STAGE == 32768, "a stage is 32 KiB");

// Buffer resource words over [base, base + bytes): loads past the end return 0.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, size_t bytes)
{
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
    const uint64_t b = (uint64_t)base;
    rsrc_t r;
    r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(b >> 32) & 0xFFFFu));   // stride 0
    r.z = __builtin_amdgcn_readfirstlane((int32_t)n);                                  // bytes
    r.w = 0x00020000;
    return r;
}

// LDS tile rows are 64 bytes (32 bf16 of K) = 4 chunks of 16 bytes.  Position
// p of tile row r holds global chunk p ^ swz(r), swz(r) = (r >> 2) & 3: the 16
// lanes of one ds_read_b128 phase (rows r0..r0+15 at one chunk, r0 % 16 == 0)
// then hit all 64 banks once, so fragment reads are conflict-free.
__device__ __forceinline__ int lds_swz(int r) { return (r >> 2) & 3; }

// Issue the copy of ROWS rows x 32 bf16 (columns k0 .. k0+31) into an LDS tile,
// 16 rows per wave instruction (buffer_load ... lds: 16 bytes per lane, lane l
// lands at M0 + 16 l).  Lane l lands at row rb*16 + l/4, position l%4, so it
// fetches the global chunk (l%4) ^ swz(l/4) (independent of rb): lane_off =
// (l/4)*row_bytes + that*16.  Written as inline assembly so the compiler's own
// tracking of LDS-bound loads, which cannot tell the four stage arrays apart,
// adds no vmcnt(0) waits; every wait on these copies is explicit.
template <int ROWS>
__device__ __forceinline__ void issue_tile(rsrc_t src, uint32_t lane_off, uint32_t row_bytes, uint32_t k0_bytes,
                                           lds_char_t *lds_tile, int wave)
{
#pragma unroll
    for (int it = 0; it < ROWS / 64; ++it) {
        const int rb = it * 4 + wave;
        const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_tile + rb * 1024));
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)rb * 16u * row_bytes + k0_bytes);
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(lane_off), "s"(src), "s"(soff)
                     : "memory", "m0");
    }
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_vmem_all() { wait_vmem<0>(); }

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedVMEM = 0x010, kSchedDSRead = 0x100;

template <class C>
__device__ __forceinline__ void load_frags(const lds_char_t *stage, int wn, int wm, int off, bf16x8_t (&fa)[C::NI],
                                           bf16x8_t (&fb)[C::MI])
{
    typedef __attribute__((address_space(3))) const bf16x8_t lds_frag_t;
    const lds_char_t *wt = stage + (wn * (C::BN / 2)) * 64;
    const lds_char_t *xt = stage + C::W_BYTES + (wm * (C::BM / 2)) * 64;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) fa[i] = *(lds_frag_t *)(wt + i * 32 * 64 + off);
#pragma unroll
    for (int j = 0; j < C::MI; ++j) fb[j] = *(lds_frag_t *)(xt + j * 32 * 64 + off);
}

template <class C>
__device__ __forceinline__ void mfma_block(const bf16x8_t (&fa)[C::NI], const bf16x8_t (&fb)[C::MI],
                                           f32x16_t (&acc)[C::NI][C::MI])
{
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// Interleave the MFMAs just emitted with the fragment reads just emitted:
// one read after each of the first NR MFMAs.
template <class C>
__device__ __forceinline__ void sched_mfma_with_reads(bool reads)
{
    constexpr int NR = C::NI + C::MI, NM = C::NI * C::MI;
    if (reads) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NM - NR, 0);
    } else {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NM, 0);
    }
}

// One BN x BM tile: token rows [row0, row0 + BM) of x_perm (rows_valid of
// them readable and stored), W rows [n0, n0 + BN) of expert e.
//
// K runs in stages of 32 through four LDS arrays (d / 32 stages, a multiple
// of 4 since d % 128 == 0).  Stage k lives in array k % 4 and has two
// sub-steps of K = 16.  Per stage:
//   sub-step 0: MFMAs on fragments fr0 while fragments fr1 (sub-step 1 of
//               this stage) are read;
//   wait for the copy of stage k+1, barrier (every wave is then past its
//               reads of stage k, and stage k+1 is visible), issue the copy of
//               stage k+4 into stage k's array;
//   sub-step 1: MFMAs on fr1 while fr0 of stage k+1 is read.
// The copy of stage k+4 therefore has three stages of lead time.  The loop is
// written out four stages at a time so every LDS array and wait count is a
// compile-time constant.
template <class C>
__device__ __forceinline__ void gemm_tile_big(const GemmArgs &a, int e, int row0, int rows_valid, int n0,
                                              const LdsStages &ls)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps M0/soffset scalar
    const int lane = threadIdx.x % kWave;
    const int wn = wave & 1, wm = wave >> 1;
    const size_t w_first = (size_t)e * a.N + n0;
    const rsrc_t wsrc =
        make_rsrc(a.w + w_first * a.d, ((size_t)a.E_local * a.N - w_first) * a.d * 2);
    // Only the tile's valid rows are readable: rows past a ragged end return 0 without a memory access
    // (they may belong to a tile that is not yet moved).
    const rsrc_t xsrc = make_rsrc(a.x_perm + (size_t)row0 * a.d, (size_t)rows_valid * a.d * 2);
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    const uint32_t lane_off = (uint32_t)(lane >> 2) * row_bytes + (uint32_t)(((lane & 3) ^ lds_swz(lane >> 2)) << 4);
    const int KT = a.d / C::BK;   // a multiple of 4 (d % 128 == 0)

    int frag_off[2];   // row (lane & 31) of a 32-row block, chunk 2kk + lane/32
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        frag_off[kk] = (lane & 31) * 64 + (((2 * kk + (lane >> 5)) ^ lds_swz(lane & 31)) << 4);

    f32x16_t acc[C::NI][C::MI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    lds_char_t *const st[4] = {ls.p[0], ls.p[1], ls.p[2], ls.p[3]};
    auto issue_stage = [&](int k, lds_char_t *dst) {
        const uint32_t k0 = (uint32_t)k * C::BK * 2;
        issue_tile<C::BN>(wsrc, lane_off, row_bytes, k0, dst, wave);
        issue_tile<C::BM>(xsrc, lane_off, row_bytes, k0, dst + C::W_BYTES, wave);
    };
    // vmcnt counts loads and stores together and they may complete out of
    // order relative to each other: the previous tile's output stores must be
    // done before a partial vmcnt wait can stand for "these copies arrived".
    wait_vmem_all();
    issue_stage(0, st[0]);
    issue_stage(1, st[1]);
    issue_stage(2, st[2]);
    issue_stage(3, st[3]);
    wait_vmem<3 * C::DMA_PER_WAVE>();
    __syncthreads();
    bf16x8_t fa0[C::NI], fb0[C::MI], fa1[C::NI], fb1[C::MI];
    load_frags<C>(st[0], wn, wm, frag_off[0], fa0, fb0);

    // One stage; ISSUE: refill CUR with stage K + 4; WAITN: copies allowed in
    // flight once stage K + 1 has arrived (-1: K is the last stage).
#define MK_GEMM_STAGE(CUR, NXT, K, ISSUE, WAITN)                                                        \
    do {                                                                                               \
        load_frags<C>(CUR, wn, wm, frag_off[1], fa1, fb1);                                             \
        mfma_block<C>(fa0, fb0, acc);                                                                  \
        sched_mfma_with_reads<C>(true);                                                                \
        if ((WAITN) >= 0) {                                                                            \
            wait_vmem<((WAITN) < 0 ? 0 : (WAITN))>();                                                  \
            __syncthreads();                                                                           \
            if (ISSUE) issue_stage((K) + 4, CUR);                                                      \
            load_frags<C>(NXT, wn, wm, frag_off[0], fa0, fb0);                                         \
        }                                                                                              \
        mfma_block<C>(fa1, fb1, acc);                                                                  \
        sched_mfma_with_reads<C>((WAITN) >= 0);                                                        \
    } while (0)

    constexpr int D2 = 2 * C::DMA_PER_WAVE;
    int kt = 0;
    for (; kt + 4 < KT; kt += 4) {   // every stage refills: four stages always in flight
        MK_GEMM_STAGE(st[0], st[1], kt, true, D2);
        MK_GEMM_STAGE(st[1], st[2], kt + 1, true, D2);
        MK_GEMM_STAGE(st[2], st[3], kt + 2, true, D2);
        MK_GEMM_STAGE(st[3], st[0], kt + 3, true, D2);
    }
    // last four stages: nothing left to issue, the pipeline drains
    MK_GEMM_STAGE(st[0], st[1], kt, false, D2);
    MK_GEMM_STAGE(st[1], st[2], kt + 1, false, C::DMA_PER_WAVE);
    MK_GEMM_STAGE(st[2], st[3], kt + 2, false, 0);
    MK_GEMM_STAGE(st[3], st[0], kt + 3, false, -1);
#undef MK_GEMM_STAGE
    __syncthreads();   // every wave is done with the stages before the next tile refills them

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
__device__ void gemm_worker(const GemmArgs &a, int w, int G, const LdsStages &ls)
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
        gemm_tile_big<C>(a, p.e, row0, rows_valid, p.nb * C::BN, ls);
    }
}

}  // namespace mk
