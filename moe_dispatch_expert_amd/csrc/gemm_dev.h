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
//   - both operands are K-contiguous in HBM.  K runs in slabs of 64: each
//     wave loads its share of a slab as whole 128-byte lines (8 rows x 128 B
//     per buffer_load_dwordx4) into registers two slabs ahead, and writes the
//     slab into one of two LDS buffers one slab ahead.  Streaming is latency
//     bound per CU, so what counts is the bytes in flight: registers hold two
//     slabs (128 KiB per workgroup) on top of the two LDS buffers;
//   - the 16-byte chunk index of each 128-byte LDS row is XOR-swizzled by
//     (row >> 1) & 7, so both the slab writes and the fragment reads are
//     conflict-free on the 64-bank LDS;
//   - fragment reads of the next K = 16 step are interleaved with the MFMAs
//     of the current one (sched_group_barrier), and the one barrier per slab
//     sits before the last step, so the next slab's first reads overlap it;
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

template <int BM_, int BN_, int WN_ = 2>
struct BigTile {
    static constexpr int BM = BM_;         // token rows per tile
    static constexpr int BN = BN_;         // W rows (output columns) per tile
    static constexpr int WN = WN_;         // waves along N (the other 4 / WN along M)
    static constexpr int WM = 4 / WN_;
    static constexpr int BK = 64;          // K per slab: one 128-byte LDS row per tile row
    static constexpr int NI = BN / WN / 32;   // 32-wide blocks per wave along N
    static constexpr int MI = BM / WM / 32;   // 32-wide blocks per wave along M
    static constexpr int WL = BN / 32;     // W loads per wave per slab (8 rows x 128 B each)
    static constexpr int XL = BM / 32;     // x loads per wave per slab
    static constexpr int STAGE = BN * BK * 2;   // bytes of one LDS array (W or x half of a slab buffer)
    static constexpr int THREADS = 256;
    static_assert(NI >= 1 && MI >= 1 && XL <= WL, "tile shape");
};
static_assert(BigTile<256, 256>::STAGE == 32768, "an LDS array is 32 KiB");

typedef int32_t v4i_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i_t lds_v4i_t;

// Buffer resource over [base, base + bytes): loads past the end return 0.
// The arguments must be wave-uniform; readfirstlane makes that visible to the
// compiler, which otherwise wraps every load in a loop over distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes)
{
    const uint64_t b = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}

// One wave's share of a slab in registers: load i < WL is W, the rest x;
// load i covers tile rows (4 (i % WL) + wave) * 8 + lane / 8, 16 bytes at
// chunk lane % 8.
template <class C>
struct SlabRegs {
    static constexpr int N = C::WL + C::XL;
    v4i_t v[N];
};

// Loads [I0, I1) of slab `slab`.  The row part of each offset is in the
// per-lane offset (voff[i] = row * row_bytes + chunk * 16), which the buffer
// range check covers, so rows past the end of a resource read 0 without a
// memory access; the K part (slab * 128 bytes, always inside the row) is the
// scalar offset.
template <class C, int I0, int I1>
__device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t wsrc, __amdgpu_buffer_rsrc_t xsrc,
                                          const uint32_t (&voff)[C::WL], int slab, SlabRegs<C> &r)
{
    const uint32_t k0 = (uint32_t)slab * C::BK * 2;
#pragma unroll
    for (int i = I0; i < I1; ++i)
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(i < C::WL ? wsrc : xsrc, voff[i < C::WL ? i : i - C::WL], k0, 0);
}

// Writes [I0, I1) of a slab from registers into an LDS buffer (128 B per row,
// chunk p of row r at position p ^ ((r >> 1) & 7)).  st_off: this lane's byte
// offset inside a block of 8 rows (the swizzle of row (4 i + wave) * 8 +
// lane / 8 depends on the lane and the wave's parity only).
template <class C, int I0, int I1>
__device__ __forceinline__ void store_part(const SlabRegs<C> &r, lds_char_t *wbuf, lds_char_t *xbuf, int wave,
                                           uint32_t st_off)
{
#pragma unroll
    for (int i = I0; i < I1; ++i)
        *(lds_v4i_t *)((i < C::WL ? wbuf : xbuf) + (4 * (i < C::WL ? i : i - C::WL) + wave) * 1024 + st_off) = r.v[i];
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
constexpr int kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100, kSchedDSWrite = 0x200;

template <class C>
__device__ __forceinline__ void load_frags(const lds_char_t *wbuf, const lds_char_t *xbuf, int wn, int wm, int off,
                                           bf16x8_t (&fa)[C::NI], bf16x8_t (&fb)[C::MI])
{
    typedef __attribute__((address_space(3))) const bf16x8_t lds_frag_t;
    const lds_char_t *wt = wbuf + (wn * (C::BN / C::WN)) * 128;
    const lds_char_t *xt = xbuf + (wm * (C::BM / C::WM)) * 128;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) fa[i] = *(lds_frag_t *)(wt + i * 32 * 128 + off);
#pragma unroll
    for (int j = 0; j < C::MI; ++j) fb[j] = *(lds_frag_t *)(xt + j * 32 * 128 + off);
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

// Order the K = 16 step just emitted: NR fragment reads, then NW slab writes
// each followed by a slab load, one after each MFMA; the rest of the MFMAs
// after them.
template <class C, int NR, int NW>
__device__ __forceinline__ void sched_step()
{
    constexpr int NM = C::NI * C::MI;
    if (NR + NW > NM) return;   // too few MFMAs to pair with: the compiler's own order
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSWrite, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, 1, 0);
    }
    if (NM - NR - NW > 0) __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NM - NR - NW, 0);
}

// One BN x BM tile: token rows [row0, row0 + BM) of x_perm (rows_valid of
// them readable and stored), W rows [n0, n0 + BN) of expert e.
//
// Slab j (K = 64 j .. 64 j + 63) is computed from LDS buffer j % 2 (W in
// ls.p[2 (j % 2)], x in ls.p[2 (j % 2) + 1]) in four K = 16 steps, with the
// fragments of step s + 1 read during the MFMAs of step s.  Between steps 2
// and 3: write slab j + 1 from registers into the other buffer (its old slab
// j - 1 was last read before the previous barrier), load slab j + 3 into the
// registers just freed, barrier, then read step 0 of slab j + 1 during step 3.
// Slab s lives in register set s % 2, loaded two slabs before it is written.
template <class C>
__device__ __forceinline__ void gemm_tile_big(const GemmArgs &a, int e, int row0, int rows_valid, int n0,
                                              const LdsStages &ls)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps soffsets scalar
    const int lane = threadIdx.x % kWave;
    const int wn = wave % C::WN, wm = wave / C::WN;
    const size_t w_first = (size_t)e * a.N + n0;
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(a.w + w_first * a.d, ((size_t)a.E_local * a.N - w_first) * a.d * 2);
    // Only the tile's valid rows are readable: rows past a ragged end return 0 without a memory access
    // (they may belong to a tile that is not yet moved).
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(a.x_perm + (size_t)row0 * a.d, (size_t)rows_valid * a.d * 2);
    // Loads of slabs past the end go to empty resources: they read 0 without a memory access, and
    // keep the number of loads in flight the same on every path.
    const __amdgpu_buffer_rsrc_t wnone = make_rsrc(a.w, 0), xnone = make_rsrc(a.x_perm, 0);
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    uint32_t voff[C::WL];
#pragma unroll
    for (int i = 0; i < C::WL; ++i)
        voff[i] = (uint32_t)((4 * i + wave) * 8 + (lane >> 3)) * row_bytes + (uint32_t)(lane & 7) * 16u;
    const uint32_t st_off = (uint32_t)(lane >> 3) * 128u + (uint32_t)(((lane & 7) ^ ((lane >> 4) + 4 * (wave & 1))) << 4);
    const int KK = __builtin_amdgcn_readfirstlane(a.d / C::BK);   // even (d % 128 == 0); uniform

    int frag_off[4];   // row (lane & 31) of a 32-row block, chunk 2 kk + lane / 32
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        frag_off[kk] = (lane & 31) * 128 + (((2 * kk + (lane >> 5)) ^ (((lane & 31) >> 1) & 7)) << 4);

    f32x16_t acc[C::NI][C::MI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    lds_char_t *const wb[2] = {ls.p[0], ls.p[2]};
    lds_char_t *const xb[2] = {ls.p[1], ls.p[3]};
    constexpr int NL = SlabRegs<C>::N;
    constexpr int P1 = (NL + 2) / 3, P2 = (2 * NL + 2) / 3;   // the slab write in three parts
    constexpr int NR = C::NI + C::MI;
    SlabRegs<C> r0, r1;
    load_part<C, 0, NL>(wsrc, xsrc, voff, 0, r0);
    load_part<C, 0, NL>(wsrc, xsrc, voff, 1, r1);
    store_part<C, 0, NL>(r0, wb[0], xb[0], wave, st_off);
    load_part<C, 0, NL>(KK > 2 ? wsrc : wnone, KK > 2 ? xsrc : xnone, voff, 2, r0);
    __syncthreads();
    bf16x8_t fa0[C::NI], fb0[C::MI], fa1[C::NI], fb1[C::MI];
    load_frags<C>(wb[0], xb[0], wn, wm, frag_off[0], fa0, fb0);

    // Slab J from buffer B; RN: the register set holding slab J + 1; NEXT
    // (compile-time): slab J + 1 exists.  During steps 0..2, slab J + 1 is
    // written from RN into the other buffer, a third per step, and each
    // register is refilled with slab J + 3 right after it is written (from
    // the empty resources if slab J + 3 does not exist).
#define MK_GEMM_SLAB(B, RN, J, NEXT)                                                                   \
    do {                                                                                               \
        const bool ahead_ = __builtin_amdgcn_readfirstlane((J) + 3 < KK);                              \
        const __amdgpu_buffer_rsrc_t wl_ = ahead_ ? wsrc : wnone, xl_ = ahead_ ? xsrc : xnone;         \
        lds_char_t *const wo_ = wb[1 - (B)];                                                           \
        lds_char_t *const xo_ = xb[1 - (B)];                                                           \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[1], fa1, fb1);                                    \
        mfma_block<C>(fa0, fb0, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, 0, P1>(RN, wo_, xo_, wave, st_off);                                          \
            load_part<C, 0, P1>(wl_, xl_, voff, (J) + 3, RN);                                          \
            sched_step<C, NR, P1>();                                                                   \
        } else {                                                                                       \
            sched_step<C, NR, 0>();                                                                    \
        }                                                                                              \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[2], fa0, fb0);                                    \
        mfma_block<C>(fa1, fb1, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, P1, P2>(RN, wo_, xo_, wave, st_off);                                         \
            load_part<C, P1, P2>(wl_, xl_, voff, (J) + 3, RN);                                         \
            sched_step<C, NR, P2 - P1>();                                                              \
        } else {                                                                                       \
            sched_step<C, NR, 0>();                                                                    \
        }                                                                                              \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[3], fa1, fb1);                                    \
        mfma_block<C>(fa0, fb0, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, P2, NL>(RN, wo_, xo_, wave, st_off);                                         \
            load_part<C, P2, NL>(wl_, xl_, voff, (J) + 3, RN);                                         \
            sched_step<C, NR, NL - P2>();                                                              \
            __builtin_amdgcn_sched_barrier(0);                                                         \
            __syncthreads();                                                                           \
            load_frags<C>(wo_, xo_, wn, wm, frag_off[0], fa0, fb0);                                    \
        } else {                                                                                       \
            sched_step<C, NR, 0>();                                                                    \
        }                                                                                              \
        mfma_block<C>(fa1, fb1, acc);                                                                  \
        if (NEXT) sched_step<C, NR, 0>();                                                              \
        else sched_step<C, 0, 0>();                                                                    \
    } while (0)

    int j = 0;
    for (; j + 2 < KK; j += 2) {
        MK_GEMM_SLAB(0, r1, j, true);
        MK_GEMM_SLAB(1, r0, j + 1, true);
    }
    MK_GEMM_SLAB(0, r1, j, true);
    MK_GEMM_SLAB(1, r0, j + 1, false);
#undef MK_GEMM_SLAB
    __syncthreads();   // every wave is done with the stages before the next tile refills them

    // epilogue: lane holds y^T[n][m] for n = base + 8*(v/4) + 4*(lane/32) + v%4, m = lane%32
    const int n_limit = a.N - n0;
#pragma unroll
    for (int j = 0; j < C::MI; ++j) {
        const int m = wm * (C::BM / C::WM) + j * 32 + (lane & 31);
        if (m >= rows_valid) continue;
        uint16_t *yrow = a.y + (size_t)(row0 + m) * a.N + n0;
#pragma unroll
        for (int i = 0; i < C::NI; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = wn * (C::BN / C::WN) + i * 32 + 8 * g + 4 * (lane >> 5);
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

// The tile heights in use: full row tiles are 256 rows; the last (ragged)
// row tile of an expert takes the smallest height that covers its rows, so a
// tail of a few rows (and every tile of a decode-sized batch) costs a fraction
// of a full tile's matrix work.
typedef BigTile<256, 256, 2> TileM256;
typedef BigTile<128, 256, 2> TileM128;
typedef BigTile<64, 256, 4> TileM64;
typedef BigTile<32, 256, 4> TileM32;

__device__ __forceinline__ void gemm_tile_any(const GemmArgs &a, int e, int row0, int rows_valid, int n0,
                                              const LdsStages &ls)
{
    if (rows_valid > 128) gemm_tile_big<TileM256>(a, e, row0, rows_valid, n0, ls);
    else if (rows_valid > 64) gemm_tile_big<TileM128>(a, e, row0, rows_valid, n0, ls);
    else if (rows_valid > 32) gemm_tile_big<TileM64>(a, e, row0, rows_valid, n0, ls);
    else gemm_tile_big<TileM32>(a, e, row0, rows_valid, n0, ls);
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
__device__ __forceinline__ void gemm_worker(const GemmArgs &a, int w, int G, const LdsStages &ls)
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
        gemm_tile_any(a, p.e, row0, rows_valid, p.nb * C::BN, ls);
    }
}

}  // namespace mk
