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
//     columns of one row; the epilogue stages the bf16 tile in LDS and stores
//     whole 512-byte row segments (16 bytes per lane);
//   - ragged tails: tile rows past the expert's count read padding or the next
//     expert's rows and are never stored; W rows past N are clamped.
#pragma once

#include "mk_args.h"
#include "mk_device.h"

namespace mk {

typedef __attribute__((address_space(3))) char lds_char_t;

// The four LDS stage arrays of a GEMM workgroup, as LDS-space pointers (their
// 32-bit LDS addresses are compile-time constants once the arrays are placed).
// The arrays are consecutive, 32 KiB each: p[k] == p[0] + k * 32768.
struct LdsStages {
    lds_char_t *p[4];
};

// Stage array k (0..3) for a runtime k (address arithmetic: an indexed load of
// p[] would put the pointer array in scratch memory).
__device__ __forceinline__ lds_char_t *stage_at(const LdsStages &ls, int k)
{
    return ls.p[0] + k * 32768;
}

struct GemmArgs {
    const uint16_t *x_perm;      // [x_perm_rows, d]
    const uint16_t *w;           // [E_local, N, d]
    uint16_t *y;                 // [R_cap, N]
    const int32_t *offsets;      // [E_local + 1]
    const int32_t *tile_off;     // [E_local + 1] exclusive prefix of row tiles
    WsHeader *hdr;
    int32_t d, N, E_local;
    // SwiGLU launches only: F features per expert; W holds 2F rows per expert (gate rows, then up rows),
    // so N == 2F, and y is h [rows, F] = silu(gate) * up.
    int32_t F;
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
// scalar offset.  SwiGLU tiles (SW): voff[i >= WL / 2] carry the up rows' skip (slab_offsets<true>);
// the x loads that share those offsets take it off again.
template <class C, int I0, int I1, bool SW = false>
__device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t wsrc, __amdgpu_buffer_rsrc_t xsrc,
                                          const uint32_t (&voff)[C::WL], int slab, SlabRegs<C> &r,
                                          uint32_t up_skip = 0)
{
    const uint32_t k0 = (uint32_t)slab * C::BK * 2;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const int vi = i < C::WL ? i : i - C::WL;
        const uint32_t vo = (SW && i >= C::WL && vi >= C::WL / 2) ? voff[vi] - up_skip : voff[vi];
        r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(i < C::WL ? wsrc : xsrc, vo, k0, 0);
    }
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

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two floats as two round-to-nearest-even bf16 in one word (lo = a), one
// conversion instruction for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
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

// Epilogue, first half: the tile's bf16 outputs go into LDS, so that the
// global stores (second half) are whole 512-byte output row segments (16 bytes
// per lane, two rows per wave store) instead of 8-byte pieces scattered over
// 32 rows per store.
//   - Lane (wave, lane) holds y^T[n][m] for n = nw + i*32 + 8*(v/4) + 4*(lane/32)
//     + v%4, m = mw + j*32 + lane%32 (32x32 MFMA accumulator layout).  Each
//     group of 4 consecutive n is one 8-byte write into LDS row m.
//   - LDS row m of the tile lives in stage array m / 64 at (m % 64) * 512 bytes;
//     its 16-byte chunk c sits at position c ^ (m % 32), so the 32 rows one
//     write touches spread over all banks and a row read back is contiguous.
//   - The caller's stage arrays are free: the main loop ends with a barrier.
template <class C>
__device__ __forceinline__ void stage_tile(const f32x16_t (&acc)[C::NI][C::MI], const LdsStages &ls, int wave,
                                           int lane)
{
    static_assert(C::BN == 256 && C::BM <= 256, "an output row segment is 512 bytes; at most 4 x 64 rows");
    const int wn = wave % C::WN, wm = wave / C::WN;
    // The swizzled offsets depend only on the lane; computed from an opaque copy of it here, so that the
    // compiler does not hoist dozens of them out of the tile loop and keep them live (spilled) throughout.
    int lo_ = lane;
    asm volatile("" : "+v"(lo_));
    lane = lo_;
#pragma unroll
    for (int j = 0; j < C::MI; ++j) {
        const int mb = wm * (C::BM / C::WM) + j * 32;   // uniform, a multiple of 32
        const int m = mb + (lane & 31);
        lds_char_t *row = stage_at(ls, __builtin_amdgcn_readfirstlane(mb >> 6)) + ((mb & 63) + (lane & 31)) * 512;
#pragma unroll
        for (int i = 0; i < C::NI; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = (wn * (C::BN / C::WN) + i * 32 + 8 * g) >> 3;
                typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
                *(lds_u32x2_t *)(row + ((c ^ (m & 31)) << 4) + ((lane >> 5) << 3)) =
                    u32x2_t{pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                            pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
            }
        }
    }
}

// Second half of the epilogue: after a barrier that follows stage_tile, wave
// w stores rows [w * BM / 4, (w + 1) * BM / 4) of the staged tile.
template <class C>
__device__ __forceinline__ void store_staged_tile(const GemmArgs &a, int row0, int rows_valid, int n0,
                                                  const LdsStages &ls, int wave, int lane)
{
    // Two rows per instruction; rows are read back in batches of up to 16, then stored, so the LDS
    // latency is paid once per batch.  (Opaque lane: see stage_tile.)
    int lo_ = lane;
    asm volatile("" : "+v"(lo_));
    lane = lo_;
    constexpr int RPW = C::BM / 4;
    constexpr int NS = RPW / 2, BATCH = NS < 8 ? NS : 8;
    static_assert(RPW % 2 == 0 && NS % BATCH == 0, "rows per wave");
    const int c = lane & 31;
    const bool col_ok = n0 + c * 8 < a.N;   // N % 8 == 0: a chunk is wholly inside or outside
    // Rows past rows_valid fall outside the resource: those stores are dropped.
    const __amdgpu_buffer_rsrc_t ysrc = make_rsrc(a.y + (size_t)row0 * a.N + n0, (size_t)rows_valid * a.N * 2);
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += BATCH) {
        v4i_t v[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int mb = wave * RPW + 2 * (s0 + b);   // uniform and even: rows mb, mb + 1 share a stage array
            const int m = mb + (lane >> 5);
            typedef __attribute__((address_space(3))) const v4i_t lds_cv4i_t;
            v[b] = *(lds_cv4i_t *)(stage_at(ls, __builtin_amdgcn_readfirstlane(mb >> 6)) +
                                   ((mb & 63) + (lane >> 5)) * 512 + ((c ^ (m & 31)) << 4));
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int m = wave * RPW + 2 * (s0 + b) + (lane >> 5);
            if (col_ok) __builtin_amdgcn_raw_buffer_store_b128(v[b], ysrc, (uint32_t)(m * a.N + c * 8) * 2u, 0, 0);
        }
    }
    __syncthreads();   // the stage arrays are free again for the next tile
}

// SwiGLU epilogue, after a barrier that follows stage_tile: staged columns 0..127 are the gate values
// and 128..255 the up values of features f0 .. f0 + 127, both already rounded to bf16 (as a gate|up
// GEMM stores them); h = bf16(silu(g) * u) in fp32, the same expression as the separate SwiGLU
// kernel, so the two routes give the same bits.  Lane: row mb + lane / 16, 8 features 8 (lane % 16).
template <class C>
__device__ __forceinline__ void store_staged_swiglu(const GemmArgs &a, int row0, int rows_valid, int f0,
                                                    const LdsStages &ls, int wave, int lane)
{
    int lo_ = lane;
    asm volatile("" : "+v"(lo_));
    lane = lo_;
    constexpr int RPW = C::BM / 4;
    static_assert(RPW % 4 == 0, "rows per wave");
    const int c = lane & 15;
    const bool col_ok = f0 + c * 8 < a.F;   // F % 8 == 0
    const __amdgpu_buffer_rsrc_t hsrc = make_rsrc(a.y + (size_t)row0 * a.F + f0, (size_t)rows_valid * a.F * 2);
#pragma unroll 2
    for (int s0 = 0; s0 < RPW; s0 += 4) {
        const int mb = wave * RPW + s0;   // uniform, a multiple of 4: rows mb .. mb + 3 share a stage array
        const int m = mb + (lane >> 4);
        typedef __attribute__((address_space(3))) const v4i_t lds_cv4i_t;
        const lds_char_t *row = stage_at(ls, __builtin_amdgcn_readfirstlane(mb >> 6)) + (m & 63) * 512;
        const v4i_t gv = *(lds_cv4i_t *)(row + ((c ^ (m & 31)) << 4));
        const v4i_t uv = *(lds_cv4i_t *)(row + (((c + 16) ^ (m & 31)) << 4));
        v4i_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float g0 = __uint_as_float((uint32_t)gv[q] << 16), g1 = __uint_as_float((uint32_t)gv[q] & 0xFFFF0000u);
            const float u0 = __uint_as_float((uint32_t)uv[q] << 16), u1 = __uint_as_float((uint32_t)uv[q] & 0xFFFF0000u);
            const float h0 = g0 / (1.0f + expf(-g0)) * u0;
            const float h1 = g1 / (1.0f + expf(-g1)) * u1;
            o[q] = (int32_t)pack_bf16x2(h0, h1);
        }
        if (col_ok) __builtin_amdgcn_raw_buffer_store_b128(o, hsrc, (uint32_t)(m * a.F + c * 8) * 2u, 0, 0);
    }
    __syncthreads();   // the stage arrays are free again for the next tile
}

// The tile heights in use: full row tiles are 256 rows; the last (ragged)
// row tile of an expert takes the smallest height that covers its rows, so a
// tail of a few rows (and every tile of a decode-sized batch) costs a fraction
// of a full tile's matrix work.
typedef BigTile<256, 256, 2> TileM256;
typedef BigTile<128, 256, 2> TileM128;
typedef BigTile<64, 256, 4> TileM64;
typedef BigTile<32, 256, 4> TileM32;

// One GEMM task: token rows [row0, row0 + BM) of x_perm (rows_valid of them
// readable and stored), W rows [n0, n0 + BN) of expert e.  rows_valid <= 0:
// no task.
struct TileJob {
    int e, row0, rows_valid, n0;
};

// The W and x buffer resources of a tile.
struct TileSrc {
    __amdgpu_buffer_rsrc_t w, x;
};

__device__ __forceinline__ TileSrc tile_src(const GemmArgs &a, const TileJob &t)
{
    TileSrc s;
    const size_t w_first = (size_t)t.e * a.N + t.n0;
    s.w = make_rsrc(a.w + w_first * a.d, ((size_t)a.E_local * a.N - w_first) * a.d * 2);
    // Only the tile's valid rows are readable: rows past a ragged end return 0 without a memory access
    // (they may belong to a tile that is not yet moved).
    s.x = make_rsrc(a.x_perm + (size_t)t.row0 * a.d, (size_t)t.rows_valid * a.d * 2);
    return s;
}

// Per-lane byte offsets of the slab loads (the same for every tile of a
// launch): load i covers tile rows (4 i + wave) * 8 + lane / 8, 16 bytes at
// chunk lane % 8 of the row's 128-byte slab segment.
struct SlabOffsets {
    uint32_t v[TileM256::WL];
};

// SwiGLU tiles (SW): tile rows 0..127 are gate rows f0.., rows 128..255 the up rows F + f0.., so the
// W loads of the second half (i >= WL / 2: rows >= 128) skip F - 128 rows.
template <bool SW = false>
__device__ __forceinline__ SlabOffsets slab_offsets(const GemmArgs &a, int wave, int lane)
{
    SlabOffsets o;
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    const uint32_t up_skip = SW ? (uint32_t)(a.F - 128) * row_bytes : 0u;
#pragma unroll
    for (int i = 0; i < TileM256::WL; ++i)
        o.v[i] = (uint32_t)((4 * i + wave) * 8 + (lane >> 3)) * row_bytes + (uint32_t)(lane & 7) * 16u +
                 (i >= TileM256::WL / 2 ? up_skip : 0u);
    return o;
}

// One tile.  After the main loop the workgroup claims its next task
// (sc.claim() into `next`; not earlier, so that no workgroup holds a second
// task while others still look for their first), then runs the epilogue.
//
// Slab j (K = 64 j .. 64 j + 63) is computed from LDS buffer j % 2 (W in
// ls.p[2 (j % 2)], x in ls.p[2 (j % 2) + 1]) in four K = 16 steps, with the
// fragments of step s + 1 read during the MFMAs of step s.  Between steps 2
// and 3: write slab j + 1 from registers into the other buffer (its old slab
// j - 1 was last read before the previous barrier), load slab j + 3 into the
// registers just freed, barrier, then read step 0 of slab j + 1 during step 3.
// Slab s lives in register set s % 2, loaded two slabs before it is written.
template <class C, bool SW, class Sched>
__device__ __forceinline__ void gemm_tile_big(const GemmArgs &a, const TileJob &job, TileJob &next, Sched &sc,
                                              const LdsStages &ls, const SlabOffsets &so)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps soffsets scalar
    const int lane = threadIdx.x % kWave;
    const int wn = wave % C::WN, wm = wave / C::WN;
    const TileSrc src = tile_src(a, job);
    const uint32_t(&voff)[TileM256::WL] = so.v;
    // Loads of slabs past the end go to empty resources: they read 0 without a memory access, and
    // keep the number of loads in flight the same on every path.
    const __amdgpu_buffer_rsrc_t wnone = make_rsrc(a.w, 0), xnone = make_rsrc(a.x_perm, 0);
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
    const uint32_t up_skip = SW ? (uint32_t)__builtin_amdgcn_readfirstlane((a.F - 128) * a.d * 2) : 0u;
    load_part<C, 0, NL, SW>(src.w, src.x, voff, 0, r0, up_skip);
    load_part<C, 0, NL, SW>(src.w, src.x, voff, 1, r1, up_skip);
    store_part<C, 0, NL>(r0, wb[0], xb[0], wave, st_off);
    load_part<C, 0, NL, SW>(KK > 2 ? src.w : wnone, KK > 2 ? src.x : xnone, voff, 2, r0, up_skip);
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
        const __amdgpu_buffer_rsrc_t wl_ = ahead_ ? src.w : wnone, xl_ = ahead_ ? src.x : xnone;       \
        lds_char_t *const wo_ = wb[1 - (B)];                                                           \
        lds_char_t *const xo_ = xb[1 - (B)];                                                           \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[1], fa1, fb1);                                    \
        mfma_block<C>(fa0, fb0, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, 0, P1>(RN, wo_, xo_, wave, st_off);                                          \
            load_part<C, 0, P1, SW>(wl_, xl_, voff, (J) + 3, RN, up_skip);                                 \
            sched_step<C, NR, P1>();                                                                   \
        } else {                                                                                       \
            sched_step<C, NR, 0>();                                                                    \
        }                                                                                              \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[2], fa0, fb0);                                    \
        mfma_block<C>(fa1, fb1, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, P1, P2>(RN, wo_, xo_, wave, st_off);                                         \
            load_part<C, P1, P2, SW>(wl_, xl_, voff, (J) + 3, RN, up_skip);                                \
            sched_step<C, NR, P2 - P1>();                                                              \
        } else {                                                                                       \
            sched_step<C, NR, 0>();                                                                    \
        }                                                                                              \
        load_frags<C>(wb[B], xb[B], wn, wm, frag_off[3], fa1, fb1);                                    \
        mfma_block<C>(fa0, fb0, acc);                                                                  \
        if (NEXT) {                                                                                    \
            store_part<C, P2, NL>(RN, wo_, xo_, wave, st_off);                                         \
            load_part<C, P2, NL, SW>(wl_, xl_, voff, (J) + 3, RN, up_skip);                                \
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

    // Distance between the last MFMA and the first read of its accumulators.  The compiler pads that
    // read to its own model of the instruction's latency; a build whose first read came 11 wait
    // states after the last 32x32x16 MFMA got stale values for that register block, one of 13 has
    // not.  Three more s_nops make the distance independent of how the epilogue is scheduled: the
    // empty statements take the accumulators as operands, so every later read or copy follows them.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j) asm volatile("" : "+a"(acc[i][j]));
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue: claim the next task, stage the outputs in LDS, store them as whole row segments.
    __syncthreads();   // every wave is done with the stages before the epilogue reuses them
    stage_tile<C>(acc, ls, wave, lane);
    next = sc.claim();
    __syncthreads();   // the staged tile is complete
    if constexpr (SW) store_staged_swiglu<C>(a, job.row0, job.rows_valid, job.n0, ls, wave, lane);
    else store_staged_tile<C>(a, job.row0, job.rows_valid, job.n0, ls, wave, lane);
}

// A Sched made of three callables.
template <class Cl, class Wa, class Do>
struct LambdaSched {
    Cl &claim_;
    Wa &wait_;
    Do &done_;
    __device__ TileJob claim() { return claim_(); }
    __device__ bool wait(const TileJob &t) { return wait_(t); }
    __device__ void done() { done_(); }
};

// The persistent tile loop.  Sched provides: claim() -> the next TileJob of
// this workgroup (rows_valid <= 0: none left); wait(job) -> false if the
// workgroup must stop (a failed wait for the job's rows); done() after each
// tile.
template <bool SW = false, class Sched>
__device__ __forceinline__ void gemm_run(const GemmArgs &a, Sched &sc, const LdsStages &ls)
{
    const SlabOffsets so = slab_offsets<SW>(a, __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), threadIdx.x % kWave);
    TileJob job = sc.claim();
    while (job.rows_valid > 0) {
        if (!sc.wait(job)) return;
        TileJob next;
        if (job.rows_valid > 128) gemm_tile_big<TileM256, SW>(a, job, next, sc, ls, so);
        else if (job.rows_valid > 64) gemm_tile_big<TileM128, SW>(a, job, next, sc, ls, so);
        else if (job.rows_valid > 32) gemm_tile_big<TileM64, SW>(a, job, next, sc, ls, so);
        else gemm_tile_big<TileM32, SW>(a, job, next, sc, ls, so);
        sc.done();
        job = next;
    }
}

// Task q -> its tile; tasks are ordered expert-major, then column block, then
// row tile, so consecutive tasks share one W tile.  q >= n_tasks: no task.
// A SwiGLU column block is 128 features (256 W rows: their gate and up rows).
template <class C, bool SW = false>
__device__ __forceinline__ TileJob job_of_task(const GemmArgs &a, const int32_t *tile_off, const int32_t *offsets,
                                               int NB, int n_tasks, int q)
{
    TileJob t{0, 0, 0, 0};
    if (q >= n_tasks) return t;
    int lo = 0, hi = a.E_local;   // find e: tile_off[e]*NB <= q < tile_off[e+1]*NB
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] * NB <= q) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int nt = tile_off[e + 1] - tile_off[e];
    const int rem = q - tile_off[e] * NB;
    const int nb = rem / nt, mt = rem % nt;
    t.e = e;
    t.row0 = offsets[e] + mt * C::BM;
    t.rows_valid = min(C::BM, offsets[e + 1] - offsets[e] - mt * C::BM);
    t.n0 = nb * (SW ? C::BN / 2 : C::BN);
    return t;
}

// Persistent workgroup loop over GEMM tasks.  Workgroup w (of G, G % 8 == 0)
// runs task round*G + slot(w); slot() gives the workgroups of one XCD
// (w % 8 == x, dispatched round-robin over the 8 XCDs) a contiguous run of
// tasks, so tasks sharing a W tile share that XCD's L2.
template <class C, bool SW = false>
__device__ __forceinline__ void gemm_worker(const GemmArgs &a, int w, int G, const LdsStages &ls)
{
    struct Sched {
        const GemmArgs &a;
        int NB, n_tasks, q, G;
        __device__ TileJob claim()
        {
            const TileJob t = job_of_task<C, SW>(a, a.tile_off, a.offsets, NB, n_tasks, q);
            q += G;
            return t;
        }
        __device__ bool wait(const TileJob &) { return true; }
        __device__ void done() {}
    };
    const int NB = SW ? (a.F + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN;
    Sched sc{a, NB, (int)a.hdr->n_tiles * NB, (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w, G};
    gemm_run<SW>(a, sc, ls);
}

}  // namespace mk
