// gemm_dev.h -- per-expert grouped GEMM on gfx950 matrix cores.
//
// y_perm[r, n] = bf16_rne(sum_i x_perm[r, i] * W[e, n, i]) for the rows r of
// expert e, fp32 accumulation: the dense-compute half of the "MoE
// Dispatch+GEMM" kernel ("mKernel UCCL fuses NVLink/RDMA/compute into one
// persistent CUDA kernel", zubnet.ai, paragraph 2).  The pages give no GEMM
// design; the one here is written for CDNA4:
//   - a workgroup of 4 waves owns a BN x BM tile of y^T (W rows x token rows);
//     each wave a (BN/2) x (BM/2) quadrant made of 32x32 v_mfma bf16 blocks
//     with K = 16 per instruction (one wave per SIMD);
//   - both operands are K-contiguous in HBM.  K runs in slabs of 64 (one
//     128-byte segment per tile row).  Slabs go from global memory straight
//     into LDS (buffer_load_dwordx4 ... lds: lane l's 16 bytes land at byte
//     16 l of a 1 KiB block), two stages, the loads of slab j + 2 issued while
//     slab j is computed, so the waves issue no LDS writes and hold no staging
//     registers: a wave's LDS issue rate (about 24 bytes per clock at one
//     wave per SIMD, measured) then serves the fragment reads alone;
//   - the 16-byte chunk index of each 128-byte LDS row is XOR-swizzled by
//     (row >> 1) & 7, so the fragment reads are conflict-free on the 64-bank
//     LDS; a load lane fetches the chunk that belongs at its LDS position;
//   - fragment reads of the next K = 16 step are interleaved with the MFMAs
//     of the current one (sched_group_barrier), and the one barrier per slab
//     sits before the last step, so the next slab's first reads and the next
//     loads overlap it;
//   - token rows come from an expert-contiguous row buffer, or straight from
//     the token matrix through the slot -> token map (a gather in the loads,
//     no copy);
//   - W is the MFMA "A" operand, so each lane ends with 4 consecutive output
//     columns of one row; the epilogue stages the bf16 tile in LDS and stores
//     whole 512-byte row segments (16 bytes per lane);
//   - ragged tails: tile rows past the expert's count read 0 (or the next
//     expert's rows) and are never stored; W rows past N likewise.
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
    const uint16_t *x_perm;      // [x_perm_rows, d] expert-contiguous rows (row mode)
    const uint16_t *x_tok;       // gather mode: the lowest source buffer (row r is token row_token[r]), or nullptr
    const int32_t *row_token;    // [R_cap] slot -> token (gather mode)
    int32_t T;                   // tokens
    // Gather mode: token t = s * x_rows_per_src + r is row r of source s, at byte x_src_off[s] + r * d * 2
    // from x_tok; the sources lie in the x_bytes (< 4 GiB) from x_tok.
    int32_t x_nsrc, x_rows_per_src;
    uint32_t x_src_off[kGatherSources];
    uint64_t x_bytes;
    // Gather mode with the tokens derived in place of row_token (nullptr: read row_token): the
    // per-64-token-block expert masks [nblk, E_local], the per-block exclusive bases of every expert
    // (16-bit ranks within the expert, LDS, same layout) and the expert offsets (LDS).
    const uint64_t *tok_mask;
    const uint16_t *tok_base;
    const int32_t *tok_off;
    int32_t tok_nblk;
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

// A tile of BM token rows x BN W rows computed by NW waves, WN of them along N
// and NW / WN along M.  A slab (K = 64) of an operand is BN / 8 (or BM / 8)
// blocks of 8 rows x 128 bytes, one 1 KiB global -> LDS load each; wave w
// loads blocks w, w + NW, w + 2 NW, ...: WS slots of W blocks, then XS slots of
// x blocks (when NW does not divide BM / 8, the last slot of some waves holds
// rows past the tile, which read 0 into a block the tile does not use).
template <int BM_, int BN_, int WN_, int NW_>
struct BigTile {
    static constexpr int BM = BM_;         // token rows per tile
    static constexpr int BN = BN_;         // W rows (output columns) per tile
    static constexpr int NW = NW_;         // waves per workgroup
    static constexpr int WN = WN_;         // waves along N (the other NW / WN along M)
    static constexpr int WM = NW_ / WN_;
    static constexpr int BK = 64;          // K per slab: one 128-byte LDS row per tile row
    static constexpr int NI = BN / WN / 32;   // 32-wide blocks per wave along N
    static constexpr int MI = BM / WM / 32;   // 32-wide blocks per wave along M
    static constexpr int WB = BN / 8;      // W blocks per slab
    static constexpr int XB = BM / 8;      // x blocks per slab
    static constexpr int WS = WB / NW;     // W load slots per wave
    static constexpr int XS = (XB + NW - 1) / NW;   // x load slots per wave
    static constexpr int NS = WS + XS;
    static constexpr int STAGE = 256 * BK * 2;   // bytes of one LDS array (the W or x half of a stage)
    static constexpr int THREADS = 64 * NW;
    static_assert(NI >= 1 && MI >= 1 && WB % NW == 0 && NW % 2 == 0 && BN <= 256 && BM <= 256, "tile shape");
};

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

// The same resource as four scalar dwords (base, stride 0, records, flags), for the slab loads below.
typedef uint32_t rsrc4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc4_t make_rsrc4(const void *base, size_t bytes)
{
    const uint64_t b = (uint64_t)base;
    return rsrc4_t{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu),
                   (uint32_t)__builtin_amdgcn_readfirstlane(bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes),
                   0x00020000u};
}

// One global -> LDS load: 16 bytes per lane from rsrc + voff (range-checked) + soff land at LDS byte
// lds_addr + 16 lane.  Written as an instruction of its own rather than the compiler builtin: for the
// builtin the compiler cannot tell that the fragment reads of the other stage do not alias the loads
// in flight, and waits for every load before each such read.  The loads have no register results; the
// caller waits for them (s_waitcnt vmcnt) before a barrier, and the compiler's own vmcnt waits only
// grow with loads it does not count.  M0 (the LDS address) is written by the compiler as an input;
// the s_nop covers the M0 -> LDS-load hazard.
// NT: non-temporal (the L2 keeps the line only briefly), for data that no other tile reads.
template <bool NT = false>
__device__ __forceinline__ void lds_load16(rsrc4_t rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff)
{
    if constexpr (NT)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                     "{m0}"(lds_addr));
    else
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                     "{m0}"(lds_addr));
}


// Global -> LDS load slot i of slab `slab` into one stage: slot i < WS is W
// block wave + NW i, the rest x block wave + NW (i - WS); block b covers
// operand rows 8 b .. 8 b + 7, i.e. LDS bytes [1024 b, 1024 b + 1024) of the
// stage array, lane l's 16 bytes at 1024 b + 16 l.  wo / xo: the lane's byte
// offsets of its row and chunk (the row part is range-checked: rows past the
// resource read 0); the K part (slab * 128 bytes) is the scalar offset.  WNT: the W
// loads are non-temporal.
template <class C, bool WNT = false>
__device__ __forceinline__ void dma_one(rsrc4_t wsrc, rsrc4_t xsrc, const uint32_t *wo, const uint32_t *xo, int i,
                                        int slab, lds_char_t *wbuf, lds_char_t *xbuf, int wave)
{
    const uint32_t k0 = __builtin_amdgcn_readfirstlane((uint32_t)slab * C::BK * 2);
    const bool isw = i < C::WS;
    const int vi = isw ? i : i - C::WS;
    // Every wave issues the same number of loads per slab, so that a wave's vmcnt waits (which count
    // its own loads) cover the slab: an x slot past the tile's XB blocks (32-row tiles of eight waves)
    // still loads, its rows lie past the tile's valid rows and read 0, and it lands in an LDS block the
    // tile never reads (block b < 8 of the 32-block x array).
    const int b = wave + C::NW * vi;
    lds_char_t *dst = (isw ? wbuf : xbuf) + b * 1024;
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    if (isw) lds_load16<WNT>(wsrc, lds_addr, wo[vi], k0);
    else lds_load16<false>(xsrc, lds_addr, xo[vi], k0);
}

template <class C, int I0, int I1>
__device__ __forceinline__ void dma_part(rsrc4_t wsrc, rsrc4_t xsrc, const uint32_t *wo, const uint32_t *xo,
                                         int slab, lds_char_t *wbuf, lds_char_t *xbuf, int wave)
{
#pragma unroll
    for (int i = I0; i < I1; ++i) dma_one<C>(wsrc, xsrc, wo, xo, i, slab, wbuf, xbuf, wave);
}

// The chunk a load lane fetches: LDS position lane % 8 of row 8 b + lane / 8 holds chunk
// (lane % 8) ^ ((row >> 1) & 7), and (row >> 1) & 7 = (4 (b % 2) + lane / 16) & 7 with b % 2 = wave % 2
// for every slot (NW is even).
__device__ __forceinline__ uint32_t dma_chunk_bytes(int wave, int lane)
{
    return (uint32_t)(((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) << 4);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kStoreNT = 2;   // cache-policy operand of the buffer store builtins: non-temporal

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


// Fragment q of a K = 16 step (q < NI: W block q of the wave's N range;
// else x block q - NI of its M range) from stage B: the LDS address is the
// lane's precomputed base for the step (row lane % 32 of the block's first
// row, chunk 2 kk + lane / 32 after the swizzle) plus immediates.
template <class C, int B>
__device__ __forceinline__ void read_frag(const lds_char_t *aw, const lds_char_t *ax, int q, bf16x8_t (&fa)[C::NI],
                                          bf16x8_t (&fb)[C::MI])
{
    typedef __attribute__((address_space(3))) const bf16x8_t lds_frag_t;
    if (q < C::NI) fa[q] = *(lds_frag_t *)(aw + B * C::STAGE + q * 32 * 128);
    else fb[q - C::NI] = *(lds_frag_t *)(ax + B * C::STAGE + (q - C::NI) * 32 * 128);
}

// The order in which a step's fragments are read: the one the next step's MFMA (0, 0) needs first,
// then the x fragments (MFMAs (0, j)), then the remaining W fragments.
template <class C>
__device__ __forceinline__ constexpr int frag_order(int r)
{
    return r == 0 ? 0 : (r <= C::MI ? C::NI + r - 1 : r - C::MI);
}

// One K = 16 step: the NI x MI MFMAs on (fa, fb) in order (i, j) row-major;
// after MFMA q, slab load q (q < NLD, ld(q)) and fragment read frag_order(q)
// of the next step (q < NRD, rd(...)).  The order is pinned: the reads and
// loads are spread over the MFMAs instead of bunching at one end.
template <class C, int NRD, int NLD, class RD, class LD>
__device__ __forceinline__ void mfma_step(const bf16x8_t (&fa)[C::NI], const bf16x8_t (&fb)[C::MI],
                                          f32x16_t (&acc)[C::NI][C::MI], RD &&rd, LD &&ld)
{
#pragma unroll
    for (int q = 0; q < C::NI * C::MI; ++q) {
        const int i = q / C::MI, j = q % C::MI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if (q < NLD) ld(q);
        if (q < NRD) rd(frag_order<C>(q));
        __builtin_amdgcn_sched_barrier(0);
    }
    // a step with fewer MFMAs than loads or reads issues the rest after them
#pragma unroll
    for (int q = C::NI * C::MI; q < NLD || q < NRD; ++q) {
        if (q < NLD) ld(q);
        if (q < NRD) rd(frag_order<C>(q));
    }
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
    static_assert(C::BN <= 256 && C::BM <= 256, "an output row segment is at most 512 bytes; at most 4 x 64 rows");
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
// w stores rows [w * BM / NW, (w + 1) * BM / NW) of the staged tile.
template <class C>
__device__ __forceinline__ void store_staged_tile(const GemmArgs &a, int row0, int rows_valid, int n0,
                                                  const LdsStages &ls, int wave, int lane)
{
    // Two rows per instruction; rows are read back in batches of up to 16, then stored, so the LDS
    // latency is paid once per batch.  (Opaque lane: see stage_tile.)
    int lo_ = lane;
    asm volatile("" : "+v"(lo_));
    lane = lo_;
    constexpr int RPW = C::BM / C::NW;
    constexpr int NS = RPW / 2, BATCH = NS < 8 ? NS : 8;
    static_assert(RPW % 2 == 0 && NS % BATCH == 0, "rows per wave");
    const int c = lane & 31;
    const bool col_ok = c * 8 < C::BN && n0 + c * 8 < a.N;   // N % 8 == 0: a chunk is wholly inside or outside
    // Rows past rows_valid fall outside the resource: those stores are dropped.  The stores are
    // non-temporal (no tile reads y back; skewed and wide-EP launches 1.5-2% shorter).
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
            if (col_ok) __builtin_amdgcn_raw_buffer_store_b128(v[b], ysrc, (uint32_t)(m * a.N + c * 8) * 2u, 0, kStoreNT);
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
    constexpr int RPW = C::BM / C::NW;
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
        if (col_ok) __builtin_amdgcn_raw_buffer_store_b128(o, hsrc, (uint32_t)(m * a.F + c * 8) * 2u, 0, kStoreNT);
    }
    __syncthreads();   // the stage arrays are free again for the next tile
}

// The tile heights in use for NW waves: full row tiles are 256 rows; the last
// (ragged) row tile of an expert takes the smallest height that covers its
// rows, so a tail of a few rows (and every tile of a decode-sized batch) costs
// a fraction of a full tile's matrix work.  Eight waves (two per SIMD): each
// wave owns 128 x 64 of a full tile; four waves: 128 x 128.
template <int NW>
struct Tiles {
    typedef BigTile<256, 256, 2, NW> M256;
    typedef BigTile<256, 128, 2, NW> M256H;   // a full row tile over the last 128 or fewer columns
    typedef BigTile<128, 256, 2, NW> M128;
    typedef BigTile<64, 256, 4, NW> M64;
    typedef BigTile<32, 256, NW == 8 ? 8 : 4, NW> M32;
};

// One GEMM task: token rows [row0, row0 + BM) of x_perm (rows_valid of them
// readable and stored), W rows [n0, n0 + BN) of expert e.  rows_valid <= 0:
// no task.
struct TileJob {
    int e, row0, rows_valid, n0;
    int w_once;   // the expert's rows fit this one short tile: no other task reads its W tile
};

// The lane's byte offsets of a tile's x rows: slot i covers tile row
// (wave + NW i) * 8 + lane / 8 (the same rows for every tile height; a
// shorter tile uses the first slots), plus its chunk.  Computed for the next task in the current one's
// epilogue, between staging its outputs and storing them.
template <int NW>
struct XOffsets {
    uint32_t v[Tiles<NW>::M256::XS];
};

// The token tables of the in-place path (tok_base, tok_off) live in LDS: read them as LDS, not through
// generic pointers (a generic load waits on both the LDS and the vector-memory counters).
typedef __attribute__((address_space(3))) const uint16_t lds_cu16_t;
typedef __attribute__((address_space(3))) const int32_t lds_ci32_t;

// Position of the j-th set bit of m (j < popcount(m)): halve the window each step.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int j)
{
    int pos = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const int c = __popcll(m & ((1ull << w) - 1ull));
        if (j >= c) {
            j -= c;
            m >>= w;
            pos += w;
        }
    }
    return pos;
}

// The tokens of ranks q[0..n) among expert e's rows: the last block b whose base is <= q holds it (bases
// grow by the block's count, so that block has more than q - base bits), at the (q - base)-th set bit of
// the block's mask.  The n searches run side by side without branches (one LDS latency per halving step
// for all of them) and the n mask loads are in flight together.  Lanes with valid[i] false get 0.
template <int NQ>
__device__ __forceinline__ void tokens_of_ranks(const GemmArgs &a, int e, const int (&q)[NQ], const bool (&valid)[NQ],
                                                int (&tok)[NQ])
{
    const int E = a.E_local;
    lds_cu16_t *base = (lds_cu16_t *)a.tok_base;
    int lo[NQ], hi[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        lo[i] = 0;
        hi[i] = a.tok_nblk;
    }
    for (int span = a.tok_nblk; span > 1; span = (span + 1) >> 1) {   // ceil(log2 nblk) halvings
        int v[NQ], mid[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            mid[i] = (lo[i] + hi[i]) >> 1;   // lo when the window is down to one block
            v[i] = base[mid[i] * E + e];
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const bool live = hi[i] - lo[i] > 1;
            lo[i] = live && v[i] <= q[i] ? mid[i] : lo[i];
            hi[i] = live && v[i] > q[i] ? mid[i] : hi[i];
        }
    }
    uint64_t m[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) m[i] = valid[i] ? a.tok_mask[(size_t)lo[i] * E + e] : 0ull;
#pragma unroll
    for (int i = 0; i < NQ; ++i) tok[i] = valid[i] ? lo[i] * 64 + nth_set_bit(m[i], q[i] - base[lo[i] * E + e]) : 0;
}

__device__ __forceinline__ int token_of_rank(const GemmArgs &a, int e, int q)
{
    const int qs[1] = {q};
    const bool valid[1] = {true};
    int tok[1];
    tokens_of_ranks<1>(a, e, qs, valid, tok);
    return tok[0];
}

template <int NW>
__device__ __forceinline__ XOffsets<NW> x_offsets(const GemmArgs &a, const TileJob &t, int wave, int lane)
{
    constexpr int XS = Tiles<NW>::M256::XS;
    XOffsets<NW> o;
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    const uint32_t ch = dma_chunk_bytes(wave, lane);
    int m[XS];
#pragma unroll
    for (int i = 0; i < XS; ++i) m[i] = (wave + NW * i) * 8 + (lane >> 3);
    if (!a.x_tok) {
#pragma unroll
        for (int i = 0; i < XS; ++i) o.v[i] = (uint32_t)m[i] * row_bytes + ch;
        return o;
    }
    // Gather: row m of the tile is token row_token[row0 + m] of the token matrix; rows past the tile's
    // valid rows point past the end of the resource and read 0 without a memory access.
    bool valid[XS];
    int tok[XS];
#pragma unroll
    for (int i = 0; i < XS; ++i) valid[i] = t.rows_valid > 0 && m[i] < t.rows_valid;
    if (a.tok_base) {
        const int r0 = t.row0 - ((lds_ci32_t *)a.tok_off)[t.e];   // rank of the tile's first row
        int q[XS];
#pragma unroll
        for (int i = 0; i < XS; ++i) q[i] = r0 + m[i];
        tokens_of_ranks<XS>(a, t.e, q, valid, tok);
    } else {
#pragma unroll
        for (int i = 0; i < XS; ++i) tok[i] = valid[i] ? a.row_token[t.row0 + m[i]] : 0;
    }
#pragma unroll
    for (int i = 0; i < XS; ++i) {
        uint32_t off = kPastResource;
        if (valid[i]) {
            const int sh = a.x_nsrc > 1 ? tok[i] / a.x_rows_per_src : 0;
            uint32_t base = a.x_src_off[0];
#pragma unroll
            for (int k = 1; k < kGatherSources; ++k)
                if (sh == k) base = a.x_src_off[k];
            off = base + (uint32_t)(tok[i] - sh * a.x_rows_per_src) * row_bytes;
        }
        o.v[i] = off + ch;
    }
    return o;
}

// The W and x buffer resources of a tile.
struct TileSrc {
    rsrc4_t w, x;
};

__device__ __forceinline__ TileSrc tile_src(const GemmArgs &a, const TileJob &t)
{
    TileSrc s;
    const size_t w_first = (size_t)t.e * a.N + t.n0;
    s.w = make_rsrc4(a.w + w_first * a.d, ((size_t)a.E_local * a.N - w_first) * a.d * 2);
    if (a.x_tok) s.x = make_rsrc4(a.x_tok, a.x_bytes);
    // Row mode: only the tile's valid rows are readable: rows past a ragged end return 0 without a
    // memory access (they may belong to a tile that is not yet moved).
    else s.x = make_rsrc4(a.x_perm + (size_t)t.row0 * a.d, (size_t)t.rows_valid * a.d * 2);
    return s;
}

// Per-lane byte offsets of the W loads (the same for every tile of a launch):
// slot i covers W tile rows (wave + NW i) * 8 + lane / 8.
template <int NW>
struct SlabOffsets {
    uint32_t v[Tiles<NW>::M256::WS];
};

// SwiGLU tiles (SW): tile rows 0..127 are gate rows f0.., rows 128..255 the up rows F + f0.., so the
// W loads of blocks 16.. (rows >= 128) skip F - 128 rows.
template <int NW, bool SW = false>
__device__ __forceinline__ SlabOffsets<NW> slab_offsets(const GemmArgs &a, int wave, int lane)
{
    SlabOffsets<NW> o;
    const uint32_t row_bytes = (uint32_t)a.d * 2;
    const uint32_t up_skip = SW ? (uint32_t)(a.F - 128) * row_bytes : 0u;
    const uint32_t ch = dma_chunk_bytes(wave, lane);
#pragma unroll
    for (int i = 0; i < Tiles<NW>::M256::WS; ++i) {
        const int b = wave + NW * i;
        o.v[i] = (uint32_t)(b * 8 + (lane >> 3)) * row_bytes + ch + (b >= 16 ? up_skip : 0u);
    }
    return o;
}

// One tile.  After the main loop the workgroup claims its next task
// (sc.claim() into `next`; not earlier, so that no workgroup holds a second
// task while others still look for their first), then runs the epilogue.
//
// Slab j (K = 64 j .. 64 j + 63) sits in stage j % 2 (W in ls.p[2 (j % 2)],
// x in ls.p[2 (j % 2) + 1]) and is computed in four K = 16 steps, the
// fragments of step s + 1 read during the MFMAs of step s.  Before step 3:
// wait for this wave's loads of slab j + 1 and for its fragment reads of step
// 3, then one barrier (every wave's slab j + 1 has landed, and no wave reads
// stage j % 2 any more); during step 3, issue the loads of slab j + 2 into
// stage j % 2 and read step 0 of slab j + 1.
template <class C, bool SW, class Sched>
__device__ __forceinline__ void gemm_tile_big(const GemmArgs &a, const TileJob &job, const XOffsets<C::NW> &xoff,
                                              TileJob &next, XOffsets<C::NW> &xoff_next, Sched &sc,
                                              const LdsStages &ls, const SlabOffsets<C::NW> &so)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform: keeps soffsets scalar
    const int lane = threadIdx.x % kWave;
    const int wn = wave % C::WN, wm = wave / C::WN;
    const TileSrc src = tile_src(a, job);
    const uint32_t *wo = so.v;
    const uint32_t *xo = xoff.v;
    const int KK = __builtin_amdgcn_readfirstlane(a.d / C::BK);   // even (d % 128 == 0); uniform

    // LDS: W of stage 0 and 1 in ls.p[0], ls.p[1]; x of stage 0 and 1 in ls.p[2], ls.p[3] (consecutive
    // 32 KiB arrays, so a stage is an immediate offset).  The lane's fragment bases, one per K = 16
    // step kk of a slab: row (lane & 31), chunk 2 kk + lane / 32 after the swizzle.
    const lds_char_t *aw[4], *ax[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        int fo = (lane & 31) * 128 + (((2 * kk + (lane >> 5)) ^ (((lane & 31) >> 1) & 7)) << 4);
        asm volatile("" : "+v"(fo));   // computed once, kept in a register (no re-adds in the loop)
        aw[kk] = ls.p[0] + wn * (C::BN / C::WN) * 128 + fo;
        ax[kk] = ls.p[2] + wm * (C::BM / C::WM) * 128 + fo;
    }

    f32x16_t acc[C::NI][C::MI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    lds_char_t *const wb[2] = {ls.p[0], ls.p[1]};
    lds_char_t *const xb[2] = {ls.p[2], ls.p[3]};
    constexpr int NL = C::NS;           // load slots per wave per slab
    constexpr int NR = C::NI + C::MI;   // fragment reads per wave per K = 16 step
    dma_part<C, 0, NL>(src.w, src.x, wo, xo, 0, wb[0], xb[0], wave);
    dma_part<C, 0, NL>(src.w, src.x, wo, xo, 1, wb[1], xb[1], wave);
    wait_vmem<NL>();   // this wave's slab 0 has landed
    __syncthreads();   // every wave's
    bf16x8_t fa0[C::NI], fb0[C::MI], fa1[C::NI], fb1[C::MI];
#pragma unroll
    for (int q = 0; q < NR; ++q) read_frag<C, 0>(aw[0], ax[0], q, fa0, fb0);

    auto none = [](int) {};
    // Slab J from stage B.  MODE (compile-time): 2 = slab J + 1 exists and slab J + 2 is loaded into
    // stage B during step 3; 1 = slab J + 1 exists, nothing more to load; 0 = the last slab.
#define MK_GEMM_SLAB(B, J, MODE)                                                                         \
    do {                                                                                                \
        mfma_step<C, NR, 0>(fa0, fb0, acc, [&](int q) { read_frag<C, B>(aw[1], ax[1], q, fa1, fb1); }, none); \
        mfma_step<C, NR, 0>(fa1, fb1, acc, [&](int q) { read_frag<C, B>(aw[2], ax[2], q, fa0, fb0); }, none); \
        mfma_step<C, NR, 0>(fa0, fb0, acc, [&](int q) { read_frag<C, B>(aw[3], ax[3], q, fa1, fb1); }, none); \
        if constexpr ((MODE) > 0) {                                                                     \
            __builtin_amdgcn_s_waitcnt(0x0070); /* vmcnt(0) lgkmcnt(0): slab J + 1 and step 3 here */   \
            __syncthreads();                                                                            \
            mfma_step<C, NR, (MODE) == 2 ? NL : 0>(                                                     \
                fa1, fb1, acc, [&](int q) { read_frag<C, 1 - (B)>(aw[0], ax[0], q, fa0, fb0); },        \
                [&](int q) {                                                                            \
                    if constexpr ((MODE) == 2)                                                          \
                        dma_one<C>(src.w, src.x, wo, xo, q, (J) + 2, wb[B], xb[B], wave);           \
                });                                                                                     \
        } else {                                                                                        \
            mfma_step<C, 0, 0>(fa1, fb1, acc, none, none);                                              \
        }                                                                                               \
    } while (0)

    int j = 0;
    for (; j + 2 < KK; j += 2) {
        MK_GEMM_SLAB(0, j, 2);
        MK_GEMM_SLAB(1, j + 1, 2);
    }
    MK_GEMM_SLAB(0, j, 1);
    MK_GEMM_SLAB(1, j + 1, 0);
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
    xoff_next = x_offsets<C::NW>(a, next, wave, lane);
    __syncthreads();   // the staged tile is complete
    if constexpr (SW) store_staged_swiglu<C>(a, job.row0, job.rows_valid, job.n0, ls, wave, lane);
    else store_staged_tile<C>(a, job.row0, job.rows_valid, job.n0, ls, wave, lane);
}

// Short tiles (BM <= 64: the ragged tail of an expert, every tile of a
// decode-sized batch) do little matrix work per slab and are bound by how
// fast a CU streams its W tile, i.e. by the bytes it has in flight.  They run
// three stages, two slabs ahead: W of stage s in ls.p[s], x of stage s at
// ls.p[3] + s * XSTAGE.  Otherwise the same step structure as gemm_tile_big
// (one barrier per slab, before its last step), with the stage index held at
// run time.  Loads of slabs past the end go to empty resources (no memory
// access; every wave keeps the same load count), and all loads are waited for
// before the epilogue reuses the stage arrays.
template <class C, bool SW, bool WNT, class Sched>
__device__ __forceinline__ void gemm_tile_stream(const GemmArgs &a, const TileJob &job, const XOffsets<C::NW> &xoff,
                                                 TileJob &next, XOffsets<C::NW> &xoff_next, Sched &sc,
                                                 const LdsStages &ls, const SlabOffsets<C::NW> &so)
{
    static_assert(C::BM <= 64, "three stages of x fit one 32 KiB array");
    constexpr int S = 3;
    constexpr int XSTAGE = (C::XB > C::XS * C::NW ? C::XB : C::XS * C::NW) * 1024;   // empty slots land inside
    static_assert(S * XSTAGE <= 32768, "x stages");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int wn = wave % C::WN, wm = wave / C::WN;
    const TileSrc src = tile_src(a, job);
    const TileSrc none{make_rsrc4(a.w, 0), make_rsrc4(a.w, 0)};
    const uint32_t *wo = so.v;
    const uint32_t *xo = xoff.v;
    const int KK = __builtin_amdgcn_readfirstlane(a.d / C::BK);

    const lds_char_t *aw[4], *ax[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        int fo = (lane & 31) * 128 + (((2 * kk + (lane >> 5)) ^ (((lane & 31) >> 1) & 7)) << 4);
        asm volatile("" : "+v"(fo));
        aw[kk] = ls.p[0] + wn * (C::BN / C::WN) * 128 + fo;
        ax[kk] = ls.p[3] + wm * (C::BM / C::WM) * 128 + fo;
    }
    f32x16_t acc[C::NI][C::MI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    constexpr int NL = C::NS;
    constexpr int NR = C::NI + C::MI;
    // stage st: W at ls.p[0] + st * 32768, x at ls.p[3] + st * XSTAGE
    auto issue = [&](int slab, int st, int i) {
        const bool real = slab < KK;
        dma_one<C, WNT>(real ? src.w : none.w, real ? src.x : none.x, wo, xo, i, real ? slab : 0,
                        ls.p[0] + st * 32768, ls.p[3] + st * XSTAGE, wave);
    };
#pragma unroll
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
        for (int i = 0; i < NL; ++i) issue(sl, sl, i);
    wait_vmem<(S - 1) * NL>();   // this wave's slab 0 has landed
    __syncthreads();
    bf16x8_t fa0[C::NI], fb0[C::MI], fa1[C::NI], fb1[C::MI];
    typedef __attribute__((address_space(3))) const bf16x8_t lds_frag_t;
    // fragment q of step kk from the stage at byte offsets (wst, xst)
    auto rd = [&](int kk, int q, int wst, int xst, bf16x8_t (&fa)[C::NI], bf16x8_t (&fb)[C::MI]) {
        if (q < C::NI) fa[q] = *(lds_frag_t *)(aw[kk] + wst + q * 32 * 128);
        else fb[q - C::NI] = *(lds_frag_t *)(ax[kk] + xst + (q - C::NI) * 32 * 128);
    };
#pragma unroll
    for (int q = 0; q < NR; ++q) rd(0, q, 0, 0, fa0, fb0);
    auto none_ld = [](int) {};
    int st = 0;
    for (int j = 0; j < KK; ++j) {
        const int wst = __builtin_amdgcn_readfirstlane(st * 32768), xst = __builtin_amdgcn_readfirstlane(st * XSTAGE);
        const int st1 = st == S - 1 ? 0 : st + 1;
        mfma_step<C, NR, 0>(fa0, fb0, acc, [&](int q) { rd(1, q, wst, xst, fa1, fb1); }, none_ld);
        mfma_step<C, NR, 0>(fa1, fb1, acc, [&](int q) { rd(2, q, wst, xst, fa0, fb0); }, none_ld);
        mfma_step<C, NR, 0>(fa0, fb0, acc, [&](int q) { rd(3, q, wst, xst, fa1, fb1); }, none_ld);
        if (j + 1 < KK) {
            // slab j + 1 has landed (slab j + 2 may still be in flight) and this wave's reads of stage st are done
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt((NL & 15) | ((NL >> 4) << 14) | 0x0070);   // vmcnt(NL) lgkmcnt(0)
            __syncthreads();
            const int wst1 = __builtin_amdgcn_readfirstlane(st1 * 32768);
            const int xst1 = __builtin_amdgcn_readfirstlane(st1 * XSTAGE);
            mfma_step<C, NR, NL>(fa1, fb1, acc, [&](int q) { rd(0, q, wst1, xst1, fa0, fb0); },
                                 [&](int i) { issue(j + S, st, i); });
        } else {
            mfma_step<C, 0, 0>(fa1, fb1, acc, none_ld, none_ld);
        }
        st = st1;
    }
    wait_vmem_all();   // the loads past the end land in the stages the epilogue reuses

    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::MI; ++j) asm volatile("" : "+a"(acc[i][j]));
    __builtin_amdgcn_sched_barrier(0);

    __syncthreads();
    stage_tile<C>(acc, ls, wave, lane);
    next = sc.claim();
    xoff_next = x_offsets<C::NW>(a, next, wave, lane);
    __syncthreads();
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
// tile.  HALF_N: the build with the half-width tile for a ragged last column
// block (a kernel of its own, so that shapes with N % 256 == 0 keep the code
// and register allocation of the build without it).
template <int NW, bool SW = false, bool HALF_N = false, class Sched>
__device__ __forceinline__ void gemm_run(const GemmArgs &a, Sched &sc, const LdsStages &ls)
{
    typedef Tiles<NW> T;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const SlabOffsets<NW> so = slab_offsets<NW, SW>(a, wave, lane);
    TileJob job = sc.claim();
    XOffsets<NW> xo = x_offsets<NW>(a, job, wave, lane);
    while (job.rows_valid > 0) {
        if (!sc.wait(job)) return;
        TileJob next;
        XOffsets<NW> xo_next;
        // The last column block of a ragged N (128 columns or fewer) runs half as many MFMAs.
        if (HALF_N && !SW && job.rows_valid > 128 && a.N - job.n0 <= 128)
            gemm_tile_big<typename T::M256H, SW>(a, job, xo, next, xo_next, sc, ls, so);
        else if (job.rows_valid > 128) gemm_tile_big<typename T::M256, SW>(a, job, xo, next, xo_next, sc, ls, so);
        else if (job.rows_valid > 64) gemm_tile_big<typename T::M128, SW>(a, job, xo, next, xo_next, sc, ls, so);
        // A W tile that only this task reads streams non-temporally, so that it does not push the
        // token rows and the other tiles' W out of the L2 (decode: 0.221 -> 0.205 ms; with W tiles
        // that several row tiles share, Mixtral-shaped, the hint made the launch 5% slower).
        else if (job.rows_valid > 32 && job.w_once)
            gemm_tile_stream<typename T::M64, SW, true>(a, job, xo, next, xo_next, sc, ls, so);
        else if (job.rows_valid > 32) gemm_tile_stream<typename T::M64, SW, false>(a, job, xo, next, xo_next, sc, ls, so);
        else if (job.w_once) gemm_tile_stream<typename T::M32, SW, true>(a, job, xo, next, xo_next, sc, ls, so);
        else gemm_tile_stream<typename T::M32, SW, false>(a, job, xo, next, xo_next, sc, ls, so);
        sc.done();
        job = next;
        xo = xo_next;
    }
}

// Task q -> its tile; tasks are ordered expert-major, then column block, then
// row tile, so consecutive tasks share one W tile.  q >= n_tasks: no task.
// A SwiGLU column block is 128 features (256 W rows: their gate and up rows).
template <class C, bool SW = false>
__device__ __forceinline__ TileJob job_of_task(const GemmArgs &a, const int32_t *tile_off, const int32_t *offsets,
                                               int NB, int n_tasks, int q)
{
    TileJob t{0, 0, 0, 0, 0};
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
    t.w_once = offsets[e + 1] - offsets[e] <= 64;
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
    gemm_run<C::NW, SW>(a, sc, ls);
}

}  // namespace mk
