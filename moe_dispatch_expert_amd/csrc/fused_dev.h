// fused_dev.h -- the persistent fused dispatch + expert GEMM kernel body.
//
// "mKernel UCCL fuses NVLink/RDMA/compute into one persistent CUDA kernel"
// (zubnet.ai), paragraph 2, describes one persistent kernel that pays the
// launch cost once and overlaps at tile granularity, so a tile that has
// arrived feeds the GEMM while the next is in flight; "UC Berkeley presenta
// mKernel ..." (edge.aivizor.me), paragraph 2, has thread blocks take roles
// (compute, communication) with the count per role set per tensor shape.
// Here, on one MI355X, a co-resident grid of workgroups runs:
//   phase 1  router logits                                  (all workgroups)
//   -- grid barrier A --
//   phase 2  top-k, gate, per-64-token histogram + ranks    (all)
//   -- grid barrier B --
//   phase 3  offsets / per-block bases by an LDS scan in every workgroup,
//            slot map and row map for the workgroup's own token blocks
//   (-- grid barrier C, only when the GEMM must read row_token: a block-base
//            table too large for LDS, or rows from the arrival simulator --)
//   rows     in place: the GEMM tiles read their token rows straight from the
//            sources, each tile first waiting (acquire) for the ready flags of
//            its rows' source chunks when rows arrive from peers; or movers
//            copy row chunks of each tile into the expert-contiguous buffer
//            (waiting on the chunk flags) and bump the tile's arrival count
//            (release), then join the compute role;
//   compute  take GEMM tasks from per-XCD queues, wait until the tile's rows are
//            there, run the tile.
//   arrival simulator (optional, the last workgroup, outside the barriers):
//            stands in for the peers and releases source-chunk flags at given
//            delays, then (in place) joins the compute role after barrier C.
#pragma once

#include "gemm_dev.h"
#include "layout_dev.h"
#include "mk_args.h"
#include "mk_device.h"
#include "route_dev.h"

namespace mk {

constexpr int kMoveRows = 32;          // rows per mover work unit
constexpr int kShortTile = 64;         // a last row tile of at most this many rows is short (tile order)
constexpr int kScanHalf = 8192;       // ints per LDS array in phase 3
constexpr int kMaxScanEntries = 2 * kScanHalf; // nblk * E_local held in LDS by phase 3
constexpr int kBaseTab = 8192;        // nblk * E_local bases kept through the GEMM (in-place path, no 3rd barrier),
                                      // as 16-bit ranks within an expert (T < 65536)

struct FusedArgs {
    RouterArgs ra;
    TopkArgs ta;
    CountArgs ca;
    GemmArgs ga;
    SrcRows src;
    SrcFlags fl;
    const int32_t *ids_in;       // nullptr: route inside
    int32_t *ids_user;           // copy of ids (given ids path) or nullptr
    int32_t *offsets;            // [E_local + 1] user
    int32_t *slot_of;            // [T, k] user
    int32_t *row_token_ws;       // [R_cap]
    int32_t *row_token_user;     // or nullptr
    uint16_t *x_perm;            // [x_perm_rows, d] the expert-contiguous row buffer
    int32_t *blkbase;            // [nblk, E_local]
    int32_t *tile_off;           // [E_local + 1]
    uint32_t *tile_cnt;          // [max_tiles] row chunks moved into each tile (reset every call)
    uint32_t *xcd_next;          // [8] per-XCD task counters (reset every call)
    uint32_t *bar_flag;          // [kBarrierWGs] grid barrier: generation each workgroup has reached
    WsHeader *hdr;
    uint64_t spin_limit;
    int32_t T, d, E, k, e_begin, E_local, nblk, bm;
    int32_t n_mover;             // workgroups that start as movers (0: gather mode)
    int32_t tails_last;          // 1: GEMM tasks of full row tiles first, the experts' short last tiles after
    int32_t gather;              // 1: no mover role; the GEMM reads token rows in place (sources inside one
                                 // buffer resource), each tile waiting for its rows' chunk flags if rows
                                 // arrive from peers
    int32_t has_sim;             // last workgroup is the arrival simulator
    int32_t max_tiles;
    uint32_t ticks_per_us;       // wall-clock ticks per microsecond
    uint64_t *trace;             // [kTraceWGs][kTraceWords] per-workgroup phase stamps
    int32_t *status_out;         // nullptr, or [2]: the call's (error code, detail), written by the last
                                 // workgroup out, which then clears the workspace's error words
};

// Trace record words (wall-clock ticks unless noted), written by thread 0.
enum TraceWord {
    kTrStart = 0, kTrRouted, kTrBarA, kTrCounted, kTrBarB, kTrSlots, kTrBarC, kTrMoved, kTrFirstTask,
    kTrDone, kTrTasks /* count */, kTrWaitTicks, kTrXcc /* hardware XCC id */, kTrUnits /* count */,
    kTrCopyTicks, kTrReleaseTicks, kTrSelected
};

__device__ __forceinline__ void trace_put(const FusedArgs &a, int word, uint64_t v)
{
    if (threadIdx.x == 0 && blockIdx.x < kTraceWGs) a.trace[blockIdx.x * kTraceWords + word] = v;
}

__device__ __forceinline__ int fused_participants(const FusedArgs &a) { return (int)gridDim.x - a.has_sim; }

// Barrier targets of a call: barrier b (1, 2, 3) of the call with epoch c waits for the value 4 c + b.
// Every workgroup reads the epoch at its start; the last workgroup to leave a call advances it
// (fused_exit), so arrival words that a failed call left behind can never satisfy a barrier of a
// later call.
__device__ __forceinline__ uint32_t barrier_target(uint32_t call, int b) { return call * 4u + (uint32_t)b; }

// Grid barrier over the participating workgroups (the simulator stays out).
__device__ __forceinline__ bool fused_barrier(const FusedArgs &a, uint32_t want, uint32_t detail)
{
    // Arrival: each workgroup publishes its writes and then its own arrival word (release store, so
    // no two workgroups contend for one counter); workgroup 0 polls all the words, then releases
    // the target value that the others wait for.
    wait_vmem_all();   // every wave's stores of the phase have reached L2
    __syncthreads();
    __shared__ int ok_shared;
    // (every value that crosses the barrier is written through to memory or by an atomic, and every
    // wave has waited for its stores above, so the arrival needs no release write-back)
    if (threadIdx.x == 0) st_relaxed(a.bar_flag + blockIdx.x, want);
    bool ok = true;
    if (blockIdx.x == 0) {
        const int G = fused_participants(a);
        const uint64_t t0 = now_ticks();
        for (;;) {
            int here = 1;
            for (int i = threadIdx.x; i < G; i += blockDim.x) here &= ld_relaxed(a.bar_flag + i) == want;
            int bad = 0;
            if (threadIdx.x == 0) {
                if (ld_relaxed(&a.hdr->err) != 0) {
                    bad = 1;
                } else if (now_ticks() - t0 > a.spin_limit) {
                    raise_error(&a.hdr->err, kErrTimeout, detail);
                    bad = 1;
                }
            }
            if (__syncthreads_and(here)) break;   // both reductions are workgroup-uniform
            if (__syncthreads_or(bad)) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ok && threadIdx.x == 0) {
            fence_acquire_agent();
            st_relaxed(&a.hdr->bar_gen, want);
        }
        __syncthreads();
        return ok;
    }
    if (threadIdx.x == 0) ok_shared = wait_flag_eq(&a.hdr->bar_gen, want, &a.hdr->err, a.spin_limit, detail) ? 1 : 0;
    __syncthreads();
    return ok_shared != 0;
}

// The epoch of the current call (uniform), read once at the start of every workgroup.
__device__ __forceinline__ uint32_t fused_call_epoch(const FusedArgs &a)
{
    __shared__ uint32_t call_sh;
    if (threadIdx.x == 0) call_sh = ld_relaxed(&a.hdr->call_epoch);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(call_sh);
}

// Every workgroup of the grid, on every path out of the call (also after a failed wait): count itself
// out; the last one resets the count and advances the epoch.  No workgroup of this call reads the epoch
// after that, and the next call on the stream starts after this one has ended.
__device__ __forceinline__ void fused_exit(const FusedArgs &a, uint32_t call)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t n = __hip_atomic_fetch_add(&a.hdr->done_cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (n + 1u == gridDim.x) {
            __hip_atomic_store(&a.hdr->done_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.hdr->call_epoch, call + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a.status_out) {   // the acq_rel count above ordered every workgroup's error write before this
                a.status_out[0] = (int32_t)ld_relaxed(&a.hdr->err);
                a.status_out[1] = (int32_t)ld_relaxed(&a.hdr->err_detail);
                __hip_atomic_store(&a.hdr->err_detail, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.hdr->err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Inclusive scan of NV values per thread over the workgroup's threads, in thread order: wave scans, then
// the waves' totals (NV ints per wave in wsum, LDS).  tot gets the workgroup's totals.  Every thread of
// the workgroup calls it (it holds two barriers).
template <int NV>
__device__ __forceinline__ void block_incl_scan(int32_t (&v)[NV], int32_t (&tot)[NV], int32_t *wsum)
{
    const int lane = (int)threadIdx.x % kWave, wv = (int)threadIdx.x / kWave, nwv = (int)blockDim.x / kWave;
    for (int dl = 1; dl < kWave; dl <<= 1) {
        int32_t u[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) u[j] = __shfl_up(v[j], dl);
        if (lane >= dl)
#pragma unroll
            for (int j = 0; j < NV; ++j) v[j] += u[j];
    }
    if (lane == kWave - 1)
#pragma unroll
        for (int j = 0; j < NV; ++j) wsum[NV * wv + j] = v[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NV; ++j) tot[j] = 0;
    for (int u = 0; u < nwv; ++u) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (u == wv) v[j] += tot[j];
            tot[j] += wsum[NV * u + j];
        }
    }
    __syncthreads();   // wsum may be rewritten after this
}

// Phase 3 in one workgroup: per-block exclusive bases for every local expert
// (into LDS and, for the blocks this workgroup owns, into the workspace),
// expert offsets and tile prefix (LDS).  The nblk*E_local counts live in two
// LDS arrays of kScanHalf ints (entry i in cnt0[i] or cnt1[i - kScanHalf]);
// part: blockDim.x ints; off/toff/uoff: E_local+1 ints each.
struct ScanLds {
    int32_t *cnt0, *cnt1;
    __device__ __forceinline__ int32_t &operator[](int i) const
    {
        return i < kScanHalf ? cnt0[i] : cnt1[i - kScanHalf];
    }
};

__device__ __forceinline__ void fused_scan(const FusedArgs &a, const ScanLds &cnt, int32_t *part, int32_t *off, int32_t *toff,
                           int32_t *uoff, bool from_masks)
{
    const int n = a.nblk * a.E_local;
    // kScanBatch loads in flight per thread before the first LDS write (through the generic LDS
    // pointers the compiler would otherwise wait for each load before the next one).
    constexpr int kScanBatch = 16;
    const int nt = (int)blockDim.x;
    for (int i0 = threadIdx.x; i0 < n; i0 += kScanBatch * nt) {
        int32_t v[kScanBatch];
        if (from_masks) {
            uint64_t m[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) m[j] = i0 + j * nt < n ? a.ca.blkmask[i0 + j * nt] : 0ull;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) v[j] = __popcll(m[j]);
        } else {
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) v[j] = i0 + j * nt < n ? a.ca.blkcnt[i0 + j * nt] : 0;
        }
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
            if (i0 + j * nt < n) cnt[i0 + j * nt] = v[j];
    }
    __syncthreads();
    // Thread (e, p): blocks [p*L, (p+1)*L) of expert column e (EC columns per pass).  The sums of the
    // P chunks of a column are prefixed by Hillis-Steele rounds in LDS (log2 P barriers, not P - 1
    // reads in a row).
    const int P = a.E_local >= (int)blockDim.x ? 1 : (int)blockDim.x / a.E_local;
    const int L = (a.nblk + P - 1) / P;
    const int EC = (int)blockDim.x / P;
    for (int base_e = 0; base_e < a.E_local; base_e += EC) {
        const int col = (int)threadIdx.x % EC;
        const int e = base_e + col;
        const int p = (int)threadIdx.x / EC;
        const bool mine = e < a.E_local && p < P;
        int32_t s = 0;
        if (mine)
            for (int b = p * L; b < min(a.nblk, (p + 1) * L); ++b) s += cnt[b * a.E_local + e];
        __syncthreads();   // the previous pass is done with part
        if (mine) part[p * EC + col] = s;
        __syncthreads();
        int32_t incl = s;   // sum of chunks 0 .. p of the column
        for (int dl = 1; dl < P; dl <<= 1) {
            const int32_t add = mine && p >= dl ? part[(p - dl) * EC + col] : 0;
            __syncthreads();
            incl += add;
            if (mine) part[p * EC + col] = incl;
            __syncthreads();
        }
        if (mine) {
            int32_t run = incl - s;
            for (int b = p * L; b < min(a.nblk, (p + 1) * L); ++b) {
                const int32_t c = cnt[b * a.E_local + e];
                cnt[b * a.E_local + e] = run;   // now the exclusive base of block b
                run += c;
            }
            if (p == P - 1) off[e + 1] = run;   // expert total (prefixed below)
        }
        __syncthreads();
    }
    // Expert offsets and the prefixes of row tiles and mover units (kMoveRows rows each) from the totals
    // in off[1 .. E_local], a pass per blockDim experts (part, done with, holds the waves' totals).
    int32_t carry[3] = {0, 0, 0};
    for (int e0 = 0; e0 < a.E_local; e0 += blockDim.x) {
        const int e = e0 + (int)threadIdx.x;
        const int32_t c = e < a.E_local ? off[e + 1] : 0;
        int32_t v[3] = {c, (c + a.bm - 1) / a.bm, (c + kMoveRows - 1) / kMoveRows}, tot[3];
        block_incl_scan<3>(v, tot, part);
        if (e < a.E_local) {
            off[e + 1] = carry[0] + v[0];
            toff[e + 1] = carry[1] + v[1];
            uoff[e + 1] = carry[2] + v[2];
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) carry[j] += tot[j];
    }
    if (threadIdx.x == 0) {
        off[0] = 0;
        toff[0] = 0;
        uoff[0] = 0;
    }
    __syncthreads();
}

// Rows [row0, row0 + nrows) of the expert buffer from their tokens (tok_lds,
// -1 = skip), NR rows per wave at a time with all their loads in flight.
template <int CPL, int NR>
__device__ __forceinline__ void move_rows(const FusedArgs &a, const int32_t *tok_lds, int row0, int nrows, int wave,
                                          int lane)
{
    const int cpr = a.d / 8;
    for (int r0 = wave * NR; r0 < nrows; r0 += (int)(blockDim.x / kWave) * NR) {
        const uint16_t *src[NR];
        uint16_t *dst[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = r0 + i;
            const int t = r < nrows ? tok_lds[r] : -1;
            src[i] = t >= 0 ? token_row(a.src, t, a.d) : nullptr;
            dst[i] = t >= 0 ? a.x_perm + (size_t)(row0 + r) * a.d : nullptr;
        }
        if (!src[0]) {   // keep a valid address in slot 0 for the clamped loads
#pragma unroll
            for (int i = 1; i < NR; ++i)
                if (src[i]) src[0] = src[i];
        }
        if (src[0]) copy_rows_wave<CPL, NR>(src, dst, cpr, lane);
    }
}

// One mover unit: ranks [q0, q1) (q1 - q0 <= kMoveRows) of local expert le,
// i.e. expert-buffer rows off[le] + q0 .. off[le] + q1 - 1.  The unit finds
// its own tokens: block b holds the expert's ranks [base_b, base_{b+1}) (bases
// from the scan, in LDS), in the token order of the set bits of the block's
// mask for the expert.  Then it waits for the arrival flags of the rows'
// source chunks (when rows come from peers) and copies the rows, one per wave
// at a time.
__device__ __forceinline__ bool fused_move_unit(const FusedArgs &a, const ScanLds &base, const int32_t *off, int le,
                                                int q0, int q1, int32_t *tok_lds)
{
    const int n_e = off[le + 1] - off[le];
    // blocks [b_lo, b_hi) hold ranks [q0, q1): b_lo is the last block with base <= q0,
    // b_hi the first block with base >= q1
    int lo = 0, hi = a.nblk;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (base[mid * a.E_local + le] <= q0) lo = mid; else hi = mid;
    }
    const int b_lo = lo;
    lo = b_lo;
    hi = a.nblk;
    while (hi - lo > 1) {   // last block with base < q1
        const int mid = (lo + hi) >> 1;
        if (base[mid * a.E_local + le] < q1) lo = mid; else hi = mid;
    }
    const int b_hi = lo + 1;
    if ((int)threadIdx.x < kMoveRows) tok_lds[threadIdx.x] = -1;   // a rank not found stays -1 and is skipped
    __syncthreads();
    for (int b = b_lo + (int)threadIdx.x; b < b_hi; b += blockDim.x) {
        uint64_t m = a.ca.blkmask[(size_t)b * a.E_local + le];
        int q = base[b * a.E_local + le];
        const int q_end = b + 1 < a.nblk ? base[(b + 1) * a.E_local + le] : n_e;
        while (m && q < q1) {
            const int bit = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            if (q >= q0 && q < q_end) tok_lds[q - q0] = b * kTokBlock + bit;
            ++q;
        }
    }
    __syncthreads();
    const int nrows = q1 - q0;
    __shared__ int ok_sh;
    if (threadIdx.x < kWave) {
        // Rows from peers: lane i checks the ready flag of row i's source chunk, all lanes at once
        // (one load latency for the unit); while some are not ready, lane 0 waits for the first of them
        // and the lanes check again.
        int ok = 1;
        static_assert(kMoveRows <= kWave, "one lane per row of a unit");
        if (a.fl.chunk_rows > 0) {
            const int i = threadIdx.x;
            int c = -1;
            if (i < nrows && tok_lds[i] >= 0) {
                const int t = tok_lds[i];
                const int sh = t / a.src.rows_per_src;
                c = sh * a.fl.chunks_per_src + (t - sh * a.src.rows_per_src) / a.fl.chunk_rows;
            }
            for (;;) {
                const bool pending = c >= 0 && ld_relaxed(a.fl.ready + c) != a.fl.epoch;
                const uint64_t pend = __ballot(pending);
                if (pend == 0ull) break;
                const int cw = __shfl(c, __ffsll((unsigned long long)pend) - 1);
                int r = 1;
                if (i == 0) r = wait_flag_eq(a.fl.ready + cw, a.fl.epoch, &a.hdr->err, a.spin_limit,
                                             0x20000000u | (uint32_t)cw) ? 1 : 0;
                if (!__shfl(r, 0)) {
                    ok = 0;
                    break;
                }
            }
            fence_acquire_agent();   // the rows' payload is read after the flags
        }
        if (threadIdx.x == 0) ok_sh = ok;
    }
    __syncthreads();
    if (!ok_sh) return false;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int cpr = a.d / 8;
    // 64 registers of row data in flight per lane (eight waves per workgroup, two per SIMD: the GEMM's
    // 128 accumulators leave 128 registers for the rest)
    if (cpr <= 4 * kWave) move_rows<4, 4>(a, tok_lds, off[le] + q0, nrows, wave, lane);
    else if (cpr <= 8 * kWave) move_rows<8, 2>(a, tok_lds, off[le] + q0, nrows, wave, lane);
    else if (cpr <= 16 * kWave) move_rows<16, 1>(a, tok_lds, off[le] + q0, nrows, wave, lane);
    else
        for (int r = wave; r < nrows; r += (int)blockDim.x / kWave) {
            const int t = tok_lds[r];
            if (t >= 0) copy_row(token_row(a.src, t, a.d), a.x_perm + (size_t)(off[le] + q0 + r) * a.d, a.d, lane);
        }
    wait_vmem_all();   // this wave's stores have reached L2 before the release below
    return true;
}

// The arrival simulator: releases chunk c at start + delay[c] microseconds, copying the chunk's
// payload into the source buffer first if one is given.  Its state lives in LDS (the workgroup's
// stage arrays, which it has no other use for): every chunk's delay and a released bit.  Each round
// the workgroup collects the chunks that are due, copies their payloads together, then releases
// them with one release fence and a flag store each, so a round costs about one LDS pass and no
// round trip to memory per chunk.  Chunks that already hold the epoch count as released.
constexpr int kSimMaxChunks = 16384;   // chunks the simulator can hold (S * chunks_per_src)
constexpr int kSimList = 256;          // chunks released per round at most

__device__ __forceinline__ void fused_arrival_sim(const FusedArgs &a, char *lds)
{
    const int n_chunks = a.src.S * a.fl.chunks_per_src;   // <= kSimMaxChunks (checked by the host)
    uint32_t *delay = (uint32_t *)lds;                    // [kSimMaxChunks] microseconds
    uint32_t *done = delay + kSimMaxChunks;               // [kSimMaxChunks / 32] released bits
    int32_t *list = (int32_t *)(done + kSimMaxChunks / 32);   // [kSimList] due this round
    __shared__ int n_due_sh, left_sh;
    __shared__ uint64_t t0_sh;
    if (threadIdx.x == 0) {
        t0_sh = now_ticks();
        left_sh = n_chunks;
    }
    for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) delay[c] = a.fl.sim_delay_us[c];
    for (int i = threadIdx.x; i < (n_chunks + 31) / 32; i += blockDim.x) done[i] = 0u;
    __syncthreads();
    for (int c = threadIdx.x; c < n_chunks; c += blockDim.x)
        if (ld_relaxed(a.fl.ready + c) == a.fl.epoch) {
            atomicOr(done + c / 32, 1u << (c % 32));
            atomicSub(&left_sh, 1);
        }
    __syncthreads();
    const uint64_t t0 = t0_sh;
    while (left_sh > 0) {   // uniform: read after a barrier
        // past the wait bound every chunk is due (the readers' own bounds report the delay)
        const uint64_t el = now_ticks() - t0;
        const bool late = el >= a.spin_limit;
        const uint64_t now_us = el / a.ticks_per_us;
        if (threadIdx.x == 0) n_due_sh = 0;
        __syncthreads();
        for (int c = threadIdx.x; c < n_chunks; c += blockDim.x)
            if (!((done[c / 32] >> (c % 32)) & 1u) && (late || delay[c] <= now_us)) {
                const int i = atomicAdd(&n_due_sh, 1);
                if (i < kSimList) list[i] = c;
            }
        __syncthreads();
        const int n = min(n_due_sh, kSimList);
        if (n == 0) {
            __builtin_amdgcn_s_sleep(2);
        } else {
            if (a.fl.has_payload) {
                for (int i = 0; i < n; ++i) {
                    const int c = list[i];
                    const int sh = c / a.fl.chunks_per_src;
                    const int r0 = (c % a.fl.chunks_per_src) * a.fl.chunk_rows;
                    const int r1 = min(a.src.rows_per_src, r0 + a.fl.chunk_rows);
                    const uint4 *src = (const uint4 *)(a.fl.sim_payload[sh] + (size_t)r0 * a.d);
                    uint4 *dst = (uint4 *)(a.src.p[sh] + (size_t)r0 * a.d);
                    const int n16 = (r1 - r0) * a.d / 8;
                    for (int q = threadIdx.x; q < n16; q += blockDim.x) dst[q] = src[q];
                }
                wait_vmem_all();   // every wave's copies have reached L2 before the release below
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                for (int i = 0; i < n; ++i)
                    __hip_atomic_store(a.fl.ready + list[i], a.fl.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                left_sh -= n;
            }
            for (int i = threadIdx.x; i < n; i += blockDim.x) atomicOr(done + list[i] / 32, 1u << (list[i] % 32));
        }
        __syncthreads();
    }
}

// The simulator's way into the GEMM role (in-place path): wait until barrier C of this call has passed
// (the expert and tile offsets and row_token are then in memory), then load the offsets into LDS.
__device__ __forceinline__ bool fused_join_layout(const FusedArgs &a, uint32_t call, int32_t *off, int32_t *toff)
{
    __shared__ int ok_sh;
    if (threadIdx.x == 0)
        ok_sh = wait_flag_eq(&a.hdr->bar_gen, barrier_target(call, 3), &a.hdr->err, 2 * a.spin_limit,
                             0x08000000u) ? 1 : 0;
    __syncthreads();
    if (!ok_sh) return false;
    for (int e = threadIdx.x; e <= a.E_local; e += blockDim.x) {
        off[e] = a.offsets[e];
        toff[e] = a.tile_off[e];
    }
    __syncthreads();
    return true;
}

// st / ls: the four GEMM stage arrays (32 KiB each; ls holds their LDS-space
// addresses for the GEMM), also used by the earlier phases; off, toff, uoff:
// LDS arrays of at least E_local + 1 ints that outlive the GEMM tiles.
template <class C, bool SW, bool HALF_N = false>
__device__ __forceinline__ void fused_kernel_body(const FusedArgs &a, uint32_t call, char *const (&st)[4],
                                                  const LdsStages &ls, int32_t *off, int32_t *toff, int32_t *uoff,
                                                  uint16_t *basetab)
{
    const int w = blockIdx.x;
    if (w < kTraceWGs && (int)threadIdx.x < kTraceWords) a.trace[w * kTraceWords + threadIdx.x] = 0;   // this call's record only
    __syncthreads();
    trace_put(a, kTrStart, now_ticks());
    trace_put(a, kTrXcc, (uint64_t)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & 0xF));
    const int G = fused_participants(a);
    GemmArgs g = a.ga;
    bool run_phases = true;
    if (a.has_sim && w == (int)gridDim.x - 1) {
        fused_arrival_sim(a, st[0]);   // the stage arrays are consecutive: 128 KiB
        // In the in-place path the simulator then joins the GEMM role, once barrier C has published the
        // layout and the slot -> token map (taken whenever rows are simulated).
        if (!a.gather || !fused_join_layout(a, call, off, toff)) {
            trace_put(a, kTrDone, now_ticks());
            return;
        }
        run_phases = false;
    }
    if (run_phases) {
    // Counters and masks that other workgroups update with atomics: cleared through to memory.
    // (each XCD's counter starts past the tasks its own workgroups take first, without an atomic)
    if (w == 0 && threadIdx.x < 8) store_through(a.xcd_next + threadIdx.x, (uint32_t)((G - (int)threadIdx.x + 7) / 8));
    for (int i = w * (int)blockDim.x + threadIdx.x; i < a.max_tiles; i += G * (int)blockDim.x)
        store_through(a.tile_cnt + i, 0u);

    // The token-per-wave selection builds the block masks with atomic ORs:
    // clear them before barrier A.
    const bool wave_topk = !a.ids_in;
    if (wave_topk)
        for (int i = w * (int)blockDim.x + threadIdx.x; i < a.nblk * a.E_local; i += G * (int)blockDim.x)
            store_through(a.ca.blkmask + i, 0ull);

    // ---- phase 1: router logits
    if (!a.ids_in) {
        const int tasks = router_tasks(a.T, a.E);
        const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
        // At most four tasks per workgroup: one per SIMD (waves 0..3), staging chunks of kRtKC steps (a
        // task's time is mostly the load latency of its chunks).  More: every wave, consecutive tasks per
        // workgroup (they share token rows), chunks of kRtKCFused steps so that eight waves' staging fits.
        static_assert(4 * RtStage<kRtKC>::LDS_PER_WAVE <= 4 * 32768, "router staging fits the stage arrays");
        static_assert(C::NW * RtStage<kRtKCFused>::LDS_PER_WAVE <= 4 * 32768, "router staging fits");
        if (tasks <= 4 * G) {
            if (wave < 4 && w * 4 + wave < tasks)
                router_task<kRtKC>(a.ra, w * 4 + wave, (lds_byte_t *)ls.p[0] + wave * RtStage<kRtKC>::LDS_PER_WAVE);
        } else if (a.E >= 4 * kRtExp) {   // four expert groups per task: four chains per lane
            // (skewed-shaped, 64 experts: routing 43 -> 36 us against two groups per task)
            static_assert(C::NW * RtStage<kRtKCPair, 4>::LDS_PER_WAVE <= 4 * 32768, "router staging fits");
            const int tasks4 = router_tasks(a.T, a.E, 4);
            lds_byte_t *rlds = (lds_byte_t *)ls.p[0] + wave * RtStage<kRtKCPair, 4>::LDS_PER_WAVE;
            for (int q = w * C::NW + wave; q < tasks4; q += G * C::NW) router_task<kRtKCPair, 4>(a.ra, q, rlds);
        } else if (a.E >= 2 * kRtExp) {   // two expert groups per task: two chains per lane
            static_assert(C::NW * RtStage<kRtKCPair, 2>::LDS_PER_WAVE <= 4 * 32768, "router staging fits");
            const int tasks2 = router_tasks(a.T, a.E, 2);
            lds_byte_t *rlds = (lds_byte_t *)ls.p[0] + wave * RtStage<kRtKCPair, 2>::LDS_PER_WAVE;
            for (int q = w * C::NW + wave; q < tasks2; q += G * C::NW) router_task<kRtKCPair, 2>(a.ra, q, rlds);
        } else {
            lds_byte_t *rlds = (lds_byte_t *)ls.p[0] + wave * RtStage<kRtKCFused>::LDS_PER_WAVE;
            for (int q = w * C::NW + wave; q < tasks; q += G * C::NW) router_task<kRtKCFused>(a.ra, q, rlds);
        }
        trace_put(a, kTrRouted, now_ticks());
        if (!fused_barrier(a, barrier_target(call, 1), 0x01000000u)) return;
        trace_put(a, kTrBarA, now_ticks());
    }
    // ---- phase 2: top-k, histogram and ranks.  Routing inside: the selection
    // runs token-parallel over every workgroup (one token per wave) and ORs
    // each token into its block's mask of every local expert it chose; after
    // the barrier the masks give the counts and ranks.  Given ids: per 64-token
    // block, copy and histogram in one workgroup.
    if (wave_topk) {
        topk_wave_loop(a.ta, w, G);
        trace_put(a, kTrSelected, now_ticks());
        trace_put(a, kTrCounted, now_ticks());
        if (!fused_barrier(a, barrier_target(call, 2), 0x04000000u)) return;
        trace_put(a, kTrBarB, now_ticks());
    } else {
        int32_t *ids_lds = (int32_t *)st[1];                          // 8 KiB
        int32_t *cnt_lds = (int32_t *)(st[1] + kTokBlock * kMaxK * 4);  // E_local ints (<= 4 KiB)
        uint64_t *mask_lds = (uint64_t *)(st[1] + 16384);               // E_local uint64 (<= 8 KiB)
        for (int blk = w; blk < a.nblk; blk += G) {
            const int base_t = blk * kTokBlock;
            const int n_t = min(kTokBlock, a.T - base_t);
            for (int i = threadIdx.x; i < n_t * a.k; i += blockDim.x) {
                const size_t o = (size_t)base_t * a.k + i;
                const int32_t id = a.ids_in[o];
                ids_lds[i] = id;
                store_through(a.ta.ids + o, id);
                if (a.ids_user) a.ids_user[o] = id;
            }
            __syncthreads();
            count_block(a.ca, blk, ids_lds, cnt_lds, mask_lds);
        }
        trace_put(a, kTrCounted, now_ticks());
        if (!fused_barrier(a, barrier_target(call, 2), 0x02000000u)) return;
        trace_put(a, kTrBarB, now_ticks());
    }

    // ---- phase 3: scan (every workgroup), slot map of own blocks.  The movers
    // need no barrier after it: they find the tokens of their rows from the
    // block masks and the bases, which every workgroup holds in LDS.
    const ScanLds cnt{(int32_t *)st[0], (int32_t *)st[1]};   // nblk * E_local (<= 64 KiB)
    int32_t *part = (int32_t *)st[2];                         // blockDim.x ints
    fused_scan(a, cnt, part, off, toff, uoff, wave_topk);
    if (w == 0) {
        for (int e = threadIdx.x; e <= a.E_local; e += blockDim.x) {
            store_through(a.offsets + e, off[e]);
            store_through(a.tile_off + e, toff[e]);
        }
        if (threadIdx.x == 0) {
            store_through(&a.hdr->R, (uint32_t)off[a.E_local]);
            store_through(&a.hdr->n_tiles, (uint32_t)toff[a.E_local]);
        }
    }
    for (int blk = w; blk < a.nblk; blk += G) {
        for (int i = threadIdx.x; i < kTokBlock * a.k; i += blockDim.x) {
            const int t = blk * kTokBlock + i / a.k;
            if (t >= a.T) break;
            const size_t o = (size_t)t * a.k + (i % a.k);
            const int le = a.ta.ids[o] - a.e_begin;
            const bool local = le >= 0 && le < a.E_local;
            int32_t rank = -1;
            if (!wave_topk) rank = a.ca.lrank[o];
            else if (local)   // tokens before t in the block with the same expert
                rank = __popcll(a.ca.blkmask[(size_t)blk * a.E_local + le] & ((1ull << (t % kTokBlock)) - 1ull));
            int32_t slot = -1;
            if (local && rank >= 0) {
                slot = off[le] + cnt[blk * a.E_local + le] + rank;
                if (slot < off[le + 1]) {
                    store_through(a.row_token_ws + slot, t);
                    if (a.row_token_user) a.row_token_user[slot] = t;
                } else {
                    slot = -1;
                }
            }
            a.slot_of[o] = slot;
        }
    }
    trace_put(a, kTrSlots, now_ticks());
    // The GEMM's row tokens: with a small block table each workgroup keeps the per-block bases it
    // scanned (the stage arrays that hold them now are reused by the GEMM) and finds the tokens of its
    // tiles from them and the block masks; otherwise it reads row_token after a barrier that publishes
    // every workgroup's slots.
    if (a.gather) {
        const int nb = a.nblk * a.E_local;
        if (nb <= kBaseTab && a.T < 65536 && !a.has_sim) {
            for (int i = threadIdx.x; i < nb; i += blockDim.x) basetab[i] = (uint16_t)cnt[i];
            __syncthreads();
            g.tok_mask = a.ca.blkmask;
            g.tok_base = basetab;
            g.tok_off = off;
            g.tok_nblk = a.nblk;
        } else {
            if (!fused_barrier(a, barrier_target(call, 3), 0x08000000u)) return;
            trace_put(a, kTrBarC, now_ticks());
        }
    }

    // ---- movers: unit u = kMoveRows ranks of one expert (tile-major, since bm % kMoveRows == 0),
    // dealt round-robin over the movers
    uint64_t n_units = 0, copy_ticks = 0, release_ticks = 0;
    if (!a.gather && w < a.n_mover) {
        int32_t *tok_lds = (int32_t *)st[2] + 1024;   // kMoveRows ints after the scan's partials
        const int n_units_all = uoff[a.E_local];
        // The arrival counter of unit u's tile.
        auto unit_tile = [&](int u, int &e, int &q0, int &q1) {
            int lo = 0, hi = a.E_local;   // expert e with uoff[e] <= u < uoff[e+1]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (uoff[mid] <= u) lo = mid; else hi = mid;
            }
            e = lo;
            q0 = (u - uoff[e]) * kMoveRows;
            q1 = min(off[e + 1] - off[e], q0 + kMoveRows);
            return a.tile_cnt + toff[e] + q0 / a.bm;
        };
        // Rows resident: one release after all of this workgroup's units (each agent-scope release
        // writes back the XCD's L2, so one per unit serialises the movers), then relaxed counter
        // bumps.  Rows from peers: a release per unit, so tiles start as their chunks arrive.
        const bool batch = a.fl.chunk_rows == 0;
        for (int u = w; u < n_units_all; u += a.n_mover) {
            int e, q0, q1;
            uint32_t *ctr = unit_tile(u, e, q0, q1);
            const uint64_t c0 = now_ticks();
            const bool ok = fused_move_unit(a, cnt, off, e, q0, q1, tok_lds);
            __syncthreads();
            if (!ok) return;
            const uint64_t c1 = now_ticks();
            if (!batch && threadIdx.x == 0)
                __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            copy_ticks += c1 - c0;
            release_ticks += now_ticks() - c1;
            ++n_units;
        }
        if (batch && n_units > 0 && threadIdx.x == 0) {   // every wave's stores reached L2 (fused_move_unit)
            const uint64_t c1 = now_ticks();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            for (int u = w; u < n_units_all; u += a.n_mover) {
                int e, q0, q1;
                __hip_atomic_fetch_add(unit_tile(u, e, q0, q1), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            release_ticks += now_ticks() - c1;
        }
    }
    trace_put(a, kTrMoved, now_ticks());
    trace_put(a, kTrUnits, n_units);
    trace_put(a, kTrCopyTicks, copy_ticks);
    trace_put(a, kTrReleaseTicks, release_ticks);
    }   // run_phases
    uint64_t n_done = 0, wait_ticks = 0;

    // ---- compute: per-XCD queues over chunks of CH consecutive tasks.  A SwiGLU tile covers BN / 2
    // features (BN / 2 gate rows and the matching up rows of W).
    constexpr int BNO = SW ? C::BN / 2 : C::BN;
    const int NB = SW ? (g.F + BNO - 1) / BNO : (g.N + BNO - 1) / BNO;
    const int n_tasks = toff[a.E_local] * NB;
    const int xcd = w % 8;
    const int CH = (G + 7) / 8;
    __shared__ int q_sh;
    // The next task index, walking this XCD's queue, then the others' (-1: none left).  A participating
    // workgroup's first task is entry w / 8 of its own queue (the queue's w / 8-th workgroup); the queue
    // counters start at the number of workgroups per XCD (the arrival simulator, not among them, claims
    // through the counter).  Once a queue comes up empty the workgroup reads all eight counters at once
    // and takes entries only from queues that still hold tasks (a counter only grows, so a queue seen
    // empty stays empty): one round trip instead of an atomic on every queue in turn.
    auto entry_task = [&](int i, int x) { return (i / CH) * 8 * CH + x * CH + (i % CH); };
    int o = 0;
    bool first = w < G;
    bool polled = false;
    uint32_t live = 0xFFu;   // queues that may still hold tasks (uniform)
    __shared__ uint32_t live_sh;
    auto claim = [&]() -> int {
        // At most one task per workgroup: every task is some workgroup's first, nothing is left to take.
        if (!first && n_tasks <= G && !a.has_sim) return -1;
        for (; o < 8; ++o) {
            const int x = (xcd + o) % 8;
            if (!((live >> x) & 1u)) continue;
            if (threadIdx.x == 0) {
                const int i = first ? w / 8
                                    : (int)__hip_atomic_fetch_add(a.xcd_next + x, 1u, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT);
                q_sh = entry_task(i, x);
            }
            first = false;
            __syncthreads();
            const int q = __builtin_amdgcn_readfirstlane(q_sh);   // uniform: keeps the tile loop scalar
            __syncthreads();
            if (q < n_tasks) return q;
            if (!polled) {
                polled = true;
                if (threadIdx.x < kWave) {   // wave 0: lane y reads queue y's counter
                    bool has = false;
                    if (threadIdx.x < 8)
                        has = entry_task((int)ld_relaxed(a.xcd_next + threadIdx.x), (int)threadIdx.x) < n_tasks;
                    const uint64_t b = __ballot(has);
                    if (threadIdx.x == 0) live_sh = (uint32_t)b;
                }
                __syncthreads();
                live = __builtin_amdgcn_readfirstlane(live_sh);
                __syncthreads();
            }
        }
        return -1;
    };
    // Task q -> expert, column block, row tile (consecutive tasks share a W tile).
    // With tails_last every expert's row tiles but a short last one (at most kShortTile rows) come
    // first, the short last tiles after them: fpre[e] = the other tiles of the experts before e (in
    // uoff, which the movers are done with); the short tiles before e are then toff[e] - fpre[e].
    int32_t *fpre = uoff;
    if (a.tails_last) {
        int32_t *wsum = (int32_t *)st[2];   // the scan's partials, done with
        int32_t carry = 0;
        __syncthreads();   // this workgroup is done with uoff (the movers' unit prefix)
        for (int e0 = 0; e0 < a.E_local; e0 += blockDim.x) {
            const int e = e0 + (int)threadIdx.x;
            const int c = e < a.E_local ? off[e + 1] - off[e] : 0;
            int32_t v[1] = {c / C::BM + (c % C::BM > kShortTile ? 1 : 0)}, tot[1];
            const int32_t mine = v[0];
            block_incl_scan<1>(v, tot, wsum);
            if (e < a.E_local) fpre[e] = carry + v[0] - mine;
            carry += tot[0];
        }
        if (threadIdx.x == 0) fpre[a.E_local] = carry;
        __syncthreads();
    }
    auto job_of = [&](int q) -> TileJob {
        TileJob t{0, 0, 0, 0, 0};
        if (q < 0) return t;
        int e, row0, rows, nb;
        if (!a.tails_last) {
            int lo = 0, hi = a.E_local;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (toff[mid] * NB <= q) lo = mid; else hi = mid;
            }
            const int nt = toff[lo + 1] - toff[lo];
            const int rem = q - toff[lo] * NB;
            const int mt = rem % nt;
            e = lo;
            row0 = off[lo] + mt * C::BM;
            rows = min(C::BM, off[lo + 1] - off[lo] - mt * C::BM);
            nb = rem / nt;
        } else if (q < fpre[a.E_local] * NB) {   // a full tile
            int lo = 0, hi = a.E_local;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (fpre[mid] * NB <= q) lo = mid; else hi = mid;
            }
            const int nf = fpre[lo + 1] - fpre[lo];
            const int rem = q - fpre[lo] * NB;
            e = lo;
            row0 = off[lo] + (rem % nf) * C::BM;
            rows = min(C::BM, off[lo + 1] - row0);
            nb = rem / nf;
        } else {                                  // a tail: one per expert that has one
            const int q2 = q - fpre[a.E_local] * NB;
            int lo = 0, hi = a.E_local;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((toff[mid] - fpre[mid]) * NB <= q2) lo = mid; else hi = mid;
            }
            const int nf = fpre[lo + 1] - fpre[lo];
            e = lo;
            row0 = off[lo] + nf * C::BM;
            rows = off[lo + 1] - row0;
            nb = q2 - (toff[lo] - fpre[lo]) * NB;
        }
        t.e = __builtin_amdgcn_readfirstlane(e);
        t.row0 = __builtin_amdgcn_readfirstlane(row0);
        t.rows_valid = __builtin_amdgcn_readfirstlane(rows);
        t.n0 = __builtin_amdgcn_readfirstlane(nb * BNO);
        t.w_once = __builtin_amdgcn_readfirstlane(off[e + 1] - off[e] <= 64 ? 1 : 0);
        return t;
    };
    // Row tile t's arrival counter and the count of moved units that completes it.
    auto tile_counter = [&](const TileJob &t) { return a.tile_cnt + toff[t.e] + (t.row0 - off[t.e]) / C::BM; };
    auto tile_units = [&](const TileJob &t) { return (uint32_t)((t.rows_valid + kMoveRows - 1) / kMoveRows); };
    // Blocking: wait until all rows of t are moved, or, rows read in place from peers, until their
    // chunks have arrived (false: give up, the error word is set).
    auto wait = [&](const TileJob &t) -> bool {
        if (n_done == 0) trace_put(a, kTrFirstTask, now_ticks());
        if (a.gather && a.fl.chunk_rows == 0) return true;   // rows read in place, all resident
        const uint64_t tw0 = now_ticks();
        int ok;
        if (a.gather) {
            // thread i waits for the ready flag of the source chunk of the tile's row i
            int fail = 0;
            const int i = threadIdx.x;
            if (i < t.rows_valid) {
                const int tok = g.tok_base ? token_of_rank(g, t.e, t.row0 - off[t.e] + i) : g.row_token[t.row0 + i];
                const int sh = tok / a.src.rows_per_src;
                const int c = sh * a.fl.chunks_per_src + (tok - sh * a.src.rows_per_src) / a.fl.chunk_rows;
                fail = wait_flag_eq(a.fl.ready + c, a.fl.epoch, &a.hdr->err, a.spin_limit,
                                    0x20000000u | (uint32_t)c) ? 0 : 1;
            }
            ok = __syncthreads_or(fail) ? 0 : 1;
        } else {
            if (threadIdx.x == 0)
                // twice the movers' bound: a withheld arrival is reported as itself, not as this wait
                q_sh = wait_flag_geq(tile_counter(t), tile_units(t), &a.hdr->err, 2 * a.spin_limit,
                                     0x10000000u | (uint32_t)(tile_counter(t) - a.tile_cnt)) ? 1 : 0;
            __syncthreads();
            ok = __builtin_amdgcn_readfirstlane(q_sh);
            __syncthreads();
        }
        wait_ticks += now_ticks() - tw0;
        return ok != 0;
    };
    auto claim_job = [&]() { return job_of(claim()); };
    auto done = [&]() { ++n_done; };
    LambdaSched<decltype(claim_job), decltype(wait), decltype(done)> sc{claim_job, wait, done};
    gemm_run<C::NW, SW, HALF_N>(g, sc, ls);
    trace_put(a, kTrDone, now_ticks());
    trace_put(a, kTrTasks, n_done);
    trace_put(a, kTrWaitTicks, wait_ticks);
}

}  // namespace mk
