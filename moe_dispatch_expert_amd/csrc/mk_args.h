// mk_args.h -- plain structs passed by value from the host launcher to the
// kernels, and the layout of the dispatch workspace.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mk {

constexpr int kMaxSources = 64;     // source shards a call may name
constexpr int kGatherSources = 8;   // sources the GEMM can read rows from in place
// A buffer offset past every resource the kernels build (their sizes stay below it): loads read 0
// without a memory access.
constexpr uint32_t kPastResource = 0xFFFFFF00u;
constexpr int kRouterSegments = 8;  // contiguous K segments of the router dot product
constexpr int kMaxK = 32;           // experts per token this build handles
constexpr int kTokBlock = 64;       // tokens per counting block (one wave, lane = token)
constexpr int kMinBM = 16;          // smallest GEMM tile height any kernel uses

// Token t lives in shard t / rows_per_src at row t % rows_per_src.
struct SrcRows {
    const uint16_t *p[kMaxSources];
    int32_t S;
    int32_t rows_per_src;
};

// Arrival flags of the source chunks (chunk_rows == 0: rows resident).
struct SrcFlags {
    uint32_t *ready;              // [S * chunks_per_src]
    const uint32_t *sim_delay_us; // NULL: flags are released by someone else
    const uint16_t *sim_payload[kMaxSources];
    int32_t has_payload;
    int32_t chunk_rows;
    int32_t chunks_per_src;
    uint32_t epoch;
};

// First 256 bytes of the dispatch workspace.
struct WsHeader {
    uint32_t err;          // 0 or an mk_status code
    uint32_t err_detail;
    uint32_t done_cnt;     // fused kernel: workgroups that have left the current call (0 between calls)
    uint32_t bar_gen;      // grid barrier: the last target value released by workgroup 0
    uint32_t n_tiles;      // GEMM row tiles of the current call
    uint32_t R;            // routed local rows of the current call
    uint32_t call_epoch;   // fused kernel: calls completed through this workspace (barrier targets derive from it)
    uint32_t xcd_next[8];  // fused kernel: per-XCD GEMM task counters
    uint32_t pad[49];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// Byte offsets of the workspace segments (all 256-byte aligned).
constexpr int kTraceWGs = 1024;   // workgroups the trace segment has room for
constexpr int kTraceWords = 32;   // uint64 records per workgroup
constexpr int kBarrierWGs = 1024; // workgroups the grid barrier's arrival words have room for

struct WsLayout {
    size_t hdr, bar_flag, part, ids, lrank, blkcnt, blkbase, blkmask, tile_off, tile_flag, row_token, trace, x_perm, total;
    int32_t nblk, max_tiles, r_cap, x_perm_rows;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// with_x_perm: the call copies rows into the expert-contiguous row buffer (mover role or staged path);
// the gather path reads rows in place and needs no such buffer.
inline WsLayout ws_layout(int32_t T, int32_t d, int32_t E, int32_t k, int32_t E_local, bool with_x_perm)
{
    WsLayout L{};
    L.nblk = (T + kTokBlock - 1) / kTokBlock;
    L.r_cap = T * (k < E_local ? k : E_local);
    L.max_tiles = L.r_cap / kMinBM + E_local + 1;
    L.x_perm_rows = with_x_perm ? L.r_cap + 256 : 0;   // a full tile past the last row stays in bounds
    size_t o = 0;
    L.hdr = o;       o += align256(sizeof(WsHeader));
    L.bar_flag = o;  o += align256((size_t)kBarrierWGs * 4);
    L.part = o;      o += align256((size_t)kRouterSegments * T * E * 4);
    L.ids = o;       o += align256((size_t)T * k * 4);
    L.lrank = o;     o += align256((size_t)T * k * 4);
    L.blkcnt = o;    o += align256((size_t)L.nblk * E_local * 4);
    L.blkbase = o;   o += align256((size_t)L.nblk * E_local * 4);
    L.blkmask = o;   o += align256((size_t)L.nblk * E_local * 8);
    L.tile_off = o;  o += align256((size_t)(E_local + 1) * 4);
    L.tile_flag = o; o += align256((size_t)L.max_tiles * 4);
    L.row_token = o; o += align256((size_t)(L.r_cap + 1) * 4);
    L.trace = o;     o += align256((size_t)kTraceWGs * kTraceWords * 8);
    L.x_perm = o;    o += align256((size_t)L.x_perm_rows * d * 2);
    L.total = o;
    return L;
}

}  // namespace mk
