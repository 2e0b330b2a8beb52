// api.cpp -- the C ABI declared in include/mk.h: argument validation,
// workspace layout, per-shape tuning and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/mk.h"
#include "fused_dev.h"
#include "gemm_dev.h"
#include "layout_dev.h"
#include "mk_args.h"
#include "mk_launch.h"
#include "route_dev.h"

static __device__ __align__(256) char scratch[MK_STATIC_SCRATCH_BYTES];

namespace {

using namespace mk;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int ticks_per_us();

// Wall-clock ticks a device-side wait may spin: MK_TIMEOUT_US (read at every
// call), default 2 s.
uint64_t spin_limit_ticks()
{
    long us = 2000000;
    if (const char *e = std::getenv("MK_TIMEOUT_US")) {
        const long v = std::strtol(e, nullptr, 10);
        if (v > 0) us = v;
    }
    return (uint64_t)us * (uint64_t)ticks_per_us();
}

mk_status check_shape(const mk_shape *s)
{
    if (!s) return MK_EINVAL;
    if (s->T < 0 || s->d <= 0 || s->E < 1 || s->k < 1 || s->k > s->E || s->e_begin < 0 || s->E_local < 1 ||
        s->e_begin + s->E_local > s->E || s->N <= 0)
        return MK_EINVAL;
    if (s->d % 8 != 0 || s->N % 8 != 0) return MK_EINVAL;
    if (s->d % 128 != 0 || s->E > 1024 || s->k > kMaxK || s->E_local > 1024) return MK_EUNSUPPORTED;
    return MK_OK;
}

mk_status check_sources(const mk_shape *s, const mk_sources *src)
{
    if (!src || src->S < 1 || src->S > kMaxSources || src->rows_per_src < 0 || !src->x) return MK_EINVAL;
    if ((long)src->S * src->rows_per_src != s->T) return MK_EINVAL;
    for (int i = 0; i < src->S; ++i)
        if (s->T > 0 && (!src->x[i] || !aligned16(src->x[i]))) return MK_EINVAL;
    if (src->chunk_rows < 0) return MK_EINVAL;
    if (src->chunk_rows > 0) {
        if (!src->chunk_ready || !aligned16(src->chunk_ready)) return MK_EINVAL;
        if (src->sim_delay_us && !aligned16(src->sim_delay_us)) return MK_EINVAL;
        // the simulator holds every chunk's delay in LDS
        const long n_chunks = (long)src->S * ((src->rows_per_src + src->chunk_rows - 1) / src->chunk_rows);
        if (src->sim_delay_us && n_chunks > kSimMaxChunks) return MK_EUNSUPPORTED;
        if (src->sim_payload) {
            if (!src->sim_delay_us) return MK_EINVAL;
            for (int i = 0; i < src->S; ++i)
                if (!src->sim_payload[i] || !aligned16(src->sim_payload[i])) return MK_EINVAL;
        }
    }
    return MK_OK;
}

SrcRows make_src_rows(const mk_sources *src)
{
    SrcRows r{};
    for (int i = 0; i < src->S; ++i) r.p[i] = (const uint16_t *)src->x[i];
    r.S = src->S;
    r.rows_per_src = src->rows_per_src > 0 ? src->rows_per_src : 1;
    return r;
}

int ticks_per_us()
{
    static int v = 0;
    if (v == 0) {
        int dev = 0, khz = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz >= 1000)
            v = khz / 1000;
        else
            v = 100;
    }
    return v;
}

// Where the GEMM can read token rows in place (no mover role): at most kGatherSources sources, all
// inside one buffer resource (< 4 GiB from the lowest one).  *lo and *span receive that window.
bool gather_window(const mk_shape *s, const mk_sources *src, uintptr_t *lo = nullptr, uint64_t *span = nullptr)
{
    if (!src || src->S < 1 || src->S > kGatherSources) return false;
    const uint64_t bytes = (uint64_t)src->rows_per_src * s->d * 2;
    uintptr_t l = (uintptr_t)src->x[0], h = l + bytes;
    for (int i = 1; i < src->S; ++i) {
        l = std::min(l, (uintptr_t)src->x[i]);
        h = std::max(h, (uintptr_t)src->x[i] + (uintptr_t)bytes);
    }
    if (lo) *lo = l;
    if (span) *span = (uint64_t)(h - l);
    return (uint64_t)(h - l) <= kPastResource;
}

// The per-shape table.  Rows readable in place (gather_window): no mover role, the GEMM reads each
// tile's token rows straight from the sources through the slot -> token map (MK_MOVERS_NONE), and
// when rows arrive from peers each tile first waits for its rows' chunk flags.  (On the one-GPU share
// of a wide EP layer, 8 sources x 2048 rows, d = 7168, 32 local experts, rows arriving in 128-row
// chunks at U[0, 100] us, moving the rows first took 0.78 / 0.77 / 0.76 / 0.75 ms with 32 / 64 / 128 /
// 256 movers: every expert tile holds rows of most chunks, so no tile is complete much before the
// last arrival.)  Otherwise every co-resident workgroup starts as a mover, then computes.
bool gather_possible(const mk_shape *s, const mk_sources *src) { return gather_window(s, src); }

// GEMM tasks a uniform routing gives: each local expert ~ T k / E rows, in 256-row tiles, times the
// 256-column blocks of N.
// Compute workgroups of the in-place path: as many as those tasks, with a quarter
// more for skew, at least 32, in multiples of 8 (one per XCD); 0 (every co-resident workgroup)
// when that reaches 256.  Fewer workgroups make the grid barriers and the phases before the GEMM
// cheaper when the GEMM cannot use the whole device: T = 256, d = 512, 8 experts, top-2, N = 1024
// (32 tasks) took 0.034 ms on 32 or 64 workgroups, 0.040 on 128 and 0.060 on 256.
long uniform_tasks(const mk_shape *s)
{
    const double rows_e = (double)s->T * s->k / s->E;
    const long tiles_e = (long)((rows_e + 255.0) / 256.0);
    return (long)s->E_local * (tiles_e > 0 ? tiles_e : 1) * ((s->N + 255) / 256);
}

int table_compute_wg(const mk_shape *s)
{
    const long tasks = uniform_tasks(s);
    long g = (tasks * 5 + 3) / 4;
    g = (g + 7) / 8 * 8;
    if (g < 32) g = 32;
    return g >= 256 ? 0 : (int)g;
}

mk_tuning table_tuning(const mk_shape *s, const mk_sources *src)
{
    mk_tuning t{};
    t.bm = 256;
    t.bn = 256;
    t.bk = Tiles<4>::M256::BK;
    // Task order: rows read in place and at most three rounds of tasks on the device's 256 workgroups:
    // the experts' short last tiles go after every other tile, so that the longer tasks are spread evenly
    // first (one GPU's share of a wide EP layer, 16384 x 8 of 256 experts, 32 local, d = 7168, N = 2048:
    // two rounds plus 112 short tasks, 0.673 -> 0.645 ms).  Otherwise every expert's tiles together, each
    // short tile beside the tiles that share its W tile (Mixtral-shaped, 7 rounds, and skewed, 4.5: 1-2%
    // faster; the same share with moved rows and arrivals: 0.742 against 0.785 ms with the short tiles last).
    t.tile_order = MK_ORDER_EXPERT;
    if (gather_possible(s, src)) {
        t.n_mover_wg = MK_MOVERS_NONE;
        t.n_compute_wg = table_compute_wg(s);
        if (uniform_tasks(s) <= 3 * 256) t.tile_order = MK_ORDER_TAILS_LAST;
    } else {
        t.n_mover_wg = 256;
        t.n_compute_wg = 0;   // 0: every co-resident workgroup
    }
    return t;
}

enum class Path { kGather, kMove, kStaged };

// How one call runs: the resolved tuning, the path, and the workspace layout it needs.
struct Plan {
    mk_tuning tu;
    Path path;
    WsLayout L;
    bool table_compute;   // tu.n_compute_wg is the table's (clamped to the device), not the caller's
};

mk_status plan_call(const mk_shape *s, const mk_sources *src, const mk_tuning *tune, Plan &p)
{
    p.tu = table_tuning(s, src);
    if (tune) {
        if ((tune->bm && tune->bm != 256) || (tune->bn && tune->bn != 256) ||
            (tune->bk && tune->bk != Tiles<4>::M256::BK))
            return MK_EUNSUPPORTED;
        if (tune->n_mover_wg < MK_MOVERS_NONE || tune->n_compute_wg < 0 || tune->cooperative < 0 ||
            tune->cooperative > 1 || tune->tile_order < 0 || tune->tile_order > MK_ORDER_TAILS_LAST)
            return MK_EINVAL;
        if (tune->n_mover_wg) p.tu.n_mover_wg = tune->n_mover_wg;
        if (tune->n_compute_wg) p.tu.n_compute_wg = tune->n_compute_wg;
        p.tu.cooperative = tune->cooperative;
        if (tune->tile_order) p.tu.tile_order = tune->tile_order;
    }
    // Phase 3 of the fused kernel keeps nblk * E_local block counts in LDS.
    const WsLayout L0 = ws_layout(s->T, s->d, s->E, s->k, s->E_local, false);
    const bool fits_fused = (long)L0.nblk * s->E_local <= kMaxScanEntries;
    if (p.tu.n_mover_wg == MK_MOVERS_STAGED || s->T == 0 || !fits_fused) {
        if (src->chunk_rows > 0) return MK_EUNSUPPORTED;   // arrival flags need the fused kernel
        p.path = Path::kStaged;
    } else if (p.tu.n_mover_wg == MK_MOVERS_NONE) {
        if (!gather_possible(s, src)) return MK_EUNSUPPORTED;
        p.path = Path::kGather;
    } else {
        p.path = Path::kMove;
    }
    // the table's compute count is for the in-place path; on another path it means every workgroup
    p.table_compute = !(tune && tune->n_compute_wg);
    if (p.path != Path::kGather && p.table_compute) p.tu.n_compute_wg = 0;
    // likewise the table's task order (tails last only where rows are read in place)
    if (p.path != Path::kGather && !(tune && tune->tile_order)) p.tu.tile_order = MK_ORDER_EXPERT;
    p.L = ws_layout(s->T, s->d, s->E, s->k, s->E_local, p.path != Path::kGather);
    return MK_OK;
}

// The dispatch call; status_out (device [2], or nullptr) receives the call's device status at its end
// (no-allocation entry point), else the error words stay in the workspace for mk_poll_error.
mk_status dispatch_impl(const mk_shape *s, const mk_sources *src, const float *w_router, const float *bias,
                        const int32_t *topk_ids_in, const void *w_experts, void *y_perm, int32_t *slot_of,
                        int32_t *expert_offsets, int32_t *topk_ids_out, float *topk_w_out, int32_t *row_token,
                        void *workspace, size_t workspace_bytes, const mk_tuning *tune, void *stream,
                        int32_t *status_out, const Plan *pre_plan, bool swiglu = false)
{
    mk_status st = check_shape(s);
    if (st != MK_OK) return st;
    // SwiGLU: w_experts holds 2F = N rows per expert (F gate rows, then F up rows), y_perm is [R_cap, F]
    if (swiglu && s->N % 16 != 0) return MK_EINVAL;
    // (the SwiGLU tiles' W row offsets are 32-bit: N + 256 rows of d bf16 stay below 2 GiB)
    if (swiglu && (int64_t)(s->N + 256) * s->d * 2 >= ((int64_t)1 << 31)) return MK_EUNSUPPORTED;
    st = check_sources(s, src);
    if (st != MK_OK) return st;
    if (!w_experts || !expert_offsets || !workspace) return MK_EINVAL;
    if (s->T > 0 && (!y_perm || !slot_of)) return MK_EINVAL;   // T == 0: empty outputs may be null
    if (!topk_ids_in && !w_router) return MK_EINVAL;
    const void *ptrs[] = {w_router, bias, topk_ids_in, w_experts, y_perm, slot_of, expert_offsets,
                          topk_ids_out, topk_w_out, row_token, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return MK_EINVAL;
    Plan plan;
    if (pre_plan) {
        plan = *pre_plan;
    } else {
        st = plan_call(s, src, tune, plan);
        if (st != MK_OK) return st;
    }
    const WsLayout &L = plan.L;
    if (workspace_bytes < L.total) return MK_EWORKSPACE;
    const mk_tuning &tu = plan.tu;
    const bool staged = plan.path == Path::kStaged;
    const bool gather = plan.path == Path::kGather;
    hipEvent_t ev_begin = tune ? (hipEvent_t)tune->ev_gemm_begin : nullptr;
    hipEvent_t ev_end = tune ? (hipEvent_t)tune->ev_gemm_end : nullptr;

    hipStream_t hs = (hipStream_t)stream;
    char *ws = (char *)workspace;
    WsHeader *hdr = (WsHeader *)(ws + L.hdr);
    float *part = (float *)(ws + L.part);
    int32_t *ids = (int32_t *)(ws + L.ids);
    int32_t *lrank = (int32_t *)(ws + L.lrank);
    int32_t *blkcnt = (int32_t *)(ws + L.blkcnt);
    uint64_t *blkmask = (uint64_t *)(ws + L.blkmask);
    int32_t *blkbase = (int32_t *)(ws + L.blkbase);
    int32_t *tile_off = (int32_t *)(ws + L.tile_off);
    int32_t *row_token_ws = (int32_t *)(ws + L.row_token);
    uint16_t *x_perm = (uint16_t *)(ws + L.x_perm);
    const SrcRows rows = make_src_rows(src);

    if (!staged) {
        const int resident = fused_max_grid();
        if (resident <= 0) return MK_EHIP;
        FusedArgs fa{};
        fa.ra.src = rows;
        fa.ra.wr = w_router;
        fa.ra.part = part;
        fa.ra.T = s->T;
        fa.ra.d = s->d;
        fa.ra.E = s->E;
        fa.ta.part = part;
        fa.ta.bias = bias;
        fa.ta.ids = ids;
        fa.ta.ids_user = topk_ids_out;
        fa.ta.w_user = topk_w_out;
        fa.ta.blkmask = blkmask;
        fa.ta.T = s->T;
        fa.ta.E = s->E;
        fa.ta.k = s->k;
        fa.ta.e_begin = s->e_begin;
        fa.ta.E_local = s->E_local;
        fa.ca.ids = ids;
        fa.ca.lrank = lrank;
        fa.ca.blkcnt = blkcnt;
        fa.ca.blkmask = blkmask;
        fa.ca.err = &hdr->err;
        fa.ca.T = s->T;
        fa.ca.E = s->E;
        fa.ca.k = s->k;
        fa.ca.e_begin = s->e_begin;
        fa.ca.E_local = s->E_local;
        fa.ga.x_perm = x_perm;
        if (gather) {
            uintptr_t lo = 0;
            uint64_t span = 0;
            gather_window(s, src, &lo, &span);
            fa.ga.x_tok = (const uint16_t *)lo;
            fa.ga.x_bytes = span;
            fa.ga.x_nsrc = src->S;
            fa.ga.x_rows_per_src = rows.rows_per_src;
            for (int i = 0; i < src->S; ++i) fa.ga.x_src_off[i] = (uint32_t)((uintptr_t)src->x[i] - lo);
            fa.ga.row_token = row_token_ws;
            fa.ga.T = s->T;
        }
        fa.ga.w = (const uint16_t *)w_experts;
        fa.ga.y = (uint16_t *)y_perm;
        fa.ga.offsets = expert_offsets;
        fa.ga.tile_off = tile_off;
        fa.ga.hdr = hdr;
        fa.ga.d = s->d;
        fa.ga.N = s->N;
        fa.ga.F = swiglu ? s->N / 2 : 0;
        fa.ga.E_local = s->E_local;
        fa.src = rows;
        if (src->chunk_rows > 0) {
            fa.fl.ready = src->chunk_ready;
            fa.fl.sim_delay_us = src->sim_delay_us;
            fa.fl.has_payload = src->sim_payload ? 1 : 0;
            for (int i = 0; src->sim_payload && i < src->S; ++i)
                fa.fl.sim_payload[i] = (const uint16_t *)src->sim_payload[i];
            fa.fl.chunk_rows = src->chunk_rows;
            fa.fl.chunks_per_src = (src->rows_per_src + src->chunk_rows - 1) / src->chunk_rows;
            fa.fl.epoch = src->epoch;
        }
        fa.ids_in = topk_ids_in;
        fa.ids_user = topk_ids_in ? topk_ids_out : nullptr;
        fa.offsets = expert_offsets;
        fa.slot_of = slot_of;
        fa.row_token_ws = row_token_ws;
        fa.row_token_user = row_token;
        fa.x_perm = x_perm;
        fa.blkbase = blkbase;
        fa.tile_off = tile_off;
        fa.tile_cnt = (uint32_t *)(ws + L.tile_flag);
        fa.xcd_next = hdr->xcd_next;
        fa.bar_flag = (uint32_t *)(ws + L.bar_flag);
        fa.hdr = hdr;
        fa.spin_limit = spin_limit_ticks();
        fa.T = s->T;
        fa.d = s->d;
        fa.E = s->E;
        fa.k = s->k;
        fa.e_begin = s->e_begin;
        fa.E_local = s->E_local;
        fa.nblk = L.nblk;
        fa.bm = tu.bm;
        static_assert(256 % kMoveRows == 0, "mover units tile the GEMM row tiles");
        fa.has_sim = (src->chunk_rows > 0 && src->sim_delay_us) ? 1 : 0;
        // Grid: every resident workgroup, or n_mover + n_compute of them (n_compute alone in the gather
        // path); all of them must be resident together (grid barriers).
        int G = resident - fa.has_sim;
        if (tu.n_compute_wg > 0) {
            const int want = tu.n_compute_wg + (gather ? 0 : tu.n_mover_wg);
            if (want + fa.has_sim <= resident) G = want;
            else if (!plan.table_compute) return MK_EUNSUPPORTED;
        }
        if (G > kBarrierWGs) return MK_EUNSUPPORTED;
        const int grid = G + fa.has_sim;
        fa.gather = gather ? 1 : 0;
        fa.tails_last = tu.tile_order == MK_ORDER_TAILS_LAST ? 1 : 0;
        fa.n_mover = gather ? 0 : (tu.n_mover_wg > G ? G : tu.n_mover_wg);
        fa.max_tiles = L.max_tiles;
        fa.ticks_per_us = (uint32_t)ticks_per_us();
        fa.trace = (uint64_t *)(ws + L.trace);
        fa.status_out = status_out;
        if (ev_begin && hipEventRecord(ev_begin, hs) != hipSuccess) return MK_EHIP;
        // Four waves per workgroup (one per SIMD, 128 x 128 per wave) where a uniform routing gives every
        // expert at most 32 rows, i.e. every GEMM task is a short weight-streaming tile: the decode-shaped
        // share (T = 128, top-8 of 256) 0.194 -> 0.184 ms.  Eight waves otherwise (Mixtral-shaped 4% and
        // skewed 5% faster with eight: their full tiles keep the matrix cores busier with two waves a SIMD).
        const bool four_waves = (long)s->T * s->k <= 32L * s->E;
        if (launch_fused(fa, grid, tu.cooperative != 0, four_waves, hs) != hipSuccess) return MK_EHIP;
        if (ev_end && hipEventRecord(ev_end, hs) != hipSuccess) return MK_EHIP;
        return MK_OK;
    }

    CountArgs ca{};
    ca.ids = ids;
    ca.lrank = lrank;
    ca.blkcnt = blkcnt;
    ca.blkmask = blkmask;
    ca.err = &hdr->err;
    ca.T = s->T;
    ca.E = s->E;
    ca.k = s->k;
    ca.e_begin = s->e_begin;
    ca.E_local = s->E_local;

    if (s->T > 0) {
        if (!topk_ids_in) {
            RouterArgs ra{};
            ra.src = rows;
            ra.wr = w_router;
            ra.part = part;
            ra.T = s->T;
            ra.d = s->d;
            ra.E = s->E;
            if (launch_router(ra, hs) != hipSuccess) return MK_EHIP;
            TopkArgs ta{};
            ta.part = part;
            ta.bias = bias;
            ta.ids = ids;
            ta.ids_user = topk_ids_out;
            ta.w_user = topk_w_out;
            ta.T = s->T;
            ta.E = s->E;
            ta.k = s->k;
            if (launch_topk(ta, ca, true, hs) != hipSuccess) return MK_EHIP;
        } else {
            if (launch_count_given(topk_ids_in, ids, topk_ids_out, ca, hs) != hipSuccess) return MK_EHIP;
        }
    }

    ScanArgs sa{};
    sa.blkcnt = blkcnt;
    sa.blkbase = blkbase;
    sa.offsets_ws = expert_offsets;
    sa.offsets_user = nullptr;
    sa.tile_off = tile_off;
    sa.hdr = hdr;
    sa.nblk = L.nblk;
    sa.E_local = s->E_local;
    sa.bm = tu.bm;
    if (launch_scan(sa, hs) != hipSuccess) return MK_EHIP;
    if (s->T == 0) return (status_out && launch_status(hdr, status_out, hs) != hipSuccess) ? MK_EHIP : MK_OK;

    SlotArgs sl{};
    sl.ids = ids;
    sl.lrank = lrank;
    sl.blkbase = blkbase;
    sl.offsets = expert_offsets;
    sl.slot_of = slot_of;
    sl.row_token_ws = row_token_ws;
    sl.row_token_user = row_token;
    sl.T = s->T;
    sl.k = s->k;
    sl.e_begin = s->e_begin;
    sl.E_local = s->E_local;
    if (launch_slots(sl, hs) != hipSuccess) return MK_EHIP;
    if (launch_move(rows, row_token_ws, x_perm, s->d, hdr, hs) != hipSuccess) return MK_EHIP;

    GemmArgs ga{};
    ga.x_perm = x_perm;
    ga.w = (const uint16_t *)w_experts;
    ga.y = (uint16_t *)y_perm;
    ga.offsets = expert_offsets;
    ga.tile_off = tile_off;
    ga.hdr = hdr;
    ga.d = s->d;
    ga.N = s->N;
    ga.F = swiglu ? s->N / 2 : 0;
    ga.E_local = s->E_local;
    int grid = gemm_max_grid(tu.bm, tu.bn);
    if (grid <= 0) return MK_EHIP;
    if (tu.n_compute_wg > 0 && tu.n_compute_wg < grid) grid = tu.n_compute_wg;
    grid -= grid % 8;
    if (grid < 8) grid = 8;
    if (ev_begin && hipEventRecord(ev_begin, hs) != hipSuccess) return MK_EHIP;
    if ((swiglu ? launch_gemm_swiglu(ga, grid, hs) : launch_gemm(ga, tu.bm, tu.bn, grid, hs)) != hipSuccess)
        return MK_EHIP;
    if (ev_end && hipEventRecord(ev_end, hs) != hipSuccess) return MK_EHIP;
    if (status_out && launch_status(hdr, status_out, hs) != hipSuccess) return MK_EHIP;
    return MK_OK;
}


// ---------------------------------------------------------------- the library's own scratch

// Device memory of the no-allocation entry point: one array per GPU the library runs on, held until the
// process ends.  Host code never uses this name as an address (in host code it is a stand-in): it takes
// the device address once per device from hipGetSymbolAddress and keeps that.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];

}  // namespace

extern "C" {

const char *mk_status_str(mk_status st)
{
    switch (st) {
    case MK_OK: return "ok";
    case MK_EINVAL: return "invalid argument";
    case MK_EUNSUPPORTED: return "unsupported shape or option";
    case MK_EWORKSPACE: return "workspace too small";
    case MK_EHIP: return "HIP runtime error";
    case MK_ETIMEOUT: return "device wait timed out";
    default: return "unknown status";
    }
}

size_t mk_route_topk_workspace_bytes(int32_t T, int32_t E)
{
    if (T < 0 || E < 1) return 0;
    return align256((size_t)kRouterSegments * T * E * 4) + 256;
}

mk_status mk_route_topk(const void *x, const float *w_router, const float *bias, int32_t T, int32_t d, int32_t E,
                        int32_t k, int32_t *topk_ids, float *topk_w, float *logits, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    if (T < 0 || d <= 0 || E < 1 || k < 1 || k > E) return MK_EINVAL;
    if (d % 8 != 0) return MK_EINVAL;
    if (d % 128 != 0 || E > 1024 || k > kMaxK) return MK_EUNSUPPORTED;
    if (T == 0) return MK_OK;
    if (!x || !w_router || !topk_ids || !workspace) return MK_EINVAL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_ids) || !aligned16(workspace) ||
        (bias && !aligned16(bias)) || (topk_w && !aligned16(topk_w)) || (logits && !aligned16(logits)))
        return MK_EINVAL;
    if (workspace_bytes < mk_route_topk_workspace_bytes(T, E)) return MK_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    RouterArgs ra{};
    ra.src.p[0] = (const uint16_t *)x;
    ra.src.S = 1;
    ra.src.rows_per_src = T;
    ra.wr = w_router;
    ra.part = (float *)workspace;
    ra.T = T;
    ra.d = d;
    ra.E = E;
    if (launch_router(ra, st) != hipSuccess) return MK_EHIP;
    TopkArgs ta{};
    ta.part = (const float *)workspace;
    ta.bias = bias;
    ta.ids = topk_ids;
    ta.ids_user = nullptr;
    ta.w_user = topk_w;
    ta.logits_user = logits;
    ta.T = T;
    ta.E = E;
    ta.k = k;
    CountArgs ca{};
    if (launch_topk(ta, ca, false, st) != hipSuccess) return MK_EHIP;
    return MK_OK;
}

size_t mk_dispatch_gemm_workspace_bytes(const mk_shape *s, const mk_sources *src, const mk_tuning *tune)
{
    if (check_shape(s) != MK_OK || check_sources(s, src) != MK_OK) return 0;
    Plan p;
    if (plan_call(s, src, tune, p) != MK_OK) return 0;
    return p.L.total;
}

mk_status mk_select_tuning(const mk_shape *s, const mk_sources *src, mk_tuning *out)
{
    mk_status st = check_shape(s);
    if (st != MK_OK) return st;
    st = check_sources(s, src);
    if (st != MK_OK) return st;
    if (!out) return MK_EINVAL;
    *out = table_tuning(s, src);
    return MK_OK;
}

mk_status mk_dispatch_gemm(const mk_shape *s, const mk_sources *src, const float *w_router, const float *bias,
                           const int32_t *topk_ids_in, const void *w_experts, void *y_perm, int32_t *slot_of,
                           int32_t *expert_offsets, int32_t *topk_ids_out, float *topk_w_out, int32_t *row_token,
                           void *workspace, size_t workspace_bytes, const mk_tuning *tune, void *stream)
{
    return dispatch_impl(s, src, w_router, bias, topk_ids_in, w_experts, y_perm, slot_of, expert_offsets,
                         topk_ids_out, topk_w_out, row_token, workspace, workspace_bytes, tune, stream, nullptr,
                         nullptr);
}

mk_status mk_dispatch_gemm_swiglu(const mk_shape *s, const mk_sources *src, const float *w_router, const float *bias,
                                  const int32_t *topk_ids_in, const void *w_gate_up, void *h_perm, int32_t *slot_of,
                                  int32_t *expert_offsets, int32_t *topk_ids_out, float *topk_w_out,
                                  int32_t *row_token, void *workspace, size_t workspace_bytes, const mk_tuning *tune,
                                  void *stream)
{
    return dispatch_impl(s, src, w_router, bias, topk_ids_in, w_gate_up, h_perm, slot_of, expert_offsets,
                         topk_ids_out, topk_w_out, row_token, workspace, workspace_bytes, tune, stream, nullptr,
                         nullptr, true);
}

mk_status mk_dispatch_gemm_static(const mk_shape *s, const mk_sources *src, const float *w_router, const float *bias,
                                  const int32_t *topk_ids_in, const void *w_experts, void *y_perm, int32_t *slot_of,
                                  int32_t *expert_offsets, int32_t *topk_ids_out, float *topk_w_out,
                                  int32_t *row_token, int32_t *status, const mk_tuning *tune, void *stream)
{
    mk_status st = check_shape(s);
    if (st != MK_OK) return st;
    st = check_sources(s, src);
    if (st != MK_OK) return st;
    if (!status || !aligned16(status)) return MK_EINVAL;
    Plan plan;
    st = plan_call(s, src, tune, plan);
    if (st != MK_OK) return st;
    if (plan.L.total > MK_STATIC_SCRATCH_BYTES) return MK_EWORKSPACE;   // before any HIP call
    // The scratch address of the current device, taken once; at that time its barrier and error words
    // are zeroed by a kernel on the caller's stream (the rest of the workspace is rewritten by every call).
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MK_EHIP;
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_dev[dev]) {
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MK_EHIP;
            if (launch_zero(ptr, plan.L.part, (hipStream_t)stream) != hipSuccess) return MK_EHIP;
            g_scratch_dev[dev] = ptr;
        }
        ws = g_scratch_dev[dev];
    }
    return dispatch_impl(s, src, w_router, bias, topk_ids_in, w_experts, y_perm, slot_of, expert_offsets,
                         topk_ids_out, topk_w_out, row_token, ws, MK_STATIC_SCRATCH_BYTES, tune, stream, status,
                         &plan);
}

mk_status mk_dispatch_gemm_trace(const mk_shape *s, const mk_sources *src, size_t *offset, int32_t *n_wg,
                                  int32_t *words, int32_t *ticks_per_us_out)
{
    (void)src;   // the trace segment sits before the row buffer, at the same offset on every path
    const mk_status st = check_shape(s);
    if (st != MK_OK) return st;
    if (offset) *offset = ws_layout(s->T, s->d, s->E, s->k, s->E_local, false).trace;
    if (n_wg) *n_wg = kTraceWGs;
    if (words) *words = kTraceWords;
    if (ticks_per_us_out) *ticks_per_us_out = ticks_per_us();
    return MK_OK;
}

mk_status mk_combine(const void *y_perm, int32_t rows, const int32_t *slot_of, const float *topk_w, int32_t T,
                     int32_t k, int32_t N, void *out, void *stream)
{
    if (T < 0 || k < 1 || k > kMaxK || rows < 0 || N <= 0 || N % 8 != 0) return MK_EINVAL;
    if (T == 0) return MK_OK;
    if (!slot_of || !topk_w || !out || (rows > 0 && !y_perm)) return MK_EINVAL;
    if (!aligned16(slot_of) || !aligned16(topk_w) || !aligned16(out) || (y_perm && !aligned16(y_perm)))
        return MK_EINVAL;
    if (launch_combine((const uint16_t *)y_perm, rows, slot_of, topk_w, T, k, N, (uint16_t *)out,
                       (hipStream_t)stream) != hipSuccess)
        return MK_EHIP;
    return MK_OK;
}

mk_status mk_swiglu(const void *gate_up, int32_t rows, int32_t F, void *h, void *stream)
{
    if (rows < 0 || F <= 0 || F % 8 != 0) return MK_EINVAL;
    if (rows == 0) return MK_OK;
    if (!gate_up || !h || !aligned16(gate_up) || !aligned16(h)) return MK_EINVAL;
    if (launch_swiglu((const uint16_t *)gate_up, rows, F, (uint16_t *)h, (hipStream_t)stream) != hipSuccess)
        return MK_EHIP;
    return MK_OK;
}

size_t mk_grouped_gemm_workspace_bytes(int32_t E_local)
{
    if (E_local < 1 || E_local > 1024) return 0;
    return sizeof(WsHeader) + align256((size_t)(E_local + 1) * 4);
}

mk_status mk_grouped_gemm(const void *a, const int32_t *expert_offsets, int32_t E_local, const void *w, int32_t K,
                          int32_t N, void *y, void *workspace, size_t workspace_bytes, void *stream)
{
    if (E_local < 1 || E_local > 1024 || K <= 0 || N <= 0 || N % 8 != 0 || K % 8 != 0) return MK_EINVAL;
    if (K % 128 != 0) return MK_EUNSUPPORTED;
    if (!a || !expert_offsets || !w || !y || !workspace) return MK_EINVAL;
    if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned16(workspace) || !aligned16(expert_offsets))
        return MK_EINVAL;
    if (workspace_bytes < mk_grouped_gemm_workspace_bytes(E_local)) return MK_EWORKSPACE;
    hipStream_t hs = (hipStream_t)stream;
    WsHeader *hdr = (WsHeader *)workspace;
    int32_t *tile_off = (int32_t *)((char *)workspace + sizeof(WsHeader));
    if (launch_tiles(expert_offsets, E_local, 256, tile_off, hdr, hs) != hipSuccess) return MK_EHIP;
    GemmArgs ga{};
    ga.x_perm = (const uint16_t *)a;
    ga.w = (const uint16_t *)w;
    ga.y = (uint16_t *)y;
    ga.offsets = expert_offsets;
    ga.tile_off = tile_off;
    ga.hdr = hdr;
    ga.d = K;
    ga.N = N;
    ga.E_local = E_local;
    int grid = gemm_max_grid(256, 256);
    if (grid <= 0) return MK_EHIP;
    grid -= grid % 8;
    if (grid < 8) grid = 8;
    if (launch_gemm(ga, 256, 256, grid, hs) != hipSuccess) return MK_EHIP;
    return MK_OK;
}

mk_status mk_grouped_gemm_swiglu(const void *a, const int32_t *expert_offsets, int32_t E_local, const void *w_gate_up,
                                 int32_t K, int32_t F, void *h, void *workspace, size_t workspace_bytes, void *stream)
{
    if (E_local < 1 || E_local > 1024 || K <= 0 || F <= 0 || F % 8 != 0 || K % 8 != 0) return MK_EINVAL;
    if (K % 128 != 0) return MK_EUNSUPPORTED;
    // the tiles' W row offsets are 32-bit: 2F + 256 rows of K bf16 must stay below 2 GiB
    if ((int64_t)(2 * (int64_t)F + 256) * K * 2 >= ((int64_t)1 << 31)) return MK_EUNSUPPORTED;
    if (!a || !expert_offsets || !w_gate_up || !h || !workspace) return MK_EINVAL;
    if (!aligned16(a) || !aligned16(w_gate_up) || !aligned16(h) || !aligned16(workspace) || !aligned16(expert_offsets))
        return MK_EINVAL;
    if (workspace_bytes < mk_grouped_gemm_workspace_bytes(E_local)) return MK_EWORKSPACE;
    hipStream_t hs = (hipStream_t)stream;
    WsHeader *hdr = (WsHeader *)workspace;
    int32_t *tile_off = (int32_t *)((char *)workspace + sizeof(WsHeader));
    if (launch_tiles(expert_offsets, E_local, 256, tile_off, hdr, hs) != hipSuccess) return MK_EHIP;
    GemmArgs ga{};
    ga.x_perm = (const uint16_t *)a;
    ga.w = (const uint16_t *)w_gate_up;
    ga.y = (uint16_t *)h;
    ga.offsets = expert_offsets;
    ga.tile_off = tile_off;
    ga.hdr = hdr;
    ga.d = K;
    ga.N = 2 * F;
    ga.F = F;
    ga.E_local = E_local;
    int grid = gemm_max_grid(256, 256);
    if (grid <= 0) return MK_EHIP;
    grid -= grid % 8;
    if (grid < 8) grid = 8;
    if (launch_gemm_swiglu(ga, grid, hs) != hipSuccess) return MK_EHIP;
    return MK_OK;
}

mk_status mk_poll_error(void *workspace, int32_t *detail)
{
    if (!workspace) return MK_EINVAL;
    uint32_t w[2] = {0, 0};
    if (hipMemcpy(w, workspace, sizeof w, hipMemcpyDeviceToHost) != hipSuccess) return MK_EHIP;
    if (detail) *detail = (int32_t)w[1];
    if (w[0] != 0) {
        const uint32_t zero[2] = {0, 0};
        if (hipMemcpy(workspace, zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return MK_EHIP;
    }
    return (mk_status)w[0];
}

}  // extern "C"
