/*
 * mk.h -- C ABI of libmk.so: fused MoE dispatch + expert GEMM for MI355X (gfx950).
 *
 * The operation is the "MoE Dispatch+GEMM" fused kernel named in "mKernel UCCL
 * fuses NVLink/RDMA/compute into one persistent CUDA kernel" (zubnet.ai),
 * paragraph 2: tokens are routed to experts, their rows are dispatched into
 * expert-contiguous buffers and every expert runs its dense GEMM, inside one
 * persistent kernel whose workgroups take roles ("UC Berkeley presenta mKernel
 * ..." (edge.aivizor.me), paragraph 2) and overlap at tile granularity
 * (zubnet.ai, paragraph 2).  The pages give no formulas; the definitions below
 * are the readings this library implements.
 *
 * Conventions for every entry point
 *   - Array pointers are DEVICE pointers unless marked HOST.
 *   - bf16 arrays hold raw bf16 bit patterns (2 bytes each), row-major.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *   - The caller allocates and owns every buffer and keeps it alive until the
 *     stream has passed the call.  The library allocates no device memory on
 *     the call path and keeps no mutable global state.
 *   - Invalid arguments are reported synchronously by the return value and
 *     nothing is launched.  No exception crosses the ABI; nothing is printed.
 *   - Every device pointer must be 16-byte aligned.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mk_status;
enum {
    MK_OK = 0,
    MK_EINVAL = 1,        /* bad shape, null pointer, misalignment, k out of range */
    MK_EUNSUPPORTED = 2,  /* legal shape this library does not handle (see each call) */
    MK_EWORKSPACE = 3,    /* workspace missing or smaller than required */
    MK_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
    MK_ETIMEOUT = 5       /* a device-side wait exceeded its bound (mk_poll_error) */
};

/* Problem shape.  Local experts are [e_begin, e_begin + E_local) of the E
 * global experts the router scores.  Requires T >= 0, d > 0, d % 128 == 0,
 * 1 <= k <= E <= 1024, 0 <= e_begin, e_begin + E_local <= E, N > 0, N % 8 == 0. */
typedef struct {
    int32_t T, d, E, k, e_begin, E_local, N;
} mk_shape;

/* Where the token rows come from.  An ordinary call has S = 1, x[0] = the
 * [T, d] bf16 token matrix and chunk_rows = 0.  For one GPU's share of an
 * expert-parallel layer the rows arrive as S source shards (one per peer),
 * token t = s * rows_per_src + r, each shard in its own buffer; a chunk of
 * chunk_rows rows of a shard may be read only once its ready flag holds
 * `epoch` (acquire), which models "a tile that has arrived feeds the GEMM
 * while the next is still in flight" (zubnet.ai, paragraph 2). */
typedef struct {
    int32_t S;                   /* >= 1 */
    int32_t rows_per_src;        /* T == S * rows_per_src */
    const void *const *x;        /* HOST array of S device pointers, each [rows_per_src, d] bf16 */
    int32_t chunk_rows;          /* rows per ready flag; 0 = all rows already resident */
    uint32_t *chunk_ready;       /* [S * ceil(rows_per_src / chunk_rows)], chunk c = s * cps + j */
    uint32_t epoch;              /* chunk c is ready iff chunk_ready[c] == epoch */
    /* Arrival simulator (one GPU standing in for its peers).  If sim_delay_us
     * is non-NULL, one workgroup of the fused kernel writes chunk_ready[c] =
     * epoch (release) sim_delay_us[c] microseconds after the kernel starts.
     * If sim_payload is also non-NULL (HOST array of S device pointers, same
     * shape as x), that workgroup first copies the chunk from sim_payload[s]
     * into x[s] (which must then be writable), so a read before the release
     * sees whatever x held before the call.  The simulator holds at most
     * 16384 chunks (S * ceil(rows_per_src / chunk_rows)); more is
     * MK_EUNSUPPORTED. */
    const uint32_t *sim_delay_us;
    const void *const *sim_payload;
} mk_sources;

/* Role split, grid and tile sizes ("UC Berkeley presenta mKernel ..."
 * (edge.aivizor.me), paragraph 2, and "mKernel : une bibliotheque de noyaux
 * fusionnes ..." (lefilia.fr), paragraph 2: the number of thread blocks per
 * role is set per tensor shape).  All zeros = the per-shape table
 * (mk_select_tuning); a zero field means "the table's value".
 *   n_mover_wg    > 0: that many workgroups start in the dispatch (mover) role:
 *                 they copy token rows into an expert-contiguous buffer tile by
 *                 tile (waiting for the source chunks' ready flags when rows
 *                 arrive from peers) and then join the GEMM role;
 *                 MK_MOVERS_NONE: no mover role: the GEMM reads each tile's
 *                 token rows in place through the slot -> token map, and
 *                 when rows arrive from peers each tile first waits for the
 *                 ready flags of its rows' chunks (at most 8 sources, all
 *                 inside 4 GiB - 256 bytes from the lowest one; else
 *                 MK_EUNSUPPORTED);
 *                 MK_MOVERS_STAGED: one kernel launch per step instead of the
 *                 persistent kernel (no overlap; for comparison).
 *   n_compute_wg  > 0: workgroups that start in the GEMM role; the grid is then
 *                 n_compute_wg (+ n_mover_wg), and must fit the device at once
 *                 (else MK_EUNSUPPORTED).  0: every workgroup the device holds.
 *   bm, bn, bk    0 or the one tile this library has: 256 token rows, 256 output
 *                 columns, K slabs of 64 (the last row tile of each expert
 *                 shrinks to 128, 64 or 32 rows by itself); else MK_EUNSUPPORTED.
 *   cooperative   1: launch the persistent kernel cooperatively, so the runtime
 *                 guarantees that all its workgroups are resident together
 *                 (for callers that share the device with other streams); about
 *                 15 us more per call.  0: an ordinary launch (see
 *                 mk_dispatch_gemm).
 *   tile_order    order of the GEMM tasks (the fused path): MK_ORDER_EXPERT,
 *                 every expert's row tiles together (its short last tile
 *                 beside the full tiles that share its weights), or
 *                 MK_ORDER_TAILS_LAST, every other row tile of all experts
 *                 first and the experts' short last tiles (at most 64 rows)
 *                 after them (the last round is then made of short tasks).
 *                 0: the table's (tails last where a uniform routing gives
 *                 at most three rounds of tasks on 256 workgroups).
 *   ev_gemm_begin / ev_gemm_end: NULL, or hipEvent_t handles the library
 *                 records on `stream` immediately before and after the launch
 *                 that runs the expert GEMM, so a caller can time that kernel. */
#define MK_MOVERS_STAGED (-1)
#define MK_MOVERS_NONE (-2)
#define MK_ORDER_EXPERT 1
#define MK_ORDER_TAILS_LAST 2
typedef struct {
    int32_t n_mover_wg, n_compute_wg, bm, bn, bk, cooperative, tile_order;
    void *ev_gemm_begin;
    void *ev_gemm_end;
} mk_tuning;

/* Router: logits l[t,e] = sum_i x[t,i] * w_router[i,e] (+ bias[e]), fp32, in a
 * fixed order: K split into 8 contiguous segments of d/8, a sequential fused
 * multiply-add chain in ascending i inside each segment, the 8 partial sums
 * added left to right, then the bias.  Top-k keeps the k experts ranked by
 * (logit descending, expert id ascending; -0 equals +0); topk_ids[t, j] is the
 * j-th best.  topk_w[t, j] is the softmax over all E logits at that expert
 * (not renormalised over the k).  Token routing is named in zubnet.ai,
 * paragraph 2, and lefilia.fr, paragraph 3; the order, tie rule and gate are
 * this library's readings.
 *   x         [T, d] bf16          w_router [d, E] fp32     bias [E] fp32 or NULL
 *   topk_ids  [T, k] int32 (out)   topk_w   [T, k] fp32 (out, may be NULL)
 *   logits    [T, E] fp32 (out, may be NULL): every logit as it entered the
 *             selection (the ordered sum above, bias included), for checking
 *   workspace mk_route_topk_workspace_bytes(T, E) bytes, any contents.
 * T == 0 is a no-op returning MK_OK. */
size_t mk_route_topk_workspace_bytes(int32_t T, int32_t E);
mk_status mk_route_topk(const void *x, const float *w_router, const float *bias,
                        int32_t T, int32_t d, int32_t E, int32_t k,
                        int32_t *topk_ids, float *topk_w, float *logits,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace mk_dispatch_gemm needs for this shape, sources and tuning
 * (tune NULL = the per-shape table); 0 on bad input.  Paths that copy rows (a
 * mover role or the staged launches) need room for the expert-contiguous row
 * buffer, [T * min(k, E_local) + 256, d] bf16; the in-place path does not. */
size_t mk_dispatch_gemm_workspace_bytes(const mk_shape *s, const mk_sources *src, const mk_tuning *tune);

/* Fused dispatch + expert GEMM, one persistent launch.
 * Steps (routing per mk_route_topk unless topk_ids_in is given):
 *   count[e']   = #{(t, j) : topk_ids[t, j] == e_begin + e'}        (histogram)
 *   offsets     = exclusive prefix sum of count; R = offsets[E_local]
 *   slot_of[t,j]= offsets[e'] + #{t' < t : e' chosen by t'}  or -1 if not local
 *   row_token[slot_of[t,j]] = t
 *   x_perm[r]   = x[row_token[r]]   (tile-chunked scatter into expert-contiguous rows)
 *   y_perm[r,n] = bf16_rne(sum_i x_perm[r,i] * w_experts[e', n, i]), fp32 accumulation
 * Arguments:
 *   w_router, bias     router inputs (used iff topk_ids_in == NULL)
 *   topk_ids_in        NULL = route inside this call; else [T, k] int32 ids routed
 *                      by the sources (validated on device: out-of-range ids -> MK_EINVAL
 *                      via mk_poll_error)
 *   w_experts          [E_local, N, d] bf16, K contiguous (y = x . W^T)
 *   y_perm             [T * min(k, E_local), N] bf16; rows >= R are not written
 *   slot_of            [T, k] int32
 *   expert_offsets     [E_local + 1] int32
 *   topk_ids_out       NULL or [T, k] int32     topk_w_out NULL or [T, k] fp32
 *   row_token          NULL or [T * min(k, E_local)] int32 (first R written)
 *   workspace          mk_dispatch_gemm_workspace_bytes(s, src, tune) bytes, ZERO-FILLED
 *                      ONCE before its first use; it carries state between calls (the
 *                      call epoch from which grid-barrier targets derive), so two calls
 *                      in flight must not share one.
 *   tune               NULL or all zeros = per-shape table
 * Device-side failures (a wait that timed out, bad topk_ids_in) are reported by
 * mk_poll_error after the stream is synchronised; outputs are then undefined.
 * The workspace stays failed until mk_poll_error has read and cleared the error:
 * every call through it before that stops early (outputs undefined).  After
 * that it needs no re-zeroing: a failed call still ends its epoch, so barrier
 * state it left behind cannot satisfy a later call's barriers.
 * The fused kernel runs one workgroup per resident slot of the device (eight
 * waves; four, one per SIMD, where T * k <= 32 * E, i.e. a uniform routing
 * gives every expert at most 32 rows, N % 256 == 0 and no SwiGLU epilogue) and
 * synchronises them with grid barriers: they must all become resident, so
 * work of other streams on the device only delays it, and a wait longer than
 * the bound (MK_TIMEOUT_US microseconds, default 2000000) ends the call with
 * MK_ETIMEOUT rather than hanging. */
mk_status mk_dispatch_gemm(const mk_shape *s, const mk_sources *src,
                           const float *w_router, const float *bias,
                           const int32_t *topk_ids_in,
                           const void *w_experts,
                           void *y_perm, int32_t *slot_of, int32_t *expert_offsets,
                           int32_t *topk_ids_out, float *topk_w_out, int32_t *row_token,
                           void *workspace, size_t workspace_bytes,
                           const mk_tuning *tune, void *stream);

/* mk_dispatch_gemm with the expert FFN's gate|up weights and the SwiGLU of
 * mk_swiglu in the GEMM's epilogue, so the first half of the expert FFN runs
 * over the dispatch's own layout in the same launch.  The pages name the MoE
 * Dispatch+GEMM kernel (zubnet.ai, paragraph 2), whose experts in MoE models
 * are gated FFNs; the gated form is this library's reading, as for mk_swiglu.
 * Everything is as for mk_dispatch_gemm (routing, layout, outputs other than
 * y_perm, workspace and its size, tuning, errors) with s->N = 2F and:
 *   w_gate_up [E_local, 2F, d] bf16 (F gate rows, then F up rows; d contiguous)
 *   h_perm    [T * min(k, E_local), F] bf16 (out; rows >= R are not written):
 *             h_perm[r, f] = bf16_rne( silu(g) * u ), g and u the bf16 outputs
 *             of mk_dispatch_gemm with w_experts = w_gate_up at columns f and
 *             F + f, i.e. bit for bit mk_dispatch_gemm followed by mk_swiglu.
 * Requires F % 8 == 0 (s->N % 16 == 0, else MK_EINVAL) and
 * (2F + 256) * d * 2 < 2^31 (else MK_EUNSUPPORTED). */
mk_status mk_dispatch_gemm_swiglu(const mk_shape *s, const mk_sources *src,
                                  const float *w_router, const float *bias,
                                  const int32_t *topk_ids_in,
                                  const void *w_gate_up,
                                  void *h_perm, int32_t *slot_of, int32_t *expert_offsets,
                                  int32_t *topk_ids_out, float *topk_w_out, int32_t *row_token,
                                  void *workspace, size_t workspace_bytes,
                                  const mk_tuning *tune, void *stream);

/* mk_dispatch_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, inputs and outputs, with the workspace replaced by the
 * library's own device array of MK_STATIC_SCRATCH_BYTES (one per GPU, held
 * until the process ends).  The call allocates nothing.
 *   status   [2] int32 (out, device): the call's device status (an mk_status:
 *            MK_OK, MK_ETIMEOUT or MK_EINVAL) and its detail, written when the
 *            call ends on the stream (read it after a sync); it takes the
 *            place of mk_poll_error for this entry point.
 * A shape, sources and tuning whose workspace (mk_dispatch_gemm_workspace_bytes)
 * exceeds MK_STATIC_SCRATCH_BYTES is refused with MK_EWORKSPACE before any
 * device work; paths that copy rows into the expert-contiguous buffer need it
 * for the rows, so in practice this is the in-place path.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and give undefined results. */
#define MK_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
mk_status mk_dispatch_gemm_static(const mk_shape *s, const mk_sources *src,
                                  const float *w_router, const float *bias,
                                  const int32_t *topk_ids_in,
                                  const void *w_experts,
                                  void *y_perm, int32_t *slot_of, int32_t *expert_offsets,
                                  int32_t *topk_ids_out, float *topk_w_out, int32_t *row_token,
                                  int32_t *status, const mk_tuning *tune, void *stream);

/* The tuning the per-shape table picks (what a NULL/zero `tune` means), keyed
 * on the shape and the sources:
 *   rows readable in place (at most 8 sources inside one 4 GiB window,
 *     resident or arriving in chunks): no mover role (MK_MOVERS_NONE), and
 *     n_compute_wg = the GEMM tasks a uniform routing gives
 *     (E_local * ceil(T k / E / 256) * ceil(N / 256)) plus a quarter,
 *     rounded up to a multiple of 8, at least 32; 0 (every co-resident
 *     workgroup) once that reaches 256;
 *   otherwise: n_mover_wg = 256 (every workgroup moves rows first, then
 *     computes), n_compute_wg = 0;
 *   bm = bn = 256, bk = 64, cooperative = 0.
 * A value the table gives that the device cannot hold at once is clamped to
 * it; one the caller gives is refused (MK_EUNSUPPORTED). */
mk_status mk_select_tuning(const mk_shape *s, const mk_sources *src, mk_tuning *out);

/* Where the fused kernel's per-workgroup trace lives inside a dispatch
 * workspace: *offset bytes from its start, *n_wg records of *words uint64
 * each (record w = workgroup w).  Words, written by every fused call:
 *   0 start, 1 router logits done, 2 barrier A passed, 3 histogram done,
 *   4 barrier B passed, 5 scan done, 6 barrier C passed (in-place path), 7 mover role
 *   done, 8 first GEMM task started, 9 workgroup done (wall-clock ticks,
 *   *ticks_per_us per microsecond); 10 GEMM tasks run, 11 ticks spent
 *   waiting for tiles, 12 hardware XCD id, 13 mover units copied, 14 ticks
 *   copying rows, 15 ticks publishing moved units, 16 token-parallel
 *   selection done (routing inside only); words 17.. are zero.
 * For profiling the overlap of the roles; the host reads it after a sync. */
mk_status mk_dispatch_gemm_trace(const mk_shape *s, const mk_sources *src, size_t *offset, int32_t *n_wg,
                                  int32_t *words, int32_t *ticks_per_us);

/* Combine, the step after the path: the weighted un-permute that brings each
 * token's expert outputs back to its own row,
 *   out[t, n] = bf16_rne( sum over j = 0 .. k-1 with 0 <= slot_of[t, j] < rows
 *                         of topk_w[t, j] * y_perm[slot_of[t, j], n] ),
 * fp32 accumulation in ascending j.  A slot of -1 (a choice that is not local)
 * adds nothing, and so does any slot outside [0, rows); a token without a local
 * choice gets a zero row.  The gates are used as given (softmax over all
 * experts, not renormalised), so the outputs of all expert-parallel ranks add
 * up to the full combine.  The pages name the dispatch kernel and the dynamic
 * routing of tokens to experts that may live elsewhere (zubnet.ai, paragraph 2;
 * lefilia.fr, paragraph 3) but do not write this step out; the sum above is
 * this library's reading.
 *   y_perm [rows, N] bf16 (mk_dispatch_gemm's output)   slot_of [T, k] int32
 *   topk_w [T, k] fp32                                  out [T, N] bf16 (out)
 * Requires T >= 0, 1 <= k <= 32, rows >= 0, N > 0, N % 8 == 0.  T == 0 is a
 * no-op returning MK_OK.  No workspace. */
mk_status mk_combine(const void *y_perm, int32_t rows, const int32_t *slot_of, const float *topk_w,
                     int32_t T, int32_t k, int32_t N, void *out, void *stream);

/* Expert FFN after the gate|up GEMM (next row: the pages name the MoE
 * Dispatch+GEMM kernel, zubnet.ai paragraph 2, whose experts in MoE models are
 * gated FFNs; the activation and the down-projection below are this library's
 * reading).  With w_experts of mk_dispatch_gemm holding the gate rows and then
 * the up rows of every expert ([E_local, 2F, d]), y_perm rows are [g | u]:
 *   h[r, f] = bf16_rne( silu(g[r, f]) * u[r, f] ),  silu(g) = g / (1 + e^-g), fp32.
 *   gate_up [rows, 2F] bf16    h [rows, F] bf16 (out)
 * Requires rows >= 0, F > 0, F % 8 == 0; rows == 0 is a no-op. */
mk_status mk_swiglu(const void *gate_up, int32_t rows, int32_t F, void *h, void *stream);

/* Grouped GEMM over an expert layout (the down-projection of the expert FFN):
 *   y[r, n] = bf16_rne( sum_i a[r, i] * w[e, n, i] ),  fp32 accumulation,
 * for every row r of expert e, offsets[e] <= r < offsets[e + 1] (the layout
 * mk_dispatch_gemm returns).  R = offsets[E_local] is read on the device.
 *   a [>= R, K] bf16    expert_offsets [E_local + 1] int32 (non-decreasing, offsets[0] = 0)
 *   w [E_local, N, K] bf16 (K contiguous)    y [>= R, N] bf16 (out; rows >= R untouched)
 *   workspace mk_grouped_gemm_workspace_bytes(E_local) bytes, any contents
 * Requires 1 <= E_local <= 1024, K % 128 == 0 (else MK_EUNSUPPORTED for K % 8 == 0),
 * N > 0, N % 8 == 0. */
size_t mk_grouped_gemm_workspace_bytes(int32_t E_local);
mk_status mk_grouped_gemm(const void *a, const int32_t *expert_offsets, int32_t E_local, const void *w, int32_t K,
                          int32_t N, void *y, void *workspace, size_t workspace_bytes, void *stream);

/* The expert FFN's gate|up GEMM with the SwiGLU of mk_swiglu in its epilogue.
 * The pages name the MoE Dispatch+GEMM kernel (zubnet.ai, paragraph 2), whose
 * experts in MoE models are gated FFNs; the gated form below is this library's
 * reading, the same as for mk_swiglu.  For every row r of expert e,
 *   g = bf16_rne( sum_i a[r, i] * w_gate_up[e, f, i] ),  u = bf16_rne( sum_i a[r, i] * w_gate_up[e, F + f, i] ),
 *   h[r, f] = bf16_rne( silu(g) * u ),  fp32 accumulation and activation,
 * i.e. bit for bit mk_grouped_gemm (N = 2F) followed by mk_swiglu, without the
 * [R, 2F] intermediate in memory.
 *   a [>= R, K] bf16    expert_offsets [E_local + 1] int32 as for mk_grouped_gemm
 *   w_gate_up [E_local, 2F, K] bf16 (gate rows, then up rows; K contiguous)
 *   h [>= R, F] bf16 (out; rows >= R untouched)
 *   workspace mk_grouped_gemm_workspace_bytes(E_local) bytes, any contents
 * Requires 1 <= E_local <= 1024, K % 128 == 0 (else MK_EUNSUPPORTED for K % 8 == 0),
 * F > 0, F % 8 == 0, (2F + 256) * K * 2 < 2^31 (else MK_EUNSUPPORTED). */
mk_status mk_grouped_gemm_swiglu(const void *a, const int32_t *expert_offsets, int32_t E_local, const void *w_gate_up,
                                 int32_t K, int32_t F, void *h, void *workspace, size_t workspace_bytes, void *stream);

/* Synchronous: reads the device error word of a dispatch workspace (the caller
 * must have synchronised the stream).  Returns MK_OK, MK_ETIMEOUT or MK_EINVAL;
 * *detail (if non-NULL) receives which wait or id failed.  Clears the word. */
mk_status mk_poll_error(void *workspace, int32_t *detail);

/* Static string for a status code. */
const char *mk_status_str(mk_status st);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
