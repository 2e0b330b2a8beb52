/*
 * oracle.c -- plain, slow, obviously correct CPU model of the fused MoE
 * dispatch + expert GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under moe_dispatch_expert_amd/) never calls it, never links it
 * and shares no code, header or constant with it.
 *
 * What is computed follows the "MoE Dispatch+GEMM" fused kernel named in
 * "mKernel UCCL fuses NVLink/RDMA/compute into one persistent CUDA kernel"
 * (zubnet.ai), paragraph 2, and "mKernel : une bibliotheque de noyaux
 * fusionnes multi-GPU et multi-noeuds ..." (lefilia.fr), paragraphs 1 and 3:
 * every token is routed to experts, its row is dispatched to them, and each
 * expert runs its dense GEMM.  The pages give no formula for any step; every
 * step below is the plainest reading, stated where it is taken:
 *
 *   1. router logits l[t,e] = sum_i x[t,i] * Wr[i,e] in fp32, in one fixed
 *      order (8 contiguous K segments, sequential fma in each, the 8 partial
 *      sums added left to right, then the optional per-expert bias);
 *   2. top-k by (logit descending, expert id ascending);
 *   3. softmax gate over all E experts, evaluated in fp64;
 *   4. per-local-expert counts;
 *   5. exclusive prefix sum -> expert offsets;
 *   6. slots: within an expert, ascending token id (stable counting sort);
 *   7. expert GEMM y[r,n] = sum_i x[row_token[r],i] * W[e,n,i] in fp64.
 *
 * Steps 1-6 are exact (integer results, or an fp32 result with one fixed
 * rounding sequence); step 7 is the exact-arithmetic reference against which
 * a bf16-output, fp32-accumulating GEMM is judged within a tolerance.
 *
 * Parity pins (checked by the CPU tests, not by re-running this code):
 *   logits      - hand-worked order examples, error bound against exact sums
 *   top-k       - brute force over all k-subsets, closed forms (x = 0, ties)
 *   gate        - closed forms (uniform, two-expert sigmoid, rational bias)
 *   layout      - sort-based brute force, bijection, closed form for x = 0
 *   GEMM        - library fp64 matmul (E = 1, k = 1), tagged identity experts
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* Number of contiguous K segments of the router dot product (reading of the
 * pages' silence on accumulation order: see the header). */
#define ORACLE_ROUTER_SEGMENTS 8

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;   /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Step 1.  x [T,d] bf16 bits row-major; wr [d,E] fp32 row-major;
 * bias [E] or NULL; logits [T,E] out.  Requires d % 8 == 0. */
int oracle_logits(const uint16_t *x, const float *wr, const float *bias,
                  int T, int d, int E, float *logits)
{
    if (d % ORACLE_ROUTER_SEGMENTS != 0 || T < 0 || d <= 0 || E <= 0)
        return 1;
    const int seg = d / ORACLE_ROUTER_SEGMENTS;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            float part[ORACLE_ROUTER_SEGMENTS];
            for (int s = 0; s < ORACLE_ROUTER_SEGMENTS; ++s) {
                float acc = 0.0f;
                for (int i = s * seg; i < (s + 1) * seg; ++i)
                    acc = fmaf(bf16_bits_to_float(x[(size_t)t * d + i]),
                               wr[(size_t)i * E + e], acc);
                part[s] = acc;
            }
            float l = part[0];
            for (int s = 1; s < ORACLE_ROUTER_SEGMENTS; ++s)
                l = l + part[s];
            if (bias)
                l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
    }
    return 0;
}

/* "a beats b": larger logit, or equal logit (float ==, so -0 == +0) and the
 * lower expert id. */
static int beats(float la, int a, float lb, int b)
{
    return la > lb || (la == lb && a < b);
}

/* Steps 2-3.  logits [T,E]; ids [T,k] out in rank order (best first);
 * w [T,k] out, fp64 softmax probability of each chosen expert over all E. */
int oracle_topk(const float *logits, int T, int E, int k, int32_t *ids, double *w)
{
    if (k < 1 || k > E || T < 0)
        return 1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || beats(l[e], e, l[best], best))
                    best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        free(taken);
        double m = (double)l[ids[(size_t)t * k]];
        double z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp((double)l[e] - m);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - m) / z;
    }
    return 0;
}

/* Steps 4-6.  ids [T,k]; local experts are [e_begin, e_begin + E_local).
 * count [E_local], offsets [E_local+1], slot_of [T,k] (-1 = not local),
 * row_token [T*k] (first R entries written).  Returns 0 or 1 on bad input. */
int oracle_layout(const int32_t *ids, int T, int k, int e_begin, int E_local,
                  int32_t *count, int32_t *offsets, int32_t *slot_of,
                  int32_t *row_token)
{
    if (T < 0 || k < 1 || E_local < 1)
        return 1;
    for (int e = 0; e < E_local; ++e)
        count[e] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j] - e_begin;
            if (e >= 0 && e < E_local)
                count[e] += 1;
        }
    offsets[0] = 0;
    for (int e = 0; e < E_local; ++e)
        offsets[e + 1] = offsets[e] + count[e];
    int32_t *cur = (int32_t *)malloc(sizeof(int32_t) * (size_t)E_local);
    for (int e = 0; e < E_local; ++e)
        cur[e] = offsets[e];
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j] - e_begin;
            if (e >= 0 && e < E_local) {
                int slot = cur[e]++;
                slot_of[(size_t)t * k + j] = slot;
                row_token[slot] = t;
            } else {
                slot_of[(size_t)t * k + j] = -1;
            }
        }
    free(cur);
    return 0;
}

/* Step 7 for a chosen list of expert-buffer rows.  x [T,d] bf16 bits;
 * w [E_local,N,d] bf16 bits (K contiguous); offsets [E_local+1];
 * row_token [R]; rows [n_rows] (each < R); y [n_rows,N] fp64 out. */
int oracle_expert_rows(const uint16_t *x, int d, const uint16_t *w, int N,
                       const int32_t *offsets, int E_local,
                       const int32_t *row_token, const int32_t *rows,
                       int n_rows, double *y)
{
    const int R = offsets[E_local];
    for (int q = 0; q < n_rows; ++q)
        if (rows[q] < 0 || rows[q] >= R)
            return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < n_rows; ++q) {
        const int r = rows[q];
        int e = 0;
        while (!(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        const uint16_t *xr = x + (size_t)row_token[r] * d;
        for (int n = 0; n < N; ++n) {
            const uint16_t *wr = w + ((size_t)e * N + n) * d;
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += (double)bf16_bits_to_float(xr[i]) * (double)bf16_bits_to_float(wr[i]);
            y[(size_t)q * N + n] = acc;
        }
    }
    return 0;
}

/* Step 8 (the next step after the path: combine).  The weighted un-permute
 * that brings a token's expert outputs back to its own row:
 *   out[t][n] = sum over j = 0 .. k-1 with slot_of[t][j] >= 0 of
 *               w[t][j] * y[row_of_slot(slot_of[t][j])][n],
 * in ascending j, fp64.  Choices that are not local (slot -1) add nothing; the
 * gate weights are the softmax over all experts (not renormalised), so the
 * sums of all ranks' partial outputs make the full combine.
 * y [n_rows,N] fp64 holds the rows of the slots listed in slot_rows [n_rows];
 * slot_of [T,k]; w [T,k] fp64; out [T,N] fp64.
 * Returns 1 if a chosen slot is not among slot_rows. */
int oracle_combine(const double *y, const int32_t *slot_rows, int n_rows, int N,
                   const int32_t *slot_of, const double *w, int T, int k,
                   double *out)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int t = 0; t < T; ++t) {
        double *o = out + (size_t)t * N;
        for (int n = 0; n < N; ++n)
            o[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            const int32_t slot = slot_of[(size_t)t * k + j];
            if (slot < 0)
                continue;
            int q = 0;
            while (q < n_rows && slot_rows[q] != slot)
                ++q;
            if (q == n_rows) {
                bad = 1;
                continue;
            }
            const double wt = w[(size_t)t * k + j];
            for (int n = 0; n < N; ++n)
                o[n] += wt * y[(size_t)q * N + n];
        }
    }
    return bad;
}

/* Next row, expert FFN.  SwiGLU of the gate|up expert output rows:
 * gu [rows, 2F] holds g = columns [0, F) and u = columns [F, 2F) of each row;
 * h[r][f] = silu(g) * u with silu(g) = g / (1 + e^-g), fp64.  gu is bf16 bits. */
int oracle_swiglu(const uint16_t *gu, int rows, int F, double *h)
{
    if (rows < 0 || F < 1)
        return 1;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int f = 0; f < F; ++f) {
            const double g = (double)bf16_bits_to_float(gu[(size_t)r * 2 * F + f]);
            const double u = (double)bf16_bits_to_float(gu[(size_t)r * 2 * F + F + f]);
            h[(size_t)r * F + f] = g / (1.0 + exp(-g)) * u;
        }
    return 0;
}

/* Next row, expert FFN.  Grouped GEMM over the expert layout for chosen rows:
 * z[q][n] = sum_i a[rows[q]][i] * w[e][n][i], e the expert whose offsets range
 * holds rows[q]; a [R, K] and w [E_local, N, K] bf16 bits, z [n_rows, N] fp64. */
int oracle_grouped_rows(const uint16_t *a, int K, const uint16_t *w, int N,
                        const int32_t *offsets, int E_local, const int32_t *rows,
                        int n_rows, double *z)
{
    const int R = offsets[E_local];
    for (int q = 0; q < n_rows; ++q)
        if (rows[q] < 0 || rows[q] >= R)
            return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < n_rows; ++q) {
        const int r = rows[q];
        int e = 0;
        while (!(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        const uint16_t *ar = a + (size_t)r * K;
        for (int n = 0; n < N; ++n) {
            const uint16_t *wr = w + ((size_t)e * N + n) * K;
            double acc = 0.0;
            for (int i = 0; i < K; ++i)
                acc += (double)bf16_bits_to_float(ar[i]) * (double)bf16_bits_to_float(wr[i]);
            z[(size_t)q * N + n] = acc;
        }
    }
    return 0;
}

/* Threads the OpenMP loops above use (reported by the CPU baseline). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
