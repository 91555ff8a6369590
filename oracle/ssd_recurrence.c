/*
 * oracle/ssd_recurrence.c -- plain fp64 CPU oracle of the Mamba-2 SSD varlen
 * forward prefill scan with in-place state-pool write-back.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  The GPU
 * library never links, loads or calls it, and this file shares no code,
 * header or constant with the GPU path.
 *
 * What it computes is the plain definition of the operation, the per-token
 * linear recurrence, written out in double precision:
 *
 *   Source: "mamba2_ssd_scan" (Modular MAX kernels docs), section
 *   "Per-token recurrence", for every head h, head_dim channel p and the
 *   group g = h / (nheads / ngroups) that serves h:
 *     dts_t      = softplus(dt[t,h] + dt_bias[h])
 *     r_t        = exp(A[h] * dts_t)
 *     state[p,n] = state[p,n] * r_t + dts_t * B[t,g,n] * x[t,h,p]
 *     y[t,h,p]   = sum_n C[t,g,n] * state[p,n] + D[h] * x[t,h,p]
 *   The state resets at each query_start_loc boundary (zero, or the initial
 *   state), so no state crosses from one sequence to the next, and the state
 *   reached at a sequence's end is its final state (same section).
 *
 *   Source: "Mamba2SSDChunkScanVarlenFwdInplace" (Modular Mojo struct docs),
 *   struct description and "Tensor shapes": the initial state of sequence b
 *   is read from ssm_pool[cache_indices[b]] when has_initial_state[b] is
 *   true, and the final state is written into that same slot; D, dt_bias and
 *   has_initial_state may be empty (absent).  The dt_softplus parameter
 *   (default true) selects whether softplus is applied to dt + dt_bias.
 *
 * Readings of points the pages leave open:
 *   - y[t] uses the state after token t's update (order of the two lines).
 *   - dt_softplus = 0: dts = dt + dt_bias (the bias is still added).
 *   - softplus(v) = log(1 + e^v) exactly, evaluated as
 *     max(v,0) + log1p(exp(-|v|)); no threshold and no clamp.
 *   - absent D / dt_bias -> 0; absent has_initial_state -> all false.
 *   - has_initial_state[b] false: the slot is not read at all.
 *   - a zero-length sequence still writes its final state (= initial state,
 *     or zeros) into its slot.
 *   - written pool values are the fp64 final state rounded to fp32
 *     (round-to-nearest-even, the C cast); every other slot is copied bit
 *     for bit.
 *
 * Data types at the boundary: x, B, C are bf16 bit patterns (uint16); they
 * are widened to double exactly.  dt, A, D, dt_bias and the pool are fp32,
 * widened to double exactly.  Outputs y and final_states are fp64.
 *
 * Parallelism: OpenMP over (sequence, head) pairs only; every pair runs the
 * recurrence token by token in order.  No blocking, fusion or reordering of
 * the recurrence.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* log(1 + e^v) without overflow: max(v, 0) + log1p(e^{-|v|}). */
double ssd_oracle_softplus(double v)
{
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

int ssd_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Returns 0 on success, a negative number on a malformed problem:
 *   -1 bad sizes, -2 query_start_loc not non-decreasing from 0 to total_len,
 *   -3 cache index out of range, -4 out of memory.
 * pool_out may be NULL (pool write-back not materialised); when given it
 * receives a bit copy of pool_in with the written slots replaced.
 * final_states may be NULL.
 * seq_lo/seq_hi restrict the work to sequences [seq_lo, seq_hi) (the y rows
 * of other sequences are left untouched); pass 0 and batch for all of them.
 */
int ssd_oracle_recurrence(int64_t total_len, int32_t batch, int32_t nheads,
                          int32_t head_dim, int32_t ngroups, int32_t dstate,
                          int32_t max_slots, int32_t dt_softplus,
                          const uint16_t *x, const float *dt, const float *A,
                          const uint16_t *B, const uint16_t *C,
                          const float *D, const float *dt_bias,
                          const float *pool_in, const int32_t *query_start_loc,
                          const uint8_t *has_initial_state,
                          const uint32_t *cache_indices,
                          int32_t seq_lo, int32_t seq_hi,
                          double *y, double *final_states, float *pool_out)
{
    const int64_t T = total_len;
    const int H = nheads, P = head_dim, G = ngroups, N = dstate;
    if (T < 0 || batch < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 ||
        H % G != 0 || max_slots < 0)
        return -1;
    if (seq_lo < 0 || seq_hi > batch || seq_lo > seq_hi)
        return -1;
    if (batch > 0 && (query_start_loc[0] != 0 || query_start_loc[batch] != T))
        return -2;
    for (int b = 0; b < batch; ++b) {
        if (query_start_loc[b + 1] < query_start_loc[b])
            return -2;
        if (cache_indices[b] >= (uint32_t)max_slots)
            return -3;
    }

    const int heads_per_group = H / G;
    const size_t slot_elems = (size_t)H * P * N;
    const size_t head_state = (size_t)P * N;

    if (pool_out != NULL && pool_in != NULL && pool_out != pool_in)
        memcpy(pool_out, pool_in, sizeof(float) * slot_elems * (size_t)max_slots);

    const int npairs = (seq_hi - seq_lo) * H;
    int failed = 0;

#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * head_state);
        double *brow = (double *)malloc(sizeof(double) * (size_t)N);
        double *crow = (double *)malloc(sizeof(double) * (size_t)N);
        if (st == NULL || brow == NULL || crow == NULL) {
#pragma omp atomic write
            failed = 1;
        }

#pragma omp for schedule(dynamic, 1)
        for (int pair = 0; pair < npairs; ++pair) {
            if (failed)
                continue;
            const int b = seq_lo + pair / H;
            const int h = pair % H;
            const int g = h / heads_per_group;
            const int64_t s = query_start_loc[b];
            const int64_t e = query_start_loc[b + 1];
            const size_t slot = cache_indices[b];
            const int init = has_initial_state != NULL && has_initial_state[b] != 0;

            /* initial state: the pool slot when flagged, zeros otherwise */
            for (size_t k = 0; k < head_state; ++k)
                st[k] = init ? (double)pool_in[slot * slot_elems + (size_t)h * head_state + k]
                             : 0.0;

            const double a_h = (double)A[h];
            const double d_h = D != NULL ? (double)D[h] : 0.0;
            const double bias_h = dt_bias != NULL ? (double)dt_bias[h] : 0.0;

            for (int64_t t = s; t < e; ++t) {
                const double v = (double)dt[t * H + h] + bias_h;
                const double dts = dt_softplus ? ssd_oracle_softplus(v) : v;
                const double r = exp(a_h * dts);
                for (int n = 0; n < N; ++n) {
                    brow[n] = bf16_bits_to_double(B[(t * G + g) * N + n]);
                    crow[n] = bf16_bits_to_double(C[(t * G + g) * N + n]);
                }
                for (int p = 0; p < P; ++p) {
                    const double xv = bf16_bits_to_double(x[(t * H + h) * P + p]);
                    double *row = st + (size_t)p * N;
                    /* state update for token t ... */
                    for (int n = 0; n < N; ++n)
                        row[n] = row[n] * r + dts * brow[n] * xv;
                    /* ... then the output reads the updated state */
                    double acc = 0.0;
                    for (int n = 0; n < N; ++n)
                        acc += crow[n] * row[n];
                    y[(t * H + h) * P + p] = acc + d_h * xv;
                }
            }

            if (final_states != NULL)
                memcpy(final_states + ((size_t)b * H + h) * head_state, st,
                       sizeof(double) * head_state);
            if (pool_out != NULL)
                for (size_t k = 0; k < head_state; ++k)
                    pool_out[slot * slot_elems + (size_t)h * head_state + k] = (float)st[k];
        }
        free(st);
        free(brow);
        free(crow);
    }
    return failed ? -4 : 0;
}
