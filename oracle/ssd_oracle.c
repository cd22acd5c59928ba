/*
 * ssd_oracle.c -- plain fp64 CPU oracle for the Mamba2 selective-state scan.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the bench's CPU
 * baseline load this library. The product path never calls it, and it shares
 * no code, header or constant with the HIP library.
 *
 * What it computes is the plain definition of the scan, one token at a time,
 * in float64, from inputs that the caller has widened exactly to float64:
 *
 *   delta_t = softplus(dt_t + dt_bias)        (or dt_t when softplus is off)
 *   h_t     = exp(delta_t * A) * h_{t-1} + delta_t * x_t (outer) B_t
 *   y_t     = C_t . h_t + D * x_t
 *
 * This is the Mamba2 recurrence that the vLLM RFC "Mamba2: exact-replay
 * decode so that prefill, chunked prefill and decode produce identical bits"
 * measures both kernels against (section 2, item 1: the fp64 reference, of
 * which the chunked scan and the recurrent update are both fp32/bf16
 * approximations). The
 * ReplaySSM reproduction page ("Core equations") writes the same recurrence
 * as S_h = gamma_h S_ckpt + sum_j gamma_{j+1:h} v_j k_j^T with
 * alpha = exp(delta A), v = delta x, k = B, q = C.
 *
 * Readings taken where the pages are silent:
 *  - decay first, then input (h_t uses exp(delta_t A) on h_{t-1});
 *  - head h reads B/C group h / (H/G) (contiguous groups);
 *  - D[h] is added after the contraction with C, no gating;
 *  - softplus(u) = log1p(exp(u)) for u <= 0, u + log1p(exp(-u)) otherwise;
 *  - the boundary state is the state after the last token whose position,
 *    counted from the sequence start, is a multiple of the chunk size.
 *
 * Layouts (row-major, contiguous): x[T,H,P], dt[T,H], B/C[T,G,N],
 * state[S,H,P,N], chunk_states[S,max_chunks,H,P,N]. cu[S+1] holds int64
 * sequence offsets into the packed token dimension.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus64(double u)
{
    if (u <= 0.0)
        return log1p(exp(u));
    return u + log1p(exp(-u));
}

int ssd_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of later scans (n >= 1): timing runs of the oracle itself, e.g.
 * one core against the host's all. The arithmetic does not depend on it. */
void ssd_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Returns 0 on success, -1 on bad arguments, -2 when out of memory.
 * init, D, dt_bias, final_state, boundary_state, boundary_len and
 * chunk_states may be NULL. chunk_states[s, c] receives the state after
 * (c+1)*Q tokens of sequence s, for c < max_chunks.
 */
int ssd_oracle_scan(int32_t S, const int64_t *cu, int32_t H, int32_t G,
                    int32_t P, int32_t N, int32_t Q,
                    const double *x, const double *dt, const double *A,
                    const double *D, const double *dt_bias, int32_t dt_softplus,
                    const double *B, const double *C, const double *init,
                    double *y, double *final_state, double *boundary_state,
                    int64_t *boundary_len, double *chunk_states,
                    int32_t max_chunks)
{
    if (S < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || Q <= 0 || H % G != 0)
        return -1;
    if (!cu || !x || !dt || !A || !B || !C || !y)
        return -1;
    const int64_t PN = (int64_t)P * N;
    const int32_t heads_per_group = H / G;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t job = 0; job < (int64_t)S * H; ++job) {
        const int64_t s = job / H;
        const int32_t h = (int32_t)(job % H);
        const int32_t g = h / heads_per_group;
        double *st = (double *)malloc(sizeof(double) * PN);
        if (!st) {
            failed |= 1;
            continue;
        }
        if (init)
            memcpy(st, init + (s * H + h) * PN, sizeof(double) * PN);
        else
            memset(st, 0, sizeof(double) * PN);
        const int64_t t0 = cu[s], t1 = cu[s + 1];
        double *bnd = boundary_state ? boundary_state + (s * H + h) * PN : NULL;
        if (bnd)
            memcpy(bnd, st, sizeof(double) * PN);
        int64_t since_boundary = 0;
        for (int64_t t = t0; t < t1; ++t) {
            const double raw = dt[t * H + h];
            const double d = dt_softplus
                                 ? softplus64(raw + (dt_bias ? dt_bias[h] : 0.0))
                                 : raw + (dt_bias ? dt_bias[h] : 0.0);
            const double a = exp(d * A[h]);
            const double *xt = x + (t * H + h) * P;
            const double *bt = B + (t * G + g) * N;
            const double *ct = C + (t * G + g) * N;
            double *yt = y + (t * H + h) * P;
            for (int32_t p = 0; p < P; ++p) {
                const double dx = d * xt[p];
                double *row = st + (int64_t)p * N;
                double acc = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    row[n] = a * row[n] + dx * bt[n];
                    acc += row[n] * ct[n];
                }
                yt[p] = acc + (D ? D[h] : 0.0) * xt[p];
            }
            const int64_t done = t - t0 + 1;
            since_boundary = done % Q;
            if (since_boundary == 0) {
                if (bnd)
                    memcpy(bnd, st, sizeof(double) * PN);
                const int64_t c = done / Q - 1;
                if (chunk_states && c < max_chunks)
                    memcpy(chunk_states + ((s * max_chunks + c) * H + h) * PN,
                           st, sizeof(double) * PN);
            }
        }
        if (boundary_len && h == 0)
            boundary_len[s] = since_boundary;
        if (final_state)
            memcpy(final_state + (s * H + h) * PN, st, sizeof(double) * PN);
        free(st);
    }
    return failed ? -2 : 0;
}
