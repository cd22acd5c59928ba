/* oracle_check.c -- the fp64 oracle (oracle/ssd_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: a varlen pack with empty
 * and chunk-multiple sequences, every optional output, and a case with a
 * closed form (one head, P = N = 1, constant decay a and input b: the state
 * after t tokens from h0 is a^t h0 + b (1 - a^t) / (1 - a)), plus the
 * argument checks. Exit status 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_oracle_scan(int32_t S, const int64_t *cu, int32_t H, int32_t G, int32_t P, int32_t N,
                    int32_t Q, const double *x, const double *dt, const double *A,
                    const double *D, const double *dt_bias, int32_t dt_softplus,
                    const double *B, const double *C, const double *init, double *y,
                    double *final_state, double *boundary_state, int64_t *boundary_len,
                    double *chunk_states, int32_t max_chunks);

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static double *filled(size_t n, unsigned *seed)
{
    double *p = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) {
        *seed = *seed * 1103515245u + 12345u;
        p[i] = ((double)((*seed >> 8) & 0xffff) / 65536.0) - 0.5;
    }
    return p;
}

int main(void)
{
    unsigned seed = 7;
    {
        const int32_t S = 4, H = 4, G = 2, P = 3, N = 5, Q = 8, MC = 3;
        const int64_t cu[] = {0, 0, 16, 21, 45};
        const int64_t T = cu[S];
        double *x = filled(T * H * P, &seed), *dt = filled(T * H, &seed);
        double *B = filled(T * G * N, &seed), *C = filled(T * G * N, &seed);
        double *A = filled(H, &seed), *D = filled(H, &seed), *bias = filled(H, &seed);
        double *init = filled(S * H * P * N, &seed);
        double *y = calloc(T * H * P, sizeof(double));
        double *fin = calloc(S * H * P * N, sizeof(double));
        double *bnd = calloc(S * H * P * N, sizeof(double));
        double *cs = calloc(S * MC * H * P * N, sizeof(double));
        int64_t blen[4];
        for (int h = 0; h < H; ++h)
            A[h] = -1.0 - 8.0 * fabs(A[h]);
        EXPECT(ssd_oracle_scan(S, cu, H, G, P, N, Q, x, dt, A, D, bias, 1, B, C, init, y, fin,
                               bnd, blen, cs, MC) == 0);
        EXPECT(blen[0] == 0 && blen[1] == 0 && blen[2] == 5 && blen[3] == 0);
        /* the empty sequence keeps its initial state */
        for (int i = 0; i < H * P * N; ++i)
            EXPECT(fin[i] == init[i] && bnd[i] == init[i]);
        /* the chunk-multiple sequence: boundary = final = its second chunk state */
        for (int i = 0; i < H * P * N; ++i) {
            EXPECT(bnd[1 * H * P * N + i] == fin[1 * H * P * N + i]);
            EXPECT(cs[(1 * MC + 1) * H * P * N + i] == fin[1 * H * P * N + i]);
        }
        EXPECT(ssd_oracle_scan(S, cu, H, G, P, N, Q, x, dt, A, NULL, NULL, 0, B, C, NULL, y,
                               NULL, NULL, NULL, NULL, 0) == 0);
        EXPECT(ssd_oracle_scan(S, cu, 3, 2, P, N, Q, x, dt, A, D, bias, 1, B, C, init, y, fin,
                               bnd, blen, cs, MC) == -1);   /* H % G != 0 */
        EXPECT(ssd_oracle_scan(S, cu, H, G, P, N, Q, NULL, dt, A, D, bias, 1, B, C, init, y, fin,
                               bnd, blen, cs, MC) == -1);
        free(x); free(dt); free(B); free(C); free(A); free(D); free(bias); free(init);
        free(y); free(fin); free(bnd); free(cs);
    }
    {
        /* closed form: delta = dt (softplus off), a = exp(delta A), input
         * delta x B per token, C = 1 so y_t = h_t + D x */
        const int64_t cu[] = {0, 40};
        double x[40], dt[40], B[40], C[40], y[40], fin, h0 = 0.75;
        const double A = -0.3, D = 0.5, d = 0.2, xv = 1.5, bv = 2.0;
        for (int t = 0; t < 40; ++t) {
            x[t] = xv; dt[t] = d; B[t] = bv; C[t] = 1.0;
        }
        EXPECT(ssd_oracle_scan(1, cu, 1, 1, 1, 1, 16, x, dt, &A, &D, NULL, 0, B, C, &h0, y, &fin,
                               NULL, NULL, NULL, 0) == 0);
        const double a = exp(d * A), b = d * xv * bv;
        for (int t = 0; t < 40; ++t) {
            const double at = pow(a, t + 1);
            const double h = at * h0 + b * (1.0 - at) / (1.0 - a);
            EXPECT(fabs(y[t] - (h + D * xv)) <= 1e-13 * fabs(h + D * xv));
        }
    }
    printf("oracle check: %d failed expectations\n", fails);
    return fails == 0 ? 0 : 1;
}
