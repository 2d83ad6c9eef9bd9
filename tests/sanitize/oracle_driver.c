/* Drives the C oracle (oracle.c) for the sanitizer test: reads a problem from
 * stdin (whitespace-separated integers), runs it, prints the bf16 result bits.
 *   gemm M N K has_res   then A (M*K), W (N*K), [R (M*N)]     -> M*N bits
 *   tail M d D has_s eps_e6 then L (M*d), gamma (d), W (D*d), [S (M*D)] -> M*D bits
 *   round count then count doubles (as %la hex floats)      -> count bits
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_round_bf16(double v);
void oracle_gemm(int M, int N, int K, const uint16_t *A, long lda, const uint16_t *W, long ldw,
                 const uint16_t *R, long ldr, double *c_exact, uint16_t *c_bf16, long ldc);
void oracle_latent_tail(int M, int d, int D, const uint16_t *L, const uint16_t *gamma, double eps,
                        const uint16_t *Wup, const uint16_t *S, int variant, double *out_exact,
                        uint16_t *out_bf16);

static uint16_t *read_u16(size_t n)
{
    uint16_t *p = malloc((n ? n : 1) * sizeof *p);
    for (size_t i = 0; i < n; ++i) {
        unsigned v;
        if (scanf("%u", &v) != 1)
            exit(2);
        p[i] = (uint16_t)v;
    }
    return p;
}

int main(void)
{
    char op[16];
    while (scanf("%15s", op) == 1) {
        if (strcmp(op, "gemm") == 0) {
            int M, N, K, hr;
            if (scanf("%d %d %d %d", &M, &N, &K, &hr) != 4)
                return 2;
            uint16_t *A = read_u16((size_t)M * K), *W = read_u16((size_t)N * K);
            uint16_t *R = hr ? read_u16((size_t)M * N) : NULL;
            double *ex = malloc(((size_t)M * N + 1) * sizeof *ex);
            uint16_t *c = malloc(((size_t)M * N + 1) * sizeof *c);
            oracle_gemm(M, N, K, A, K, W, K, R, N, ex, c, N);
            for (size_t i = 0; i < (size_t)M * N; ++i)
                printf("%u\n", c[i]);
            free(A); free(W); free(R); free(ex); free(c);
        } else if (strcmp(op, "tail") == 0) {
            int M, d, D, hs, eps6;
            if (scanf("%d %d %d %d %d", &M, &d, &D, &hs, &eps6) != 5)
                return 2;
            uint16_t *L = read_u16((size_t)M * d), *g = read_u16((size_t)d);
            uint16_t *W = read_u16((size_t)D * d);
            uint16_t *S = hs ? read_u16((size_t)M * D) : NULL;
            uint16_t *o = malloc(((size_t)M * D + 1) * sizeof *o);
            for (int variant = 0; variant <= 1; ++variant) {
                oracle_latent_tail(M, d, D, L, g, eps6 * 1e-6, W, S, variant, NULL, o);
                for (size_t i = 0; i < (size_t)M * D; ++i)
                    printf("%u\n", o[i]);
            }
            free(L); free(g); free(W); free(S); free(o);
        } else if (strcmp(op, "round") == 0) {
            int n;
            if (scanf("%d", &n) != 1)
                return 2;
            for (int i = 0; i < n; ++i) {
                double v;
                if (scanf("%la", &v) != 1)
                    return 2;
                printf("%u\n", oracle_round_bf16(v));
            }
        } else {
            return 2;
        }
    }
    return 0;
}
