/*
 * Oracle for the bf16 skinny-GEMM hot path (Kimi-K3 KDA decode projections and
 * the latent-MoE tail).  TEST INFRASTRUCTURE ONLY: nothing in the product path
 * links, loads or calls this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.
 *
 * Plain, slow, obviously correct: every result is a sequential k-loop in IEEE
 * double over the exact widening of the bf16 inputs, followed by one
 * round-to-nearest-even to bf16 at exactly the points the method rounds.  A
 * bf16 x bf16 product has at most 16 significant bits, so every product is
 * exact in double; only the running sum rounds (relative error ~K * 2^-53).
 * OpenMP splits the independent output elements across threads; it does not
 * change the arithmetic of any single element.
 *
 * Sources (vLLM pull-request summaries on prhub.com.cn):
 *  - "Kimi K3 support, phase 1" (#50089), key source snippets,
 *    _skinny_gemm.py CuteSkinnyGemm docstring: C[M,N] = A[M,K] @ B[N,K]^T
 *    + residual, bf16 inputs, fp32 accumulation; the residual is added to the
 *    accumulator before the single store.
 *  - same page, latent_moe_runner.py LatentMoERunner docstring: the latent
 *    partial is RMS-normed and up-projected by a replicated up-projection; the
 *    shared-expert partial is added in the GEMM epilogue (addmm).
 *  - "Overlap low-M TP8 KDA projections" (#54697), key source snippets,
 *    low_latency_gemm.py run_kda_projection_overlap: the F_A/beta projection is
 *    split into f_a (rank 128) and beta, and the bf16 f_a tensor feeds the F_B
 *    GEMM that yields g1.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Exact widening of a bf16 bit pattern: the bf16 bits are the top half of an
 * IEEE binary32, and binary32 -> binary64 is exact. */
static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, binary32 exponent
 * range), ties to an even last significand bit.  Written from the definition:
 * find the binade [2^E, 2^(E+1)) of |v|, the bf16 spacing there is 2^(E-7)
 * (fixed at 2^-133 below the normal range), scale |v| to a count of spacings
 * (exact, a power-of-two scaling), round that count to the nearest integer
 * with ties to even, and scale back.  A count of 256 at E = 127 is 2^128,
 * which is beyond the largest bf16 and becomes +-inf. */
uint16_t oracle_round_bf16(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t sign = (uint16_t)(neg ? 0x8000u : 0u);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e2;
    (void)frexp(a, &e2);  /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;       /* 2^E <= a < 2^(E+1) */
    if (E < -126)
        E = -126;
    double spacing = ldexp(1.0, E - 7);
    double q = a / spacing;          /* exact: division by a power of two */
    double fl = floor(q);
    double frac = q - fl;            /* exact */
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double res = r * spacing;
    if (res >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)res;            /* exact: res has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

double oracle_bf16_to_f64(uint16_t b) { return bf16_to_f64(b); }

/* Skinny GEMM with optional residual (CuteSkinnyGemm docstring, #50089):
 *   C[m,n] = round_bf16( sum_k A[m,k] * W[n,k] + R[m,n] )
 * A is [M,K] with row stride lda, W is [N,K] (nn.Linear layout) with row stride
 * ldw, R is [M,N] with row stride ldr or NULL.  c_exact (nullable) receives
 * the unrounded double value, c_bf16 (nullable) the rounded bits; both have
 * row stride ldc. */
void oracle_gemm(int M, int N, int K,
                 const uint16_t *A, long lda,
                 const uint16_t *W, long ldw,
                 const uint16_t *R, long ldr,
                 double *c_exact, uint16_t *c_bf16, long ldc)
{
    long total = (long)M * (long)N;
#pragma omp parallel for schedule(static)
    for (long idx = 0; idx < total; ++idx) {
        int m = (int)(idx / N);
        int n = (int)(idx % N);
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
            acc += bf16_to_f64(A[(long)m * lda + k]) * bf16_to_f64(W[(long)n * ldw + k]);
        if (R)
            acc += bf16_to_f64(R[(long)m * ldr + n]);
        if (c_exact)
            c_exact[(long)m * ldc + n] = acc;
        if (c_bf16)
            c_bf16[(long)m * ldc + n] = oracle_round_bf16(acc);
    }
}

/* RMSNorm of one latent row (LatentMoERunner docstring, #50089; standard
 * RMSNorm over the whole latent dimension, eps inside the square root):
 *   r = 1 / sqrt( (1/d) * sum_k L[k]^2 + eps ),   n[k] = L[k] * r * gamma[k]. */
static double rms_scale(const uint16_t *Lrow, int d, double eps)
{
    double ss = 0.0;
    for (int k = 0; k < d; ++k) {
        double v = bf16_to_f64(Lrow[k]);
        ss += v * v;
    }
    return 1.0 / sqrt(ss / (double)d + eps);
}

/* Per-row RMSNorm scale r[m] for an [M,d] latent with row stride ldl. */
void oracle_rms_scale(int M, int d, const uint16_t *L, long ldl, double eps, double *r)
{
    for (int m = 0; m < M; ++m)
        r[m] = rms_scale(L + (long)m * ldl, d, eps);
}

/* Latent-MoE tail (LatentMoERunner docstring, #50089):
 *   out[m,j] = round_bf16( S[m,j] + sum_k n[m,k] * Wup[j,k] ),
 *   n[m,k]   = L[m,k] * r[m] * gamma[k].
 * variant 1 rounds n to bf16 before the up-projection: the RMSNorm output is
 * a bf16 tensor that the up-projection GEMM consumes, as in the runner's
 * unfused path (norm, then a bf16 addmm).  This is the reading the library is
 * held to.  variant 0 keeps n in double (the exact-arithmetic value, used to
 * bound how far the two readings can drift apart).  S may be NULL (no
 * shared-expert add).  L is [M,d], Wup is [D,d], S and out are [M,D]; all
 * row-major and contiguous. */
void oracle_latent_tail(int M, int d, int D,
                        const uint16_t *L, const uint16_t *gamma, double eps,
                        const uint16_t *Wup, const uint16_t *S,
                        int variant, double *out_exact, uint16_t *out_bf16)
{
    for (int m = 0; m < M; ++m) {
        const uint16_t *Lrow = L + (long)m * d;
        double r = rms_scale(Lrow, d, eps);
        double nrow[d > 0 ? d : 1];
        for (int k = 0; k < d; ++k) {
            double nk = bf16_to_f64(Lrow[k]) * r * bf16_to_f64(gamma[k]);
            if (variant == 1)
                nk = bf16_to_f64(oracle_round_bf16(nk));
            nrow[k] = nk;
        }
#pragma omp parallel for schedule(static)
        for (int j = 0; j < D; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += nrow[k] * bf16_to_f64(Wup[(long)j * d + k]);
            if (S)
                acc += bf16_to_f64(S[(long)m * D + j]);
            if (out_exact)
                out_exact[(long)m * D + j] = acc;
            if (out_bf16)
                out_bf16[(long)m * D + j] = oracle_round_bf16(acc);
        }
    }
}
