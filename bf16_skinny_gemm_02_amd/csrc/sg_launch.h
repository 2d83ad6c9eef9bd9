// Internal launch interface between the host layer (abi.cpp) and the kernel
// translation units.  Arguments are validated by the caller before any of
// these is invoked; the launchers only pick the template instance and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "skinny_gemm.h"

namespace sg {

// One dot-product problem out[m,n] = sum_k a[m,k] * w[n,k] with one of the
// epilogues below.
struct DotProblem {
  const uint16_t* a;       // [M,K] activations (the latent L when gamma != NULL)
  int64_t lda;
  const uint16_t* w;       // [N,K] weights
  int64_t ldw;
  const uint16_t* res;     // [M,N] residual / shared-expert partial, nullable
  int64_t ldr;
  uint16_t* out;           // [M,N] bf16 output (unused when partial != NULL)
  int64_t ldc;
  int M, N, K;
  // RMSNorm fold (latent-MoE tail, GEMV kernel only): the activation is
  // replaced by bf16(a * r[m] * gamma) with r[m] = rsqrt(mean_k a[m,k]^2 + eps).
  const uint16_t* gamma;   // [K], non-NULL enables the fold
  float eps;
  // Split-K partials: when non-NULL the kernel writes fp32 partial sums
  // partial[s][m][n] (s < k_split) instead of the bf16 output.
  float* partial;
};

// Workspace layout for split-K partials of a [M,N] problem with S splits.
inline size_t partial_floats(int S, int M, int N) { return (size_t)S * M * N; }

hipError_t launch_gemv(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);
hipError_t launch_smallk(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);
hipError_t launch_mfma(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);

// out[m,n] = bf16( sum_{s<S} partial[s][m][n] + res[m,n] ).  The sum runs
// over s = 0..S-1 in order (deterministic).
struct ReduceProblem {
  const float* partial;
  int S, M, N;
  const uint16_t* res;      // nullable
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
};
hipError_t launch_reduce(const ReduceProblem& p, hipStream_t s);

// F_B stage of the KDA F_A/beta -> F_B branch: reduces the F_A/beta split-K
// partials (fixed order), rounds P to bf16, stores beta (and f_a when
// requested), and computes g1 = bf16(f_a @ w_b^T) with f_a held in LDS.
struct FbProblem {
  const float* partial;     // [S][M][n_ab]
  int S, M, n_ab, rank, n_b;
  const uint16_t* w_b;      // [n_b, rank]
  uint16_t* f_a;            // [M, rank], nullable
  uint16_t* beta;           // [M, n_ab - rank]
  uint16_t* g1;             // [M, n_b]
};
hipError_t launch_fab_fb_tail(const FbProblem& p, hipStream_t s);

// RMSNorm of the latent rows into a bf16 buffer: n[m,k] = bf16(L[m,k] * r[m] *
// gamma[k]), r[m] = rsqrt(mean_k L[m,k]^2 + eps).
struct NormProblem {
  const uint16_t* latent;   // [M,d] contiguous
  const uint16_t* gamma;    // [d]
  uint16_t* out;            // [M,d] contiguous
  int M, d;
  float eps;
};
hipError_t launch_rmsnorm(const NormProblem& p, hipStream_t s);

// Largest M * rank the F_B stage keeps in LDS.
constexpr int kFbMaxMRank = 32768;

}  // namespace sg
