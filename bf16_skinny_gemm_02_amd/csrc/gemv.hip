// Row-parallel and split-K GEMV for M <= 16 (gfx950).
//
// out[m,n] = sum_k a[m,k] * w[n,k]  for a handful of activation rows m, the
// decode-time projection of "Kimi K3 support, phase 1" (CuteSkinnyGemm, where
// M is fixed at compile time and fully unrolled) and the F_A/beta small-N
// projection of "Overlap low-M TP8 KDA projections" (_KdaSkinnyNGemm, which
// splits the work finely because N is small).
//
// Mapping: one wave owns R consecutive weight rows and a range of K.  The 64
// lanes cover 64 consecutive 16-byte chunks of each row per step (one fully
// coalesced 1 KiB global_load_dwordx4 per row), so a step covers 512 K.  Each
// lane keeps U steps of weight chunks in flight (non-temporal loads), reads the
// matching activation chunks through the cache (they are shared by every
// wave), and accumulates acc[m][r] in fp32 with v_dot2c_f32_bf16.  The 64
// per-lane partial sums are then combined with a DPP / permlane butterfly and
// lane (m*R + r) stores output (m, r).  No LDS and no barriers.
//
// Split-K (grid.y > 1): wave (row group, s) covers steps
// [s*sps, (s+1)*sps) and stores fp32 partials for a later fixed-order sum.
//
// Fold (latent-MoE tail, RMSNorm -> up-projection): the activation is the
// latent L.  The wave first sums L[m,k]^2 over the whole row (its lanes hold
// every chunk of it), forms r[m] = rsqrt(sum / K + eps), and then feeds the
// dot product with n = bf16(L * r * gamma), the bf16 normalised latent the
// up-projection consumes.  One launch, no workspace.
#include "sg_device.h"
#include "sg_launch.h"

namespace sg {
namespace {

struct GemvArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* w;
  int64_t ldw;
  const uint16_t* res;
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
  const uint16_t* gamma;
  float* partial;
  int N, K;
  int sps;  // steps per split
  float eps;
};

constexpr int kGemvWaves = 4;

template <int M, int R, int U, bool FOLD>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_kernel(GemvArgs g) {
  const int lane = lane_id();
  const int n0 = (static_cast<int>(blockIdx.x) * kGemvWaves + wave_id()) * R;
  if (n0 >= g.N) return;  // wave-uniform; the kernel uses no barriers

  const int K8 = g.K >> 3;
  const int nsteps = (K8 + kWave - 1) / kWave;
  const int s_begin = static_cast<int>(blockIdx.y) * g.sps;
  const int s_end = min(nsteps, s_begin + g.sps);

  const uint16_t* wrow[R];
  bool rvalid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rvalid[r] = (n0 + r) < g.N;
    wrow[r] = g.w + static_cast<int64_t>(rvalid[r] ? n0 + r : n0) * g.ldw;
  }

  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.f;

  // RMSNorm scale of each latent row over the full K (every split needs it).
  float rscale[M];
  if constexpr (FOLD) {
#pragma unroll
    for (int m = 0; m < M; ++m) rscale[m] = 0.f;
    for (int st = 0; st < nsteps; ++st) {
      const int c = st * kWave + lane;
      if (c < K8) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 lv = load_cached(g.a + m * g.lda + static_cast<int64_t>(c) * 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float l0 = bf16_lo(lv[i]), l1 = bf16_hi(lv[i]);
            rscale[m] = fmaf(l0, l0, rscale[m]);
            rscale[m] = fmaf(l1, l1, rscale[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
      rscale[m] = __frsqrt_rn(wave_allreduce(rscale[m]) / static_cast<float>(g.K) + g.eps);
  }

  for (int s0 = s_begin; s0 < s_end; s0 += U) {
    u32x4 wv[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (s0 + u) * kWave + lane;
      const bool ok = (s0 + u < s_end) && (c < K8);
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[u][r] = (ok && rvalid[r]) ? load_nt(wrow[r] + static_cast<int64_t>(c) * 8) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (s0 + u) * kWave + lane;
      const bool ok = (s0 + u < s_end) && (c < K8);
      u32x4 xv[M];
#pragma unroll
      for (int m = 0; m < M; ++m)
        xv[m] = ok ? load_cached(g.a + m * g.lda + static_cast<int64_t>(c) * 8) : zero4();
      if constexpr (FOLD) {
        const u32x4 gv = ok ? load_cached(g.gamma + static_cast<int64_t>(c) * 8) : zero4();
#pragma unroll
        for (int m = 0; m < M; ++m) {
          u32x4 nv;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            nv[i] = pack_bf16x2(bf16_lo(xv[m][i]) * rscale[m] * bf16_lo(gv[i]),
                                bf16_hi(xv[m][i]) * rscale[m] * bf16_hi(gv[i]));
          xv[m] = nv;
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = dot8(xv[m], wv[u][r], acc[m][r]);
      // Keep the next step's activation loads below this point: only one
      // step of activation chunks is live at a time.
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Cross-lane sums: every lane ends up with every (m, r) total.
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_allreduce(acc[m][r]);

  if (g.partial != nullptr) {
    // Lane j stores partial (m, r) = (j / R, j % R).
    float v = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) v = (lane == m * R + r) ? acc[m][r] : v;
    if (lane < M * R) {
      const int m = lane / R, r = lane % R;
      if (n0 + r < g.N)
        g.partial[(static_cast<int64_t>(blockIdx.y) * M + m) * g.N + n0 + r] = v;
    }
    return;
  }

  float v = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) v = (lane == m * R + r) ? acc[m][r] : v;
  if (lane < M * R) {
    const int m = lane / R, r = lane % R;
    const int n = n0 + r;
    if (n < g.N) {
      if (g.res != nullptr) v += bf16_to_f32(g.res[m * g.ldr + n]);
      g.out[m * g.ldc + n] = f32_to_bf16(v);
    }
  }
}

// Steps of 16-byte chunks each lane keeps in flight: R * U = 16 chunks
// (64 VGPRs of weights).
template <int R>
constexpr int unroll_for() { return 16 / R; }

template <int M, int R, bool FOLD>
hipError_t launch_mr(const GemvArgs& g, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<M, R, unroll_for<R>(), FOLD>), grid, dim3(kGemvWaves * kWave), 0,
                     s, g);
  return hipGetLastError();
}

template <int M, bool FOLD>
hipError_t launch_m(const GemvArgs& g, int R, dim3 grid, hipStream_t s) {
  switch (R) {
    case 1: return launch_mr<M, 1, FOLD>(g, grid, s);
    case 2: return launch_mr<M, 2, FOLD>(g, grid, s);
    case 4: return launch_mr<M, 4, FOLD>(g, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool FOLD>
hipError_t launch_fold(const GemvArgs& g, int M, int R, dim3 grid, hipStream_t s) {
  switch (M) {
#define SG_CASE(mm) \
  case mm: return launch_m<mm, FOLD>(g, R, grid, s);
    SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
    SG_CASE(9) SG_CASE(10) SG_CASE(11) SG_CASE(12) SG_CASE(13) SG_CASE(14) SG_CASE(15) SG_CASE(16)
#undef SG_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(const DotProblem& p, const sg_config_t& cfg, hipStream_t s) {
  GemvArgs g;
  g.a = p.a;
  g.lda = p.lda;
  g.w = p.w;
  g.ldw = p.ldw;
  g.res = p.res;
  g.ldr = p.ldr;
  g.out = p.out;
  g.ldc = p.ldc;
  g.gamma = p.gamma;
  g.partial = p.partial;
  g.N = p.N;
  g.K = p.K;
  g.eps = p.eps;
  const int K8 = p.K >> 3;
  const int nsteps = (K8 + kWave - 1) / kWave;
  const int S = cfg.k_split > 0 ? cfg.k_split : 1;
  g.sps = (nsteps + S - 1) / S;
  if (g.sps < 1) g.sps = 1;
  const int rows_per_wg = kGemvWaves * cfg.rows;
  const dim3 grid((p.N + rows_per_wg - 1) / rows_per_wg, S);
  if (p.gamma != nullptr) return launch_fold<true>(g, p.M, cfg.rows, grid, s);
  return launch_fold<false>(g, p.M, cfg.rows, grid, s);
}

}  // namespace sg
