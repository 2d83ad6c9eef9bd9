// bf16 MFMA tile path for 16 < M <= 256 (gfx950, v_mfma_f32_16x16x32_bf16).
//
// out[m,n] = sum_k a[m,k] * w[n,k] is a dense contraction once M exceeds a
// GEMV's handful of rows, so it goes to the matrix cores.  Operand layout of
// the 16x16x32 instruction: lane l supplies row (l % 16) and the eight
// consecutive k of group (l / 16) of the 16x32 A operand, and the same for
// the columns of B; lane l receives D[4*(l/16) + v][l % 16], v = 0..3.
// Because the weights are [N,K] with K contiguous, a lane's eight k of one
// weight row are one 16-byte global load, so the A operand (weights, rows =
// n) is loaded straight from HBM into registers in MFMA order -- no LDS
// transpose.  The B operand is the activation (columns = m), loaded the same
// way from the cache.  D[n][m] then gives each lane four consecutive n of one
// output row.
//
// Workgroup = 4 waves on one 16*NB-row weight tile.  The workgroup's K-range
// (all of K, or 1/k_split of it) is cut into 4 contiguous pieces, one per
// wave; each wave keeps U k-steps of weights in flight.  The four wave
// partials are summed through LDS in the fixed order 0,1,2,3, so results do
// not depend on timing.
//
// The latent-MoE tail reaches this kernel with its activation already
// normalised (bf16 RMSNorm output from the norm kernel), so the epilogue only
// adds the shared-expert partial.
#include "sg_device.h"
#include "sg_launch.h"

namespace sg {
namespace {

struct MfmaArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* w;
  int64_t ldw;
  const uint16_t* res;
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
  float* partial;
  int M, N, K;
  int sps;  // k-steps per split
};

constexpr int kMfmaWaves = 4;
constexpr int kKStep = 32;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int MB, int NB, int U>
__global__ __launch_bounds__(kMfmaWaves * kWave) void mfma_kernel(MfmaArgs g) {
  constexpr int kRegs = MB * NB * 4;
  __shared__ float red[(kMfmaWaves - 1) * kRegs * kWave];

  const int lane = lane_id();
  const int wave = wave_id();
  const int rl = lane & 15;
  const int kg = lane >> 4;
  const int n_base = static_cast<int>(blockIdx.x) * 16 * NB;
  const int K8 = g.K >> 3;
  const int KS = (g.K + kKStep - 1) / kKStep;
  const int s_begin = static_cast<int>(blockIdx.y) * g.sps;
  const int s_end = min(KS, s_begin + g.sps);
  const int len = max(0, s_end - s_begin);
  const int per = (len + kMfmaWaves - 1) / kMfmaWaves;
  const int w_begin = s_begin + wave * per;
  const int w_end = min(s_end, w_begin + per);

  const uint16_t* wrow[NB];
  bool nvalid[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n = n_base + 16 * b + rl;
    nvalid[b] = n < g.N;
    wrow[b] = g.w + static_cast<int64_t>(nvalid[b] ? n : 0) * g.ldw;
  }
  const uint16_t* arow[MB];
  bool mvalid[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int m = 16 * a + rl;
    mvalid[a] = m < g.M;
    arow[a] = g.a + static_cast<int64_t>(mvalid[a] ? m : 0) * g.lda;
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ks0 = w_begin; ks0 < w_end; ks0 += U) {
    u32x4 wv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (ks0 + u) * 4 + kg;
      const bool ok = (ks0 + u < w_end) && (c < K8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        wv[u][b] = (ok && nvalid[b]) ? load_nt(wrow[b] + static_cast<int64_t>(c) * 8) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (ks0 + u) * 4 + kg;
      const bool ok = (ks0 + u < w_end) && (c < K8);
      u32x4 xv[MB];
#pragma unroll
      for (int a = 0; a < MB; ++a)
        xv[a] = (ok && mvalid[a]) ? load_cached(arow[a] + static_cast<int64_t>(c) * 8) : zero4();
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = mfma16(wv[u][b], xv[a], acc[a][b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Fixed-order sum of the four wave partials.
  if (wave > 0) {
    float* dst = red + (wave - 1) * kRegs * kWave;
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[((a * NB + b) * 4 + v) * kWave + lane] = acc[a][b][v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kMfmaWaves - 1; ++w) {
    const float* src = red + w * kRegs * kWave;
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[a][b][v] += src[((a * NB + b) * 4 + v) * kWave + lane];
  }

  if (g.partial != nullptr) {
    const int64_t s = blockIdx.y;
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      const int m = 16 * a + rl;
      if (m >= g.M) continue;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = n_base + 16 * b + 4 * kg + v;
          if (n < g.N) g.partial[(s * g.M + m) * g.N + n] = acc[a][b][v];
        }
    }
    return;
  }

#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int m = 16 * a + rl;
    if (m >= g.M) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = n_base + 16 * b + 4 * kg + v;
        if (n < g.N) {
          float val = acc[a][b][v];
          if (g.res != nullptr) val += bf16_to_f32(g.res[m * g.ldr + n]);
          g.out[m * g.ldc + n] = f32_to_bf16(val);
        }
      }
  }
}

template <int MB>
hipError_t launch_mb(const MfmaArgs& g, int NB, dim3 grid, hipStream_t s) {
  if (NB != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mfma_kernel<MB, 1, 8>), grid, dim3(kMfmaWaves * kWave), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const DotProblem& p, const sg_config_t& cfg, hipStream_t s) {
  MfmaArgs g;
  g.a = p.a;
  g.lda = p.lda;
  g.w = p.w;
  g.ldw = p.ldw;
  g.res = p.res;
  g.ldr = p.ldr;
  g.out = p.out;
  g.ldc = p.ldc;
  g.partial = p.partial;
  g.M = p.M;
  g.N = p.N;
  g.K = p.K;
  const int KS = (p.K + kKStep - 1) / kKStep;
  const int S = cfg.k_split > 0 ? cfg.k_split : 1;
  g.sps = (KS + S - 1) / S;
  if (g.sps < 1) g.sps = 1;
  const int MB = cfg.m_tile / 16;
  const int NB = cfg.rows;
  const int rows_per_wg = 16 * NB;
  const dim3 grid((p.N + rows_per_wg - 1) / rows_per_wg, S);
  switch (MB) {
#define SG_CASE(mb) \
  case mb: return launch_mb<mb>(g, NB, grid, s);
    SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
    SG_CASE(9) SG_CASE(10) SG_CASE(11) SG_CASE(12) SG_CASE(13) SG_CASE(14) SG_CASE(15) SG_CASE(16)
#undef SG_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sg
