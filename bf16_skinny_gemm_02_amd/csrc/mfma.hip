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
// wave; each wave keeps a ring of D k-steps of weight and activation
// fragments in flight.  The four wave partials are summed through LDS in the
// fixed order 0,1,2,3, so results do not depend on timing.
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
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
  int M, N, K;
  int row_origin;  // absolute index of weight row 0 (sets the k-order rotation)
  int sps;  // k-steps per split
};

constexpr int kMfmaWaves = 4;
constexpr int kKStep = 32;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int MB, int NB, int D, int NKT>
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
  const int nk = max(0, w_end - w_begin);

  // Buffer resources: the workgroup's weight tile and the activation.  A
  // row past N or M, a chunk past K and a step past the wave's range all map
  // to kOob and read as zero.
  const int tile_rows = min(16 * NB, g.N - n_base);
  const rsrc_t wres = make_rsrc(g.w + static_cast<int64_t>(n_base) * g.ldw,
                                static_cast<uint32_t>(((tile_rows - 1) * g.ldw + g.K) * 2));
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
  uint32_t wbase[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = 16 * b + rl;
    wbase[b] = row < tile_rows ? static_cast<uint32_t>(row * g.ldw * 2) : kOob;
  }
  uint32_t xbase[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int m = 16 * a + rl;
    xbase[a] = m < g.M ? static_cast<uint32_t>(m * g.lda * 2) : kOob;
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of D k-steps: weight and activation fragments of step t are issued
  // together, D steps before they are consumed, so waiting for one step never
  // waits on a load issued for a later step.  No load sits in a branch.
  // Every workgroup reads the same activation lines; if all of them walked K
  // in the same order they would request the same lines at the same moment
  // and queue at one L2 channel.  Each wave therefore starts its K-range at
  // an offset set by its absolute 16-row tile (workgroups of one XCD are 8
  // tiles apart) and wraps around.  The offset depends only on which rows the
  // tile holds, so a row's sum is formed in the same order in every launch.
  const int tile = (g.row_origin + n_base) >> 4;
  const int rot = nk > 0 ? ((tile >> 3) * 23 + (tile & 7) * 7) % nk : 0;
  auto koff = [&](int t) -> uint32_t {
    int tt = t + rot;
    tt = tt >= nk ? tt - nk : tt;
    const int c = (w_begin + tt) * 4 + kg;
    return (t < nk && c < K8) ? static_cast<uint32_t>(c * 16) : kOob;
  };
  auto wfrag = [&](uint32_t ko, int b) -> u32x4 {
    return buf_load_nt(wres, (ko == kOob || wbase[b] == kOob) ? kOob : wbase[b] + ko);
  };
  auto xfrag = [&](uint32_t ko, int a) -> u32x4 {
    return buf_load(xres, (ko == kOob || xbase[a] == kOob) ? kOob : xbase[a] + ko);
  };

  u32x4 wr[D][NB];
  u32x4 xr[D][MB];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const uint32_t ko = koff(j);
#pragma unroll
    for (int b = 0; b < NB; ++b) wr[j][b] = wfrag(ko, b);
#pragma unroll
    for (int a = 0; a < MB; ++a) xr[j][a] = xfrag(ko, a);
  }

  // One ring pass: consume slot j, refill it with the step D ahead, in
  // program order, so the loads complete in the order the steps need them.
  auto pass = [&](int tb) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int t = tb + j;
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = mfma16(wr[j][b], xr[j][a], acc[a][b]);
      const uint32_t ko = koff(t + D);
#pragma unroll
      for (int b = 0; b < NB; ++b) wr[j][b] = wfrag(ko, b);
#pragma unroll
      for (int a = 0; a < MB; ++a) xr[j][a] = xfrag(ko, a);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (NKT > 0) {
    // Known step count: straight-line code, so every wait is exact (a loop
    // head would merge the pending-load state of two paths and drain).
#pragma unroll
    for (int tb = 0; tb < NKT; tb += D) pass(tb);
  } else {
    for (int tb = 0; tb < nk; tb += D) pass(tb);
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
          if (g.n_split > 0 && n >= g.n_split)
            g.out2[m * g.ldc2 + (n - g.n_split)] = f32_to_bf16(val);
          else
            g.out[m * g.ldc + n] = f32_to_bf16(val);
        }
      }
  }
}

// Ring depth: the weight fragment plus MB activation fragments per k-step,
// D steps deep, within the register budget of one wave per SIMD.
template <int MB>
constexpr int ring_depth() {
  return MB <= 2 ? 12 : (MB <= 4 ? 8 : (MB <= 8 ? 4 : 2));
}

template <int MB>
hipError_t launch_mb(const MfmaArgs& g, int NB, int per_wave, dim3 grid, hipStream_t s) {
  if (NB != 1) return hipErrorInvalidValue;
  constexpr int D = ring_depth<MB>();
  // Straight-line instances for the per-wave step counts of the model's
  // shapes (K = 7168 and K = 2048 without a split); a loop otherwise.
  if (per_wave > 16 && per_wave <= 56)
    hipLaunchKernelGGL((mfma_kernel<MB, 1, D, 56>), grid, dim3(kMfmaWaves * kWave), 0, s, g);
  else if (per_wave <= 16)
    hipLaunchKernelGGL((mfma_kernel<MB, 1, D, 16>), grid, dim3(kMfmaWaves * kWave), 0, s, g);
  else
    hipLaunchKernelGGL((mfma_kernel<MB, 1, D, 0>), grid, dim3(kMfmaWaves * kWave), 0, s, g);
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
  g.out2 = p.out2;
  g.ldc2 = p.ldc2;
  g.n_split = p.n_split;
  g.M = p.M;
  g.N = p.N;
  g.K = p.K;
  g.row_origin = p.row_origin;
  const int KS = (p.K + kKStep - 1) / kKStep;
  const int S = cfg.k_split > 0 ? cfg.k_split : 1;
  g.sps = (KS + S - 1) / S;
  if (g.sps < 1) g.sps = 1;
  const int MB = cfg.m_tile / 16;
  const int NB = cfg.rows;
  const int rows_per_wg = 16 * NB;
  const dim3 grid((p.N + rows_per_wg - 1) / rows_per_wg, S);
  const int per_wave = (g.sps + kMfmaWaves - 1) / kMfmaWaves;
  switch (MB) {
#define SG_CASE(mb) \
  case mb: return launch_mb<mb>(g, NB, per_wave, grid, s);
    SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
    SG_CASE(9) SG_CASE(10) SG_CASE(11) SG_CASE(12) SG_CASE(13) SG_CASE(14) SG_CASE(15) SG_CASE(16)
#undef SG_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sg
