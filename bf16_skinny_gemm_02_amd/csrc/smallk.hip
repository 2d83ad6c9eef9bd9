// Small-K GEMV, the F_B stage of the KDA F_A/beta -> F_B branch, the
// fixed-order split-K reduction and the latent RMSNorm (gfx950).
//
// Small K (K <= 256 for skinny_gemm, K = rank = 128 for F_B): a weight row is
// at most 32 chunks of 16 bytes, so a group of G lanes (G = next power of two
// >= K/8) covers one row and a wave covers 64/G rows at once.  Each lane loads
// its weight chunk once and reuses it for every activation row; the G-lane sum
// uses DPP within a 16-lane row (plus a permlane swap for G = 32, 64).
//
// The F_B stage follows "Overlap low-M TP8 KDA projections"
// (run_kda_projection_overlap / run_fab_fb): P = bf16(x @ W_ab^T) is split into
// f_a = P[:, :rank] and beta = P[:, rank:], and the bf16 f_a feeds F_B.  Here
// the F_A/beta kernel leaves fp32 split-K partials; every F_B workgroup sums
// them in the same fixed order (so all agree bit for bit), rounds f_a to bf16
// into LDS and workgroup 0 also stores beta (and f_a if asked).  This replaces
// a separate reduction launch: the F_B kernel is launched anyway.
#include "sg_device.h"
#include "sg_launch.h"

namespace sg {
namespace {

constexpr int kSmallkWaves = 4;

// Sum over aligned groups of G lanes (G a power of two, 1..64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<0xB1>(v);
  if constexpr (G >= 4) v += dpp<0x4E>(v);
  if constexpr (G >= 8) v += dpp<0x141>(v);
  if constexpr (G >= 16) v += dpp<0x140>(v);
  if constexpr (G >= 32) v = xor16_sum(v);
  if constexpr (G >= 64) v = xor32_sum(v);
  return v;
}

struct SmallkArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* w;
  int64_t ldw;
  const uint16_t* res;
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
  int M, N, K;
};

// One row per group of G lanes; lane j of the group holds chunk j of the row.
template <int G>
__global__ __launch_bounds__(kSmallkWaves * kWave) void smallk_kernel(SmallkArgs g) {
  const int lane = lane_id();
  const int j = lane & (G - 1);
  const int rows_per_wave = kWave / G;
  const int n = (static_cast<int>(blockIdx.x) * kSmallkWaves + wave_id()) * rows_per_wave + lane / G;
  const int K8 = g.K >> 3;
  const bool nvalid = n < g.N;
  const bool cvalid = j < K8;
  const u32x4 wv = (nvalid && cvalid) ? load_nt(g.w + static_cast<int64_t>(n) * g.ldw + j * 8) : zero4();
  for (int m = 0; m < g.M; ++m) {
    const u32x4 xv = cvalid ? load_cached(g.a + m * g.lda + j * 8) : zero4();
    float v = group_sum<G>(dot8(xv, wv, 0.f));
    if (nvalid && j == 0) {
      if (g.res != nullptr) v += bf16_to_f32(g.res[m * g.ldr + n]);
      if (g.n_split > 0 && n >= g.n_split)
        g.out2[m * g.ldc2 + (n - g.n_split)] = f32_to_bf16(v);
      else
        g.out[m * g.ldc + n] = f32_to_bf16(v);
    }
  }
}

struct FbArgs {
  const float* partial;
  int S, M, n_ab, rank, n_b;
  const uint16_t* w_b;
  uint16_t* f_a;
  uint16_t* beta;
  uint16_t* g1;
};

// Sum of the S split-K partials p[0], p[plane], ..., in the fixed order
// s = 0, 1, ..., S-1.  Loads go out kSumBatch at a time, so a sum over S
// partials costs ceil(S / kSumBatch) memory round trips, not S.
constexpr int kSumBatch = 16;
constexpr int kRedBatch = 8;  // f32x4 partial loads per straight-line batch per thread
// How reduce_block requests the partials (see there).
constexpr int kRedGroups = 0, kRedPredicated = 1, kRedStraight = 2;
// The F_B launch's reduction role takes kRedStraight up to this many workgroups
// (measured: 0.3 us faster with 128 of them, M = 32; 0.4 us slower with 256).
constexpr int kRedStraightMaxWgs = 128;

__device__ __forceinline__ float sum_splits(const float* p, int64_t plane, int S) {
  float acc = 0.f;
  for (int s = 0; s < S; s += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) v[i] = (s + i < S) ? p[(s + i) * plane] : 0.f;
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i)
      if (s + i < S) acc += v[i];
  }
  return acc;
}

struct ReduceArgs {
  const float* partial;
  int S, M, N;
  const uint16_t* res;
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
};

// Four consecutive elements (flat index over [M][N]) per thread.  The
// residual is requested before the partial sums so the two loads overlap;
// the S partials are summed in the fixed order s = 0..S-1.
// RV (N % 4 == 0): the four elements lie in one row, so their residual
// comes as one aligned-block load (load4_bf16).
template <bool VEC, bool RES, int MODE, bool RV = false>
__device__ __forceinline__ void reduce_block(const ReduceArgs& g, int block) {
  const int64_t total = static_cast<int64_t>(g.M) * g.N;
  const int64_t e0 = (static_cast<int64_t>(block) * 256 + threadIdx.x) * 4;
  if (e0 >= total) return;
  int mm[4], nn[4];
  float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    // Past the end the index is clamped to the last element: it is loaded
    // (a valid address) but neither added nor stored.  Loads outside
    // branches go out together instead of one memory round trip each.
    const int64_t e = min(e0 + v, total - 1);
    mm[v] = static_cast<int>(e / g.N);
    nn[v] = static_cast<int>(e - static_cast<int64_t>(mm[v]) * g.N);
  }
  // RES (g.res != NULL): the residual is requested first, outside any
  // branch, and widened only after the partials are summed, so its loads and
  // the partials' share one memory round trip.
  uint16_t rv[4] = {0, 0, 0, 0};
  if constexpr (RES) {
    if constexpr (RV) {
      load4_bf16(g.res, static_cast<int64_t>(g.M - 1) * g.ldr + g.N,
                 static_cast<int64_t>(mm[0]) * g.ldr + nn[0], true, true, rv);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) rv[v] = g.res[mm[v] * g.ldr + nn[v]];
    }
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (VEC) {
    // total % 4 == 0: every plane starts 16-byte aligned.  Three ways to
    // request the S partials, each adding them in the order s = 0, 1, ...,
    // S-1 (so all give the same bits), chosen by measurement:
    //  * kRedGroups: groups of four requested together, then the remainder
    //    one by one (fewest registers: the many-workgroup reduction role of
    //    the F_B launch at larger M);
    //  * kRedPredicated: predicated groups of four, non-temporal (the
    //    reduction launch: each partial is read once; in the F_B launch's
    //    roles non-temporal loads measured slower);
    //  * kRedStraight: straight-line batches of kRedBatch whose loads are
    //    unconditional (indices past S - 1 repeat the last split) and kept
    //    ahead of the first addition by a scheduling barrier, one memory
    //    round trip per batch (the few-workgroup reduction role at small M,
    //    where its latency is the launch's critical path).
    const f32x4* p = reinterpret_cast<const f32x4*>(g.partial + e0);
    const int64_t plane4 = total / 4;
    if constexpr (MODE == kRedStraight) {
      auto batch = [&](int s0) {
        f32x4 t[kRedBatch];
#pragma unroll
        for (int k = 0; k < kRedBatch; ++k)
          t[k] = p[static_cast<int64_t>(min(s0 + k, g.S - 1)) * plane4];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kRedBatch; ++k)
          if (s0 + k < g.S)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += t[k][v];
      };
      batch(0);
      if (g.S > kRedBatch) batch(kRedBatch);
      for (int s0 = 2 * kRedBatch; s0 < g.S; s0 += kRedBatch) batch(s0);
    } else {
      const int grouped = MODE == kRedPredicated ? g.S : (g.S / 4) * 4;
      for (int s = 0; s < grouped; s += 4) {
        f32x4 t[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          t[k] = (s + k < g.S) ? (MODE == kRedPredicated ? __builtin_nontemporal_load(p + (s + k) * plane4)
                                                         : p[(s + k) * plane4])
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (s + k < g.S)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] += t[k][v];
      }
      for (int s = grouped; s < g.S; ++s) {
        const f32x4 t = p[s * plane4];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += t[v];
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (e0 + v < total) acc[v] = sum_splits(g.partial + e0 + v, total, g.S);
  }
  if constexpr (RES) {
#pragma unroll
    for (int v = 0; v < 4; ++v) r[v] = (e0 + v < total) ? bf16_to_f32(rv[v]) : 0.f;
  }
  // The four outputs in one row of one output: one 8-byte store if aligned.
  if (g.N % 4 == 0 && e0 + 3 < total &&
      !(g.n_split > 0 && nn[0] < g.n_split && nn[0] + 3 >= g.n_split)) {
    uint16_t* dst = (g.n_split > 0 && nn[0] >= g.n_split)
                        ? g.out2 + mm[0] * g.ldc2 + (nn[0] - g.n_split)
                        : g.out + mm[0] * g.ldc + nn[0];
    if ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
      float v4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) v4[v] = RES ? acc[v] + r[v] : acc[v];
      uint2 packed;
      packed.x = pack_bf16x2(v4[0], v4[1]);
      packed.y = pack_bf16x2(v4[2], v4[3]);
      *reinterpret_cast<uint2*>(dst) = packed;
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (e0 + v >= total) break;
    const float val = RES ? acc[v] + r[v] : acc[v];
    if (g.n_split > 0 && nn[v] >= g.n_split)
      g.out2[mm[v] * g.ldc2 + (nn[v] - g.n_split)] = f32_to_bf16(val);
    else
      g.out[mm[v] * g.ldc + nn[v]] = f32_to_bf16(val);
  }
}

template <bool VEC, bool RES, bool RV = false>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs g) {
  reduce_block<VEC, RES, kRedPredicated, RV>(g, static_cast<int>(blockIdx.x));
}

// Rows of w_b one F_B workgroup covers: one row per group of G lanes, every
// lane of the workgroup busy, a single pass.
template <int G>
constexpr int fb_rows_per_wg() { return kSmallkWaves * (kWave / G); }

// P elements one F_B thread forms per pass (4 rows x 136 columns = 544 fit in
// one pass of 256 threads x 3).
constexpr int kFbPer = 3;
// Splits the F_B stage requests per batch when it sums the F_A/beta partials.
constexpr int kFbBatch = 8;

// Workgroup (x, y) computes g1 rows [x*R, (x+1)*R), R = fb_rows_per_wg<G>(),
// for activation rows [y*kFbMGroup, (y+1)*kFbMGroup).  Its w_b chunk is
// requested first, so that load overlaps forming P: the rows' bf16 P (the
// F_A/beta partials summed in fixed order, so every workgroup agrees bit for
// bit); f_a goes to LDS, and workgroups with x == 0 also store beta (and
// f_a).
//
// RED (0 none, 1 vector, 2 scalar, 3 vector straight-line): the first red_wgs workgroups instead run
// the split-K reduction of another problem (the Q/K/V/G projection that ran
// beside F_A/beta), so both epilogues take one launch.
template <int G, int RED>
__global__ __launch_bounds__(kSmallkWaves * kWave) void fab_fb_tail_kernel(FbArgs g, ReduceArgs red,
                                                                           int red_wgs, int fbx) {
  __shared__ __attribute__((aligned(16))) uint16_t fa_lds[kFbMGroup * kFbMaxRank];
  int b = static_cast<int>(blockIdx.x);
  if constexpr (RED != 0) {
    if (b < red_wgs) {
      // The projection's rows: no residual.
      reduce_block<RED != 2, false, RED == 3 ? kRedStraight : kRedGroups>(red, b);
      return;
    }
    b -= red_wgs;
  }
  const int bx = b % fbx;
  const int by = b / fbx;
  const int tid = static_cast<int>(threadIdx.x);
  const int nthreads = kSmallkWaves * kWave;
  const int64_t plane = static_cast<int64_t>(g.M) * g.n_ab;
  const int m0 = by * kFbMGroup;
  const int mg = min(kFbMGroup, g.M - m0);
  const bool first = bx == 0;

  const int lane = lane_id();
  const int j = lane & (G - 1);
  const int K8 = g.rank >> 3;
  const bool cvalid = j < K8;
  const int i = bx * fb_rows_per_wg<G>() + wave_id() * (kWave / G) + lane / G;
  const bool ivalid = i < g.n_b;
  const u32x4 wv =
      (ivalid && cvalid) ? load_nt(g.w_b + static_cast<int64_t>(i) * g.rank + j * 8) : zero4();

  // 1. P = bf16(sum_s partial[s][m][j]) for this workgroup's rows; all n_ab
  //    columns in the first column of workgroups, the rank f_a columns
  //    elsewhere.  kFbPer elements per thread per pass.  The first pass
  //    (every element when mg * cols <= kFbPer * nthreads, the usual case)
  //    is straight-line code for up to kSumBatch splits: batches of kFbBatch
  //    splits whose loads go out together (the first behind the w_b load),
  //    one memory round trip per batch.  Past the end of the rows a thread
  //    loads element 0 (in bounds) and discards it.  More splits, or a
  //    second pass, take the loop below.
  const int cols = first ? g.n_ab : g.rank;
  const int count = mg * cols;
  auto place = [&](int idx, uint16_t b) {
    if (idx >= count) return;
    const int mm = idx / cols, jj = idx - mm * cols;
    const int m = m0 + mm;
    if (jj < g.rank) {
      fa_lds[mm * g.rank + jj] = b;
      if (first && g.f_a != nullptr) g.f_a[static_cast<int64_t>(m) * g.rank + jj] = b;
    } else {
      g.beta[static_cast<int64_t>(m) * (g.n_ab - g.rank) + (jj - g.rank)] = b;
    }
  };
  auto element = [&](int idx) -> int64_t {
    if (idx >= count) return 0;
    const int mm = idx / cols, jj = idx - mm * cols;
    return static_cast<int64_t>(m0 + mm) * g.n_ab + jj;
  };
  int base = 0;
  if (g.S <= kSumBatch) {
    int64_t off[kFbPer];
#pragma unroll
    for (int e = 0; e < kFbPer; ++e) off[e] = element(e * nthreads + tid);
    uint16_t b[kFbPer];
    {
      // Splits in two straight-line batches of kFbBatch (the second only
      // when S > kFbBatch); a batch's loads are unconditional (split indices
      // past S - 1 repeat the last one) and the scheduling barrier keeps
      // every load of a batch ahead of its first addition.  The additions
      // run in the order s = 0, 1, ..., S-1.
      float acc[kFbPer] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < kSumBatch / kFbBatch; ++h) {
        if (h > 0 && g.S <= h * kFbBatch) break;
        float v[kFbPer][kFbBatch];
#pragma unroll
        for (int i = 0; i < kFbBatch; ++i) {
          const int64_t si = min(h * kFbBatch + i, g.S - 1);
#pragma unroll
          for (int e = 0; e < kFbPer; ++e) v[e][i] = g.partial[off[e] + si * plane];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < kFbPer; ++e)
#pragma unroll
          for (int i = 0; i < kFbBatch; ++i)
            if (h * kFbBatch + i < g.S) acc[e] += v[e][i];
      }
#pragma unroll
      for (int e = 0; e < kFbPer; ++e) b[e] = f32_to_bf16(acc[e]);
    }
#pragma unroll
    for (int e = 0; e < kFbPer; ++e) place(e * nthreads + tid, b[e]);
    base = kFbPer * nthreads;
  }
  for (; base < count; base += kFbPer * nthreads) {
    uint16_t b[kFbPer];
#pragma unroll
    for (int e = 0; e < kFbPer; ++e) {
      const int idx = base + e * nthreads + tid;
      b[e] = 0;
      if (idx < count) b[e] = f32_to_bf16(sum_splits(g.partial + element(idx), plane, g.S));
    }
#pragma unroll
    for (int e = 0; e < kFbPer; ++e) place(base + e * nthreads + tid, b[e]);
  }
  __syncthreads();

  // 2. g1[m, i] = bf16(sum_r f_a[m, r] * w_b[i, r]): the weight chunk is used
  //    for every activation row of the group.
  for (int mm = 0; mm < mg; ++mm) {
    const u32x4 xv = cvalid ? *reinterpret_cast<const u32x4*>(fa_lds + mm * g.rank + j * 8) : zero4();
    const float v = group_sum<G>(dot8(xv, wv, 0.f));
    if (ivalid && j == 0) g.g1[static_cast<int64_t>(m0 + mm) * g.n_b + i] = f32_to_bf16(v);
  }
}

// One workgroup per latent row.  The row and gamma are loaded once, into
// registers (up to kNormChunks 16-byte chunks per thread, d <= 8192), then
// the sum of squares in a fixed-order tree (per-thread order, wave
// butterfly, the four wave sums in order) and the bf16 output.
constexpr int kNormChunks = 4;

__global__ __launch_bounds__(256) void rmsnorm_kernel(NormProblem p) {
  __shared__ float wsum[4];
  const int m = static_cast<int>(blockIdx.x);
  const uint16_t* row = p.latent + static_cast<int64_t>(m) * p.d;
  uint16_t* orow = p.out + static_cast<int64_t>(m) * p.d;
  const int d8 = p.d >> 3;
  const int tid = static_cast<int>(threadIdx.x);
  u32x4 v[kNormChunks], gv[kNormChunks];
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = tid + 256 * i;
    v[i] = c < d8 ? load_cached(row + c * 8) : zero4();
    gv[i] = c < d8 ? load_cached(p.gamma + c * 8) : zero4();
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float l0 = bf16_lo(v[i][q]), l1 = bf16_hi(v[i][q]);
      ss = fmaf(l0, l0, ss);
      ss = fmaf(l1, l1, ss);
    }
  ss = wave_allreduce(ss);
  if (lane_id() == 0) wsum[wave_id()] = ss;
  __syncthreads();
  const float total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float r = __frsqrt_rn(total / static_cast<float>(p.d) + p.eps);
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = tid + 256 * i;
    if (c >= d8) break;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(bf16_lo(v[i][q]) * r * bf16_lo(gv[i][q]), bf16_hi(v[i][q]) * r * bf16_hi(gv[i][q]));
    *reinterpret_cast<u32x4*>(orow + c * 8) = o;
  }
}

int lanes_for(int K8) {
  int G = 1;
  while (G < K8) G <<= 1;
  return G;
}

template <int G>
hipError_t launch_smallk_g(const SmallkArgs& g, hipStream_t s) {
  const int rows_per_wg = kSmallkWaves * (kWave / G);
  const dim3 grid((g.N + rows_per_wg - 1) / rows_per_wg);
  return launch_kernel(smallk_kernel<G>, grid, dim3(kSmallkWaves * kWave), 0, s, g);
}

template <int G>
hipError_t launch_fb_g(const FbArgs& g, const ReduceArgs& r, int red_wgs, int red_mode, hipStream_t s) {
  // At least one column of workgroups: it also stores beta and f_a.
  constexpr int R = fb_rows_per_wg<G>();
  const int bx = (g.n_b + R - 1) / R;
  const int fbx = bx > 0 ? bx : 1;
  const int fby = (g.M + kFbMGroup - 1) / kFbMGroup;
  const dim3 grid(red_wgs + fbx * fby);
  const dim3 block(kSmallkWaves * kWave);
  switch (red_mode) {
    case 1: return launch_kernel(fab_fb_tail_kernel<G, 1>, grid, block, 0, s, g, r, red_wgs, fbx);
    case 2: return launch_kernel(fab_fb_tail_kernel<G, 2>, grid, block, 0, s, g, r, red_wgs, fbx);
    case 3: return launch_kernel(fab_fb_tail_kernel<G, 3>, grid, block, 0, s, g, r, red_wgs, fbx);
    default: return launch_kernel(fab_fb_tail_kernel<G, 0>, grid, block, 0, s, g, r, red_wgs, fbx);
  }
}

int reduce_blocks(const ReduceProblem& p) {
  const int64_t total = static_cast<int64_t>(p.M) * p.N;
  return static_cast<int>((total + 1023) / 1024);
}

bool reduce_vec(const ReduceProblem& p) {
  const int64_t total = static_cast<int64_t>(p.M) * p.N;
  return (total % 4) == 0 && (reinterpret_cast<uintptr_t>(p.partial) & 15u) == 0;
}

ReduceArgs reduce_args(const ReduceProblem& p) {
  return ReduceArgs{p.partial, p.S, p.M, p.N, p.res, p.ldr, p.out, p.ldc, p.out2, p.ldc2, p.n_split};
}

}  // namespace

hipError_t launch_smallk(const DotProblem& p, const sg_config_t& cfg, hipStream_t s) {
  (void)cfg;
  SmallkArgs g{p.a,    p.lda,  p.w,       p.ldw, p.res, p.ldr, p.out,
               p.ldc,  p.out2, p.ldc2,    p.n_split, p.M, p.N, p.K};
  switch (lanes_for(p.K >> 3)) {
    case 1: return launch_smallk_g<1>(g, s);
    case 2: return launch_smallk_g<2>(g, s);
    case 4: return launch_smallk_g<4>(g, s);
    case 8: return launch_smallk_g<8>(g, s);
    case 16: return launch_smallk_g<16>(g, s);
    case 32: return launch_smallk_g<32>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fab_fb_tail(const FbProblem& p, hipStream_t s) {
  if (p.partial == nullptr || p.S < 1) return hipErrorInvalidValue;
  FbArgs g{p.partial, p.S, p.M, p.n_ab, p.rank, p.n_b, p.w_b, p.f_a, p.beta, p.g1};
  ReduceArgs r{};
  int red_wgs = 0, red_mode = 0;
  if (p.red != nullptr && p.red->res != nullptr) return hipErrorInvalidValue;  // no residual role
  if (p.red != nullptr && reduce_blocks(*p.red) > 0) {
    r = reduce_args(*p.red);
    red_wgs = reduce_blocks(*p.red);
    red_mode = reduce_vec(*p.red) ? (red_wgs <= kRedStraightMaxWgs ? 3 : 1) : 2;
  }
  switch (lanes_for(p.rank >> 3)) {
    case 1: return launch_fb_g<1>(g, r, red_wgs, red_mode, s);
    case 2: return launch_fb_g<2>(g, r, red_wgs, red_mode, s);
    case 4: return launch_fb_g<4>(g, r, red_wgs, red_mode, s);
    case 8: return launch_fb_g<8>(g, r, red_wgs, red_mode, s);
    case 16: return launch_fb_g<16>(g, r, red_wgs, red_mode, s);
    case 32: return launch_fb_g<32>(g, r, red_wgs, red_mode, s);
    case 64: return launch_fb_g<64>(g, r, red_wgs, red_mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const ReduceProblem& p, hipStream_t s) {
  const int blocks = reduce_blocks(p);
  if (blocks < 1) return hipSuccess;
  const ReduceArgs g = reduce_args(p);
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool res = p.res != nullptr;
  if (res && p.N % 4 == 0)
    return reduce_vec(p) ? launch_kernel(reduce_kernel<true, true, true>, grid, dim3(256), 0, s, g)
                         : launch_kernel(reduce_kernel<false, true, true>, grid, dim3(256), 0, s, g);
  if (reduce_vec(p))
    return res ? launch_kernel(reduce_kernel<true, true>, grid, dim3(256), 0, s, g)
               : launch_kernel(reduce_kernel<true, false>, grid, dim3(256), 0, s, g);
  return res ? launch_kernel(reduce_kernel<false, true>, grid, dim3(256), 0, s, g)
             : launch_kernel(reduce_kernel<false, false>, grid, dim3(256), 0, s, g);
}

hipError_t launch_rmsnorm(const NormProblem& p, hipStream_t s) {
  if ((p.d >> 3) > 256 * kNormChunks) return hipErrorInvalidValue;
  return launch_kernel(rmsnorm_kernel, dim3(static_cast<unsigned>(p.M)), dim3(256), 0, s, p);
}

}  // namespace sg
