// Internal launch interface between the host layer (abi.cpp) and the kernel
// translation units.  Arguments are validated by the caller before any of
// these is invoked; the launchers only pick the template instance and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "skinny_gemm.h"

namespace sg {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device: `done` is the kernel instance's own table of devices already
// set (static storage, so it starts all false).  Devices past the table are
// set on every call.
constexpr int kLdsAttrDevices = 64;
inline hipError_t ensure_lds_limit(const void* kernel, size_t bytes, std::atomic<bool>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kLdsAttrDevices;
  if (tracked && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess && tracked) done[dev].store(true, std::memory_order_release);
  return e;
}

// Enqueues kern<<<grid, block, lds, s>>>(args...) through hipLaunchKernel
// and returns that call's own status.  (Reading the runtime's last-error
// slot after a launch would also report an error some earlier, unrelated
// call of the caller left there.)
template <typename T>
struct arg_ident {
  using type = T;
};
template <typename... P>
inline hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                                typename arg_ident<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s);
}

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
  // RMSNorm fold (latent-MoE tail; the GEMV kernel at M = 1 and the
  // wave-split MFMA tile): the activation is replaced by
  // bf16((a * r[m]) * gamma) with r[m] = rsqrt(mean_k a[m,k]^2 + eps).
  const uint16_t* gamma;   // [K], non-NULL enables the fold
  float eps;
  // Split-K partials: when non-NULL the kernel writes fp32 partial sums
  // partial[s][m][n] (s < k_split) instead of the bf16 output.
  float* partial;
  // Split output: rows n >= n_split go to out2[m * ldc2 + (n - n_split)]
  // instead of out (used by the packed KDA projection, whose F_A/beta rows
  // form a separate tensor).  n_split <= 0 disables it.
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
  // In-launch hand-off (with `partial`, in a fused launch): the workspace's
  // flag header.  The partials are stored device-coherently and each wave
  // (GEMV) or workgroup (wave-split) then advances its flag, for an F_B role
  // later in the same grid (sg_fused.h).
  unsigned* arrive;
  // In-launch K-split sum (the 4-wave tile kernel with exactly two K splits,
  // bf16 out): the first split's workgroups store their fp32 sums with the
  // call's generation as 8-byte pairs in `pairs` (in thread order, 8 KiB per
  // 16 activation rows of a 64-row tile), the second split's
  // workgroups read them, add them to their own and store the output; the
  // generations live in the hand-off header `sync` (sg_fused.h: zero before
  // the first call on a workspace).  No split-K partials, no second launch.
  uint64_t* pairs;
  unsigned* sync;
};

// The F_B role of a fused launch (see sg_fused.h): workgroups that wait for
// the arrivals of the segment whose `arrive` is set, then sum its partials
// (S of them, [S][M][n_ab]) into bf16 P and compute g1 = bf16(f_a W_b^T).
struct FusedFb {
  const float* partial;     // the arriving segment's partials
  unsigned* sync;           // the workspace's flag header, zero before the first call
  int S, M, n_ab, rank, n_b;
  const uint16_t* w_b;      // [n_b, rank]
  uint16_t* f_a;            // [M, rank], nullable
  uint16_t* beta;           // [M, n_ab - rank]
  uint16_t* g1;             // [M, n_b]
};

// Workspace regions start on 256-byte boundaries.
size_t ws_round(size_t bytes);

// Workspace layout for split-K partials of a [M,N] problem with S splits.
inline size_t partial_floats(int S, int M, int N) { return (size_t)S * M * N; }

// floor(2^32 / d) for the kernels' workgroup-index quotient (2^32 - 1 for
// d = 1): n * floor(2^32/d) / 2^32 falls short of n / d by less than
// n / 2^32 < 1, so its integer part is the quotient or one less, and
// quotient_by() corrects it.
inline unsigned quotient_magic(int d) {
  if (d <= 1) return 0xFFFFFFFFu;
  return static_cast<unsigned>(0x100000000ull / static_cast<unsigned>(d));
}

hipError_t launch_gemv(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);
hipError_t launch_smallk(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);
hipError_t launch_mfma(const DotProblem& p, const sg_config_t& cfg, hipStream_t s);

// Segmented launches: nseg (1 or 2) independent problems in one grid, each
// with its own configuration (k_split, grid); both must name the same kernel
// instance (*_same_instance), which lets two shapes that would each leave the
// chip partly idle, or spill a few workgroups into a second wave, run as one
// wave of work.
bool gemv_same_instance(const sg_config_t& a, const sg_config_t& b);
bool mfma_same_instance(const sg_config_t& a, const sg_config_t& b);
hipError_t launch_gemv(const DotProblem* segs, const sg_config_t* cfgs, int nseg, hipStream_t s);
hipError_t launch_mfma(const DotProblem* segs, const sg_config_t* cfgs, int nseg, hipStream_t s);

// Fused launches: the segments in grid order, plus the F_B role's
// workgroups placed after the first `fb_after` segments (0 <= fb_after <=
// nseg).  Exactly one segment has `arrive` and `partial` set (the F_A/beta
// rows); GEMV instances with 4 waves (M == 1) and the wave-split MFMA tile
// host the role.
hipError_t launch_gemv_fused(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                             const FusedFb& fb, int fb_after, hipStream_t s);
hipError_t launch_mfma_fused(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                             const FusedFb& fb, int fb_after, hipStream_t s);
// Geometry of the one-launch KDA projection's helper wave (sg_help.h): W_ab
// rows per producer unit, 512-k steps per unit at most, K-ranges at most (so
// K <= 8192), the largest M, activation rows and g1 rows per F_B host at
// most, and the largest rank (k-steps of 32 for the MFMA F_B).
constexpr int kHelpRows = 4;
constexpr int kHelpSteps = 4;
constexpr int kHelpMaxS = 4;
constexpr int kHelpMaxM = 16;
constexpr int kHelpHostM = 8;
constexpr int kHelpHostRows = 64;
constexpr int kHelpMaxRank = 128;
// K-ranges of the F_A/beta partials: one unit covers at most kHelpSteps
// steps of 512 k.
inline int help_ranges(int K) {
  const int wsteps = (K / 8 + 63) / 64;
  return (wsteps + kHelpSteps - 1) / kHelpSteps;
}
// A host's P rows in LDS: n_ab columns padded to whole 16-byte pieces, so
// that every row's f_a starts 16-byte aligned for the MFMA operand reads.
__host__ __device__ inline int help_p_stride(int n_ab) { return (n_ab + 7) / 8 * 8; }
// LDS of the helper behind the four rings: a unit's activation rows
// (kHelpSteps KiB per row, 4 * XQ rows), or a host's W_b rows (room for
// kHelpHostRows rows of kHelpMaxRank) and its P [<= kHelpHostM]
// [help_p_stride(n_ab)], all bf16.
inline size_t help_lds_bytes(int M, int rank, int n_ab) {
  (void)rank;
  const size_t xq = static_cast<size_t>((M + 3) / 4);
  const size_t unit = static_cast<size_t>(kHelpSteps) * 4 * xq * 1024;
  const size_t hm = static_cast<size_t>(M < kHelpHostM ? M : kHelpHostM);
  const size_t host = static_cast<size_t>(kHelpHostRows) * kHelpMaxRank * 2 +
                      hm * static_cast<size_t>(help_p_stride(n_ab)) * 2;
  return unit > host ? unit : host;
}

// The one-launch KDA projection: the Q/K/V/G rows of `q` (bf16 out, 16 rows
// per wave-split workgroup over all of K, M <= 16), each workgroup with a
// helper wave that runs the F_A/beta -> F_B chain (sg_help.h).  w_ab [n_ab,K]
// shares q's K; the tagged partials and the hand-off header `sync`
// (zero before the first call) live in the workspace.
struct OneLaunchProj {
  DotProblem q;
  const uint16_t* w_ab;
  int n_ab, rank, n_b;
  const uint16_t* w_b;
  uint16_t* beta;
  uint16_t* g1;
  uint32_t* pairs;   // [S][M][n_ab] (fp32 bits, generation)
  unsigned* sync;
};
// The helper geometry: `groups` units of 4 W_ab rows per K-range, S
// K-ranges of `per` 512-k steps (units = groups * S producer workgroups),
// then `hosts` F_B hosts, row_hosts of host_rows g1 rows for each group of
// kHelpHostM activation rows, all within the wgs Q/K/V/G workgroups.  False
// when the shapes do not fit it.
struct HelpPlan {
  int wgs, groups, S, per, units, hosts, row_hosts, host_rows;
};
bool help_plan(int M, int K, int n_qkvg, int n_ab, int rank, int n_b, HelpPlan* out);
hipError_t launch_proj_one(const OneLaunchProj& p, const HelpPlan& plan, hipStream_t s);

// Bytes at the start of a kda_fab_fb_proj(_fused) workspace that hold the
// hand-off header (4096 producer flags and 512 consumer cursors, uint32);
// the fp32 partials follow.
constexpr size_t kSyncBytes = 18432;

// LDS of the MFMA ring kernels: the shared-activation tile (nw waves, c ring
// slots, 4*xq activation rows) and the wave-split tile (4 private rings).
// The configuration table keeps both within kMfmaMaxLds.
constexpr size_t kMfmaMaxLds = 160 * 1024;
size_t tile_lds_bytes(int nw, int c, int xq);
size_t wsplit_lds_bytes(int c, int xq, bool norm, int nt);
// Whether the wave-split kernel can fold the RMSNorm for this K and K split
// (the launcher's own guard).
bool wsplit_fold_fits(int K, int k_split);
// Whether latent_moe_tail folds the RMSNorm into the GEMM for configuration c
// (the single decision the entry point and the workspace size both use).
bool tail_folds(const sg_config_t& c, int K);
// Whether latent_moe_tail_fused sums the GEMM's two K splits in the launch.
bool tail_tags(const sg_config_t& c, int N);
size_t block_lds_bytes(int c);

// out[m,n] = bf16( sum_{s<S} partial[s][m][n] + res[m,n] ).  The sum runs
// over s = 0..S-1 in order (deterministic).  Columns n >= n_split (when
// n_split > 0) go to out2[m * ldc2 + n - n_split] instead.
struct ReduceProblem {
  const float* partial;
  int S, M, N;
  const uint16_t* res;      // nullable
  int64_t ldr;
  uint16_t* out;
  int64_t ldc;
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
};
hipError_t launch_reduce(const ReduceProblem& p, hipStream_t s);

// F_B stage of the KDA F_A/beta -> F_B branch.  The F_A/beta projection
// P [M, n_ab] arrives as fp32 split-K partials, summed in fixed order.  The
// stage stores beta = P[:, rank:] (and f_a = P[:, :rank] when requested) and
// g1 = bf16(f_a @ w_b^T).
struct FbProblem {
  const float* partial;     // [S][M][n_ab]
  int S, M, n_ab, rank, n_b;
  const uint16_t* w_b;      // [n_b, rank]
  uint16_t* f_a;            // [M, rank], nullable
  uint16_t* beta;           // [M, n_ab - rank]
  uint16_t* g1;             // [M, n_b]
  // Optional: a split-K reduction run by extra workgroups of the same
  // launch (the Q/K/V/G partials of the packed projection).
  const ReduceProblem* red;
};
hipError_t launch_fab_fb_tail(const FbProblem& p, hipStream_t s);

// RMSNorm of the latent rows into a bf16 buffer: n[m,k] = bf16(L[m,k] * r[m] *
// gamma[k]), r[m] = rsqrt(mean_k L[m,k]^2 + eps).  d <= kNormMaxD.
struct NormProblem {
  const uint16_t* latent;   // [M,d] contiguous
  const uint16_t* gamma;    // [d]
  uint16_t* out;            // [M,d] contiguous
  int M, d;
  float eps;
};
hipError_t launch_rmsnorm(const NormProblem& p, hipStream_t s);
constexpr int kNormMaxD = 8192;

// F_B stage tiling: activation rows per workgroup, largest rank (f_a width)
// it supports.
constexpr int kFbMGroup = 4;
constexpr int kFbMaxRank = 512;

// GEMV activation staging: a workgroup keeps its K-range of the activation in
// LDS (at most this many bytes) and holds every weight step of that range in
// registers; the table sizes k_split so that both fit.
constexpr size_t kGemvMaxLds = 128 * 1024;
size_t gemv_lds_bytes(int M, int K, int k_split, bool fold);
bool gemv_fits(int M, int K, int k_split, int rows, bool fold);

}  // namespace sg
