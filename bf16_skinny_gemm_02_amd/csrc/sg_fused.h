// In-launch F_A/beta -> F_B hand-off for the KDA projection (gfx950).
//
// "Overlap low-M TP8 KDA projections" (run_kda_projection_overlap, run_fab_fb)
// computes P = bf16(x @ W_ab^T), splits it into f_a = P[:, :rank] and
// beta = P[:, rank:], and feeds the bf16 f_a to F_B: g1 = bf16(f_a @ W_b^T).
// On its hardware the F_B GEMM is launched behind F_A/beta with programmatic
// dependent launch.  HIP has no such launch; here both stages are roles of one
// grid instead:
//
//  * the F_A/beta segment's workgroups store their fp32 split-K partials with
//    device-coherent stores (written through to the device's point of
//    coherence, so a workgroup on another XCD reads them), wait until the
//    stores have completed, and then count their arrival with one atomic add;
//  * F_B workgroups (the FB role, later in the grid) request their rows of
//    W_b, wait -- a bounded spin -- until every F_A/beta arrival is counted,
//    then sum the partials in the fixed order s = 0..S-1 with device-coherent
//    loads, round f_a to bf16 (every FB workgroup forms the same bits), and
//    compute their rows of g1; the first FB workgroup also stores beta (and
//    f_a when asked).
//
// No fence that writes back or invalidates a whole L2 is used: only the
// hand-off data itself bypasses the non-coherent caches.
//
// Progress does not depend on co-residency: producers never wait, and a
// waiter only waits for producers that do not wait.  The spin is bounded
// anyway (kFbSpinLimit polls); on a time-out the waiter writes NaN to its
// outputs, so a failed hand-off is visible and every wave still ends.
//
// The two counters live in the caller's workspace: zero before the first
// launch that uses them, and every launch leaves them zero (the last FB
// workgroup to finish resets both).
#pragma once

#include "sg_device.h"

namespace sg {

// FB role arguments, part of the kernel argument block of a fused launch.
struct FbFuse {
  const float* partial;  // [S][M][n_ab] F_A/beta partial sums
  unsigned* sync;        // [0] arrivals, [1] finished FB workgroups
  int S;                 // K splits of the F_A/beta segment
  int arrivals;          // arrivals to wait for
  int M, n_ab, rank, n_b;
  const uint16_t* w_b;   // [n_b, rank]
  uint16_t* f_a;         // [M, rank], nullable
  uint16_t* beta;        // [M, n_ab - rank]
  uint16_t* g1;          // [M, n_b]
  int wg_begin, wg_end;  // FB workgroups [wg_begin, wg_end); wg_begin == wg_end: none
};

constexpr int kFbThreads = 256;   // threads of every kernel that hosts the FB role
constexpr int kFbSpinLimit = 1 << 18;
constexpr uint16_t kBf16NaN = 0x7FC0;

// ---- device-coherent accesses --------------------------------------------------

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by each arriving wave once its own coherent stores are issued:
// waits until they have completed, then counts one arrival.
__device__ __forceinline__ void arrive(unsigned* sync) {
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if ((threadIdx.x & (kWave - 1)) == 0)
    __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lanes per W_b row: the smallest power of two >= rank / 8 (rank <= 512).
template <int G>
__device__ __forceinline__ float fb_group_sum(float v) {
  if constexpr (G >= 2) v += dpp<0xB1>(v);
  if constexpr (G >= 4) v += dpp<0x4E>(v);
  if constexpr (G >= 8) v += dpp<0x141>(v);
  if constexpr (G >= 16) v += dpp<0x140>(v);
  if constexpr (G >= 32) v = xor16_sum(v);
  if constexpr (G >= 64) v = xor32_sum(v);
  return v;
}

// Partial-sum loads per batch (one memory round trip each), and P elements
// per thread per pass.
constexpr int kFbSumBatch = 8;
constexpr int kFbPerPass = 4;

// The FB role of workgroup `b` (b in [f.wg_begin, f.wg_end)).  lds: at least
// M * rank * 2 bytes of the kernel's dynamic LDS, 16-byte aligned.
template <int G>
__device__ void fb_role_g(const FbFuse& f, int b, void* lds_raw) {
  constexpr int kRowsPerWg = kFbThreads / G;
  uint16_t* fa_lds = static_cast<uint16_t*>(lds_raw);
  __shared__ int ok_flag;
  const int tid = static_cast<int>(threadIdx.x);
  const int local = b - f.wg_begin;
  const bool first = local == 0;
  const int j = tid & (G - 1);
  const int K8 = f.rank >> 3;
  const bool cvalid = j < K8;
  const int i = local * kRowsPerWg + tid / G;
  const bool ivalid = i < f.n_b;
  // This workgroup's rows of W_b, requested before the wait.
  const u32x4 wv = (ivalid && cvalid) ? load_nt(f.w_b + static_cast<int64_t>(i) * f.rank + j * 8)
                                      : zero4();

  if (tid == 0) {
    int n = 0;
    unsigned seen = __hip_atomic_load(f.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (seen < static_cast<unsigned>(f.arrivals) && n < kFbSpinLimit) {
      __builtin_amdgcn_s_sleep(2);
      seen = __hip_atomic_load(f.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++n;
    }
    ok_flag = seen >= static_cast<unsigned>(f.arrivals);
  }
  __syncthreads();
  const bool ok = ok_flag != 0;

  // P for this workgroup's needs: all n_ab columns in the first FB workgroup
  // (it stores beta, and f_a when asked), the rank f_a columns elsewhere.
  // kFbPerPass elements per thread per pass; all their loads of one batch of
  // splits go out together (unused slots load element 0 and are discarded),
  // and each element's splits are added in the order s = 0..S-1.
  const int cols = first ? f.n_ab : f.rank;
  const int count = f.M * cols;
  const int64_t plane = static_cast<int64_t>(f.M) * f.n_ab;
  for (int base = 0; base < count; base += kFbPerPass * kFbThreads) {
    int64_t off[kFbPerPass];
#pragma unroll
    for (int e = 0; e < kFbPerPass; ++e) {
      const int idx = base + e * kFbThreads + tid;
      const int m = idx / cols;
      off[e] = idx < count ? static_cast<int64_t>(m) * f.n_ab + (idx - m * cols) : 0;
    }
    float acc[kFbPerPass];
#pragma unroll
    for (int e = 0; e < kFbPerPass; ++e) acc[e] = 0.f;
    if (ok) {
      for (int s0 = 0; s0 < f.S; s0 += kFbSumBatch) {
        float v[kFbPerPass][kFbSumBatch];
#pragma unroll
        for (int e = 0; e < kFbPerPass; ++e)
#pragma unroll
          for (int t = 0; t < kFbSumBatch; ++t)
            v[e][t] = load_coherent(f.partial + off[e] + static_cast<int64_t>(min(s0 + t, f.S - 1)) * plane);
#pragma unroll
        for (int e = 0; e < kFbPerPass; ++e)
#pragma unroll
          for (int t = 0; t < kFbSumBatch; ++t)
            if (s0 + t < f.S) acc[e] += v[e][t];
      }
    }
#pragma unroll
    for (int e = 0; e < kFbPerPass; ++e) {
      const int idx = base + e * kFbThreads + tid;
      if (idx >= count) continue;
      const int m = idx / cols;
      const int jj = idx - m * cols;
      const uint16_t bits = ok ? f32_to_bf16(acc[e]) : kBf16NaN;
      if (jj < f.rank) {
        fa_lds[m * f.rank + jj] = bits;
        if (first && f.f_a != nullptr) f.f_a[static_cast<int64_t>(m) * f.rank + jj] = bits;
      } else {
        f.beta[static_cast<int64_t>(m) * (f.n_ab - f.rank) + (jj - f.rank)] = bits;
      }
    }
  }
  __syncthreads();

  // g1[m, i] = bf16(sum_r f_a[m, r] * w_b[i, r]), one W_b row per G lanes.
  for (int m = 0; m < f.M; ++m) {
    const u32x4 xv = cvalid ? *reinterpret_cast<const u32x4*>(fa_lds + m * f.rank + j * 8) : zero4();
    const float v = fb_group_sum<G>(dot8(xv, wv, 0.f));
    if (ivalid && j == 0) f.g1[static_cast<int64_t>(m) * f.n_b + i] = f32_to_bf16(v);
  }

  // Every FB workgroup has passed its wait (all arrivals are in, or it timed
  // out); the last one to finish returns both counters to zero.
  if (tid == 0) {
    const unsigned nfb = static_cast<unsigned>(f.wg_end - f.wg_begin);
    const unsigned done = __hip_atomic_fetch_add(f.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == nfb - 1) {
      __hip_atomic_store(f.sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__device__ __forceinline__ void fb_role(const FbFuse& f, int b, void* lds) {
  const int g = f.rank >> 3;  // chunks per W_b row
  if (g <= 8) fb_role_g<8>(f, b, lds);
  else if (g <= 16) fb_role_g<16>(f, b, lds);
  else if (g <= 32) fb_role_g<32>(f, b, lds);
  else fb_role_g<64>(f, b, lds);
}

}  // namespace sg
