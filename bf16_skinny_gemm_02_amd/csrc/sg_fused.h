// In-launch F_A/beta -> F_B hand-off: the one-launch F_A/beta -> F_B branch
// of kda_fab_fb_proj_fused (gfx950).
//
// "Overlap low-M TP8 KDA projections" (run_kda_projection_overlap, run_fab_fb)
// computes P = bf16(x @ W_ab^T), splits it into f_a = P[:, :rank] and
// beta = P[:, rank:], and feeds the bf16 f_a to F_B: g1 = bf16(f_a @ W_b^T).
// On its hardware the F_B GEMM is launched behind F_A/beta with programmatic
// dependent launch.  HIP has no such launch; here both stages are roles of one
// grid instead:
//
//  * the F_A/beta segment's waves (producers) store their fp32 split-K
//    partials with device-coherent stores (written through to the device's
//    point of coherence, so a workgroup on another XCD reads them), wait until
//    the stores have completed, and then advance their own flag;
//  * F_B workgroups (consumers, the FB role, later in the grid) request their
//    rows of W_b, wait -- a bounded spin -- until every producer flag has
//    advanced, then sum the partials in the fixed order s = 0..S-1 with
//    device-coherent loads, round f_a to bf16 (every FB workgroup forms the
//    same bits), and compute their rows of g1; the first FB workgroup also
//    stores beta (and f_a when asked).
//
// Flags and cursors, not a counter: every producer slot has its own flag and
// every consumer its own cursor, each written by one party only, so no two
// workgroups ever update one word (arrivals counted with atomics on one word
// serialise at the point of coherence: ~20 ns each, ~19 us for 952 waves).
// Invariant between launches: every flag and every cursor of the header
// holds L, the number of one-launch calls so far on this workspace (all zero
// at first).  A launch moves every one of them to L + 1 exactly once:
//  - producer p reads its flag (L) early and writes L + 1 once its partials
//    are stored; producer 0 also writes L + 1 to the flags of the slots this
//    launch has no producer for;
//  - consumer k reads its cursor (L), waits until flags 0..n-1 reach L + 1,
//    then writes L + 1 to its cursor; consumer 0 also advances the cursors
//    of the absent consumers.
// So the header needs no reset, whatever the shapes of successive launches.
// No fence that writes back or invalidates a whole L2 is used: only the
// hand-off data itself bypasses the non-coherent caches.
//
// Progress does not depend on co-residency: producers never wait, and a
// waiter only waits for producers that do not wait.  The spin is bounded
// anyway (kFbSpinLimit polls); on a time-out the waiter writes NaN to its
// outputs, so a failed hand-off is visible and every wave still ends (and the
// invariant holds again once the late producers have written).
#pragma once

#include "sg_device.h"

namespace sg {

// Header of the F_A/beta workspace: kFbMaxProducers flags, then
// kFbMaxConsumers cursors (uint32 each), zero before the first one-launch call.
constexpr int kFbMaxProducers = 4096;
constexpr int kFbMaxConsumers = 512;

// FB role arguments, part of the kernel argument block of a fused launch.
struct FbFuse {
  const float* partial;  // [S][M][n_ab] F_A/beta partial sums
  unsigned* sync;        // the workspace header (flags, then cursors)
  int S;                 // K splits of the F_A/beta segment
  int arrivals;          // producer slots in this launch (<= kFbMaxProducers)
  int M, n_ab, rank, n_b;
  const uint16_t* w_b;   // [n_b, rank]
  uint16_t* f_a;         // [M, rank], nullable
  uint16_t* beta;        // [M, n_ab - rank]
  uint16_t* g1;          // [M, n_b]
  int wg_begin, wg_end;  // FB workgroups [wg_begin, wg_end)
};

constexpr int kFbThreads = 256;   // threads of every kernel that hosts the FB role
constexpr int kFbSpinLimit = 1 << 18;
constexpr int kFbPollBatch = 16;  // flag loads per lane per round trip of a poll
constexpr uint16_t kBf16NaN = 0x7FC0;

// W_b rows of one FB workgroup: passes of 256 / G rows (G lanes per row),
// up to 64 rows and 8 passes.
__host__ __device__ constexpr int fb_passes(int G) {
  return (64 * G / kFbThreads) < 8 ? (64 * G / kFbThreads) : 8;
}
// Lanes per W_b row: the smallest power of two >= max(8, rank / 8).
inline int fb_lanes(int rank) {
  int g = 8;
  while (g < (rank >> 3)) g <<= 1;
  return g;
}
// FB workgroups for n_b rows of W_b (at least one: it also stores beta).
inline int fused_fb_wgs(int rank, int n_b) {
  const int g = fb_lanes(rank);
  const int rows = fb_passes(g) * (kFbThreads / g);
  const int w = (n_b + rows - 1) / rows;
  return w > 0 ? w : 1;
}

// Host side: the role's kernel arguments for workgroups [wg_begin, wg_end).
template <typename FusedFbT>
inline FbFuse make_fb_fuse(const FusedFbT& f, int wg_begin, int wg_end, int arrivals) {
  FbFuse r;
  r.partial = f.partial;
  r.sync = f.sync;
  r.S = f.S;
  r.arrivals = arrivals;
  r.M = f.M;
  r.n_ab = f.n_ab;
  r.rank = f.rank;
  r.n_b = f.n_b;
  r.w_b = f.w_b;
  r.f_a = f.f_a;
  r.beta = f.beta;
  r.g1 = f.g1;
  r.wg_begin = wg_begin;
  r.wg_end = wg_end;
  return r;
}

inline FbFuse no_fb_fuse() {
  FbFuse r{};
  r.wg_begin = r.wg_end = 0;
  return r;
}

// ---- device-coherent accesses --------------------------------------------------

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_flag(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_flag(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Producer slot `slot` of a launch with `nslots` producer slots, called by
// the whole wave once its coherent partial stores are issued; `prev` is the
// slot's flag as read before (L).  Waits until the wave's stores have
// completed, then writes L + 1 to the slot's flag; slot 0 also writes it to
// the flags of the slots [nslots, kFbMaxProducers) that have no producer.
__device__ __forceinline__ void produce(unsigned* sync, int slot, int nslots, unsigned prev) {
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const unsigned next = prev + 1u;
  if (lane == 0) store_flag(sync + slot, next);
  if (slot == 0)
    for (int q = nslots + lane; q < kFbMaxProducers; q += kWave) store_flag(sync + q, next);
}

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

// Partial-sum loads per round trip, and P elements per thread per pass.
constexpr int kFbSumBatch = 8;
constexpr int kFbPerPass = 2;

// LDS the role needs from its kernel's dynamic LDS: f_a as bf16, then one
// flag.  (The role declares no LDS of its own: a kernel with static LDS
// could not raise its dynamic limit to the whole 160 KiB.)
__host__ __device__ inline size_t fb_lds_bytes(int M, int rank) {
  return ((static_cast<size_t>(M) * rank * 2 + 15) & ~static_cast<size_t>(15)) + 16;
}

// The FB role of workgroup `b` (b in [f.wg_begin, f.wg_end)).  lds: at least
// fb_lds_bytes(M, rank) of the kernel's dynamic LDS, 16-byte aligned.
template <int G>
__device__ void fb_role_g(const FbFuse& f, int b, void* lds_raw) {
  constexpr int kPasses = fb_passes(G);
  constexpr int kRowsPerPass = kFbThreads / G;
  uint16_t* fa_lds = static_cast<uint16_t*>(lds_raw);
  int& ok_flag = *reinterpret_cast<int*>(static_cast<char*>(lds_raw) + fb_lds_bytes(f.M, f.rank) - 16);
  const int tid = static_cast<int>(threadIdx.x);
  const int local = b - f.wg_begin;
  const bool first = local == 0;
  const int j = tid & (G - 1);
  const int K8 = f.rank >> 3;
  const bool cvalid = j < K8;
  // This workgroup's rows of W_b (kPasses of kRowsPerPass rows) and its
  // cursor, requested before the wait.
  int irow[kPasses];
  u32x4 wv[kPasses];
#pragma unroll
  for (int q = 0; q < kPasses; ++q) {
    irow[q] = (local * kPasses + q) * kRowsPerPass + tid / G;
    wv[q] = (irow[q] < f.n_b && cvalid) ? load_nt(f.w_b + static_cast<int64_t>(irow[q]) * f.rank + j * 8)
                                        : zero4();
  }
  unsigned* cursors = f.sync + kFbMaxProducers;
  const unsigned target = load_flag(cursors + local) + 1u;

  // Wave 0 waits: each lane watches every 64th producer flag until all have
  // reached target.  A poll requests its flags in straight-line batches
  // (indices past the last slot repeat it): one memory round trip per
  // kFbPollBatch * 64 slots.
  if (tid < kWave) {
    int polls = 0;
    bool all = false;
    for (;;) {
      bool mine = true;
      for (int q0 = 0; q0 < f.arrivals; q0 += kFbPollBatch * kWave) {
        unsigned v[kFbPollBatch];
#pragma unroll
        for (int t = 0; t < kFbPollBatch; ++t)
          v[t] = load_flag(f.sync + min(q0 + t * kWave + tid, f.arrivals - 1));
#pragma unroll
        for (int t = 0; t < kFbPollBatch; ++t) mine = mine && static_cast<int>(v[t] - target) >= 0;
      }
      all = __builtin_amdgcn_ballot_w64(!mine) == 0;  // no lane saw a flag behind
      if (all || ++polls >= kFbSpinLimit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0) ok_flag = all ? 1 : 0;
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

  // g1[m, i] = bf16(sum_r f_a[m, r] * w_b[i, r]), one W_b row per G lanes
  // (NaN f_a after a time-out makes g1 NaN too).
  for (int m = 0; m < f.M; ++m) {
    const u32x4 xv = cvalid ? *reinterpret_cast<const u32x4*>(fa_lds + m * f.rank + j * 8) : zero4();
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const float v = fb_group_sum<G>(dot8(xv, wv[q], 0.f));
      if (irow[q] < f.n_b && j == 0)
        f.g1[static_cast<int64_t>(m) * f.n_b + irow[q]] = ok ? f32_to_bf16(v) : kBf16NaN;
    }
  }

  // This consumer is done: its cursor moves to target; consumer 0 also moves
  // the cursors of the absent consumers.
  const int nfb = f.wg_end - f.wg_begin;
  if (tid == 0) store_flag(cursors + local, target);
  if (local == 0)
    for (int q = nfb + tid; q < kFbMaxConsumers; q += kFbThreads) store_flag(cursors + q, target);
}

__device__ __forceinline__ void fb_role(const FbFuse& f, int b, void* lds) {
  const int g = f.rank >> 3;  // chunks per W_b row
  if (g <= 8) fb_role_g<8>(f, b, lds);
  else if (g <= 16) fb_role_g<16>(f, b, lds);
  else if (g <= 32) fb_role_g<32>(f, b, lds);
  else fb_role_g<64>(f, b, lds);
}

}  // namespace sg
