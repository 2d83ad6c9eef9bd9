// Row-parallel and split-K GEMV for one activation row (gfx950).
//
// out[m,n] = sum_k a[m,k] * w[n,k]  for a handful of activation rows m, the
// decode-time projection of "Kimi K3 support, phase 1" (CuteSkinnyGemm, where
// M is fixed at compile time and fully unrolled) and the F_A/beta small-N
// projection of "Overlap low-M TP8 KDA projections" (_KdaSkinnyNGemm, which
// splits the work finely because N is small).
//
// Mapping.  A workgroup of NW waves owns NW*R consecutive weight rows and one
// K-range (all of K, or 1/k_split of it).  A "step" is 512 consecutive k: the
// 64 lanes of a wave read 64 consecutive 16-byte chunks of one weight row,
// one fully coalesced 1 KiB global_load_dwordx4.
//
//  1. The workgroup stages its activation rows for the K-range in LDS with
//     direct global->LDS copies (no registers); the products read them back
//     with ds_read_b128.  The copies go out first: a wave's vector memory
//     operations complete in issue order, so the wait for them (and the
//     RMSNorm fold below) does not wait for the weight stream.
//  2. Each wave issues every weight chunk of its R rows over the workgroup's
//     K-range at once (non-temporal loads: each weight byte is used once).
//     The table keeps the K-range within D steps (a whole 7168-wide row for
//     R <= 2), so the whole weight stream is requested before the first
//     product and there is nothing to refill; each step's products start as
//     soon as it lands.  On MI355X a plain streaming read of the same bytes
//     is only ~5% faster.
//  3. acc[m][r] accumulates in fp32 with v_dot2c_f32_bf16; a DPP / permlane
//     butterfly sums the 64 lanes and lane (m*R + r) stores output (m, r).
//
// Split-K (grid.y > 1): workgroup (row group, s) covers steps
// [s*sps, (s+1)*sps) and stores fp32 partials for a later fixed-order sum.
//
// Fold (latent-MoE tail, RMSNorm -> up-projection): the staged activation is
// the latent L over the whole row, with gamma staged behind it in the same
// step (both land with one round trip).  Every wave sums L[m,k]^2 from LDS in the
// same order, r[m] = rsqrt(sum / K + eps), and the workgroup rewrites LDS in
// place with n = bf16(L * r * gamma), the bf16 normalised latent the
// up-projection consumes.  One launch, no workspace.
#include "sg_device.h"
#include "sg_fused.h"
#include "sg_launch.h"

namespace sg {

static_assert(kSyncBytes == static_cast<size_t>(kFbMaxProducers + kFbMaxConsumers) * sizeof(unsigned),
              "hand-off header size");

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
  uint16_t* out2;
  int64_t ldc2;
  int n_split;
  unsigned* arrive;  // in-launch hand-off (FB instances, sg_fused.h): the flag header
  int nslots;        // producer slots of the launch (every wave of the F_A/beta segment)
  int N, K;
  int sps;  // steps per split
  float eps;
};

// One launch covers one or two segments (independent problems sharing a
// flat grid), and optionally the F_B role of a fused launch.  Within a
// segment, workgroup `local` takes row group local % groups of K-range
// local / groups.
struct GemvSeg {
  GemvArgs g;
  int groups;
  unsigned groups_magic;  // quotient_magic(groups)
  int wg_begin, wg_end;  // the segment's workgroups (empty range: unused)
};
struct GemvLaunch {
  GemvSeg seg[2];
  FbFuse fb;
};

// FB (instances of the one-launch F_A/beta -> F_B branch only): workgroups
// in L.fb's range run the F_B role, and a segment with `arrive` set hands
// its partials over (sg_fused.h).  Other instances carry none of that code.
//
// RES (instances launched for a problem with a residual and bf16 output):
// the residual is requested first; other instances load none.
template <int M, int R, int NW, int D, bool FOLD, bool FB, bool RES>
__global__ __launch_bounds__(NW * kWave) void gemv_kernel(GemvLaunch L) {
  extern __shared__ u32x4 xs[];  // [M][row_chunks] 16-byte chunks of the activation
  const int b = static_cast<int>(blockIdx.x);
  if constexpr (FB) {
    static_assert(NW * kWave == kFbThreads && !FOLD, "F_B role instances");
    if (b >= L.fb.wg_begin && b < L.fb.wg_end) {
      fb_role(L.fb, b, xs);
      return;
    }
  }
  // FOLD instances take one segment: no selection, and every argument the
  // first copies need requested in one round of scalar loads (left to itself
  // the compiler issues a second round behind a wait for the first).
  if constexpr (FOLD) {
    const GemvSeg& s0 = L.seg[0];
    asm volatile("" ::"s"(s0.g.a), "s"(s0.g.lda), "s"(s0.g.w), "s"(s0.g.ldw), "s"(s0.g.res), "s"(s0.g.ldr),
                 "s"(s0.g.gamma), "s"(s0.g.N), "s"(s0.g.K), "s"(s0.g.sps), "s"(s0.groups), "s"(s0.groups_magic),
                 "s"(s0.wg_begin));
  }
  const GemvSeg sgm = (FOLD || !(b >= L.seg[1].wg_begin && b < L.seg[1].wg_end)) ? L.seg[0] : L.seg[1];
  const GemvArgs g = sgm.g;
  const int local = b - sgm.wg_begin;
  const int split = quotient_by(local, sgm.groups, sgm.groups_magic);
  const int group = local - split * sgm.groups;
  constexpr int kThreads = NW * kWave;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = wave_id();
  const int n0 = (group * NW + wave) * R;
  const bool active = n0 < g.N;

  // Hand-off: this wave's producer flag, read before anything else is in
  // flight (so the counted waits below are unchanged).
  const int slot = local * NW + wave;
  unsigned prev = 0u;
  if constexpr (FB) prev = g.arrive != nullptr ? load_flag(g.arrive + slot) : 0u;

  const int K8 = g.K >> 3;
  const int nsteps = (K8 + kWave - 1) / kWave;
  const int s_begin = split * g.sps;
  const int s_end = min(nsteps, s_begin + g.sps);
  const int nst = max(0, s_end - s_begin);  // <= D (the table guarantees it)
  const int row_chunks = nst * kWave;
  const int total = M * row_chunks;
  const int c_base = s_begin * kWave;

  // 0. The residual this lane adds in the epilogue (lane m * R + r adds
  //    res[m, n0 + r]), requested before anything else: it lands with the
  //    first round trip instead of costing one of its own at the end.  The
  //    load is unconditional (index clamped; the activation stands in when
  //    there is no residual) so that no wait is attached to it.
  uint16_t res_bits = 0;
  if constexpr (RES) {
    const bool use = g.res != nullptr && g.partial == nullptr;
    const int mr = min(lane / R, M - 1);
    const int nr = min(n0 + lane % R, g.N - 1);
    res_bits = use ? g.res[static_cast<int64_t>(mr) * g.ldr + nr] : g.a[0];
  }

  // 1. Activation rows of the range into LDS, one 1 KiB step-block per wave
  //    copy, straight from global memory (no registers; chunks past K read
  //    zeros), and with the fold gamma over the same range behind them.
  //    They go out before the weights: a wave's vector memory operations
  //    complete in issue order, so staging issued after the weight stream
  //    would land only after all of it, and the normalisation below would
  //    wait for the whole stream.
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(((M - 1) * g.lda + g.K) * 2));
#pragma unroll
  for (int m = 0; m < M; ++m) {
    for (int t = wave; t < nst; t += NW) {
      const int c = c_base + t * kWave + lane;
      copy16_to_lds(xres, xs + m * row_chunks + t * kWave,
                    c < K8 ? static_cast<uint32_t>((m * g.lda + c * 8) * 2) : kOob);
    }
  }
  if constexpr (FOLD) {
    const rsrc_t gres = make_rsrc(g.gamma, static_cast<uint32_t>(g.K * 2));
    for (int t = wave; t < nst; t += NW) {
      const int c = c_base + t * kWave + lane;
      copy16_to_lds(gres, xs + total + t * kWave, c < K8 ? static_cast<uint32_t>(c * 16) : kOob);
    }
  }

  // 2. Every weight chunk of the workgroup's K-range, issued up front (the
  //    range is at most D steps, so nothing is reloaded later).  Buffer
  //    loads: rows past N, chunks past K and steps past the range read zero.
  const int wg_row0 = group * NW * R;
  const int wg_rows = min(NW * R, g.N - wg_row0);
  const rsrc_t wres = make_rsrc(g.w + static_cast<int64_t>(wg_row0) * g.ldw,
                                static_cast<uint32_t>(((wg_rows - 1) * g.ldw + g.K) * 2));
  u32x4 wr[D][R];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int c = c_base + j * kWave + lane;
    const bool kok = (j < nst) && (c < K8);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = wave * R + r;
      const uint32_t off =
          (kok && row < wg_rows) ? static_cast<uint32_t>((row * g.ldw + c * 8) * 2) : kOob;
      wr[j][r] = buf_load_nt(wres, off);
    }
  }

  // This wave's staging has landed once at most its D * R weight loads are
  // outstanding; the barrier makes that so for every wave.  (A full
  // __syncthreads would also wait for the weights.)
  wait_vmcnt<D * R>();
  __builtin_amdgcn_s_barrier();

  if constexpr (FOLD) {
    // RMSNorm over the whole row (the host runs the fold with one split).
    float rs[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float ss = 0.f;
      for (int c = lane; c < row_chunks; c += kWave) {
        const u32x4 v = xs[m * row_chunks + c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float l0 = bf16_lo(v[i]), l1 = bf16_hi(v[i]);
          ss = fmaf(l0, l0, ss);
          ss = fmaf(l1, l1, ss);
        }
      }
      rs[m] = __frsqrt_rn(wave_allreduce(ss) / static_cast<float>(g.K) + g.eps);
    }
    __builtin_amdgcn_s_barrier();  // every wave has read the raw latent
    for (int q = tid; q < total; q += kThreads) {
      const int m = q / row_chunks;
      const int c = q - m * row_chunks;
      if (c < K8) {
        const u32x4 v = xs[q];
        const u32x4 gv = xs[total + c];
        float r = 0.f;
#pragma unroll
        for (int mm = 0; mm < M; ++mm) r = (mm == m) ? rs[mm] : r;
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = pack_bf16x2(bf16_lo(v[i]) * r * bf16_lo(gv[i]), bf16_hi(v[i]) * r * bf16_hi(gv[i]));
        xs[q] = o;
      }
    }
    wait_lgkmcnt0();  // the normalised latent is in LDS
    __builtin_amdgcn_s_barrier();
  }
  if (!active) {  // no barrier follows; in a hand-off every wave is a producer
    if constexpr (FB) {
      if (g.arrive != nullptr) produce(g.arrive, slot, g.nslots, prev);
    }
    return;
  }

  // 3. Products: every weight step is already in flight; each is used as
  //    soon as it lands.
  float acc[M][R];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < nst) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4 xv = xs[m * row_chunks + j * kWave + lane];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = dot8(xv, wr[j][r], acc[m][r]);
      }
    }
  }

  // 4. Cross-lane sums: every lane ends up with every (m, r) total.
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_allreduce(acc[m][r]);

  float v = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) v = (lane == m * R + r) ? acc[m][r] : v;
  if (lane < M * R) {
    const int m = lane / R, r = lane % R;
    const int n = n0 + r;
    if (n < g.N) {
      if (g.partial != nullptr) {
        float* dst = g.partial + (static_cast<int64_t>(split) * M + m) * g.N + n;
        if constexpr (FB) {
          if (g.arrive != nullptr) store_coherent(dst, v);
          else *dst = v;
        } else {
          *dst = v;
        }
      } else {
        if constexpr (RES) {
          if (g.res != nullptr) v += bf16_to_f32(res_bits);
        }
        if (g.n_split > 0 && n >= g.n_split)
          g.out2[m * g.ldc2 + (n - g.n_split)] = f32_to_bf16(v);
        else
          g.out[m * g.ldc + n] = f32_to_bf16(v);
      }
    }
  }
  if constexpr (FB) {
    if (g.arrive != nullptr) produce(g.arrive, slot, g.nslots, prev);
  }
}

// Weight steps a wave holds (the largest K-range, in 512-wide steps, the
// table gives one workgroup): 16, 14, 7, 4 steps for R = 1, 2, 4, 7 rows,
// i.e. at most 112 VGPRs of weights; a whole 7168-wide row for R <= 2, a
// whole 2048-wide one for R = 7.
constexpr int gemv_depth(int R) { return R == 1 ? 16 : (R == 2 ? 14 : (R == 4 ? 7 : 4)); }

template <int M, int R, int NW, bool FOLD, bool FB, bool RES>
hipError_t launch_inst(const GemvLaunch& g, dim3 grid, size_t lds, hipStream_t s) {
  constexpr int D = gemv_depth(R);
  auto kern = gemv_kernel<M, R, NW, D, FOLD, FB, RES>;
  static std::atomic<bool> lds_set[kLdsAttrDevices];
  const hipError_t attr = ensure_lds_limit(reinterpret_cast<const void*>(kern), kGemvMaxLds, lds_set);
  if (attr != hipSuccess) return attr;
  return launch_kernel(kern, grid, dim3(NW * kWave), lds, s, g);
}

// The table sends only M = 1 here (4 waves; one weight row per wave, or four
// when a whole row fits in 7 steps); wider M goes to the MFMA kernels.
template <bool FOLD, bool RES>
hipError_t launch_fold(const GemvLaunch& g, int M, int R, int NW, dim3 grid, size_t lds,
                       hipStream_t s) {
  if (M == 1 && R == 1 && NW == 4) return launch_inst<1, 1, 4, FOLD, false, RES>(g, grid, lds, s);
  if (M == 1 && R == 4 && NW == 4) return launch_inst<1, 4, 4, FOLD, false, RES>(g, grid, lds, s);
  if (M == 1 && R == 7 && NW == 4) return launch_inst<1, 7, 4, FOLD, false, RES>(g, grid, lds, s);
  return hipErrorInvalidValue;
}

// The one-launch F_A/beta -> F_B instances (M = 1, 4 waves, no fold).
hipError_t launch_fb(const GemvLaunch& g, int M, int R, int NW, dim3 grid, size_t lds,
                     hipStream_t s) {
  if (M == 1 && R == 1 && NW == 4) return launch_inst<1, 1, 4, false, true, false>(g, grid, lds, s);
  if (M == 1 && R == 4 && NW == 4) return launch_inst<1, 4, 4, false, true, false>(g, grid, lds, s);
  if (M == 1 && R == 7 && NW == 4) return launch_inst<1, 7, 4, false, true, false>(g, grid, lds, s);
  return hipErrorInvalidValue;
}

}  // namespace

// The activation rows of one K-range, plus gamma's when the RMSNorm is folded.
size_t gemv_lds_bytes(int M, int K, int k_split, bool fold) {
  const int K8 = K >> 3;
  const int nsteps = (K8 + kWave - 1) / kWave;
  const int S = k_split > 0 ? k_split : 1;
  const int sps = nsteps > 0 ? (nsteps + S - 1) / S : 0;
  return static_cast<size_t>(M + (fold ? 1 : 0)) * sps * kWave * 16;
}

bool gemv_fits(int M, int K, int k_split, int rows, bool fold) {
  const int K8 = K >> 3;
  const int nsteps = (K8 + kWave - 1) / kWave;
  const int S = k_split > 0 ? k_split : 1;
  const int sps = nsteps > 0 ? (nsteps + S - 1) / S : 0;
  return gemv_lds_bytes(M, K, k_split, fold) <= kGemvMaxLds && sps <= gemv_depth(rows);
}

bool gemv_same_instance(const sg_config_t& a, const sg_config_t& b) {
  return (a.kind == SG_KIND_GEMV_ROW || a.kind == SG_KIND_GEMV_SPLITK) &&
         (b.kind == SG_KIND_GEMV_ROW || b.kind == SG_KIND_GEMV_SPLITK) && a.rows == b.rows &&
         a.waves == b.waves && a.m_tile == b.m_tile;
}

namespace {

// Segments in grid order, and the F_B role (fb != NULL) after the first
// fb_after of them.
hipError_t launch_gemv_impl(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                            const FusedFb* fb, int fb_after, hipStream_t s) {
  if (nseg < 1 || nseg > 2) return hipErrorInvalidValue;
  // The fold instances read one segment only.
  if (nseg == 2 && (!gemv_same_instance(cfgs[0], cfgs[1]) || segs[0].M != segs[1].M ||
                    segs[0].gamma != nullptr || segs[1].gamma != nullptr))
    return hipErrorInvalidValue;
  if (fb != nullptr && (fb_after < 0 || fb_after > nseg || cfgs[0].waves * kWave != kFbThreads ||
                        segs[0].gamma != nullptr))
    return hipErrorInvalidValue;
  GemvLaunch L;
  L.fb = no_fb_fuse();
  const int nfb = fb != nullptr ? fused_fb_wgs(fb->rank, fb->n_b) : 0;
  int wgs = 0, arrivals = 0, arriving = 0;
  size_t lds = 0;
  for (int i = 0; i < 2; ++i) {
    GemvSeg& sgm = L.seg[i];
    if (i >= nseg) {
      sgm = L.seg[0];
      sgm.wg_begin = sgm.wg_end = 0;
      continue;
    }
    if (fb != nullptr && i == fb_after) {
      L.fb = make_fb_fuse(*fb, wgs, wgs + nfb, 0);
      wgs += nfb;
    }
    const DotProblem& p = segs[i];
    const sg_config_t& cfg = cfgs[i];
    GemvArgs& g = sgm.g;
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
    g.out2 = p.out2;
    g.ldc2 = p.ldc2;
    g.n_split = p.n_split;
    g.arrive = fb != nullptr ? p.arrive : nullptr;
    g.nslots = 0;
    g.N = p.N;
    g.K = p.K;
    g.eps = p.eps;
    const int K8 = p.K >> 3;
    const int nsteps = (K8 + kWave - 1) / kWave;
    const int S = cfg.k_split > 0 ? cfg.k_split : 1;
    g.sps = nsteps > 0 ? (nsteps + S - 1) / S : 1;
    const bool fold = p.gamma != nullptr;
    if (!gemv_fits(p.M, p.K, S, cfg.rows, fold)) return hipErrorInvalidValue;
    const size_t seg_lds = gemv_lds_bytes(p.M, p.K, S, fold);
    if (seg_lds > lds) lds = seg_lds;
    const int rows_per_wg = cfg.waves * cfg.rows;
    sgm.groups = (p.N + rows_per_wg - 1) / rows_per_wg;
    if (sgm.groups <= 0) return hipErrorInvalidValue;
    sgm.groups_magic = quotient_magic(sgm.groups);
    sgm.wg_begin = wgs;
    wgs += sgm.groups * S;
    sgm.wg_end = wgs;
    if (g.arrive != nullptr) {
      if (p.partial == nullptr || p.partial != fb->partial || S != fb->S || p.arrive != fb->sync)
        return hipErrorInvalidValue;
      arrivals += sgm.groups * S * cfg.waves;  // every wave of the segment is a producer
      ++arriving;
    }
  }
  if (fb != nullptr) {
    if (fb_after == nseg) {
      L.fb = make_fb_fuse(*fb, wgs, wgs + nfb, 0);
      wgs += nfb;
    }
    if (arriving != 1 || arrivals > kFbMaxProducers || nfb > kFbMaxConsumers) return hipErrorInvalidValue;
    L.fb.arrivals = arrivals;
    for (int i = 0; i < nseg; ++i) L.seg[i].g.nslots = arrivals;
    const size_t fa_bytes = fb_lds_bytes(fb->M, fb->rank);
    if (fa_bytes > lds) lds = fa_bytes;
    if (lds > kGemvMaxLds) return hipErrorInvalidValue;
  }
  if (wgs <= 0) return hipSuccess;
  const dim3 grid(wgs);
  if (fb != nullptr) return launch_fb(L, segs[0].M, cfgs[0].rows, cfgs[0].waves, grid, lds, s);
  // Instances that load a residual only where a segment has one and stores bf16.
  bool res = false;
  for (int i = 0; i < nseg; ++i) res = res || (segs[i].res != nullptr && segs[i].partial == nullptr);
  const int M = segs[0].M, R = cfgs[0].rows, NW = cfgs[0].waves;
  if (segs[0].gamma != nullptr)
    return res ? launch_fold<true, true>(L, M, R, NW, grid, lds, s) : launch_fold<true, false>(L, M, R, NW, grid, lds, s);
  return res ? launch_fold<false, true>(L, M, R, NW, grid, lds, s) : launch_fold<false, false>(L, M, R, NW, grid, lds, s);
}

}  // namespace

hipError_t launch_gemv(const DotProblem* segs, const sg_config_t* cfgs, int nseg, hipStream_t s) {
  return launch_gemv_impl(segs, cfgs, nseg, nullptr, 0, s);
}

hipError_t launch_gemv_fused(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                             const FusedFb& fb, int fb_after, hipStream_t s) {
  return launch_gemv_impl(segs, cfgs, nseg, &fb, fb_after, s);
}

hipError_t launch_gemv(const DotProblem& p, const sg_config_t& cfg, hipStream_t s) {
  return launch_gemv(&p, &cfg, 1, s);
}

}  // namespace sg
