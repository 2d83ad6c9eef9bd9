// Configuration table, overlap gate and workspace sizing (host-only, pure).
//
// The analogue of ShapeDynamicSkinnyGemm._config(m, n, k) ("Kimi K3 support,
// phase 1", skinny_gemm.py), which picks a launch configuration from the
// problem shape, and of the KDA_QKVG_CONFIGS / KDA_PROJECTION_OVERLAP_MAX_TOKENS
// constants ("Overlap low-M TP8 KDA projections", low_latency_gemm.py).  The
// rule and its values are this library's own, written for MI355X: 256 compute
// units, 64-lane waves, 16-byte loads.  Nothing here touches the GPU, so the
// table can be tested on any host.
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "skinny_gemm.h"

namespace {

constexpr int kWaves = 4;            // waves per workgroup unless a kind sets its own
constexpr int kGemvRowMinN = 1024;   // below this N the M = 1 GEMV splits K
constexpr int kGemvWaveTarget = 2048;  // waves the split-K GEMV aims for
constexpr int kSmallK = 256;         // K at or below this: small-K GEMV
constexpr int kGemvDepth = 16;       // 512-wide weight steps an M = 1 GEMV wave holds
// MFMA ring kernels.  A chunk is 4 k-steps of 32 (128 k).
constexpr int kWgTarget = 224;       // workgroups a launch aims for (256 CUs, one each)
constexpr int kNoSplitTiles = 192;   // this many tiles fill the chip without a K split
constexpr int kSplitMaxTiles = 320;  // WAVESPLIT up to this many 16-row tiles
constexpr int kSplitRing = 4;        // WAVESPLIT ring slots
constexpr int kWideRing = 4;         // TILE ring slots for M <= 16 (2 waves, 32 rows)
constexpr int kTileRing = 3;         // TILE ring slots for 16 < M <= 64 (4 waves, 64 rows)
// Largest M for which the two-stream projection is worth its fork/join.  On
// MI355X the concurrent schedule measured slower than the single-stream one
// (two segments in one launch, then F_B) at every decode M from 1 to 64:
// the event pair costs more than the overlap recovers, and the LDS-resident
// main kernel leaves no room beside it for the aux branch's workgroups.  The
// gate therefore stays closed; the concurrent path remains available.
constexpr int kOverlapMaxTokens = 0;

int ceil_div(int a, int b) { return (a + b - 1) / b; }

int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Split `steps` units of work into at most `want` contiguous ranges of equal
// length; returns the number of non-empty ranges.
int effective_split(int steps, int want) {
  if (steps <= 0 || want <= 1) return 1;
  if (want > steps) want = steps;
  const int per = ceil_div(steps, want);
  return ceil_div(steps, per);
}

// K split for `tiles` workgroup tiles: none once the tiles fill the chip,
// otherwise enough ranges for about kWgTarget workgroups, each range at
// least min_steps k-steps long.
int mfma_split(int tiles, int ksteps, int min_steps) {
  if (tiles >= kNoSplitTiles) return 1;
  int cap = ksteps / min_steps;
  if (cap < 1) cap = 1;
  int want = ceil_div(kWgTarget, tiles);
  if (want > cap) want = cap;
  return effective_split(ksteps, want);
}

int direct_ring_depth(int mb) { return mb <= 8 ? 4 : 2; }

}  // namespace

extern "C" int sg_select(int M, int N, int K, int has_residual, sg_config_t* out) {
  (void)has_residual;
  if (out == nullptr) return SG_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return SG_ERR_INVALID_ARG;
  if (K % 8 != 0) return SG_ERR_UNSUPPORTED;
  if (M > 256) return SG_ERR_UNSUPPORTED;
  sg_config_t c;
  memset(&c, 0, sizeof c);
  if (M == 0 || N == 0) {
    c.kind = SG_KIND_NONE;
    *out = c;
    return SG_OK;
  }
  const int K8 = K / 8;
  const int ksteps = ceil_div(K, 32);
  c.waves = kWaves;
  c.nt_weights = 1;
  if (M <= 16 && K <= kSmallK) {
    c.kind = SG_KIND_GEMV_SMALLK;
    c.m_tile = M;
    const int G = pow2_ceil(K8 > 0 ? K8 : 1);
    c.rows = 64 / G;
    c.k_split = 1;
    c.k_unroll = 1;
    c.grid = ceil_div(N, kWaves * c.rows);
  } else if (M == 1) {
    // A workgroup holds every weight step of its K-range in registers (at
    // most kGemvDepth steps of 512) and the activation for that range in
    // LDS: K is split across workgroups until both fit.
    const int steps = ceil_div(K8, 64);
    int want;
    if (N >= kGemvRowMinN) {
      c.kind = SG_KIND_GEMV_ROW;
      want = 1;
    } else {
      c.kind = SG_KIND_GEMV_SPLITK;
      want = ceil_div(kGemvWaveTarget, N);
    }
    c.m_tile = 1;
    c.rows = 1;
    const int need = ceil_div(steps, kGemvDepth);
    c.k_split = effective_split(steps, want > need ? want : need);
    c.k_unroll = kGemvDepth;
    c.grid = ceil_div(N, c.waves * c.rows) * c.k_split;
  } else if (M <= 16) {
    c.m_tile = 4 * ceil_div(M, 4);
    const int tiles16 = ceil_div(N, 16);
    if (tiles16 <= kSplitMaxTiles) {
      // Each wave walks a quarter of the workgroup's K-range: at least one
      // chunk (4 k-steps) per wave.
      c.kind = SG_KIND_MFMA_WAVESPLIT;
      c.rows = 16;
      c.waves = 4;
      c.k_unroll = kSplitRing;
      c.k_split = mfma_split(tiles16, ksteps, 16);
      c.grid = tiles16 * c.k_split;
    } else {
      c.kind = SG_KIND_MFMA_TILE;
      c.rows = 32;
      c.waves = 2;
      c.k_unroll = kWideRing;
      const int tiles = ceil_div(N, c.rows);
      c.k_split = mfma_split(tiles, ksteps, 8);
      c.grid = tiles * c.k_split;
    }
  } else if (M <= 64) {
    c.kind = SG_KIND_MFMA_TILE;
    c.m_tile = 16 * ceil_div(M, 16);
    c.rows = 64;
    c.waves = 4;
    c.k_unroll = kTileRing;
    const int tiles = ceil_div(N, c.rows);
    c.k_split = mfma_split(tiles, ksteps, 8);
    c.grid = tiles * c.k_split;
  } else {
    c.kind = SG_KIND_MFMA_DIRECT;
    const int mb = ceil_div(M, 16);
    c.m_tile = 16 * mb;
    c.rows = 1;
    c.k_unroll = direct_ring_depth(mb);
    const int tiles = ceil_div(N, 16);
    c.k_split = mfma_split(tiles, ksteps, 32);
    c.grid = tiles * c.k_split;
  }
  *out = c;
  return SG_OK;
}

extern "C" int sg_overlap_max_tokens(void) { return kOverlapMaxTokens; }

extern "C" int sg_overlap_gate(int M, int x_contiguous, int have_aux_stream, int have_events,
                               int enabled) {
  return (enabled && M > 0 && M <= kOverlapMaxTokens && x_contiguous && have_aux_stream &&
          have_events)
             ? 1
             : 0;
}

namespace sg {

// Workspace regions start on 256-byte boundaries.
size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
size_t ws_round(size_t b) { return round256(b); }

}  // namespace sg

extern "C" size_t sg_workspace_bytes(int op, int M, int N, int K) {
  sg_config_t c;
  if (sg_select(M, N, K, 0, &c) != SG_OK) return 0;
  if (c.kind == SG_KIND_NONE) return 0;
  const size_t S = static_cast<size_t>(c.k_split > 0 ? c.k_split : 1);
  const size_t plane = static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float);
  switch (op) {
    case SG_OP_GEMM:
      return c.k_split > 1 ? sg::round256(S * plane) : 0;
    case SG_OP_FAB_FB: {
      // The F_A/beta stage always leaves partials for the F_B stage to sum.
      const size_t s = (c.kind == SG_KIND_GEMV_SMALLK) ? 1 : S;
      return sg::round256(s * plane);
    }
    case SG_OP_LATENT_TAIL: {
      // M = 1 with the whole row in one workgroup: the GEMV normalises the
      // latent in LDS (no workspace).  Otherwise the bf16 normalised latent
      // [M,K] goes to the workspace first, followed by any split partials.
      const bool gemv1 = (M == 1) && (c.kind == SG_KIND_GEMV_SMALLK ||
                                      ((c.kind == SG_KIND_GEMV_ROW || c.kind == SG_KIND_GEMV_SPLITK) &&
                                       c.k_split == 1));
      if (gemv1) return 0;
      const size_t part = (c.k_split > 1 && c.kind != SG_KIND_GEMV_SMALLK) ? sg::round256(S * plane) : 0;
      return sg::round256(static_cast<size_t>(M) * static_cast<size_t>(K) * 2) + part;
    }
    default:
      return 0;
  }
}

extern "C" const char* sg_strerror(int status) {
  switch (status) {
    case SG_OK: return "ok";
    case SG_ERR_INVALID_ARG: return "invalid argument";
    case SG_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case SG_ERR_MISALIGNED: return "misaligned pointer or row stride";
    case SG_ERR_WORKSPACE: return "workspace missing or too small";
    case SG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* sg_version(void) { return "0.1.0"; }

extern "C" size_t sg_kda_workspace_bytes(int which, int M, int K, int n_qkvg, int n_ab) {
  if (M <= 0 || K < 0 || n_qkvg < 0 || n_ab <= 0) return 0;
  if (which == 0) {  // main: Q/K/V/G split-K partials
    sg_config_t c;
    if (n_qkvg == 0 || sg_select(M, n_qkvg, K, 0, &c) != SG_OK || c.kind == SG_KIND_NONE) return 0;
    return sg_workspace_bytes(SG_OP_GEMM, M, n_qkvg, K);
  }
  if (which == 1)  // aux: F_A/beta partials, as kda_fab_fb_proj
    return sg_workspace_bytes(SG_OP_FAB_FB, M, n_ab, K);
  return 0;
}
