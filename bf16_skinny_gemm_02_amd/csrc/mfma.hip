// bf16 MFMA paths for 2 <= M <= 256 (gfx950, v_mfma_f32_16x16x32_bf16).
//
// out[m,n] = sum_k a[m,k] * w[n,k] is a dense contraction once more than one
// activation row shares each weight byte, so the products go to the matrix
// cores; the weight stream from HBM stays the bound up to M = 64.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16)
// and the eight consecutive k of group (l / 16) of the 16x32 A operand, the
// same for the 16 columns of B, and receives D[4*(l/16) + v][l % 16],
// v = 0..3.  A = 16 weight rows (n), B = 16 activation rows (m): each lane
// ends with four consecutive n of one output row m.
//
// Three kernels, all staging both operands through an LDS ring filled by
// direct global->LDS copies:
//
//  * tile_kernel (SG_KIND_MFMA_TILE): a workgroup of NW waves owns 16*NW
//    weight rows (wave w: rows 16w..16w+15) and one K-range (all of K, or
//    1/k_split of it).  The range is walked in chunks of 4 k-steps (128 k,
//    256 bytes of a row).  For every chunk the weight tile and the activation
//    rows are copied straight from global memory into one slot of a C-slot
//    LDS ring (buffer_load ... lds, no registers, 1 KiB per instruction:
//    4 rows x 256 contiguous bytes), C-1 chunks ahead of the products.  All
//    waves share the activation copy; one barrier per chunk.
//  * wsplit_kernel (SG_KIND_MFMA_WAVESPLIT, M <= 16): a workgroup owns 16
//    weight rows; its 4 waves each walk a quarter of the K-range with a
//    private LDS ring (16 weight rows + the M activation rows per slot), so
//    the loop has no barrier.  The four wave sums meet in LDS in the fixed
//    order 0,1,2,3 at the end: no split-K partials and no second launch.
//  * block_kernel (SG_KIND_MFMA_BLOCK, M > 64): tile_kernel's ring over a
//    two-dimensional block, 64 weight rows x 128 activation rows, each wave
//    a 32 x 64 corner of it.
//
// LDS layout of one ring slot: rows of 16 pieces of 16 bytes.  Piece c of row
// r is stored at position c ^ (r & 15): the 16 lanes that read piece c of 16
// consecutive rows (one MFMA operand) hit 16 different 16-byte bank groups.
// The copies realise the swizzle on the global side: the lane that fills
// position p of row r loads piece p ^ (r & 15).
//
// Every kernel either stores bf16 (with the optional residual and the split
// output of the packed KDA projection) or fp32 split-K partials
// partial[s][m][n] for a later fixed-order sum.  Each output element's sum is
// formed in an order that depends only on K and the configuration, never on
// timing or on which tile holds the row.
#include "sg_device.h"
#include "sg_fused.h"
#include "sg_help.h"
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
  int sps;        // k-steps (32 k) per split
  int tile_rows;  // wave-split kernel: weight rows per workgroup (16, or 17..32 with NT = 2)
  const uint16_t* gamma;  // RMSNorm fold (wave-split kernel): gamma[K], else unused
  float eps;
  unsigned* arrive;  // in-launch hand-off (FB wave-split instances, sg_fused.h): the flag header
  int nslots;        // producer slots of the launch (one per workgroup of the F_A/beta segment)
  uint64_t* pairs;   // tile kernel, TAG instances: the first split's tagged sums (thread order)
  unsigned* sync;    // and the hand-off header (flag per tile of split 0, cursor per tile of split 1)
  int ntiles;        // tiles per K split (TAG instances)
};

// One launch covers one or two segments (independent problems whose
// workgroups share a flat grid) and, for the wave-split tile, optionally the
// F_B role of a fused launch.  Within a segment, workgroup `local` takes tile
// local % tiles of K-range local / tiles.
struct MfmaSeg {
  MfmaArgs g;
  int tiles;
  unsigned tiles_magic;  // quotient_magic(tiles)
  int wg_begin, wg_end;  // the segment's workgroups (empty range: unused)
};
struct MfmaLaunch {
  MfmaSeg seg[2];
  FbFuse fb;
};

// The segment's arguments are copied into registers once (uniform values in
// SGPRs), so nothing re-reads the kernel arguments inside the loops.  ONE
// (instances only ever launched with one segment): no selection, so the
// kernel arguments come in one round of scalar loads and the first copies
// go out sooner (measured: 0.1-0.5 us per launch).  The K-range index is
// quotient_by(): no division, and no branch for the compiler to schedule
// the argument loads around.
template <bool ONE = false>
__device__ __forceinline__ MfmaArgs pick_segment(const MfmaLaunch& L, int& tile, int& split,
                                                 int& local) {
  const int b = static_cast<int>(blockIdx.x);
  const MfmaSeg sg = (ONE || !(b >= L.seg[1].wg_begin && b < L.seg[1].wg_end)) ? L.seg[0] : L.seg[1];
  local = b - sg.wg_begin;
  split = quotient_by(local, sg.tiles, sg.tiles_magic);
  tile = local - split * sg.tiles;
  return sg.g;
}
template <bool ONE = false>
__device__ __forceinline__ MfmaArgs pick_segment(const MfmaLaunch& L, int& tile, int& split) {
  int local;
  return pick_segment<ONE>(L, tile, split, local);
}

constexpr int kKStep = 32;       // k per MFMA
constexpr int kChunkSteps = 4;   // k-steps per LDS ring chunk
constexpr int kPieces = 16;      // 16-byte pieces of a row per chunk (256 bytes)

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The residual values of the four outputs (m, n0 .. n0+3) a lane will store,
// requested when the kernel starts (before the ring's first chunks: loads
// complete in issue order, so no chunk wait waits for them) and widened only
// in the epilogue.  RES (a kernel instance launched for a segment with a
// residual and bf16 output): load4_bf16 (n0 is a multiple of 4).  Rows past
// M, a lane that stores nothing (`active` false, uniform per wave) and a
// segment without a residual read zeros and fetch nothing.  The loads are
// unconditional: a load under a branch would get a wait for every load in
// flight at the branch's end.  Without RES nothing is loaded.
struct Res4 {
  uint16_t v[4];
};

template <bool RES>
__device__ __forceinline__ Res4 load_res4(const MfmaArgs& g, int m, int n0, bool active = true) {
  Res4 r = {{0, 0, 0, 0}};
  if constexpr (RES) {
    const bool use = g.res != nullptr && g.partial == nullptr && active;
    load4_bf16(g.res, static_cast<int64_t>(g.M - 1) * g.ldr + g.N, static_cast<int64_t>(m) * g.ldr + n0,
               use, m < g.M, r.v);
  }
  return r;
}

// Stores the four outputs (m, n0 .. n0+3) a lane holds.
// Four consecutive outputs go out as one 16-byte (partials) or 8-byte (bf16)
// store when they lie in one row of one output and the address is aligned;
// otherwise element by element.  Partials are stored non-temporally: every
// workgroup writes them at its very end and the next launch reads them once.
// COHERENT (the F_A/beta segment of a one-launch F_A/beta -> F_B call): the
// partials go out as device-coherent stores for the F_B role to read.
// Rows n >= nlim (the next workgroup's, or past N) are not stored.
template <bool COHERENT = false>
__device__ __forceinline__ void store4(const MfmaArgs& g, const f32x4& acc, int m, int n0, int split,
                                       const Res4& res, int nlim = INT32_MAX) {
  if (m >= g.M) return;
  nlim = min(nlim, g.N);
  const bool whole = n0 + 3 < nlim;
  if (g.partial != nullptr) {
    float* p = g.partial + (static_cast<int64_t>(split) * g.M + m) * g.N + n0;
    if constexpr (COHERENT) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (n0 + v < nlim) store_coherent(p + v, acc[v]);
      return;
    }
    if (whole && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(p));
      return;
    }
  } else if (whole && !(g.n_split > 0 && n0 < g.n_split && n0 + 3 >= g.n_split)) {
    uint16_t* p = (g.n_split > 0 && n0 >= g.n_split) ? g.out2 + m * g.ldc2 + (n0 - g.n_split)
                                                       : g.out + m * g.ldc + n0;
    if ((reinterpret_cast<uintptr_t>(p) & 7u) == 0) {
      float v0 = acc[0], v1 = acc[1], v2 = acc[2], v3 = acc[3];
      if (g.res != nullptr) {
        v0 += bf16_to_f32(res.v[0]);
        v1 += bf16_to_f32(res.v[1]);
        v2 += bf16_to_f32(res.v[2]);
        v3 += bf16_to_f32(res.v[3]);
      }
      uint2 packed;
      packed.x = pack_bf16x2(v0, v1);
      packed.y = pack_bf16x2(v2, v3);
      *reinterpret_cast<uint2*>(p) = packed;
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int n = n0 + v;
    if (n >= nlim) continue;
    if (g.partial != nullptr) {
      g.partial[(static_cast<int64_t>(split) * g.M + m) * g.N + n] = acc[v];
    } else {
      float val = acc[v];
      if (g.res != nullptr) val += bf16_to_f32(res.v[v]);
      if (g.n_split > 0 && n >= g.n_split)
        g.out2[m * g.ldc2 + (n - g.n_split)] = f32_to_bf16(val);
      else
        g.out[m * g.ldc + n] = f32_to_bf16(val);
    }
  }
}

// ---- shared-activation LDS tile ------------------------------------------------

// MB: 16-row activation blocks (m_tile = 16*MB); NW: waves = 16-row weight
// blocks per workgroup; C: ring slots; XQ: activation rows copied per chunk,
// in groups of 4 (XQ*4 >= M).
//
// TAG (two K splits, bf16 out, one segment): the K-split sum happens in the
// launch.  A workgroup of split 0 (a producer) stores its fp32 sums as
// 8-byte pairs (value, generation), one atomic store each, in thread order,
// and advances its
// tile's flag without waiting; the workgroup of split 1 for the same tile (a
// consumer, dispatched after every producer) reads the pairs of the outputs
// it holds until each carries the generation (a bounded wait: NaN after a
// time-out), adds them to its own sums -- split 0's then split 1's, the order
// of the reduction launch -- and stores out = bf16(sum + residual).
// Generations as in sg_fused.h: the producer's is its flag + 1, the
// consumer waits for its cursor + 1; both advance, and the tiles share out
// the absent flags and cursors.
template <int MB, int NW, int C, int XQ, bool RES, bool TAG = false>
__global__ __launch_bounds__(NW * kWave) void tile_kernel(MfmaLaunch L) {
  extern __shared__ u32x4 lds[];
  int tile, split;
  const MfmaArgs g = pick_segment<TAG>(L, tile, split);
  // TAG: this call's generation, read before anything else is in flight.
  unsigned gen = 0u;
  if constexpr (TAG) gen = load_flag(g.sync + (split == 0 ? tile : kFbMaxProducers + tile)) + 1u;
  constexpr int WROWS = 16 * NW;
  constexpr int XROWS = 4 * XQ;
  constexpr int SLOT = (WROWS + XROWS) * kPieces;
  constexpr int XJ = (XQ + NW - 1) / NW;  // activation copies per wave per chunk
  constexpr int P = 4 + XJ;               // copies per wave per chunk
  constexpr int kInFlight = (C - 2) * P;  // copies allowed pending when a chunk is read
  static_assert(XROWS <= 16 * MB && XROWS > 16 * (MB - 1), "activation rows");
  static_assert(C >= 2, "ring");

  const int lane = lane_id();
  const int wave = wave_id();
  const int rl = lane & 15;
  const int kg = lane >> 4;
  const int K8 = g.K >> 3;
  const int KS = (g.K + kKStep - 1) / kKStep;
  const int s_begin = split * g.sps;
  const int nk = max(0, min(KS, s_begin + g.sps) - s_begin);
  const int npieces = nk * 4;
  const int nch = (nk + kChunkSteps - 1) / kChunkSteps;
  const int c0 = s_begin * 4;
  const int tile_row0 = tile * WROWS;
  const int tile_rows = min(WROWS, g.N - tile_row0);

  const rsrc_t wres = make_rsrc(g.w + static_cast<int64_t>(tile_row0) * g.ldw,
                                static_cast<uint32_t>(((tile_rows - 1) * g.ldw + g.K) * 2));
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
  const int dr = lane >> 4;   // row within a 4-row copy
  const int dp = lane & 15;   // position within the row

  // Copies of chunk q into slot q % C: this wave's 16 weight rows (4 copies)
  // and its share of the activation row groups.  Chunks past the range read
  // zeros (no memory traffic), so every wave issues the same count.
  auto issue = [&](int q) {
    u32x4* slot = lds + (q % C) * SLOT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + dr;
      const int pc = kPieces * q + (dp ^ (r & 15));
      const uint32_t off = (r < tile_rows && pc < npieces && c0 + pc < K8)
                               ? static_cast<uint32_t>((r * g.ldw + (c0 + pc) * 8) * 2)
                               : kOob;
      copy16_to_lds_nt(wres, slot + (16 * wave + 4 * i) * kPieces, off);
    }
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int grp = (wave + NW * j) % XQ;  // a repeated group rewrites identical bytes
      const int m = 4 * grp + dr;
      const int pc = kPieces * q + (dp ^ (m & 15));
      const uint32_t off = (m < g.M && pc < npieces && c0 + pc < K8)
                               ? static_cast<uint32_t>((m * g.lda + (c0 + pc) * 8) * 2)
                               : kOob;
      copy16_to_lds(xres, slot + (WROWS + 4 * grp) * kPieces, off);
    }
  };

  // The residual goes out before the ring's first chunks: loads complete in
  // issue order, so the chunk waits below never wait for it.  (TAG: only the
  // consumer stores, so only it loads the residual.)
  // Eight waves over 128 weight rows x 64 activation rows (QUAD): wave w
  // reads weight rows 32 (w & 3) .. +31 and activation rows 32 (w >> 2) ..
  // +31, four fragments per k-step instead of one weight and four activation
  // fragments, 20% fewer LDS reads for the same MFMAs (each output keeps its
  // k order).  The copies are the same.  acc[2 f + a]: weight fragment f,
  // activation fragment a.
  constexpr bool QUAD = NW == 8 && MB == 4 && !TAG;
  const int wq = wave & 3;
  const int wm = wave >> 2;
  const int n0 = tile_row0 + 16 * wave + 4 * kg;
  Res4 res[MB];
  if constexpr (QUAD) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        res[2 * f + a] = load_res4<RES>(g, 32 * wm + 16 * a + rl, tile_row0 + 32 * wq + 16 * f + 4 * kg);
  } else {
#pragma unroll
    for (int a = 0; a < MB; ++a) res[a] = load_res4<RES>(g, 16 * a + rl, n0, !TAG || split == 1);
  }

#pragma unroll
  for (int q = 0; q < C - 1; ++q) issue(q);

  f32x4 acc[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wrow = (16 * wave + rl) * kPieces;
  for (int q = 0; q < nch; ++q) {
    // Chunk q has landed for this wave; the barrier makes it so for all, and
    // also means every wave has finished reading slot (q - 1) % C, which the
    // next copy overwrites.
    wait_vmcnt<kInFlight>();
    __builtin_amdgcn_s_barrier();
    issue(q + C - 1);
    const u32x4* slot = lds + (q % C) * SLOT;
    if constexpr (QUAD) {
      u32x4 wf[kChunkSteps][2], xf[kChunkSteps][2];
#pragma unroll
      for (int t = 0; t < kChunkSteps; ++t) {
#pragma unroll
        for (int f = 0; f < 2; ++f) wf[t][f] = slot[(32 * wq + 16 * f + rl) * kPieces + ((4 * t + kg) ^ rl)];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int x0 = 32 * wm + 16 * a + rl;
          const int xr = x0 < XROWS ? x0 : XROWS - 1;
          xf[t][a] = slot[(WROWS + xr) * kPieces + ((4 * t + kg) ^ (xr & 15))];
        }
      }
#pragma unroll
      for (int t = 0; t < kChunkSteps; ++t)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int a = 0; a < 2; ++a) acc[2 * f + a] = mfma16(wf[t][f], xf[t][a], acc[2 * f + a]);
    } else {
      u32x4 wf[kChunkSteps], xf[kChunkSteps][MB];
#pragma unroll
      for (int t = 0; t < kChunkSteps; ++t) {
        wf[t] = slot[wrow + ((4 * t + kg) ^ rl)];
#pragma unroll
        for (int a = 0; a < MB; ++a) {
          // Rows past the copied ones only feed outputs that are not stored.
          const int xr = (16 * a + rl < XROWS) ? 16 * a + rl : XROWS - 1;
          xf[t][a] = slot[(WROWS + xr) * kPieces + ((4 * t + kg) ^ (xr & 15))];
        }
      }
#pragma unroll
      for (int t = 0; t < kChunkSteps; ++t)
#pragma unroll
        for (int a = 0; a < MB; ++a) acc[a] = mfma16(wf[t], xf[t][a], acc[a]);
    }
  }
  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released

  if constexpr (TAG) {
    // The pairs of one tile in thread order: pair (a, v) of thread t at
    // ((tile * MB + a) * 4 + v) * 64 NW + t, so that every store and every
    // load of them is one contiguous 512-byte access per wave.  Producer and
    // consumer threads hold the same outputs (same tile, same code).
    const int lane64 = lane_id();
    const int t = static_cast<int>(threadIdx.x);
    uint64_t* tp = g.pairs + static_cast<int64_t>(tile) * MB * 4 * (NW * kWave) + t;
    if (split == 0) {
      // Producer: the sums of the outputs (m, n0 .. n0 + 3) this thread holds
      // (every slot written, outputs past M or N included: the consumer
      // ignores them).
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const float v4[4] = {acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint64_t pair = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, v4[v])) |
                                (static_cast<uint64_t>(gen) << 32);
          __hip_atomic_store(tp + (a * 4 + v) * (NW * kWave), pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // The tile's flag (nothing in this launch waits for it: it keeps the
      // generations for later calls), and this tile's share of the absent
      // slots, at most one store per lane.
      if (wave == 0) {
        if (lane64 == 0) store_flag(g.sync + tile, gen);
        for (int q = g.ntiles + tile + g.ntiles * lane64; q < kFbMaxProducers; q += g.ntiles * kWave)
          store_flag(g.sync + q, gen);
      }
      return;
    }
    // Consumer: read the producer's pairs of this thread's outputs until all
    // carry the generation, then add them first.
    uint64_t pv[MB][4];
    bool ok = false;
    for (int polls = 0;;) {
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          pv[a][v] = __hip_atomic_load(tp + (a * 4 + v) * (NW * kWave), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool mine = true;
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) mine = mine && static_cast<unsigned>(pv[a][v] >> 32) == gen;
      ok = __builtin_amdgcn_ballot_w64(!mine) == 0;
      if (ok || ++polls >= kFbSpinLimit) break;
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      const f32x4 p0 = f32x4{__builtin_bit_cast(float, static_cast<uint32_t>(pv[a][0])),
                             __builtin_bit_cast(float, static_cast<uint32_t>(pv[a][1])),
                             __builtin_bit_cast(float, static_cast<uint32_t>(pv[a][2])),
                             __builtin_bit_cast(float, static_cast<uint32_t>(pv[a][3]))};
      acc[a] = ok ? p0 + acc[a] : f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
#pragma unroll
    for (int a = 0; a < MB; ++a) store4(g, acc[a], 16 * a + rl, n0, split, res[a]);
    if (wave == 0) {
      unsigned* cursors = g.sync + kFbMaxProducers;
      if (lane64 == 0) store_flag(cursors + tile, gen);
      for (int q = g.ntiles + tile + g.ntiles * lane64; q < kFbMaxConsumers; q += g.ntiles * kWave)
        store_flag(cursors + q, gen);
    }
    return;
  }
  if constexpr (QUAD) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        store4(g, acc[2 * f + a], 32 * wm + 16 * a + rl, tile_row0 + 32 * wq + 16 * f + 4 * kg, split,
               res[2 * f + a]);
  } else {
#pragma unroll
    for (int a = 0; a < MB; ++a) store4(g, acc[a], 16 * a + rl, n0, split, res[a]);
  }
}

// ---- wave-split LDS tile (M <= 16) ------------------------------------------------

constexpr int kSplitWaves = 4;
constexpr int kHelpRing = 3;  // ring slots of the one-launch projection's tile
// RMSNorm fold: the latent row is read in at most this many 16-byte chunks
// per lane (d_latent <= 2048).
constexpr int kFoldChunks = 4;
constexpr int kFoldMaxK = kFoldChunks * kWave * 8;
// 16-byte pieces per normalised activation row in LDS (the longest row).
constexpr int kFoldStride = kFoldChunks * kWave;

// NORM (the latent-MoE tail): the activation rows are the raw latent L.  Each
// wave reads whole rows of it into registers (rows m = wave + 4j), with the
// whole of gamma, while its ring's first chunks are in flight; it computes
// r[m] = 1/sqrt(mean(L[m,:]^2) + eps) and writes n = bf16((L * r) * gamma),
// the rounding of the bf16 normalised latent that a separate RMSNorm kernel
// would store, into an LDS region behind the rings that holds every
// activation row over all of K.  One barrier, and the chunk loop reads its
// activation fragments from there: the rings carry the weight rows only, so
// no chunk refill waits for normalisation arithmetic and the latent crosses
// L2 once per workgroup.
//
// FB (instances of the one-launch F_A/beta -> F_B branch only): workgroups in
// L.fb's range run the F_B role, and the segment with `arrive` set hands its
// partials over (sg_fused.h).  Other instances carry none of that code.
//
// NT: 16-row weight fragments per workgroup (1, or 2 for a workgroup of
// 17..32 rows: the second fragment's rows past g.tile_rows read zeros and are
// not stored), so that e.g. 7168 rows make exactly 256 workgroups of 28.
template <int XQ, int C, bool NORM, bool RES, bool FB, int NT, bool ONE = true>
__device__ __forceinline__ void wsplit_body(const MfmaLaunch& L, u32x4* lds) {
  if constexpr (FB) {
    static_assert(kSplitWaves * kWave == kFbThreads && !NORM && !RES, "F_B role instances");
    const int b = static_cast<int>(blockIdx.x);
    if (b >= L.fb.wg_begin && b < L.fb.wg_end) {
      fb_role(L.fb, b, lds);
      return;
    }
  }
  int tile, split, slot;
  const MfmaArgs g = pick_segment<ONE>(L, tile, split, slot);
  // Every argument the ring's first copies need, requested in one round of
  // scalar loads (left to itself the compiler issues a second round behind
  // a wait for the first, which holds back the copies).
  if constexpr (ONE)
    asm volatile("" ::"s"(g.w), "s"(g.ldw), "s"(g.a), "s"(g.lda), "s"(g.M), "s"(g.N), "s"(g.K), "s"(g.sps),
                 "s"(g.tile_rows), "s"(g.res), "s"(g.ldr), "s"(g.out), "s"(g.ldc), "s"(g.gamma));
  // Hand-off: this workgroup's producer flag (slot = its index in the
  // segment), read before anything else is in flight.
  unsigned prev = 0u;
  if constexpr (FB) prev = g.arrive != nullptr ? load_flag(g.arrive + slot) : 0u;
  constexpr int XROWS = 4 * XQ;
  constexpr int WROWS = 16 * NT;
  constexpr int SLOT = (WROWS + (NORM ? 0 : XROWS)) * kPieces;  // NORM: weight rows only
  constexpr int P = 4 * NT + (NORM ? 0 : XQ);                  // copies per chunk
  constexpr int kInFlight = (C - 2) * P;
  static_assert(XQ >= 1 && XQ <= 4 && C >= 2 && (NT == 1 || NT == 2), "configuration");

  const int lane = lane_id();
  const int wave = wave_id();
  const int rl = lane & 15;
  const int kg = lane >> 4;
  const int K8 = g.K >> 3;
  const int KS = (g.K + kKStep - 1) / kKStep;
  const int s_begin = split * g.sps;
  const int len = max(0, min(KS, s_begin + g.sps) - s_begin);
  const int per = (len + kSplitWaves - 1) / kSplitWaves;
  const int w_begin = s_begin + wave * per;
  const int nk = max(0, min(s_begin + len, w_begin + per) - w_begin);
  const int npieces = nk * 4;
  const int nch = (nk + kChunkSteps - 1) / kChunkSteps;
  const int c0 = w_begin * 4;
  const int row0 = tile * g.tile_rows;
  const int rows = min(g.tile_rows, g.N - row0);
  u32x4* ring = lds + wave * C * SLOT;

  const rsrc_t wres = make_rsrc(g.w + static_cast<int64_t>(row0) * g.ldw,
                                static_cast<uint32_t>(((rows - 1) * g.ldw + g.K) * 2));
  const rsrc_t xres = make_rsrc(g.a, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
  const int dr = lane >> 4;
  const int dp = lane & 15;
  // Behind the rings (NORM): the normalised activation, XROWS rows of
  // kFoldStride 16-byte pieces, piece p of row m at (p & ~15) | ((p ^ m) & 15)
  // so that the 16 rows of a fragment read fall in distinct banks.
  u32x4* xs = lds + kSplitWaves * C * SLOT;
  auto issue = [&](int q) {
    u32x4* slot = ring + (q % C) * SLOT;
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i) {
      const int r = 4 * i + dr;
      const int pc = kPieces * q + (dp ^ (r & 15));
      const uint32_t off = (r < rows && pc < npieces && c0 + pc < K8)
                               ? static_cast<uint32_t>((r * g.ldw + (c0 + pc) * 8) * 2)
                               : kOob;
      copy16_to_lds_nt(wres, slot + 4 * i * kPieces, off);
    }
    if constexpr (!NORM) {
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        const int m = 4 * j + dr;
        const int pc = kPieces * q + (dp ^ m);
        const uint32_t off = (m < g.M && pc < npieces && c0 + pc < K8)
                                 ? static_cast<uint32_t>((m * g.lda + (c0 + pc) * 8) * 2)
                                 : kOob;
        copy16_to_lds(xres, slot + (WROWS + 4 * j) * kPieces, off);
      }
    }
  };

  // The residual and (NORM) gamma and the whole latent rows go out before the
  // ring's first chunks: loads complete in issue order, so neither the
  // RMSNorm below nor the chunk waits of the loop wait for the other's loads.
  Res4 res[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) res[nt] = load_res4<RES>(g, rl, row0 + 16 * nt + 4 * kg, wave == 0);
  u32x4 gv[NORM ? kFoldChunks : 1];
  u32x4 lv[NORM ? XQ : 1][kFoldChunks];
  if constexpr (NORM) {
    const rsrc_t gres = make_rsrc(g.gamma, static_cast<uint32_t>(g.K * 2));
#pragma unroll
    for (int i = 0; i < kFoldChunks; ++i) {
      const int c = lane + kWave * i;
      gv[i] = buf_load(gres, c < K8 ? static_cast<uint32_t>(c * 16) : kOob);
    }
#pragma unroll
    for (int j = 0; j < XQ; ++j) {
      const int m = wave + 4 * j;
#pragma unroll
      for (int i = 0; i < kFoldChunks; ++i) {
        const int c = lane + kWave * i;
        const uint32_t off =
            (m < g.M && c < K8) ? static_cast<uint32_t>((m * g.lda + c * 8) * 2) : kOob;
        lv[j][i] = buf_load(xres, off);
      }
    }
  }

#pragma unroll
  for (int q = 0; q < C - 1; ++q) issue(q);
  // Nothing below moves above the ring's first copies (the RMSNorm's waits
  // for the latent rows would otherwise hold them back).
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NORM) {
#pragma unroll
    for (int j = 0; j < XQ; ++j) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < kFoldChunks; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l0 = bf16_lo(lv[j][i][e]), l1 = bf16_hi(lv[j][i][e]);
          ss = fmaf(l0, l0, ss);
          ss = fmaf(l1, l1, ss);
        }
      ss = wave_allreduce(ss);
      const int m = wave + 4 * j;
      const float r = m < g.M ? __frsqrt_rn(ss / static_cast<float>(g.K) + g.eps) : 0.f;
#pragma unroll
      for (int i = 0; i < kFoldChunks; ++i) {
        const int c = lane + kWave * i;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(bf16_lo(lv[j][i][e]) * r * bf16_lo(gv[i][e]),
                             bf16_hi(lv[j][i][e]) * r * bf16_hi(gv[i][e]));
        xs[m * kFoldStride + ((c & ~15) | ((c ^ m) & 15))] = o;
      }
    }
    // Every activation row is in LDS.  A plain barrier after the LDS writes:
    // a __syncthreads would also wait for the ring's chunks in flight (the
    // global->LDS copies count as memory loads), which no other wave reads.
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
  }

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int xr = rl < XROWS ? rl : XROWS - 1;
  for (int q = 0; q < nch; ++q) {
    wait_vmcnt<kInFlight>();  // this wave's chunk q has landed (its own ring)
    const u32x4* slot = ring + (q % C) * SLOT;
    u32x4 wf[kChunkSteps][NT], xf[kChunkSteps];
#pragma unroll
    for (int t = 0; t < kChunkSteps; ++t) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wf[t][nt] = slot[(16 * nt + rl) * kPieces + ((4 * t + kg) ^ rl)];
      if constexpr (NORM) {
        // Pieces past the wave's K-range meet zero weights; the clamp keeps
        // the read inside the row.
        const int p = min(c0 + kPieces * q + 4 * t + kg, kFoldStride - 1);
        xf[t] = xs[xr * kFoldStride + ((p & ~15) | ((p ^ xr) & 15))];
      } else {
        xf[t] = slot[(WROWS + xr) * kPieces + ((4 * t + kg) ^ xr)];
      }
    }
    wait_lgkmcnt0();  // the slot is in registers before the copy below refills the ring
    issue(q + C - 1);
#pragma unroll
    for (int t = 0; t < kChunkSteps; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16(wf[t][nt], xf[t], acc[nt]);
  }
  wait_vmcnt<0>();
  __syncthreads();  // every ring is drained: LDS is reused for the wave sums

  float* red = reinterpret_cast<float*>(lds);
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(((wave - 1) * NT + nt) * 4 + v) * kWave + lane] = acc[nt][v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kSplitWaves - 1; ++w)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[nt][v] += red[((w * NT + nt) * 4 + v) * kWave + lane];
  const int nlim = row0 + rows;
  if constexpr (FB) {
    if (g.arrive != nullptr) {  // wave 0 alone stores: one producer slot per workgroup
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        store4<true>(g, acc[nt], rl, row0 + 16 * nt + 4 * kg, split, res[nt], nlim);
      produce(g.arrive, slot, g.nslots, prev);
      return;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) store4(g, acc[nt], rl, row0 + 16 * nt + 4 * kg, split, res[nt], nlim);
}

template <int XQ, int C, bool NORM, bool RES, bool FB, int NT>
__global__ __launch_bounds__(kSplitWaves * kWave) void wsplit_kernel(MfmaLaunch L) {
  extern __shared__ u32x4 lds[];
  wsplit_body<XQ, C, NORM, RES, FB, NT>(L, lds);
}

// The one-launch KDA projection (sg_help.h): the four waves of the wave-split
// tile stream the Q/K/V/G rows (16 per workgroup, all of K, bf16 out); a
// fifth wave runs the F_A/beta -> F_B chain in LDS behind the four rings, at
// the highest issue priority among the workgroup's waves, so that its few
// loads go out ahead of the rings' copies (the chain, not the stream, ends
// the launch).  The helper meets the tile's two epilogue barriers once its
// own work is done.
template <int XQ>
__global__ __launch_bounds__((kSplitWaves + 1) * kWave) void wsplit_help_kernel(MfmaLaunch L, HelpArgs H) {
  extern __shared__ u32x4 lds[];
  if (wave_id() == kSplitWaves) {
    __builtin_amdgcn_s_setprio(3);
    constexpr int kRing = kSplitWaves * kHelpRing * (16 + 4 * XQ) * kPieces;
    help_wave<XQ>(H, static_cast<int>(blockIdx.x), lds + kRing);
    __syncthreads();
    __syncthreads();
    return;
  }
  // The main waves' quicker start (one segment, one round of argument
  // loads) measured even at M <= 4, 0.5 us faster at M = 9..16 and 0.4 us
  // slower at M = 5..8 (with every host sleep tried there), where the units'
  // loads then queue behind more ring copies.
  wsplit_body<XQ, kHelpRing, false, false, false, 1, XQ != 2>(L, lds);
}

// ---- two-dimensional LDS block tile (M > 64) ----------------------------------------

// A workgroup of 4 waves owns a block of kBlkRows weight rows x kBlkM
// activation rows and one K-range; wave w computes weight rows 32 (w & 1) ..
// +31 against activation rows 64 (w >> 1) .. +63 (2 x 4 MFMA tiles), so each
// k-step reads 6 fragments from LDS for 8 MFMAs.  The ring is tile_kernel's:
// chunks of 128 k, both operands copied global->LDS (weights non-temporal),
// one barrier per chunk.
constexpr int kBlkRows = 64;
constexpr int kBlkM = 128;
constexpr int kBlkWaves = 4;

// Workgroup -> (weight tile, activation block).  Consecutive workgroups go to
// the 8 XCDs in turn, so the activation blocks of one weight tile are given
// to workgroups 8 apart: the same XCD, whose L2 then serves the tile's second
// read.
__device__ __forceinline__ void block_coords(int tile, int ntiles, int mblocks, int& nt, int& mb) {
  const int G = 8 * mblocks;
  const int grp = tile / G;
  const int r = tile - grp * G;
  const int nrem = min(8, ntiles - grp * 8);
  mb = r / nrem;
  nt = grp * 8 + (r - mb * nrem);
}

// RES: 0 no residual; 1 the residual in the MFMA layout (load_res4); 2 a
// residual with 16-byte aligned rows, read in row order (16-byte pieces of
// whole rows, the pieces each thread stores) and added in the row-order
// epilogue.
template <int C, int RES>
__global__ __launch_bounds__(kBlkWaves * kWave) void block_kernel(MfmaLaunch L) {
  extern __shared__ u32x4 lds[];
  int tile, split;
  // RES == 2 (one segment with row-aligned residual and output) takes the
  // single-segment selection.
  const MfmaArgs g = pick_segment<RES == 2>(L, tile, split);
  constexpr int SLOT = (kBlkRows + kBlkM) * kPieces;
  constexpr int WC = kBlkRows / 4 / kBlkWaves;  // weight copies per wave per chunk
  constexpr int XC = kBlkM / 4 / kBlkWaves;     // activation copies per wave per chunk
  constexpr int kInFlight = (C - 2) * (WC + XC);
  static_assert(C >= 2, "ring");

  const int lane = lane_id();
  const int wave = wave_id();
  const int rl = lane & 15;
  const int kg = lane >> 4;
  const int ntiles = (g.N + kBlkRows - 1) / kBlkRows;
  const int mblocks = (g.M + kBlkM - 1) / kBlkM;
  int nt, mb;
  block_coords(tile, ntiles, mblocks, nt, mb);
  const int K8 = g.K >> 3;
  const int KS = (g.K + kKStep - 1) / kKStep;
  const int s_begin = split * g.sps;
  const int nk = max(0, min(KS, s_begin + g.sps) - s_begin);
  const int npieces = nk * 4;
  const int nch = (nk + kChunkSteps - 1) / kChunkSteps;
  const int c0 = s_begin * 4;
  const int row0 = nt * kBlkRows;
  const int tile_rows = min(kBlkRows, g.N - row0);
  const int m0 = mb * kBlkM;
  const int m_rows = min(kBlkM, g.M - m0);

  const rsrc_t wres = make_rsrc(g.w + static_cast<int64_t>(row0) * g.ldw,
                                static_cast<uint32_t>(((tile_rows - 1) * g.ldw + g.K) * 2));
  const rsrc_t xres = make_rsrc(g.a + static_cast<int64_t>(m0) * g.lda,
                                static_cast<uint32_t>(((m_rows - 1) * g.lda + g.K) * 2));
  const int dr = lane >> 4;
  const int dp = lane & 15;
  auto issue = [&](int q) {
    u32x4* slot = lds + (q % C) * SLOT;
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      const int r = 4 * (wave * WC + i) + dr;
      const int pc = kPieces * q + (dp ^ (r & 15));
      const uint32_t off = (r < tile_rows && pc < npieces && c0 + pc < K8)
                               ? static_cast<uint32_t>((r * g.ldw + (c0 + pc) * 8) * 2)
                               : kOob;
      copy16_to_lds_nt(wres, slot + 4 * (wave * WC + i) * kPieces, off);
    }
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int m = 4 * (wave * XC + j) + dr;
      const int pc = kPieces * q + (dp ^ (m & 15));
      const uint32_t off = (m < m_rows && pc < npieces && c0 + pc < K8)
                               ? static_cast<uint32_t>((m * g.lda + (c0 + pc) * 8) * 2)
                               : kOob;
      copy16_to_lds(xres, slot + (kBlkRows + 4 * (wave * XC + j)) * kPieces, off);
    }
  };

  // The residual goes out before the ring's first chunks (see tile_kernel).
  const int wr0 = 32 * (wave & 1);   // this wave's first weight row in the block
  const int xr0 = 64 * (wave >> 1);  // and first activation row
  Res4 res[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      res[i][j] = load_res4<RES == 1>(g, m0 + xr0 + 16 * j + rl, row0 + wr0 + 16 * i + 4 * kg);
  constexpr int kPer = kBlkRows / 8;                       // 16-byte pieces per block row
  constexpr int kRowPieces = kBlkM * kPer / (kBlkWaves * kWave);  // per thread
  u32x4 rrow[RES == 2 ? kRowPieces : 1];
  if constexpr (RES == 2) {
    // Buffer from the residual to its end rounded up to 16 bytes: every
    // piece lies wholly inside or outside it, and none crosses a page.
    const int64_t span = (static_cast<int64_t>(g.M - 1) * g.ldr + g.N) * 2;
    const rsrc_t rres = make_rsrc(g.res, static_cast<uint32_t>((span + 15) & ~static_cast<int64_t>(15)));
#pragma unroll
    for (int q = 0; q < kRowPieces; ++q) {
      const int c = static_cast<int>(threadIdx.x) + q * kBlkWaves * kWave;
      const int ml = c / kPer, nl = (c - ml * kPer) * 8;
      const int m = m0 + ml, n = row0 + nl;
      rrow[q] = buf_load(rres, (m < g.M && n < g.N)
                                   ? static_cast<uint32_t>((static_cast<int64_t>(m) * g.ldr + n) * 2)
                                   : kOob);
    }
  }

#pragma unroll
  for (int q = 0; q < C - 1; ++q) issue(q);

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < nch; ++q) {
    wait_vmcnt<kInFlight>();
    __builtin_amdgcn_s_barrier();
    issue(q + C - 1);
    const u32x4* slot = lds + (q % C) * SLOT;
#pragma unroll
    for (int t = 0; t < kChunkSteps; ++t) {
      const int pos = (4 * t + kg) ^ rl;  // every fragment row is 16-aligned + rl
      u32x4 wf[2], xf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) wf[i] = slot[(wr0 + 16 * i + rl) * kPieces + pos];
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = slot[(kBlkRows + xr0 + 16 * j + rl) * kPieces + pos];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(wf[i], xf[j], acc[i][j]);
    }
  }
  wait_vmcnt<0>();  // no copy may land after the workgroup's LDS is released

  // bf16 output with 16-byte aligned rows: the block goes through LDS in row
  // order, so each output row leaves as whole 16-byte pieces (8 lanes per
  // 128-byte row segment) instead of 8-byte pieces of 16 rows per store.
  const bool rows16 = g.partial == nullptr && g.n_split <= 0 &&
                      (reinterpret_cast<uintptr_t>(g.out) & 15u) == 0 && (g.ldc & 7) == 0;
  if constexpr (RES == 2) {
    // (the launcher picks RES 2 only for 16-byte aligned output rows)
    constexpr int LDF = kBlkRows + 4;  // fp32 per LDS row (padded against bank conflicts)
    float* tf = reinterpret_cast<float*>(lds);
    __syncthreads();  // every wave has finished reading the ring
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(tf + (xr0 + 16 * j + rl) * LDF + wr0 + 16 * i + 4 * kg) = acc[i][j];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kRowPieces; ++q) {
      const int c = static_cast<int>(threadIdx.x) + q * kBlkWaves * kWave;
      const int ml = c / kPer, nl = (c - ml * kPer) * 8;
      const int m = m0 + ml, n = row0 + nl;
      if (m >= g.M || n >= g.N) continue;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(tf + ml * LDF + nl);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(tf + ml * LDF + nl + 4);
      const u32x4 r = rrow[q];
      u32x4 o;
      o[0] = pack_bf16x2(a0[0] + bf16_lo(r[0]), a0[1] + bf16_hi(r[0]));
      o[1] = pack_bf16x2(a0[2] + bf16_lo(r[1]), a0[3] + bf16_hi(r[1]));
      o[2] = pack_bf16x2(a1[0] + bf16_lo(r[2]), a1[1] + bf16_hi(r[2]));
      o[3] = pack_bf16x2(a1[2] + bf16_lo(r[3]), a1[3] + bf16_hi(r[3]));
      uint16_t* dst = g.out + static_cast<int64_t>(m) * g.ldc + n;
      if (n + 7 < g.N) {
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        for (int e = 0; e < g.N - n; ++e) dst[e] = static_cast<uint16_t>(o[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
  if (rows16) {
    constexpr int LD = kBlkRows + 8;  // bf16 per LDS row (padded against bank conflicts)
    uint16_t* tl = reinterpret_cast<uint16_t*>(lds);
    __syncthreads();  // every wave has finished reading the ring
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = xr0 + 16 * j + rl, nl = wr0 + 16 * i + 4 * kg;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = acc[i][j][e] + ((RES == 1 && g.res != nullptr) ? bf16_to_f32(res[i][j].v[e]) : 0.f);
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(tl + ml * LD + nl) = pk;
      }
    __syncthreads();
    constexpr int kPer = kBlkRows / 8;  // 16-byte pieces per row
    for (int c = static_cast<int>(threadIdx.x); c < kBlkM * kPer; c += kBlkWaves * kWave) {
      const int ml = c / kPer, nl = (c - ml * kPer) * 8;
      const int m = m0 + ml, n = row0 + nl;
      if (m >= g.M || n >= g.N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(tl + ml * LD + nl);
      uint16_t* dst = g.out + static_cast<int64_t>(m) * g.ldc + n;
      if (n + 7 < g.N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        const uint16_t* sv = tl + ml * LD + nl;
        for (int e = 0; e < g.N - n; ++e) dst[e] = sv[e];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store4(g, acc[i][j], m0 + xr0 + 16 * j + rl, row0 + wr0 + 16 * i + 4 * kg, split, res[i][j]);
}

// ---- launchers -------------------------------------------------------------------

// One attribute call per kernel instance and device (the ring can exceed the default
// 64 KiB of dynamic LDS).
template <int MB, int NW, int C, int XQ, bool RES, bool TAG = false>
hipError_t launch_tile_inst(const MfmaLaunch& L, int wgs, hipStream_t s) {
  auto kern = tile_kernel<MB, NW, C, XQ, RES, TAG>;
  static std::atomic<bool> lds_set[kLdsAttrDevices];
  const hipError_t attr = ensure_lds_limit(reinterpret_cast<const void*>(kern), kMfmaMaxLds, lds_set);
  if (attr != hipSuccess) return attr;
  return launch_kernel(kern, dim3(wgs), dim3(NW * kWave), tile_lds_bytes(NW, C, XQ), s, L);
}

template <int XQ, int C, bool NORM, bool RES, bool FB = false, int NT = 1>
hipError_t launch_wsplit_inst(const MfmaLaunch& L, int wgs, hipStream_t s) {
  auto kern = wsplit_kernel<XQ, C, NORM, RES, FB, NT>;
  static std::atomic<bool> lds_set[kLdsAttrDevices];
  const hipError_t attr = ensure_lds_limit(reinterpret_cast<const void*>(kern), kMfmaMaxLds, lds_set);
  if (attr != hipSuccess) return attr;
  return launch_kernel(kern, dim3(wgs), dim3(kSplitWaves * kWave), wsplit_lds_bytes(C, XQ, NORM, NT), s,
                       L);
}

template <bool NORM, bool RES>
hipError_t launch_wsplit_xq(const MfmaLaunch& L, int XQ, int C, int NT, int wgs, hipStream_t s) {
  if (NT == 2) {  // 17..32 rows per workgroup, one workgroup per CU
    if (C != 3) return hipErrorInvalidValue;
    switch (XQ) {
      case 1: return launch_wsplit_inst<1, 3, NORM, RES, false, 2>(L, wgs, s);
      case 2: return launch_wsplit_inst<2, 3, NORM, RES, false, 2>(L, wgs, s);
      case 3: return launch_wsplit_inst<3, 3, NORM, RES, false, 2>(L, wgs, s);
      case 4: return launch_wsplit_inst<4, 3, NORM, RES, false, 2>(L, wgs, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (NT != 1) return hipErrorInvalidValue;
  if (C == 2) {  // 9 <= M <= 16, two workgroups per CU
    switch (XQ) {
      case 3: return launch_wsplit_inst<3, 2, NORM, RES>(L, wgs, s);
      case 4: return launch_wsplit_inst<4, 2, NORM, RES>(L, wgs, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (C != 3) return hipErrorInvalidValue;
  switch (XQ) {
    case 1: return launch_wsplit_inst<1, 3, NORM, RES>(L, wgs, s);
    case 2: return launch_wsplit_inst<2, 3, NORM, RES>(L, wgs, s);
    case 3: return launch_wsplit_inst<3, 3, NORM, RES>(L, wgs, s);
    case 4: return launch_wsplit_inst<4, 3, NORM, RES>(L, wgs, s);
    default: return hipErrorInvalidValue;
  }
}

// The one-launch F_A/beta -> F_B instances (no fold, no residual).
hipError_t launch_wsplit_fb(const MfmaLaunch& L, int XQ, int C, int wgs, hipStream_t s) {
  if (C == 2) {
    switch (XQ) {
      case 3: return launch_wsplit_inst<3, 2, false, false, true>(L, wgs, s);
      case 4: return launch_wsplit_inst<4, 2, false, false, true>(L, wgs, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (C != 3) return hipErrorInvalidValue;
  switch (XQ) {
    case 1: return launch_wsplit_inst<1, 3, false, false, true>(L, wgs, s);
    case 2: return launch_wsplit_inst<2, 3, false, false, true>(L, wgs, s);
    case 3: return launch_wsplit_inst<3, 3, false, false, true>(L, wgs, s);
    case 4: return launch_wsplit_inst<4, 3, false, false, true>(L, wgs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int C, int RES>
hipError_t launch_block_inst(const MfmaLaunch& L, int wgs, hipStream_t s) {
  auto kern = block_kernel<C, RES>;
  static std::atomic<bool> lds_set[kLdsAttrDevices];
  const hipError_t attr = ensure_lds_limit(reinterpret_cast<const void*>(kern), kMfmaMaxLds, lds_set);
  if (attr != hipSuccess) return attr;
  return launch_kernel(kern, dim3(wgs), dim3(kBlkWaves * kWave), block_lds_bytes(C), s, L);
}

int ksteps_of(int K) { return (K + kKStep - 1) / kKStep; }

// Workgroup tiles of one K-range: c.rows weight rows each (16 * NW for
// TILE, 16 or 17..32 for WAVESPLIT), or (BLOCK) 64 weight rows x 128
// activation rows.
int tiles_of(const sg_config_t& c, int M, int N) {
  if (c.kind == SG_KIND_MFMA_BLOCK)
    return ((N + kBlkRows - 1) / kBlkRows) * ((M + kBlkM - 1) / kBlkM);
  return (N + c.rows - 1) / c.rows;
}

}  // namespace

size_t tile_lds_bytes(int nw, int c, int xq) {
  return static_cast<size_t>(c) * (16 * nw + 4 * xq) * kPieces * 16;
}

size_t block_lds_bytes(int c) {
  return static_cast<size_t>(c) * (kBlkRows + kBlkM) * kPieces * 16;
}

size_t wsplit_lds_bytes(int c, int xq, bool norm, int nt) {
  // NORM: weight rows only in the rings, then the normalised activation rows.
  const size_t rings = static_cast<size_t>(kSplitWaves) * c * (16 * nt + (norm ? 0 : 4 * xq)) * kPieces * 16;
  return rings + (norm ? static_cast<size_t>(4 * xq) * kFoldStride * 16 : 0);
}

bool wsplit_fold_fits(int K, int k_split) {
  // Whole latent rows in kFoldChunks chunks per lane, and at most 16 k-steps
  // per wave.
  const int ks = ksteps_of(K);
  const int S = k_split > 0 ? k_split : 1;
  const int sps = (ks + S - 1) / S;
  return K > 0 && K <= kFoldMaxK && (sps + kSplitWaves - 1) / kSplitWaves <= 16;
}

bool mfma_same_instance(const sg_config_t& a, const sg_config_t& b) {
  return a.kind == b.kind && a.m_tile == b.m_tile && a.rows == b.rows && a.waves == b.waves &&
         a.k_unroll == b.k_unroll;
}

namespace {

// Segments in grid order, and the F_B role (fb != NULL, wave-split tile
// only) after the first fb_after of them.
hipError_t launch_mfma_impl(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                            const FusedFb* fb, int fb_after, hipStream_t s) {
  if (nseg < 1 || nseg > 2) return hipErrorInvalidValue;
  const sg_config_t& cfg = cfgs[0];
  if (nseg == 2 && !mfma_same_instance(cfgs[0], cfgs[1])) return hipErrorInvalidValue;
  if (fb != nullptr && (fb_after < 0 || fb_after > nseg || cfg.kind != SG_KIND_MFMA_WAVESPLIT))
    return hipErrorInvalidValue;
  MfmaLaunch L;
  L.fb = no_fb_fuse();
  const int nfb = fb != nullptr ? fused_fb_wgs(fb->rank, fb->n_b) : 0;
  int wgs = 0, arrivals = 0, arriving = 0;
  int max_sps = 0;
  for (int i = 0; i < 2; ++i) {
    MfmaSeg& sgm = L.seg[i];
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
    const sg_config_t& c = cfgs[i];
    if (p.M > c.m_tile || c.m_tile <= 0) return hipErrorInvalidValue;
    MfmaArgs& g = sgm.g;
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
    g.gamma = p.gamma;
    g.eps = p.eps;
    g.arrive = fb != nullptr ? p.arrive : nullptr;
    g.nslots = 0;
    g.tile_rows = c.rows;
    g.pairs = p.pairs;
    g.sync = p.sync;
    const int KS = ksteps_of(p.K);
    const int S = c.k_split > 0 ? c.k_split : 1;
    g.sps = (KS + S - 1) / S;
    if (g.sps < 1) g.sps = 1;
    if (g.sps > max_sps) max_sps = g.sps;
    sgm.tiles = tiles_of(c, p.M, p.N);
    sgm.tiles_magic = quotient_magic(sgm.tiles);
    g.ntiles = sgm.tiles;
    sgm.wg_begin = wgs;
    if (sgm.tiles <= 0) return hipErrorInvalidValue;
    wgs += sgm.tiles * S;
    sgm.wg_end = wgs;
    if (g.arrive != nullptr) {
      if (p.partial == nullptr || p.partial != fb->partial || S != fb->S || p.gamma != nullptr ||
          p.res != nullptr || p.arrive != fb->sync)
        return hipErrorInvalidValue;
      arrivals += sgm.tiles * S;  // one producer slot per workgroup
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
    if (fb_lds_bytes(fb->M, fb->rank) > wsplit_lds_bytes(cfg.k_unroll, cfg.m_tile / 4, false, 1))
      return hipErrorInvalidValue;
    for (int i = 0; i < nseg; ++i)
      if (segs[i].gamma != nullptr || segs[i].res != nullptr) return hipErrorInvalidValue;
  }
  if (wgs <= 0) return hipSuccess;
  if (cfg.kind != SG_KIND_MFMA_WAVESPLIT && (segs[0].gamma != nullptr || (nseg == 2 && segs[1].gamma != nullptr)))
    return hipErrorInvalidValue;

  // Instances that load a residual (RES) only where a segment has one and
  // stores bf16; the packed KDA projection (8-wave tiles) never does.
  const bool res = (segs[0].res != nullptr && segs[0].partial == nullptr) ||
                   (nseg == 2 && segs[1].res != nullptr && segs[1].partial == nullptr);
  if (cfg.kind == SG_KIND_MFMA_TILE) {
    const int NW = cfg.waves, C = cfg.k_unroll, XQ = cfg.m_tile / 4;
    if (cfg.rows != 16 * NW || (cfg.m_tile % 4) != 0) return hipErrorInvalidValue;
    // The instances the configuration table uses.
    if (NW == 2 && C == 4) {
      switch (XQ) {
        case 1: return res ? launch_tile_inst<1, 2, 4, 1, true>(L, wgs, s) : launch_tile_inst<1, 2, 4, 1, false>(L, wgs, s);
        case 2: return res ? launch_tile_inst<1, 2, 4, 2, true>(L, wgs, s) : launch_tile_inst<1, 2, 4, 2, false>(L, wgs, s);
        case 3: return res ? launch_tile_inst<1, 2, 4, 3, true>(L, wgs, s) : launch_tile_inst<1, 2, 4, 3, false>(L, wgs, s);
        case 4: return res ? launch_tile_inst<1, 2, 4, 4, true>(L, wgs, s) : launch_tile_inst<1, 2, 4, 4, false>(L, wgs, s);
        default: break;
      }
    }
    // The in-launch K-split sum: one segment, two K splits, bf16 out.
    if (segs[0].pairs != nullptr) {
      const int S = cfg.k_split;
      if (nseg != 1 || NW != 4 || C != 3 || S != 2 || segs[0].partial != nullptr || segs[0].sync == nullptr ||
          L.seg[0].tiles > kFbMaxConsumers)
        return hipErrorInvalidValue;
      switch (XQ) {
        case 8: return launch_tile_inst<2, 4, 3, 8, true, true>(L, wgs, s);
        case 12: return launch_tile_inst<3, 4, 3, 12, true, true>(L, wgs, s);
        case 16: return launch_tile_inst<4, 4, 3, 16, true, true>(L, wgs, s);
        default: return hipErrorInvalidValue;
      }
    }
    if (NW == 4 && C == 3) {
      switch (XQ) {
        case 8: return res ? launch_tile_inst<2, 4, 3, 8, true>(L, wgs, s) : launch_tile_inst<2, 4, 3, 8, false>(L, wgs, s);
        case 12: return res ? launch_tile_inst<3, 4, 3, 12, true>(L, wgs, s) : launch_tile_inst<3, 4, 3, 12, false>(L, wgs, s);
        case 16: return res ? launch_tile_inst<4, 4, 3, 16, true>(L, wgs, s) : launch_tile_inst<4, 4, 3, 16, false>(L, wgs, s);
        default: break;
      }
    }
    if (NW == 8 && C == 3 && res) {  // table entries at 17 <= M <= 64
      switch (XQ) {
        case 8: return launch_tile_inst<2, 8, 3, 8, true>(L, wgs, s);
        case 12: return launch_tile_inst<3, 8, 3, 12, true>(L, wgs, s);
        case 16: return launch_tile_inst<4, 8, 3, 16, true>(L, wgs, s);
        default: break;
      }
    }
    if (NW == 8 && C == 3 && !res) {  // the packed KDA projection, 2 <= M <= 64, and table entries
      switch (XQ) {
        case 1: return launch_tile_inst<1, 8, 3, 1, false>(L, wgs, s);
        case 2: return launch_tile_inst<1, 8, 3, 2, false>(L, wgs, s);
        case 3: return launch_tile_inst<1, 8, 3, 3, false>(L, wgs, s);
        case 4: return launch_tile_inst<1, 8, 3, 4, false>(L, wgs, s);
        case 8: return launch_tile_inst<2, 8, 3, 8, false>(L, wgs, s);
        case 12: return launch_tile_inst<3, 8, 3, 12, false>(L, wgs, s);
        case 16: return launch_tile_inst<4, 8, 3, 16, false>(L, wgs, s);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  }
  if (cfg.kind == SG_KIND_MFMA_WAVESPLIT) {
    // One segment: the instances read only the first (pick_segment<true>).
    if (nseg != 1) return hipErrorInvalidValue;
    const int C = cfg.k_unroll, XQ = cfg.m_tile / 4;
    // 16 rows per workgroup (one fragment), or 17..32 in steps of 4 (two).
    const int NT = cfg.rows == 16 ? 1 : 2;
    if (cfg.rows < 16 || cfg.rows > 32 || cfg.rows % 4 != 0 || cfg.waves != kSplitWaves ||
        (cfg.m_tile % 4) != 0 || (C != 2 && C != 3))
      return hipErrorInvalidValue;
    if (fb != nullptr) {
      if (NT != 1) return hipErrorInvalidValue;
      return launch_wsplit_fb(L, XQ, C, wgs, s);
    }
    if (segs[0].gamma != nullptr) {
      // The RMSNorm fold: one segment whose whole rows fit the prologue.
      if (nseg != 1 || !wsplit_fold_fits(segs[0].K, cfg.k_split)) return hipErrorInvalidValue;
      return res ? launch_wsplit_xq<true, true>(L, XQ, C, NT, wgs, s)
                 : launch_wsplit_xq<true, false>(L, XQ, C, NT, wgs, s);
    }
    if (nseg == 2 && segs[1].gamma != nullptr) return hipErrorInvalidValue;
    return res ? launch_wsplit_xq<false, true>(L, XQ, C, NT, wgs, s)
               : launch_wsplit_xq<false, false>(L, XQ, C, NT, wgs, s);
  }
  if (cfg.kind == SG_KIND_MFMA_BLOCK) {
    if (cfg.rows != kBlkRows || cfg.waves != kBlkWaves || cfg.m_tile % kBlkM != 0) return hipErrorInvalidValue;
    if (cfg.k_unroll != 3) return hipErrorInvalidValue;
    // One segment with a residual, bf16 output and 16-byte aligned output and
    // residual rows: the residual in row order.
    const DotProblem& p0 = segs[0];
    const bool rows16 = nseg == 1 && res && p0.n_split <= 0 &&
                        (reinterpret_cast<uintptr_t>(p0.out) & 15u) == 0 && (p0.ldc & 7) == 0 &&
                        (reinterpret_cast<uintptr_t>(p0.res) & 15u) == 0 && (p0.ldr & 7) == 0;
    if (rows16) return launch_block_inst<3, 2>(L, wgs, s);
    return res ? launch_block_inst<3, 1>(L, wgs, s) : launch_block_inst<3, 0>(L, wgs, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma(const DotProblem* segs, const sg_config_t* cfgs, int nseg, hipStream_t s) {
  return launch_mfma_impl(segs, cfgs, nseg, nullptr, 0, s);
}

hipError_t launch_mfma_fused(const DotProblem* segs, const sg_config_t* cfgs, int nseg,
                             const FusedFb& fb, int fb_after, hipStream_t s) {
  return launch_mfma_impl(segs, cfgs, nseg, &fb, fb_after, s);
}

hipError_t launch_mfma(const DotProblem& p, const sg_config_t& cfg, hipStream_t s) {
  return launch_mfma(&p, &cfg, 1, s);
}

// ---- the one-launch KDA projection -------------------------------------------------

bool help_plan(int M, int K, int n_qkvg, int n_ab, int rank, int n_b, HelpPlan* out) {
  if (M < 1 || M > kHelpMaxM || K <= 0 || K % 8 != 0 || n_qkvg <= 0 || rank <= 0 || n_ab <= rank ||
      n_ab % 4 != 0 || rank % 8 != 0 || rank > kHelpMaxRank || n_b <= 0)
    return false;
  HelpPlan p;
  p.wgs = (n_qkvg + 15) / 16;
  const int wsteps = (K / 8 + kWave - 1) / kWave;
  p.S = help_ranges(K);
  if (p.S > kHelpMaxS) return false;
  p.per = (wsteps + p.S - 1) / p.S;
  p.groups = (n_ab + kHelpRows - 1) / kHelpRows;
  p.units = p.groups * p.S;
  // As few hosts as the rows allow (every host reads all the partials of its
  // activation rows), for each group of kHelpHostM activation rows.
  p.row_hosts = (n_b + kHelpHostRows - 1) / kHelpHostRows;
  p.host_rows = ((n_b + p.row_hosts - 1) / p.row_hosts + 3) / 4 * 4;
  p.hosts = p.row_hosts * ((M + kHelpHostM - 1) / kHelpHostM);
  if (p.units > kFbMaxProducers || p.hosts > kFbMaxConsumers || p.units + p.hosts > p.wgs) return false;
  // Each lane of a host polls at most kHelpPollItems 16-byte loads per K-range.
  if ((M < kHelpHostM ? M : kHelpHostM) * (n_ab / 2) > kHelpPollItems * kWave) return false;
  const int XQ = (M + 3) / 4;
  if (wsplit_lds_bytes(kHelpRing, XQ, false, 1) + help_lds_bytes(M, rank, n_ab) > kMfmaMaxLds) return false;
  *out = p;
  return true;
}

namespace {

template <int XQ>
hipError_t launch_help_inst(const MfmaLaunch& L, const HelpArgs& H, int wgs, hipStream_t s) {
  auto kern = wsplit_help_kernel<XQ>;
  static std::atomic<bool> lds_set[kLdsAttrDevices];
  const hipError_t attr = ensure_lds_limit(reinterpret_cast<const void*>(kern), kMfmaMaxLds, lds_set);
  if (attr != hipSuccess) return attr;
  const size_t lds = wsplit_lds_bytes(kHelpRing, XQ, false, 1) + help_lds_bytes(H.M, H.rank, H.n_ab);
  return launch_kernel(kern, dim3(wgs), dim3((kSplitWaves + 1) * kWave), lds, s, L, H);
}

}  // namespace

hipError_t launch_proj_one(const OneLaunchProj& p, const HelpPlan& plan, hipStream_t s) {
  const DotProblem& q = p.q;
  if (q.M < 1 || q.M > kHelpMaxM || plan.wgs != (q.N + 15) / 16) return hipErrorInvalidValue;
  MfmaLaunch L;
  L.fb = no_fb_fuse();
  MfmaArgs& g = L.seg[0].g;
  g = MfmaArgs{};
  g.a = q.a;
  g.lda = q.lda;
  g.w = q.w;
  g.ldw = q.ldw;
  g.ldr = q.ldc;
  g.out = q.out;
  g.ldc = q.ldc;
  g.M = q.M;
  g.N = q.N;
  g.K = q.K;
  g.sps = ksteps_of(q.K);
  g.tile_rows = 16;
  L.seg[0].tiles = plan.wgs;
  L.seg[0].tiles_magic = quotient_magic(plan.wgs);
  L.seg[0].wg_begin = 0;
  L.seg[0].wg_end = plan.wgs;
  L.seg[1] = L.seg[0];
  L.seg[1].wg_begin = L.seg[1].wg_end = 0;

  HelpArgs H;
  H.x = q.a;
  H.lda = q.lda;
  H.w_ab = p.w_ab;
  H.ldw = q.K;
  H.pairs = p.pairs;
  H.sync = p.sync;
  H.w_b = p.w_b;
  H.beta = p.beta;
  H.g1 = p.g1;
  H.M = q.M;
  H.K = q.K;
  H.n_ab = p.n_ab;
  H.rank = p.rank;
  H.n_b = p.n_b;
  H.groups = plan.groups;
  H.S = plan.S;
  H.per = plan.per;
  H.units = plan.units;
  H.h_begin = plan.units;
  H.h_end = plan.units + plan.hosts;
  H.row_hosts = plan.row_hosts;
  H.host_rows = plan.host_rows;
  switch ((q.M + 3) / 4) {
    case 1: return launch_help_inst<1>(L, H, plan.wgs, s);
    case 2: return launch_help_inst<2>(L, H, plan.wgs, s);
    case 3: return launch_help_inst<3>(L, H, plan.wgs, s);
    case 4: return launch_help_inst<4>(L, H, plan.wgs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sg
