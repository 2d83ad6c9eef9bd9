// The helper wave of the one-launch KDA projection (gfx950).
//
// "Overlap low-M TP8 KDA projections" (run_kda_projection_overlap,
// run_fab_fb) computes, from one decode activation x,
//   qkvg = bf16(x W_qkvg^T),
//   P    = bf16(x W_ab^T),  f_a = P[:, :rank],  beta = P[:, rank:],
//   g1   = bf16(f_a W_b^T),
// with the small F_A/beta -> F_B chain on an auxiliary stream beside the
// Q/K/V/G GEMM.  Here the chain rides inside the Q/K/V/G launch instead: each
// wave-split workgroup (four waves streaming 16 Q/K/V/G rows) carries a fifth
// wave, the helper, which
//
//  * in workgroups [0, units) computes one producer unit of P -- four W_ab
//    rows over one K-range of at most 2048 -- as a GEMV (weights straight
//    into registers, the activation rows through LDS, fp32 dot products, a
//    transposing wave sum) and stores each fp32 partial together with the
//    call's generation as one 8-byte device-coherent store;
//  * in workgroups [h_begin, h_end) (none of them a producer) acts as an F_B
//    host: loads its rows of W_b, then reads every partial it needs until all
//    carry this call's generation (a bounded spin), sums them in the fixed
//    order s = 0..S-1 into a bf16 P tile in LDS (f_a, and in the group's
//    first host beta, which it then stores), and computes its rows of g1 on
//    the matrix cores.
//
// A partial tagged with the generation needs no separate flag: its producer
// never waits for its store to complete, and the host's wait is the load of
// the data itself, one round trip to the point of coherence per poll.  The
// units spread the F_A/beta bytes evenly over the chip at the start of the
// launch, and no workgroup beyond the Q/K/V/G tiles is launched.
//
// Generations: the workspace header of sg_fused.h (one flag per producer
// slot, one cursor per consumer, each advanced by one per call, zero before
// the first call).  A unit tags its partials with its flag + 1 and then
// advances the flag; a host waits for its cursor + 1 and then advances the
// cursor; the units share out the absent slots and the hosts the absent
// cursors, so every flag and cursor holds the number of calls so far,
// whatever the shapes of the calls and whichever one-launch entry point made
// them.  Producers never wait, and
// every host is dispatched after every producer (dispatch follows the
// workgroup index), so the wait ends even when the workgroups do not all fit
// the chip at once.
#pragma once

#include "sg_fused.h"
#include "sg_launch.h"

namespace sg {

constexpr int kHelpPollItems = 9;   // 16-byte loads (two tagged partials) per lane per K-range

struct HelpArgs {
  const uint16_t* x;       // [M, K]
  int64_t lda;
  const uint16_t* w_ab;    // [n_ab, K]
  int64_t ldw;
  uint32_t* pairs;         // [S][M][n_ab] pairs (fp32 bits, generation)
  unsigned* sync;          // hand-off header: flags, then cursors
  const uint16_t* w_b;     // [n_b, rank], rank % 8 == 0, rank <= kHelpMaxRank
  uint16_t* beta;          // [M, n_ab - rank]
  uint16_t* g1;            // [M, n_b]
  int M, K, n_ab, rank, n_b;
  int groups;              // units per K-range: ceil(n_ab / kHelpRows)
  int S;                   // K-ranges of P, each `per` 512-k steps
  int per;
  int units;               // groups * S: workgroup u < units runs unit (u % groups, u / groups)
  int h_begin, h_end;      // F_B hosts: row_hosts per group of kHelpHostM activation rows
  int row_hosts;
  int host_rows;           // g1 rows per host, a multiple of 4, <= kHelpHostRows
};

// Coherent 16-byte load (sc1: served from the device's point of coherence,
// so partials another XCD stored are seen).
__device__ __forceinline__ u32x4 buf_load_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 16));
}

// Lane l receives the sum over all 64 lanes of v[l].  At distance d = 32, 16,
// .., 1 lanes l and l ^ d each keep one half of their remaining values (the
// lane with bit d set the upper half) and add the partner's copy of it, so
// after six steps the single value left in lane l belongs to index l.  Each
// total is formed by the same tree of additions on every call.
__device__ __forceinline__ float transpose_sum64(float (&v)[64]) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const bool up = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < d; ++i) {
      // Values, not array elements, are selected: a conditional between two
      // elements would select their address and put v in scratch memory.
      const float lo = v[i], hi = v[i + d];
      const float keep = up ? hi : lo;
      const float give = up ? lo : hi;
      v[i] = keep + __shfl_xor(give, d);
    }
  }
  return v[0];
}

// Producer unit `b`: four rows of W_ab over one K-range against the M
// activation rows (4 * XQ >= M), stored as tagged fp32 partial[s][m][row].
// lds: kHelpSteps * 4 * XQ KiB of the helper's LDS.
template <int XQ>
__device__ __forceinline__ void help_unit(const HelpArgs& h, int b, void* lds) {
  const int lane = lane_id();
  const unsigned gen = load_flag(h.sync + b) + 1u;
  const int grp = b % h.groups;
  const int s = b / h.groups;
  const int r0 = grp * kHelpRows;
  const int rows = min(kHelpRows, h.n_ab - r0);
  const int K8 = h.K >> 3;
  const int st0 = s * h.per;
  const rsrc_t wres = make_rsrc(h.w_ab + static_cast<int64_t>(r0) * h.ldw,
                                static_cast<uint32_t>(((rows - 1) * h.ldw + h.K) * 2));
  const rsrc_t xres = make_rsrc(h.x, static_cast<uint32_t>(((h.M - 1) * h.lda + h.K) * 2));
  // The activation rows of the K-range go global->LDS (step i, row m: 1 KiB
  // at xs + (i * 4 XQ + m) * 64), the weights into registers; all requested
  // at once (one round trip).  Pieces past the range, the rows or K read
  // zeros.
  u32x4* xs = static_cast<u32x4*>(lds);
  u32x4 wv[kHelpRows][kHelpSteps];
#pragma unroll
  for (int i = 0; i < kHelpSteps; ++i) {
    const int c = (st0 + i) * kWave + lane;
    const bool ok = i < h.per && c < K8;
#pragma unroll
    for (int m = 0; m < 4 * XQ; ++m)
      copy16_to_lds(xres, xs + (i * 4 * XQ + m) * kWave,
                    (ok && m < h.M) ? static_cast<uint32_t>((m * h.lda + c * 8) * 2) : kOob);
#pragma unroll
    for (int r = 0; r < kHelpRows; ++r)
      wv[r][i] = buf_load_nt(wres, (ok && r < rows) ? static_cast<uint32_t>((r * h.ldw + c * 8) * 2) : kOob);
  }
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the LDS reads below follow the copies
  float v[64];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    u32x4 xv[kHelpSteps];
#pragma unroll
    for (int i = 0; i < kHelpSteps; ++i) xv[i] = m < 4 * XQ ? xs[(i * 4 * XQ + m) * kWave + lane] : zero4();
#pragma unroll
    for (int r = 0; r < kHelpRows; ++r) {
      float a = 0.f;
      if (m < 4 * XQ) {
#pragma unroll
        for (int i = 0; i < kHelpSteps; ++i) a = dot8(wv[r][i], xv[i], a);
      }
      v[r * 16 + m] = a;
    }
  }
  const float t = transpose_sum64(v);
  const int r = lane >> 4, m = lane & 15;
  if (m < h.M && r < rows) {
    const uint64_t pair = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, t)) | (static_cast<uint64_t>(gen) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(h.pairs) + (static_cast<int64_t>(s) * h.M + m) * h.n_ab + r0 + r,
                       pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The slot's flag (nothing in this launch waits for it; it keeps the
  // header's generations for later calls), and its share of the absent
  // slots' (unit b: slots units + b + j * units), at most one store per lane.
  if (lane == 0) store_flag(h.sync + b, gen);
  for (int q = h.units + b + h.units * lane; q < kFbMaxProducers; q += h.units * kWave) store_flag(h.sync + q, gen);
}

// F_B host `hid` (XQ: the launch's activation tile): g1 rows
// [rg * host_rows, +host_rows) of the activation
// rows [mg * kHelpHostM, +kHelpHostM) (hid = mg * row_hosts + rg) as four
// 16-row MFMA tiles.  lds: the helper's LDS, W_b rows [kHelpHostRows]
// [kHelpMaxRank] (swizzled) then the group's P [kHelpHostM][help_p_stride
// (n_ab)] (f_a then beta columns), both bf16.
template <int XQ>
__device__ __forceinline__ void help_host(const HelpArgs& h, int hid, void* lds_raw) {
  const int lane = lane_id();
  uint16_t* wb_lds = static_cast<uint16_t*>(lds_raw);
  uint16_t* p_lds = wb_lds + kHelpHostRows * kHelpMaxRank;
  const int pst = help_p_stride(h.n_ab);
  const int mg = hid / h.row_hosts;
  const int rg = hid - mg * h.row_hosts;
  const int m0 = mg * kHelpHostM;
  const int mc = min(kHelpHostM, h.M - m0);
  const int row_base = rg * h.host_rows;
  const int nrows = max(0, min(h.host_rows, h.n_b - row_base));
  const int K8b = h.rank >> 3;
  const int rl = lane & 15;
  const int kg = lane >> 4;
  // The host's W_b rows copied global->LDS before the wait, 16 pieces of 8
  // per row (zeros past rank and past the host's rows), piece c of row r at
  // position c ^ (r & 15): the 16 lanes that read one MFMA operand (16 rows,
  // one piece) hit 16 different bank groups.  Each copy fills 4 rows; the
  // lane that fills position p of row r loads piece p ^ (r & 15).
  const rsrc_t bres = make_rsrc(h.w_b + static_cast<int64_t>(row_base) * h.rank,
                                static_cast<uint32_t>(nrows * h.rank * 2));
#pragma unroll
  for (int r0 = 0; r0 < kHelpHostRows; r0 += 4) {
    const int r = r0 + (lane >> 4);
    const int pc = (lane & 15) ^ (r & 15);
    copy16_to_lds_nt(bres, wb_lds + r0 * kHelpMaxRank,
                     (r < nrows && pc < K8b) ? static_cast<uint32_t>((r * h.rank + pc * 8) * 2) : kOob);
  }
  unsigned* cursors = h.sync + kFbMaxProducers;
  const unsigned target = load_flag(cursors + hid) + 1u;

  // The partials this host needs: the rank f_a columns of its activation
  // rows (all n_ab in the group's first host, which also stores their
  // beta), two columns per 16-byte load, of every K-range.  A poll loads
  // them all and succeeds when every one carries generation `target`.
  const int cols = rg == 0 ? h.n_ab : h.rank;
  const int q2 = cols >> 1;
  const int count = mc * q2;
  const uint32_t plane = static_cast<uint32_t>(h.M * h.n_ab * 8);
  const rsrc_t pres = make_rsrc(h.pairs, static_cast<uint32_t>(h.S) * plane);
  uint32_t off[kHelpPollItems];
  int lo[kHelpPollItems];  // each load's two columns in p_lds (bf16 units)
#pragma unroll
  for (int e = 0; e < kHelpPollItems; ++e) {
    const int idx = e * kWave + lane;
    const int m = idx / q2;
    const int c = 2 * (idx - m * q2);
    off[e] = idx < count ? static_cast<uint32_t>(((m0 + m) * h.n_ab + c) * 8) : 0u;
    lo[e] = m * pst + c;
  }
  u32x4 pv[kHelpPollItems][kHelpMaxS];
  bool ok = false;
  // The units' partials land 3.5-6.5 us into the launch (measured): a poll
  // before then only adds coherent loads to this workgroup's own stream.
  // The first poll therefore waits about that long (s_sleep counts 64
  // clocks per unit): measured best among none / 1.8 / 2.8 / 3.9 / 4.8 /
  // 5.8 / 7.7 us of sleep, 0.4-0.9 us per call faster than polling at once.
  // Larger units land later: beyond 127 units, 30 more at M = 5..8, 100 at
  // 9..12 (best among 30 / 60 / 100 / 127 / 180 / 254, 0.6-1 us faster than
  // 30) and 16 (M - 4) at 13..16 (against 12 (M - 4) and 14 (M - 4)).
  __builtin_amdgcn_s_sleep(127);
  if constexpr (XQ == 2) __builtin_amdgcn_s_sleep(30);
  if constexpr (XQ == 3) __builtin_amdgcn_s_sleep(100);
  if constexpr (XQ == 4)
    for (int z = 0; z < 16 * (h.M - 4); z += 16) __builtin_amdgcn_s_sleep(16);
  {
    int polls = 0;
    for (;;) {
#pragma unroll
      for (int e = 0; e < kHelpPollItems; ++e)
#pragma unroll
        for (int s = 0; s < kHelpMaxS; ++s)
          pv[e][s] = buf_load_coherent(pres, off[e] + static_cast<uint32_t>(min(s, h.S - 1)) * plane);
      bool mine = true;
#pragma unroll
      for (int e = 0; e < kHelpPollItems; ++e)
#pragma unroll
        for (int s = 0; s < kHelpMaxS; ++s)
          mine = mine && (pv[e][s][1] == target) && (pv[e][s][3] == target);
      ok = __builtin_amdgcn_ballot_w64(!mine) == 0;
      if (ok || ++polls >= kFbSpinLimit) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  // Every load of this wave has completed (the poll's loads waited for, the
  // W_b copies issued before them): the wait below costs nothing, and no
  // later wait for the copies has to wait for the beta stores.
  wait_vmcnt<0>();
  // P in the order s = 0..S-1, rounded to bf16, into LDS (row m - m0; the
  // beta columns only in the group's first host); NaN after a time-out.
  // One LDS store per load, no branch on the column: the per-item work is
  // the sum, the rounding and the store.
  const uint32_t nan2 = static_cast<uint32_t>(kBf16NaN) * 0x10001u;
#pragma unroll
  for (int e = 0; e < kHelpPollItems; ++e) {
    if (e * kWave + lane >= count) break;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int s = 0; s < kHelpMaxS; ++s) {
      const f32x4 f = __builtin_bit_cast(f32x4, pv[e][s]);
      a0 += s < h.S ? f[0] : 0.f;
      a1 += s < h.S ? f[2] : 0.f;
    }
    *reinterpret_cast<uint32_t*>(p_lds + lo[e]) = ok ? pack_bf16x2(a0, a1) : nan2;
  }
  // P was written to LDS by this wave (in order for the LDS unit); keep the
  // compiler from moving the reads below above those writes.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (rg == 0) {  // the group's beta columns, from LDS to memory
    const int nbeta = h.n_ab - h.rank;
    for (int i = lane; i < mc * nbeta; i += kWave) {
      const int m = i / nbeta;
      const int j = i - m * nbeta;
      h.beta[static_cast<int64_t>(m0 + m) * nbeta + j] = p_lds[m * pst + h.rank + j];
    }
  }

  // g1[m, row] = bf16(sum_r f_a[m, r] * w_b[row, r]) on the matrix cores:
  // A = W_b (lane l: row l % 16 of the tile, k group l / 16, zero past rank),
  // B = f_a (lane l: row m0 + l % 16, zero past the group's rows), the
  // k-steps in order; lane l ends with rows 4 (l / 16) .. +3 of each tile for
  // m = m0 + l % 16 (NaN f_a after a time-out makes g1 NaN too).
  u32x4 fb[kHelpMaxRank / 32];
#pragma unroll
  for (int s = 0; s < kHelpMaxRank / 32; ++s) {
    const int kc = 4 * s + kg;
    const u32x4 v = *reinterpret_cast<const u32x4*>(p_lds + min(rl, mc - 1) * pst + min(kc, K8b - 1) * 8);
    fb[s] = (rl < mc && kc < K8b) ? v : zero4();
  }
  const bool vec = ((reinterpret_cast<uintptr_t>(h.g1) | (static_cast<uintptr_t>(h.n_b) * 2)) & 7u) == 0;
#pragma unroll
  for (int tt = 0; tt < kHelpHostRows / 16; ++tt) {
    if (16 * tt >= nrows) break;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kHelpMaxRank / 32; ++s) {
      const int kc = 4 * s + kg;  // zeros past rank
      const u32x4 w = *reinterpret_cast<const u32x4*>(wb_lds + (16 * tt + rl) * kHelpMaxRank + (kc ^ rl) * 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                   __builtin_bit_cast(bf16x8, fb[s]), acc, 0, 0, 0);
    }
    const int r0 = 16 * tt + 4 * kg;
    if (rl >= mc || r0 >= nrows) continue;
    uint16_t* dst = h.g1 + static_cast<int64_t>(m0 + rl) * h.n_b + row_base + r0;
    if (vec && r0 + 3 < nrows) {
      uint2 packed;
      packed.x = pack_bf16x2(acc[0], acc[1]);
      packed.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<uint2*>(dst) = packed;
    } else {
      const float a[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (r0 + v < nrows) dst[v] = f32_to_bf16(a[v]);
    }
  }

  // This host is done: its cursor moves to target, and its share of the
  // absent hosts' cursors (nhosts + hid + j * nhosts).
  const int nhosts = h.h_end - h.h_begin;
  if (lane == 0) store_flag(cursors + hid, target);
  for (int q = nhosts + hid + nhosts * lane; q < kFbMaxConsumers; q += nhosts * kWave) store_flag(cursors + q, target);
}

// The helper wave of workgroup b.  lds: help_lds_bytes(M, rank, n_ab) of dynamic
// LDS no other wave uses.
template <int XQ>
__device__ __forceinline__ void help_wave(const HelpArgs& h, int b, void* lds) {
  if (b < h.units)
    help_unit<XQ>(h, b, lds);
  else if (b >= h.h_begin && b < h.h_end)
    help_host<XQ>(h, b - h.h_begin, lds);
}

}  // namespace sg
