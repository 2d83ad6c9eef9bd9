// Device helpers shared by the gfx950 kernels of libskinny_gemm.
//
// Data movement is in 16-byte chunks (8 bf16), the widest per-lane global load
// (global_load_dwordx4).  Weights are streamed with non-temporal loads, the
// analogue of the reference's STREAMING cache mode for B (CuteSkinnyGemm copy
// atoms, "Kimi K3 support, phase 1"): each weight byte is used once, so it
// should not displace the activations from the caches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- loads -----------------------------------------------------------------

__device__ __forceinline__ u32x4 load_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 load_cached(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// ---- buffer loads ------------------------------------------------------------
//
// A buffer resource bounds a region of num_records bytes; a load whose offset
// lies past it returns zeros without touching memory.  Ragged rows, the K
// tail and steps past a wave's range therefore become an integer select on
// the offset (kOob) instead of a branch around the load.  Loads outside
// branches let the compiler wait for exactly the loads a value depends on
// rather than for every outstanding load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;  // any offset >= num_records reads zeros

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // 0x00020000: raw (untyped) 32-bit data, the gfx9 descriptor word 3 value.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Non-temporal (streaming) 16-byte load: weights, each byte used once.
__device__ __forceinline__ u32x4 buf_load_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2));
}

// Cached 16-byte load: activations, reused by every workgroup.
__device__ __forceinline__ u32x4 buf_load(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

// Four consecutive bf16 values base[idx .. idx+3] of a buffer of `elems`
// elements with any 2-byte alignment, as two 8-byte buffer loads of the
// 8-byte-aligned blocks that hold them (the second only when they straddle
// two): the buffer runs from the 8-byte boundary at or below `base` to its
// end rounded up to 8 bytes, so every block lies wholly inside or outside it
// and none crosses a page.  `use` false (uniform across the wave: it sizes
// the buffer, which must stay in scalar registers) or `lane` false reads
// zeros and fetches nothing.  Values past the end read zeros or are unused.
__device__ __forceinline__ void load4_bf16(const uint16_t* base, int64_t elems, int64_t idx, bool use,
                                           bool lane, uint16_t (&out)[4]) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(base);
  const uintptr_t rb = b & ~static_cast<uintptr_t>(7);
  const int64_t span = static_cast<int64_t>(b - rb) + elems * 2;
  const rsrc_t rr = make_rsrc(reinterpret_cast<const void*>(rb),
                              use ? static_cast<uint32_t>((span + 7) & ~static_cast<int64_t>(7)) : 0u);
  const uint32_t a = static_cast<uint32_t>(static_cast<int64_t>(b - rb) + idx * 2);
  const uint32_t s0 = lane ? (a & ~7u) : kOob;
  const uint32_t s1 = lane ? (a & ~7u) + ((a & 7u) != 0u ? 8u : 0u) : kOob;
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, static_cast<int>(s0), 0, 0));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, static_cast<int>(s1), 0, 0));
  const bool k = ((a >> 2) & 1u) != 0;  // the first value's word in the first block: 0 or 1
  const uint32_t bb = a & 3u;           // and its byte within it: 0 or 2
  const uint32_t w0 = k ? lo[1] : lo[0];
  const uint32_t w1 = k ? hi[0] : lo[1];
  const uint32_t w2 = k ? hi[1] : hi[0];
  const uint32_t v01 = __builtin_amdgcn_alignbyte(w1, w0, bb);
  const uint32_t v23 = __builtin_amdgcn_alignbyte(w2, w1, bb);
  out[0] = static_cast<uint16_t>(v01 & 0xFFFFu);
  out[1] = static_cast<uint16_t>(v01 >> 16);
  out[2] = static_cast<uint16_t>(v23 & 0xFFFFu);
  out[3] = static_cast<uint16_t>(v23 >> 16);
}

// ---- bf16 <-> fp32 ---------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- 8-element dot product, fp32 accumulate ---------------------------------

// acc + sum_{i<8} a[i]*b[i] for two 16-byte chunks of bf16, four
// v_dot2c_f32_bf16 (two bf16 products per instruction, fp32 accumulate).
// The pairs are taken with whole-vector casts and shuffles: this compiler
// mis-lowers __builtin_bit_cast applied directly to a vector element
// expression (it reads element 0), so element-wise casts are avoided
// throughout these kernels.
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a);
  const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 0, 1),
                                        __builtin_shufflevector(bv, bv, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 2, 3),
                                        __builtin_shufflevector(bv, bv, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 4, 5),
                                        __builtin_shufflevector(bv, bv, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 6, 7),
                                        __builtin_shufflevector(bv, bv, 6, 7), acc, false);
  return acc;
}

// Sum of the two halves returned by v_permlane{16,32}_swap (a 2-vector),
// read through a scalar copy of each element (see dot8).
template <typename V>
__device__ __forceinline__ float swap_pair_sum(V s) {
  const uint32_t s0 = s[0];
  const uint32_t s1 = s[1];
  return __builtin_bit_cast(float, s0) + __builtin_bit_cast(float, s1);
}

__device__ __forceinline__ float xor16_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return swap_pair_sum(__builtin_amdgcn_permlane16_swap(u, u, false, false));
}

__device__ __forceinline__ float xor32_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return swap_pair_sum(__builtin_amdgcn_permlane32_swap(u, u, false, false));
}

// ---- wave-level reductions ---------------------------------------------------

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets it.
// DPP quad_perm [1,0,3,2] and [2,3,0,1] sum a quad, row_half_mirror pairs the
// two quads of an 8-lane half, row_mirror pairs the two halves of a 16-lane row.
__device__ __forceinline__ float row16_allreduce(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// n / d for 0 <= n, d with n + d < 2^32, given magic = quotient_magic(d)
// (the host's): a multiply-high and one branch-free correction, no division.
__device__ __forceinline__ int quotient_by(int n, int d, unsigned magic) {
  const unsigned q = __umulhi(static_cast<unsigned>(n), magic);
  return static_cast<int>((q + 1u) * static_cast<unsigned>(d) <= static_cast<unsigned>(n) ? q + 1u : q);
}

// Sum over all 64 lanes; every lane gets it.  After the 16-lane sums,
// v_permlane16_swap exchanges odd and even rows and v_permlane32_swap the two
// 32-lane halves.
__device__ __forceinline__ float wave_allreduce(float v) {
  return xor32_sum(xor16_sum(row16_allreduce(v)));
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }
// The wave index is the same for all 64 lanes; reading it through
// readfirstlane puts it (and everything derived from it: K-ranges, trip
// counts) in scalar registers, so loops over it are scalar loops.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// ---- global -> LDS copies ----------------------------------------------------
//
// buffer_load_dwordx4 ... lds: each lane's 16 bytes go from the buffer offset
// it names straight into LDS at dst + 16 * lane (dst is the same for the whole
// wave), without passing through registers.  An offset past the buffer writes
// zeros.  The copy is counted by vmcnt; the compiler does not order LDS reads
// after it, so callers wait with wait_vmcnt<> (and a barrier when another
// wave reads the data).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void copy16_to_lds(rsrc_t r, void* lds_dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_dst, 16, static_cast<int>(off), 0, 0, 0);
}
// Same, non-temporal (weights).
__device__ __forceinline__ void copy16_to_lds_nt(rsrc_t r, void* lds_dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_dst, 16, static_cast<int>(off), 0, 0, 2);
}

// s_waitcnt with only one counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace sg
