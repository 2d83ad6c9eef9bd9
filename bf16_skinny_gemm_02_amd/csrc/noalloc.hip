// kda_projection_noalloc: the KDA projection with its workspaces in a
// library-owned device array instead of caller-supplied buffers, for callers
// that cannot allocate (code under graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// `scratch` is a file-scope device array of SG_NOALLOC_SCRATCH_BYTES.  Each
// GPU holds its own copy, zero-filled when the code object is loaded (static
// storage), until the process ends.  Host code never uses the array's name
// as an address: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in `g_scratch`; only
// that address reaches a kernel.  The projection's workspaces are carved
// from it: the F_A/beta region first (its leading counters must be zero
// before a call; every call leaves them zero), then the Q/K/V/G partials.
// Every call on one GPU uses the same array, so calls that overlap on one GPU
// (two streams, or two threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>

#include "sg_launch.h"
#include "skinny_gemm.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of this device's `scratch` (looked up on first use).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SG_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SG_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);  // every thread finds the same address
  }
  *out = p;
  return SG_OK;
}

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

extern "C" int kda_projection_noalloc(const sg_bf16* x, const sg_bf16* packed_w, const sg_bf16* w_b,
                                      sg_bf16* qkvg, sg_bf16* beta, sg_bf16* g1, int M, int K,
                                      int n_qkvg, int n_ab, int rank, int n_b,
                                      sg_stream_t main_stream, sg_stream_t aux_stream,
                                      sg_event_t fork, sg_event_t join) {
  if (M < 0 || K < 0 || n_qkvg < 0 || n_ab < 0) return SG_ERR_INVALID_ARG;
  // The scratch size is checked before anything touches the GPU.
  const size_t aux = round256(sg_kda_workspace_bytes(SG_KDA_FAB, M, K, n_qkvg, n_ab));
  const size_t main = round256(sg_kda_workspace_bytes(SG_KDA_QKVG, M, K, n_qkvg, n_ab));
  if (aux + main > SG_NOALLOC_SCRATCH_BYTES) return SG_ERR_WORKSPACE;
  if (M == 0) {  // the existing entry point validates the rest and enqueues nothing
    return kda_projection_overlap(x, packed_w, w_b, qkvg, beta, g1, M, K, n_qkvg, n_ab, rank, n_b,
                                  nullptr, 0, nullptr, 0, main_stream, aux_stream, fork, join);
  }
  void* base = nullptr;
  const int st = scratch_ptr(&base);
  if (st != SG_OK) return st;
  unsigned char* b = static_cast<unsigned char*>(base);
  return kda_projection_overlap(x, packed_w, w_b, qkvg, beta, g1, M, K, n_qkvg, n_ab, rank, n_b,
                                main > 0 ? b + aux : nullptr, main, b, aux, main_stream, aux_stream,
                                fork, join);
}
