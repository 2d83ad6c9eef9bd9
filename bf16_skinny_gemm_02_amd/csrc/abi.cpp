// extern "C" entry points of libskinny_gemm (declared in include/skinny_gemm.h).
//
// Every entry point validates all of its arguments on the host before it
// enqueues anything, then launches the kernels the configuration table names.
// Argument checks are explicit branches that return a status (never assert),
// so they hold in every build mode.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "sg_fused.h"
#include "sg_launch.h"
#include "skinny_gemm.h"

namespace {

using sg::DotProblem;

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? SG_OK : SG_ERR_HIP; }

// Checks shared by every dot-product call once sizes are known non-negative
// and the problem is non-empty.
int check_operand16(const void* p, int64_t ld, int64_t min_ld) {
  if (p == nullptr) return SG_ERR_INVALID_ARG;
  if (ld < min_ld) return SG_ERR_INVALID_ARG;
  if (!al16(p) || (ld % 8) != 0) return SG_ERR_MISALIGNED;
  return SG_OK;
}

int check_output2(const void* p, int64_t ld, int64_t min_ld) {
  if (p == nullptr) return SG_ERR_INVALID_ARG;
  if (ld < min_ld) return SG_ERR_INVALID_ARG;
  if (!al2(p)) return SG_ERR_MISALIGNED;
  return SG_OK;
}

// Kernels address a weight tile (at most 128 rows) and the whole activation
// through 32-bit buffer offsets: both spans must stay below 2^31 bytes.
constexpr int64_t kMaxTileRows = 128;
bool spans_ok(int64_t rows, int64_t ld, int64_t K) {
  if (ld < 0 || K < 0) return false;
  if (rows <= 0) return true;
  return ((rows - 1) * ld + K) * 2 < (int64_t(1) << 31);
}

int check_workspace(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SG_OK;
  if (ws == nullptr || ws_bytes < need) return SG_ERR_WORKSPACE;
  if (!al16(ws)) return SG_ERR_MISALIGNED;
  return SG_OK;
}

bool is_mfma(int kind) {
  return kind == SG_KIND_MFMA_TILE || kind == SG_KIND_MFMA_WAVESPLIT || kind == SG_KIND_MFMA_BLOCK;
}

// Whether the F_A/beta rows of configuration f can hand their partials to an
// F_B role in the same launch: the kernels that host the role (the 4-wave
// GEMV, M = 1, and the wave-split MFMA tile, M <= 16), with a flag for every
// producer (each GEMV wave, each wave-split workgroup) and a cursor for every
// F_B workgroup in the workspace header.
bool hosts_fb(const sg_config_t& f, int rank, int n_b) {
  int64_t producers;
  if (f.kind == SG_KIND_GEMV_ROW || f.kind == SG_KIND_GEMV_SPLITK) {
    if (f.waves != 4 || f.m_tile != 1) return false;
    producers = static_cast<int64_t>(f.grid) * f.waves;
  } else if (f.kind == SG_KIND_MFMA_WAVESPLIT && f.rows == 16) {  // one-fragment instances
    producers = f.grid;
  } else {
    return false;
  }
  return producers <= sg::kFbMaxProducers && sg::fused_fb_wgs(rank, n_b) <= sg::kFbMaxConsumers;
}

// The main kernel of configuration c, with the problem's epilogue as given
// (p.partial set means fp32 partials).
hipError_t launch_main(const DotProblem& p, const sg_config_t& c, hipStream_t s) {
  if (is_mfma(c.kind)) return sg::launch_mfma(p, c, s);
  if (c.kind == SG_KIND_GEMV_SMALLK) return sg::launch_smallk(p, c, s);
  return sg::launch_gemv(p, c, s);
}

// Enqueue out = a @ w^T (+res) with configuration c.  ws holds the split-K
// partials when c.k_split > 1 (size checked by the caller).
int enqueue_dot(DotProblem p, const sg_config_t& c, void* ws, hipStream_t s) {
  if (c.kind == SG_KIND_NONE) return SG_OK;
  if (c.kind == SG_KIND_GEMV_SMALLK) return hip_status(sg::launch_smallk(p, c, s));
  if (c.kind != SG_KIND_GEMV_ROW && c.kind != SG_KIND_GEMV_SPLITK && !is_mfma(c.kind))
    return SG_ERR_UNSUPPORTED;
  const bool split = c.k_split > 1;
  if (split) p.partial = static_cast<float*>(ws);
  if (launch_main(p, c, s) != hipSuccess) return SG_ERR_HIP;
  if (!split) return SG_OK;
  sg::ReduceProblem r{};
  r.partial = p.partial;
  r.S = c.k_split;
  r.M = p.M;
  r.N = p.N;
  r.res = p.res;
  r.ldr = p.ldr;
  r.out = p.out;
  r.ldc = p.ldc;
  r.out2 = p.out2;
  r.ldc2 = p.ldc2;
  r.n_split = p.n_split;
  return hip_status(sg::launch_reduce(r, s));
}

// Validation of skinny_gemm arguments; fills *cfg on success.
int validate_gemm(const sg_bf16* A, int64_t lda, const sg_bf16* W, int64_t ldw, const sg_bf16* R,
                  int64_t ldr, sg_bf16* C, int64_t ldc, int M, int N, int K,
                  const sg_config_t* user_cfg, void* ws, size_t ws_bytes, sg_config_t* cfg,
                  bool* empty) {
  *empty = false;
  if (M < 0 || N < 0 || K < 0) return SG_ERR_INVALID_ARG;
  int st = sg_select(M, N, K, R != nullptr, cfg);
  if (st != SG_OK) return st;
  if (cfg->kind == SG_KIND_NONE) {
    *empty = true;
    return SG_OK;
  }
  // Row strides are at least K (so never negative) whatever K is: the MFMA
  // kernels build 32-bit buffer bounds from them even when K == 0.
  if (lda < K || ldw < K) return SG_ERR_INVALID_ARG;
  if (K > 0) {  // with K == 0 the operands are never read
    if ((st = check_operand16(A, lda, K)) != SG_OK) return st;
    if ((st = check_operand16(W, ldw, K)) != SG_OK) return st;
  }
  if ((st = check_output2(C, ldc, N)) != SG_OK) return st;
  if (R != nullptr && (st = check_output2(R, ldr, N)) != SG_OK) return st;
  if (user_cfg != nullptr) {
    if (sg_config_supported(user_cfg, M, N, K) != SG_OK) return SG_ERR_UNSUPPORTED;
    *cfg = *user_cfg;
  }
  if (!spans_ok(M, lda, K) || !spans_ok(kMaxTileRows, ldw, K)) return SG_ERR_UNSUPPORTED;
  return check_workspace(ws, ws_bytes, user_cfg != nullptr ? sg_config_workspace_bytes(cfg, M, N)
                                                           : sg_workspace_bytes(SG_OP_GEMM, M, N, K));
}

// The F_A/beta stage configuration of kda_fab_fb_proj (the table's choice,
// run in partial mode).
sg_config_t fab_config(int M, int n_ab, int K) {
  sg_config_t c;
  if (sg_kda_select(SG_KDA_FAB_ALONE, M, K, 0, n_ab, &c) != SG_OK) memset(&c, 0, sizeof c);
  return c;
}

int validate_fab_fb(const sg_bf16* x, const sg_bf16* w_ab, const sg_bf16* w_b, sg_bf16* beta,
                    sg_bf16* g1, sg_bf16* f_a, int M, int K, int n_ab, int rank, int n_b,
                    void* ws, size_t ws_bytes, bool* empty) {
  *empty = false;
  if (M < 0 || K < 0 || n_b < 0 || rank <= 0 || n_ab <= rank) return SG_ERR_INVALID_ARG;
  if (rank % 8 != 0 || rank > sg::kFbMaxRank) return SG_ERR_UNSUPPORTED;
  if (K % 8 != 0 || M > 256) return SG_ERR_UNSUPPORTED;
  if (M == 0) {
    *empty = true;
    return SG_OK;
  }
  int st;
  if ((st = check_operand16(x, K, K)) != SG_OK) return st;
  if ((st = check_operand16(w_ab, K, K)) != SG_OK) return st;
  if ((st = check_operand16(w_b, rank, rank)) != SG_OK) return st;
  if ((st = check_output2(beta, n_ab - rank, n_ab - rank)) != SG_OK) return st;
  if (n_b > 0 && (st = check_output2(g1, n_b, n_b)) != SG_OK) return st;
  if (n_b == 0 && g1 != nullptr && !al2(g1)) return SG_ERR_MISALIGNED;
  if (f_a != nullptr && !al2(f_a)) return SG_ERR_MISALIGNED;
  if (!spans_ok(M, K, K) || !spans_ok(kMaxTileRows, K, K)) return SG_ERR_UNSUPPORTED;
  return check_workspace(ws, ws_bytes, sg_workspace_bytes(SG_OP_FAB_FB, M, n_ab, K));
}

// The F_A/beta -> F_B branch.  Its workspace: the hand-off header
// (kSyncBytes), then the F_A/beta partials.  one_launch: the F_B role runs in
// the F_A/beta launch where a kernel hosts it (else F_B is a second launch).
int enqueue_fab_fb(const sg_bf16* x, const sg_bf16* w_ab, const sg_bf16* w_b, sg_bf16* f_a,
                   sg_bf16* beta, sg_bf16* g1, int M, int K, int n_ab, int rank, int n_b, void* ws,
                   bool one_launch, hipStream_t s) {
  const sg_config_t c = fab_config(M, n_ab, K);
  unsigned* sync = static_cast<unsigned*>(ws);
  DotProblem p{};
  p.a = x;
  p.lda = K;
  p.w = w_ab;
  p.ldw = K;
  p.M = M;
  p.N = n_ab;
  p.K = K;
  p.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + sg::kSyncBytes);
  if (one_launch && hosts_fb(c, rank, n_b)) {
    // One grid: the F_A/beta workgroups, then the F_B role.
    p.arrive = sync;
    const sg::FusedFb ff{p.partial, sync, c.k_split, M, n_ab, rank, n_b, w_b, f_a, beta, g1};
    const DotProblem segs[1] = {p};
    const sg_config_t cfgs[1] = {c};
    const bool gemv = c.kind != SG_KIND_MFMA_WAVESPLIT;
    return hip_status(gemv ? sg::launch_gemv_fused(segs, cfgs, 1, ff, 1, s)
                           : sg::launch_mfma_fused(segs, cfgs, 1, ff, 1, s));
  }
  if (launch_main(p, c, s) != hipSuccess) return SG_ERR_HIP;
  sg::FbProblem fb{};
  fb.partial = p.partial;
  fb.S = c.k_split;
  fb.M = M;
  fb.n_ab = n_ab;
  fb.rank = rank;
  fb.n_b = n_b;
  fb.w_b = w_b;
  fb.f_a = f_a;
  fb.beta = beta;
  fb.g1 = g1;
  return hip_status(sg::launch_fab_fb_tail(fb, s));
}

}  // namespace

extern "C" int skinny_gemm(const sg_bf16* A, int64_t lda, const sg_bf16* W, int64_t ldw,
                           const sg_bf16* R, int64_t ldr, sg_bf16* C, int64_t ldc, int M, int N,
                           int K, const sg_config_t* cfg, void* ws, size_t ws_bytes,
                           sg_stream_t stream) {
  sg_config_t c;
  bool empty = false;
  int st = validate_gemm(A, lda, W, ldw, R, ldr, C, ldc, M, N, K, cfg, ws, ws_bytes, &c, &empty);
  if (st != SG_OK || empty) return st;
  DotProblem p{};
  p.a = A;
  p.lda = lda;
  p.w = W;
  p.ldw = ldw;
  p.res = R;
  p.ldr = ldr;
  p.out = C;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  return enqueue_dot(p, c, ws, static_cast<hipStream_t>(stream));
}

extern "C" int kda_qkvg_proj(const sg_bf16* x, const sg_bf16* w_qkvg, sg_bf16* qkvg, int M, int N,
                             int K, void* ws, size_t ws_bytes, sg_stream_t stream) {
  return skinny_gemm(x, K, w_qkvg, K, nullptr, N, qkvg, N, M, N, K, nullptr, ws, ws_bytes, stream);
}

extern "C" int kda_fab_fb_proj(const sg_bf16* x, const sg_bf16* w_ab, const sg_bf16* w_b,
                               sg_bf16* f_a, sg_bf16* beta, sg_bf16* g1, int M, int K, int n_ab,
                               int rank, int n_b, void* ws, size_t ws_bytes, sg_stream_t stream) {
  bool empty = false;
  int st = validate_fab_fb(x, w_ab, w_b, beta, g1, f_a, M, K, n_ab, rank, n_b, ws, ws_bytes, &empty);
  if (st != SG_OK || empty) return st;
  return enqueue_fab_fb(x, w_ab, w_b, f_a, beta, g1, M, K, n_ab, rank, n_b, ws, false,
                        static_cast<hipStream_t>(stream));
}

extern "C" int kda_fab_fb_proj_fused(const sg_bf16* x, const sg_bf16* w_ab, const sg_bf16* w_b,
                                     sg_bf16* f_a, sg_bf16* beta, sg_bf16* g1, int M, int K,
                                     int n_ab, int rank, int n_b, void* ws, size_t ws_bytes,
                                     sg_stream_t stream) {
  bool empty = false;
  int st = validate_fab_fb(x, w_ab, w_b, beta, g1, f_a, M, K, n_ab, rank, n_b, ws, ws_bytes, &empty);
  if (st != SG_OK || empty) return st;
  return enqueue_fab_fb(x, w_ab, w_b, f_a, beta, g1, M, K, n_ab, rank, n_b, ws, true,
                        static_cast<hipStream_t>(stream));
}

extern "C" int kda_projection_overlap(const sg_bf16* x, const sg_bf16* packed_w,
                                      const sg_bf16* w_b, sg_bf16* qkvg, sg_bf16* beta,
                                      sg_bf16* g1, int M, int K, int n_qkvg, int n_ab, int rank,
                                      int n_b, void* ws_main, size_t ws_main_bytes, void* ws_aux,
                                      size_t ws_aux_bytes, sg_stream_t main_stream,
                                      sg_stream_t aux_stream, sg_event_t fork, sg_event_t join) {
  // ---- validation of both branches, before anything is enqueued ----
  if (M < 0 || K < 0 || n_qkvg < 0 || n_b < 0 || rank <= 0 || n_ab <= rank)
    return SG_ERR_INVALID_ARG;
  if (rank % 8 != 0 || rank > sg::kFbMaxRank) return SG_ERR_UNSUPPORTED;
  sg_config_t cq, cf;  // the two row ranges' configurations
  int st = sg_kda_select(SG_KDA_QKVG, M, K, n_qkvg, n_ab, &cq);
  if (st != SG_OK) return st;
  if (M == 0) return SG_OK;
  if ((st = sg_kda_select(SG_KDA_FAB, M, K, n_qkvg, n_ab, &cf)) != SG_OK) return st;
  if ((st = check_operand16(x, K, K)) != SG_OK) return st;
  if ((st = check_operand16(packed_w, K, K)) != SG_OK) return st;
  if ((st = check_operand16(w_b, rank, rank)) != SG_OK) return st;
  if (n_qkvg > 0 && (st = check_output2(qkvg, n_qkvg, n_qkvg)) != SG_OK) return st;
  if ((st = check_output2(beta, n_ab - rank, n_ab - rank)) != SG_OK) return st;
  if (n_b > 0 && (st = check_output2(g1, n_b, n_b)) != SG_OK) return st;
  if (!spans_ok(M, K, K) || !spans_ok(kMaxTileRows, K, K)) return SG_ERR_UNSUPPORTED;
  const size_t need_main = sg_kda_workspace_bytes(SG_KDA_QKVG, M, K, n_qkvg, n_ab);
  const size_t need_aux = sg_kda_workspace_bytes(SG_KDA_FAB, M, K, n_qkvg, n_ab);
  if ((st = check_workspace(ws_main, ws_main_bytes, need_main)) != SG_OK) return st;
  if ((st = check_workspace(ws_aux, ws_aux_bytes, need_aux)) != SG_OK) return st;
  if (need_main > 0) {  // the two workspaces may be used concurrently
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(ws_main), a1 = a0 + need_main;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(ws_aux), b1 = b0 + need_aux;
    if (a0 < b1 && b0 < a1) return SG_ERR_INVALID_ARG;
  }

  hipStream_t sm = static_cast<hipStream_t>(main_stream);
  hipStream_t sa = static_cast<hipStream_t>(aux_stream);
  hipEvent_t ef = static_cast<hipEvent_t>(fork);
  hipEvent_t ej = static_cast<hipEvent_t>(join);
  const bool concurrent = sa != nullptr && ef != nullptr && ej != nullptr;
  const bool have_q = n_qkvg > 0 && cq.kind != SG_KIND_NONE;
  const bool split_q = have_q && cq.k_split > 1;

  // Q/K/V/G rows with their own configuration (split-K partials in ws_main).
  DotProblem q{};
  q.a = x;
  q.lda = K;
  q.w = packed_w;
  q.ldw = K;
  q.out = qkvg;
  q.ldc = n_qkvg;
  q.ldr = n_qkvg;
  q.M = M;
  q.N = n_qkvg;
  q.K = K;
  if (split_q) q.partial = static_cast<float*>(ws_main);
  sg::ReduceProblem red{};
  red.partial = static_cast<const float*>(ws_main);
  red.S = cq.k_split;
  red.M = M;
  red.N = n_qkvg;
  red.out = qkvg;
  red.ldc = n_qkvg;

  // F_A/beta rows: always fp32 partials in ws_aux, summed by the F_B stage.
  DotProblem f{};
  f.a = x;
  f.lda = K;
  f.w = packed_w + static_cast<int64_t>(n_qkvg) * K;
  f.ldw = K;
  f.M = M;
  f.N = n_ab;
  f.K = K;
  f.partial = static_cast<float*>(ws_aux);

  sg::FbProblem fb{};
  fb.partial = f.partial;
  fb.S = cf.k_split;
  fb.M = M;
  fb.n_ab = n_ab;
  fb.rank = rank;
  fb.n_b = n_b;
  fb.w_b = w_b;
  fb.beta = beta;
  fb.g1 = g1;

  // Each output element is computed by the same kernel code over the same
  // K-ranges, and every split-K sum runs in the same fixed order, in both
  // schedules: the results are bitwise identical.
  if (!concurrent) {
    // One launch for both row ranges when their configurations name the same
    // kernel instance (two segments of one grid: the small F_A/beta problem
    // fills in beside the Q/K/V/G tiles instead of trailing them), then one
    // launch for F_B and the Q/K/V/G split-K reduction.
    const DotProblem segs[2] = {q, f};
    const sg_config_t cfgs[2] = {cq, cf};
    hipError_t e = hipSuccess;
    if (have_q && is_mfma(cq.kind) && is_mfma(cf.kind) && cq.kind != SG_KIND_MFMA_WAVESPLIT &&
        sg::mfma_same_instance(cq, cf)) {
      e = sg::launch_mfma(segs, cfgs, 2, sm);
    } else if (have_q && !is_mfma(cq.kind) && cq.kind != SG_KIND_GEMV_SMALLK &&
               !is_mfma(cf.kind) && sg::gemv_same_instance(cq, cf)) {
      e = sg::launch_gemv(segs, cfgs, 2, sm);
    } else {
      if (have_q && launch_main(q, cq, sm) != hipSuccess) return SG_ERR_HIP;
      e = launch_main(f, cf, sm);
    }
    if (e != hipSuccess) return SG_ERR_HIP;
    if (split_q) fb.red = &red;
    return hip_status(sg::launch_fab_fb_tail(fb, sm));
  }

  if (hipEventRecord(ef, sm) != hipSuccess) return SG_ERR_HIP;
  if (hipStreamWaitEvent(sa, ef, 0) != hipSuccess) return SG_ERR_HIP;
  if (have_q) {
    if (launch_main(q, cq, sm) != hipSuccess) return SG_ERR_HIP;
    if (split_q && sg::launch_reduce(red, sm) != hipSuccess) return SG_ERR_HIP;
  }
  if (launch_main(f, cf, sa) != hipSuccess) return SG_ERR_HIP;
  if (sg::launch_fab_fb_tail(fb, sa) != hipSuccess) return SG_ERR_HIP;
  if (hipEventRecord(ej, sa) != hipSuccess) return SG_ERR_HIP;
  if (hipStreamWaitEvent(sm, ej, 0) != hipSuccess) return SG_ERR_HIP;
  return SG_OK;
}

// The workspace query (dispatch.cpp, host-only code) restates these.
static_assert(sg::kSyncBytes == SG_FAB_HEADER_BYTES, "hand-off header size");
static_assert(sg::kHelpSteps == 4, "one-launch K-ranges: four 512-k steps per unit");

extern "C" int sg_kda_one_launch_fits(int M, int K, int n_qkvg, int n_ab, int rank, int n_b) {
  sg::HelpPlan plan;
  return sg::help_plan(M, K, n_qkvg, n_ab, rank, n_b, &plan) ? 1 : 0;
}

extern "C" int kda_projection_fused(const sg_bf16* x, const sg_bf16* packed_w, const sg_bf16* w_b,
                                    sg_bf16* qkvg, sg_bf16* beta, sg_bf16* g1, int M, int K,
                                    int n_qkvg, int n_ab, int rank, int n_b, void* ws,
                                    size_t ws_bytes, sg_stream_t stream) {
  if (M < 0 || K < 0 || n_qkvg < 0 || n_b < 0 || rank <= 0 || n_ab <= rank)
    return SG_ERR_INVALID_ARG;
  if (rank % 8 != 0 || rank > sg::kFbMaxRank) return SG_ERR_UNSUPPORTED;
  sg_config_t cq;  // the one-stream schedule's shape checks, for either path
  int st = sg_kda_select(SG_KDA_QKVG, M, K, n_qkvg, n_ab, &cq);
  if (st != SG_OK) return st;
  if (M == 0) return SG_OK;
  if ((st = check_operand16(x, K, K)) != SG_OK) return st;
  if ((st = check_operand16(packed_w, K, K)) != SG_OK) return st;
  if ((st = check_operand16(w_b, rank, rank)) != SG_OK) return st;
  if (n_qkvg > 0 && (st = check_output2(qkvg, n_qkvg, n_qkvg)) != SG_OK) return st;
  if ((st = check_output2(beta, n_ab - rank, n_ab - rank)) != SG_OK) return st;
  if (n_b > 0 && (st = check_output2(g1, n_b, n_b)) != SG_OK) return st;
  if (!spans_ok(M, K, K) || !spans_ok(kMaxTileRows, K, K)) return SG_ERR_UNSUPPORTED;
  if ((st = check_workspace(ws, ws_bytes, sg_kda_workspace_bytes(SG_KDA_ONE_LAUNCH, M, K, n_qkvg, n_ab))) != SG_OK)
    return st;
  sg::HelpPlan plan;
  if (!sg::help_plan(M, K, n_qkvg, n_ab, rank, n_b, &plan)) {
    // The one-stream schedule, its two workspaces behind the header.
    const size_t need_main = sg_kda_workspace_bytes(SG_KDA_QKVG, M, K, n_qkvg, n_ab);
    const size_t need_aux = sg_kda_workspace_bytes(SG_KDA_FAB, M, K, n_qkvg, n_ab);
    char* base = static_cast<char*>(ws) + sg::kSyncBytes;
    return kda_projection_overlap(x, packed_w, w_b, qkvg, beta, g1, M, K, n_qkvg, n_ab, rank, n_b,
                                  need_main > 0 ? base : nullptr, need_main,
                                  need_aux > 0 ? base + need_main : nullptr, need_aux, stream,
                                  nullptr, nullptr, nullptr);
  }
  sg::OneLaunchProj p{};
  p.q.a = x;
  p.q.lda = K;
  p.q.w = packed_w;
  p.q.ldw = K;
  p.q.out = qkvg;
  p.q.ldc = n_qkvg;
  p.q.M = M;
  p.q.N = n_qkvg;
  p.q.K = K;
  p.w_ab = packed_w + static_cast<int64_t>(n_qkvg) * K;
  p.n_ab = n_ab;
  p.rank = rank;
  p.n_b = n_b;
  p.w_b = w_b;
  p.beta = beta;
  p.g1 = g1;
  p.sync = static_cast<unsigned*>(ws);
  p.pairs = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + sg::kSyncBytes);
  return hip_status(sg::launch_proj_one(p, plan, static_cast<hipStream_t>(stream)));
}

namespace {

// Validation shared by the two tail entry points: fills the configuration
// and its RMSNorm placement; *empty when there is nothing to do.
int validate_tail(const sg_bf16* latent, const sg_bf16* gamma, float eps, const sg_bf16* w_up,
                  const sg_bf16* shared, sg_bf16* out, int M, int d_latent, int d_hidden,
                  sg_config_t* cfg, bool* fold, bool* mfma_fold, bool* empty) {
  *empty = false;
  if (M < 0 || d_latent < 0 || d_hidden < 0) return SG_ERR_INVALID_ARG;
  if (!isfinite(eps) || !(eps > 0.f)) return SG_ERR_INVALID_ARG;
  sg_config_t& c = *cfg;
  int st = sg_select(M, d_hidden, d_latent, shared != nullptr, &c);
  if (st != SG_OK) return st;
  if (c.kind == SG_KIND_NONE) {
    *empty = true;
    return SG_OK;
  }
  if (d_latent == 0) return SG_ERR_INVALID_ARG;  // RMS of an empty row is undefined
  if ((st = check_operand16(latent, d_latent, d_latent)) != SG_OK) return st;
  if ((st = check_operand16(gamma, d_latent, d_latent)) != SG_OK) return st;
  if ((st = check_operand16(w_up, d_latent, d_latent)) != SG_OK) return st;
  if ((st = check_output2(out, d_hidden, d_hidden)) != SG_OK) return st;
  if (shared != nullptr && (st = check_output2(shared, d_hidden, d_hidden)) != SG_OK) return st;
  *fold = (M == 1) && (c.kind == SG_KIND_GEMV_SMALLK ||
                       ((c.kind == SG_KIND_GEMV_ROW || c.kind == SG_KIND_GEMV_SPLITK) && c.k_split == 1));
  // 2 <= M <= 16 on the wave-split MFMA tile: the kernel normalises in registers.
  *mfma_fold = sg::tail_folds(c, d_latent);
  if (!*fold && !*mfma_fold && d_latent > sg::kNormMaxD) return SG_ERR_UNSUPPORTED;
  if (!*fold && !spans_ok(kMaxTileRows, d_latent, d_latent)) return SG_ERR_UNSUPPORTED;
  return SG_OK;
}

}  // namespace

extern "C" int latent_moe_tail(const sg_bf16* latent, const sg_bf16* gamma, float eps,
                               const sg_bf16* w_up, const sg_bf16* shared, sg_bf16* out, int M,
                               int d_latent, int d_hidden, void* ws, size_t ws_bytes,
                               sg_stream_t stream) {
  sg_config_t c;
  bool fold = false, mfma_fold = false, empty = false;
  int st = validate_tail(latent, gamma, eps, w_up, shared, out, M, d_latent, d_hidden, &c, &fold,
                         &mfma_fold, &empty);
  if (st != SG_OK || empty) return st;
  const size_t need = sg_workspace_bytes(SG_OP_LATENT_TAIL, M, d_hidden, d_latent);
  if ((st = check_workspace(ws, ws_bytes, need)) != SG_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma_fold) {
    DotProblem p{};
    p.a = latent;
    p.lda = d_latent;
    p.w = w_up;
    p.ldw = d_latent;
    p.res = shared;
    p.ldr = d_hidden;
    p.out = out;
    p.ldc = d_hidden;
    p.M = M;
    p.N = d_hidden;
    p.K = d_latent;
    p.gamma = gamma;
    p.eps = eps;
    return enqueue_dot(p, c, ws, s);
  }
  if (!fold) {
    // RMSNorm into a bf16 buffer at the start of the workspace, then the GEMM
    // with the shared-expert add in its epilogue.
    const size_t norm_bytes = (static_cast<size_t>(M) * d_latent * sizeof(uint16_t) + 255) & ~size_t(255);
    sg::NormProblem np{latent, gamma, static_cast<uint16_t*>(ws), M, d_latent, eps};
    if (sg::launch_rmsnorm(np, s) != hipSuccess) return SG_ERR_HIP;
    DotProblem p{};
    p.a = static_cast<const uint16_t*>(ws);
    p.lda = d_latent;
    p.w = w_up;
    p.ldw = d_latent;
    p.res = shared;
    p.ldr = d_hidden;
    p.out = out;
    p.ldc = d_hidden;
    p.M = M;
    p.N = d_hidden;
    p.K = d_latent;
    return enqueue_dot(p, c, static_cast<char*>(ws) + norm_bytes, s);
  }
  // One GEMV launch (M = 1, whole row in one workgroup) that stages the
  // latent in LDS and normalises it there.  The small-K GEMV has no fold, so
  // a small latent uses the GEMV kernel too.
  if (c.kind == SG_KIND_GEMV_SMALLK) {
    c.kind = SG_KIND_GEMV_SPLITK;
    c.m_tile = 1;
    c.rows = 1;
    c.waves = 4;
    c.k_split = 1;
  }
  DotProblem p{};
  p.a = latent;
  p.lda = d_latent;
  p.w = w_up;
  p.ldw = d_latent;
  p.res = shared;
  p.ldr = d_hidden;
  p.out = out;
  p.ldc = d_hidden;
  p.M = M;
  p.N = d_hidden;
  p.K = d_latent;
  p.gamma = gamma;
  p.eps = eps;
  return enqueue_dot(p, c, ws, s);
}

extern "C" int latent_moe_tail_fused(const sg_bf16* latent, const sg_bf16* gamma, float eps,
                                     const sg_bf16* w_up, const sg_bf16* shared, sg_bf16* out,
                                     int M, int d_latent, int d_hidden, void* ws, size_t ws_bytes,
                                     sg_stream_t stream) {
  sg_config_t c;
  bool fold = false, mfma_fold = false, empty = false;
  int st = validate_tail(latent, gamma, eps, w_up, shared, out, M, d_latent, d_hidden, &c, &fold,
                         &mfma_fold, &empty);
  if (st != SG_OK || empty) return st;
  const size_t need = sg_workspace_bytes(SG_OP_LATENT_TAIL_FUSED, M, d_hidden, d_latent);
  if ((st = check_workspace(ws, ws_bytes, need)) != SG_OK) return st;
  char* base = static_cast<char*>(ws) + sg::kSyncBytes;
  if (fold || mfma_fold || !sg::tail_tags(c, d_hidden))
    return latent_moe_tail(latent, gamma, eps, w_up, shared, out, M, d_latent, d_hidden, base,
                           ws_bytes - sg::kSyncBytes, stream);
  // RMSNorm into a bf16 buffer behind the header, then the GEMM whose second
  // K split sums the first's tagged sums, adds the shared-expert partial and
  // stores out.
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t tail_bytes = sg_workspace_bytes(SG_OP_LATENT_TAIL, M, d_hidden, d_latent);
  sg::NormProblem np{latent, gamma, reinterpret_cast<uint16_t*>(base), M, d_latent, eps};
  if (sg::launch_rmsnorm(np, s) != hipSuccess) return SG_ERR_HIP;
  DotProblem p{};
  p.a = reinterpret_cast<const uint16_t*>(base);
  p.lda = d_latent;
  p.w = w_up;
  p.ldw = d_latent;
  p.res = shared;
  p.ldr = d_hidden;
  p.out = out;
  p.ldc = d_hidden;
  p.M = M;
  p.N = d_hidden;
  p.K = d_latent;
  p.pairs = reinterpret_cast<uint64_t*>(base + tail_bytes);
  p.sync = static_cast<unsigned*>(ws);
  return hip_status(launch_main(p, c, s));
}
