/*
 * skinny_gemm.h -- C ABI of libskinny_gemm.so, low-M bf16 GEMMs for gfx950
 * (AMD Instinct MI355X): the Kimi-K3 KDA decode projections and the
 * latent-MoE tail.
 *
 * Sources for what each call computes (vLLM pull-request summaries on
 * prhub.com.cn):
 *   [P1] "Kimi K3 support, phase 1" (vLLM #50089), key source snippets:
 *        _skinny_gemm.py (CuteSkinnyGemm), skinny_gemm.py
 *        (SkinnyGemmConfig, ShapeDynamicSkinnyGemm._config) and
 *        latent_moe_runner.py (LatentMoERunner).
 *   [P3] "Overlap low-M TP8 KDA projections" (vLLM #54697), key source
 *        snippets: low_latency_gemm.py (run_kda_projection_overlap, run_qkvg,
 *        run_fab_fb), kda_skinny_gemm.py (_KdaSkinnyNGemm) and kda.py
 *        (KimiK3DeltaAttention.forward gate).
 *
 * Conventions that hold for every call below:
 *  - Element type: bf16, passed as its 16-bit pattern (sg_bf16).  Arithmetic:
 *    products and sums in fp32, one round-to-nearest-even to bf16 per output.
 *  - Layout: every matrix is row-major with unit column stride.  Activations
 *    are [M, K]; weights are [N, K] (the nn.Linear layout), so y = x * W^T and
 *    each output is the dot product of two contiguous K-vectors.  lda/ldw/ldr/
 *    ldc are row strides in elements.
 *  - Pointers: every matrix pointer is a DEVICE pointer (hipMalloc'd or a
 *    torch CUDA tensor) owned by the caller.  Base pointers and row strides
 *    must keep every row 16-byte aligned (pointer % 16 == 0 and ld % 8 == 0)
 *    for inputs and weights; outputs and residuals need 2-byte alignment and
 *    ld % 8 == 0 is not required for them.
 *  - Workspace: some paths keep fp32 split-K partial sums in a caller-owned
 *    device workspace; query its size with sg_workspace_bytes().  Its contents
 *    need no initialisation and are dead after the call, except for the
 *    hand-off header of kda_fab_fb_proj(_fused) workspaces (see there).  Two
 *    calls that may run concurrently must not share one workspace.
 *  - Streams/events: sg_stream_t is a hipStream_t (NULL = the legacy default
 *    stream); sg_event_t is a hipEvent_t.  Both are owned by the caller.
 *  - Asynchrony: calls validate every argument on the host, then enqueue
 *    kernels and return without synchronising.  All calls are capturable
 *    into a hipGraph (no allocation, no memset, no host synchronisation).
 *  - Errors: every argument is validated before anything is enqueued, so an
 *    error return means no work was enqueued.  A launch the runtime refuses
 *    is returned as SG_ERR_HIP; each launch's own status is read, so an error
 *    some earlier, unrelated call left pending in the runtime is neither
 *    reported as this call's nor cleared.  (If a later launch of a
 *    multi-launch call fails, the earlier ones stay enqueued.)  M == 0 (or an
 *    empty N) is a valid no-op that returns SG_OK.
 *  - Every output element is written on every successful path, and nothing
 *    outside the outputs and the workspace is written.
 *  - State: the library allocates nothing.  Its process state is, per
 *    kernel instance and per device, a flag that the kernel's dynamic-LDS
 *    limit has been raised (hipFuncSetAttribute, on first use; kept for the
 *    device current at the call, so a call must be made with its stream's
 *    device current, as torch does), the per-device address of the
 *    no-allocation scratch array (kda_projection_noalloc), and the
 *    configuration override a tuner may install (sg_set_table_override;
 *    empty unless set).  The entry points are thread-safe as long as the
 *    override does not change during calls.
 *  - Environment, read once by the first configuration call of the process
 *    (sg_select, sg_kda_select, sg_set_table_override or any entry point):
 *    SKINNY_GEMM_LOG (set, not "0") prints every configuration choice on
 *    stderr with its source (rule, measured table, override, KDA pairing);
 *    SKINNY_GEMM_TABLE installs override entries, each nine integers
 *    "N,K,m_lo,m_hi,kind,rows,waves,k_unroll,k_split" (the fields of
 *    sg_table_entry_t), entries separated by ';', checked as
 *    sg_set_table_override checks them; a malformed or unsupported value is
 *    reported on stderr and ignored.  sg_set_table_override replaces what
 *    the environment installed.  The one-launch entry points
 *    (kda_fab_fb_proj_fused, kda_projection_fused, latent_moe_tail_fused)
 *    keep their hand-off generations in a header at the start of the
 *    caller's workspace: zero before the first call on it, left consistent
 *    by every call, and not to be altered between calls.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t sg_bf16;   /* bf16 bit pattern */
typedef void *sg_stream_t;  /* hipStream_t */
typedef void *sg_event_t;   /* hipEvent_t */

/* Status codes. */
enum {
    SG_OK = 0,
    SG_ERR_INVALID_ARG = -1,  /* NULL pointer, negative size, bad eps, ... */
    SG_ERR_UNSUPPORTED = -2,  /* shape outside what the kernels cover */
    SG_ERR_MISALIGNED = -3,   /* pointer / row stride alignment violated */
    SG_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than required */
    SG_ERR_HIP = -5           /* the HIP runtime reported a launch error */
};

/* Kernel families a configuration can name. */
enum {
    SG_KIND_NONE = 0,           /* empty problem: nothing to launch */
    SG_KIND_GEMV_ROW = 1,       /* M == 1: one wave streams whole weight rows */
    SG_KIND_GEMV_SPLITK = 2,    /* M == 1, small N: K split across workgroups */
    SG_KIND_GEMV_SMALLK = 3,    /* M <= 16, K <= 256: several rows per wave */
    SG_KIND_MFMA_TILE = 4,      /* bf16 MFMA, weight and activation chunks staged
                                   in an LDS ring shared by the workgroup */
    SG_KIND_MFMA_WAVESPLIT = 5, /* bf16 MFMA, M <= 16: 16 weight rows per
                                   workgroup, each wave a private LDS ring over
                                   a quarter of K, summed in LDS */
    SG_KIND_MFMA_BLOCK = 6      /* bf16 MFMA, M > 64: 64 weight rows x 128
                                   activation rows per workgroup, both staged
                                   in an LDS ring */
};

/* Launch configuration chosen per (M, N, K): the analogue of the reference's
 * SkinnyGemmConfig [P1 skinny_gemm.py].  Fields not used by a kind are 0.
 *   kind     SG_KIND_*
 *   m_tile   activation rows the kernel instance is built for: M (GEMV),
 *            M rounded up to 4 (TILE and WAVESPLIT with M <= 16), M rounded
 *            up to 16 (TILE otherwise), M rounded up to 128 (BLOCK: blocks of
 *            128 activation rows, one per workgroup)
 *   rows     weight rows per wave (GEMV) or per workgroup (MFMA TILE and
 *            WAVESPLIT, BLOCK: 64 with 128 activation rows)
 *   waves    waves (64 lanes) per workgroup
 *   k_split  workgroups that split K; > 1 means fp32 partials in workspace
 *   k_unroll GEMV: 512-wide weight steps a wave holds; TILE / WAVESPLIT: LDS
 *            ring slots (chunks of 128 k); BLOCK: the same
 *   grid     workgroups launched by the main kernel
 *   nt_weights 1 = weights are read with non-temporal (streaming) loads */
typedef struct {
    int32_t kind;
    int32_t m_tile;
    int32_t rows;
    int32_t waves;
    int32_t k_split;
    int32_t k_unroll;
    int32_t grid;
    int32_t nt_weights;
} sg_config_t;

/* Operation identifiers for sg_workspace_bytes(). */
enum {
    SG_OP_GEMM = 0,         /* skinny_gemm / kda_qkvg_proj:  N = N            */
    SG_OP_FAB_FB = 1,       /* kda_fab_fb_proj:              N = n_ab         */
    SG_OP_LATENT_TAIL = 2,  /* latent_moe_tail:   N = d_hidden, K = d_latent  */
    SG_OP_LATENT_TAIL_FUSED = 3  /* latent_moe_tail_fused: the same N, K       */
};

/* Host-only: the configuration the library uses for C[M,N] = A[M,K] *
 * W[N,K]^T.  Plays the role of ShapeDynamicSkinnyGemm._config(m, n, k)
 * [P1 skinny_gemm.py] with a table of this library's own (the reference's
 * values were tuned for other hardware): a rule by shape, replaced where a
 * measured table entry covers (N, K, M) (sg_tuned_table; the analogue of the
 * autotuned KDA_QKVG_CONFIGS [P3 low_latency_gemm.py autotune_kda_qkvg]),
 * and before that where an entry of the caller's override covers it
 * (sg_set_table_override).  has_residual does not change the choice today;
 * it is part of the key so that it may.
 * Returns SG_OK and fills *out, SG_ERR_INVALID_ARG for negative sizes or a
 * NULL out, SG_ERR_UNSUPPORTED for K % 8 != 0 or M > 256.  An empty problem
 * (M == 0 or N == 0) returns SG_OK with kind SG_KIND_NONE. */
int sg_select(int M, int N, int K, int has_residual, sg_config_t *out);

/* One entry of the measured configuration table: problems with this N and K
 * and m_lo <= M <= m_hi take this kind, rows, waves, k_unroll and k_split
 * (m_tile and grid follow from them and M). */
typedef struct {
    int32_t N, K, m_lo, m_hi;
    int32_t kind, rows, waves, k_unroll, k_split;
} sg_table_entry_t;

/* Host-only, pure: SG_OK if the kernels can run *cfg on an M x N x K
 * problem (an instance exists for its kind, waves, rows, ring slots and
 * activation tile, m_tile and grid are the ones that follow from it, the K
 * split has no empty range, a GEMV K-range fits the steps a wave holds; the
 * small-K kind only as sg_select gives it), SG_ERR_UNSUPPORTED if not,
 * SG_ERR_INVALID_ARG for a NULL cfg or negative sizes. */
int sg_config_supported(const sg_config_t *cfg, int M, int N, int K);

/* Host-only, pure: workspace bytes skinny_gemm needs with configuration *cfg
 * at M x N (fp32 split-K partials, 0 without a K split or for a NULL cfg). */
size_t sg_config_workspace_bytes(const sg_config_t *cfg, int M, int N);

/* Host-only, pure: the compiled measured table.  Returns its number of
 * entries and, if entries != NULL, points *entries at them (static storage,
 * owned by the library). */
int sg_tuned_table(const sg_table_entry_t **entries);

/* Host-only: replaces the process-wide override table (n = 0 clears it),
 * which sg_select consults before the measured table; for a tuner that
 * times candidate configurations through the entry points.  Every entry must
 * satisfy sg_config_supported for every M of its range (else
 * SG_ERR_UNSUPPORTED, and the override is unchanged); n <= 64
 * (SG_ERR_INVALID_ARG otherwise).  This is the library's one piece of
 * mutable configuration: it must not change while other calls are in flight
 * or being captured, and workspaces sized before a change may no longer fit. */
int sg_set_table_override(const sg_table_entry_t *entries, int n);

/* Host-only, pure: whether the two-stream KDA projection should be used, the
 * analogue of the gate in KimiK3DeltaAttention.forward [P3 kda.py]:
 *   enabled && 0 < M <= sg_overlap_max_tokens() && x_contiguous &&
 *   have_aux_stream && have_events.
 * (The reference also requires CUDA-graph capture; capture state is the
 * caller's to test.)  Returns 1 or 0. */
int sg_overlap_gate(int M, int x_contiguous, int have_aux_stream, int have_events, int enabled);

/* The largest M for which sg_overlap_gate() opens (the analogue of
 * KDA_PROJECTION_OVERLAP_MAX_TOKENS [P3 low_latency_gemm.py]), compiled with
 * the measured table: the largest M up to which the two-stream schedule
 * measured faster at every M on MI355X (0: it never did, the gate stays
 * closed). */
int sg_overlap_max_tokens(void);

/* Bytes of device workspace the operation needs at this shape (0 if none).
 * Returns 0 for invalid arguments as well; the entry point then reports the
 * error. */
size_t sg_workspace_bytes(int op, int M, int N, int K);

/* Row ranges of the KDA projection, for sg_kda_select() and
 * sg_kda_workspace_bytes(). */
enum {
    SG_KDA_QKVG = 0,       /* Q/K/V/G rows in kda_projection_overlap */
    SG_KDA_FAB = 1,        /* F_A/beta rows in kda_projection_overlap */
    SG_KDA_FAB_ALONE = 2,  /* F_A/beta rows in kda_fab_fb_proj */
    SG_KDA_ONE_LAUNCH = 3  /* kda_projection_fused's workspace (sg_kda_workspace_bytes only) */
};

/* Host-only, pure: the configurations the KDA projection entry points use,
 * the analogue of the per-M KDA_QKVG_CONFIGS table and of the small-N
 * kernel's own choice [P3 low_latency_gemm.py, kda_skinny_gemm.py].
 *   SG_KDA_FAB_ALONE: sg_select(M, n_ab, K, 0), except that the small-K
 *     kind, which has no partial output, becomes GEMV_SPLITK (M == 1) or
 *     MFMA_WAVESPLIT (M > 1) over one K-range: the F_B stage always sums
 *     fp32 partials.  More than 8 K-ranges become split(steps, max(need,
 *     8)) with the grid scaled to match (steps = ceil((K/8)/64), need =
 *     ceil(steps/16) for the GEMV kinds; steps = ceil(K/32), need = 1
 *     otherwise): the F_B stage then sums them in one batch of loads.
 *   SG_KDA_QKVG / SG_KDA_FAB: sg_select(M, n_qkvg, K, 0) and the
 *     SG_KDA_FAB_ALONE configuration, except that
 *     - where the Q/K/V/G rows run whole on GEMV_ROW (k_split 1, M == 1)
 *       the F_A/beta rows take that configuration as GEMV_SPLITK with
 *       k_split = split(ceil((K/8)/64), 7), grid ceil(n_ab / (waves * rows))
 *       * k_split;
 *     - where both are MFMA_WAVESPLIT or MFMA_TILE (2 <= M <= 64) both
 *       ranges use MFMA_TILE with 128-row tiles of 8 waves (m_tile M rounded
 *       up to 4 for M <= 16, to 16 above) and one K split S =
 *       split(ceil(K/32), min(256 / (t_q + t_f), max(1, ceil(K/32) / 8))),
 *       t = ceil(rows / 128), so that the two segments of the single-stream
 *       launch run in one round of workgroups.
 * Returns SG_OK, SG_ERR_INVALID_ARG (NULL out, unknown which, negative
 * sizes) or the status of sg_select for either range. */
int sg_kda_select(int which, int M, int K, int n_qkvg, int n_ab, sg_config_t *out);

/* Bytes of device workspace kda_projection_overlap needs: which =
 * SG_KDA_QKVG for ws_main (the Q/K/V/G split-K partials, k_split * M *
 * n_qkvg * 4 rounded up to 256, 0 when unsplit), SG_KDA_FAB for ws_aux (the
 * F_A/beta partials, k_split * M * n_ab * 4 rounded up to 256), with the
 * configurations of sg_kda_select().  SG_KDA_ONE_LAUNCH: the workspace of
 * kda_projection_fused, SG_FAB_HEADER_BYTES of hand-off header followed by
 * the larger of its tagged F_A/beta partials (ceil(ceil(K/512)/4) * M *
 * n_ab * 8, rounded up to 256) and the SG_KDA_QKVG + SG_KDA_FAB workspaces.
 * 0 for any other which. */
size_t sg_kda_workspace_bytes(int which, int M, int K, int n_qkvg, int n_ab);

/* Human-readable name of a status code (static string, never NULL). */
const char *sg_strerror(int status);

/* Library version, "MAJOR.MINOR.PATCH" (static string). */
const char *sg_version(void);

/* ---- Entry points ------------------------------------------------------- */

/* Generic skinny GEMM [P1 _skinny_gemm.py CuteSkinnyGemm]:
 *   C[m,n] = bf16( sum_k A[m,k] * W[n,k] + R[m,n] )   (R omitted when NULL)
 * A [M,K] lda, W [N,K] ldw, R [M,N] ldr (nullable), C [M,N] ldc.
 * cfg: NULL = sg_select(M, N, K, R != NULL); otherwise any configuration
 * that sg_config_supported accepts for this shape (else SG_ERR_UNSUPPORTED),
 * with ws of at least sg_config_workspace_bytes(cfg, M, N) bytes (the
 * analogue of passing a config to shape_dynamic_skinny_gemm [P1]).  C may
 * alias R exactly (in-place add); any other overlap of C with an input is
 * undefined. */
int skinny_gemm(const sg_bf16 *A, int64_t lda, const sg_bf16 *W, int64_t ldw,
                const sg_bf16 *R, int64_t ldr, sg_bf16 *C, int64_t ldc,
                int M, int N, int K, const sg_config_t *cfg,
                void *ws, size_t ws_bytes, sg_stream_t stream);

/* KDA packed Q/K/V/G projection [P3 low_latency_gemm.py run_qkvg]:
 *   qkvg[m,n] = bf16( sum_k x[m,k] * w_qkvg[n,k] )
 * x [M,K] contiguous, w_qkvg [N,K] contiguous (N = 4096 for one TP8 rank:
 * q, k, v, g, 1024 columns each), qkvg [M,N] contiguous. */
int kda_qkvg_proj(const sg_bf16 *x, const sg_bf16 *w_qkvg, sg_bf16 *qkvg,
                  int M, int N, int K, void *ws, size_t ws_bytes, sg_stream_t stream);

/* KDA F_A/beta -> F_B branch [P3 low_latency_gemm.py run_fab_fb,
 * kda_skinny_gemm.py]:
 *   P[m,j]    = bf16( sum_k x[m,k] * w_ab[j,k] ),   j < n_ab
 *   f_a       = P[:, 0:rank]        (low-rank gate input, bf16)
 *   beta      = P[:, rank:n_ab]     (raw beta heads, no activation)
 *   g1[m,i]   = bf16( sum_r f_a[m,r] * w_b[i,r] ),  i < n_b
 * x [M,K], w_ab [n_ab,K], w_b [n_b,rank], f_a [M,rank] (nullable: not
 * stored), beta [M,n_ab-rank], g1 [M,n_b]; all contiguous.  Requires
 * 0 < rank < n_ab, rank % 8 == 0, rank <= 512.  Needs workspace
 * sg_workspace_bytes(SG_OP_FAB_FB, M, n_ab, K): SG_FAB_HEADER_BYTES of
 * hand-off header (used by kda_fab_fb_proj_fused only; this call neither
 * reads nor writes it), then the F_A/beta partials.  Two launches: F_A/beta
 * (split-K partials), then the F_B stage. */
#define SG_FAB_HEADER_BYTES 18432
int kda_fab_fb_proj(const sg_bf16 *x, const sg_bf16 *w_ab, const sg_bf16 *w_b,
                    sg_bf16 *f_a, sg_bf16 *beta, sg_bf16 *g1,
                    int M, int K, int n_ab, int rank, int n_b,
                    void *ws, size_t ws_bytes, sg_stream_t stream);

/* The F_A/beta -> F_B branch of kda_fab_fb_proj as ONE launch [P3
 * low_latency_gemm.py run_fab_fb, which chains its two GEMMs with
 * programmatic dependent launch]: same arguments, same workspace size and
 * bit-for-bit the same results.  Where the F_A/beta configuration runs on a
 * kernel that hosts the in-launch hand-off (the 4-wave GEMV at M == 1, the
 * wave-split MFMA tile at M <= 16 for these shapes) and the header has room
 * (at most 4096 producers and 512 F_B workgroups), the F_A/beta workgroups
 * store their partials device-coherently and each advances a flag in the
 * workspace header; F_B workgroups later in the same grid wait for every
 * flag (a bounded wait: on a time-out they write NaN to g1, beta and f_a),
 * sum the partials in fixed order and compute g1.  Elsewhere it is
 * kda_fab_fb_proj.  The header (the first SG_FAB_HEADER_BYTES of ws) must
 * be zero before the first call on a workspace; each call then keeps it
 * consistent by itself (it is not zero afterwards and must not be
 * altered), so zero-filling a workspace once when it is allocated
 * suffices, whatever the shapes of later calls.
 * On MI355X under graph replay the single launch is slower than
 * kda_fab_fb_proj's two (the in-launch hand-off costs more than a launch
 * boundary); it is for callers that count launches. */
int kda_fab_fb_proj_fused(const sg_bf16 *x, const sg_bf16 *w_ab, const sg_bf16 *w_b,
                          sg_bf16 *f_a, sg_bf16 *beta, sg_bf16 *g1,
                          int M, int K, int n_ab, int rank, int n_b,
                          void *ws, size_t ws_bytes, sg_stream_t stream);

/* Concurrent KDA projection [P3 low_latency_gemm.py
 * run_kda_projection_overlap; kda.py forward fallback]:
 *   qkvg = bf16(x @ packed_w[0:n_qkvg]^T)                    on `main`
 *   P    = bf16(x @ packed_w[n_qkvg:n_qkvg+n_ab]^T), beta = P[:, rank:],
 *   g1   = bf16(P[:, :rank] @ w_b^T)                          on `aux`
 * Fork: `fork` is recorded on main and waited on by aux; join: `join` is
 * recorded on aux and waited on by main, so every output is complete in
 * main's order once the call's work retires.  If aux, fork or join is NULL
 * the call runs on main alone (the reference's sequential path): the
 * Q/K/V/G rows and the F_A/beta rows as two segments of one launch, then one
 * launch for F_B (and the Q/K/V/G split-K reduction).  Both schedules use the
 * configurations sg_kda_select(SG_KDA_QKVG / SG_KDA_FAB, ...), so their
 * outputs are bitwise identical; where those equal the standalone
 * configurations (sg_select and SG_KDA_FAB_ALONE) they are also bitwise
 * identical to kda_qkvg_proj + kda_fab_fb_proj.
 * packed_w [n_qkvg + n_ab, K] contiguous; qkvg [M,n_qkvg]; beta
 * [M,n_ab-rank]; g1 [M,n_b]; w_b [n_b,rank]; 0 < rank < n_ab, rank % 8 == 0,
 * rank <= 512.  ws_main needs sg_kda_workspace_bytes(SG_KDA_QKVG, ...) bytes
 * (often 0) and ws_aux sg_kda_workspace_bytes(SG_KDA_FAB, ...); they must
 * not overlap. */
int kda_projection_overlap(const sg_bf16 *x, const sg_bf16 *packed_w, const sg_bf16 *w_b,
                           sg_bf16 *qkvg, sg_bf16 *beta, sg_bf16 *g1,
                           int M, int K, int n_qkvg, int n_ab, int rank, int n_b,
                           void *ws_main, size_t ws_main_bytes,
                           void *ws_aux, size_t ws_aux_bytes,
                           sg_stream_t main_stream, sg_stream_t aux_stream,
                           sg_event_t fork, sg_event_t join);

/* The KDA projection of kda_projection_overlap as ONE launch on one stream
 * [P3 low_latency_gemm.py run_kda_projection_overlap, which runs the
 * F_A/beta -> F_B chain beside the Q/K/V/G GEMM; the chain's two GEMMs are
 * themselves linked by programmatic dependent launch there]:
 * same outputs (qkvg, beta, g1; no f_a), same argument conventions.  Where
 * the shapes fit (1 <= M <= 16, K <= 8192, n_qkvg / 16 wave-split
 * workgroups of 16 Q/K/V/G rows that outnumber the F_A/beta units and F_B
 * hosts, n_ab % 4 == 0, min(M, 8) * n_ab <= 1152, rank <= 128), every Q/K/V/G
 * workgroup carries a fifth wave: in the first ceil(n_ab/4) *
 * ceil(ceil(K/512)/4) workgroups it computes fp32 partials of 4 F_A/beta
 * rows over one K-range (at most 2048 k) and stores each with the call's
 * generation (workspace header) in one 8-byte store; in the next
 * ceil(n_b/64) workgroups per group of up to 8 activation rows it reads
 * the partials of its rows until all carry the
 * generation (a bounded wait: on a time-out it writes NaN to g1 and beta),
 * sums them in fixed order into bf16 f_a and beta and computes its share of
 * g1 (at most 64 rows).  The Q/K/V/G rows are those of the wave-split tile
 * over all of K.  Elsewhere (M > 16, other shapes) the call runs the
 * one-stream schedule of kda_projection_overlap with its two workspaces
 * behind the header.
 * Results: qkvg as the wave-split tile computes it; beta and g1 from the
 * same products summed in another order than kda_projection_overlap's (both
 * within the oracle's tolerance, not bitwise equal).
 * Workspace: sg_kda_workspace_bytes(SG_KDA_ONE_LAUNCH, ...) bytes.  Its
 * header (the first SG_FAB_HEADER_BYTES) must be zero before the first call
 * on a workspace; each call keeps it consistent by itself (it is not zero
 * afterwards and must not be altered), whatever the shapes of later calls.
 * Calls that share a workspace must not run concurrently. */
int kda_projection_fused(const sg_bf16 *x, const sg_bf16 *packed_w, const sg_bf16 *w_b,
                         sg_bf16 *qkvg, sg_bf16 *beta, sg_bf16 *g1,
                         int M, int K, int n_qkvg, int n_ab, int rank, int n_b,
                         void *ws, size_t ws_bytes, sg_stream_t stream);

/* Host-only, pure: 1 if kda_projection_fused runs these shapes as one launch
 * (the conditions above), 0 if it takes the one-stream schedule. */
int sg_kda_one_launch_fits(int M, int K, int n_qkvg, int n_ab, int rank, int n_b);

/* Latent-MoE tail [P1 latent_moe_runner.py LatentMoERunner: RMS-norm of the
 * latent partial, replicated up-projection, shared-expert add folded into
 * the GEMM epilogue]:
 *   r[m]     = 1 / sqrt( (1/d_latent) * sum_k L[m,k]^2 + eps )
 *   n[m,k]   = bf16( L[m,k] * r[m] * gamma[k] )      (the bf16 RMSNorm output)
 *   out[m,j] = bf16( S[m,j] + sum_k n[m,k] * w_up[j,k] )
 * latent [M,d_latent], gamma [d_latent], w_up [d_hidden,d_latent], shared
 * [M,d_hidden] (nullable: no add), out [M,d_hidden]; all contiguous.  eps
 * must be finite and > 0, d_latent > 0.  out may alias shared exactly.
 * For M == 1 (when one workgroup covers the whole latent row) one GEMV
 * kernel normalises on the fly, and so does the wave-split MFMA tile
 * (2 <= M <= 16, at most 512 tiles of 16 rows of w_up) when d_latent <=
 * 2048; otherwise the normalised latent is written to the workspace by a
 * norm kernel and consumed by the GEMM, which needs d_latent <= 8192
 * (SG_ERR_UNSUPPORTED otherwise).  Workspace: sg_workspace_bytes(
 * SG_OP_LATENT_TAIL, M, d_hidden, d_latent), 0 unless the GEMM splits K or
 * the norm kernel runs. */
int latent_moe_tail(const sg_bf16 *latent, const sg_bf16 *gamma, float eps,
                    const sg_bf16 *w_up, const sg_bf16 *shared, sg_bf16 *out,
                    int M, int d_latent, int d_hidden,
                    void *ws, size_t ws_bytes, sg_stream_t stream);

/* latent_moe_tail with the up-projection's K-split sum inside its launch:
 * same arguments and results, bit for bit.  Where latent_moe_tail splits
 * the GEMM's K in two on the 4-wave MFMA tile (17 <= M <= 64 at the Kimi-K3
 * shapes) and then sums the splits in a second launch, here each workgroup
 * of the first split stores its fp32 sums with the call's generation
 * (workspace header) as 8-byte pairs, and the workgroup of the second split
 * for the same tile reads them until all carry the generation (a bounded
 * wait: NaN outputs on a time-out), adds them first and stores out =
 * bf16(sum + S) -- the order of the reduction launch.  Elsewhere it runs
 * latent_moe_tail with its workspace behind the header.
 * Workspace: sg_workspace_bytes(SG_OP_LATENT_TAIL_FUSED, M, d_hidden,
 * d_latent) = SG_FAB_HEADER_BYTES + latent_moe_tail's workspace + (where
 * the splits are summed in the launch) ceil(d_hidden/64) * ceil(M/16) *
 * 8192 bytes (the tagged sums of every 64-row tile and 16-row block).
 * Its header (the first SG_FAB_HEADER_BYTES) must be zero before the first
 * call on a workspace; each call keeps it consistent by itself (it is not
 * zero afterwards and must not be altered), whatever the shapes of later
 * calls.  Calls that share a workspace must not run concurrently. */
int latent_moe_tail_fused(const sg_bf16 *latent, const sg_bf16 *gamma, float eps,
                          const sg_bf16 *w_up, const sg_bf16 *shared, sg_bf16 *out,
                          int M, int d_latent, int d_hidden,
                          void *ws, size_t ws_bytes, sg_stream_t stream);

/* For callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * projection of kda_projection_overlap, same arguments and results, with
 * both workspaces taken from a device array the library owns instead of the
 * caller's ws_main / ws_aux.
 * The array holds SG_NOALLOC_SCRATCH_BYTES per GPU, zero-filled when the
 * library is loaded and kept until the process ends.  A call whose two
 * workspaces (sg_kda_workspace_bytes(SG_KDA_FAB, ...) and
 * sg_kda_workspace_bytes(SG_KDA_QKVG, ...), each rounded up to 256 bytes)
 * need more returns SG_ERR_WORKSPACE before anything is enqueued (at the
 * Kimi-K3 shapes, M <= 256 needs less than 10 MiB).  It calls no allocating
 * routine; its first call on a device looks up that device's array address
 * (hipGetSymbolAddress).  All calls on one GPU share the array: calls that
 * may overlap on one GPU (two streams, two host threads) race on it and
 * must not be issued.  Returns the statuses of kda_projection_overlap. */
#define SG_NOALLOC_SCRATCH_BYTES (16u << 20)
int kda_projection_noalloc(const sg_bf16 *x, const sg_bf16 *packed_w, const sg_bf16 *w_b,
                           sg_bf16 *qkvg, sg_bf16 *beta, sg_bf16 *g1,
                           int M, int K, int n_qkvg, int n_ab, int rank, int n_b,
                           sg_stream_t main_stream, sg_stream_t aux_stream,
                           sg_event_t fork, sg_event_t join);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
