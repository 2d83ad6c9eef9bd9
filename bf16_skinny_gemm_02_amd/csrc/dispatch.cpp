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
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "skinny_gemm.h"

namespace {

constexpr int kWaves = 4;            // waves per workgroup unless a kind sets its own
constexpr int kGemvRowMinN = 1024;   // below this N the M = 1 GEMV splits K
constexpr int kGemvWaveTarget = 2048;  // waves the split-K GEMV aims for
constexpr int kSmallK = 256;         // K at or below this: small-K GEMV
constexpr int kGemvDepth = 16;       // 512-wide weight steps an M = 1 GEMV wave holds
constexpr int kGemvDepth4 = 7;       // the same with four weight rows per wave
constexpr int kGemvDepth7 = 4;       // ... and with seven
// MFMA ring kernels.  A chunk is 4 k-steps of 32 (128 k).
constexpr int kWgTarget = 224;       // workgroups a launch aims for (256 CUs, one each)
constexpr int kNoSplitTiles = 192;   // this many tiles fill the chip without a K split
constexpr int kSplitMaxTiles = 320;  // WAVESPLIT up to this many 16-row tiles
constexpr int kSplitPairTiles = 512; // ... or this many when two workgroups fit a CU (M <= 8)
constexpr int kSplitRing = 3;        // WAVESPLIT ring slots
constexpr int kSplitRing2 = 2;       // ... for 9 <= M <= 16 with two workgroups per CU
constexpr int kCus = 256;            // compute units (8 XCDs of 32)
constexpr int kSplitWideRows = 32;   // WAVESPLIT: most weight rows per workgroup (two fragments)
constexpr int kWideRing = 4;         // TILE ring slots for M <= 16 (2 waves, 32 rows)
constexpr int kTileRing = 3;         // TILE ring slots for 16 < M <= 64 (4 waves, 64 rows)
constexpr int kBlockRows = 64;       // BLOCK (M > 64): weight rows per workgroup
constexpr int kBlockM = 128;         // ... and activation rows per workgroup
constexpr int kBlockRing = 3;
// The packed KDA projection at 2 <= M <= 64: both row ranges in 128-row tiles
// (8 waves) with one K split, so that the two segments of the launch fit in a
// single round of workgroups on 256 CUs.
constexpr int kPairRows = 128;
constexpr int kPairWaves = 8;
constexpr int kPairRing = 3;
constexpr int kPairWgs = 256;
// K-ranges of the packed projection's F_A/beta rows beside the M = 1 GEMV (at
// most the F_B stage's batch of 8 splits, one memory round trip).
constexpr int kFabGemvSplit = 7;
// Most K-ranges of the standalone F_A/beta rows (the F_B stage's batch).
constexpr int kFabMaxSplit = 8;
// The measured table (tuned_table.inc, written by the tuner from its measured
// table, tuned_table.json): per (N, K) and range of M, the configuration that
// measured fastest on MI355X among the candidates the kernels support, and
// the overlap gate derived from timing both projection schedules.
#include "tuned_table.inc"
// Largest M for which the two-stream projection is worth its fork/join: the
// largest M up to which the fork/join schedule measured faster than the
// single-stream one at every M (0: it never did on MI355X).
constexpr int kOverlapMaxTokens = kTunedOverlapMaxTokens;
constexpr int kTunedCount = static_cast<int>(sizeof(kTunedTable) / sizeof(kTunedTable[0]));
// Process-wide override (sg_set_table_override), consulted before the table.
constexpr int kMaxOverride = 64;
sg_table_entry_t g_override[kMaxOverride];
std::atomic<int> g_override_n{0};
// Bytes at the start of a kda_fab_fb_proj(_fused) workspace: the hand-off
// header of the one-launch F_A/beta -> F_B path (4096 producer flags and 512
// consumer cursors, uint32), then the partials.
constexpr size_t kFabHeaderBytes = 18432;

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


// m_tile and grid of a configuration with the given kind, rows, waves and
// k_split for an M x N problem (the table entries leave them implicit).
int m_tile_for(int kind, int waves, int M) {
  switch (kind) {
    case SG_KIND_MFMA_WAVESPLIT: return 4 * ceil_div(M, 4);
    case SG_KIND_MFMA_TILE: return waves == 2 ? 4 * ceil_div(M, 4) : 16 * ceil_div(M, 16);
    case SG_KIND_MFMA_BLOCK: return kBlockM * ceil_div(M, kBlockM);
    default: return M;
  }
}

int grid_for(const sg_config_t& c, int M, int N) {
  const int S = c.k_split > 0 ? c.k_split : 1;
  switch (c.kind) {
    case SG_KIND_GEMV_ROW:
    case SG_KIND_GEMV_SPLITK: return ceil_div(N, c.waves * c.rows) * S;
    case SG_KIND_GEMV_SMALLK: return ceil_div(N, c.waves * c.rows);
    case SG_KIND_MFMA_BLOCK: return ceil_div(N, kBlockRows) * ceil_div(M, kBlockM) * S;
    default: return ceil_div(N, c.rows) * S;
  }
}

sg_config_t from_entry(const sg_table_entry_t& e, int M, int N) {
  sg_config_t c;
  memset(&c, 0, sizeof c);
  c.kind = e.kind;
  c.rows = e.rows;
  c.waves = e.waves;
  c.k_unroll = e.k_unroll;
  c.k_split = e.k_split;
  c.nt_weights = 1;
  c.m_tile = m_tile_for(c.kind, c.waves, M);
  c.grid = grid_for(c, M, N);
  return c;
}

int rule_select(int M, int N, int K, sg_config_t* out);

// Whether the kernels can run configuration c on an M x N x K problem (an
// instance exists for its kind, waves, rows, ring and activation tile; a
// GEMV K-range fits the steps a wave holds).  The small-K GEMV has no free
// parameter: only the rule's own configuration.
bool supported(const sg_config_t& c, int M, int N, int K) {
  if (M < 1 || M > 256 || N < 1 || K < 8 || K % 8 != 0) return false;
  if (c.nt_weights != 1 || c.k_split < 1) return false;
  if (c.m_tile != m_tile_for(c.kind, c.waves, M) || c.grid != grid_for(c, M, N)) return false;
  const int ksteps = ceil_div(K, 32);
  switch (c.kind) {
    case SG_KIND_GEMV_ROW:
    case SG_KIND_GEMV_SPLITK: {
      const int steps = ceil_div(K / 8, 64);
      const int depth = c.rows == 1 ? kGemvDepth : (c.rows == 4 ? kGemvDepth4 : kGemvDepth7);
      return M == 1 && c.waves == kWaves && (c.rows == 1 || c.rows == 4 || c.rows == 7) &&
             c.k_unroll == kGemvDepth && c.k_split <= steps &&
             effective_split(steps, c.k_split) == c.k_split && ceil_div(steps, c.k_split) <= depth;
    }
    case SG_KIND_GEMV_SMALLK: {
      sg_config_t r;
      if (rule_select(M, N, K, &r) != SG_OK) return false;
      return memcmp(&r, &c, sizeof r) == 0;
    }
    case SG_KIND_MFMA_WAVESPLIT:
      if (M > 16 || c.waves != 4) return false;
      // 2-slot rings are built for 9 <= M <= 16 only; two fragments with 3.
      if (!((c.rows == 16 && (c.k_unroll == kSplitRing || (c.k_unroll == kSplitRing2 && M > 8))) ||
            (c.rows > 16 && c.rows <= kSplitWideRows && c.rows % 4 == 0 && c.k_unroll == kSplitRing)))
        return false;
      break;
    case SG_KIND_MFMA_TILE:
      if (!((c.waves == 2 && c.rows == 32 && c.k_unroll == kWideRing && M <= 16) ||
            (c.waves == 4 && c.rows == 64 && c.k_unroll == kTileRing && M >= 17 && M <= 64) ||
            (c.waves == kPairWaves && c.rows == kPairRows && c.k_unroll == kPairRing && M >= 17 && M <= 64)))
        return false;
      break;
    case SG_KIND_MFMA_BLOCK:
      if (c.waves != 4 || c.rows != kBlockRows || c.k_unroll != kBlockRing || M < 17) return false;
      break;
    default:
      return false;
  }
  return c.k_split <= ksteps && effective_split(ksteps, c.k_split) == c.k_split;
}

// The first entry of `t` that covers (M, N, K) and whose configuration the
// kernels support there.
bool lookup(const sg_table_entry_t* t, int n, int M, int N, int K, sg_config_t* out) {
  for (int i = 0; i < n; ++i) {
    const sg_table_entry_t& e = t[i];
    if (e.N != N || e.K != K || M < e.m_lo || M > e.m_hi) continue;
    const sg_config_t c = from_entry(e, M, N);
    if (!supported(c, M, N, K)) continue;
    *out = c;
    return true;
  }
  return false;
}

// Checks the entries as sg_set_table_override documents and, if all pass,
// makes them the override table.
int install_override(const sg_table_entry_t* entries, int n) {
  if (n < 0 || n > kMaxOverride || (n > 0 && entries == nullptr)) return SG_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    const sg_table_entry_t& e = entries[i];
    if (e.N < 1 || e.K < 8 || e.K % 8 != 0 || e.m_lo < 1 || e.m_hi < e.m_lo || e.m_hi > 256)
      return SG_ERR_INVALID_ARG;
    for (int M = e.m_lo; M <= e.m_hi; ++M)
      if (!supported(from_entry(e, M, e.N), M, e.N, e.K)) return SG_ERR_UNSUPPORTED;
  }
  g_override_n.store(0, std::memory_order_release);
  for (int i = 0; i < n; ++i) g_override[i] = entries[i];
  g_override_n.store(n, std::memory_order_release);
  return SG_OK;
}

// Parses "N,K,m_lo,m_hi,kind,rows,waves,k_unroll,k_split" entries separated
// by ';' (blanks allowed around the numbers, an empty entry skipped).
// Returns the number of entries, or -1 if the text is malformed or holds
// more than kMaxOverride entries.
int parse_table(const char* text, sg_table_entry_t* out) {
  int n = 0;
  const char* p = text;
  while (*p != '\0') {
    while (*p == ' ' || *p == ';') ++p;
    if (*p == '\0') break;
    if (n == kMaxOverride) return -1;
    int32_t v[9];
    for (int f = 0; f < 9; ++f) {
      char* end = nullptr;
      const long x = strtol(p, &end, 10);
      if (end == p || x < INT32_MIN || x > INT32_MAX) return -1;
      v[f] = static_cast<int32_t>(x);
      p = end;
      while (*p == ' ') ++p;
      if (f < 8) {
        if (*p != ',') return -1;
        ++p;
      }
    }
    if (*p != ';' && *p != '\0') return -1;
    out[n++] = sg_table_entry_t{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], v[8]};
  }
  return n;
}

// The environment, read once, by the first configuration call of the
// process:
//   SKINNY_GEMM_LOG      non-empty and not "0": every sg_select and
//                        sg_kda_select prints its choice on stderr.
//   SKINNY_GEMM_TABLE    override entries (parse_table's format), installed
//                        as sg_set_table_override would; a malformed or
//                        unsupported value is reported on stderr and ignored.
// Later sg_set_table_override calls replace what the environment installed.
struct EnvState {
  bool log;
};

const EnvState& env() {
  static const EnvState state = [] {
    EnvState s{false};
    const char* log = getenv("SKINNY_GEMM_LOG");
    s.log = log != nullptr && log[0] != '\0' && strcmp(log, "0") != 0;
    const char* table = getenv("SKINNY_GEMM_TABLE");
    if (table != nullptr && table[0] != '\0') {
      sg_table_entry_t entries[kMaxOverride];
      const int n = parse_table(table, entries);
      const int st = n < 0 ? SG_ERR_INVALID_ARG : install_override(entries, n);
      if (st != SG_OK)
        fprintf(stderr, "skinny_gemm: SKINNY_GEMM_TABLE ignored (%s)\n",
                n < 0 ? "malformed" : (st == SG_ERR_UNSUPPORTED ? "unsupported entry" : "invalid entry"));
      else if (s.log)
        fprintf(stderr, "skinny_gemm: SKINNY_GEMM_TABLE installed %d entries\n", n);
    }
    return s;
  }();
  return state;
}

const char* kind_name(int kind) {
  static const char* const names[] = {"none", "gemv_row", "gemv_splitk", "gemv_smallk",
                                      "mfma_tile", "mfma_wavesplit", "mfma_block"};
  return (kind >= 0 && kind < 7) ? names[kind] : "?";
}

void log_choice(const char* what, int M, int N, int K, const sg_config_t& c, const char* source) {
  fprintf(stderr,
          "skinny_gemm: %s M=%d N=%d K=%d -> %s m_tile=%d rows=%d waves=%d k_unroll=%d "
          "k_split=%d grid=%d (%s)\n",
          what, M, N, K, kind_name(c.kind), c.m_tile, c.rows, c.waves, c.k_unroll, c.k_split,
          c.grid, source);
}

// sg_select without the log line; *source names where the choice came from.
int select_impl(int M, int N, int K, sg_config_t* out, const char** source) {
  *source = "rule";
  const int st = rule_select(M, N, K, out);
  if (st != SG_OK || out->kind == SG_KIND_NONE) return st;
  // The override, then the measured table, replace the rule's choice where
  // they cover the shape.
  const int n_over = g_override_n.load(std::memory_order_acquire);
  if (n_over > 0 && lookup(g_override, n_over, M, N, K, out)) {
    *source = "override";
    return SG_OK;
  }
  if (lookup(kTunedTable, kTunedCount, M, N, K, out)) *source = "measured table";
  return SG_OK;
}

}  // namespace

extern "C" int sg_select(int M, int N, int K, int has_residual, sg_config_t* out) {
  (void)has_residual;
  if (out == nullptr) return SG_ERR_INVALID_ARG;
  const bool log = env().log;
  const char* source;
  const int st = select_impl(M, N, K, out, &source);
  if (log && st == SG_OK) log_choice("select", M, N, K, *out, source);
  return st;
}

extern "C" int sg_config_supported(const sg_config_t* cfg, int M, int N, int K) {
  if (cfg == nullptr || M < 0 || N < 0 || K < 0) return SG_ERR_INVALID_ARG;
  return supported(*cfg, M, N, K) ? SG_OK : SG_ERR_UNSUPPORTED;
}

extern "C" size_t sg_config_workspace_bytes(const sg_config_t* cfg, int M, int N) {
  if (cfg == nullptr || M <= 0 || N <= 0) return 0;
  if (cfg->k_split <= 1 || cfg->kind == SG_KIND_GEMV_SMALLK) return 0;
  const size_t plane = static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float);
  return (static_cast<size_t>(cfg->k_split) * plane + 255) & ~static_cast<size_t>(255);
}

extern "C" int sg_tuned_table(const sg_table_entry_t** entries) {
  // A table with no entries is compiled as one sentinel entry of N = 0
  // (which no problem matches).
  const int n = (kTunedCount == 1 && kTunedTable[0].N == 0) ? 0 : kTunedCount;
  if (entries != nullptr) *entries = kTunedTable;
  return n;
}

extern "C" int sg_set_table_override(const sg_table_entry_t* entries, int n) {
  env();  // the environment's entries, if any, are in place before these replace them
  return install_override(entries, n);
}

namespace {

// The rule: the configuration by shape alone.
int rule_select(int M, int N, int K, sg_config_t* out) {
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
    // Several rows per wave when a whole short row fits in a shallower
    // register ring: fewer, longer workgroups (each stages the activation
    // once).  Seven rows of up to four steps (28 rows per workgroup: 7168
    // rows, the latent-MoE up-projection, are exactly 256 workgroups), else
    // four rows of up to seven.
    c.rows = 1;
    if (c.kind == SG_KIND_GEMV_ROW && steps <= kGemvDepth7) c.rows = 7;
    else if (c.kind == SG_KIND_GEMV_ROW && steps <= kGemvDepth4) c.rows = 4;
    const int need = ceil_div(steps, kGemvDepth);
    c.k_split = effective_split(steps, want > need ? want : need);
    c.k_unroll = kGemvDepth;
    c.grid = ceil_div(N, c.waves * c.rows) * c.k_split;
  } else if (M <= 16) {
    c.m_tile = 4 * ceil_div(M, 4);
    const int tiles16 = ceil_div(N, 16);
    // Past kSplitMaxTiles 16-row tiles, one workgroup per CU with 17..32 rows
    // (two fragments, a multiple of 4) while that covers N in one round:
    // e.g. 7168 rows are 256 workgroups of 28.
    const int wide_rows = 4 * ceil_div(ceil_div(N, kCus), 4);
    if (tiles16 > kSplitMaxTiles && wide_rows <= kSplitWideRows) {
      c.kind = SG_KIND_MFMA_WAVESPLIT;
      c.rows = wide_rows;
      c.waves = 4;
      c.k_unroll = kSplitRing;
      const int tiles = ceil_div(N, c.rows);
      c.k_split = mfma_split(tiles, ksteps, 16);
      c.grid = tiles * c.k_split;
    } else if (tiles16 <= kSplitMaxTiles || (c.m_tile <= 8 && tiles16 <= kSplitPairTiles)) {
      // Each wave walks a quarter of the workgroup's K-range: at least one
      // chunk (4 k-steps) per wave.  Up to M = 8 the 3-slot rings of two
      // workgroups fit one CU's LDS, so up to 512 tiles run in one round.
      c.kind = SG_KIND_MFMA_WAVESPLIT;
      c.rows = 16;
      c.waves = 4;
      c.k_unroll = kSplitRing;
      c.k_split = mfma_split(tiles16, ksteps, 16);
      c.grid = tiles16 * c.k_split;
    } else if (tiles16 <= kSplitPairTiles) {
      // 9 <= M <= 16: 2-slot rings, so that two workgroups again fit one CU
      // and up to 512 tiles run in one round.
      c.kind = SG_KIND_MFMA_WAVESPLIT;
      c.rows = 16;
      c.waves = 4;
      c.k_unroll = kSplitRing2;
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
    // Two-dimensional blocks: the activation is shared by 64 weight rows and
    // each weight tile by 128 activation rows.
    c.kind = SG_KIND_MFMA_BLOCK;
    c.m_tile = kBlockM * ceil_div(M, kBlockM);
    c.rows = kBlockRows;
    c.k_unroll = kBlockRing;
    const int tiles = ceil_div(N, kBlockRows) * ceil_div(M, kBlockM);
    c.k_split = mfma_split(tiles, ksteps, 8);
    c.grid = tiles * c.k_split;
  }
  *out = c;
  return SG_OK;
}

}  // namespace

extern "C" int sg_overlap_max_tokens(void) { return kOverlapMaxTokens; }

extern "C" int sg_overlap_gate(int M, int x_contiguous, int have_aux_stream, int have_events,
                               int enabled) {
  return (enabled && M > 0 && M <= kOverlapMaxTokens && x_contiguous && have_aux_stream &&
          have_events)
             ? 1
             : 0;
}

namespace sg {

// The one decision on the wave-split tile's RMSNorm fold (latent-MoE tail),
// shared by the entry point and the workspace size: whole latent rows of at
// most 2048 (4 16-byte chunks per lane, normalised once into LDS), and at
// most 16 k-steps per wave.  The kernel launcher checks the same limits
// again before it launches.
bool tail_folds(const sg_config_t& c, int K) {
  if (c.kind != SG_KIND_MFMA_WAVESPLIT) return false;
  const int ks = ceil_div(K, 32);
  const int S = c.k_split > 0 ? c.k_split : 1;
  const int sps = ceil_div(ks, S);
  return K > 0 && K <= 2048 && ceil_div(sps, 4) <= 16;
}

// Whether latent_moe_tail_fused sums the two K splits of the tail's GEMM in
// the launch (the tile kernel's tagged hand-off), shared by the entry point
// and the workspace size: the 4-wave tile with a 3-slot ring, exactly two K
// splits, an activation tile of 8, 12 or 16 row groups (17 <= M <= 64), N
// even (16-byte loads of two pairs), and at most 512 tiles per split (one
// consumer cursor each in the hand-off header).
bool tail_tags(const sg_config_t& c, int N) {
  if (c.kind != SG_KIND_MFMA_TILE || c.k_split != 2 || c.waves != 4 || c.k_unroll != 3) return false;
  if (c.m_tile != 32 && c.m_tile != 48 && c.m_tile != 64) return false;
  return N > 0 && N % 2 == 0 && c.rows > 0 && ceil_div(N, c.rows) <= 512;
}

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
      // The F_A/beta stage always leaves partials for the F_B stage to sum,
      // with the configuration sg_kda_select gives it alone, behind the
      // hand-off header of the one-launch path (kFabHeaderBytes).
      sg_config_t f;
      if (sg_kda_select(SG_KDA_FAB_ALONE, M, K, 0, N, &f) != SG_OK) return 0;
      return kFabHeaderBytes + sg::round256(static_cast<size_t>(f.k_split > 0 ? f.k_split : 1) * plane);
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
      // The wave-split tile normalises in registers: no normalised copy.
      if (sg::tail_folds(c, K)) return part;
      return sg::round256(static_cast<size_t>(M) * static_cast<size_t>(K) * 2) + part;
    }
    case SG_OP_LATENT_TAIL_FUSED: {
      // The hand-off header, latent_moe_tail's own workspace behind it, and
      // the first K split's tagged sums where the GEMM sums its splits in the
      // launch: 8 bytes per output of every 64-row tile and 16-row activation
      // block (256 threads x 4 outputs per block).
      const size_t base = sg_workspace_bytes(SG_OP_LATENT_TAIL, M, N, K);
      const size_t pairs = sg::tail_tags(c, N)
                               ? static_cast<size_t>(ceil_div(N, 64)) * static_cast<size_t>(c.m_tile / 16) * 8192
                               : 0;
      return kFabHeaderBytes + base + pairs;
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

extern "C" int sg_kda_select(int which, int M, int K, int n_qkvg, int n_ab, sg_config_t* out) {
  if (out == nullptr || which < SG_KDA_QKVG || which > SG_KDA_FAB_ALONE) return SG_ERR_INVALID_ARG;
  if (M < 0 || K < 0 || n_qkvg < 0 || n_ab < 0) return SG_ERR_INVALID_ARG;
  const bool log = env().log;
  sg_config_t q, f;
  const char *src_q, *src_f;
  int st = select_impl(M, n_qkvg, K, &q, &src_q);
  if (st != SG_OK) return st;
  if ((st = select_impl(M, n_ab, K, &f, &src_f)) != SG_OK) return st;
  // The F_A/beta rows always leave fp32 partials for the F_B stage to sum, so
  // the small-K kind (which has no partial output) is replaced by the kind
  // the table uses for these M at larger K, over one K-range.
  if (f.kind == SG_KIND_GEMV_SMALLK) {
    if (M == 1) {
      f.kind = SG_KIND_GEMV_SPLITK;
      f.m_tile = 1;
      f.rows = 1;
      f.waves = kWaves;
      f.k_unroll = kGemvDepth;
      f.grid = ceil_div(n_ab, kWaves);
    } else {
      f.kind = SG_KIND_MFMA_WAVESPLIT;
      f.m_tile = 4 * ceil_div(M, 4);
      f.rows = 16;
      f.waves = 4;
      f.k_unroll = kSplitRing;
      f.grid = ceil_div(n_ab, 16);
    }
    f.k_split = 1;
    src_f = "small-K replaced";
  }
  if (f.k_split < 1) f.k_split = 1;
  // At most one batch of partials for the F_B stage (kFabMaxSplit, one memory
  // round trip): longer F_A/beta workgroups cost less than a second round
  // trip.  A GEMV range still fits the steps a wave holds.
  if (f.k_split > kFabMaxSplit) {
    const bool gemv = f.kind == SG_KIND_GEMV_SPLITK || f.kind == SG_KIND_GEMV_ROW;
    const int steps = gemv ? ceil_div(K / 8, 64) : ceil_div(K, 32);
    const int need = gemv ? ceil_div(steps, kGemvDepth) : 1;
    const int tiles = f.grid / f.k_split;
    f.k_split = effective_split(steps, need > kFabMaxSplit ? need : kFabMaxSplit);
    f.grid = tiles * f.k_split;
  }
  if (which == SG_KDA_FAB_ALONE) {
    *out = f;
    if (log) log_choice("kda F_A/beta alone", M, n_ab, K, f, src_f);
    return SG_OK;
  }
  // M = 1 with the Q/K/V/G rows on the whole-row GEMV: the F_A/beta rows join
  // them as a second segment of the same instance with kFabGemvSplit K-ranges:
  // short workgroups that fill the CUs the Q/K/V/G rows leave idle at the end
  // of the launch, and few enough partials for the F_B stage to sum in one
  // batch.
  if (q.kind == SG_KIND_GEMV_ROW && q.k_split == 1) {
    f = q;
    f.kind = SG_KIND_GEMV_SPLITK;
    f.k_split = effective_split(ceil_div(K / 8, 64), kFabGemvSplit);
    f.grid = ceil_div(n_ab, q.waves * q.rows) * f.k_split;
    src_f = "second GEMV segment";
  }
  // 2 <= M <= 64: the table's wave-split and 64-row tiles give the Q/K/V/G
  // rows alone 256 workgroups, one per CU, so the F_A/beta segment would start
  // a second round.  Both ranges move to 128-row tiles with one K split sized
  // so that all their workgroups run in one round.
  const bool q_small = q.kind == SG_KIND_MFMA_WAVESPLIT || q.kind == SG_KIND_MFMA_TILE;
  const bool f_small = f.kind == SG_KIND_MFMA_WAVESPLIT || f.kind == SG_KIND_MFMA_TILE;
  if (q_small && f_small) {
    const int tq = ceil_div(n_qkvg, kPairRows), tf = ceil_div(n_ab, kPairRows);
    const int ksteps = ceil_div(K, 32);
    int want = kPairWgs / (tq + tf);
    int cap = ksteps / 8;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    const int S = effective_split(ksteps, want);
    sg_config_t* both[2] = {&q, &f};
    const int tiles[2] = {tq, tf};
    for (int i = 0; i < 2; ++i) {
      both[i]->kind = SG_KIND_MFMA_TILE;
      both[i]->m_tile = M <= 16 ? 4 * ceil_div(M, 4) : 16 * ceil_div(M, 16);
      both[i]->rows = kPairRows;
      both[i]->waves = kPairWaves;
      both[i]->k_unroll = kPairRing;
      both[i]->k_split = S;
      both[i]->grid = tiles[i] * S;
    }
    src_q = src_f = "one-round 128-row pairing";
  }
  *out = (which == SG_KDA_QKVG) ? q : f;
  if (log)
    log_choice(which == SG_KDA_QKVG ? "kda Q/K/V/G" : "kda F_A/beta", M,
               which == SG_KDA_QKVG ? n_qkvg : n_ab, K, *out,
               which == SG_KDA_QKVG ? src_q : src_f);
  return SG_OK;
}

extern "C" size_t sg_kda_workspace_bytes(int which, int M, int K, int n_qkvg, int n_ab) {
  if (M <= 0 || K < 0 || n_qkvg < 0 || n_ab <= 0) return 0;
  if (which == SG_KDA_ONE_LAUNCH) {
    // The hand-off header, then the larger of the one-launch F_A/beta
    // partials and the two workspaces of the one-stream schedule it falls
    // back to.
    // Its K-ranges: ceil(ceil(K/512) / 4), a unit covering four 512-k
    // steps; each partial is 8 bytes (fp32 and a generation tag).
    const int ranges = ((K / 8 + 63) / 64 + 3) / 4;
    const size_t one = sg::round256(static_cast<size_t>(ranges) * static_cast<size_t>(M) *
                                    static_cast<size_t>(n_ab) * 8);
    const size_t two = sg_kda_workspace_bytes(SG_KDA_QKVG, M, K, n_qkvg, n_ab) +
                       sg_kda_workspace_bytes(SG_KDA_FAB, M, K, n_qkvg, n_ab);
    return kFabHeaderBytes + (one > two ? one : two);
  }
  if (which != SG_KDA_QKVG && which != SG_KDA_FAB) return 0;
  sg_config_t c;
  if (sg_kda_select(which, M, K, n_qkvg, n_ab, &c) != SG_OK || c.kind == SG_KIND_NONE) return 0;
  const int N = (which == SG_KDA_QKVG) ? n_qkvg : n_ab;
  const size_t plane = static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float);
  // Q/K/V/G: split-K partials only when K is split.  F_A/beta: always partials.
  if (which == SG_KDA_QKVG && c.k_split <= 1) return 0;
  return sg::round256(static_cast<size_t>(c.k_split) * plane);
}
