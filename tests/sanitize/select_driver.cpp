// Drives the host-only configuration table (dispatch.cpp) over a grid of
// shapes for the sanitizer test: one line per query, printed as
//   <fn> <args...> : <status> <fields...>
// The test compares every line with the independent selection mirror.
#include <stdio.h>

#include "skinny_gemm.h"

static void print_cfg(const sg_config_t& c) {
  printf(" %d %d %d %d %d %d %d %d", c.kind, c.m_tile, c.rows, c.waves, c.k_split, c.k_unroll,
         c.grid, c.nt_weights);
}

int main() {
  const int shapes[][2] = {{4096, 7168}, {136, 7168}, {1024, 128}, {7168, 2048}, {4232, 7168},
                           {1, 8},       {300, 264},  {5, 256},    {17, 0},      {2048, 520}};
  for (const auto& nk : shapes) {
    for (int M = -1; M <= 260; ++M) {
      for (int res = 0; res <= 1; ++res) {
        sg_config_t c = {};
        const int st = sg_select(M, nk[0], nk[1], res, &c);
        printf("select %d %d %d %d : %d", M, nk[0], nk[1], res, st);
        if (st == SG_OK) print_cfg(c);
        printf("\n");
      }
      for (int op = 0; op <= 2; ++op)
        printf("ws %d %d %d %d : %zu\n", op, M, nk[0], nk[1], sg_workspace_bytes(op, M, nk[0], nk[1]));
    }
  }
  const int kda[][3] = {{7168, 4096, 136}, {7168, 4096, 144}, {2048, 1024, 136}, {16384, 256, 136},
                        {8, 8, 8},         {7168, 0, 136}};
  for (const auto& s : kda) {
    for (int M = -1; M <= 260; ++M) {
      for (int which = -1; which <= 3; ++which) {
        sg_config_t c = {};
        const int st = sg_kda_select(which, M, s[0], s[1], s[2], &c);
        printf("kda %d %d %d %d %d : %d", which, M, s[0], s[1], s[2], st);
        if (st == SG_OK) print_cfg(c);
        printf("\n");
        printf("kdaws %d %d %d %d %d : %zu\n", which, M, s[0], s[1], s[2],
               sg_kda_workspace_bytes(which, M, s[0], s[1], s[2]));
      }
    }
  }
  for (int M = -1; M <= 70; ++M)
    for (int bits = 0; bits < 16; ++bits)
      printf("gate %d %d %d %d %d : %d\n", M, bits & 1, (bits >> 1) & 1, (bits >> 2) & 1,
             (bits >> 3) & 1, sg_overlap_gate(M, bits & 1, (bits >> 1) & 1, (bits >> 2) & 1, (bits >> 3) & 1));
  // a NULL out and the string tables
  printf("null : %d\n", sg_select(1, 1, 8, 0, nullptr));
  for (int st = -6; st <= 1; ++st) printf("strerror %d : %s\n", st, sg_strerror(st));
  return 0;
}
