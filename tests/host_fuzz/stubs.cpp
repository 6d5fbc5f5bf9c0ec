// Host-only stand-ins for the kernel launchers (sanitizer test of the host
// code, tests/test_host_fuzz.py): they check the launch
// parameters against the kernels' limits instead of launching.
#include <cstdio>
#include <cstdlib>
#include "internal.h"
#define REQUIRE(c) do { if (!(c)) { fprintf(stderr, "contract violated: %s (%s:%d)\n", #c, __FILE__, __LINE__); abort(); } } while (0)
namespace ditango {
int partial_rows_per_block(int d, int S) { (void)d; return S > 300 ? 256 : 128; }
long g_partial = 0, g_merge = 0, g_stats = 0, g_drift = 0;
// the last per-pair work list, for the driver to compare with its mask
int g_last_n = -1, g_last_blocks = -1, g_last_qtiles = -1;
uint16_t g_last_pairs[DITANGO_MAX_P * DITANGO_MAX_P];
hipError_t launch_partial(PartialParams& p, int rows, hipStream_t) {
  REQUIRE(p.n_pairs >= 1 && p.n_pairs <= DITANGO_MAX_P * DITANGO_MAX_P);
  REQUIRE(p.P >= 1 && p.P <= DITANGO_MAX_P && p.S >= 1 && p.N >= p.P);
  REQUIRE(p.q_tiles == (p.S + rows - 1) / rows);
  REQUIRE(static_cast<long long>(p.n_blocks) == static_cast<long long>(p.H) * p.n_pairs * p.q_tiles);
  for (int i = 0; i < p.n_pairs; ++i) {
    if (!p.grouped) REQUIRE(p.pairs[i] < p.P * p.P);
    else { int q = p.pairs[i] >> 6, s = p.pairs[i] & 63; REQUIRE(q < p.P && s < DITANGO_MAX_SLOTS && p.gO[s] && p.gLSE[s]); }
  }
  if (!p.grouped) {
    g_last_n = p.n_pairs;
    g_last_blocks = p.n_blocks;
    g_last_qtiles = p.q_tiles;
    for (int i = 0; i < p.n_pairs; ++i) g_last_pairs[i] = p.pairs[i];
  }
  ++g_partial; return hipSuccess;
}
hipError_t launch_merge(const MergeParams& m, hipStream_t) {
  REQUIRE(m.n_in >= 1 && m.n_in <= DITANGO_MAX_SLOTS);
  for (int q = 0; q < m.P; ++q) {
    REQUIRE(m.n_in == 32 || (m.live[q] >> m.n_in) == 0);
    for (int k = 0; k < m.n_in; ++k) if ((m.live[q] >> k) & 1u) REQUIRE(m.in_O[k] && m.in_L[k]);
  }
  ++g_merge; return hipSuccess;
}
hipError_t launch_stats(const StatsParams& p, hipStream_t) {
  REQUIRE(p.n_pairs >= 0 && p.n_pairs <= DITANGO_MAX_P * DITANGO_MAX_P);
  for (int i = 0; i < p.n_pairs; ++i) REQUIRE(p.pairs[i] < p.P * p.P);
  ++g_stats; return hipSuccess;
}
hipError_t launch_drift(const DriftParams& p, hipStream_t) {
  REQUIRE(p.n_pairs >= 0 && p.n_pairs <= DITANGO_MAX_P * DITANGO_MAX_P && p.P >= 1 && p.P <= DITANGO_MAX_P);
  for (int i = 0; i < p.n_pairs; ++i) REQUIRE(p.pairs[i] < p.P * p.P);
  ++g_drift; return hipSuccess;
}
}  // namespace ditango
