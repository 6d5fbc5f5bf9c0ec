// Host-only stand-ins for the kernel launchers (sanitizer test of the host
// code, tests/test_host_fuzz.py): they check the launch
// parameters against the kernels' limits instead of launching.
#include <cstdio>
#include <cstdlib>
#include "internal.h"
#define REQUIRE(c) do { if (!(c)) { fprintf(stderr, "contract violated: %s (%s:%d)\n", #c, __FILE__, __LINE__); abort(); } } while (0)
namespace ditango {
// same rule as the kernels': 128 rows for d = 64 and 72; d = 128 picks 256
// or 128 by the waste of the last query tile
int partial_rows_per_block(int d, int S) {
  if (d != 128) return 128;
  const long ww = (S + 255) / 256 * 256L - S, wn = (S + 127) / 128 * 128L - S;
  return wn * 10 + S < ww * 10 ? 128 : 256;
}
long g_partial = 0, g_merge = 0, g_stats = 0, g_drift = 0;
// the last per-pair work list, for the driver to compare with its mask
int g_last_n = -1, g_last_blocks = -1, g_last_qtiles = -1;
uint16_t g_last_pairs[DITANGO_MAX_P * DITANGO_MAX_P];
hipError_t launch_partial(PartialParams& p, int rows, hipStream_t) {
  REQUIRE(p.n_pairs >= 1 && p.n_pairs <= DITANGO_MAX_P * DITANGO_MAX_P);
  REQUIRE(p.P >= 1 && p.P <= DITANGO_MAX_P && p.S >= 1 && p.N >= p.P);
  REQUIRE(rows == (p.d == 128 ? rows : 128) && (rows == 128 || rows == 256));
  REQUIRE(p.q_tiles == (p.S + rows - 1) / rows);
  // K/V byte offsets of one head fit the 32-bit buffer descriptors
  REQUIRE(static_cast<long long>(p.N) * p.d * 2 < (1LL << 31));
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
long g_step = 0;
hipError_t launch_step(StepParams& p, int rows, hipStream_t) {
  REQUIRE(p.P >= 1 && p.P <= DITANGO_MAX_P && p.S >= 1 && p.N >= p.P && p.H >= 1);
  REQUIRE(rows == partial_rows_per_block(p.d, p.S));
  REQUIRE(p.q_tiles == (p.S + rows - 1) / rows);
  REQUIRE(static_cast<long long>(p.n_blocks) == static_cast<long long>(p.H) * p.P * p.q_tiles);
  REQUIRE(static_cast<long long>(p.N) * p.d * 2 < (1LL << 31));
  for (int q = 0; q < p.P; ++q) {
    REQUIRE(p.nf[q] <= p.P);
    for (int i = 0; i < p.nf[q]; ++i) {
      REQUIRE(p.fresh[q][i] < p.P);
      if (i) REQUIRE(p.fresh[q][i] > p.fresh[q][i - 1]);
    }
  }
  REQUIRE(p.O && p.LSE && p.Oout && p.LSEout);
  ++g_step; return hipSuccess;
}
long g_gstep = 0;
hipError_t launch_group_step(GroupStepParams& p, int rows, hipStream_t) {
  REQUIRE(p.P >= 1 && p.P <= DITANGO_MAX_P && p.S >= 1 && p.N >= p.P && p.H >= 1 && p.g >= 1);
  REQUIRE(rows == partial_rows_per_block(p.d, p.S));
  REQUIRE(p.q_tiles == (p.S + rows - 1) / rows);
  REQUIRE(static_cast<long long>(p.n_blocks) == static_cast<long long>(p.H) * p.P * p.q_tiles);
  REQUIRE(static_cast<long long>(p.N) * p.d * 2 < (1LL << 31));
  REQUIRE(p.Oout && p.LSEout);
  for (int q = 0; q < p.P; ++q) {
    REQUIRE(p.nl[q] >= 1 && p.nl[q] <= DITANGO_MAX_SLOTS && p.nc[q] <= p.nl[q]);
    REQUIRE(p.lslot[q][0] == 0);                       // the local slot always takes part
    for (int i = 0; i < p.nl[q]; ++i) {
      REQUIRE(p.lslot[q][i] < DITANGO_MAX_SLOTS && p.gO[p.lslot[q][i]] && p.gLSE[p.lslot[q][i]]);
      if (i) REQUIRE(p.lslot[q][i] > p.lslot[q][i - 1]);
    }
    for (int i = 0; i < p.nc[q]; ++i) {
      bool listed = false;
      for (int j = 0; j < p.nl[q]; ++j) listed = listed || p.lslot[q][j] == p.cslot[q][i];
      REQUIRE(listed);                                 // a computed slot is a live one
    }
  }
  ++g_gstep; return hipSuccess;
}
hipError_t launch_merge(const MergeParams& m, hipStream_t) {
  REQUIRE(m.n_in >= 1 && m.n_in <= DITANGO_MAX_SLOTS);
  REQUIRE((m.O != nullptr) != (m.Os != nullptr) && m.LSE);   // one output: fp32 rows or a bf16 group slot
  REQUIRE(m.res_mode == 0 || (m.O && m.res));
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
