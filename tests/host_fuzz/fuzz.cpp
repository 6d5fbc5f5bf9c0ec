// Seeded fuzz of the library's host logic (masks, planner, t_c bookkeeping,
// work lists, grouped slots) under ASan/UBSan; kernels are stubbed.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <random>
#include <vector>
#include "ditango.h"
namespace ditango {
extern long g_partial, g_merge, g_stats, g_drift, g_step, g_gstep;
extern int g_last_n, g_last_blocks, g_last_qtiles;
extern uint16_t g_last_pairs[DITANGO_MAX_P * DITANGO_MAX_P];
}

// The per-pair work list of the last launch holds exactly the fresh pairs
// of `mask`, once each, and the grid is heads x pairs x query tiles.
static void check_work_list(const ditango_states_t& st, const uint8_t* mask) {
  const int P = st.shape.P;
  std::vector<int> seen(P * P, 0);
  int fresh = 0;
  for (int i = 0; i < P * P; ++i) fresh += mask[i] == 1;
  bool ok = ditango::g_last_n == fresh;
  for (int i = 0; ok && i < ditango::g_last_n; ++i) {
    const int id = ditango::g_last_pairs[i];
    ok = id < P * P && mask[id] == 1 && seen[id]++ == 0;
  }
  ok = ok && static_cast<long long>(ditango::g_last_blocks) ==
                 static_cast<long long>(st.shape.H) * fresh * ditango::g_last_qtiles;
  if (!ok) {
    fprintf(stderr, "work list does not match the mask (P=%d, fresh=%d, listed=%d)\n", P, fresh, ditango::g_last_n);
    abort();
  }
}

static std::mt19937_64 rng(12345);
static int ri(int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); }
static float rf() { return std::uniform_real_distribution<float>(0.f, 1.f)(rng); }
static float* fake(uintptr_t a) { return reinterpret_cast<float*>(a); }
static void* fakev(uintptr_t a) { return reinterpret_cast<void*>(a); }

static float wild() {   // finite, zero, inf, NaN, negative
  switch (ri(0, 9)) {
    case 0: return NAN; case 1: return INFINITY; case 2: return 0.0f; case 3: return -rf();
    default: return rf();
  }
}

int main() {
  long calls = 0, oks = 0;
  std::vector<uint8_t> m(40 * 40), m2(40 * 40);
  // masks
  for (int it = 0; it < 20000; ++it) {
    int pol = ri(-1, 5), P = ri(-1, 34), n = ri(-2, 36);
    oks += ditango_mask_build(pol, P, n, rng(), static_cast<int32_t>(rng() % 12) - 1, m.data()) == 0; ++calls;
    oks += ditango_group_mask_build(P, ri(-1, 36), n, m.data()) == 0; ++calls;
    ditango_group_slots(P, ri(-2, 40));
  }
  // planner
  for (int it = 0; it < 3000; ++it) {
    ditango_planner_t pl;
    std::memset(&pl, 0, sizeof pl);
    int P = ri(0, 33), g = ri(0, 34), H = ri(0, 3);
    float rho = ri(0, 5) == 0 ? wild() : rf(), dm = ri(0, 5) == 0 ? wild() : rf() * 0.5f;
    int rc = ditango_planner_init(&pl, P, g, H, rho, dm, ri(1, 3));
    ++calls;
    if (rc) continue;
    std::vector<float> D(P), W(static_cast<size_t>(H) * P * P), e(P * P);
    for (int t = 0; t < 12; ++t) {
      for (auto& x : D) x = ri(0, 3) ? rf() * 0.3f : wild();
      int32_t anchor = 0;
      rc = ditango_planner_plan(&pl, t, (t && ri(0, 9)) ? D.data() : nullptr, m.data(), &anchor);
      ++calls;
      if (rc) continue;
      for (int i = 0; i < P * P; ++i) m2[i] = ri(0, 9) == 0 ? 3 : m[i];
      for (auto& x : W) x = ri(0, 9) ? rf() : wild();
      for (auto& x : e) x = ri(0, 6) ? rf() : wild();
      rc = ditango_planner_update(&pl, t, ri(0, 9) ? m.data() : m2.data(), ri(0, 9) ? W.data() : nullptr,
                                  ri(0, 3) ? e.data() : nullptr);
      ++calls; oks += rc == 0;
    }
  }
  // per-pair cache
  const int dims[] = {64, 72, 128, 65};
  for (int it = 0; it < 3000; ++it) {
    ditango_shape_t sh = {ri(0, 3), ri(0, 3000), dims[ri(0, 3)], ri(0, 33), ri(0, 20) ? 0.125f : wild(),
                          ri(0, 20) ? ri(0, 1) : ri(-1, 3)};
    // now and then a sequence at the 32-bit K/V offset limit (N * d around 2^30)
    if (ri(0, 9) == 0) sh.N = (1 << 30) / sh.d + ri(-2, 1);
    ditango_states_t st;
    std::memset(&st, 0, sizeof st);
    std::vector<int32_t> tc(40 * 40, 7);
    size_t ob = 0, lb = 0;
    ditango_states_bytes(&sh, &ob, &lb);
    int rc = ditango_states_init(&st, &sh, fakev(0x100000), fake(0x200000 + (ri(0, 20) ? 0 : 4)), tc.data());
    ++calls;
    if (rc) continue;
    int P = sh.P;
    for (int t = 0; t < 6; ++t) {
      for (int i = 0; i < P * P; ++i) m[i] = t == 0 ? 1 : (ri(0, 30) ? ri(0, 1) : 2);
      for (int q = 0; q < P; ++q) m[q * P + q] = m[q * P + q] ? m[q * P + q] : (ri(0, 4) ? 1 : 0);
      std::vector<uint8_t> reused(P * P);
      ditango::g_last_n = -1;
      int prc = ditango_attn_partial(fake(0x300000), fake(0x400000), fake(0x500000), m.data(), &st, nullptr);
      ++calls; oks += prc == 0;
      if (prc == 0 && ditango::g_last_n >= 0) check_work_list(st, m.data());
      if (prc == 0) {   // no launch only when nothing is fresh
        bool any = false;
        for (int i = 0; i < P * P; ++i) any = any || m[i];
        if (any != (ditango::g_last_n >= 0)) { fprintf(stderr, "launch presence does not match the mask\n"); abort(); }
      }
      ++calls; oks += ditango_state_cache_update(&st, m.data(), ri(0, 4) ? t : ri(-2, 10), reused.data()) == 0;
      ++calls; oks += ditango_state_merge(&st, fake(0x600000), fake(0x700000), nullptr) == 0;
      ++calls; oks += ditango_attn_partial_merge(ri(0, 20) ? fake(0x300000) : nullptr, fake(0x400000), fake(0x500000),
                                                 m.data(), &st, fake(0x600000), ri(0, 20) ? fake(0x700000) : nullptr,
                                                 nullptr) == 0;
      ++calls; oks += ditango_step(fake(0x300000), fake(0x400000), fake(0x500000), m.data(), t + 10, &st, fake(0x600000),
                                   fake(0x700000), reused.data(), nullptr) == 0;
      ++calls; oks += ditango_window_residual_merge(&st, m.data(), ri(-1, 2), fake(0x800000), fake(0x600000),
                                                    fake(0x700000), nullptr) == 0;
      ++calls; oks += ditango_pair_stats(&st, ri(0, 5) ? fake(0x900000) : nullptr, m.data(),
                                         ri(0, 1) ? fake(0xa00000) : nullptr, ri(0, 5) ? fake(0xb00000) : nullptr,
                                         nullptr) == 0;
      ++calls; oks += ditango_sig_drift(fake(0xc00000), fake(0xd00000), ri(0, 3), ri(0, 34), dims[ri(0, 3)], m.data(),
                                        fake(0xe00000), nullptr) == 0;
    }
  }
  // grouped cache
  for (int it = 0; it < 3000; ++it) {
    ditango_shape_t sh = {ri(1, 3), ri(1, 3000), dims[ri(0, 2)], ri(0, 33), 0.125f, ri(0, 20) ? ri(0, 1) : ri(-1, 3)};
    ditango_gstates_t st;
    std::memset(&st, 0, sizeof st);
    std::vector<int32_t> tc(40 * DITANGO_MAX_SLOTS, 9);
    std::vector<void*> O(DITANGO_MAX_SLOTS);
    std::vector<float*> L(DITANGO_MAX_SLOTS);
    for (int s = 0; s < DITANGO_MAX_SLOTS; ++s) { O[s] = fakev(0x1000000 + 0x10000 * s); L[s] = fake(0x3000000 + 0x10000 * s); }
    int g = ri(0, 34);
    int rc = ditango_gstates_init(&st, &sh, g, O.data(), L.data(), tc.data());
    ++calls;
    if (rc) continue;
    int P = sh.P;
    for (int t = 0; t < 8; ++t) {
      for (int i = 0; i < P * P; ++i) m[i] = t == 0 ? 1 : (ri(0, 30) ? ri(0, 1) : 2);
      std::vector<uint8_t> comp(P * DITANGO_MAX_SLOTS + 8);
      ++calls; oks += ditango_group_attn_partial(fake(0x300000), fake(0x400000), fake(0x500000), m.data(), &st, nullptr) == 0;
      ++calls; oks += ditango_group_cache_update(&st, m.data(), t, comp.data()) == 0;
      ++calls; oks += ditango_group_merge(&st, fake(0x600000), fake(0x700000), nullptr) == 0;
      ++calls; oks += ditango_group_attn_partial_merge(fake(0x300000), fake(0x400000), ri(0, 20) ? fake(0x500000) : nullptr,
                                                       m.data(), &st, fake(0x600000),
                                                       ri(0, 20) ? fake(0x700000) : fake(0x700004), nullptr) == 0;
      if (ri(0, 3) == 0) { ++calls; oks += ditango_group_compose(&st, ri(0, 5), nullptr) == 0; }
      if (ri(0, 3) == 0) {
        const size_t sb = ditango_gstates_slot_bytes(&st.shape, nullptr, nullptr);
        int32_t merges = -1;
        ++calls; oks += ditango_group_fit(&st, sb * static_cast<size_t>(ri(0, 34)), ri(0, 5), nullptr,
                                          ri(0, 5) ? &merges : nullptr) == 0;
      }
      if (ri(0, 7) == 0) { ++calls; oks += ditango_group_reset(&st, O.data(), L.data()) == 0; }
    }
  }
  printf("calls %ld ok %ld; launches fused_step %ld group_step %ld partial %ld merge %ld stats %ld drift %ld\n", calls, oks,
         ditango::g_step, ditango::g_gstep, ditango::g_partial,
         ditango::g_merge, ditango::g_stats, ditango::g_drift);
  return 0;
}
