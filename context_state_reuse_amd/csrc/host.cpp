// Host half of the C ABI: argument checks, the fresh-pair work list, the
// last-computation timestamps t_c, the selection-mask builders and errors.
//
// Method: "DiTango: Cost-Effective Parallel Diffusion Generation with
// Selective Attention State Reuse" -- state selection (COMPUTE/REUSE per
// unit, t_c = last computation step), anchor steps (all compute, t_c <- t),
// selective compute and reuse (Fig. 6).  The unit is one (query partition,
// KV partition) pair in the per-pair cache, one slot (the local pair or a
// group of adjacent partitions) in the grouped cache, whose groups can be
// merged k at a time (Dynamic Group State Compose).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "ditango.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DITANGO_OK;
}

// Validates a shape and returns S = ceil(N/P) through *S_out.
int check_shape(const ditango_shape_t* s, int32_t* S_out) {
  if (!s) return fail(DITANGO_EINVAL, "shape is NULL");
  if (s->H < 1 || s->N < 1) return fail(DITANGO_EINVAL, "H=%d and N=%d must be >= 1", s->H, s->N);
  if (s->P < 1 || s->P > DITANGO_MAX_P)
    return fail(DITANGO_EINVAL, "P=%d outside 1..%d", s->P, DITANGO_MAX_P);
  if (s->d != 64 && s->d != 72 && s->d != 128)
    return fail(DITANGO_EINVAL, "head dim d=%d not supported (64, 72 or 128)", s->d);
  if (!(s->scale > 0.0f) || !std::isfinite(s->scale))
    return fail(DITANGO_EINVAL, "scale must be finite and > 0");
  if (s->N < s->P) return fail(DITANGO_EINVAL, "N=%d < P=%d leaves an empty partition", s->N, s->P);
  if (s->state_dtype != DITANGO_STATE_F32 && s->state_dtype != DITANGO_STATE_BF16)
    return fail(DITANGO_EINVAL, "state_dtype=%d is neither DITANGO_STATE_F32 nor DITANGO_STATE_BF16", s->state_dtype);
  // K/V of one head are addressed through buffer descriptors with 32-bit
  // byte offsets: N * d * 2 bytes must stay below 2^31.
  if (static_cast<int64_t>(s->N) * s->d >= (int64_t{1} << 30))
    return fail(DITANGO_EINVAL, "N=%d x d=%d must stay below 2^30 elements per head", s->N, s->d);
  const int64_t S = (static_cast<int64_t>(s->N) + s->P - 1) / s->P;
  if (static_cast<int64_t>(s->P - 1) * S >= s->N)
    return fail(DITANGO_EINVAL, "N=%d, P=%d: partitions of %lld tokens leave the last one empty",
                s->N, s->P, static_cast<long long>(S));
  *S_out = static_cast<int32_t>(S);
  return DITANGO_OK;
}

int check_states(const ditango_states_t* st) {
  if (!st) return fail(DITANGO_EINVAL, "states is NULL");
  int32_t S = 0;
  int rc = check_shape(&st->shape, &S);
  if (rc) return rc;
  if (S != st->S) return fail(DITANGO_EINVAL, "states.S=%d does not match ceil(N/P)=%d", st->S, S);
  if (!st->O || !st->LSE || !st->tc) return fail(DITANGO_EINVAL, "states buffers are NULL");
  return DITANGO_OK;
}

int check_mask(const uint8_t* mask, int P) {
  if (!mask) return fail(DITANGO_EINVAL, "mask is NULL");
  for (int i = 0; i < P * P; ++i)
    if (mask[i] > 1) return fail(DITANGO_EINVAL, "mask[%d][%d]=%d is not 0 or 1", i / P, i % P, mask[i]);
  return DITANGO_OK;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014), mix64 variant.
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// ---- grouped cache: slot s of query partition q (0 = local pair,
// 1 + j = group j = partitions [j g, min((j+1) g, P)) without q)

int group_slots(int P, int g) {
  if (P < 1 || P > DITANGO_MAX_P || g < 1) return 0;
  const int n = 1 + (P + g - 1) / g;
  return n > DITANGO_MAX_SLOTS ? 0 : n;
}

void group_range(int P, int g, int s, int q, int* a, int* b) {
  if (s == 0) {
    *a = q;
    *b = q + 1;
  } else {
    *a = (s - 1) * g;
    *b = std::min(*a + g, P);
  }
}

// The slot holds a state of at least one partition (group {q} alone does not).
bool slot_live(int P, int g, int q, int s) {
  int a, b;
  group_range(P, g, s, q, &a, &b);
  return s == 0 || b - a > 1 || a != q;
}

// COMPUTE when any member is fresh in the pair mask.
bool slot_fresh(const uint8_t* mask, int P, int g, int q, int s) {
  int a, b;
  group_range(P, g, s, q, &a, &b);
  for (int k = a; k < b; ++k)
    if ((s == 0 || k != q) && mask[q * P + k]) return true;
  return false;
}

// Key tokens of slot s of q (the state's reduction length).
int64_t slot_keys(int N, int P, int S, int g, int q, int s) {
  int a, b;
  group_range(P, g, s, q, &a, &b);
  int64_t n = std::min<int64_t>(static_cast<int64_t>(b) * S, N) - static_cast<int64_t>(a) * S;
  if (s != 0 && a <= q && q < b) n -= std::min<int64_t>(S, N - static_cast<int64_t>(q) * S);
  return n;
}

int& gtc(const ditango_gstates_t* st, int q, int s) { return st->tc[q * DITANGO_MAX_SLOTS + s]; }

// Bytes of one cached OUT element, and the element offset of a slot block
// as a byte pointer.
size_t out_elem_bytes(const ditango_shape_t& s) { return s.state_dtype == DITANGO_STATE_BF16 ? 2 : 4; }
const void* elem_offset(const void* base, size_t elems, const ditango_shape_t& s) {
  return static_cast<const char*>(base) + elems * out_elem_bytes(s);
}

int check_slot_buffers(void* const* O, float* const* LSE, int n) {
  if (!O || !LSE) return fail(DITANGO_EINVAL, "slot buffer tables are NULL");
  for (int s = 0; s < n; ++s) {
    if (!O[s] || !LSE[s]) return fail(DITANGO_EINVAL, "slot %d buffers are NULL", s);
    if ((reinterpret_cast<uintptr_t>(O[s]) | reinterpret_cast<uintptr_t>(LSE[s])) & 15u)
      return fail(DITANGO_EINVAL, "slot %d buffers must be 16-byte aligned", s);
  }
  return DITANGO_OK;
}

int check_gstates(const ditango_gstates_t* st, int* n_slots) {
  if (!st) return fail(DITANGO_EINVAL, "states is NULL");
  int32_t S = 0;
  int rc = check_shape(&st->shape, &S);
  if (rc) return rc;
  if (S != st->S) return fail(DITANGO_EINVAL, "states.S=%d does not match ceil(N/P)=%d", st->S, S);
  if (st->g0 < 1 || st->g < st->g0 || st->g % st->g0)
    return fail(DITANGO_EINVAL, "group sizes g0=%d, g=%d are inconsistent", st->g0, st->g);
  const int n = group_slots(st->shape.P, st->g);
  if (!n) return fail(DITANGO_EINVAL, "group size %d gives too many slots for P=%d", st->g, st->shape.P);
  if (!st->tc) return fail(DITANGO_EINVAL, "tc is NULL");
  if ((rc = check_slot_buffers(st->O, st->LSE, n))) return rc;
  *n_slots = n;
  return DITANGO_OK;
}

hipError_t launch_group_merge(ditango::MergeParams& m, const ditango_gstates_t* st, int n_in,
                              hipStream_t stream) {
  m.in_hs = st->shape.P;
  m.in_qs = 1;
  m.n_in = n_in;
  m.H = st->shape.H;
  m.N = st->shape.N;
  m.P = st->shape.P;
  m.S = st->S;
  m.d = st->shape.d;
  return ditango::launch_merge(m, stream);
}

}  // namespace

extern "C" {

const char* ditango_last_error(void) { return g_err.c_str(); }

int32_t ditango_version(void) { return 6; }

size_t ditango_states_bytes(const ditango_shape_t* shape, size_t* o_bytes, size_t* lse_bytes) {
  int32_t S = 0;
  if (check_shape(shape, &S)) return 0;
  const size_t slots = static_cast<size_t>(shape->H) * shape->P * shape->P;
  const size_t ob = slots * S * shape->d * out_elem_bytes(*shape);
  const size_t lb = slots * S * sizeof(float);
  if (o_bytes) *o_bytes = ob;
  if (lse_bytes) *lse_bytes = lb;
  ok();
  return ob + lb;
}

int ditango_states_init(ditango_states_t* st, const ditango_shape_t* shape, void* O, float* LSE,
                        int32_t* tc) {
  if (!st) return fail(DITANGO_EINVAL, "states is NULL");
  int32_t S = 0;
  int rc = check_shape(shape, &S);
  if (rc) return rc;
  if (!O || !LSE || !tc) return fail(DITANGO_EINVAL, "O, LSE and tc must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  st->shape = *shape;
  st->S = S;
  st->O = O;
  st->LSE = LSE;
  st->tc = tc;
  for (int i = 0; i < shape->P * shape->P; ++i) tc[i] = -1;
  return ok();
}

int ditango_attn_partial(const void* Q, const void* K, const void* V, const uint8_t* mask,
                         ditango_states_t* st, void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(mask, P))) return rc;
  if (!Q || !K || !V) return fail(DITANGO_EINVAL, "Q, K and V must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15u)
    return fail(DITANGO_EINVAL, "Q, K and V must be 16-byte aligned");
  // Every REUSE pair must hold a state before anything is launched.
  for (int i = 0; i < P * P; ++i)
    if (!mask[i] && st->tc[i] < 0)
      return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) is marked REUSE but was never computed", i / P, i % P);

  ditango::PartialParams p;
  std::memset(&p, 0, sizeof p);
  // Fresh pairs grouped by KV partition so that blocks sharing K/V run close
  // together in time (and on one L2 slice after the XCD remap).
  int n = 0;
  for (int k = 0; k < P; ++k)
    for (int q = 0; q < P; ++q)
      if (mask[q * P + k]) p.pairs[n++] = static_cast<uint16_t>(q * P + k);
  if (n == 0) return ok();  // everything reused: no work
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.O = st->O;
  p.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  p.LSE = st->LSE;
  p.H = st->shape.H;
  p.N = st->shape.N;
  p.P = P;
  p.S = st->S;
  p.d = st->shape.d;
  p.scale_log2 = st->shape.scale * 1.4426950408889634f;
  p.n_pairs = n;
  const int rows = ditango::partial_rows_per_block(p.d, p.S);
  p.q_tiles = (p.S + rows - 1) / rows;
  const int64_t blocks = static_cast<int64_t>(p.H) * n * p.q_tiles;
  if (blocks > 0x7fffffff) return fail(DITANGO_EINVAL, "grid of %lld blocks is too large", (long long)blocks);
  p.n_blocks = static_cast<int32_t>(blocks);
  hipError_t e = ditango::launch_partial(p, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "partial kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_state_cache_update(ditango_states_t* st, const uint8_t* mask, int32_t step,
                               uint8_t* reused_out) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(mask, P))) return rc;
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  for (int i = 0; i < P * P; ++i) {
    if (st->tc[i] > step)
      return fail(DITANGO_EINVAL, "step=%d is earlier than pair %d's last computation step %d", step, i,
                  st->tc[i]);
    if (!mask[i] && st->tc[i] < 0)
      return fail(DITANGO_EINVAL, "pair (q=%d, k=%d) reused but never computed", i / P, i % P);
  }
  for (int i = 0; i < P * P; ++i) {
    if (mask[i]) st->tc[i] = step;
    if (reused_out) reused_out[i] = mask[i] ? 0 : 1;
  }
  return ok();
}

int ditango_state_merge(const ditango_states_t* st, float* O, float* LSE, void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  if (!O || !LSE) return fail(DITANGO_EINVAL, "O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  const int P = st->shape.P;
  for (int i = 0; i < P * P; ++i)
    if (st->tc[i] < 0) return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) holds no state", i / P, i % P);
  // State k of the rows of (h, q) is slot h*P*P + q*P + k.
  ditango::MergeParams m;
  std::memset(&m, 0, sizeof m);
  m.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  const size_t slot_o = static_cast<size_t>(st->S) * st->shape.d;
  for (int k = 0; k < P; ++k) {
    m.in_O[k] = elem_offset(st->O, k * slot_o, st->shape);
    m.in_L[k] = st->LSE + static_cast<size_t>(k) * st->S;
  }
  for (int q = 0; q < P; ++q) m.live[q] = P == 32 ? 0xffffffffu : (1u << P) - 1u;
  m.in_hs = static_cast<int64_t>(P) * P;
  m.in_qs = P;
  m.out_hs = st->shape.N;
  m.out_qs = st->S;
  m.O = O;
  m.LSE = LSE;
  m.n_in = P;
  m.H = st->shape.H;
  m.N = st->shape.N;
  m.P = P;
  m.S = st->S;
  m.d = st->shape.d;
  hipError_t e = ditango::launch_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_pair_stats(const ditango_states_t* st, const float* LSE, const uint8_t* select, float* W, float* SIG,
                       void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(select, P))) return rc;
  if (W && !LSE) return fail(DITANGO_EINVAL, "LSE must be non-NULL when W is wanted");
  bool any = false;
  for (int i = 0; i < P * P; ++i) any |= select[i] != 0;
  if (any && !SIG) return fail(DITANGO_EINVAL, "SIG must be non-NULL when pairs are selected");
  if (reinterpret_cast<uintptr_t>(SIG) & 15u) return fail(DITANGO_EINVAL, "SIG must be 16-byte aligned");
  for (int i = 0; i < P * P; ++i)
    if (st->tc[i] < 0) return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) holds no state", i / P, i % P);
  ditango::StatsParams sp;
  std::memset(&sp, 0, sizeof sp);
  sp.O = st->O;
  sp.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  sp.LSE_slot = st->LSE;
  sp.LSE = LSE;
  sp.W = W;
  sp.SIG = SIG;
  for (int q = 0; q < P; ++q)
    for (int k = 0; k < P; ++k)
      if (select[q * P + k]) {
        sp.sel[q] |= 1u << k;
        sp.pairs[sp.n_pairs++] = static_cast<uint16_t>(q * P + k);
      }
  sp.H = st->shape.H;
  sp.N = st->shape.N;
  sp.P = P;
  sp.S = st->S;
  sp.d = st->shape.d;
  hipError_t e = ditango::launch_stats(sp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "stats kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_sig_drift(const float* A, const float* B, int32_t H, int32_t P, int32_t d, const uint8_t* select,
                      float* out, void* stream) {
  if (!A || !B || !out) return fail(DITANGO_EINVAL, "A, B and out must be non-NULL");
  if (H < 1 || d < 1) return fail(DITANGO_EINVAL, "H=%d and d=%d must be >= 1", H, d);
  if (P < 1 || P > DITANGO_MAX_P) return fail(DITANGO_EINVAL, "P=%d outside 1..%d", P, DITANGO_MAX_P);
  if (static_cast<int64_t>(H) * d > 0x7fffffff)
    return fail(DITANGO_EINVAL, "H=%d x d=%d values per pair exceed 2^31 - 1", H, d);
  int rc = check_mask(select, P);
  if (rc) return rc;
  ditango::DriftParams dp;
  std::memset(&dp, 0, sizeof dp);
  dp.A = A;
  dp.B = B;
  dp.out = out;
  dp.H = H;
  dp.P = P;
  dp.d = d;
  for (int i = 0; i < P * P; ++i)
    if (select[i]) dp.pairs[dp.n_pairs++] = static_cast<uint16_t>(i);
  hipError_t e = ditango::launch_drift(dp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "drift kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// ---- anchor-guided planner (host only) ----
//
// DiTango page, error-analysis and state-selection sections (Eq. 5-9,
// Algorithm 1): ASE of a cached state = importance w times an error that
// grows with the cache age; groups (local state apart, always computed) are
// computed when their summed ASE exceeds eps, reused otherwise; anchor steps
// compute everything when the local state drifts too far, and re-measure w,
// the scale ratios alpha and eps.  The page's equations are lost; the
// concrete model is the one stated in ditango.h.  The planner works on
// scalars only (drifts and importances reduced on the GPU).

namespace {

int planner_groups(const ditango_planner_t* pl) { return (pl->P + pl->g - 1) / pl->g; }

// Members of group j for query partition q: [j g, min((j+1) g, P)) without q.
int group_members(const ditango_planner_t* pl, int q, int j, int* out) {
  int n = 0;
  for (int k = j * pl->g; k < std::min((j + 1) * pl->g, pl->P); ++k)
    if (k != q) out[n++] = k;
  return n;
}

int check_planner(const ditango_planner_t* pl) {
  if (!pl) return fail(DITANGO_EINVAL, "planner is NULL");
  if (pl->P < 1 || pl->P > DITANGO_MAX_P || pl->g < 1 || pl->g > pl->P || pl->H < 1 || pl->warmup < 2)
    return fail(DITANGO_EINVAL, "planner is not initialised");
  return DITANGO_OK;
}

}  // namespace

int ditango_planner_init(ditango_planner_t* pl, int32_t P, int32_t g, int32_t H, float target_reuse,
                         float drift_max, int32_t warmup) {
  if (!pl) return fail(DITANGO_EINVAL, "planner is NULL");
  if (P < 1 || P > DITANGO_MAX_P) return fail(DITANGO_EINVAL, "P=%d outside 1..%d", P, DITANGO_MAX_P);
  if (g < 1 || g > P) return fail(DITANGO_EINVAL, "group size g=%d outside 1..P", g);
  if (H < 1) return fail(DITANGO_EINVAL, "H=%d must be >= 1", H);
  if (!(target_reuse >= 0.0f && target_reuse <= 1.0f)) return fail(DITANGO_EINVAL, "target_reuse outside [0, 1]");
  if (!(drift_max >= 0.0f)) return fail(DITANGO_EINVAL, "drift_max must be >= 0");
  if (warmup < 2) return fail(DITANGO_EINVAL, "warmup=%d must be >= 2", warmup);
  std::memset(pl, 0, sizeof *pl);
  pl->P = P;
  pl->g = g;
  pl->H = H;
  pl->target_reuse = target_reuse;
  pl->drift_max = drift_max;
  pl->warmup = warmup;
  pl->eps = HUGE_VAL;
  pl->last_anchor = -1;
  return ok();
}

int ditango_planner_plan(ditango_planner_t* pl, int32_t step, const float* drift, uint8_t* mask_out,
                         int32_t* anchor_out) {
  int rc = check_planner(pl);
  if (rc) return rc;
  if (!mask_out) return fail(DITANGO_EINVAL, "mask_out must be non-NULL");
  if (pl->n_anchors > 0 && !drift) return fail(DITANGO_EINVAL, "drift must be non-NULL after the first anchor");
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  const int P = pl->P;
  bool beyond = false;
  for (int q = 0; q < P; ++q) {
    pl->D[q] = pl->n_anchors > 0 ? static_cast<double>(drift[q]) : 0.0;
    beyond = beyond || !(pl->D[q] <= pl->drift_max);   // NaN counts as beyond any bound
  }
  pl->anchor = step < pl->warmup || pl->n_anchors == 0 || beyond;
  if (anchor_out) *anchor_out = pl->anchor;
  if (pl->anchor) {
    std::memset(mask_out, 1, static_cast<size_t>(P) * P);
    return ok();
  }
  std::memset(mask_out, 0, static_cast<size_t>(P) * P);
  for (int q = 0; q < P; ++q) {
    mask_out[q * P + q] = 1;
    for (int j = 0; j < planner_groups(pl); ++j) {
      int mem[DITANGO_MAX_P];
      const int n = group_members(pl, q, j, mem);
      if (n == 0) continue;
      const double grow = std::max(0.0, pl->D[q] - pl->Dc[q][j]);
      // no growth predicts no error, and a member of zero importance adds
      // none (also when its scale ratio is +inf)
      double ase = 0.0;
      if (grow > 0.0)
        for (int i = 0; i < n; ++i)
          if (pl->W[q][mem[i]] > 0.0) ase += pl->W[q][mem[i]] * pl->alpha[q][mem[i]] * grow;
      if (ase > pl->eps)
        for (int i = 0; i < n; ++i) mask_out[q * P + mem[i]] = 1;
    }
  }
  return ok();
}

int ditango_planner_update(ditango_planner_t* pl, int32_t step, const uint8_t* mask, const float* W,
                           const float* e) {
  int rc = check_planner(pl);
  if (rc) return rc;
  const int P = pl->P, H = pl->H;
  if ((rc = check_mask(mask, P))) return rc;
  if (pl->anchor && !W) return fail(DITANGO_EINVAL, "W must be non-NULL at an anchor step");
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  if (pl->anchor) {
    // Statistics are checked before anything changes: a NaN would leave the
    // errors below without an order.  A drift may be +inf (a signature that
    // was zero has moved).
    for (size_t i = 0; i < static_cast<size_t>(H) * P * P; ++i)
      if (!(W[i] >= 0.0f) || !std::isfinite(W[i]))
        return fail(DITANGO_EINVAL, "W[%zu] = %g is not a finite importance >= 0", i, static_cast<double>(W[i]));
    if (e && pl->n_anchors > 0)
      for (int i = 0; i < P * P; ++i)
        if (i / P != i % P && !(e[i] >= 0.0f))
          return fail(DITANGO_EINVAL, "e[%d][%d] = %g is not a drift >= 0", i / P, i % P, static_cast<double>(e[i]));
  }
  if (pl->anchor) {
    for (int q = 0; q < P; ++q)
      for (int k = 0; k < P; ++k) {
        double s = 0.0;
        for (int h = 0; h < H; ++h) s += W[(static_cast<size_t>(h) * P + q) * P + k];
        pl->W[q][k] = s / H;
      }
    if (e && pl->n_anchors > 0) {
      for (int q = 0; q < P; ++q)
        for (int k = 0; k < P; ++k)
          if (k != q) pl->alpha[q][k] = pl->D[q] > 0.0 ? static_cast<double>(e[q * P + k]) / pl->D[q] : 0.0;
      std::vector<double> E;
      for (int q = 0; q < P; ++q)
        for (int j = 0; j < planner_groups(pl); ++j) {
          int mem[DITANGO_MAX_P];
          const int n = group_members(pl, q, j, mem);
          if (n == 0) continue;
          double s = 0.0;
          // a pair of zero importance adds nothing, whatever its drift
          for (int i = 0; i < n; ++i)
            if (pl->W[q][mem[i]] > 0.0) s += pl->W[q][mem[i]] * static_cast<double>(e[q * P + mem[i]]);
          E.push_back(s);
        }
      std::sort(E.begin(), E.end());
      const long kq = E.empty() ? 0 : static_cast<long>(std::ceil(pl->target_reuse * static_cast<double>(E.size()) - 1e-12));
      pl->eps = E.empty() ? HUGE_VAL : kq <= 0 ? -HUGE_VAL : E[std::min<size_t>(kq, E.size()) - 1];
    }
    for (int q = 0; q < P; ++q)
      for (int j = 0; j < DITANGO_MAX_P; ++j) pl->Dc[q][j] = 0.0;
    pl->n_anchors += 1;
    pl->last_anchor = step;
  } else {
    for (int q = 0; q < P; ++q)
      for (int j = 0; j < planner_groups(pl); ++j) {
        int mem[DITANGO_MAX_P];
        const int n = group_members(pl, q, j, mem);
        bool all = n > 0;
        for (int i = 0; i < n; ++i) all = all && mask[q * P + mem[i]];
        if (all) pl->Dc[q][j] = pl->D[q];
      }
  }
  return ok();
}

// The fused launch of a step: checks, then one step_kernel launch (fresh
// pairs per query-partition row, states stored, rows composed).
static int launch_fused_step(const void* Q, const void* K, const void* V, const uint8_t* mask,
                             const ditango_states_t* st, float* O, float* LSE, void* stream) {
  const int P = st->shape.P;
  ditango::StepParams sp;
  std::memset(&sp, 0, sizeof sp);
  for (int q = 0; q < P; ++q) {
    int n = 0;
    for (int k = 0; k < P; ++k)
      if (mask[q * P + k]) sp.fresh[q][n++] = static_cast<uint8_t>(k);
    sp.nf[q] = static_cast<uint8_t>(n);
  }
  sp.Q = static_cast<const __bf16*>(Q);
  sp.K = static_cast<const __bf16*>(K);
  sp.V = static_cast<const __bf16*>(V);
  sp.O = st->O;
  sp.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  sp.LSE = st->LSE;
  sp.Oout = O;
  sp.LSEout = LSE;
  sp.H = st->shape.H;
  sp.N = st->shape.N;
  sp.P = P;
  sp.S = st->S;
  sp.d = st->shape.d;
  sp.scale_log2 = st->shape.scale * 1.4426950408889634f;
  const int rows = ditango::partial_rows_per_block(sp.d, sp.S);
  sp.q_tiles = (sp.S + rows - 1) / rows;
  const int64_t blocks = static_cast<int64_t>(sp.H) * P * sp.q_tiles;
  if (blocks > 0x7fffffff) return fail(DITANGO_EINVAL, "grid of %lld blocks is too large", (long long)blocks);
  sp.n_blocks = static_cast<int32_t>(blocks);
  hipError_t e = ditango::launch_step(sp, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "step kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_attn_partial_merge(const void* Q, const void* K, const void* V, const uint8_t* mask,
                               ditango_states_t* st, float* O, float* LSE, void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(mask, P))) return rc;
  if (!Q || !K || !V) return fail(DITANGO_EINVAL, "Q, K and V must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15u)
    return fail(DITANGO_EINVAL, "Q, K and V must be 16-byte aligned");
  if (!O || !LSE) return fail(DITANGO_EINVAL, "O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  for (int i = 0; i < P * P; ++i)
    if (!mask[i] && st->tc[i] < 0)
      return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) is marked REUSE but was never computed", i / P, i % P);
  return launch_fused_step(Q, K, V, mask, st, O, LSE, stream);
}

int ditango_step(const void* Q, const void* K, const void* V, const uint8_t* mask, int32_t step,
                 ditango_states_t* st, float* O, float* LSE, uint8_t* reused_out, void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(mask, P))) return rc;
  if (!O || !LSE) return fail(DITANGO_EINVAL, "O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  for (int i = 0; i < P * P; ++i) {
    if (st->tc[i] > step)
      return fail(DITANGO_EINVAL, "step=%d is earlier than pair %d's last computation step %d", step, i,
                  st->tc[i]);
    if (!mask[i] && st->tc[i] < 0)
      return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) is marked REUSE but was never computed", i / P, i % P);
  }
  if (!Q || !K || !V) return fail(DITANGO_EINVAL, "Q, K and V must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15u)
    return fail(DITANGO_EINVAL, "Q, K and V must be 16-byte aligned");
  // After the checks above only a launch error remains, reported as EHIP
  // before t_c changes.
  if ((rc = launch_fused_step(Q, K, V, mask, st, O, LSE, stream))) return rc;
  return ditango_state_cache_update(st, mask, step, reused_out);
}

int ditango_window_residual_merge(const ditango_states_t* st, const uint8_t* window, int32_t mode, float* R,
                                  float* O, float* LSE, void* stream) {
  int rc = check_states(st);
  if (rc) return rc;
  const int P = st->shape.P;
  if ((rc = check_mask(window, P))) return rc;
  if (mode != DITANGO_WR_FULL && mode != DITANGO_WR_WINDOW)
    return fail(DITANGO_EINVAL, "window-residual mode %d is neither FULL nor WINDOW", mode);
  if (!R || !O || !LSE) return fail(DITANGO_EINVAL, "R, O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(R) | reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "R, O and LSE must be 16-byte aligned");
  ditango::MergeParams m;
  std::memset(&m, 0, sizeof m);
  m.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  for (int q = 0; q < P; ++q) {
    for (int k = 0; k < P; ++k)
      if (window[q * P + k]) m.wlive[q] |= 1u << k;
    if (!m.wlive[q]) return fail(DITANGO_EINVAL, "query partition %d has an empty window", q);
    m.live[q] = mode == DITANGO_WR_FULL ? (P == 32 ? 0xffffffffu : (1u << P) - 1u) : m.wlive[q];
  }
  for (int q = 0; q < P; ++q)
    for (int k = 0; k < P; ++k)
      if (((m.live[q] >> k) & 1u) && st->tc[q * P + k] < 0)
        return fail(DITANGO_ENOCACHE, "pair (q=%d, k=%d) holds no state", q, k);
  const size_t slot_o = static_cast<size_t>(st->S) * st->shape.d;
  for (int k = 0; k < P; ++k) {
    m.in_O[k] = elem_offset(st->O, k * slot_o, st->shape);
    m.in_L[k] = st->LSE + static_cast<size_t>(k) * st->S;
  }
  m.in_hs = static_cast<int64_t>(P) * P;
  m.in_qs = P;
  m.out_hs = st->shape.N;
  m.out_qs = st->S;
  m.O = O;
  m.LSE = LSE;
  m.res = R;
  m.res_mode = mode == DITANGO_WR_FULL ? 1 : 2;
  m.n_in = P;
  m.H = st->shape.H;
  m.N = st->shape.N;
  m.P = P;
  m.S = st->S;
  m.d = st->shape.d;
  hipError_t e = ditango::launch_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t ditango_group_slots(int32_t P, int32_t g) { return group_slots(P, g); }

size_t ditango_gstates_slot_bytes(const ditango_shape_t* shape, size_t* o_bytes, size_t* lse_bytes) {
  int32_t S = 0;
  if (check_shape(shape, &S)) return 0;
  const size_t rows = static_cast<size_t>(shape->H) * shape->P * S;
  if (o_bytes) *o_bytes = rows * shape->d * out_elem_bytes(*shape);
  if (lse_bytes) *lse_bytes = rows * sizeof(float);
  ok();
  return rows * (shape->d * out_elem_bytes(*shape) + sizeof(float));
}

int ditango_gstates_init(ditango_gstates_t* st, const ditango_shape_t* shape, int32_t g, void* const* O,
                         float* const* LSE, int32_t* tc) {
  if (!st) return fail(DITANGO_EINVAL, "states is NULL");
  int32_t S = 0;
  int rc = check_shape(shape, &S);
  if (rc) return rc;
  const int n = group_slots(shape->P, g);
  if (!n) return fail(DITANGO_EINVAL, "group size g=%d invalid for P=%d (at most %d slots)", g, shape->P,
                      DITANGO_MAX_SLOTS);
  if (!tc) return fail(DITANGO_EINVAL, "tc is NULL");
  if ((rc = check_slot_buffers(O, LSE, n))) return rc;
  st->shape = *shape;
  st->S = S;
  st->g0 = st->g = g;
  for (int s = 0; s < DITANGO_MAX_SLOTS; ++s) {
    st->O[s] = s < n ? O[s] : nullptr;
    st->LSE[s] = s < n ? LSE[s] : nullptr;
  }
  st->tc = tc;
  for (int i = 0; i < shape->P * DITANGO_MAX_SLOTS; ++i) tc[i] = -1;
  return ok();
}

int ditango_group_attn_partial(const void* Q, const void* K, const void* V, const uint8_t* mask,
                               ditango_gstates_t* st, void* stream) {
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  const int P = st->shape.P, g = st->g;
  if ((rc = check_mask(mask, P))) return rc;
  if (!Q || !K || !V) return fail(DITANGO_EINVAL, "Q, K and V must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15u)
    return fail(DITANGO_EINVAL, "Q, K and V must be 16-byte aligned");
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s)
      if (slot_live(P, g, q, s) && !slot_fresh(mask, P, g, q, s) && gtc(st, q, s) < 0)
        return fail(DITANGO_ENOCACHE, "slot (q=%d, s=%d) is REUSE but was never computed", q, s);

  ditango::PartialParams p;
  std::memset(&p, 0, sizeof p);
  // Items with the longest key ranges first (whole groups before the local
  // pair and the group that lost q), so the longest blocks start first.
  std::vector<std::pair<int64_t, int>> items;
  for (int s = 0; s < ns; ++s)
    for (int q = 0; q < P; ++q)
      if (slot_live(P, g, q, s) && slot_fresh(mask, P, g, q, s))
        items.push_back({-slot_keys(st->shape.N, P, st->S, g, q, s), (q << 6) | s});
  if (items.empty()) return ok();
  std::stable_sort(items.begin(), items.end(),
                   [](const std::pair<int64_t, int>& x, const std::pair<int64_t, int>& y) { return x.first < y.first; });
  for (size_t i = 0; i < items.size(); ++i) p.pairs[i] = static_cast<uint16_t>(items[i].second);
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.H = st->shape.H;
  p.N = st->shape.N;
  p.P = P;
  p.S = st->S;
  p.d = st->shape.d;
  p.scale_log2 = st->shape.scale * 1.4426950408889634f;
  p.n_pairs = static_cast<int32_t>(items.size());
  p.grouped = 1;
  p.g = g;
  p.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  for (int s = 0; s < ns; ++s) {
    p.gO[s] = st->O[s];
    p.gLSE[s] = st->LSE[s];
  }
  const int rows = ditango::partial_rows_per_block(p.d, p.S);
  p.q_tiles = (p.S + rows - 1) / rows;
  const int64_t blocks = static_cast<int64_t>(p.H) * p.n_pairs * p.q_tiles;
  if (blocks > 0x7fffffff) return fail(DITANGO_EINVAL, "grid of %lld blocks is too large", (long long)blocks);
  p.n_blocks = static_cast<int32_t>(blocks);
  hipError_t e = ditango::launch_partial(p, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "partial kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_group_attn_partial_merge(const void* Q, const void* K, const void* V, const uint8_t* mask,
                                     ditango_gstates_t* st, float* O, float* LSE, void* stream) {
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  const int P = st->shape.P, g = st->g;
  if ((rc = check_mask(mask, P))) return rc;
  if (!Q || !K || !V) return fail(DITANGO_EINVAL, "Q, K and V must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15u)
    return fail(DITANGO_EINVAL, "Q, K and V must be 16-byte aligned");
  if (!O || !LSE) return fail(DITANGO_EINVAL, "O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s)
      if (slot_live(P, g, q, s) && !slot_fresh(mask, P, g, q, s) && gtc(st, q, s) < 0)
        return fail(DITANGO_ENOCACHE, "slot (q=%d, s=%d) is REUSE but was never computed", q, s);

  ditango::GroupStepParams p;
  std::memset(&p, 0, sizeof p);
  for (int q = 0; q < P; ++q) {
    int nc = 0, nl = 0;
    for (int s = 0; s < ns; ++s) {
      if (!slot_live(P, g, q, s)) continue;
      p.lslot[q][nl++] = static_cast<uint8_t>(s);
      if (slot_fresh(mask, P, g, q, s)) p.cslot[q][nc++] = static_cast<uint8_t>(s);
    }
    p.nc[q] = static_cast<uint8_t>(nc);
    p.nl[q] = static_cast<uint8_t>(nl);
  }
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  for (int s = 0; s < ns; ++s) {
    p.gO[s] = st->O[s];
    p.gLSE[s] = st->LSE[s];
  }
  p.Oout = O;
  p.LSEout = LSE;
  p.H = st->shape.H;
  p.N = st->shape.N;
  p.P = P;
  p.S = st->S;
  p.d = st->shape.d;
  p.g = g;
  p.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  p.scale_log2 = st->shape.scale * 1.4426950408889634f;
  const int rows = ditango::partial_rows_per_block(p.d, p.S);
  p.q_tiles = (p.S + rows - 1) / rows;
  const int64_t blocks = static_cast<int64_t>(p.H) * P * p.q_tiles;
  if (blocks > 0x7fffffff) return fail(DITANGO_EINVAL, "grid of %lld blocks is too large", (long long)blocks);
  p.n_blocks = static_cast<int32_t>(blocks);
  hipError_t e = ditango::launch_group_step(p, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "group step kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_group_cache_update(ditango_gstates_t* st, const uint8_t* mask, int32_t step, uint8_t* computed_out) {
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  const int P = st->shape.P, g = st->g;
  if ((rc = check_mask(mask, P))) return rc;
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s) {
      if (!slot_live(P, g, q, s)) continue;
      if (gtc(st, q, s) > step)
        return fail(DITANGO_EINVAL, "step=%d is earlier than slot (q=%d, s=%d)'s last computation step %d", step,
                    q, s, gtc(st, q, s));
      if (!slot_fresh(mask, P, g, q, s) && gtc(st, q, s) < 0)
        return fail(DITANGO_EINVAL, "slot (q=%d, s=%d) reused but never computed", q, s);
    }
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s) {
      const bool c = slot_live(P, g, q, s) && slot_fresh(mask, P, g, q, s);
      if (c) gtc(st, q, s) = step;
      if (computed_out) computed_out[q * ns + s] = c ? 1 : 0;
    }
  return ok();
}

int ditango_group_merge(const ditango_gstates_t* st, float* O, float* LSE, void* stream) {
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  if (!O || !LSE) return fail(DITANGO_EINVAL, "O and LSE must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(O) | reinterpret_cast<uintptr_t>(LSE)) & 15u)
    return fail(DITANGO_EINVAL, "O and LSE must be 16-byte aligned");
  const int P = st->shape.P, g = st->g;
  ditango::MergeParams m;
  std::memset(&m, 0, sizeof m);
  m.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s)
      if (slot_live(P, g, q, s)) {
        if (gtc(st, q, s) < 0) return fail(DITANGO_ENOCACHE, "slot (q=%d, s=%d) holds no state", q, s);
        m.live[q] |= 1u << s;
      }
  for (int s = 0; s < ns; ++s) {
    m.in_O[s] = st->O[s];
    m.in_L[s] = st->LSE[s];
  }
  m.out_hs = st->shape.N;
  m.out_qs = st->S;
  m.O = O;
  m.LSE = LSE;
  hipError_t e = launch_group_merge(m, st, ns, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_group_compose(ditango_gstates_t* st, int32_t k, void* stream) {
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  if (k < 2) return fail(DITANGO_EINVAL, "merge factor k=%d must be >= 2", k);
  const int P = st->shape.P, g = st->g;
  if (static_cast<int64_t>(g) * k > DITANGO_MAX_P * 2)
    return fail(DITANGO_EINVAL, "group size %d * %d is beyond any partition count", g, k);
  const int g_new = g * k;
  const int m_old = ns - 1, m_new = group_slots(P, g_new) - 1;
  for (int q = 0; q < P; ++q)
    for (int s = 0; s < ns; ++s)
      if (slot_live(P, g, q, s) && gtc(st, q, s) < 0)
        return fail(DITANGO_ENOCACHE, "slot (q=%d, s=%d) holds no state to merge", q, s);
  std::vector<int> tc_new(static_cast<size_t>(P) * m_new, -1);
  // New group i is written over slot 1 + i after every earlier launch has
  // read that slot (stream order); group 0 reads and writes slot 1 element
  // by element in the same thread.
  for (int i = 0; i < m_new; ++i) {
    const int j0 = k * i, j1 = std::min(k * i + k, m_old);
    ditango::MergeParams m;
    std::memset(&m, 0, sizeof m);
    m.state_bf16 = st->shape.state_dtype == DITANGO_STATE_BF16;
    bool any = false;
    for (int j = j0; j < j1; ++j) {
      m.in_O[j - j0] = st->O[1 + j];
      m.in_L[j - j0] = st->LSE[1 + j];
    }
    for (int q = 0; q < P; ++q) {
      int t = -1;
      for (int j = j0; j < j1; ++j)
        if (slot_live(P, g, q, 1 + j)) {
          m.live[q] |= 1u << (j - j0);
          t = t < 0 ? gtc(st, q, 1 + j) : std::min(t, gtc(st, q, 1 + j));
        }
      tc_new[static_cast<size_t>(q) * m_new + i] = t;
      any = any || m.live[q];
    }
    if (!any) continue;
    m.out_hs = static_cast<int64_t>(P) * st->S;
    m.out_qs = st->S;
    m.Os = st->O[1 + i];
    m.LSE = st->LSE[1 + i];
    hipError_t e = launch_group_merge(m, st, j1 - j0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DITANGO_EHIP, "group merge kernel launch: %s", hipGetErrorString(e));
  }
  for (int q = 0; q < P; ++q)
    for (int s = 1; s < DITANGO_MAX_SLOTS; ++s)
      gtc(st, q, s) = s <= m_new ? tc_new[static_cast<size_t>(q) * m_new + s - 1] : -1;
  for (int s = 1 + m_new; s < DITANGO_MAX_SLOTS; ++s) {
    st->O[s] = nullptr;
    st->LSE[s] = nullptr;
  }
  st->g = g_new;
  return ok();
}

int ditango_group_fit(ditango_gstates_t* st, size_t budget_bytes, int32_t k, void* stream, int32_t* merges_out) {
  if (merges_out) *merges_out = 0;
  int ns = 0;
  int rc = check_gstates(st, &ns);
  if (rc) return rc;
  if (k < 2) return fail(DITANGO_EINVAL, "merge factor k=%d must be >= 2", k);
  const size_t slot_bytes = ditango_gstates_slot_bytes(&st->shape, nullptr, nullptr);
  const int P = st->shape.P;
  // Merges needed: group sizes g, k g, k^2 g, ... until the slot memory fits.
  // The coarsest grouping (one group of all P partitions) has 2 slots.
  int n = 0;
  for (int64_t g = st->g;; g *= k, ++n) {
    const int64_t slots = 1 + (P + g - 1) / g;
    if (static_cast<size_t>(slots) * slot_bytes <= budget_bytes) break;
    if (g >= P)
      return fail(DITANGO_EINVAL, "the state cache needs %zu bytes at least (2 slots of %zu), above the budget of %zu",
                  2 * slot_bytes, slot_bytes, budget_bytes);
  }
  for (int i = 0; i < n; ++i) {
    if ((rc = ditango_group_compose(st, k, stream))) return rc;
    if (merges_out) *merges_out = i + 1;
  }
  return ok();
}

int ditango_group_reset(ditango_gstates_t* st, void* const* O, float* const* LSE) {
  if (!st) return fail(DITANGO_EINVAL, "states is NULL");
  int32_t S = 0;
  int rc = check_shape(&st->shape, &S);
  if (rc) return rc;
  const int n = group_slots(st->shape.P, st->g0);
  if (!n || !st->tc) return fail(DITANGO_EINVAL, "states were not initialised");
  if ((rc = check_slot_buffers(O, LSE, n))) return rc;
  for (int s = 0; s < DITANGO_MAX_SLOTS; ++s) {
    st->O[s] = s < n ? O[s] : nullptr;
    st->LSE[s] = s < n ? LSE[s] : nullptr;
  }
  st->g = st->g0;
  for (int i = 0; i < st->shape.P * DITANGO_MAX_SLOTS; ++i) st->tc[i] = -1;
  return ok();
}

int ditango_group_mask_build(int32_t P, int32_t g, int32_t n, uint8_t* mask_out) {
  if (!mask_out) return fail(DITANGO_EINVAL, "mask_out is NULL");
  if (P < 1 || P > DITANGO_MAX_P) return fail(DITANGO_EINVAL, "P=%d outside 1..%d", P, DITANGO_MAX_P);
  if (g < 1 || n < 0) return fail(DITANGO_EINVAL, "group size g=%d must be >= 1 and n=%d >= 0", g, n);
  std::memset(mask_out, 0, static_cast<size_t>(P) * P);
  const int m = (P + g - 1) / g;
  std::vector<std::pair<int, int>> cand;   // (distance, group)
  for (int q = 0; q < P; ++q) {
    mask_out[q * P + q] = 1;
    cand.clear();
    for (int j = 0; j < m; ++j) {
      int dist = -1;
      for (int k = j * g; k < std::min((j + 1) * g, P); ++k)
        if (k != q && (dist < 0 || std::abs(q - k) < dist)) dist = std::abs(q - k);
      if (dist >= 0) cand.push_back({dist, j});
    }
    std::sort(cand.begin(), cand.end());
    for (int i = 0; i < std::min<int>(n, static_cast<int>(cand.size())); ++i) {
      const int j = cand[i].second;
      for (int k = j * g; k < std::min((j + 1) * g, P); ++k) mask_out[q * P + k] = 1;
    }
  }
  return ok();
}

int ditango_mask_build(int32_t policy, int32_t P, int32_t n, uint64_t seed, int32_t step, uint8_t* mask_out) {
  if (!mask_out) return fail(DITANGO_EINVAL, "mask_out is NULL");
  if (P < 1 || P > DITANGO_MAX_P) return fail(DITANGO_EINVAL, "P=%d outside 1..%d", P, DITANGO_MAX_P);
  if (step < 0) return fail(DITANGO_EINVAL, "step=%d must be >= 0", step);
  if (policy < DITANGO_MASK_ALL || policy > DITANGO_MASK_RANDOM)
    return fail(DITANGO_EINVAL, "unknown mask policy %d", policy);
  // The count n matters from step 1 on (step 0 is the all-fresh anchor).
  if (step > 0) {
    if (policy == DITANGO_MASK_RADIUS && n < 0) return fail(DITANGO_EINVAL, "radius n=%d must be >= 0", n);
    if ((policy == DITANGO_MASK_NEAREST || policy == DITANGO_MASK_RANDOM) && (n < 1 || n > P))
      return fail(DITANGO_EINVAL, "%s n=%d outside 1..P", policy == DITANGO_MASK_NEAREST ? "nearest" : "random", n);
  }
  // Step 0 is an anchor step: every pair computes.
  const int pol = step == 0 ? DITANGO_MASK_ALL : policy;
  std::memset(mask_out, pol == DITANGO_MASK_ALL ? 1 : 0, static_cast<size_t>(P) * P);
  if (pol == DITANGO_MASK_RADIUS) {
    for (int q = 0; q < P; ++q)
      for (int k = 0; k < P; ++k) mask_out[q * P + k] = (q - k <= n && k - q <= n) ? 1 : 0;
  } else if (pol == DITANGO_MASK_NEAREST) {
    for (int q = 0; q < P; ++q) {
      // walk outward from q: distance 0, then for each distance the lower
      // index first (ties go to the lower k)
      int taken = 0;
      for (int dist = 0; taken < n; ++dist) {
        if (q - dist >= 0 && taken < n) { mask_out[q * P + (q - dist)] = 1; ++taken; }
        if (dist > 0 && q + dist < P && taken < n) { mask_out[q * P + (q + dist)] = 1; ++taken; }
      }
    }
  } else if (pol == DITANGO_MASK_RANDOM) {
    SplitMix64 rng{seed + static_cast<uint64_t>(step)};
    std::vector<int> c;
    for (int q = 0; q < P; ++q) {
      c.clear();
      for (int k = 0; k < P; ++k)
        if (k != q) c.push_back(k);
      for (int i = 0; i < n - 1; ++i) {
        const int j = i + static_cast<int>(rng.next() % static_cast<uint64_t>(P - 1 - i));
        const int t = c[i];
        c[i] = c[j];
        c[j] = t;
      }
      mask_out[q * P + q] = 1;
      for (int i = 0; i < n - 1; ++i) mask_out[q * P + c[i]] = 1;
    }
  }
  return ok();
}

}  // extern "C"
