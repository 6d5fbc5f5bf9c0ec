// Host half of the C ABI: argument checks, the fresh-pair work list, the
// last-computation timestamps t_c, the selection-mask builders and errors.
//
// Method: "DiTango: Cost-Effective Parallel Diffusion Generation with
// Selective Attention State Reuse" -- state selection (COMPUTE/REUSE per
// unit, t_c = last computation step), anchor steps (all compute, t_c <- t),
// selective compute and reuse (Fig. 6).  The unit here is one
// (query partition, KV partition) pair.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
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

}  // namespace

extern "C" {

const char* ditango_last_error(void) { return g_err.c_str(); }

int32_t ditango_version(void) { return 1; }

size_t ditango_states_bytes(const ditango_shape_t* shape, size_t* o_bytes, size_t* lse_bytes) {
  int32_t S = 0;
  if (check_shape(shape, &S)) return 0;
  const size_t slots = static_cast<size_t>(shape->H) * shape->P * shape->P;
  const size_t ob = slots * S * shape->d * sizeof(float);
  const size_t lb = slots * S * sizeof(float);
  if (o_bytes) *o_bytes = ob;
  if (lse_bytes) *lse_bytes = lb;
  ok();
  return ob + lb;
}

int ditango_states_init(ditango_states_t* st, const ditango_shape_t* shape, float* O, float* LSE,
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
  ditango::MergeParams m;
  m.Os = st->O;
  m.LSEs = st->LSE;
  m.O = O;
  m.LSE = LSE;
  m.H = st->shape.H;
  m.N = st->shape.N;
  m.P = P;
  m.S = st->S;
  m.d = st->shape.d;
  hipError_t e = ditango::launch_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DITANGO_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int ditango_mask_build(int32_t policy, int32_t P, int32_t n, uint64_t seed, uint8_t* mask_out) {
  if (!mask_out) return fail(DITANGO_EINVAL, "mask_out is NULL");
  if (P < 1 || P > DITANGO_MAX_P) return fail(DITANGO_EINVAL, "P=%d outside 1..%d", P, DITANGO_MAX_P);
  std::memset(mask_out, 0, static_cast<size_t>(P) * P);
  switch (policy) {
    case DITANGO_MASK_ALL:
      std::memset(mask_out, 1, static_cast<size_t>(P) * P);
      return ok();
    case DITANGO_MASK_NONE:
      return ok();
    case DITANGO_MASK_RADIUS:
      if (n < 0) return fail(DITANGO_EINVAL, "radius n=%d must be >= 0", n);
      for (int q = 0; q < P; ++q)
        for (int k = 0; k < P; ++k) mask_out[q * P + k] = (q - k <= n && k - q <= n) ? 1 : 0;
      return ok();
    case DITANGO_MASK_NEAREST:
      if (n < 1 || n > P) return fail(DITANGO_EINVAL, "nearest n=%d outside 1..P", n);
      for (int q = 0; q < P; ++q) {
        // walk outward from q: distance 0, then for each distance the lower
        // index first (ties go to the lower k)
        int taken = 0;
        for (int dist = 0; taken < n; ++dist) {
          if (q - dist >= 0 && taken < n) { mask_out[q * P + (q - dist)] = 1; ++taken; }
          if (dist > 0 && q + dist < P && taken < n) { mask_out[q * P + (q + dist)] = 1; ++taken; }
        }
      }
      return ok();
    case DITANGO_MASK_RANDOM: {
      if (n < 1 || n > P) return fail(DITANGO_EINVAL, "random n=%d outside 1..P", n);
      SplitMix64 rng{seed};
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
      return ok();
    }
    default:
      return fail(DITANGO_EINVAL, "unknown mask policy %d", policy);
  }
}

}  // extern "C"
