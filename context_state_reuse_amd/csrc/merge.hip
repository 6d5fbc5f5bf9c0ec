// Composition of the P pair states of every row (DiTango page, Eq. 4, the
// n-ary form of its associative and commutative state composition):
//   m = max_k LSE_k,  w_k = exp(LSE_k - m),  Z = sum_k w_k
//   OUT = sum_k w_k OUT_k / Z,  LSE = m + log Z
// The P slots of a row mix states written this step (fresh) and states
// written at earlier steps (reused); the merge does not distinguish them.
//
// HBM-bound: per row and head it reads P*(d+1) floats and writes d+1.
// Each thread owns 4 consecutive dims of one row, so a wave reads whole
// rows of each slot as contiguous 16-byte-per-lane runs; the row's LSE
// values are the same address for all its threads (one broadcast load).

#include <hip/hip_runtime.h>

#include "internal.h"

namespace ditango {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int D, int PMAX>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t total = static_cast<int64_t>(p.H) * p.N * TPR;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= total) return;
  const int ch = static_cast<int>(gid % TPR);
  const int64_t hr = gid / TPR;                 // h * N + r
  const int r = static_cast<int>(hr % p.N);
  const int h = static_cast<int>(hr / p.N);
  const int q = r / p.S;
  const int i = r - q * p.S;
  const size_t slot0 = (static_cast<size_t>(h) * p.P + q) * p.P;  // slot of pair (q, 0)
  const float* L = p.LSEs + slot0 * p.S + i;                         // + k * S
  const float* Ob = p.Os + (slot0 * p.S + i) * D + ch * 4;           // + k * S * D
  const size_t ostride = static_cast<size_t>(p.S) * D;

  float lse[PMAX];
  f32x4 o[PMAX];
  float m = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.P) {
      lse[k] = L[static_cast<size_t>(k) * p.S];
      o[k] = *reinterpret_cast<const f32x4*>(Ob + k * ostride);
      m = fmaxf(m, lse[k]);
    }
  }
  const float log2e = 1.4426950408889634f;
  float z = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.P) {
      const float w = __builtin_amdgcn_exp2f((lse[k] - m) * log2e);
      z += w;
      acc += w * o[k];
    }
  }
  const float inv = 1.0f / z;
  *reinterpret_cast<f32x4*>(p.O + hr * D + ch * 4) = acc * inv;
  if (ch == 0) p.LSE[hr] = m + __builtin_amdgcn_logf(z) * 0.69314718055994531f;
}

template <int D, int PMAX>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.H) * p.N * (D / 4);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_kernel<D, PMAX>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const MergeParams& p, hipStream_t stream) {
  if (p.P <= 4) return launch<D, 4>(p, stream);
  if (p.P <= 8) return launch<D, 8>(p, stream);
  if (p.P <= 16) return launch<D, 16>(p, stream);
  return launch<D, 32>(p, stream);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 72: return launch_d<72>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
