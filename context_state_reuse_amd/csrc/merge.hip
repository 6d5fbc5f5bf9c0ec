// Composition of the P pair states of every row (DiTango page, Eq. 4, the
// n-ary form of its associative and commutative state composition):
//   m = max_k LSE_k,  w_k = exp(LSE_k - m) / Z,  Z = sum_k exp(LSE_k - m)
//   OUT = sum_k w_k OUT_k,  LSE = m + log Z
// The P slots of a row mix states written this step (fresh) and states
// written at earlier steps (reused); the merge does not distinguish them.
//
// HBM-bound: per row and head it reads P*(d+1) floats and writes d+1.
// A block owns R consecutive rows of one query partition of one head.
//   1. one lane per (row, slot) loads LSE_k, the row's lanes reduce max and
//      sum with cross-lane shuffles, and the normalised weights go to LDS;
//   2. for every slot k the block streams the R*d contiguous floats of rows
//      [i0, i0+R) of slot (q, k) with 16-byte loads -- all P slots' loads are
//      issued before the first is used, about 32 per thread -- and
//      accumulates w_k * OUT_k in registers;
//   3. the R*d outputs are written contiguously.
// R = 256 / PMAX keeps 32 independent loads in flight per thread at every P.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace ditango {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

#ifndef DITANGO_MERGE_NT
#define DITANGO_MERGE_NT 1
#endif

// Streaming access: every slot byte is read once and every output written
// once per step, so the non-temporal variants keep them from evicting
// reusable lines (selected by measurement).
__device__ inline f32x4 load_stream(const float* p) {
  if constexpr (DITANGO_MERGE_NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ inline void store_stream(float* p, f32x4 v) {
  if constexpr (DITANGO_MERGE_NT) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

template <int D, int PMAX>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p, int row_tiles) {
  constexpr int R = kThreads / PMAX;                  // rows per block
  constexpr int CH = R * D / 4;                       // float4 chunks per slot block
  constexpr int PER = (CH + kThreads - 1) / kThreads; // chunks per thread
  __shared__ float w_lds[R][PMAX];

  const int tid = threadIdx.x;
  const int rt = blockIdx.x % row_tiles;
  const int hq = blockIdx.x / row_tiles;              // h * P + q
  const int q = hq % p.P;
  const int h = hq / p.P;
  const int len_q = min(p.S, p.N - q * p.S);
  const int i0 = rt * R;
  const int rows = min(R, len_q - i0);
  const size_t slot0 = static_cast<size_t>(hq) * p.P;  // slot of pair (q, 0) of head h

  // 1. weights
  {
    const int r = tid / PMAX, k = tid % PMAX;
    const bool live = k < p.P && r < rows;
    float l = live ? p.LSEs[(slot0 + k) * p.S + i0 + r] : -__builtin_inff();
    float m = l;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float e = live ? __builtin_amdgcn_exp2f((l - m) * 1.4426950408889634f) : 0.0f;
    float z = e;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) z += __shfl_xor(z, off);
    w_lds[r][k] = e / z;
    if (k == 0 && r < rows)
      p.LSE[static_cast<size_t>(h) * p.N + q * p.S + i0 + r] =
          m + __builtin_amdgcn_logf(z) * 0.69314718055994531f;
  }
  __syncthreads();

  // 2. stream the slots
  const int valid = rows * (D / 4);
  f32x4 acc[PER];
  f32x4 o[PMAX][PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.P) {
      const float* src = p.Os + ((slot0 + k) * p.S + i0) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) o[k][j] = load_stream(src + 4 * c);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.P) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) acc[j] += w_lds[c / (D / 4)][k] * o[k][j];
      }
    }
  }

  // 3. write
  float* dst = p.O + (static_cast<size_t>(h) * p.N + q * p.S + i0) * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = tid + j * kThreads;
    if (c < valid) store_stream(dst + 4 * c, acc[j]);
  }
}

template <int D, int PMAX>
hipError_t launch(const MergeParams& p, hipStream_t stream) {
  constexpr int R = kThreads / PMAX;
  const int row_tiles = (p.S + R - 1) / R;
  const int64_t blocks = static_cast<int64_t>(p.H) * p.P * row_tiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_kernel<D, PMAX>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, p,
                     row_tiles);
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
