// Composition of the states of every row (DiTango page, Eq. 4, the n-ary
// form of its associative and commutative state composition):
//   m = max_k LSE_k,  w_k = exp(LSE_k - m) / Z,  Z = sum_k exp(LSE_k - m)
//   OUT = sum_k w_k OUT_k,  LSE = m + log Z
// Instances: the row merge of the per-pair cache (the P pair states of a
// row, fresh ones written this step and reused ones from earlier steps
// alike), the row merge of the grouped cache (local slot plus group slots),
// and the in-place merge of groups (Dynamic Group State Compose), whose
// output is a group slot.  Where the states are and which take part come
// from tables in the launch parameters.
//
// HBM-bound: per row and head it reads n*(d+1) floats and writes d+1.
// A block owns R consecutive rows of one query partition of one head.
//   1. one lane per (row, state) loads LSE_k, the row's lanes reduce max and
//      sum with cross-lane shuffles, and the normalised weights go to LDS;
//   2. for every state k the block streams the R*d contiguous floats of its
//      rows with 16-byte loads -- all states' loads are issued before the
//      first is used, about 32 per thread -- and accumulates w_k * OUT_k in
//      registers;
//   3. the R*d outputs are written contiguously.
// R = 256 / PMAX keeps up to 32 independent loads in flight per thread; the
// template chosen for a state count is in launch_d.  Each output element is written by the thread that read that
// element of every input, after reading it, so an output may overwrite the
// rows of one of its inputs (the in-place group merge).

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
  constexpr int CH = R * D / 4;                       // float4 chunks per state block
  constexpr int PER = (CH + kThreads - 1) / kThreads; // chunks per thread
  __shared__ float w_lds[R][PMAX];

  const int tid = threadIdx.x;
  const int rt = blockIdx.x % row_tiles;
  const int hq = blockIdx.x / row_tiles;              // h * P + q
  const int q = hq % p.P;
  const int h = hq / p.P;
  const uint32_t live = p.live[q];
  const int len_q = min(p.S, p.N - q * p.S);
  const int i0 = rt * R;
  const int rows = min(R, len_q - i0);
  if (live == 0 || rows <= 0) return;                 // block-uniform
  const int64_t in_row0 = (h * p.in_hs + q * p.in_qs) * p.S + i0;
  const int64_t out_row0 = h * p.out_hs + q * p.out_qs + i0;

  // 1. weights
  {
    const int r = tid / PMAX, k = tid % PMAX;
    const bool lv = k < p.n_in && ((live >> k) & 1u) && r < rows;
    float l = lv ? p.in_L[k][in_row0 + r] : -__builtin_inff();
    float m = l;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float e = lv ? __builtin_amdgcn_exp2f((l - m) * 1.4426950408889634f) : 0.0f;
    float z = e;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) z += __shfl_xor(z, off);
    w_lds[r][k] = e / z;
    if (k == 0 && r < rows) p.LSE[out_row0 + r] = m + __builtin_amdgcn_logf(z) * 0.69314718055994531f;
  }
  __syncthreads();

  // 2. stream the states
  const int valid = rows * (D / 4);
  f32x4 acc[PER];
  f32x4 o[PMAX][PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.n_in && ((live >> k) & 1u)) {
      const float* src = p.in_O[k] + in_row0 * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) o[k][j] = load_stream(src + 4 * c);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < p.n_in && ((live >> k) & 1u)) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) acc[j] += w_lds[c / (D / 4)][k] * o[k][j];
      }
    }
  }

  // 3. write
  float* dst = p.O + out_row0 * D;
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

// State-count template per head dim, from a sweep on MI355X (row merges and
// group merges of 2 to 32 states): the instantiations that the compiler
// builds at 256 VGPRs -- d = 128 with 4 lanes per row, d = 64 with 2 --
// reach only 55-65% of the bandwidth of their neighbours, so those counts
// use the next template up.
template <int D>
hipError_t launch_d(const MergeParams& p, hipStream_t stream) {
  const int n = p.n_in;
  if constexpr (D == 128) {
    if (n <= 2) return launch<D, 2>(p, stream);
  } else if constexpr (D == 64) {
    if (n <= 4) return launch<D, 4>(p, stream);
  }
  if (n <= 8) return launch<D, 8>(p, stream);
  if (n <= 16) return launch<D, 16>(p, stream);
  return launch<D, 32>(p, stream);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  if (p.n_in < 1 || p.n_in > 32) return hipErrorInvalidValue;
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 72: return launch_d<72>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
