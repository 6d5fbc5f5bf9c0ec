// Per-pair statistics of the state cache for the anchor-guided planner
// (DiTango page, error-analysis and state-selection sections), and the
// drift of pair signatures between two signature tables:
//   W[h][q][k]   = mean over the rows r of query partition q of
//                  exp(LSE_qk[r] - LSE[r]) -- the normalised weight of
//                  partition k in the composed state, i.e. the share of q's
//                  attention mass on k's keys (the importance w of the
//                  error model);
//   SIG[h][q][k] = mean over q's rows of OUT_qk, for the selected pairs --
//                  the signature on which the planner measures how far a
//                  state has drifted.
// One block per (head, q, k) -- per selected pair only when W is not
// wanted -- of 1024 threads, so that a step's few blocks (one per head and
// local pair) keep enough loads in flight; every sum is taken in a fixed
// order (per-thread strided partial sums over four interleaved
// accumulators, then a fixed tree), so results do not vary from run to run.  Reads the LSE of every slot and the OUT of the
// selected ones: a few per cent of one merge.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace ditango {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;        // drift kernel
constexpr int kStatsThreads = 1024;  // stats kernel

template <int D, typename ST>
__global__ __launch_bounds__(kStatsThreads) void stats_kernel(const StatsParams p) {
  constexpr int C = D / 4;                  // chunks of 4 values per row (8 bytes of bf16)
  constexpr int RG = kStatsThreads / C;     // rows summed in parallel
  __shared__ f32x4 part[RG][C];
  __shared__ float wpart[kStatsThreads / 64];

  const int tid = threadIdx.x;
  const int n = p.W ? p.P * p.P : p.n_pairs;          // blocks per head
  const int pair = p.W ? static_cast<int>(blockIdx.x % n) : static_cast<int>(p.pairs[blockIdx.x % n]);
  const int h = blockIdx.x / n;
  const int q = pair / p.P, k = pair % p.P;
  const int len_q = min(p.S, p.N - q * p.S);
  const size_t slot = static_cast<size_t>(h) * p.P * p.P + pair;
  // importance (block-uniform branch)
  if (p.W) {
    const float* ls = p.LSE_slot + slot * p.S;
    const float* lm = p.LSE + static_cast<size_t>(h) * p.N + static_cast<size_t>(q) * p.S;
    float acc = 0.0f;
    for (int r = tid; r < len_q; r += kStatsThreads) acc += __expf(ls[r] - lm[r]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((tid & 63) == 0) wpart[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kStatsThreads / 64; ++i) s += wpart[i];
      p.W[slot] = s / static_cast<float>(len_q);
    }
  }

  // signature (block-uniform branch)
  if (!((p.sel[q] >> k) & 1u)) return;
  const ST* o = static_cast<const ST*>(p.O) + slot * p.S * D;
  const int rg = tid / C, c = tid % C;
  if (rg < RG) {
    // four independent accumulators: four loads in flight per thread
    // bf16 -> fp32 is exact: the pattern in the high half of a word
    auto row = [&](int r) {
      if constexpr (std::is_same<ST, __bf16>::value) {
        const u32x2 u = *reinterpret_cast<const u32x2*>(o + static_cast<size_t>(r) * D + 4 * c);
        return f32x4{__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
                     __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u)};
      } else {
        return *reinterpret_cast<const f32x4*>(o + static_cast<size_t>(r) * D + 4 * c);
      }
    };
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
    int r = rg;
    for (; r + 3 * RG < len_q; r += 4 * RG) {
      a0 += row(r);
      a1 += row(r + RG);
      a2 += row(r + 2 * RG);
      a3 += row(r + 3 * RG);
    }
    for (; r < len_q; r += RG) a0 += row(r);
    part[rg][c] = (a0 + a1) + (a2 + a3);
  }
  __syncthreads();
  if (tid < C) {
    f32x4 s = part[0][tid];
    for (int i = 1; i < RG; ++i) s += part[i][tid];
    const float inv = 1.0f / static_cast<float>(len_q);
    *reinterpret_cast<f32x4*>(p.SIG + slot * D + 4 * tid) = s * inv;
  }
}

// One block per listed pair: every thread sums its strided share of the
// pair's H*d elements, then a fixed tree.
__global__ __launch_bounds__(kThreads) void drift_kernel(const DriftParams p) {
  __shared__ float lnum[kThreads / 64], lden[kThreads / 64];
  const int tid = threadIdx.x;
  const int pair = p.pairs[blockIdx.x];
  const int n = p.H * p.d;
  float num = 0.0f, den = 0.0f;
  for (int i = tid; i < n; i += kThreads) {
    const int h = i / p.d, c = i - h * p.d;
    const size_t off = (static_cast<size_t>(h) * p.P * p.P + pair) * p.d + c;
    const float b = p.B[off], x = p.A[off] - b;
    num += x * x;
    den += b * b;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    num += __shfl_xor(num, off);
    den += __shfl_xor(den, off);
  }
  if ((tid & 63) == 0) {
    lnum[tid >> 6] = num;
    lden[tid >> 6] = den;
  }
  __syncthreads();
  if (tid == 0) {
    float sn = 0.0f, sd = 0.0f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      sn += lnum[i];
      sd += lden[i];
    }
    p.out[pair] = sd == 0.0f ? (sn == 0.0f ? 0.0f : __builtin_inff()) : __builtin_sqrtf(sn) / __builtin_sqrtf(sd);
  }
}

}  // namespace

hipError_t launch_drift(const DriftParams& p, hipStream_t stream) {
  if (p.n_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(drift_kernel, dim3(p.n_pairs), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(p.H) * (p.W ? p.P * p.P : p.n_pairs);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kStatsThreads);
  const bool bf = p.state_bf16 != 0;
  switch (p.d) {
    case 64:
      if (bf) hipLaunchKernelGGL((stats_kernel<64, __bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((stats_kernel<64, float>), grid, block, 0, stream, p);
      break;
    case 72:
      if (bf) hipLaunchKernelGGL((stats_kernel<72, __bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((stats_kernel<72, float>), grid, block, 0, stream, p);
      break;
    case 128:
      if (bf) hipLaunchKernelGGL((stats_kernel<128, __bf16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((stats_kernel<128, float>), grid, block, 0, stream, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ditango
