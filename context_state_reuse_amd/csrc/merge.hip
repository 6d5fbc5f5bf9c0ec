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
// HBM-bound: per row and head it reads n states of d OUT values (fp32, or
// bf16 when the cache keeps them so) and one fp32 LSE each, and writes d
// fp32 values (a group slot: in the states' format) and an LSE.  A block
// owns R consecutive rows of one query partition of one head.
//   1. one lane per (row, state) loads LSE_k, the row's lanes reduce max and
//      sum with cross-lane shuffles, and the normalised weights go to LDS;
//   2. for every state k the block streams the R*d contiguous OUT values of
//      its rows in 16-byte chunks -- all states' loads are issued before the
//      first is used -- and accumulates w_k * OUT_k in fp32 registers
//      (bf16 -> fp32 is exact);
//   3. the R*d outputs are written contiguously.
// R = 256 / PMAX rows (times the passes of weight_passes) keep up to 32
// independent loads in flight per thread; the template chosen for a state
// count is in launch_d.  Each output element is written by the thread that read that
// element of every input, after reading it, so an output may overwrite the
// rows of one of its inputs (the in-place group merge).
//
// RES = 1 (full step of window attention with residual sharing, DiTFastAttn
// page): a second weight set renormalised over the window states gives the
// window composition in the same pass, and res = OUT - OUT_window is
// written beside OUT.  RES = 2 (window step): OUT of the window states plus
// the cached res.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace ditango {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__device__ inline u32x4 load_chunk(const void* p) {
  if constexpr (DITANGO_MERGE_NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ inline void store_stream(float* p, f32x4 v) {
  if constexpr (DITANGO_MERGE_NT) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
__device__ inline void store_chunk(void* p, u32x4 v) {
  if constexpr (DITANGO_MERGE_NT) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  } else {
    *reinterpret_cast<u32x4*>(p) = v;
  }
}

// The 8 bf16 values of a 16-byte chunk as fp32 (exact: the pattern in the
// high half of a word), and back (round to nearest even).
__device__ inline void unpack8(u32x4 u, f32x4& lo, f32x4& hi) {
  lo = f32x4{__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
             __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u)};
  hi = f32x4{__builtin_bit_cast(float, u.z << 16), __builtin_bit_cast(float, u.z & 0xffff0000u),
             __builtin_bit_cast(float, u.w << 16), __builtin_bit_cast(float, u.w & 0xffff0000u)};
}
__device__ inline u32x4 pack8(f32x4 lo, f32x4 hi) {
  const bf16x2 a = {(__bf16)lo.x, (__bf16)lo.y}, b = {(__bf16)lo.z, (__bf16)lo.w};
  const bf16x2 c = {(__bf16)hi.x, (__bf16)hi.y}, d = {(__bf16)hi.z, (__bf16)hi.w};
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// COMPACT: lanes walk the compacted live list idx[q][0 .. cnt[q]) (one more
// indirection per state) instead of state indices 0 .. n_in with liveness
// bits; chosen only when it lets a narrower template (fewer lanes per row)
// serve the launch.
// Rows per block: the weight pass covers kThreads / PMAX rows (one lane per
// (row, state)); it runs RM times so that a state's rows give every thread
// at least one 16-byte chunk to stream (bf16 rows of d = 64 are only 8
// chunks).
template <int D, int PMAX, typename ST>
constexpr int weight_passes() {
  constexpr int R1 = kThreads / PMAX, CPR = D / (16 / static_cast<int>(sizeof(ST)));
  return R1 * CPR >= kThreads ? 1 : kThreads / (R1 * CPR);
}
template <int D, int PMAX, typename ST>
constexpr int rows_per_block() { return kThreads / PMAX * weight_passes<D, PMAX, ST>(); }

template <int D, int PMAX, int RES, bool COMPACT, typename ST>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p, int row_tiles) {
  constexpr bool kBF = std::is_same<ST, __bf16>::value;
  constexpr int EPC = 16 / sizeof(ST);                // OUT elements per 16-byte chunk
  constexpr int NQ = EPC / 4;                         // fp32 quads per chunk
  constexpr int R1 = kThreads / PMAX;                 // rows per weight pass
  constexpr int RM = weight_passes<D, PMAX, ST>();
  constexpr int R = rows_per_block<D, PMAX, ST>();    // rows per block
  constexpr int CPR = D / EPC;                        // 16-byte chunks per row
  constexpr int CH = R * CPR;                         // chunks per state block
  constexpr int PER = (CH + kThreads - 1) / kThreads; // chunks per thread
  __shared__ float w_lds[R][PMAX];
  __shared__ float wr_lds[RES == 1 ? R : 1][PMAX];     // weights of res = OUT - OUT_window

  const int tid = threadIdx.x;
  const int rt = blockIdx.x % row_tiles;
  const int hq = blockIdx.x / row_tiles;              // h * P + q
  const int q = hq % p.P;
  const int h = hq / p.P;
  const int cnt = COMPACT ? p.cnt[q] : p.n_in;        // lanes in use per row
  const uint32_t live = COMPACT ? 0xffffffffu : p.live[q];
  const int len_q = min(p.S, p.N - q * p.S);
  const int i0 = rt * R;
  const int rows = min(R, len_q - i0);
  if (cnt == 0 || (live & (cnt >= 32 ? 0xffffffffu : (1u << cnt) - 1u)) == 0 || rows <= 0) return;   // block-uniform
  auto state = [&](int k) __attribute__((always_inline)) { return COMPACT ? static_cast<int>(p.idx[q][k]) : k; };
  const int64_t in_row0 = (h * p.in_hs + q * p.in_qs) * p.S + i0;
  const int64_t out_row0 = h * p.out_hs + q * p.out_qs + i0;

  // 1. weights
#pragma unroll
  for (int pass = 0; pass < RM; ++pass) {
    const int r = pass * R1 + tid / PMAX, k = tid % PMAX;
    const bool lv = k < cnt && ((live >> k) & 1u) && r < rows;
    // Lanes without a state take -FLT_MAX and weight 0, so no infinity or
    // NaN arises even in rows past the end of the block's rows.
    float l = lv ? p.in_L[state(k)][in_row0 + r] : -3.4028234663852886e38f;
    float m = l;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float e = lv ? __builtin_amdgcn_exp2f((l - m) * 1.4426950408889634f) : 0.0f;
    float z = e;
#pragma unroll
    for (int off = 1; off < PMAX; off <<= 1) z += __shfl_xor(z, off);
    w_lds[r][k] = e / (z > 0.0f ? z : 1.0f);
    if constexpr (RES == 1) {
      const bool win = lv && (((COMPACT ? p.wpos[q] : p.wlive[q]) >> k) & 1u);
      float mw = win ? l : -3.4028234663852886e38f;
#pragma unroll
      for (int off = 1; off < PMAX; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
      const float ew = win ? __builtin_amdgcn_exp2f((l - mw) * 1.4426950408889634f) : 0.0f;
      float zw = ew;
#pragma unroll
      for (int off = 1; off < PMAX; off <<= 1) zw += __shfl_xor(zw, off);
      wr_lds[r][k] = e / (z > 0.0f ? z : 1.0f) - ew / (zw > 0.0f ? zw : 1.0f);
    }
    if (k == 0 && r < rows) p.LSE[out_row0 + r] = m + __builtin_amdgcn_logf(z) * 0.69314718055994531f;
  }
  __syncthreads();

  // 2. stream the states
  const int valid = rows * CPR;
  f32x4 acc[PER][NQ];
  f32x4 racc[RES == 1 ? PER : 1][NQ];
  u32x4 o[PMAX][PER];
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int u = 0; u < NQ; ++u) acc[j][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (RES == 1) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
      for (int u = 0; u < NQ; ++u) racc[j][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < cnt && ((live >> k) & 1u)) {
      const ST* src = static_cast<const ST*>(p.in_O[state(k)]) + in_row0 * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) o[k][j] = load_chunk(src + EPC * c);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    if (k < cnt && ((live >> k) & 1u)) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * kThreads;
        if (c < valid) {
          f32x4 x[NQ];
          if constexpr (kBF) {
            unpack8(o[k][j], x[0], x[NQ - 1]);
          } else {
            x[0] = __builtin_bit_cast(f32x4, o[k][j]);
          }
          const float wt = w_lds[c / CPR][k];
#pragma unroll
          for (int u = 0; u < NQ; ++u) acc[j][u] += wt * x[u];
          if constexpr (RES == 1) {
            const float wr = wr_lds[c / CPR][k];
#pragma unroll
            for (int u = 0; u < NQ; ++u) racc[j][u] += wr * x[u];
          }
        }
      }
    }
  }

  // 3. write
  float* rdst = p.res + out_row0 * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = tid + j * kThreads;
    if (c < valid) {
      if constexpr (RES == 2) {
#pragma unroll
        for (int u = 0; u < NQ; ++u) acc[j][u] += load_stream(rdst + EPC * c + 4 * u);
      }
      if (p.Os) {                                      // block-uniform: a group slot, in the states' format
        ST* dst = static_cast<ST*>(p.Os) + out_row0 * D + EPC * c;
        if constexpr (kBF) {
          store_chunk(dst, pack8(acc[j][0], acc[j][NQ - 1]));
        } else {
          store_stream(reinterpret_cast<float*>(dst), acc[j][0]);
        }
      } else {
        float* dst = p.O + out_row0 * D;
#pragma unroll
        for (int u = 0; u < NQ; ++u) store_stream(dst + EPC * c + 4 * u, acc[j][u]);
      }
      if constexpr (RES == 1) {
#pragma unroll
        for (int u = 0; u < NQ; ++u) store_stream(rdst + EPC * c + 4 * u, racc[j][u]);
      }
    }
  }
}

template <int D, int PMAX, typename ST>
hipError_t launch_st(const MergeParams& p, bool compact, hipStream_t stream) {
  constexpr int R = rows_per_block<D, PMAX, ST>();
  const int row_tiles = (p.S + R - 1) / R;
  const int64_t blocks = static_cast<int64_t>(p.H) * p.P * row_tiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (p.res_mode == 1) {          // every state of a row takes part: never compacted
    hipLaunchKernelGGL((merge_kernel<D, PMAX, 1, false, ST>), grid, block, 0, stream, p, row_tiles);
  } else if (p.res_mode == 2) {
    if (compact) hipLaunchKernelGGL((merge_kernel<D, PMAX, 2, true, ST>), grid, block, 0, stream, p, row_tiles);
    else hipLaunchKernelGGL((merge_kernel<D, PMAX, 2, false, ST>), grid, block, 0, stream, p, row_tiles);
  } else if (p.res_mode == 0) {
    if (compact) hipLaunchKernelGGL((merge_kernel<D, PMAX, 0, true, ST>), grid, block, 0, stream, p, row_tiles);
    else hipLaunchKernelGGL((merge_kernel<D, PMAX, 0, false, ST>), grid, block, 0, stream, p, row_tiles);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int PMAX>
hipError_t launch(const MergeParams& p, bool compact, hipStream_t stream) {
  return p.state_bf16 ? launch_st<D, PMAX, __bf16>(p, compact, stream) : launch_st<D, PMAX, float>(p, compact, stream);
}

// State-count template per head dim, from a sweep on MI355X (row merges and
// group merges of 2 to 32 states): the instantiations that the compiler
// builds at 256 VGPRs -- d = 128 with 4 lanes per row, d = 64 with 2 --
// reach only 55-65% of the bandwidth of their neighbours, so those counts
// use the next template up.
template <int D>
int lanes_per_row(int n) {
  if (D == 128 && n <= 2) return 2;
  if (D == 64 && n <= 4) return 4;
  if (n <= 8) return 8;
  if (n <= 16) return 16;
  return 32;
}

template <int D>
hipError_t launch_d(const MergeParams& p, int most, hipStream_t stream) {
  const bool compact = lanes_per_row<D>(most) < lanes_per_row<D>(p.n_in);
  switch (lanes_per_row<D>(compact ? most : p.n_in)) {
    case 2:
      if constexpr (D == 128) return launch<D, 2>(p, compact, stream);
      break;
    case 4:
      if constexpr (D == 64) return launch<D, 4>(p, compact, stream);
      break;
    case 8: return launch<D, 8>(p, compact, stream);
    case 16: return launch<D, 16>(p, compact, stream);
    default: return launch<D, 32>(p, compact, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p_in, hipStream_t stream) {
  if (p_in.n_in < 1 || p_in.n_in > DITANGO_MAX_SLOTS || p_in.P > DITANGO_MAX_P) return hipErrorInvalidValue;
  MergeParams p = p_in;
  int most = 0;
  for (int q = 0; q < p.P; ++q) {
    int c = 0;
    uint32_t wp = 0;
    for (int k = 0; k < p.n_in; ++k)
      if ((p.live[q] >> k) & 1u) {
        if ((p.wlive[q] >> k) & 1u) wp |= 1u << c;
        p.idx[q][c++] = static_cast<uint8_t>(k);
      }
    p.cnt[q] = static_cast<uint8_t>(c);
    p.wpos[q] = wp;
    most = c > most ? c : most;
  }
  if (most == 0) return hipSuccess;                   // no state takes part anywhere
  switch (p.d) {
    case 64: return launch_d<64>(p, most, stream);
    case 72: return launch_d<72>(p, most, stream);
    case 128: return launch_d<128>(p, most, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
