// Fresh partial attention states on CDNA4 (gfx950), bf16 MFMA.
//
// For every fresh (query partition q, KV partition k) pair and head, one
// block computes the attention state (OUT, LSE) of a tile of query rows of
// partition q against all keys of partition k (DiTango page, attention-state
// section; the per-step partial attention of its ring-based composed
// attention) and stores it into the pair's cache slot.
//
// Formulation.  The scores are built transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 (A = a 32-key block of K from LDS, B = Q^T held in
// registers for the whole block).  In the accumulator layout each lane then
// owns one query (column) and 16 keys of it, so the row statistics are
// lane-local plus one exchange between the two half-waves, and the lane's
// softmax probabilities are already the B operand of the second product
// O^T += V^T P^T (keys permuted inside each group of 16, which the V^T
// operand reproduces).  V stays row-major in LDS and is read transposed with
// ds_read_b64_tr_b16.  O^T accumulates in fp32 and P is rounded to bf16 for
// the product.  Two row sums are kept: the fp32 sum of the unrounded
// probabilities gives LSE, and the sum of the rounded ones (v_dot2c_f32_bf16)
// normalises OUT, so the weights applied to V sum to one as used.
//
// Softmax runs in base 2 with the scale folded into one FMA.  The running
// max is only raised when a tile's max exceeds it by more than 8 (a factor of
// 256), which keeps every probability <= 256 and skips most rescales of the
// accumulator; the final division by the row sum makes the result exact.
//
// Block = 4 or 8 waves of 32 query rows each (128 or 256 rows), two waves
// per SIMD (<= 256 VGPRs each, no accumulator spills to AGPRs), so one wave's
// MFMAs overlap the other's softmax.  K/V tiles of 64 keys are
// double-buffered in LDS: the next tile's global loads are in flight while
// the current tile is multiplied.  The grid is the compacted list of
// fresh (head, pair, query tile) items: no block exists for a reused pair.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace ditango {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBc = 64;             // keys per K/V tile
constexpr float kRescaleSlack = 8.0f;  // base-2 headroom before the running max moves

template <int D>
struct Geometry {
  static constexpr int DK = (D + 15) / 16 * 16;   // Q.K contraction, 16 per MFMA
  static constexpr int DV = (D + 31) / 32 * 32;   // rows of O^T, 32 per MFMA tile
  static constexpr int kSteps = DK / 16;
  static constexpr int vTiles = DV / 32;
  static constexpr int chunks = D / 8;            // 16-byte chunks per global row
  // LDS row strides in bf16.  K rows are read 16 B per lane, 8 keys per LDS
  // pass: a stride of 4 (mod 8) dwords per row spreads them over all banks.
  // V rows are read 8 B per lane, 4 keys x 32 B per 16-lane group: a stride
  // of 8 or 24 (mod 32) dwords puts the four rows on disjoint banks.
  static constexpr int KS = DK + 8;
  static constexpr int VS = DV + 16;
};

typedef __attribute__((address_space(3))) bf16x4_v lds_bf16x4;

__device__ inline bf16x8 read_v_operand(const __bf16* p0, const __bf16* p1) {
  bf16x4_v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  bf16x4_v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  u32x4 w = {ua.x, ua.y, ub.x, ub.y};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

template <int D, int WAVES>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES), amdgpu_waves_per_eu(2, 2)))
void partial_kernel(const PartialParams p) {
  using G = Geometry<D>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int BR = 32 * WAVES;                   // query rows per block
  constexpr int kLoads = (kBc * G::chunks + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kBc * G::KS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kBc * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;   // half-wave
  const int l32 = lane & 31;

  // Blocks are dealt round-robin to the 8 XCDs; remap so each XCD runs a
  // contiguous range of work items (items sharing K/V then share its L2).
  const int nb = p.n_blocks;
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int per = nb >> 3, rem = nb & 7;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + (b >> 3);

  const int qt = item % p.q_tiles;
  const int rest = item / p.q_tiles;
  const int pi = rest % p.n_pairs;
  const int h = rest / p.n_pairs;
  const int pair = p.pairs[pi];
  const int qp = pair / p.P, kp = pair - qp * p.P;
  const int q0 = qp * p.S, k0 = kp * p.S;
  const int len_q = min(p.S, p.N - q0);
  const int len_k = min(p.S, p.N - k0);
  const size_t head = static_cast<size_t>(h) * p.N * D;
  const __bf16* Qh = p.Q + head + static_cast<size_t>(q0) * D;
  const __bf16* Kh = p.K + head + static_cast<size_t>(k0) * D;
  const __bf16* Vh = p.V + head + static_cast<size_t>(k0) * D;
  const float sl2 = p.scale_log2;
  const int my_row = qt * BR + wave * 32 + l32;   // this lane's query row in the partition

  // Q^T operand: lane holds 8 consecutive dims of its query per k-step.
  bf16x8 qf[G::kSteps];
  {
    const __bf16* qrow = Qh + static_cast<size_t>(min(my_row, len_q - 1)) * D;
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      const int dim = s * 16 + hw * 8;
      if (dim < D) {
        qf[s] = *reinterpret_cast<const bf16x8*>(qrow + dim);
      } else {
        qf[s] = bf16x8{};
      }
    }
  }

  // K columns beyond d (d = 72 pads the contraction to 80) must read as zero.
  if constexpr (G::DK > D) {
    for (int i = tid; i < 2 * kBc; i += kThreads)
      *reinterpret_cast<u32x4*>(&k_lds[i / kBc][(i % kBc) * G::KS + D]) = u32x4{0u, 0u, 0u, 0u};
  }

  const int n_tiles = (len_k + kBc - 1) / kBc;
  u32x4 kreg[kLoads], vreg[kLoads];

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kBc * G::chunks) {
        const int key = c / G::chunks, ch = c % G::chunks;
        const int krow = min(kt * kBc + key, len_k - 1);
        kreg[i] = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(krow) * D + ch * 8);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vh + static_cast<size_t>(krow) * D + ch * 8);
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kBc * G::chunks) {
        const int key = c / G::chunks, ch = c % G::chunks;
        *reinterpret_cast<u32x4*>(&k_lds[buf][key * G::KS + ch * 8]) = kreg[i];
        *reinterpret_cast<u32x4*>(&v_lds[buf][key * G::VS + ch * 8]) = vreg[i];
      }
    }
  };

  f32x16 oacc[G::vTiles];
#pragma unroll
  for (int v = 0; v < G::vTiles; ++v) oacc[v] = f32x16{};
  float m_run = -__builtin_inff();   // running max (base-2 units)
  float l_run = 0.0f;                // exact sum of probabilities
  float lr_run = 0.0f;               // sum of bf16-rounded probabilities
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ds_read_b64_tr_b16 addressing for the V^T operand: in each 16-lane group
  // lane 4r+c supplies key row r, dims 4c..4c+3 of the group's 16 dims, and
  // receives dim (lane % 16) of the four rows.
  const int tr_r = (lane & 15) >> 2;
  const int tr_dim = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < n_tiles;
    if (more) gload(kt + 1);
    const __bf16* kl = k_lds[buf];
    const __bf16* vl = v_lds[buf];

    // S^T = K Q^T for two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[(kb * 32 + l32) * G::KS + s * 16 + hw * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }

    // Keys past the end of a ragged partition get score -inf.
    const int lim = len_k - kt * kBc;
    if (lim < kBc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + hw * 4 + (i & 3);
          if (key >= lim) sacc[kb][i] = -__builtin_inff();
        }
    }

    // Tile max (this lane's 32 keys, then the other half-wave's 32).
    float mx = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[0][i], sacc[0][i + 1]));
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[1][i], sacc[1][i + 1]));
    mx = fmaxf(mx, xor32(mx));
    const float m_new = mx * sl2;
    // Raise the running max only when the tile exceeds it by the slack.
    const bool need = m_new > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = need ? m_new : m_run;
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int v = 0; v < G::vTiles; ++v) oacc[v] *= alpha;
    }

    // P = exp2(s * scale * log2e - m), rounded to bf16 for the product.
    // pb[u] is the B operand of key step u (16 keys).
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * half + j], sl2, -m_run));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * half + j + 1], sl2, -m_run));
          bf16x2 pr;
          pr[0] = (__bf16)e0;
          pr[1] = (__bf16)e1;
          pb[2 * kb + half][j] = pr[0];
          pb[2 * kb + half][j + 1] = pr[1];
          l_run += e0 + e1;
          lr_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lr_run, false);
        }

    // O^T += V^T P^T.
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const __bf16* p0 = &vl[(u * 16 + 4 * hw + tr_r) * G::VS + v * 32 + tr_dim];
        const __bf16* p1 = &vl[(u * 16 + 8 + 4 * hw + tr_r) * G::VS + v * 32 + tr_dim];
        oacc[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v_operand(p0, p1), pb[u], oacc[v], 0, 0, 0);
      }
    }

    if (more) swrite(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: OUT = O / l_rounded, LSE = ln2 * (m + log2 l), into the slot.
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.0f / (lr_run + xor32(lr_run));
  if (my_row < len_q) {
    const size_t slot = static_cast<size_t>(h) * p.P * p.P + pair;
    float* orow = p.O + (slot * p.S + my_row) * D;
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = v * 32 + 8 * g + 4 * hw;
        if (dim < D) {
          const f32x4 o = {oacc[v][4 * g] * inv, oacc[v][4 * g + 1] * inv, oacc[v][4 * g + 2] * inv,
                           oacc[v][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + dim) = o;
        }
      }
    if (hw == 0) p.LSE[slot * p.S + my_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int WAVES>
hipError_t launch(PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((partial_kernel<D, WAVES>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int partial_rows_per_block(int d, int S) {
  (void)d;
  // 256 rows per block unless 128-row blocks waste clearly less of a ragged
  // partition (e.g. S = 549: 3 x 256 rows hold 71% useful work, 5 x 128 hold 86%).
  const long waste256 = (S + 255) / 256 * 256L - S;
  const long waste128 = (S + 127) / 128 * 128L - S;
  return (waste128 * 10 + S < waste256 * 10) ? 128 : 256;
}

hipError_t launch_partial(PartialParams& p, int rows, hipStream_t stream) {
  const bool wide = rows == 256;
  switch (p.d) {
    case 64: return wide ? launch<64, 8>(p, stream) : launch<64, 4>(p, stream);
    case 72: return wide ? launch<72, 8>(p, stream) : launch<72, 4>(p, stream);
    case 128: return wide ? launch<128, 8>(p, stream) : launch<128, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
