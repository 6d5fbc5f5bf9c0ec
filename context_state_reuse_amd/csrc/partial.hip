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
  // LDS row strides in bf16, chosen with a bank-conflict counter sweep on
  // gfx950 (64 banks of 4 bytes).  K rows are read 16 B per lane, 16 keys
  // per pass: a stride of an odd multiple of 4 dwords spreads them over all
  // banks.  V rows are read by ds_read_b64_tr_b16, 32 lanes per pass = 8 key
  // rows x 32 B: a stride of 16 or 48 (mod 64) dwords puts those rows on
  // disjoint banks (d=128: 80 dwords; d=72 and d=64: 48 dwords).
  static constexpr int KS = DK + 8;
  static constexpr int VS = DV == 128 ? 160 : 96;
  static_assert(DV <= VS, "V row must fit its stride");
  static_assert((KS / 2) % 8 == 4, "K stride must be an odd multiple of 4 dwords");
  static_assert((VS / 2) % 64 == 16 || (VS / 2) % 64 == 48, "V stride must be 16 or 48 mod 64 dwords");
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

// Per-wave pieces of the key-tile loop.  A wave owns 32 queries (one MFMA
// column tile); see the file comment for the operand layouts.
template <int D, int NQT>
struct WaveState {
  using G = Geometry<D>;
  bf16x8 qf[NQT][G::kSteps];      // Q^T operand, per 32-query column tile
  f32x16 oacc[G::vTiles][NQT];    // O^T accumulator
  f32x16 sacc[2][NQT];            // S^T of the current tile (two 32-key blocks)
  bf16x8 pb[4][NQT];              // P^T operand of the tile's four 16-key steps
  float m_run[NQT], l_run[NQT], lr_run[NQT];
};

// S^T = K Q^T for the 64 keys of one LDS tile into `sacc`; each K operand
// read from LDS feeds the NQT column tiles.
template <int D, int NQT>
__device__ inline void tile_scores(f32x16 (&sacc)[2][NQT], const WaveState<D, NQT>& w, const __bf16* kl, int l32,
                                   int hw) {
  using G = Geometry<D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < NQT; ++c) sacc[kb][c] = f32x16{};
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[(kb * 32 + l32) * G::KS + s * 16 + hw * 8]);
#pragma unroll
      for (int c = 0; c < NQT; ++c)
        sacc[kb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[c][s], sacc[kb][c], 0, 0, 0);
    }
  }
}

// Online softmax of the tile held in sacc, first half: tile max, lazily
// raised running max, rescale of the accumulators when it moves.
// MASK: keys at or past `lim` in this tile score -inf (ragged last tile).
template <bool MASK, int D, int NQT>
__device__ inline void tile_max(WaveState<D, NQT>& w, int lim, int hw, float sl2) {
  using G = Geometry<D>;
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NQT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + hw * 4 + (i & 3);
          if (key >= lim) w.sacc[kb][c][i] = -__builtin_inff();
        }
  }
  float m_new[NQT];
  bool need_any = false;
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    float mx = fmaxf(w.sacc[0][c][0], w.sacc[0][c][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(w.sacc[0][c][i], w.sacc[0][c][i + 1]));
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(w.sacc[1][c][i], w.sacc[1][c][i + 1]));
    mx = fmaxf(mx, xor32(mx));
    m_new[c] = mx * sl2;
    need_any |= m_new[c] > w.m_run[c] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
    // Rare after the first tile.  The empty volatile asm keeps the compiler
    // from if-converting this block into unconditional multiplies.
    asm volatile("; rescale" ::);
#pragma unroll
    for (int c = 0; c < NQT; ++c) {
      const bool need = m_new[c] > w.m_run[c] + kRescaleSlack;
      const float alpha = need ? __builtin_amdgcn_exp2f(w.m_run[c] - m_new[c]) : 1.0f;
      w.m_run[c] = need ? m_new[c] : w.m_run[c];
      w.l_run[c] *= alpha;
      w.lr_run[c] *= alpha;
#pragma unroll
      for (int v = 0; v < G::vTiles; ++v) w.oacc[v][c] *= alpha;
    }
  }
}

// Second half: probabilities exp2(s * scale * log2e - m) into pb (rounded
// to bf16 for the product) and the two row sums.
template <int D, int NQT>
__device__ inline void tile_exp(WaveState<D, NQT>& w, float sl2) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int c = 0; c < NQT; ++c)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t words[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(w.sacc[kb][c][8 * half + j], sl2, -w.m_run[c]));
          const float e1 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(w.sacc[kb][c][8 * half + j + 1], sl2, -w.m_run[c]));
          const bf16x2 pr = {(__bf16)e0, (__bf16)e1};   // one v_cvt_pk_bf16_f32
          words[j / 2] = __builtin_bit_cast(uint32_t, pr);
          w.l_run[c] += e0 + e1;
          w.lr_run[c] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, w.lr_run[c], false);
        }
        const u32x4 wv = {words[0], words[1], words[2], words[3]};
        w.pb[2 * kb + half][c] = __builtin_bit_cast(bf16x8, wv);
      }
}

template <bool MASK, int D, int NQT>
__device__ inline void tile_softmax(WaveState<D, NQT>& w, int lim, int hw, float sl2) {
  tile_max<MASK>(w, lim, hw, sl2);
  tile_exp(w, sl2);
}

// O^T += V^T P^T for the tile whose V sits in `vl`; each V operand read from
// LDS feeds the NQT column tiles.
template <int D, int NQT>
__device__ inline void tile_pv(WaveState<D, NQT>& w, const __bf16* vl, int hw, int tr_r, int tr_dim) {
  using G = Geometry<D>;
#pragma unroll
  for (int v = 0; v < G::vTiles; ++v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const __bf16* p0 = &vl[(u * 16 + 4 * hw + tr_r) * G::VS + v * 32 + tr_dim];
      const __bf16* p1 = &vl[(u * 16 + 8 + 4 * hw + tr_r) * G::VS + v * 32 + tr_dim];
      const bf16x8 a = read_v_operand(p0, p1);
#pragma unroll
      for (int c = 0; c < NQT; ++c)
        w.oacc[v][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.pb[u][c], w.oacc[v][c], 0, 0, 0);
    }
  }
}

// Block = WAVES waves, each owning NQT column tiles of 32 queries.  NQT = 1
// runs two waves per SIMD (<= 256 registers each); NQT = 2 halves the LDS
// operand traffic per MFMA and runs one wave per SIMD.  K/V tiles of 64 keys
// are double-buffered in LDS: the next tile's global loads are in flight
// while the current tile is multiplied; one barrier per tile.
template <int D, int WAVES, int NQT, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(NQT == 1 ? 2 : 1, NQT == 1 ? 2 : 1)))
void partial_kernel(const PartialParams p) {
  using G = Geometry<D>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int QPW = 32 * NQT;                    // query rows per wave
  constexpr int BR = QPW * WAVES;                  // query rows per block
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
  const int row0 = qt * BR + wave * QPW + l32;    // this lane's query row of column tile 0

  WaveState<D, NQT> w;
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    const __bf16* qrow = Qh + static_cast<size_t>(min(row0 + 32 * c, len_q - 1)) * D;
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      const int dim = s * 16 + hw * 8;
      if (dim < D) {
        w.qf[c][s] = *reinterpret_cast<const bf16x8*>(qrow + dim);
      } else {
        w.qf[c][s] = bf16x8{};
      }
    }
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v) w.oacc[v][c] = f32x16{};
    w.m_run[c] = -__builtin_inff();
    w.l_run[c] = 0.0f;
    w.lr_run[c] = 0.0f;
  }

  // K columns beyond d (d = 72 pads the contraction to 80) must read as zero.
  if constexpr (G::DK > D) {
    for (int i = tid; i < 2 * kBc; i += kThreads)
      *reinterpret_cast<u32x4*>(&k_lds[i / kBc][(i % kBc) * G::KS + D]) = u32x4{0u, 0u, 0u, 0u};
  }

  const int n_tiles = (len_k + kBc - 1) / kBc;
  u32x4 kreg[kLoads], vreg[kLoads];

  // Global -> register staging of one K tile and one V tile (tile index -1:
  // skip), and register -> LDS stores into the given buffers (-1: skip).
  auto gload = [&](int kt_k, int kt_v) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kBc * G::chunks) {
        const int key = c / G::chunks, ch = c % G::chunks;
        if (kt_k >= 0) {
          const int krow = min(kt_k * kBc + key, len_k - 1);
          kreg[i] = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(krow) * D + ch * 8);
        }
        if (kt_v >= 0) {
          const int vrow = min(kt_v * kBc + key, len_k - 1);
          vreg[i] = *reinterpret_cast<const u32x4*>(Vh + static_cast<size_t>(vrow) * D + ch * 8);
        }
      }
    }
  };
  auto swrite = [&](int kbuf, int vbuf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kBc * G::chunks) {
        const int key = c / G::chunks, ch = c % G::chunks;
        if (kbuf >= 0) *reinterpret_cast<u32x4*>(&k_lds[kbuf][key * G::KS + ch * 8]) = kreg[i];
        if (vbuf >= 0) *reinterpret_cast<u32x4*>(&v_lds[vbuf][key * G::VS + ch * 8]) = vreg[i];
      }
    }
  };

  // ds_read_b64_tr_b16 addressing for the V^T operand: in each 16-lane group
  // lane 4r+c supplies key row r, dims 4c..4c+3 of the group's 16 dims, and
  // receives dim (lane % 16) of the four rows.
  const int tr_r = (lane & 15) >> 2;
  const int tr_dim = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  auto softmax = [&](int kt) {
    if (kt + 1 < n_tiles) {
      tile_softmax<false>(w, kBc, hw, sl2);
    } else {
      tile_softmax<true>(w, len_k - kt * kBc, hw, sl2);
    }
  };

  if constexpr (SCHED == 0) {
    // Plain: per tile, scores -> softmax -> PV, one barrier.
    gload(0, 0);
    swrite(0, 0);
    __syncthreads();
    for (int kt = 0; kt + 1 < n_tiles; ++kt) {
      const int buf = kt & 1;
      gload(kt + 1, kt + 1);
      tile_scores(w.sacc, w, k_lds[buf], l32, hw);
      tile_softmax<false>(w, kBc, hw, sl2);
      tile_pv(w, v_lds[buf], hw, tr_r, tr_dim);
      swrite(buf ^ 1, buf ^ 1);
      __syncthreads();
    }
    const int kt = n_tiles - 1;
    tile_scores(w.sacc, w, k_lds[kt & 1], l32, hw);
    tile_softmax<true>(w, len_k - kt * kBc, hw, sl2);
    tile_pv(w, v_lds[kt & 1], hw, tr_r, tr_dim);
  } else if constexpr (SCHED == 1) {
    // Two groups of WAVES/2 waves offset by half a tile: phase ph runs, per
    // group, either M(i) = {scores of tile i, PV of tile i-1} or X(i) =
    // softmax of tile i; group 0 runs M(i) while group 1 runs X(i-1) and
    // vice versa, a block barrier after every phase.  K runs one tile ahead
    // of V: K(j+1), V(j) are fetched in phase 2j and stored in phase 2j+1.
    const int group = wave / (WAVES / 2);
    gload(0, -1);
    swrite(0, -1);
    __syncthreads();
    const int last = 2 * n_tiles + 1;
    for (int ph = 0; ph <= last; ++ph) {
      const int j = ph >> 1;
      if ((ph & 1) == 0) gload(j + 1 < n_tiles ? j + 1 : -1, j < n_tiles ? j : -1);
      const int t = ph - group;
      if (t >= 0 && t <= 2 * n_tiles) {
        const int i = t >> 1;
        if ((t & 1) == 0) {
          if (i < n_tiles) tile_scores(w.sacc, w, k_lds[i & 1], l32, hw);
          if (i >= 1) tile_pv(w, v_lds[(i - 1) & 1], hw, tr_r, tr_dim);
        } else {
          softmax(i);
        }
      }
      if (ph & 1) swrite(j + 1 < n_tiles ? (j + 1) & 1 : -1, j < n_tiles ? j & 1 : -1);
      __syncthreads();
    }
  } else {
    // Software pipeline inside each wave: iteration j runs the softmax of
    // tile j in the same instruction stream as the scores of tile j+1 (MFMA),
    // then the PV product of tile j.  K runs one tile ahead of V: iteration
    // j reads K(j+1) and V(j) and stages K(j+2) and V(j+1).
    f32x16 nx[2][NQT];      // scores of the next tile
    gload(0, 0);
    swrite(0, 0);
    __syncthreads();
    gload(1 < n_tiles ? 1 : -1, -1);
    tile_scores(w.sacc, w, k_lds[0], l32, hw);
    swrite(1 < n_tiles ? 1 : -1, -1);
    __syncthreads();
    for (int j = 0; j + 1 < n_tiles; ++j) {
      gload(j + 2 < n_tiles ? j + 2 : -1, j + 1);
      tile_max<false>(w, kBc, hw, sl2);
      tile_scores(nx, w, k_lds[(j + 1) & 1], l32, hw);
      tile_exp(w, sl2);
      tile_pv(w, v_lds[j & 1], hw, tr_r, tr_dim);
      swrite(j + 2 < n_tiles ? j & 1 : -1, (j + 1) & 1);
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NQT; ++c) w.sacc[kb][c] = nx[kb][c];
    }
    const int j = n_tiles - 1;
    tile_max<true>(w, len_k - j * kBc, hw, sl2);
    tile_exp(w, sl2);
    tile_pv(w, v_lds[j & 1], hw, tr_r, tr_dim);
  }

  // Epilogue: OUT = O / l_rounded, LSE = ln2 * (m + log2 l), into the slot.
  const size_t slot = static_cast<size_t>(h) * p.P * p.P + pair;
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    const float l_tot = w.l_run[c] + xor32(w.l_run[c]);
    const float inv = 1.0f / (w.lr_run[c] + xor32(w.lr_run[c]));
    const int row = row0 + 32 * c;
    if (row < len_q) {
      float* orow = p.O + (slot * p.S + row) * D;
#pragma unroll
      for (int v = 0; v < G::vTiles; ++v)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = v * 32 + 8 * g + 4 * hw;
          if (dim < D) {
            const f32x4 o = {w.oacc[v][c][4 * g] * inv, w.oacc[v][c][4 * g + 1] * inv,
                             w.oacc[v][c][4 * g + 2] * inv, w.oacc[v][c][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + dim) = o;
          }
        }
      if (hw == 0) p.LSE[slot * p.S + row] = (w.m_run[c] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
  }
}

// Loop schedule per head dim, from side-by-side measurement on MI355X: the
// in-wave pipeline (2) wins at d = 64 and 72, the plain loop (0) at d = 128
// (where the pipeline's second score buffer leaves fewer registers for LDS
// prefetch).  The two-group ping-pong (1) measured slower everywhere.
#ifndef DITANGO_SCHED
#define DITANGO_SCHED -1
#endif

template <int D, int WAVES, int NQT>
hipError_t launch(PartialParams& p, hipStream_t stream) {
  constexpr int chosen = DITANGO_SCHED >= 0 ? DITANGO_SCHED : (D == 128 ? 0 : 2);
  constexpr int sched = (chosen == 1 && WAVES != 8) ? 0 : chosen;
  hipLaunchKernelGGL((partial_kernel<D, WAVES, NQT, sched>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Query rows per wave for d = 128 (32 or 64); 64 halves LDS operand traffic
// per MFMA at one wave per SIMD.
#ifndef DITANGO_D128_QPW
#define DITANGO_D128_QPW 32
#endif

int partial_rows_per_block(int d, int S) {
  const int qpw = d == 128 ? DITANGO_D128_QPW : 32;
  const int wide = 4 * 2 * 32, narrow = 4 * 32;   // 8 or 4 column tiles per block
  (void)qpw;
  // 256 rows per block unless 128-row blocks waste clearly less of a ragged
  // partition (e.g. S = 549: 3 x 256 rows hold 71% useful work, 5 x 128 hold 86%).
  const long waste_w = (S + wide - 1) / wide * static_cast<long>(wide) - S;
  const long waste_n = (S + narrow - 1) / narrow * static_cast<long>(narrow) - S;
  return (waste_n * 10 + S < waste_w * 10) ? narrow : wide;
}

hipError_t launch_partial(PartialParams& p, int rows, hipStream_t stream) {
  const bool wide = rows == 256;
  switch (p.d) {
    case 64: return wide ? launch<64, 8, 1>(p, stream) : launch<64, 4, 1>(p, stream);
    case 72: return wide ? launch<72, 8, 1>(p, stream) : launch<72, 4, 1>(p, stream);
#if DITANGO_D128_QPW == 64
    case 128: return wide ? launch<128, 4, 2>(p, stream) : launch<128, 4, 1>(p, stream);
#else
    case 128: return wide ? launch<128, 8, 1>(p, stream) : launch<128, 4, 1>(p, stream);
#endif
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
