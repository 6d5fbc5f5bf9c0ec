// Fresh partial attention states on CDNA4 (gfx950), bf16 MFMA.
//
// For every fresh (query partition q, KV partition k) pair and head, one
// block computes the attention state (OUT, LSE) of a tile of query rows of
// partition q against all keys of partition k (DiTango page, attention-state
// section; the per-step partial attention of its ring-based composed
// attention) and stores it into the pair's cache slot.  For the grouped
// cache a work item is (q, slot) instead and its keys are those of all the
// slot's member partitions, which yields their composed state (Eq. 4) in
// one pass.
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
// probabilities gives LSE, and the sum of the rounded ones (v_dot2c_f32_bf16,
// or for d = 72 a ones column of V that makes it a row of O^T) normalises
// OUT, so the weights applied to V sum to one as used.
//
// Softmax runs in base 2 with the scale folded into one FMA.  A tile's
// probabilities are taken against the running max without first computing
// the tile max; only when a lane's tile sum leaves [0, 2^64] (first tile,
// or a score far above the running max) is the max recomputed and the state
// rescaled.  The final division by the row sum makes the result exact.
//
// Block = 4 or 8 waves of 32 query rows each (128 or 256 rows), two waves
// per SIMD at d = 128 (<= 256 VGPRs each, no accumulator spills to AGPRs),
// three at d = 64 and 72 (4-wave blocks, <= 168 VGPRs), so a SIMD can issue
// one wave's softmax while another's MFMAs run.  K/V tiles of 64 keys are double-buffered in LDS and filled by
// direct buffer-to-LDS loads (buffer_load ... lds): the next tile's loads
// are in flight while the current tile is multiplied.
// The grid is the compacted list of fresh work items: no block exists for a
// reused pair.

#include <hip/hip_runtime.h>

#include <type_traits>

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


// Direct tile loads as buffer_load ... lds (1) or global_load_lds (0).
#ifndef DITANGO_BUFFER_LDS
#define DITANGO_BUFFER_LDS 1
#endif
#ifndef DITANGO_ONES_ROW
#define DITANGO_ONES_ROW 1
#endif
#ifndef DITANGO_D72_DIRECT
#define DITANGO_D72_DIRECT 1
#endif

template <int D>
struct Geometry {
  static constexpr int DK = (D + 15) / 16 * 16;   // Q.K contraction, 16 per MFMA
  static constexpr int DV = (D + 31) / 32 * 32;   // rows of O^T, 32 per MFMA tile
  // When O^T has spare rows (d = 72 pads to 96), V column d holds 1.0 in
  // LDS, so O^T row d accumulates the sum of the rounded probabilities for
  // free and the per-element v_dot2c is skipped.
  static constexpr bool ones_row = DITANGO_ONES_ROW && DV > D;
  static constexpr int kSteps = DK / 16;
  static constexpr int vTiles = DV / 32;
  static constexpr int chunks = D / 8;            // 16-byte chunks per global row
  // Staged layout (global -> registers -> LDS; kept as an alternative for
  // d = 72): rows padded, strides chosen with a bank-conflict counter sweep
  // on gfx950 (64 banks of 4 bytes).  K rows are read 16 B per lane, 16 keys
  // per pass: a stride of an odd multiple of 4 dwords spreads them over all
  // banks.  V rows are read by ds_read_b64_tr_b16, 32 lanes per pass = 4 key
  // rows x 64 B: a stride of 16 or 48 (mod 64) dwords puts those rows on
  // disjoint banks.
  //
  // Direct layout: filled by 16-byte direct loads to LDS (a wave writes 64
  // consecutive 16-byte chunks, so a row's stride is a whole number of
  // chunks).  For d = 64 and 128 rows are unpadded and the 16-byte chunk c
  // of row r sits at position c ^ f(r); the global load of position p
  // fetches chunk p ^ f(r).
  //   K: f = r mod 16 (d=128) or (r/2) mod 8 (d=64): the 16 rows of a
  //      16-lane pass land on distinct banks.
  //   V: f = 4 (r mod 4) (d=128) or 4 ((r/2) mod 2) (d=64): the 4 rows x 4
  //      chunks of a 32-lane transpose-read pass land on distinct banks.
  //   d = 72: no swizzle.  K rows of 72 (36 dwords, an odd multiple of 4);
  //      the contraction pad 72..79 reads the next row's first chunk, which
  //      is finite and meets Q's zero pad.  V rows of 96 (48 dwords) whose
  //      chunks 9..11 -- the ones column and zeros -- are written once and
  //      skipped by the loads.
  static constexpr bool direct = D == 64 || D == 128 || (D == 72 && DITANGO_D72_DIRECT);
  static constexpr int KS = direct ? D : DK + 8;
  static constexpr int VS = direct ? DV : (DV == 128 ? 160 : 96);
  static constexpr int kcpr = KS / 8;             // 16-byte chunks per LDS row (direct layout)
  static constexpr int vcpr = VS / 8;
  static constexpr int kpad = direct && DK > D ? 8 : 0;   // elements past a K tile read by the last row
  static_assert(DV <= VS, "V row must fit its stride");
  static_assert((direct && D != 72) || (KS / 2) % 8 == 4, "K stride must be an odd multiple of 4 dwords");
  static_assert((direct && D != 72) || (VS / 2) % 64 == 16 || (VS / 2) % 64 == 48,
                "V stride must be 16 or 48 mod 64 dwords");
  __device__ static int kswz(int r) { return D == 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : 0; }
  __device__ static int vswz(int r) { return D == 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0; }
};

typedef __attribute__((address_space(3))) bf16x4_v lds_bf16x4;

__device__ __attribute__((always_inline)) inline bf16x8 read_v_operand(const __bf16* p0, const __bf16* p1) {
  bf16x4_v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  bf16x4_v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  u32x4 w = {ua.x, ua.y, ub.x, ub.y};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __attribute__((always_inline)) inline float xor32(float x) { return __shfl_xor(x, 32); }

// Element offset of 16-byte chunk `c` of K row `r` in an LDS tile.  The K
// swizzle depends on r mod 16, so rows 32 apart share it.
template <int D>
__device__ __attribute__((always_inline)) inline int k_operand_offset(int r, int c) {
  using G = Geometry<D>;
  if constexpr (G::direct) {
    return r * G::KS + ((c ^ G::kswz(r)) << 3);
  } else {
    return r * G::KS + c * 8;
  }
}

// Element offset of the 4 bf16 at dims [dim, dim+4) of V row `r` (dim % 4 == 0).
template <int D>
__device__ __attribute__((always_inline)) inline int v_operand_offset(int r, int dim) {
  using G = Geometry<D>;
  if constexpr (G::direct) {
    return r * G::VS + (((dim >> 3) ^ G::vswz(r)) << 3) + (dim & 7);
  } else {
    return r * G::VS + dim;
  }
}

// Per-wave pieces of the key-tile loop.  A wave owns 32 queries (one MFMA
// column tile); see the file comment for the operand layouts.
template <int D, int NQT, int NKB>
struct WaveState {
  using G = Geometry<D>;
  static constexpr int nkb = NKB;  // 32-key blocks per tile
  bf16x8 qf[NQT][G::kSteps];      // Q^T operand, per 32-query column tile
  f32x16 oacc[G::vTiles][NQT];    // O^T accumulator
  f32x16 sacc[NKB][NQT];          // S^T of the current tile
  bf16x8 pb[2 * NKB][NQT];        // P^T operand of the tile's 16-key steps
  float m_run[NQT], l_run[NQT], lr_run[NQT];
};

// Per-lane LDS element offsets of the MFMA operands, fixed for the whole
// kernel: koff[s] = K operand of k-step s (32-key block 0; block 1 is +32
// rows), voff[v] = first transpose read of 32-dim tile v (key step u adds
// 16 rows, the second read of a step 8 rows).
template <int D>
struct OperandOffsets {
  using G = Geometry<D>;
  int koff[G::kSteps];
  int voff[G::vTiles];
  __device__ OperandOffsets(int l32, int hw, int tr_r, int tr_dim) {
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) koff[s] = k_operand_offset<D>(l32, 2 * s + hw);
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v) voff[v] = v_operand_offset<D>(4 * hw + tr_r, v * 32 + tr_dim);
  }
};

// S^T = K Q^T for the 64 keys of one LDS tile into `sacc`; each K operand
// read from LDS feeds the NQT column tiles.
template <int D, int NQT, int NKB>
__device__ __attribute__((always_inline)) inline void tile_scores(f32x16 (&sacc)[NKB][NQT], const WaveState<D, NQT, NKB>& w,
                                                                  const __bf16* kl, const OperandOffsets<D>& off) {
  using G = Geometry<D>;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int c = 0; c < NQT; ++c) sacc[kb][c] = f32x16{};
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[kb * 32 * G::KS + off.koff[s]]);
#pragma unroll
      for (int c = 0; c < NQT; ++c)
        sacc[kb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[c][s], sacc[kb][c], 0, 0, 0);
    }
  }
}

// Online softmax of the tile held in sacc, into the P operand pb and the row
// sums.  Probabilities are exp2(s * scale * log2e - m) against the running
// max m WITHOUT first taking the tile's max: the fp32 sums and bf16
// probabilities stay exact in relative terms up to huge magnitudes, so m
// only has to keep every probability below 2^64.  Each lane checks the sum
// of its probabilities in the tile; if any lane's sum is not <= 2^64 (this
// includes inf and NaN, e.g. on the first tile where m = -inf) the tile
// takes the slow path: exact tile max, m raised to it, accumulated state
// rescaled, probabilities recomputed.  After the first tile this is rare.
// MASK: keys at or past `lim` in this tile score -inf (ragged last tile).
#ifndef DITANGO_INTERLEAVE_VALU
#define DITANGO_INTERLEAVE_VALU 9
#endif

template <int D, int NQT, int NKB>
__device__ __attribute__((always_inline)) inline void tile_probs(WaveState<D, NQT, NKB>& w, float sl2, float (&tl)[NQT],
                                                                 float (&tlr)[NQT]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    tl[c] = 0.0f;
    tlr[c] = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
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
          tl[c] += e0 + e1;
          if constexpr (!Geometry<D>::ones_row) tlr[c] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, tlr[c], false);
        }
        const u32x4 wv = {words[0], words[1], words[2], words[3]};
        w.pb[2 * kb + half][c] = __builtin_bit_cast(bf16x8, wv);
      }
  }
}

// Interleave the MFMAs and VALU instructions of the current scheduling
// region: n_mfma groups of (1 MFMA, per VALU).  Used where the next tile's
// score MFMAs and this tile's probabilities are independent, so one wave
// keeps the matrix core busy while it issues the softmax arithmetic.
template <int n_mfma, int per>
__device__ __attribute__((always_inline)) inline void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < n_mfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, per, 0);  // then `per` VALU
  }
}

template <bool MASK, bool INTERLEAVE = false, int D, int NQT, int NKB>
__device__ __attribute__((always_inline)) inline void tile_softmax(WaveState<D, NQT, NKB>& w, int lim, int hw,
                                                                   float sl2) {
  using G = Geometry<D>;
  constexpr uint32_t kSumLimitBits = 0x5f800000u;   // 2^64 as fp32 bits
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < NQT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i >> 2) + hw * 4 + (i & 3);
          if (key >= lim) w.sacc[kb][c][i] = -__builtin_inff();
        }
  }
  float tl[NQT], tlr[NQT];
  tile_probs(w, sl2, tl, tlr);
  if constexpr (INTERLEAVE) interleave_mfma_valu<NKB * G::kSteps * NQT, DITANGO_INTERLEAVE_VALU>();
  // Integer test on the magnitude bits: true for sums above 2^64, inf and
  // NaN alike, independent of how the compiler treats NaN comparisons.
  bool bad = false;
#pragma unroll
  for (int c = 0; c < NQT; ++c) bad |= (__builtin_bit_cast(uint32_t, tl[c]) & 0x7fffffffu) > kSumLimitBits;
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {
    asm volatile("; raise running max" ::);
#pragma unroll
    for (int c = 0; c < NQT; ++c) {
      float mx = w.sacc[0][c][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, w.sacc[kb][c][i]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(mx * sl2, w.m_run[c]);
      const float alpha = __builtin_amdgcn_exp2f(w.m_run[c] - m_new);   // 0 when m was -inf
      w.m_run[c] = m_new;
      w.l_run[c] *= alpha;
      w.lr_run[c] *= alpha;
#pragma unroll
      for (int v = 0; v < G::vTiles; ++v) w.oacc[v][c] *= alpha;
    }
    tile_probs(w, sl2, tl, tlr);
  }
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    w.l_run[c] += tl[c];
    w.lr_run[c] += tlr[c];
  }
}

// O^T += V^T P^T for the tile whose V sits in `vl`; each V operand read from
// LDS feeds the NQT column tiles.  Rows u*16 (+8) added to the base offsets
// keep the swizzle: it depends on the row only modulo 4 (d=128) or through
// (row/2) mod 2 (d=64), which adding a multiple of 8 rows leaves unchanged.
template <int D, int NQT, int NKB>
__device__ __attribute__((always_inline)) inline void tile_pv(WaveState<D, NQT, NKB>& w, const __bf16* vl,
                                                              const OperandOffsets<D>& off) {
  using G = Geometry<D>;
#pragma unroll
  for (int v = 0; v < G::vTiles; ++v) {
#pragma unroll
    for (int u = 0; u < 2 * NKB; ++u) {
      const __bf16* p0 = &vl[u * 16 * G::VS + off.voff[v]];
      const __bf16* p1 = &vl[(u * 16 + 8) * G::VS + off.voff[v]];
      const bf16x8 a = read_v_operand(p0, p1);
#pragma unroll
      for (int c = 0; c < NQT; ++c)
        w.oacc[v][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.pb[u][c], w.oacc[v][c], 0, 0, 0);
    }
  }
}

// One 16-byte chunk per lane of a key tile into LDS (buffer_load ... lds):
// the descriptor starts at the tile's first key t0 of `base` (rows of d
// bf16) and ends at key `len`, so a lane's offset is its fixed element
// offset `elem` in the tile and rows at or past `len` read zeros.  Built
// here rather than in the kernel's lambdas, which are also compiled for the
// host, where the descriptor builtin does not exist.
template <int D>
__device__ __attribute__((always_inline)) inline void tile_load_lds(const __bf16* base, int t0, int len, int elem,
                                                                    __bf16* dst) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(base) + static_cast<size_t>(t0) * D, 0, (len - t0) * D * 2, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, elem * 2, 0, 0, 0);
}

// Waves per SIMD.  d = 64 and 72 fit in 168 VGPRs (d = 72 with the plain
// loop; 8 bytes per lane spill, outside the tile loop) and run 4-wave
// blocks at three waves per SIMD (three blocks per CU): one wave alone
// issues VALU at about half rate, so the third wave keeps the VALU busy
// while the others wait (+7-11% at d = 64, +6-9% at d = 72; four spill).
// d = 128 needs about 250 VGPRs, and three of its blocks would need more
// LDS than a CU has, so it runs two (<= 256 VGPRs each).
#ifndef DITANGO_D64_WAVES_PER_SIMD
#define DITANGO_D64_WAVES_PER_SIMD 3
#endif
#ifndef DITANGO_D72_WAVES_PER_SIMD
#define DITANGO_D72_WAVES_PER_SIMD 3
#endif
template <int D, int NQT, int WAVES>
constexpr int waves_per_simd() {
  return NQT == 2 ? 1
         : (D == 64 && WAVES == 4) ? DITANGO_D64_WAVES_PER_SIMD
         : (D == 72 && WAVES == 4) ? DITANGO_D72_WAVES_PER_SIMD
                                   : 2;
}

// Block = WAVES waves, each owning NQT column tiles of 32 queries.  NQT = 1
// runs two waves per SIMD (<= 256 registers each; three at d = 64 and 72); NQT = 2
// halves the LDS operand traffic per MFMA and runs one wave per SIMD.  K/V tiles of 64 keys
// are double-buffered in LDS: the next tile's global loads are in flight
// while the current tile is multiplied; one barrier per tile.
template <int D, int WAVES, int NQT, int SCHED, int BC, bool GROUPED>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(waves_per_simd<D, NQT, WAVES>(), waves_per_simd<D, NQT, WAVES>())))
void partial_kernel(const PartialParams p) {
  using G = Geometry<D>;
  constexpr int kBc = BC;                          // keys per K/V tile (32, 64 or 128)
  static_assert(BC == 32 || BC == 64 || BC == 128, "key tile of 32, 64 or 128");
  constexpr int kThreads = 64 * WAVES;
  constexpr int QPW = 32 * NQT;                    // query rows per wave
  constexpr int BR = QPW * WAVES;                  // query rows per block
  constexpr int kLoads = (kBc * G::chunks + kThreads - 1) / kThreads;
  // Four separate LDS buffers (not one array indexed at run time): distinct
  // variables get distinct alias scopes, so the compiler can see that reads
  // of one buffer never alias the direct loads filling the other and does not
  // make them wait for the prefetch.  The tile loop is unrolled by two so the
  // buffer of every access is a compile-time choice.
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kBc * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kBc * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kBc * G::VS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kBc * G::VS];

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
  const int it = p.pairs[pi];
  // Keys of the item: the concatenated key index j < len_k lives at token
  // k0 + j, or k0 + j + S once j >= len0 (a gap over query partition q when
  // it sits strictly inside a group; len0 = len_k otherwise).
  int qp, k0, len_k, len0;
  float* obase;   // OUT row 0 of this item's state
  float* lbase;   // LSE row 0
  if constexpr (!GROUPED) {
    qp = it / p.P;
    const int kp = it - qp * p.P;
    k0 = kp * p.S;
    len_k = min(p.S, p.N - k0);
    len0 = len_k;
    const size_t slot = static_cast<size_t>(h) * p.P * p.P + it;
    obase = p.O + slot * p.S * D;
    lbase = p.LSE + slot * p.S;
  } else {
    qp = it >> 6;
    const int s = it & 63;
    const int a = s == 0 ? qp : (s - 1) * p.g;                 // member partitions [a, b)
    const int b = s == 0 ? qp + 1 : min(a + p.g, p.P);
    int kb = a * p.S, ke = min(b * p.S, p.N);
    len0 = -1;
    if (s != 0 && a <= qp && qp < b) {                          // the group holds q: leave it out
      if (qp == a) {
        kb = (a + 1) * p.S;
      } else if (qp == b - 1) {
        ke = qp * p.S;
      } else {
        len0 = qp * p.S - kb;                                   // q is interior, so its partition is full
      }
    }
    k0 = kb;
    len_k = ke - kb - (len0 >= 0 ? p.S : 0);
    if (len0 < 0) len0 = len_k;
    const size_t row0 = (static_cast<size_t>(h) * p.P + qp) * p.S;
    obase = p.gO[s] + row0 * D;
    lbase = p.gLSE[s] + row0;
  }
  const int q0 = qp * p.S;
  const int len_q = min(p.S, p.N - q0);
  const size_t head = static_cast<size_t>(h) * p.N * D;
  const __bf16* Qh = p.Q + head + static_cast<size_t>(q0) * D;
  const __bf16* Kh = p.K + head + static_cast<size_t>(k0) * D;
  const __bf16* Vh = p.V + head + static_cast<size_t>(k0) * D;
  const float sl2 = p.scale_log2;
  const int row0 = qt * BR + wave * QPW + l32;    // this lane's query row of column tile 0

  WaveState<D, NQT, BC / 32> w;
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

  // K columns beyond d (d = 72 pads the contraction to 80) must read as
  // zero (staged layout), or as finite values (direct layout: the next row,
  // and past the last row this zeroed pad).
  if constexpr (G::DK > D) {
    if constexpr (G::direct) {
      if (tid < 2) *reinterpret_cast<u32x4*>(&(tid == 0 ? k_lds0 : k_lds1)[kBc * G::KS]) = u32x4{0u, 0u, 0u, 0u};
    } else {
      for (int i = tid; i < 2 * kBc; i += kThreads)
        *reinterpret_cast<u32x4*>(&(i < kBc ? k_lds0 : k_lds1)[(i % kBc) * G::KS + D]) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (G::ones_row) {
    if constexpr (G::direct) {
      // Chunks D/8 .. vcpr-1 of every V row: 1.0 at column D, zeros after.
      constexpr int padc = G::vcpr - D / 8;
      static_assert(D % 8 == 0 && padc >= 1, "ones column starts a spare chunk");
      for (int i = tid; i < 2 * kBc * padc; i += kThreads) {
        const int j = i % (kBc * padc);
        const int r = j / padc, c = D / 8 + j % padc;
        const u32x4 val = {c == D / 8 ? 0x3f80u : 0u, 0u, 0u, 0u};   // bf16 1.0 in element 0
        *reinterpret_cast<u32x4*>(&(i < kBc * padc ? v_lds0 : v_lds1)[r * G::VS + c * 8]) = val;
      }
    } else {
      for (int i = tid; i < 2 * kBc; i += kThreads) (i < kBc ? v_lds0 : v_lds1)[(i % kBc) * G::VS + D] = (__bf16)1.0f;
    }
  }

  const int n_tiles = (len_k + kBc - 1) / kBc;
  u32x4 kreg[G::direct ? 1 : kLoads], vreg[G::direct ? 1 : kLoads];

  // Tile transfers.  gload(kt_k, kt_v) starts fetching K tile kt_k and V
  // tile kt_v (-1: none); swrite(kbuf, vbuf) completes them into those LDS
  // buffers.  Direct layout: gload itself streams global memory into the
  // buffers (16-byte direct loads to LDS) and swrite only waits for it; the
  // buffers passed to swrite must be the ones given to the matching gload.
  // Staged layout: gload fills registers and swrite stores them.

  // Direct-load geometry: round i of a tile covers LDS chunk positions
  // [(i*WAVES + wave)*64, +64) (lane L writes position +L); per-lane element
  // offsets of the global source (swizzled) are fixed for the kernel.  V
  // positions past column d (the d = 72 ones/zero chunks) are not loaded.
  constexpr int kGroupsK = G::direct ? kBc * G::kcpr / 64 : 1;          // 64-chunk groups per K tile
  constexpr int kGroupsV = G::direct ? kBc * G::vcpr / 64 : 1;
  constexpr int kRoundsK = (kGroupsK + WAVES - 1) / WAVES;               // groups per wave (last may idle)
  constexpr int kRoundsV = (kGroupsV + WAVES - 1) / WAVES;
  static_assert(!G::direct || (kBc * G::kcpr % 64 == 0 && kBc * G::vcpr % 64 == 0),
                "tiles must split into 64-chunk groups");
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  int krow_of[kRoundsK], kgoff[kRoundsK], vrow_of[kRoundsV], vgoff[kRoundsV];
#pragma unroll
  for (int i = 0; i < kRoundsK; ++i) {
    const int idx = min((i * WAVES + wave) * 64 + lane, kBc * G::kcpr - 1);
    const int r = G::direct ? idx / G::kcpr : 0, pos = G::direct ? idx % G::kcpr : 0;
    krow_of[i] = r;
    kgoff[i] = r * D + ((pos ^ G::kswz(r)) << 3);
  }
#pragma unroll
  for (int i = 0; i < kRoundsV; ++i) {
    const int idx = min((i * WAVES + wave) * 64 + lane, kBc * G::vcpr - 1);
    const int r = G::direct ? idx / G::vcpr : 0, pos = G::direct ? idx % G::vcpr : 0;
    vrow_of[i] = r;
    vgoff[i] = pos < D / 8 ? r * D + ((pos ^ G::vswz(r)) << 3) : -1;   // -1: spare chunk, not loaded
  }
  // Global source of LDS row r of key tile kt (element offset `goff` of
  // that row): the tile's first token is a scalar unless the tile runs past
  // the last key (rows there repeat the last key) or straddles the gap;
  // those tiles map each row on its own.
  auto tile_src = [&](const __bf16* base, int kt, int r, int goff) __attribute__((always_inline)) {
    const int t0 = kt * kBc;
    if constexpr (!GROUPED) {
      if (t0 + kBc > len_k && t0 + r >= len_k) return base + static_cast<size_t>(len_k - 1 - r) * D + goff;
      return base + static_cast<size_t>(t0) * D + goff;
    } else {
      if (t0 + kBc <= len_k && (t0 + kBc <= len0 || t0 >= len0)) {
        return base + static_cast<size_t>(t0 + (t0 >= len0 ? p.S : 0)) * D + goff;
      }
      int j = min(t0 + r, len_k - 1);
      j += j >= len0 ? p.S : 0;
      return base + static_cast<size_t>(j) * D + (goff - r * D);
    }
  };
  // Buffer descriptors over this item's keys, from token k0 to the end of the
  // sequence (fewer than 2^31 bytes: the host limits N * d to 2^30).  The
  // direct loads go through buffer_load ... lds: the compiler's wait-count
  // tracking keeps its LDS writes apart from the operand reads, whereas a
  // global_load_lds in flight makes it wait for every outstanding LDS read
  // before each use (+7-8% at d = 72 and 128).  Offsets past the end read 0.
  const int kv_bytes = (p.N - k0) * D * 2;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Kh), 0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Vh), 0, kv_bytes, 0x00020000);
  auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, const __bf16* base, const __bf16* src, __bf16* dst)
                 __attribute__((always_inline)) {
#if DITANGO_BUFFER_LDS
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                             static_cast<int>(src - base) * 2, 0, 0, 0);
#else
    (void)rsrc;
    (void)base;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
#endif
  };
  // With buffer loads a tile gets a descriptor of its own, based at the
  // tile's first key and ending at the last key of its contiguous run
  // (scalar arithmetic), so each lane's offset is its fixed in-tile offset
  // and rows past the end read zeros (their scores are masked): no per-lane
  // address math.  A grouped item's tile that straddles the gap over q keeps
  // the per-lane row mapping.
  constexpr bool kTileRsrc = DITANGO_BUFFER_LDS;
  auto tile_load = [&](const __bf16* base, __amdgpu_buffer_rsrc_t whole, int kt, int elem, int r, __bf16* dst)
                       __attribute__((always_inline)) {
    const int t0 = kt * kBc;
    if constexpr (!GROUPED) {
      (void)whole;
      (void)r;
      tile_load_lds<D>(base, t0, len_k, elem, dst);
    } else {
      if (t0 + kBc <= len0 || t0 >= len0 || len0 == len_k) {   // one side of the gap (block-uniform)
        const bool after = t0 >= len0;
        tile_load_lds<D>(base, t0 + (after ? p.S : 0), after ? len_k + p.S : len0, elem, dst);
      } else {
        dma(whole, base, tile_src(base, kt, r, elem), dst);
      }
    }
  };
  auto gload_direct = [&](int kt_k, __bf16* kdst, int kt_v, __bf16* vdst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < (G::direct ? kRoundsK : 0); ++i) {
      if (kGroupsK % WAVES != 0 && i * WAVES + swave >= kGroupsK) break;   // wave-uniform
      const int lds_elem0 = (i * WAVES + swave) * 64 * 8;   // first element this wave writes
      if (kt_k >= 0) {
        if constexpr (kTileRsrc) {
          tile_load(Kh, krsrc, kt_k, kgoff[i], krow_of[i], kdst + lds_elem0);
        } else {
          dma(krsrc, Kh, tile_src(Kh, kt_k, krow_of[i], kgoff[i]), kdst + lds_elem0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (G::direct ? kRoundsV : 0); ++i) {
      if (kGroupsV % WAVES != 0 && i * WAVES + swave >= kGroupsV) break;   // wave-uniform
      const int lds_elem0 = (i * WAVES + swave) * 64 * 8;
      if (kt_v >= 0 && (G::vcpr == D / 8 || vgoff[i] >= 0)) {
        if constexpr (kTileRsrc) {
          tile_load(Vh, vrsrc, kt_v, vgoff[i], vrow_of[i], vdst + lds_elem0);
        } else {
          dma(vrsrc, Vh, tile_src(Vh, kt_v, vrow_of[i], vgoff[i]), vdst + lds_elem0);
        }
      }
    }
  };
  auto gload = [&](int kt_k, int kt_v) __attribute__((always_inline)) {
    if constexpr (G::direct) {
      (void)kt_k;
      (void)kt_v;
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int c = tid + i * kThreads;
        if (c < kBc * G::chunks) {
          const int key = c / G::chunks, ch = c % G::chunks;
          if (kt_k >= 0) {
            int krow = min(kt_k * kBc + key, len_k - 1);
            if constexpr (GROUPED) krow += krow >= len0 ? p.S : 0;
            kreg[i] = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(krow) * D + ch * 8);
          }
          if (kt_v >= 0) {
            int vrow = min(kt_v * kBc + key, len_k - 1);
            if constexpr (GROUPED) vrow += vrow >= len0 ? p.S : 0;
            vreg[i] = *reinterpret_cast<const u32x4*>(Vh + static_cast<size_t>(vrow) * D + ch * 8);
          }
        }
      }
    }
  };
  auto swrite = [&](__bf16* kdst, __bf16* vdst) __attribute__((always_inline)) {
    if constexpr (G::direct) {
      (void)kdst;
      (void)vdst;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int c = tid + i * kThreads;
        if (c < kBc * G::chunks) {
          const int key = c / G::chunks, ch = c % G::chunks;
          if (kdst) *reinterpret_cast<u32x4*>(&kdst[key * G::KS + ch * 8]) = kreg[i];
          if (vdst) *reinterpret_cast<u32x4*>(&vdst[key * G::VS + ch * 8]) = vreg[i];
        }
      }
    }
  };
  // Start fetching K tile kt_k into kdst and V tile kt_v into vdst (a tile
  // index of -1 fetches nothing; its destination must then be nullptr).
  __bf16* pend_k = nullptr;
  __bf16* pend_v = nullptr;
  auto fetch = [&](int kt_k, __bf16* kdst, int kt_v, __bf16* vdst) __attribute__((always_inline)) {
    if constexpr (G::direct) {
      gload_direct(kt_k, kdst, kt_v, vdst);
    } else {
      gload(kt_k, kt_v);
    }
    pend_k = kdst;
    pend_v = vdst;
  };
  // Complete the transfers started by the last fetch.
  auto land = [&]() __attribute__((always_inline)) { swrite(pend_k, pend_v); };

  // ds_read_b64_tr_b16 addressing for the V^T operand: in each 16-lane group
  // lane 4r+c supplies key row r, dims 4c..4c+3 of the group's 16 dims, and
  // receives dim (lane % 16) of the four rows.
  const int tr_r = (lane & 15) >> 2;
  const int tr_dim = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const OperandOffsets<D> off(l32, hw, tr_r, tr_dim);
  // Buffer pair B (0 or 1) as compile-time pointers.
  auto kb_ = [&](auto B) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(B)::value == 0) return k_lds0; else return k_lds1; };
  auto vb_ = [&](auto B) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(B)::value == 0) return v_lds0; else return v_lds1; };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  if constexpr (SCHED == 0) {
    // Plain: per tile, scores -> softmax -> PV, one barrier.  Tile kt lives
    // in buffer pair kt & 1; the next tile is fetched into the other pair.
    auto full_tile = [&](auto B, int kt) __attribute__((always_inline)) {
      constexpr int b = decltype(B)::value;
      using NB = std::integral_constant<int, 1 - b>;
      fetch(kt + 1, kb_(NB{}), kt + 1, vb_(NB{}));
      tile_scores(w.sacc, w, kb_(B), off);
      tile_softmax<false>(w, kBc, hw, sl2);
      tile_pv(w, vb_(B), off);
      land();
      __syncthreads();
    };
    auto last_tile = [&](auto B, int kt) __attribute__((always_inline)) {
      tile_scores(w.sacc, w, kb_(B), off);
      tile_softmax<true>(w, len_k - kt * kBc, hw, sl2);
      tile_pv(w, vb_(B), off);
    };
    fetch(0, k_lds0, 0, v_lds0);
    land();
    __syncthreads();
    int kt = 0;
    for (; kt + 2 < n_tiles; kt += 2) {
      full_tile(B0{}, kt);
      full_tile(B1{}, kt + 1);
    }
    if (kt + 1 < n_tiles) {
      full_tile(B0{}, kt);
      last_tile(B1{}, kt + 1);
    } else {
      last_tile(B0{}, kt);
    }
  } else {
    // Software pipeline inside each wave: iteration j runs the softmax of
    // tile j in the same instruction stream as the scores of tile j+1 (MFMA),
    // then the PV product of tile j.  K runs one tile ahead of V: iteration
    // j reads K(j+1) from pair (j+1)&1 and V(j) from pair j&1, and fetches
    // K(j+2) into pair j&1 and V(j+1) into pair (j+1)&1.
    f32x16 nx[BC / 32][NQT];   // scores of the next tile
    auto iter = [&](auto B, int j) __attribute__((always_inline)) {   // B = j & 1
      constexpr int b = decltype(B)::value;
      using NB = std::integral_constant<int, 1 - b>;
      const bool k2 = j + 2 < n_tiles;
      fetch(k2 ? j + 2 : -1, k2 ? kb_(B) : nullptr, j + 1, vb_(NB{}));
      tile_scores(nx, w, kb_(NB{}), off);
      tile_softmax<false, true>(w, kBc, hw, sl2);
      tile_pv(w, vb_(B), off);
      land();
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int c = 0; c < NQT; ++c) w.sacc[kb][c] = nx[kb][c];
    };
    auto last = [&](auto B, int j) __attribute__((always_inline)) {
      tile_softmax<true>(w, len_k - j * kBc, hw, sl2);
      tile_pv(w, vb_(B), off);
    };
    fetch(0, k_lds0, 0, v_lds0);
    land();
    __syncthreads();
    fetch(1 < n_tiles ? 1 : -1, 1 < n_tiles ? k_lds1 : nullptr, -1, nullptr);
    tile_scores(w.sacc, w, k_lds0, off);
    land();
    __syncthreads();
    int j = 0;
    for (; j + 2 < n_tiles; j += 2) {
      iter(B0{}, j);
      iter(B1{}, j + 1);
    }
    if (j + 1 < n_tiles) {
      iter(B0{}, j);
      last(B1{}, j + 1);
    } else {
      last(B0{}, j);
    }
  }

  // Epilogue: OUT = O / l_rounded, LSE = ln2 * (m + log2 l), into the slot.
#pragma unroll
  for (int c = 0; c < NQT; ++c) {
    const float l_tot = w.l_run[c] + xor32(w.l_run[c]);
    float lr_tot;
    if constexpr (G::ones_row) {
      // O^T row D sits in tile D/32, element 4*((D%32)/8) of the lanes of
      // half-wave 0 (D % 8 == 0); broadcast it to the query's other half.
      static_assert(D % 8 == 0, "ones row must start a 4-row group of half-wave 0");
      lr_tot = __shfl(w.oacc[D / 32][c][4 * ((D % 32) / 8)], l32);
    } else {
      lr_tot = w.lr_run[c] + xor32(w.lr_run[c]);
    }
    const float inv = 1.0f / lr_tot;
    const int row = row0 + 32 * c;
    if (row < len_q) {
      float* orow = obase + static_cast<size_t>(row) * D;
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
      if (hw == 0) lbase[row] = (w.m_run[c] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
  }
}

// Loop schedule per head dim, from side-by-side measurement on MI355X: the
// plain loop (0) at d = 64 (about 4% ahead of the pipeline) and d = 128
// (where the pipeline's second score buffer leaves fewer registers for LDS
// prefetch); at d = 72 the in-wave pipeline (2) is about 2% ahead at two
// waves per SIMD but spills at three, where the plain loop runs.  A two-group ping-pong
// (FA3-style, one group on MFMA while the other runs the softmax, two
// barriers per tile) was measured slower on every head dim and is not kept.
#ifndef DITANGO_SCHED
#define DITANGO_SCHED -1
#endif

// Keys per tile: 64 (32 leaves registers for scheduling; 128 was measured
// slower at d = 64 and spills at d = 72).
#ifndef DITANGO_BC
#define DITANGO_BC 64
#endif

template <int D, int WAVES, int NQT>
hipError_t launch(PartialParams& p, hipStream_t stream) {
  constexpr int sched =
      DITANGO_SCHED >= 0 ? DITANGO_SCHED : (D == 72 && waves_per_simd<D, NQT, WAVES>() == 2 ? 2 : 0);
  constexpr int bc = DITANGO_BC;
  static_assert(sched == 0 || sched == 2, "loop schedules: 0 (plain) or 2 (software-pipelined)");
  if (p.grouped) {
    hipLaunchKernelGGL((partial_kernel<D, WAVES, NQT, sched, bc, true>), dim3(p.n_blocks), dim3(64 * WAVES), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((partial_kernel<D, WAVES, NQT, sched, bc, false>), dim3(p.n_blocks), dim3(64 * WAVES), 0,
                       stream, p);
  }
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
  if (d == 64 && DITANGO_D64_WAVES_PER_SIMD > 2) return narrow;   // 4-wave blocks, three per CU
  if (d == 72 && DITANGO_D72_WAVES_PER_SIMD > 2) return narrow;
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
