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
// the product.  The fp32 sum of the unrounded probabilities gives LSE and
// normalises OUT; at d = 72, where O^T is padded to 96 rows anyway, a ones
// column of V makes the sum of the rounded probabilities a row of O^T for
// free, and OUT is normalised by that one (the weights applied to V then
// sum to one as used).
//
// Softmax runs in base 2 with the scale folded into one FMA.  A tile's
// probabilities are taken against the running max without first computing
// the tile max; only when a lane's tile sum leaves [0, 2^64] (the first
// tile, where the running max is -inf and the sums overflow to +inf, or a
// score far above the max so far) is the max recomputed and the state
// rescaled.  The final division by the row sum makes the result exact.
// Keys past the end of a ragged last tile score -FLT_MAX, so the arithmetic
// meets infinities only on the first tile and never a NaN.
//
// Block = 4 or 8 waves of 32 query rows each (128 or 256 rows); at d = 128
// two waves per SIMD (<= 256 registers each), at d = 64 and 72 4-wave blocks
// three per CU, three waves per SIMD (<= 168 registers): a lone wave issues
// VALU at about half rate, so more waves keep the VALU busy while others
// wait.  Per 64-key tile a wave issues its score MFMAs, the softmax of the
// tile and its PV MFMAs; the waves of a SIMD overlap one wave's MFMAs with
// another's softmax.  K/V tiles of 64 keys are double-buffered in LDS and
// filled by direct buffer-to-LDS loads (buffer_load ... lds): the next
// tile's loads are in flight while the current tile is multiplied; one
// barrier per tile.  The grid is the compacted list of fresh work items: no
// block exists for a reused pair.

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

constexpr int kTile = 64;                                // keys per LDS tile
constexpr float kMaskScore = -3.4028234663852886e38f;   // -FLT_MAX

template <int D>
struct Geometry {
  static constexpr int DK = (D + 15) / 16 * 16;   // Q.K contraction, 16 per MFMA
  static constexpr int DV = (D + 31) / 32 * 32;   // rows of O^T, 32 per MFMA tile
  // When O^T has spare rows (d = 72 pads to 96), V column d holds 1.0 in
  // LDS, so O^T row d accumulates the sum of the rounded probabilities for
  // free and the per-element v_dot2c is skipped.
  static constexpr bool ones_row = DV > D;
  static constexpr int kSteps = DK / 16;
  static constexpr int vTiles = DV / 32;
  // LDS rows are filled by 16-byte direct loads (a wave writes 64
  // consecutive 16-byte chunks, so a row's stride is a whole number of
  // chunks).  For d = 64 and 128 rows are unpadded and the 16-byte chunk c
  // of row r sits at position c ^ f(r); the global load of position p
  // fetches chunk p ^ f(r).  gfx950 LDS has 64 banks of 4 bytes.
  //   K: f = r mod 16 (d=128) or (r/2) mod 8 (d=64): the 16 rows of a
  //      16-lane pass land on distinct banks.
  //   V: f = 4 (r mod 4) (d=128) or 4 ((r/2) mod 2) (d=64): the 4 rows x 4
  //      chunks of a 32-lane transpose-read pass land on distinct banks.
  //   d = 72: no swizzle.  K rows of 72 (36 dwords, an odd multiple of 4);
  //      the contraction pad 72..79 reads the next row's first chunk, which
  //      is finite and meets Q's zero pad.  V rows of 96 (48 dwords) whose
  //      chunks 9..11 -- the ones column and zeros -- are written once and
  //      skipped by the loads.
  static constexpr int KS = D;
  static constexpr int VS = DV;
  static constexpr int kcpr = KS / 8;             // 16-byte chunks per LDS row
  static constexpr int vcpr = VS / 8;
  static constexpr int kpad = DK > D ? 8 : 0;     // elements past a K tile read by its last row
  static_assert(D == 64 || D == 72 || D == 128, "head dims 64, 72, 128");
  static_assert(D != 72 || (KS / 2) % 8 == 4, "d = 72 K rows must be an odd multiple of 4 dwords");
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

// Per-lane LDS element offsets of the MFMA operands, fixed for the whole
// kernel: koff[s] = K operand of contraction step s in a tile's first 32
// keys (the second 32 are +32 rows), voff[v] = first transpose read of
// 32-dim tile v (key step u adds 16 rows, the second read of a step 8
// rows).  The swizzles depend on the row only modulo 16 (K) or 4 (V), so
// block and key-step offsets are plain row offsets.
template <int D>
struct OperandOffsets {
  using G = Geometry<D>;
  int koff[G::kSteps];
  int voff[G::vTiles];
  __device__ OperandOffsets(int l32, int hw, int tr_r, int tr_dim) {
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) koff[s] = l32 * G::KS + (((2 * s + hw) ^ G::kswz(l32)) << 3);
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v) {
      const int r = 4 * hw + tr_r, dim = v * 32 + tr_dim;
      voff[v] = r * G::VS + (((dim >> 3) ^ G::vswz(r)) << 3) + (dim & 7);
    }
  }
};

// Registers of one wave: Q^T operand (32 queries), O^T accumulator, the
// scores of one 64-key tile (two 32-key blocks), its P^T operand (four
// 16-key steps) and the running statistics.
template <int D>
struct WaveState {
  using G = Geometry<D>;
  bf16x8 qf[G::kSteps];
  f32x16 oacc[G::vTiles];
  f32x16 sacc[2];
  bf16x8 pb[4];
  float m_run, l_run;
};

// S^T = K Q^T for the 64 keys of one LDS tile.
template <int D>
__device__ __attribute__((always_inline)) inline void tile_scores(WaveState<D>& w, const __bf16* kl,
                                                                  const OperandOffsets<D>& off) {
  using G = Geometry<D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    w.sacc[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kl[kb * 32 * G::KS + off.koff[s]]);
      w.sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[s], w.sacc[kb], 0, 0, 0);
    }
  }
}

// Probabilities exp2(s * scale * log2e - m) of the tile against the running
// max m, as the bf16 P^T operand, with the lane's sum of the unrounded
// probabilities (tl).
template <int D>
__device__ __attribute__((always_inline)) inline void tile_probs(WaveState<D>& w, float sl2, float& tl) {
  tl = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t words[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(w.sacc[kb][8 * half + j], sl2, -w.m_run));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(w.sacc[kb][8 * half + j + 1], sl2, -w.m_run));
        const bf16x2 pr = {(__bf16)e0, (__bf16)e1};   // one v_cvt_pk_bf16_f32
        words[j / 2] = __builtin_bit_cast(uint32_t, pr);
        tl += e0 + e1;
      }
      const u32x4 wv = {words[0], words[1], words[2], words[3]};
      w.pb[2 * kb + half] = __builtin_bit_cast(bf16x8, wv);
    }
}

// Online softmax of the tile held in sacc into the P operand and the row
// sums.  The probabilities are taken against the running max without first
// computing the tile max: the fp32 sums and bf16 probabilities stay exact
// in relative terms up to huge magnitudes, so the max only has to keep every
// probability below 2^64.  If any lane's tile sum is above 2^64 (always on
// the first tile, where the running max is -inf and the sums are +inf) the
// tile takes the slow path: exact tile max, the max raised to it, the state
// rescaled (by 0 on the first tile), the probabilities recomputed.  After
// the first tile this is rare.  MASK: keys at or past `lim` in the tile
// score -FLT_MAX (ragged last tile; key 0 of a tile always exists, so the
// tile max is finite).
template <bool MASK, int D>
__device__ __attribute__((always_inline)) inline void tile_softmax(WaveState<D>& w, int lim, int hw, float sl2) {
  using G = Geometry<D>;
  constexpr uint32_t kSumLimitBits = 0x5f800000u;   // 2^64 as fp32 bits
  if constexpr (MASK) {
    // element i of block kb holds key 32 kb + 8 (i / 4) + 4 hw + i % 4
    const int lim_l = lim - 4 * hw;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i >> 2) + (i & 3) >= lim_l) w.sacc[kb][i] = kMaskScore;
  }
  float tl;
  tile_probs<D>(w, sl2, tl);
  // Sums are >= 0 (never NaN): an integer compare of the bits is true above
  // 2^64 and for +inf.
  if (__builtin_amdgcn_ballot_w64(__builtin_bit_cast(uint32_t, tl) > kSumLimitBits) != 0) {
    asm volatile("; raise running max" ::);
    float mx = w.sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, w.sacc[kb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(mx * sl2, w.m_run);
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);   // 0 when the max was -inf
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v) w.oacc[v] *= alpha;
    tile_probs<D>(w, sl2, tl);
  }
  w.l_run += tl;
}

// O^T += V^T P^T for the tile whose V sits in `vl`.  Rows u*16 (+8) added
// to the base offsets keep the swizzle: it depends on the row only modulo 4
// (d=128) or through (row/2) mod 2 (d=64), which adding a multiple of 8 rows
// leaves unchanged.
template <int D>
__device__ __attribute__((always_inline)) inline void tile_pv(WaveState<D>& w, const __bf16* vl,
                                                              const OperandOffsets<D>& off) {
  using G = Geometry<D>;
#pragma unroll
  for (int v = 0; v < G::vTiles; ++v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x8 a = read_v_operand(&vl[u * 16 * G::VS + off.voff[v]], &vl[(u * 16 + 8) * G::VS + off.voff[v]]);
      w.oacc[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.pb[u], w.oacc[v], 0, 0, 0);
    }
  }
}

// One 16-byte chunk per lane of a key tile into LDS (buffer_load ... lds):
// the descriptor starts at the tile's first key t0 of `base` (rows of d
// bf16) and ends at key `len`, so a lane's offset is its fixed element
// offset `elem` in the tile and rows at or past `len` read zeros.  Byte
// counts stay below 2^31: the host keeps N * d below 2^30.
template <int D>
__device__ __attribute__((always_inline)) inline void tile_load_lds(const __bf16* base, int t0, int len, int elem,
                                                                    __bf16* dst) {
  const uint32_t bytes = static_cast<uint32_t>(max(len - t0, 0)) * (D * 2u);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(base) + static_cast<size_t>(t0) * D, 0, static_cast<int>(bytes), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, elem * 2, 0, 0, 0);
}

// Waves per SIMD: d = 64 and 72 fit in 168 VGPRs and run 4-wave blocks at
// three per CU; d = 128 needs up to 256 VGPRs and runs two.
template <int D>
constexpr int waves_per_simd() {
  return D == 128 ? 2 : 3;
}

// Per-lane map of a block's direct tile loads, fixed for the kernel.  Round
// i of a tile covers LDS chunk positions [(i*WAVES + wave)*64, +64) (lane L
// writes position +L); the global source offsets are swizzled as the LDS
// layout requires.  V positions past column d (the d = 72 ones/zero chunks)
// are not loaded.
template <int D, int WAVES>
struct TileLoadMap {
  using G = Geometry<D>;
  static constexpr int kGroupsK = kTile * G::kcpr / 64;            // 64-chunk groups per K tile
  static constexpr int kGroupsV = kTile * G::vcpr / 64;
  static constexpr int kRoundsK = (kGroupsK + WAVES - 1) / WAVES;  // groups per wave (the last may idle)
  static constexpr int kRoundsV = (kGroupsV + WAVES - 1) / WAVES;
  static_assert(kTile * G::kcpr % 64 == 0 && kTile * G::vcpr % 64 == 0, "tiles must split into 64-chunk groups");
  int krow_of[kRoundsK], kgoff[kRoundsK], vrow_of[kRoundsV], vgoff[kRoundsV];
  int swave;
  __device__ TileLoadMap(int wave, int lane) {
    swave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < kRoundsK; ++i) {
      const int idx = min((i * WAVES + wave) * 64 + lane, kTile * G::kcpr - 1);
      const int r = idx / G::kcpr, pos = idx % G::kcpr;
      krow_of[i] = r;
      kgoff[i] = r * D + ((pos ^ G::kswz(r)) << 3);
    }
#pragma unroll
    for (int i = 0; i < kRoundsV; ++i) {
      const int idx = min((i * WAVES + wave) * 64 + lane, kTile * G::vcpr - 1);
      const int r = idx / G::vcpr, pos = idx % G::vcpr;
      vrow_of[i] = r;
      vgoff[i] = pos < D / 8 ? r * D + ((pos ^ G::vswz(r)) << 3) : -1;   // -1: spare chunk, not loaded
    }
  }
};

// d = 72: the contraction pad 72..79 of a tile's last K row reads past the
// tile: zeros there.  V chunks D/8 .. vcpr-1 of every row: 1.0 at column D,
// zeros after (the ones row of O^T); the tile loads never write them.
template <int D, int kThreads>
__device__ __attribute__((always_inline)) inline void init_lds_pads(int tid, __bf16* k_lds0, __bf16* k_lds1,
                                                                    __bf16* v_lds0, __bf16* v_lds1) {
  using G = Geometry<D>;
  if constexpr (G::kpad > 0) {
    if (tid < 2) *reinterpret_cast<u32x4*>(&(tid == 0 ? k_lds0 : k_lds1)[kTile * G::KS]) = u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (G::ones_row) {
    constexpr int padc = G::vcpr - D / 8;
    static_assert(D % 8 == 0 && padc >= 1, "ones column starts a spare chunk");
    for (int i = tid; i < 2 * kTile * padc; i += kThreads) {
      const int j = i % (kTile * padc);
      const int r = j / padc, c = D / 8 + j % padc;
      const u32x4 val = {c == D / 8 ? 0x3f80u : 0u, 0u, 0u, 0u};   // bf16 1.0 in element 0
      *reinterpret_cast<u32x4*>(&(i < kTile * padc ? v_lds0 : v_lds1)[r * G::VS + c * 8]) = val;
    }
  }
}

// Q^T operand of this lane's query row (row `row` of the partition, clamped
// to its last row) and an empty state.
template <int D>
__device__ __attribute__((always_inline)) inline void load_q(WaveState<D>& w, const __bf16* Qh, int row, int len_q,
                                                             int hw) {
  using G = Geometry<D>;
  const __bf16* qrow = Qh + static_cast<size_t>(min(row, len_q - 1)) * D;
#pragma unroll
  for (int s = 0; s < G::kSteps; ++s) {
    const int dim = s * 16 + hw * 8;
    if (dim < D) {
      w.qf[s] = *reinterpret_cast<const bf16x8*>(qrow + dim);
    } else {
      w.qf[s] = bf16x8{};
    }
  }
}

template <int D>
__device__ __attribute__((always_inline)) inline void reset_state(WaveState<D>& w) {
  using G = Geometry<D>;
#pragma unroll
  for (int v = 0; v < G::vTiles; ++v) w.oacc[v] = f32x16{};
  w.m_run = -__builtin_inff();
  w.l_run = 0.0f;
}

// Attention of the block's query rows (Q^T in w.qf, state reset) over one
// key range: the concatenated key index j < len_k lives at row k0 + j of
// Kh0 / Vh0 (the head's K and V), or k0 + j + S once j >= len0 (a gap over
// the query partition when it sits strictly inside a group; len0 = len_k
// otherwise).  Per 64-key tile: scores -> softmax -> PV, one barrier; tile
// kt lives in buffer pair kt & 1 and the next tile is fetched into the other
// pair; the last (possibly ragged) tile is peeled so only it carries the key
// mask.  Every LDS read of the range is done when it returns (the caller
// meets the other waves before reusing the buffers).  A wave whose 32 query
// rows all lie past the end of a ragged partition (live = false) only loads
// its share of the tiles and meets the barriers, leaving its SIMD to the
// waves that have work.
template <int D, int WAVES, bool GAP>
__device__ __attribute__((always_inline)) inline void attend_keys(
    WaveState<D>& w, const __bf16* Kh0, const __bf16* Vh0, int N, int S, int k0, int len_k, int len0,
    __bf16* k_lds0, __bf16* k_lds1, __bf16* v_lds0, __bf16* v_lds1, const TileLoadMap<D, WAVES>& map,
    const OperandOffsets<D>& off, int hw, float sl2, bool live) {
  using G = Geometry<D>;
  using M = TileLoadMap<D, WAVES>;
  const __bf16* Kh = Kh0 + static_cast<size_t>(k0) * D;
  const __bf16* Vh = Vh0 + static_cast<size_t>(k0) * D;
  const int n_tiles = (len_k + kTile - 1) / kTile;
  // A tile that straddles the gap maps each LDS row to its token on its own,
  // through a descriptor over the range's keys from k0 to the end of the
  // sequence (< 2^31 bytes).  Every other tile gets a descriptor of its own,
  // based at the tile's first key and ending at the last key of its
  // contiguous run (scalar arithmetic): a lane's offset is its fixed in-tile
  // offset and rows past the end read zeros (their scores are masked).
  const uint32_t kv_bytes = static_cast<uint32_t>(N - k0) * (D * 2u);
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Kh), 0, static_cast<int>(kv_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Vh), 0, static_cast<int>(kv_bytes), 0x00020000);
  auto tile_load = [&](const __bf16* base, __amdgpu_buffer_rsrc_t whole, int kt, int elem, int r, __bf16* dst)
                       __attribute__((always_inline)) {
    const int t0 = kt * kTile;
    if constexpr (!GAP) {
      (void)whole;
      (void)r;
      tile_load_lds<D>(base, t0, len_k, elem, dst);
    } else {
      if (t0 + kTile <= len0 || t0 >= len0 || len0 == len_k) {   // one side of the gap (block-uniform)
        const bool after = t0 >= len0 && len0 != len_k;
        tile_load_lds<D>(base, t0 + (after ? S : 0), after ? len_k + S : len0, elem, dst);
      } else {
        int j = min(t0 + r, len_k - 1);
        j += j >= len0 ? S : 0;
        const int src = j * D + (elem - r * D);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(whole, (__attribute__((address_space(3))) void*)dst, 16, src * 2,
                                                 0, 0, 0);
      }
    }
  };
  // Start fetching K tile kt into kdst and V tile kt into vdst; land() waits
  // for this wave's loads and meets the other waves, after which every
  // wave's part of the tiles is visible.
  auto fetch = [&](int kt, __bf16* kdst, __bf16* vdst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < M::kRoundsK; ++i) {
      if (M::kGroupsK % WAVES != 0 && i * WAVES + map.swave >= M::kGroupsK) break;   // wave-uniform
      tile_load(Kh, krsrc, kt, map.kgoff[i], map.krow_of[i], kdst + (i * WAVES + map.swave) * 64 * 8);
    }
#pragma unroll
    for (int i = 0; i < M::kRoundsV; ++i) {
      if (M::kGroupsV % WAVES != 0 && i * WAVES + map.swave >= M::kGroupsV) break;   // wave-uniform
      if (G::vcpr == D / 8 || map.vgoff[i] >= 0)
        tile_load(Vh, vrsrc, kt, map.vgoff[i], map.vrow_of[i], vdst + (i * WAVES + map.swave) * 64 * 8);
    }
  };
  auto land = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
    __syncthreads();
  };
  // Buffer pair B (0 or 1) as compile-time pointers.
  auto kb_ = [&](auto B) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(B)::value == 0) return k_lds0; else return k_lds1; };
  auto vb_ = [&](auto B) __attribute__((always_inline)) -> __bf16* { if constexpr (decltype(B)::value == 0) return v_lds0; else return v_lds1; };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  auto full_tile = [&](auto B, int kt) __attribute__((always_inline)) {
    using NB = std::integral_constant<int, 1 - decltype(B)::value>;
    fetch(kt + 1, kb_(NB{}), vb_(NB{}));
    if (live) {
      tile_scores<D>(w, kb_(B), off);
      tile_softmax<false, D>(w, kTile, hw, sl2);
      tile_pv<D>(w, vb_(B), off);
    }
    land();
  };
  auto last_tile = [&](auto B, int kt) __attribute__((always_inline)) {
    if (live) {
      tile_scores<D>(w, kb_(B), off);
      tile_softmax<true, D>(w, len_k - kt * kTile, hw, sl2);
      tile_pv<D>(w, vb_(B), off);
    }
  };
  fetch(0, k_lds0, v_lds0);
  land();
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
}

// OUT = O / l, LSE = ln2 * (m + log2 l) of this lane's query row `row` into
// a state's rows at obase / lbase (rows at or past len_q are not stored); OUT
// in fp32, or rounded to bf16 when ST is __bf16.  l is the fp32 sum of the
// unrounded probabilities, except at d = 72, where O^T's ones row gives the
// sum of the rounded ones for free and normalises by it.
template <int D, typename ST>
__device__ __attribute__((always_inline)) inline void store_state(const WaveState<D>& w, ST* obase, float* lbase,
                                                                  int row, int len_q, int hw, int l32) {
  using G = Geometry<D>;
  const float l_tot = w.l_run + xor32(w.l_run);
  float lr_tot;
  if constexpr (G::ones_row) {
    // O^T row D sits in tile D/32, element 4*((D%32)/8) of the lanes of
    // half-wave 0 (D % 8 == 0); broadcast it to the query's other half.
    static_assert(D % 8 == 0, "ones row must start a 4-row group of half-wave 0");
    lr_tot = __shfl(w.oacc[D / 32][4 * ((D % 32) / 8)], l32);
  } else {
    lr_tot = l_tot;
  }
  const float inv = 1.0f / lr_tot;
  if (row < len_q) {
    ST* orow = obase + static_cast<size_t>(row) * D;
#pragma unroll
    for (int v = 0; v < G::vTiles; ++v)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = v * 32 + 8 * g + 4 * hw;
        if (dim < D) {
          if constexpr (std::is_same<ST, __bf16>::value) {
            const bf16x2 lo = {(__bf16)(w.oacc[v][4 * g] * inv), (__bf16)(w.oacc[v][4 * g + 1] * inv)};
            const bf16x2 hi = {(__bf16)(w.oacc[v][4 * g + 2] * inv), (__bf16)(w.oacc[v][4 * g + 3] * inv)};
            const u32x2 o = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            *reinterpret_cast<u32x2*>(orow + dim) = o;
          } else {
            const f32x4 o = {w.oacc[v][4 * g] * inv, w.oacc[v][4 * g + 1] * inv, w.oacc[v][4 * g + 2] * inv,
                             w.oacc[v][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + dim) = o;
          }
        }
      }
    if (hw == 0) lbase[row] = (w.m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

// Keys of slot s of query partition q in the grouped cache: slot 0 is the
// local partition q, slot 1 + j the member partitions [j g, min(j g + g, P))
// of group j without q.  The concatenated key index j < len_k lives at token
// k0 + j, or k0 + j + S once j >= len0 (a gap over q's partition when q sits
// strictly inside the group; len0 = len_k otherwise).
__device__ __attribute__((always_inline)) inline void group_keys(int N, int P, int S, int g, int q, int s, int& k0,
                                                                 int& len_k, int& len0) {
  const int a = s == 0 ? q : (s - 1) * g;                     // member partitions [a, bnd)
  const int bnd = s == 0 ? q + 1 : min(a + g, P);
  int kb = a * S, ke = min(bnd * S, N);
  len0 = -1;
  if (s != 0 && a <= q && q < bnd) {                          // the group holds q: leave it out
    if (q == a) {
      kb = (a + 1) * S;
    } else if (q == bnd - 1) {
      ke = q * S;
    } else {
      len0 = q * S - kb;                                      // q is interior, so its partition is full
    }
  }
  k0 = kb;
  len_k = ke - kb - (len0 >= 0 ? S : 0);
  if (len0 < 0) len0 = len_k;
}

// XCD-aware block order: blocks are dealt round-robin to the 8 XCDs; remap
// so each XCD runs a contiguous range of work items (items sharing K/V then
// share its L2).
__device__ __attribute__((always_inline)) inline int xcd_item(int nb) {
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + (b >> 3);
}

template <int D, int WAVES, bool GROUPED, typename ST>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>())))
void partial_kernel(const PartialParams p) {
  using G = Geometry<D>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int BR = 32 * WAVES;                   // query rows per block
  // Four separate LDS buffers (not one array indexed at run time): distinct
  // variables get distinct alias scopes, so the compiler can see that reads
  // of one buffer never alias the direct loads filling the other and does not
  // make them wait for the prefetch.  The tile loop is unrolled by two so the
  // buffer of every access is a compile-time choice.
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kTile * G::VS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kTile * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;   // half-wave
  const int l32 = lane & 31;

  const int item = xcd_item(p.n_blocks);
  const int qt = item % p.q_tiles;
  const int rest = item / p.q_tiles;
  const int pi = rest % p.n_pairs;
  const int h = rest / p.n_pairs;
  const int it = p.pairs[pi];
  // Keys of the item: k0 .. k0 + len_k, with a gap of S tokens over query
  // partition q at concatenated index len0 when it sits strictly inside a
  // group (len0 = len_k otherwise).
  int qp, k0, len_k, len0;
  ST* obase;      // OUT row 0 of this item's state
  float* lbase;   // LSE row 0
  if constexpr (!GROUPED) {
    qp = it / p.P;
    const int kp = it - qp * p.P;
    k0 = kp * p.S;
    len_k = min(p.S, p.N - k0);
    len0 = len_k;
    const size_t slot = static_cast<size_t>(h) * p.P * p.P + it;
    obase = static_cast<ST*>(p.O) + slot * p.S * D;
    lbase = p.LSE + slot * p.S;
  } else {
    qp = it >> 6;
    const int s = it & 63;
    group_keys(p.N, p.P, p.S, p.g, qp, s, k0, len_k, len0);
    const size_t row0 = (static_cast<size_t>(h) * p.P + qp) * p.S;
    obase = static_cast<ST*>(p.gO[s]) + row0 * D;
    lbase = p.gLSE[s] + row0;
  }
  const int q0 = qp * p.S;
  const int len_q = min(p.S, p.N - q0);
  const size_t head = static_cast<size_t>(h) * p.N * D;
  const int row0 = qt * BR + wave * 32 + l32;     // this lane's query row
  const bool live = __builtin_amdgcn_readfirstlane(qt * BR + wave * 32) < len_q;   // any row of the wave

  WaveState<D> w;
  load_q<D>(w, p.Q + head + static_cast<size_t>(q0) * D, row0, len_q, hw);
  reset_state<D>(w);
  init_lds_pads<D, kThreads>(tid, k_lds0, k_lds1, v_lds0, v_lds1);
  const TileLoadMap<D, WAVES> map(wave, lane);
  // ds_read_b64_tr_b16 addressing for the V^T operand: in each 16-lane group
  // lane 4r+c supplies key row r, dims 4c..4c+3 of the group's 16 dims, and
  // receives dim (lane % 16) of the four rows.
  const OperandOffsets<D> off(l32, hw, (lane & 15) >> 2, ((lane >> 4) & 1) * 16 + 4 * (lane & 3));
  attend_keys<D, WAVES, GROUPED>(w, p.K + head, p.V + head, p.N, p.S, k0, len_k, len0, k_lds0, k_lds1, v_lds0,
                                 v_lds1, map, off, hw, p.scale_log2, live);
  store_state<D, ST>(w, obase, lbase, row0, len_q, hw, l32);
}

// Composition (Eq. 4) of the n states of this wave's rows (nv <= 32 of
// them) into the output rows at dst_o / dst_l: m = max_k LSE_k,
// w_k = exp(LSE_k - m) / sum_k exp(LSE_k - m), OUT = sum_k w_k OUT_k,
// LSE = m + log sum.  so(k) / sl(k) give state k's OUT (ST: fp32 or bf16)
// and LSE at the wave's first row, for a uniform k < n.  Lane l owns row
// l % 32 and the states k = 2i + l / 32, so all n LSE loads of a row are in
// flight at once and the weights stay in registers.  The rows' OUT values of
// a state are nv*d contiguous elements, streamed in 16-byte chunks (4 fp32
// or 8 bf16; chunk c = lane + 64 j holds row c / (d / chunk)),
// non-temporal; a lane takes its chunk's weight from the lane that owns the
// row and the state's parity.  Fresh states among them were written by
// this wave (the caller has fenced those stores).
template <int D, typename ST, typename SO, typename SL>
__device__ __attribute__((always_inline)) inline void merge_rows(int n, SO so, SL sl, float* dst_o, float* dst_l,
                                                                 int nv, int lane) {
  constexpr bool kBF = std::is_same<ST, __bf16>::value;
  constexpr int EPC = 16 / sizeof(ST);             // elements per 16-byte chunk
  constexpr int NQ = EPC / 4;                      // fp32 quads per chunk
  constexpr int CPR = D / EPC;                     // 16-byte chunks per row
  constexpr int J = (32 * CPR + 63) / 64;          // chunks per lane for 32 rows
  constexpr int KH = DITANGO_MAX_SLOTS / 2;        // states per half-wave
  constexpr float kLog2e = 1.4426950408889634f;
  const int hw = lane >> 5;
  const int rr = min(lane & 31, nv - 1);
  float wk[KH];
#pragma unroll
  for (int i = 0; i < KH; ++i) {
    const int k = 2 * i + hw;
    const float* la = sl(min(2 * i, n - 1));
    const float* lb = sl(min(2 * i + 1, n - 1));
    wk[i] = k < n ? (hw ? lb : la)[rr] : 0.0f;
  }
  float m = hw < n ? wk[0] : kMaskScore;          // half-wave 0 always holds state 0
#pragma unroll
  for (int i = 1; i < KH; ++i)
    if (2 * i + hw < n) m = fmaxf(m, wk[i]);
  m = fmaxf(m, xor32(m));
  float zh = 0.0f;
#pragma unroll
  for (int i = 0; i < KH; ++i) {
    wk[i] = 2 * i + hw < n ? __builtin_amdgcn_exp2f((wk[i] - m) * kLog2e) : 0.0f;
    zh += wk[i];
  }
  const float z = zh + xor32(zh);
  const float invz = 1.0f / z;
#pragma unroll
  for (int i = 0; i < KH; ++i) wk[i] *= invz;

  int crow[J];
#pragma unroll
  for (int j = 0; j < J; ++j) crow[j] = min((lane + 64 * j) / CPR, 31);
  f32x4 acc[J][NQ];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < NQ; ++u) acc[j][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int valid = nv * CPR;                      // chunks of the valid rows
  // Each state's rows are read through a buffer descriptor ending at the
  // last valid row: chunks past it read as zeros (never stored), so the
  // loads need no branches or clamps, and chunk j's offset is the lane's
  // offset plus a constant.  Cache policy 2: non-temporal.
  auto load_state = [&](u32x4(&o)[J], int k) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<ST*>(so(k)), 0, valid * 16, 0x00020000);
#pragma unroll
    for (int j = 0; j < J; ++j)
      o[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + j * 1024, 0, 2));
  };
  // bf16 -> fp32 is exact: the pattern in the high half of a word.
  auto accumulate = [&](const u32x4(&o)[J], float w, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float wt = __shfl(w, crow[j] + 32 * b);
      if constexpr (kBF) {
        const f32x4 lo = {__builtin_bit_cast(float, o[j].x << 16), __builtin_bit_cast(float, o[j].x & 0xffff0000u),
                          __builtin_bit_cast(float, o[j].y << 16), __builtin_bit_cast(float, o[j].y & 0xffff0000u)};
        const f32x4 hi = {__builtin_bit_cast(float, o[j].z << 16), __builtin_bit_cast(float, o[j].z & 0xffff0000u),
                          __builtin_bit_cast(float, o[j].w << 16), __builtin_bit_cast(float, o[j].w & 0xffff0000u)};
        acc[j][0] += wt * lo;
        acc[j][NQ - 1] += wt * hi;
      } else {
        acc[j][0] += wt * __builtin_bit_cast(f32x4, o[j]);
      }
    }
  };
  // States 2i (half-wave 0's weights) and 2i + 1 (half-wave 1's) per
  // iteration, each state's loads issued one state ahead of its use; the
  // weights shift down one register per iteration so the current pair's
  // are always wk[0].  The scheduling barriers keep each load batch after
  // the arithmetic that frees its registers, so the batch in flight stays in
  // the same registers across the loop's back edge (no copy that would wait
  // for it).
  u32x4 oa[J], ob[J];
  load_state(oa, 0);
#pragma nounroll
  for (int i = 0; 2 * i < n; ++i) {
    load_state(ob, min(2 * i + 1, n - 1));       // n odd: the last pair's second state has weight 0
    __builtin_amdgcn_sched_barrier(0);
    accumulate(oa, wk[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_state(oa, min(2 * i + 2, n - 1));
    __builtin_amdgcn_sched_barrier(0);
    accumulate(ob, wk[0], 1);
#pragma unroll
    for (int t = 0; t + 1 < KH; ++t) wk[t] = wk[t + 1];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = lane + 64 * j;
    if (c < valid) {
#pragma unroll
      for (int u = 0; u < NQ; ++u) __builtin_nontemporal_store(acc[j][u], reinterpret_cast<f32x4*>(dst_o + EPC * c + 4 * u));
    }
  }
  if (hw == 0 && lane < nv) dst_l[lane] = m + __builtin_amdgcn_logf(z) * 0.69314718055994531f;
}

// The whole step of the per-pair cache for one (head, query partition,
// row tile): the fresh pairs of the partition's row of the mask, one after
// the other over the same query rows, each state stored into its slot; then
// each wave composes its rows' P states (the fresh ones just stored and the
// cached ones) into the output.  The composition needs no pass of its own
// over the states: at d = 64 and 72 (three blocks per CU) it overlaps the
// other blocks' matrix work; at d = 128 a block fills its CU and the phase
// runs at that CU's memory rate while the other CUs keep multiplying.
template <int D, int WAVES, typename ST>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>())))
void step_kernel(const StepParams p) {
  using G = Geometry<D>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int BR = 32 * WAVES;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kTile * G::VS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kTile * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;
  const int l32 = lane & 31;

  const int item = xcd_item(p.n_blocks);
  const int qt = item % p.q_tiles;
  const int rest = item / p.q_tiles;
  const int q = rest % p.P;
  const int h = rest / p.P;
  const int q0 = q * p.S;
  const int len_q = min(p.S, p.N - q0);
  const size_t head = static_cast<size_t>(h) * p.N * D;
  const int wrow0 = qt * BR + wave * 32;          // this wave's first query row
  const int row0 = wrow0 + l32;                   // this lane's query row
  const bool live = __builtin_amdgcn_readfirstlane(wrow0) < len_q;   // any row of the wave
  const int nf = p.nf[q];

  if (nf > 0) {
    WaveState<D> w;
    load_q<D>(w, p.Q + head + static_cast<size_t>(q0) * D, row0, len_q, hw);
    init_lds_pads<D, kThreads>(tid, k_lds0, k_lds1, v_lds0, v_lds1);
    const TileLoadMap<D, WAVES> map(wave, lane);
    const OperandOffsets<D> off(l32, hw, (lane & 15) >> 2, ((lane >> 4) & 1) * 16 + 4 * (lane & 3));
    for (int i = 0; i < nf; ++i) {
      if (i > 0) __syncthreads();   // every wave is done with the previous pair's tiles
      const int k = p.fresh[q][i];
      const int k0 = k * p.S;
      const int len_k = min(p.S, p.N - k0);
      reset_state<D>(w);
      attend_keys<D, WAVES, false>(w, p.K + head, p.V + head, p.N, p.S, k0, len_k, len_k, k_lds0, k_lds1, v_lds0,
                                   v_lds1, map, off, hw, p.scale_log2, live);
      const size_t slot = static_cast<size_t>(h) * p.P * p.P + static_cast<size_t>(q) * p.P + k;
      store_state<D, ST>(w, static_cast<ST*>(p.O) + slot * p.S * D, p.LSE + slot * p.S, row0, len_q, hw, l32);
    }
    // the wave's state stores complete before it reads them back
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  }
  const int r0 = __builtin_amdgcn_readfirstlane(wrow0);   // uniform per wave: keeps the descriptors scalar
  const int nv = min(32, len_q - r0);
  if (nv > 0) {
    const size_t slot0 = static_cast<size_t>(h) * p.P * p.P + static_cast<size_t>(q) * p.P;   // pair (q, 0)
    const size_t out0 = static_cast<size_t>(h) * p.N + static_cast<size_t>(q0) + r0;
    merge_rows<D, ST>(
        p.P, [&](int k) { return static_cast<const ST*>(p.O) + ((slot0 + k) * p.S + r0) * D; },
        [&](int k) { return p.LSE + (slot0 + k) * p.S + r0; }, p.Oout + out0 * D, p.LSEout + out0, nv, lane);
  }
}

// The step of the grouped cache for one (head, query partition, row tile):
// the COMPUTE slots of q one after the other over the same query rows (each
// over its members' keys, with the gap over q when q sits inside the
// group), each state stored into its slot buffer; then each wave composes
// its rows over q's live slots, as step_kernel does for the pair slots.
template <int D, int WAVES, typename ST>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>())))
void group_step_kernel(const GroupStepParams p) {
  using G = Geometry<D>;
  constexpr int kThreads = 64 * WAVES;
  constexpr int BR = 32 * WAVES;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kTile * G::KS + G::kpad];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kTile * G::VS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kTile * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = lane >> 5;
  const int l32 = lane & 31;

  const int item = xcd_item(p.n_blocks);
  const int qt = item % p.q_tiles;
  const int rest = item / p.q_tiles;
  const int q = rest % p.P;
  const int h = rest / p.P;
  const int q0 = q * p.S;
  const int len_q = min(p.S, p.N - q0);
  const size_t head = static_cast<size_t>(h) * p.N * D;
  const size_t row_base = (static_cast<size_t>(h) * p.P + q) * p.S;   // row 0 of (h, q) in a slot buffer
  const int wrow0 = qt * BR + wave * 32;
  const int row0 = wrow0 + l32;
  const bool live = __builtin_amdgcn_readfirstlane(wrow0) < len_q;
  const int nc = p.nc[q];

  if (nc > 0) {
    WaveState<D> w;
    load_q<D>(w, p.Q + head + static_cast<size_t>(q0) * D, row0, len_q, hw);
    init_lds_pads<D, kThreads>(tid, k_lds0, k_lds1, v_lds0, v_lds1);
    const TileLoadMap<D, WAVES> map(wave, lane);
    const OperandOffsets<D> off(l32, hw, (lane & 15) >> 2, ((lane >> 4) & 1) * 16 + 4 * (lane & 3));
    for (int i = 0; i < nc; ++i) {
      if (i > 0) __syncthreads();   // every wave is done with the previous slot's tiles
      const int s = p.cslot[q][i];
      int k0, len_k, len0;
      group_keys(p.N, p.P, p.S, p.g, q, s, k0, len_k, len0);
      reset_state<D>(w);
      attend_keys<D, WAVES, true>(w, p.K + head, p.V + head, p.N, p.S, k0, len_k, len0, k_lds0, k_lds1, v_lds0,
                                  v_lds1, map, off, hw, p.scale_log2, live);
      store_state<D, ST>(w, static_cast<ST*>(p.gO[s]) + row_base * D, p.gLSE[s] + row_base, row0, len_q, hw, l32);
    }
    // the wave's state stores complete before it reads them back
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  }
  const int r0 = __builtin_amdgcn_readfirstlane(wrow0);
  const int nv = min(32, len_q - r0);
  if (nv > 0) {
    const size_t out0 = static_cast<size_t>(h) * p.N + static_cast<size_t>(q0) + r0;
    merge_rows<D, ST>(
        p.nl[q], [&](int k) { return static_cast<const ST*>(p.gO[p.lslot[q][k]]) + (row_base + r0) * D; },
        [&](int k) { return p.gLSE[p.lslot[q][k]] + row_base + r0; }, p.Oout + out0 * D, p.LSEout + out0, nv, lane);
  }
}

template <int D, int WAVES, typename ST>
void launch_st(PartialParams& p, hipStream_t stream) {
  if (p.grouped) {
    hipLaunchKernelGGL((partial_kernel<D, WAVES, true, ST>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  } else {
    hipLaunchKernelGGL((partial_kernel<D, WAVES, false, ST>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  }
}

template <int D, int WAVES>
hipError_t launch(PartialParams& p, hipStream_t stream) {
  if (p.state_bf16) {
    launch_st<D, WAVES, __bf16>(p, stream);
  } else {
    launch_st<D, WAVES, float>(p, stream);
  }
  return hipGetLastError();
}

template <int D, int WAVES>
hipError_t launch_step_d(StepParams& p, hipStream_t stream) {
  if (p.state_bf16) {
    hipLaunchKernelGGL((step_kernel<D, WAVES, __bf16>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  } else {
    hipLaunchKernelGGL((step_kernel<D, WAVES, float>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, int WAVES>
hipError_t launch_group_step_d(GroupStepParams& p, hipStream_t stream) {
  if (p.state_bf16) {
    hipLaunchKernelGGL((group_step_kernel<D, WAVES, __bf16>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  } else {
    hipLaunchKernelGGL((group_step_kernel<D, WAVES, float>), dim3(p.n_blocks), dim3(64 * WAVES), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

// Query rows per block: 128 (4 waves) for d = 64 and 72; for d = 128, 256
// (8 waves) unless 128-row blocks waste clearly less of a ragged partition
// (e.g. S = 549: 3 x 256 rows hold 71% useful work, 5 x 128 hold 86%).
int partial_rows_per_block(int d, int S) {
  const int wide = 256, narrow = 128;
  if (d != 128) return narrow;
  const long waste_w = (S + wide - 1) / wide * static_cast<long>(wide) - S;
  const long waste_n = (S + narrow - 1) / narrow * static_cast<long>(narrow) - S;
  return (waste_n * 10 + S < waste_w * 10) ? narrow : wide;
}

hipError_t launch_partial(PartialParams& p, int rows, hipStream_t stream) {
  switch (p.d) {
    case 64: return rows == 128 ? launch<64, 4>(p, stream) : hipErrorInvalidValue;
    case 72: return rows == 128 ? launch<72, 4>(p, stream) : hipErrorInvalidValue;
    case 128: return rows == 256 ? launch<128, 8>(p, stream) : rows == 128 ? launch<128, 4>(p, stream)
                                                                           : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango

namespace ditango {

hipError_t launch_step(StepParams& p, int rows, hipStream_t stream) {
  switch (p.d) {
    case 64: return rows == 128 ? launch_step_d<64, 4>(p, stream) : hipErrorInvalidValue;
    case 72: return rows == 128 ? launch_step_d<72, 4>(p, stream) : hipErrorInvalidValue;
    case 128: return rows == 256 ? launch_step_d<128, 8>(p, stream) : rows == 128 ? launch_step_d<128, 4>(p, stream)
                                                                                  : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_group_step(GroupStepParams& p, int rows, hipStream_t stream) {
  switch (p.d) {
    case 64: return rows == 128 ? launch_group_step_d<64, 4>(p, stream) : hipErrorInvalidValue;
    case 72: return rows == 128 ? launch_group_step_d<72, 4>(p, stream) : hipErrorInvalidValue;
    case 128: return rows == 256   ? launch_group_step_d<128, 8>(p, stream)
                     : rows == 128 ? launch_group_step_d<128, 4>(p, stream)
                                   : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ditango
