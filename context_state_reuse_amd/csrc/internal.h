// Internal interface between the host half of the library (host.cpp) and the
// HIP kernels (partial.hip, merge.hip, stats.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ditango.h"

namespace ditango {

// Launch parameters of the fresh partial-attention kernel.  The work list
// travels in the kernel arguments (at most 32 x 32 items), so a launch needs
// no device-side work list and no allocation.
//
// Per-pair cache (grouped = 0): item = pair id q*P + k; the state goes to
// slot h*P*P + item of O/LSE ([H][P*P][S][d]).
// Grouped cache (grouped = 1): item = (q << 6) | s for slot s of query
// partition q; the keys are those of the slot's members (slot 0: partition
// q; slot 1 + j: group j of size g without q -- one contiguous range, or two
// when q sits strictly inside the group); the state goes to gO[s] / gLSE[s]
// at (h*P + q)*S.
struct PartialParams {
  const __bf16* Q;          // [H][N][d]
  const __bf16* K;          // [H][N][d]
  const __bf16* V;          // [H][N][d]
  void* O;                  // per-pair cache [H][P*P][S][d], fp32 or bf16 (state_bf16)
  float* LSE;               // per-pair cache [H][P*P][S]
  int32_t H, N, P, S, d;
  int32_t state_bf16;       // cached OUT in bf16 (1) or fp32 (0)
  float scale_log2;         // scale * log2(e): scores in base-2 units
  int32_t n_pairs;          // work items in `pairs`
  int32_t q_tiles;          // query tiles per partition, ceil(S / rows per block)
  int32_t n_blocks;         // H * n_pairs * q_tiles
  int32_t grouped;          // 0: per-pair cache, 1: grouped cache
  int32_t g;                // group size (grouped)
  void* gO[DITANGO_MAX_SLOTS];     // grouped: slot buffers [H][P][S][d]
  float* gLSE[DITANGO_MAX_SLOTS];  // grouped: [H][P][S]
  uint16_t pairs[DITANGO_MAX_P * DITANGO_MAX_P];  // work items (see above)
};

// Launch parameters of the fused step kernel (per-pair cache): one block per
// (head, query partition q, query-row tile).  The block computes the fresh
// pairs (q, fresh[q][i]), i < nf[q], one after the other over the same
// query rows, stores each state into its cache slot, and then composes
// (Eq. 4) the P states of its rows -- fresh and cached alike -- into the
// output O [H][N][d], LSE [H][N].
struct StepParams {
  const __bf16* Q;          // [H][N][d]
  const __bf16* K;
  const __bf16* V;
  void* O;                  // per-pair cache [H][P*P][S][d], fp32 or bf16 (state_bf16)
  float* LSE;               // per-pair cache [H][P*P][S]
  float* Oout;              // [H][N][d]
  float* LSEout;            // [H][N]
  int32_t H, N, P, S, d;
  int32_t state_bf16;
  float scale_log2;
  int32_t q_tiles;          // query tiles per partition
  int32_t n_blocks;         // H * P * q_tiles
  uint8_t nf[DITANGO_MAX_P];
  uint8_t fresh[DITANGO_MAX_P][DITANGO_MAX_P];
};

// Launch parameters of the fused step kernel of the grouped cache: one block
// per (head, query partition q, query-row tile) computes the COMPUTE slots
// cslot[q][0 .. nc[q]) one after the other (slot keys as in PartialParams'
// grouped items), stores each state into its slot buffer, then composes the
// live slots lslot[q][0 .. nl[q]) of its rows into O [H][N][d], LSE [H][N].
struct GroupStepParams {
  const __bf16* Q;          // [H][N][d]
  const __bf16* K;
  const __bf16* V;
  void* gO[DITANGO_MAX_SLOTS];     // slot buffers [H][P][S][d], fp32 or bf16 (state_bf16)
  float* gLSE[DITANGO_MAX_SLOTS];  // [H][P][S]
  float* Oout;              // [H][N][d]
  float* LSEout;            // [H][N]
  int32_t H, N, P, S, d, g;
  int32_t state_bf16;
  float scale_log2;
  int32_t q_tiles;          // query tiles per partition
  int32_t n_blocks;         // H * P * q_tiles
  uint8_t nc[DITANGO_MAX_P];
  uint8_t cslot[DITANGO_MAX_P][DITANGO_MAX_SLOTS];
  uint8_t nl[DITANGO_MAX_P];
  uint8_t lslot[DITANGO_MAX_P][DITANGO_MAX_SLOTS];
};

// Composition (Eq. 4) of n_in states per row.  State k of the rows of
// (head h, query partition q) starts at in_O[k] + (h*in_hs + q*in_qs)*S*d
// (LSE: in_L[k] + (h*in_hs + q*in_qs)*S); it takes part when bit k of
// live[q] is set.  Row r of (h, q) is written to O (or, for a group slot,
// Os in bf16) + (h*out_hs + q*out_qs + r)*d and LSE + h*out_hs + q*out_qs
// + r.  A (h, q) with no live state is
// skipped.  The row merge of both caches and the in-place group merge of
// the grouped cache are instances.
//
// Window attention with residual sharing (res_mode != 0; res laid out like
// O): res_mode 1 also writes res = OUT - (composition of the states in
// wlive[q]); res_mode 2 adds res to OUT.
struct MergeParams {
  const void* in_O[DITANGO_MAX_SLOTS];  // fp32 or bf16 (state_bf16)
  const float* in_L[DITANGO_MAX_SLOTS];
  uint32_t live[DITANGO_MAX_P];
  uint32_t wlive[DITANGO_MAX_P];
  // Filled by launch_merge from live/wlive: the live states of query
  // partition q as a list idx[q][0 .. cnt[q]), and the window bits over
  // that list, so a row's lanes cover only its live states.
  uint8_t idx[DITANGO_MAX_P][DITANGO_MAX_SLOTS];
  uint8_t cnt[DITANGO_MAX_P];
  uint32_t wpos[DITANGO_MAX_P];
  int64_t in_hs, in_qs;     // in units of S rows
  int64_t out_hs, out_qs;   // in rows
  float* O;                 // fp32 output rows, or
  void* Os;                 // output rows in the states' format (a group slot) when not null
  float* LSE;
  float* res;
  int32_t res_mode;
  int32_t state_bf16;       // the states (and Os) hold OUT in bf16 (1) or fp32 (0)
  int32_t n_in;             // <= DITANGO_MAX_SLOTS
  int32_t H, N, P, S, d;
};

// Per-pair statistics of the per-pair cache for the anchor-guided planner:
// for every pair (q, k) and head h, W[h][q][k] = mean over q's rows r of
// exp(LSE_slot[r] - LSE[q*S + r]); for the pairs with bit k of sel[q] set,
// SIG[h][q][k][0..d) = mean over q's rows of OUT_slot.
// W == nullptr: importance not wanted; the grid then covers the selected
// pairs only, listed in pairs[0 .. n_pairs).
struct StatsParams {
  const void* O;            // per-pair cache [H][P*P][S][d], fp32 or bf16 (state_bf16)
  int32_t state_bf16;
  const float* LSE_slot;    // [H][P*P][S]
  const float* LSE;         // merged [H][N]
  float* W;                 // [H][P][P] or nullptr
  float* SIG;               // [H][P][P][d]
  uint32_t sel[DITANGO_MAX_P];
  int32_t H, N, P, S, d;
  int32_t n_pairs;
  uint16_t pairs[DITANGO_MAX_P * DITANGO_MAX_P];
};

// Drift of pair signatures between two tables A and B ([H][P][P][d]): for
// the listed pairs, out[q*P + k] = ||A - B|| / ||B|| over the pair's heads
// and dims (0 when both are 0, +inf when only B is).
struct DriftParams {
  const float* A;
  const float* B;
  float* out;               // [P][P]
  int32_t H, P, d;
  int32_t n_pairs;
  uint16_t pairs[DITANGO_MAX_P * DITANGO_MAX_P];
};

// Query rows handled by one block of the partial kernel for head dim d
// (chosen by the launcher); the host uses it to size the grid.
int partial_rows_per_block(int d, int S);

// Enqueue kernels; return hipSuccess or the launch error.
hipError_t launch_partial(PartialParams& p, int rows_per_block, hipStream_t stream);
hipError_t launch_step(StepParams& p, int rows_per_block, hipStream_t stream);
hipError_t launch_group_step(GroupStepParams& p, int rows_per_block, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_stats(const StatsParams& p, hipStream_t stream);
hipError_t launch_drift(const DriftParams& p, hipStream_t stream);

}  // namespace ditango
