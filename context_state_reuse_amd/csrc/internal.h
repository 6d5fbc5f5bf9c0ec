// Internal interface between the host half of the library (host.cpp) and the
// HIP kernels (partial.hip, merge.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ditango.h"

namespace ditango {

// Launch parameters of the fresh partial-attention kernel.  The fresh-pair
// list travels in the kernel arguments (at most 32 x 32 pairs), so a launch
// needs no device-side work list and no allocation.
struct PartialParams {
  const __bf16* Q;          // [H][N][d]
  const __bf16* K;          // [H][N][d]
  const __bf16* V;          // [H][N][d]
  float* O;                 // cache [H][P*P][S][d]
  float* LSE;               // cache [H][P*P][S]
  int32_t H, N, P, S, d;
  float scale_log2;         // scale * log2(e): scores in base-2 units
  int32_t n_pairs;          // fresh pairs in `pairs`
  int32_t q_tiles;          // query tiles per partition, ceil(S / rows per block)
  int32_t n_blocks;         // H * n_pairs * q_tiles
  uint16_t pairs[DITANGO_MAX_P * DITANGO_MAX_P];  // pair ids q*P+k, grouped by k
};

struct MergeParams {
  const float* Os;          // cache [H][P*P][S][d]
  const float* LSEs;        // cache [H][P*P][S]
  float* O;                 // [H][N][d]
  float* LSE;               // [H][N]
  int32_t H, N, P, S, d;
};

// Query rows handled by one block of the partial kernel for head dim d
// (chosen by the launcher); the host uses it to size the grid.
int partial_rows_per_block(int d, int S);

// Enqueue kernels; return hipSuccess or the launch error.
hipError_t launch_partial(PartialParams& p, int rows_per_block, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

}  // namespace ditango
