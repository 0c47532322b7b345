// Internal interface of the bookkeeping kernels (lite_attn_aux.hip) used by the C-ABI host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lite_attn {

// Zero `words` uint32 words with a fill kernel (no memset node, so it may be captured).
hipError_t launch_mask_fill_zero(uint32_t* mask, size_t words, hipStream_t stream);

// Schedule of the query tiles of a step from their visit counts (heavy tiles first, then heads by
// decreasing work, each in traversal direction, then at most min(tail_max, non-heavy / 4) short
// tiles in traversal order): the workspace receives the queue position -> tile permutation
// (n_tiles uint32 at offset 0) and the per-tile counts after it.
size_t plan_workspace_bytes(int64_t n_tiles);
hipError_t launch_plan(const uint32_t* mask, int n_tiles, int Tq, int W, int Tk, int descending,
                       int tail_max, void* workspace, hipStream_t stream);
// counts[x] = set valid bits of the Tq * W mask words of head x (x < heads_total).
hipError_t launch_mask_popcount(const uint32_t* mask, uint32_t* counts, int heads_total,
                                int Tq, int Tk, int W, hipStream_t stream);

// *result = max |a - b| over the valid elements of two [B][H][N][D] tensors with element strides
// (sb, sh, sn), in fp32, NaN when any difference is NaN, 0 for an empty shape. Both pointers
// 16-byte aligned, strides multiples of 8 elements.
hipError_t launch_output_max_abs_diff(const void* a, const void* b, bool bf16, int B, int H,
                                      int N, int D, int64_t sb, int64_t sh, int64_t sn,
                                      float* result, hipStream_t stream);

}  // namespace lite_attn
