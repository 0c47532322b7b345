// Internal interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lite_attn {

constexpr int kTileK = 64;          // keys per tile (two 32-key MFMA blocks)
constexpr int kMaxTilesK = 2048;    // visiting list capacity per query tile (LDS)
constexpr int kMaxWords = kMaxTilesK / 32;
// Tile queues per device for persistent launches: the first kEagerQueueSlots go to streams
// (one per stream), the rest to launches captured into graphs (one per captured launch).
constexpr int kQueueSlots = 4096;
constexpr int kEagerQueueSlots = 64;

// Everything one forward launch needs. Strides are in elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  uint32_t* mask;
  int64_t sb, sh, sn;
  int B, H, N;
  int Tq, Tk, W;
  float scale;        // softmax scale (natural-log units)
  float scale_log2;   // scale * log2(e), for exp2-based softmax
  float log_eps;      // QK-Skip budget in natural-log units (may be -inf)
  int descending;     // traversal direction of this step
  int dense_prefix;   // tokens [0, dense_prefix) are exempt from flagging
  const uint32_t* perm;   // block -> query tile (B*H*Tq entries), or nullptr for the identity
  float* stats;           // divergence-refresh references (B*H*Tq), or nullptr: no refresh
  float refresh_delta;    // largest move of the statistic that keeps a mask row
  // Persistent launch: a tile queue (two uint32: next tile, finished workgroups; both zero
  // between launches) and the device's compute-unit count, which sizes the grid. With
  // queue == nullptr every workgroup takes the one tile of its block index.
  uint32_t* queue;
  int n_cu;
};

// Launches the attention kernel; *grid receives the number of workgroups launched.
using FwdLauncher = hipError_t (*)(const FwdParams&, hipStream_t, unsigned* grid);

// Launcher for (dtype, head_dim, tile_q, in-step skip) or nullptr when no kernel is built for
// it. dtype: 0 = bf16, 1 = fp32.
FwdLauncher get_fwd_launcher(int dtype, int head_dim, int tile_q, bool in_step_skip);

// Device address of tile queue `slot` (0 <= slot < kQueueSlots) on the current device.
hipError_t tile_queue_address(int slot, uint32_t** out);

}  // namespace lite_attn
