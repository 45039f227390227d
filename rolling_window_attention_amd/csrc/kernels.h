// Kernel argument blocks and launchers of librfattn (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace rfattn {

constexpr int kHeadDim = 128;
constexpr int kMaxSegments = 8;

struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  int64_t x_ld, y_ld;
  int64_t t0, n_tokens;
  int N, gw, H;
  RopeTables tab;
};

struct RollArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t k_ld, v_ld;
  uint16_t* k_ring;      // [W][H][N][D]
  uint16_t* v_ring;      // [W][H][D][N]
  int64_t slot_elems;    // H*N*D
  int64_t t0;            // first new frame
  int slot0;             // t0 % W
  int n_frames, W, N, gw, H;
  RopeTables tab;
};

struct SegDev {
  const uint16_t* q;
  uint16_t* o;
  int64_t q_ld, o_ld;
  int64_t q_t0;          // frame of the first query token
  int q_tokens;          // q_frames * N
  int q_tiles;           // ceil(q_tokens / kBlockM)
  int tile_begin;        // first work-group id of this segment
  int ctx_keys;          // ctx_frames * N
  int ctx_slot0;         // ring slot of the first context frame
};

struct AttnArgs {
  SegDev seg[kMaxSegments];
  int n_segs;
  int total_tiles;
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  int64_t slot_elems;
  int W, N, gw, H;
  float c_log2;          // scale * log2(e)
  RopeTables tab;
};

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s);
hipError_t launch_roll(const RollArgs& a, hipStream_t s);
hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s);
hipError_t prepare_window_attn();  // once per device, before the first launch
int window_attn_block_m();

}  // namespace rfattn
