// Kernel argument blocks and launchers of librfattn (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace rfattn {

constexpr int kHeadDim = 128;
constexpr int kMaxSegments = 8;
constexpr int kAttnBlockM = 256;   // query rows per attention work item
constexpr int kAttnBlockN = 64;    // keys per key tile (one work unit per key tile)
constexpr int kWorkersPerCu = 1;   // persistent attention work-groups per CU
// One partial result of a split query tile: unnormalised O as [head_dim / 8][rows][8]
// (dims 8c .. 8c+7 of every row in chunk c), then m [rows], l [rows].
constexpr int kPartRows = kAttnBlockM;
constexpr int kPartFloats = kPartRows * kHeadDim + 2 * kPartRows;

// Frame shift of a steady-state step replayed from a graph: *p (device memory,
// read when the kernel runs) clamped to [0, max], added to every absolute frame
// index of the launch (RoPE positions, ring slots); 0 when p is null.
struct FrameShift {
  const int64_t* p;
  int64_t max;
};
__device__ __forceinline__ int64_t frame_shift(const FrameShift& s) {
  if (!s.p) return 0;
  const int64_t v = *s.p;
  return v < 0 ? 0 : (v > s.max ? s.max : v);
}

// A ring descriptor in device memory (rf_kvcache_dev of the C ABI): the
// buffers and capacity are written by the upload kernel only, the window
// (first, count) also by the rolls that use the descriptor.
struct DevRing {
  uint16_t* k;       // [W][H][N][D]
  uint16_t* v;       // [W][H][N/8][D][8]
  int64_t first;
  int32_t count;
  int32_t capacity;  // W
};
static_assert(sizeof(DevRing) == 32, "rf_kvcache_dev layout");

__device__ __forceinline__ int64_t mod_pos(int64_t a, int64_t m) {
  const int64_t r = a % m;
  return r < 0 ? r + m : r;
}

struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  int64_t x_ld, y_ld;
  int64_t t0, n_tokens;
  int N, gw, H;
  RopeTables tab;
  FrameShift fs;
};

struct RollArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t k_ld, v_ld;
  int64_t k_layer_stride, v_layer_stride;  // elements between layers' inputs (grid.y = layer)
  DevRing* rings;        // per-layer device descriptors (NULL: the one ring below)
  uint16_t* k_ring;      // [W][H][N][D]
  uint16_t* v_ring;      // [W][H][N/8][D][8]
  int64_t slot_elems;    // H*N*D
  int64_t t0;            // first new frame
  int slot0;             // t0 % W
  int n_frames, W, N, gw, H;
  int n_layers;          // rings written by one launch (grid.y); 1 without descriptors
  RopeTables tab;
  FrameShift fs;
};

struct SegDev {
  const uint16_t* q;
  uint16_t* o;
  int64_t q_ld, o_ld;
  int64_t q_t0;          // frame of the first query token
  int q_tok0;            // the first query token's index inside frame q_t0
  int q_tokens;          // query tokens (rows of q and o)
  int q_tiles;           // ceil(q_tokens / kAttnBlockM)
  int ctx_keys;          // ctx_frames * N
  int ctx_slot0;         // ring slot of the first context frame
  int64_t ctx_t0;        // the first context frame (for keys rotated on load)
  int key_tiles;         // ceil(ctx_keys / kAttnBlockN)
  int tile_begin;        // first query tile of this segment (over all segments)
};

struct AttnArgs {
  SegDev seg[kMaxSegments];
  int n_segs;
  int total_tiles;       // sum over segments of heads * q_tiles
  int dp_tiles;          // tiles run whole, one work-group each (full rounds)
  int split_tiles;       // the remaining tiles (total_tiles - dp_tiles), each cut into
  int n_split;           // n_split equal key ranges (pieces), one work-group per piece
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  int64_t slot_elems;
  int W, N, gw, H;
  float c_log2;          // scale * log2(e)
  float* partial;        // workspace: split_tiles * n_split partial results of kPartFloats
  // Window mode (non-NULL): the ring's buffers and window come from this device
  // descriptor when the kernels run, and every segment attends over the whole
  // window (per-segment context fields are then derived on the device).
  const DevRing* ring_dev;
  int rot_k;             // measurement variant: the ring holds un-rotated keys, rotated per K tile on load
  RopeTables tab;
  FrameShift fs;
};

// Fused QKV projection: y = x W^T, q token-major, k rotated into K ring slots,
// v transposed into V ring slots (tiles of 256 tokens x 256 features; each of
// q, k, v has tiles_per_part = ceil(C / 256) feature tiles).
struct ProjArgs {
  const uint16_t* x;     // [M][x_ld], M = n_frames * N tokens of frames t0..
  const uint16_t* w;     // [3C][w_ld]
  uint16_t* q;           // [M][q_ld]
  uint16_t* k_ring;      // [W][H][N][D]
  uint16_t* v_ring;      // [W][H][N/8][D][8]
  int64_t x_ld, w_ld, q_ld;
  int64_t slot_elems;    // H*N*D
  int64_t t0;            // frame of token 0
  int M, C, N, gw, W, slot0;
  int n_tiles, f_tiles, tiles_per_part;
  int n_workers;         // persistent work-groups: one per CU, a multiple of 8
  float inv_n, inv_gw;   // 1/N, 1/gw for the exact small divisions
  RopeTables tab;
  FrameShift fs;
};

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s);
hipError_t launch_roll(const RollArgs& a, hipStream_t s);
hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s);
hipError_t prepare_window_attn();  // once per device, before the first launch
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s);
hipError_t prepare_qkv_proj();     // once per device, before the first launch
hipError_t launch_add_shift(int64_t* p, int64_t delta, hipStream_t s);
// Write n <= kUploadMax descriptors into device memory (a kernel: stream-ordered, capturable).
constexpr int kUploadMax = 32;
struct UploadArgs {
  DevRing d[kUploadMax];
  int n;
};
hipError_t launch_upload_rings(DevRing* dst, const UploadArgs& a, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, uint64_t bytes, hipStream_t s);

}  // namespace rfattn
