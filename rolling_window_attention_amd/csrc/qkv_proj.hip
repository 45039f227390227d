// Fused QKV projection for gfx950 (CDNA4), bf16 MFMA: y = x W^T for the
// layer input x [L][C] (C = H*D, token-major) and the weight W [3C][C] (q rows,
// then k rows, then v rows; feature h*D + d of a block is dimension d of head
// h), with an epilogue that writes the queries token-major and the keys and
// values straight into their ring slots: keys rotated by the 3D-RoPE
// (head-major [slot][h][n][d]), values transposed into 8-token blocks
// ([slot][h][n/8][d][8]).  The cache
// thus receives exactly what a roll of bf16 k and v would write, without k
// and v ever reaching memory as tensors of their own.
//
// Sources: every layer reads and writes a rolling KV cache and rotates its
// queries and keys over time, height and width ("Amazon and Reactor tune
// Trainium for real-time video generation", section "Three problems for
// generic compilers"); the layer attends over 12 heads (ai4snews digest,
// second paragraph).  The projection itself is the standard one of
// multi-head self-attention; the pages do not print it.
//
// Tiling.  A work-group computes a 256-token x 256-feature tile over the whole
// reduction (C = 1,536: 24 steps of 64), eight waves of 128 x 64 each (two per
// SIMD), 8 accumulator blocks of 32 x 32 per wave (v_mfma_f32_32x32x16_bf16).
// Both operand tiles (256 rows x 64 k of x and of W, k contiguous) are staged
// through LDS in two buffers: the next step's global loads are issued during
// the current step's first MFMAs and written to the other buffer during its
// last ones, and each substep's MFMAs run while the next substep's fragments are
// read, in an order fixed with scheduling groups.  The product is computed
// transposed for q and k tiles (A = W, B = x: a lane ends with 4 consecutive
// features of one token, i.e. two rotation pairs) and plainly for v tiles
// (A = x, B = W: 4 consecutive tokens of one feature, the order of a value row
// in the ring).  Either way the epilogue writes the accumulators as bf16 into an
// LDS image whose rows are the B-side index, and copies it out in 16-byte
// chunks with non-temporal stores: token rows of 256 features for q and k (k
// rotated on the way, with the roll's arithmetic), feature rows of 256 tokens
// for v.  One persistent work-group per CU walks the tiles, and puts the next
// tile's first loads in flight before its epilogue.  Tiles are numbered in groups
// of kGroupM token tiles x all feature tiles, token tile fastest (tile_ref), and
// dealt XCD-contiguously, so the work-groups of one XCD share a few token and
// weight panels in its L2 at every reduction step.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"


namespace rfattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Eight waves (two per SIMD) of 128 x 64: four waves of 128 x 128 (one per SIMD)
// fill all 256 accumulation registers of a wave and ran slower.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;               // tokens and features per tile
constexpr int kBW = kTile / (kWaves / 2);  // B-side columns per wave: 128 or 64
constexpr int kNB = kBW / 32;            // B-side 32-blocks per wave
constexpr int kSRows = kThreads / 8;     // operand rows staged per pass (8 chunks of 16 B a row)
constexpr int kSPass = kTile / kSRows;   // staging passes per operand tile
constexpr int kStepK = 64;               // reduction per staged step
constexpr int kSRow = kStepK + 8;        // LDS row stride of a staged operand (144 B)
constexpr int kSTile = kTile * kSRow;    // elements of one staged operand tile
constexpr int kORow = kTile + 8;         // LDS row stride of the output image (528 B)
constexpr size_t kLds = 2 * 2 * kSTile * sizeof(uint16_t);  // 2 buffers x (x, W)
static_assert((size_t)kTile * kORow * sizeof(uint16_t) <= kLds, "output image fits the staging buffers");
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Output stores: non-temporal (the outputs are not read again by this kernel;
// measured 6-10% faster than ordinary stores for the whole kernel).
__device__ __forceinline__ void out_store(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Work-group id -> tile index, each XCD walking a contiguous run (a bijection).
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int x = bid % kXcds, idx = bid / kXcds;
  if (rem == 0 || x < rem) return x * per + idx;
  return rem * per + (x - rem) * (per - 1) + idx;
}

}  // namespace

// A tile's coordinates and operand buffers.
struct TileRef {
  int part;      // 0: q, 1: k, 2: v (uniform)
  int fl0;       // first feature inside the part
  int m0;        // first token
  int rows_x;    // valid tokens
  int rows_w;    // valid features
  __amdgpu_buffer_rsrc_t xrs, wrs;  // rows past the valid ones read 0
};

// Tiles are numbered in groups of kGroupM token tiles x all feature tiles, token
// tile fastest inside a group: the 32 work-groups of an XCD (consecutive numbers)
// then share about 8 token panels and 4 feature panels at each reduction step
// instead of 2 and 18, so more of their operand reads hit the XCD's L2.  (Group
// sizes 2, 4, 8, 16 measured; 8 was fastest.)
constexpr int kGroupM = 8;

__device__ __forceinline__ TileRef tile_ref(const ProjArgs& a, int tile) {
  TileRef t;
  const int m_tiles = a.n_tiles / a.f_tiles;
  const int group = tile / (kGroupM * a.f_tiles);
  const int in_group = tile - group * (kGroupM * a.f_tiles);
  const int gm = min(kGroupM, m_tiles - group * kGroupM);  // token tiles in this group
  const int ft = in_group / gm;
  const int mt = group * kGroupM + (in_group - ft * gm);
  t.part = ft / a.tiles_per_part;
  t.fl0 = (ft - t.part * a.tiles_per_part) * kTile;
  t.m0 = mt * kTile;
  t.rows_x = min(kTile, a.M - t.m0);
  t.rows_w = min(kTile, a.C - t.fl0);
  t.xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x + (int64_t)t.m0 * a.x_ld), 0,
                                            (int)((uint32_t)t.rows_x * (uint32_t)a.x_ld * 2u), kBufferWord3);
  t.wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.w + ((int64_t)t.part * a.C + t.fl0) * a.w_ld),
                                            0, (int)((uint32_t)t.rows_w * (uint32_t)a.w_ld * 2u), kBufferWord3);
  return t;
}

// Step kt's operand rows of tile t into registers: thread -> rows (tid >> 3) +
// kSRows i, 16-byte chunk tid & 7 of the step's 64 k.  The whole offset goes in
// the vector operand: the buffer's range check (which turns rows past the valid
// ones into zeros) does not include the scalar offset.
__device__ __forceinline__ void load_step(const ProjArgs& a, const TileRef& t, int kt, u32x4 (&xs)[kSPass],
                                          u32x4 (&ws)[kSPass]) {
  const int srow = threadIdx.x >> 3, schunk = threadIdx.x & 7;
  const uint32_t x_lane = (uint32_t)srow * (uint32_t)a.x_ld * 2u + 16u * schunk + (uint32_t)kt * 128u;
  const uint32_t w_lane = (uint32_t)srow * (uint32_t)a.w_ld * 2u + 16u * schunk + (uint32_t)kt * 128u;
  const uint32_t x_rows = (uint32_t)kSRows * (uint32_t)a.x_ld * 2u, w_rows = (uint32_t)kSRows * (uint32_t)a.w_ld * 2u;
#pragma unroll
  for (int i = 0; i < kSPass; ++i) {
    xs[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(t.xrs, x_lane + (uint32_t)i * x_rows, 0, 0));
    ws[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(t.wrs, w_lane + (uint32_t)i * w_rows, 0, 0));
  }
}

// One 256 x 256 output tile whose first step is already in xs/ws: main loop, then
// (with the next tile's first step put in flight in xs/ws, if there is one) the
// epilogue through LDS.
__device__ __forceinline__ void proj_tile(const ProjArgs& a, uint16_t* lds, const TileRef& t, bool has_next,
                                          const TileRef& next, u32x4 (&xs)[kSPass], u32x4 (&ws)[kSPass]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int hf = lane >> 5;
  const int wa = wave & 1, wb = wave >> 1;  // wave's 128-row A block and kBW-column B block
  const int part = t.part, fl0 = t.fl0, m0 = t.m0, rows_x = t.rows_x, rows_w = t.rows_w;
  const bool is_v = part == 2;
  const int srow = tid >> 3, schunk = tid & 7;
  auto stage = [&](int buf) {
    uint16_t* X = lds + buf * 2 * kSTile;
    uint16_t* Wt = X + kSTile;
#pragma unroll
    for (int i = 0; i < kSPass; ++i) {
      *(u32x4*)(X + (srow + kSRows * i) * kSRow + 8 * schunk) = xs[i];
      *(u32x4*)(Wt + (srow + kSRows * i) * kSRow + 8 * schunk) = ws[i];
    }
  };

  f32x16 acc[4][kNB];
#pragma unroll
  for (int ia = 0; ia < 4; ++ia)
#pragma unroll
    for (int ib = 0; ib < kNB; ++ib) acc[ia][ib] = f32x16{};

  const int nk = a.C / kStepK;
  stage(0);
  __syncthreads();
  // One reduction step on LDS buffer kt & 1; with `more`, the next step's global
  // loads are issued during the first substep's MFMAs and staged into the other
  // buffer during the last one.  Each substep's MFMAs run while the next
  // substep's fragments are read.  The interleave is fixed with scheduling
  // groups: one fragment read, global load or staging write after each MFMA
  // (left to the compiler, the reads sat right before their MFMAs: 4% slower).
  auto kstep = [&](int kt, auto more) {
    constexpr bool kMore = decltype(more)::value;
    constexpr int kSub = kStepK / 16;
    constexpr int kMf = 4 * kNB;        // MFMAs per substep
    constexpr int kRd = 4 + kNB;        // fragment reads per substep
    constexpr int kVm = 2 * kSPass;     // global loads (and staging writes) per step
    if constexpr (kMore) load_step(a, t, kt + 1, xs, ws);
    const uint16_t* X = lds + (kt & 1) * 2 * kSTile;
    const uint16_t* At = is_v ? X : X + kSTile;
    const uint16_t* Bt = is_v ? X + kSTile : X;
    bf16x8 af[2][4], bfr[2][kNB];
    auto frags = [&](int set, int s) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[set][i] = *(const bf16x8*)(At + (128 * wa + 32 * i + lr) * kSRow + 16 * s + 8 * hf);
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        bfr[set][i] = *(const bf16x8*)(Bt + (kBW * wb + 32 * i + lr) * kSRow + 16 * s + 8 * hf);
    };
    frags(0, 0);
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const int set = s & 1;
      if (s + 1 < kSub) frags(set ^ 1, s + 1);
#pragma unroll
      for (int ia = 0; ia < 4; ++ia)
#pragma unroll
        for (int ib = 0; ib < kNB; ++ib)
          acc[ia][ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][ia], bfr[set][ib], acc[ia][ib], 0, 0, 0);
    }
    if constexpr (kMore) stage((kt + 1) & 1);
    __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);  // substep 0's fragments first
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
#pragma unroll
      for (int i = 0; i < kMf; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA
        if (s + 1 < kSub && i < kRd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        if (kMore && s == 0 && i < kVm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        if (kMore && s == kSub - 1 && i < kVm) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
    }
  };
  for (int kt = 0; kt + 1 < nk; ++kt) {
    kstep(kt, std::true_type{});
    __syncthreads();
  }
  kstep(nk - 1, std::false_type{});
  __syncthreads();

  if (has_next) load_step(a, next, 0, xs, ws);  // in flight during the epilogue

  // ---- epilogue: bf16 image [B-side row][A-side column] in LDS ---------------------
  // Accumulator register 4 g + j of block (ia, ib) holds A-side row
  // 32 ia + 8 g + 4 hf + j and B-side column 32 ib + lr.
  uint16_t* T = lds;
#pragma unroll
  for (int ia = 0; ia < 4; ++ia)
#pragma unroll
    for (int ib = 0; ib < kNB; ++ib)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2(acc[ia][ib][4 * g + 0], acc[ia][ib][4 * g + 1]);
        w[1] = pack2(acc[ia][ib][4 * g + 2], acc[ia][ib][4 * g + 3]);
        *(u32x2*)(T + (kBW * wb + 32 * ib + lr) * kORow + 128 * wa + 32 * ia + 8 * g + 4 * hf) = w;
      }
  __syncthreads();

  const int N = a.N;
  const int64_t head_elems = (int64_t)N * kHeadDim;
  const int64_t sh = frame_shift(a.fs);
  int slot0 = a.slot0 + (int)(sh % a.W);
  if (slot0 >= a.W) slot0 -= a.W;
  if (part == 0) {
    // token rows: 32 chunks of 8 features each
    for (int idx = tid; idx < kTile * 32; idx += kThreads) {
      const int ml = idx >> 5, c = idx & 31;
      if (ml >= rows_x || 8 * c >= rows_w) continue;
      out_store((u32x4*)(a.q + (int64_t)(m0 + ml) * a.q_ld + fl0 + 8 * c), *(const u32x4*)(T + ml * kORow + 8 * c));
    }
  } else if (part == 1) {
    // token rows: a thread takes chunk column cc (pairs 4cc..4cc+3) of one token in
    // both heads of the tile, sharing the pairs' cos/sin
    for (int idx = tid; idx < kTile * 16; idx += kThreads) {
      const int ml = idx >> 4, cc = idx & 15;
      if (ml >= rows_x) continue;
      const int mg = m0 + ml;
      uint32_t pin, col;
      const uint32_t fr = small_div((uint32_t)mg, (uint32_t)N, a.inv_n, &pin);
      const uint32_t row = small_div(pin, (uint32_t)a.gw, a.inv_gw, &col);
      int slot = slot0 + (int)fr;
      if (slot >= a.W) slot -= a.W;  // slot0 < W and fr < W
      const ChunkCS cs = rope_chunk_cs_of(a.tab, 4 * cc, a.t0 + sh + fr, (int)row, (int)col);
      uint16_t* kdst = a.k_ring + (int64_t)slot * a.slot_elems + (int64_t)pin * kHeadDim + 8 * cc;
#pragma unroll
      for (int hh = 0; hh < kTile / kHeadDim; ++hh) {
        const int f = fl0 + hh * kHeadDim;  // first feature of the head inside the part
        if (hh * kHeadDim >= rows_w) break;
        const u32x4 v = *(const u32x4*)(T + ml * kORow + hh * kHeadDim + 8 * cc);
        out_store((u32x4*)(kdst + (f / kHeadDim) * head_elems), rope_chunk_cs(v, cs));
      }
    }
  } else {
    // 8-token chunks of feature rows (N % 8 == 0: a chunk stays in one frame) to the
    // ring's [h][n/8][d][8] blocks; consecutive threads take consecutive features of
    // one token group, so a wave writes 1 KB runs
    for (int idx = tid; idx < kTile * 32; idx += kThreads) {
      const int c = idx >> 8, fl = idx & (kTile - 1);
      if (fl >= rows_w || 8 * c >= rows_x) continue;
      const u32x4 v = *(const u32x4*)(T + fl * kORow + 8 * c);
      uint32_t n0;
      const uint32_t fr = small_div((uint32_t)(m0 + 8 * c), (uint32_t)N, a.inv_n, &n0);
      int slot = slot0 + (int)fr;
      if (slot >= a.W) slot -= a.W;
      const int f = fl0 + fl;
      const int h = f / kHeadDim, d = f - h * kHeadDim;
      out_store((u32x4*)(a.v_ring + (int64_t)slot * a.slot_elems + h * head_elems + (int64_t)(n0 / 8) * 1024 + d * 8),
                v);
    }
  }
}

// Persistent: one work-group per CU walks tiles i = blockIdx.x, + gridDim.x, ...;
// a tile's stores drain while the next tile computes.  Tile i goes to XCD i % 8
// with the grid a multiple of 8, and xcd_tile gives each XCD a contiguous run.
__global__ __launch_bounds__(kThreads, 1) void qkv_proj_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  int i = blockIdx.x;
  if (i >= a.n_tiles) return;
  u32x4 xs[kSPass], ws[kSPass];
  TileRef cur = tile_ref(a, xcd_tile(i, a.n_tiles));
  load_step(a, cur, 0, xs, ws);
  for (;;) {
    const int nxt = i + (int)gridDim.x;
    const bool has_next = nxt < a.n_tiles;
    const TileRef next = tile_ref(a, xcd_tile(has_next ? nxt : i, a.n_tiles));
    proj_tile(a, lds, cur, has_next, next, xs, ws);
    if (!has_next) break;
    __syncthreads();  // the LDS image is read out before the next tile stages into it
    i = nxt;
    cur = next;
  }
}

hipError_t prepare_qkv_proj() {
  return hipFuncSetAttribute((const void*)qkv_proj_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)kLds);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  if (a.n_tiles == 0) return hipSuccess;
  const int grid = min(a.n_tiles, a.n_workers);
  hipLaunchKernelGGL(qkv_proj_kernel, dim3((unsigned)grid), dim3(kThreads), kLds, s, a);
  return hipGetLastError();
}

}  // namespace rfattn
