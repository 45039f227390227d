// Fused QKV projection for gfx950 (CDNA4), bf16 MFMA: y = x W^T for the
// layer input x [L][C] (C = H*D, token-major) and the weight W [3C][C] (q rows,
// then k rows, then v rows; feature h*D + d of a block is dimension d of head
// h), with an epilogue that writes the queries token-major and the keys and
// values straight into their ring slots: keys rotated by the 3D-RoPE
// (head-major [slot][h][n][d]), values transposed ([slot][h][d][n]).  The cache
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
// reduction (C = 1,536: 24 steps of 64), four waves of 128 x 128 each, 16
// accumulator blocks of 32 x 32 per wave (v_mfma_f32_32x32x16_bf16).  Both
// operand tiles (256 rows x 64 k of x and of W, k contiguous) are staged
// through LDS in two buffers: the next step's global loads are issued before
// the current step's MFMAs and written to the other buffer after them.  The
// product is computed transposed for q and k tiles (A = W, B = x: a lane ends
// with 4 consecutive features of one token, i.e. two rotation pairs) and
// plainly for v tiles (A = x, B = W: 4 consecutive tokens of one feature, the
// order of a value row in the ring).  Either way the epilogue writes the
// accumulators as bf16 into an LDS image whose rows are the B-side index, and
// copies it out in 16-byte chunks: token rows of 256 features for q and k (k
// rotated on the way, with the roll's arithmetic), feature rows of 256 tokens
// for v.  Tiles are numbered so that each XCD walks consecutive feature tiles
// of one token tile (x rows reused from L2).
#include "device_common.h"
#include "kernels.h"

namespace rfattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 256;               // tokens and features per tile
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

// Work-group id -> tile index, each XCD walking a contiguous run (a bijection).
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int x = bid % kXcds, idx = bid / kXcds;
  if (rem == 0 || x < rem) return x * per + idx;
  return rem * per + (x - rem) * (per - 1) + idx;
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void qkv_proj_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int hf = lane >> 5;
  const int wa = wave & 1, wb = wave >> 1;  // wave's 128-row block of the A and B sides

  const int tile = xcd_tile(blockIdx.x, a.n_tiles);
  const int mt = tile / a.f_tiles;
  const int ft = tile - mt * a.f_tiles;
  const int part = ft / a.tiles_per_part;   // 0: q, 1: k, 2: v (wave-uniform)
  const int fl0 = (ft - part * a.tiles_per_part) * kTile;  // first feature inside the part
  const int m0 = mt * kTile;
  const int rows_x = min(kTile, a.M - m0);   // valid tokens of the tile
  const int rows_w = min(kTile, a.C - fl0);  // valid features of the tile
  const bool is_v = part == 2;

  // operand tiles through raw buffer loads: rows past the valid ones read 0
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x + (int64_t)m0 * a.x_ld), 0, (int)((uint32_t)rows_x * (uint32_t)a.x_ld * 2u),
      kBufferWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w + ((int64_t)part * a.C + fl0) * a.w_ld), 0,
      (int)((uint32_t)rows_w * (uint32_t)a.w_ld * 2u), kBufferWord3);
  // thread -> rows (tid >> 3) + 32 i, 16-byte chunk tid & 7 of the step's 64 k
  const int srow = tid >> 3, schunk = tid & 7;
  const uint32_t x_lane = (uint32_t)srow * (uint32_t)a.x_ld * 2u + 16u * schunk;
  const uint32_t w_lane = (uint32_t)srow * (uint32_t)a.w_ld * 2u + 16u * schunk;
  const uint32_t x_row32 = 32u * (uint32_t)a.x_ld * 2u, w_row32 = 32u * (uint32_t)a.w_ld * 2u;
  u32x4 xs[8], ws[8];
  // The whole offset goes in the vector operand: the buffer's range check (which
  // turns rows past the valid ones into zeros) does not include the scalar offset.
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xrs, x_lane + (uint32_t)i * x_row32 + (uint32_t)kt * 128u, 0, 0));
      ws[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            wrs, w_lane + (uint32_t)i * w_row32 + (uint32_t)kt * 128u, 0, 0));
    }
  };
  auto stage = [&](int buf) {
    uint16_t* X = lds + buf * 2 * kSTile;
    uint16_t* Wt = X + kSTile;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(u32x4*)(X + (srow + 32 * i) * kSRow + 8 * schunk) = xs[i];
      *(u32x4*)(Wt + (srow + 32 * i) * kSRow + 8 * schunk) = ws[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int ia = 0; ia < 4; ++ia)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) acc[ia][ib] = f32x16{};

  const int nk = a.C / kStepK;
  load(0);
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const uint16_t* X = lds + (kt & 1) * 2 * kSTile;
    const uint16_t* At = is_v ? X : X + kSTile;
    const uint16_t* Bt = is_v ? X + kSTile : X;
#pragma unroll
    for (int s = 0; s < kStepK / 16; ++s) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *(const bf16x8*)(At + (128 * wa + 32 * i + lr) * kSRow + 16 * s + 8 * hf);
        bfr[i] = *(const bf16x8*)(Bt + (128 * wb + 32 * i + lr) * kSRow + 16 * s + 8 * hf);
      }
#pragma unroll
      for (int ia = 0; ia < 4; ++ia)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          acc[ia][ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ia], bfr[ib], acc[ia][ib], 0, 0, 0);
    }
    if (kt + 1 < nk) stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: bf16 image [B-side row][A-side column] in LDS ---------------------
  // Accumulator register 4 g + j of block (ia, ib) holds A-side row
  // 32 ia + 8 g + 4 hf + j and B-side column 32 ib + lr.
  uint16_t* T = lds;
#pragma unroll
  for (int ia = 0; ia < 4; ++ia)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack2(acc[ia][ib][4 * g + 0], acc[ia][ib][4 * g + 1]);
        w[1] = pack2(acc[ia][ib][4 * g + 2], acc[ia][ib][4 * g + 3]);
        *(u32x2*)(T + (128 * wb + 32 * ib + lr) * kORow + 128 * wa + 32 * ia + 8 * g + 4 * hf) = w;
      }
  __syncthreads();

  const int N = a.N;
  const int64_t head_elems = (int64_t)N * kHeadDim;
  if (!is_v) {
    // token rows: 32 chunks of 8 features each
    for (int idx = tid; idx < kTile * 32; idx += kThreads) {
      const int ml = idx >> 5, c = idx & 31;
      if (ml >= rows_x || 8 * c >= rows_w) continue;
      const u32x4 v = *(const u32x4*)(T + ml * kORow + 8 * c);
      const int mg = m0 + ml;
      const int f = fl0 + 8 * c;  // feature inside the part
      if (part == 0) {
        *(u32x4*)(a.q + (int64_t)mg * a.q_ld + f) = v;
      } else {
        uint32_t pin, col;
        const uint32_t fr = small_div((uint32_t)mg, (uint32_t)N, a.inv_n, &pin);
        const uint32_t row = small_div(pin, (uint32_t)a.gw, a.inv_gw, &col);
        int slot = a.slot0 + (int)fr;
        if (slot >= a.W) slot -= a.W;  // slot0 < W and fr < W
        const int h = f / kHeadDim, d = f - h * kHeadDim;
        const ChunkCS cs = rope_chunk_cs_of(a.tab, d / 2, a.t0 + fr, (int)row, (int)col);
        *(u32x4*)(a.k_ring + (int64_t)slot * a.slot_elems + h * head_elems + (int64_t)pin * kHeadDim + d) =
            rope_chunk_cs(v, cs);
      }
    }
  } else {
    // feature rows: 32 chunks of 8 tokens each (N % 8 == 0: a chunk stays in one frame)
    for (int idx = tid; idx < kTile * 32; idx += kThreads) {
      const int fl = idx >> 5, c = idx & 31;
      if (fl >= rows_w || 8 * c >= rows_x) continue;
      const u32x4 v = *(const u32x4*)(T + fl * kORow + 8 * c);
      uint32_t n0;
      const uint32_t fr = small_div((uint32_t)(m0 + 8 * c), (uint32_t)N, a.inv_n, &n0);
      int slot = a.slot0 + (int)fr;
      if (slot >= a.W) slot -= a.W;
      const int f = fl0 + fl;
      const int h = f / kHeadDim, d = f - h * kHeadDim;
      *(u32x4*)(a.v_ring + (int64_t)slot * a.slot_elems + h * head_elems + (int64_t)d * N + n0) = v;
    }
  }
}

hipError_t prepare_qkv_proj() {
  return hipFuncSetAttribute((const void*)qkv_proj_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)kLds);
}

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  if (a.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_proj_kernel, dim3((unsigned)a.n_tiles), dim3(kThreads), kLds, s, a);
  return hipGetLastError();
}

}  // namespace rfattn
