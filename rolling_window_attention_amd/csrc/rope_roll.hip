// Bandwidth-bound kernels of librfattn (gfx950):
//   rope3d_kernel  -- 3D-RoPE of a token-major bf16 tensor;
//   roll_kernel    -- one-pass KV-cache roll: RoPE'd keys to head-major ring
//                     slots, values transposed into 8-token blocks
//                     [head][token/8][dim][8] of their slots.
//
// Sources: 3D-RoPE over time/height/width and the per-layer rolling KV cache
// ("Amazon and Reactor tune Trainium for real-time video generation",
// section "Three problems for generic compilers"); the pages report
// hand-written kernels for both (section "Results with the Neuron Kernel
// Interface") and no standalone transposes (vibeleaderboard digest, key
// takeaways).
#include "device_common.h"
#include "kernels.h"


namespace rfattn {

// Both kernels rotate 16-byte chunks (8 bf16, 4 rotation pairs).  A thread owns
// one chunk column c (pairs 4c..4c+3) of one token and a group of kRopeHpt of the
// token's heads: the pairs' (cos, sin), their table lookups and float64 widening
// are shared by the group, which leaves the rotation itself as the thread's
// arithmetic.  A work-group is 16 (token, head group) rows x 16 columns, so each
// load or store instruction of a wave covers four 256-byte head rows.  Three
// heads per thread with all three loads in flight measured fastest: more heads
// per thread leave too few threads, fewer repeat the shared work.

// (frame offset, row, column) of token `tok` of a range whose token 0 starts
// frame 0; frames have N tokens of gw columns.
struct TokPos {
  uint32_t f, row, col;
};
__device__ __forceinline__ TokPos tok_pos(uint32_t tok, uint32_t N, float inv_n, uint32_t gw, float inv_gw) {
  uint32_t pin, col;
  const uint32_t f = small_div(tok, N, inv_n, &pin);
  const uint32_t row = small_div(pin, gw, inv_gw, &col);
  return {f, row, col};
}

constexpr int kRopeThreads = 256;
constexpr int kRopeRows = kRopeThreads / 16;     // (token, head group) rows per work-group
constexpr int kRopeHpt = 3;                      // heads per thread (a head group)
constexpr int kRopeBatch = 3;                    // head chunks loaded before the first is rotated

// Row R of the [tokens][head groups] grid -> token and the group's first head.
__device__ __forceinline__ void rope_row(uint32_t R, int H, uint32_t* tok, int* h0) {
  const uint32_t ng = (uint32_t)((H + kRopeHpt - 1) / kRopeHpt);
  *tok = R / ng;
  *h0 = (int)(R - *tok * ng) * kRopeHpt;
}

// Heads [h0, h1) of one (token, column): y[h] = RoPE(x[h]), kRopeBatch loads in
// flight.  Element offset of head h's chunk: base + h * 128.
template <typename Store>
__device__ __forceinline__ void rotate_heads(const uint16_t* x, int h0, int h1, const ChunkCS& cs, Store store) {
  for (int hb = h0; hb < h1; hb += kRopeBatch) {
    u32x4 v[kRopeBatch];
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u)
      if (hb + u < h1) v[u] = __builtin_nontemporal_load((const u32x4*)(x + (hb + u) * 128));
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u)
      if (hb + u < h1) store(hb + u, rope_chunk_cs(v[u], cs));
  }
}

// ---------------------------------------------------------------------------
// rope3d: tokens [tok_base, tok_base + n) of the range; thread = (token, column).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(RopeArgs a, uint32_t tok_base, uint32_t n) {
  uint32_t tl;
  int h0;
  rope_row(blockIdx.x * (uint32_t)kRopeRows + (threadIdx.x >> 4), a.H, &tl, &h0);
  const uint32_t c = threadIdx.x & 15u;
  if (tl >= n) return;
  const uint32_t tok = tok_base + tl;
  const TokPos p = tok_pos(tok, (uint32_t)a.N, 1.0f / (float)a.N, (uint32_t)a.gw, 1.0f / (float)a.gw);
  const ChunkCS cs = rope_chunk_cs_of(a.tab, (int)c * 4, a.t0 + frame_shift(a.fs) + p.f, (int)p.row, (int)p.col);
  uint16_t* yrow = a.y + (int64_t)tok * a.y_ld + c * 8;
  rotate_heads(a.x + (int64_t)tok * a.x_ld + c * 8, h0, min(h0 + kRopeHpt, a.H), cs,
               [&](int h, u32x4 y) { __builtin_nontemporal_store(y, (u32x4*)(yrow + h * 128)); });
}

// ---------------------------------------------------------------------------
// roll: key work-groups rotate like rope3d and store head-major; value
// work-groups give a thread an 8-token x 8-dim block of one (frame, head).
// Values: the 8x8 bf16 block is transposed in registers so that each dim's 8
// tokens form one 16-byte chunk, the chunk that V[slot][h][n/8][d][8] holds
// for (token group n/8, dim d) -- the transpose costs no extra pass.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // in[j] = 8 dims of token j (word w holds dims 2w, 2w+1);
  // out[i] = 8 tokens of dim i (word u holds tokens 2u, 2u+1).
  uint32_t w[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) { w[j][0] = in[j][0]; w[j][1] = in[j][1]; w[j][2] = in[j][2]; w[j][3] = in[j][3]; }
  uint32_t o[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t a0 = w[2 * u][i >> 1], a1 = w[2 * u + 1][i >> 1];
      uint32_t lo = (i & 1) ? (a0 >> 16) : (a0 & 0xFFFFu);
      uint32_t hi = (i & 1) ? (a1 & 0xFFFF0000u) : (a1 << 16);
      o[i][u] = lo | hi;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) { u32x4 r = {o[i][0], o[i][1], o[i][2], o[i][3]}; out[i] = r; }
}

// Values: a value work-group owns (frame, head, 64-dim half, block of kVBlock
// tokens).  Each thread loads 8 tokens x 8 dims (every load instruction of a
// wave reads whole 128-byte lines, one per token), transposes them in
// registers and writes the result into an LDS image [dim][token] of the block;
// then each 8-token group leaves as its 64 dims' chunks, one contiguous 1 KB
// run (the value layout [h][n/8][d][8] makes a token group's dims adjacent).
// With the earlier [h][d][n] layout each dim row of the block was a 256-byte
// run at a 3,120-byte stride, none line-aligned, and the 16-frame roll took
// 62-64 us cold against 55.6 us with whole 1 KB runs.  Work-groups owning
// fewer dims per token read partial lines that a work-group on another XCD
// fetches again, which measured much slower.
constexpr int kVBlock = 128;  // tokens per value work-group (multiple of 8)
static_assert(kVBlock % 8 == 0, "value block");

// The window a roll of frames t0..t0+n-1 leaves (the host's ring rule, applied on
// the device to a device-resident descriptor): overwrite inside the window,
// append after it, evict the oldest frames beyond the capacity.
__device__ void advance_window(DevRing* r, int64_t t0, int n) {
  const int W = r->capacity > 0 ? r->capacity : 1;
  int64_t first = r->first;
  int64_t end = first + (r->count > 0 ? r->count : 0);
  if (r->count <= 0) first = end = t0;
  const int64_t new_end = end > t0 + n ? end : t0 + n;
  int64_t count = new_end - first;
  if (count > W) {
    first = new_end - W;
    count = W;
  }
  r->first = first;
  r->count = (int32_t)count;
}

// Work-groups [0, v_blocks): value blocks as above.  Work-groups from v_blocks
// on: keys of tokens [tok_base, tok_base + k_tokens), a thread per (token, head
// group, 16-byte column) as in rope3d, rotated and stored to K[slot][h][n][d].
// The longer value work-groups come first so that they do not form a tail.
// blockIdx.y is the layer: its inputs sit layer_stride elements further, its
// ring is a.rings[layer] when per-layer device descriptors are given (whose
// window the layer's first work-group advances when `advance` is set).
__global__ __launch_bounds__(256) void roll_kernel(RollArgs a, uint32_t v_blocks, uint32_t tok_base,
                                                   uint32_t k_tokens, int advance) {
  const int64_t sh = frame_shift(a.fs);
  if (a.rings) {
    DevRing* r = a.rings + blockIdx.y;
    a.k_ring = r->k;
    a.v_ring = r->v;
    a.W = r->capacity > 0 ? r->capacity : 1;
    a.slot0 = (int)mod_pos(a.t0, a.W);
    a.k_new += (int64_t)blockIdx.y * a.k_layer_stride;
    a.v_new += (int64_t)blockIdx.y * a.v_layer_stride;
    if (advance && blockIdx.x == 0 && threadIdx.x == 0) advance_window(r, a.t0 + sh, a.n_frames);
  }
  if (blockIdx.x >= v_blocks) {
    uint32_t tl;
    int h0;
    rope_row((blockIdx.x - v_blocks) * (uint32_t)kRopeRows + (threadIdx.x >> 4), a.H, &tl, &h0);
    const uint32_t c = threadIdx.x & 15u;
    if (tl >= k_tokens) return;
    const uint32_t tok = tok_base + tl;
    const TokPos p = tok_pos(tok, (uint32_t)a.N, 1.0f / (float)a.N, (uint32_t)a.gw, 1.0f / (float)a.gw);
    int slot = a.slot0 + (int)(sh % a.W);
    if (slot >= a.W) slot -= a.W;
    slot += (int)p.f;
    if (slot >= a.W) slot -= a.W;  // both terms below W
    const ChunkCS cs = rope_chunk_cs_of(a.tab, (int)c * 4, a.t0 + sh + p.f, (int)p.row, (int)p.col);
    const uint32_t n = tok - p.f * (uint32_t)a.N;
    uint16_t* krow = a.k_ring + (int64_t)slot * a.slot_elems + (int64_t)n * 128 + c * 8;  // head 0
    const int64_t head_stride = (int64_t)a.N * 128;
    rotate_heads(a.k_new + (int64_t)tok * a.k_ld + c * 8, h0, min(h0 + kRopeHpt, a.H), cs, [&](int h, u32x4 y) {
      __builtin_nontemporal_store(y, (u32x4*)(krow + h * head_stride));
    });
    return;
  }
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][kVBlock + 8];
  const uint32_t N = (uint32_t)a.N;
  const uint32_t nblk = (N + kVBlock - 1) / kVBlock;
  const uint32_t fhd = blockIdx.x / nblk;  // (frame, head, half)
  const uint32_t b = blockIdx.x - fhd * nblk;
  const uint32_t fh = fhd >> 1, dh = fhd & 1u;
  const int f = (int)fh / a.H;
  const int h = (int)fh - f * a.H;
  int slot = a.slot0 + (int)(sh % a.W);
  if (slot >= a.W) slot -= a.W;
  slot += f;
  if (slot >= a.W) slot -= a.W;
  const uint32_t t0 = b * (uint32_t)kVBlock;
  const uint32_t ng = (min((uint32_t)kVBlock, N - t0)) >> 3;  // 8-token groups in the block
  const uint16_t* vin = a.v_new + ((int64_t)f * N + t0) * a.v_ld + h * 128 + dh * 64;
  for (uint32_t t = threadIdx.x; t < ng * 8; t += 256) {  // (group, 8-dim chunk)
    const uint32_t c = t & 7u, g = t >> 3;
    u32x4 in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      in[j] = __builtin_nontemporal_load((const u32x4*)(vin + (int64_t)(g * 8 + j) * a.v_ld + c * 8));
    u32x4 vt[8];
    transpose8x8(in, vt);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)&tile[c * 8 + i][g * 8] = vt[i];
  }
  __syncthreads();
  // token group t0/8 + g, dims dh*64 + r: [h][n/8][d][8]
  uint16_t* vout = a.v_ring + (int64_t)slot * a.slot_elems + (int64_t)h * N * 128 + (int64_t)(t0 / 8) * 1024 + dh * 512;
  for (uint32_t q = threadIdx.x; q < 64 * ng; q += 256) {  // (group, dim row): a wave writes 1 KB runs
    const uint32_t g = q >> 6, r = q & 63u;
    *(u32x4*)(vout + (int64_t)g * 1024 + r * 8) = *(const u32x4*)&tile[r][g * 8];
  }
}

// Tokens per launch: keeps the (token, head group) row index, token * groups,
// below 2^30.
uint32_t tokens_per_launch(int H) { return (1u << 30) / (uint32_t)((H + kRopeHpt - 1) / kRopeHpt); }

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s) {
  const uint32_t per_launch = tokens_per_launch(a.H);
  for (uint32_t t = 0; t < (uint32_t)a.n_tokens; t += per_launch) {
    const uint32_t n = min(per_launch, (uint32_t)a.n_tokens - t);
    const uint64_t rows = (uint64_t)n * (uint64_t)((a.H + kRopeHpt - 1) / kRopeHpt);
    dim3 grid((unsigned)((rows + kRopeRows - 1) / kRopeRows));
    hipLaunchKernelGGL(rope3d_kernel, grid, dim3(kRopeThreads), 0, s, a, t, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_roll(const RollArgs& a, hipStream_t s) {
  const uint32_t tokens = (uint32_t)a.n_frames * (uint32_t)a.N;
  const uint32_t v_blocks = (uint32_t)a.n_frames * (uint32_t)a.H * 2u * (((uint32_t)a.N + kVBlock - 1) / kVBlock);
  const uint32_t per_launch = tokens_per_launch(a.H);
  for (uint32_t t = 0; t < tokens; t += per_launch) {
    const uint32_t n = min(per_launch, tokens - t);
    const uint64_t rows = (uint64_t)n * (uint64_t)((a.H + kRopeHpt - 1) / kRopeHpt);
    const uint32_t k_blocks = (uint32_t)((rows + kRopeRows - 1) / kRopeRows);
    const uint32_t vb = t == 0 ? v_blocks : 0u;  // value blocks ride with the first piece
    hipLaunchKernelGGL(roll_kernel, dim3(vb + k_blocks, (unsigned)a.n_layers), dim3(256), 0, s, a, vb, t, n,
                       t == 0 ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Plain device copy, one 16-byte chunk per thread, non-temporal both ways: the
// bandwidth one launch of a given size reaches when it only moves bytes (the
// ceiling the RoPE and roll kernels are measured against).
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                   uint64_t n16, uint64_t base) {
  const uint64_t i = base + (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_copy(void* dst, const void* src, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  const uint64_t per_launch = (uint64_t)1 << 31;  // chunks per launch: the grid stays below 2^23 blocks
  for (uint64_t b = 0; b < n16; b += per_launch) {
    const uint64_t n = n16 - b < per_launch ? n16 - b : per_launch;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (u32x4*)dst,
                       (const u32x4*)src, b + n, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ void upload_rings_kernel(DevRing* dst, UploadArgs a) {
  if ((int)threadIdx.x < a.n) dst[threadIdx.x] = a.d[threadIdx.x];
}

hipError_t launch_upload_rings(DevRing* dst, const UploadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(upload_rings_kernel, dim3(1), dim3(kUploadMax), 0, s, dst, a);
  return hipGetLastError();
}

// *p += delta on the stream (a one-thread kernel: stream-ordered and capturable).
__global__ void add_shift_kernel(int64_t* p, int64_t delta) { p[threadIdx.x] += delta; }

hipError_t launch_add_shift(int64_t* p, int64_t delta, hipStream_t s) {
  hipLaunchKernelGGL(add_shift_kernel, dim3(1), dim3(1), 0, s, p, delta);
  return hipGetLastError();
}

}  // namespace rfattn
