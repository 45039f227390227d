// Flash-style non-causal window attention for gfx950 (CDNA4), bf16 MFMA.
//
// Source: the DiT self-attention of 23,400 query tokens over 32,760 context
// tokens in 12 heads that dominates the step (ai4snews digest of "A
// kernel-centric path to real-time video generation on Trainium", second
// paragraph); attention transposes live inside the attention kernel
// (vibeleaderboard digest, key takeaways); the denoise and cache-update
// passes are batched ("Optimizing Real-Time Video Generation on Trainium
// Chips", section 8) -- here as several query segments in one grid.
//
// Work decomposition: one work-group = (segment, head, 128 query rows), four
// waves of 32 query rows each.  Per 64-key tile:
//   S^T[key][q] = K_tile . Q^T      v_mfma_f32_32x32x16_bf16, 2 tiles x 8 k-steps
//   online softmax in float32, exp2 with scale*log2(e) folded into one FMA
//   O^T[d][q]  += V^T_tile . P^T    4 dim tiles x 4 k-steps
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators, so the row max needs one cross-half exchange, the row
// sum none until the end, and the rescale is a per-lane scalar.  The key
// order inside a tile is permuted (kappa below) so that each lane's 16
// softmax values are 16 consecutive keys, which is what the P^T operand of
// the value product needs; the softmax is order-free over keys.
//
// K/V tiles are gathered from ring slots (a tile may straddle frames), staged
// through LDS with register prefetch of the next tile, two LDS buffers and
// one barrier per tile.  Q is loaded once per work-group with 3D-RoPE applied
// on the fly (bit-identical to rf_rope3d_apply); keys are stored rotated.
#include "device_common.h"
#include "kernels.h"

namespace rfattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockM = 128;               // query rows per work-group
constexpr int kBlockN = 64;                // keys per tile
constexpr int kThreads = 256;              // 4 waves
constexpr int kKRow = kHeadDim + 8;        // LDS row stride of K tile (272 B: conflict-free 16 B reads)
constexpr int kVRow = kBlockN + 8;         // LDS row stride of V^T tile (144 B)
constexpr int kKTile = kBlockN * kKRow;    // elements
constexpr int kVTile = kHeadDim * kVRow;   // elements
constexpr int kStage = kKTile + kVTile;    // one LDS buffer, elements
constexpr size_t kLdsBytes = 2 * kStage * sizeof(uint16_t);
constexpr float kRescaleLog2 = 8.0f;       // rescale O only when a row max grows by > 2^8
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;   // buffer offset past the end: the load returns 0
constexpr int kXcds = 8;                   // MI355X: work-groups go round-robin over 8 XCDs

int window_attn_block_m() { return kBlockM; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Combine a per-lane value with the lane 32 positions away (the other half of the
// wave holds the other 16 keys of the same query).
__device__ __forceinline__ float xhalf_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Work-group id -> tile index such that each XCD walks a contiguous run of tiles
// (consecutive query tiles of one head), so the work-groups resident on an XCD at
// any time share their head's K/V in that XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int x = bid % kXcds, idx = bid / kXcds;
  if (rem == 0 || x < rem) return x * per + idx;
  return rem * per + (x - rem) * (per - 1) + idx;
}

// kSmallN: frames shorter than a key tile (a tile may cover 3+ frames); the
// general per-row frame walk is used.  Otherwise a tile straddles at most one
// frame boundary and each row picks one of two bases.
template <bool kSmallN>
__global__ __launch_bounds__(kThreads, 2) void window_attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // query column of this lane in the 32x32 tiles
  const int hf = lane >> 5;  // lane half: selects k-slots 0-7 / 8-15 of an MFMA step

  // ---- work-group -> (segment, head, query tile) ---------------------------
  const int tile = xcd_tile(blockIdx.x, a.total_tiles);
  int si = 0;
#pragma unroll
  for (int s = 1; s < kMaxSegments; ++s)
    if (s < a.n_segs && tile >= a.seg[s].tile_begin) si = s;
  const SegDev& sg = a.seg[si];
  const int local = tile - sg.tile_begin;
  const int h = local / sg.q_tiles;
  const int qt = local - h * sg.q_tiles;

  // ---- Q fragment, RoPE'd on load: lane holds query row lr, dims 16s+8hf..+7 --
  const int qi = qt * kBlockM + wave * 32 + lr;
  const bool qvalid = qi < sg.q_tokens;
  bf16x8 qf[8];
  if (qvalid) {
    const int f = qi / a.N;
    const int pin = qi - f * a.N;
    const int row = pin / a.gw;
    const int col = pin - row * a.gw;
    const uint16_t* qrow = sg.q + (int64_t)qi * sg.q_ld + h * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + hf;
      u32x4 x = *(const u32x4*)(qrow + 8 * c);
      qf[s] = as_bf16x8(rope_chunk(x, 4 * c, sg.q_t0 + f, row, col, a.tab));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  // ---- tile loaders (byte offsets into the rings, raw buffer loads) ------------
  const int nkeys = sg.ctx_keys;
  const int ntiles = (nkeys + kBlockN - 1) / kBlockN;
  const int N = a.N;
  const int W = a.W;
  const uint32_t slot_b = (uint32_t)a.slot_elems * 2u;
  const uint32_t ring_b = slot_b * (uint32_t)W;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k_ring), 0, (int)ring_b, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v_ring), 0, (int)ring_b, kBufferWord3);
  const uint32_t k_head = (uint32_t)h * (uint32_t)N * (kHeadDim * 2u);  // K: [H][N][D]
  const uint32_t v_head = (uint32_t)h * kHeadDim * (uint32_t)N * 2u;    // V: [H][D][N]
  // K: rows (tid>>4) + 16i, 16-byte chunk tid&15.  V^T: dims (tid>>3) + 32i, key chunk tid&7.
  const int k_r0 = tid >> 4, k_c = tid & 15;
  const int v_d0 = tid >> 3, v_kc = tid & 7;
  u32x4 kst[4], vst[4];

  // Cursor of the tile start in the key stream (uniform): slot and token offset.
  int cur_slot = sg.ctx_slot0;
  int cur_n = 0;

  auto load_tile = [&](int kt) {
    const int key_lim = nkeys - kt * kBlockN;  // valid keys in this tile
    uint32_t koff[4], voff[4];
    if constexpr (!kSmallN) {
      const int b = N - cur_n;  // keys of this tile still in the current frame
      const int nxt = (cur_slot + 1 == W) ? 0 : cur_slot + 1;
      const uint32_t ka = (uint32_t)cur_slot * slot_b + k_head + (uint32_t)cur_n * (kHeadDim * 2u);
      const uint32_t kb = (uint32_t)nxt * slot_b + k_head - (uint32_t)b * (kHeadDim * 2u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = k_r0 + 16 * i;
        koff[i] = (uint32_t)r * (kHeadDim * 2u) + 16u * k_c + (r < b ? ka : kb);
      }
      const uint32_t vbase = (8 * v_kc < b)
                                 ? (uint32_t)cur_slot * slot_b + v_head + (uint32_t)cur_n * 2u
                                 : (uint32_t)nxt * slot_b + v_head - (uint32_t)b * 2u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        voff[i] = vbase + (uint32_t)(v_d0 + 32 * i) * (uint32_t)N * 2u + 16u * v_kc;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = cur_n + k_r0 + 16 * i, slot = cur_slot;
        while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
        koff[i] = (uint32_t)slot * slot_b + k_head + (uint32_t)n * (kHeadDim * 2u) + 16u * k_c;
      }
      int n = cur_n + 8 * v_kc, slot = cur_slot;
      while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        voff[i] = (uint32_t)slot * slot_b + v_head + (uint32_t)(v_d0 + 32 * i) * (uint32_t)N * 2u +
                  (uint32_t)n * 2u;
    }
    if (key_lim < kBlockN) {  // last tile: keys past the end read as zeros
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k_r0 + 16 * i >= key_lim) koff[i] = kOutOfRange;
        if (8 * v_kc >= key_lim) voff[i] = kOutOfRange;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) kst[i] = bload(krs, koff[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vst[i] = bload(vrs, voff[i]);
    // advance the cursor by one tile
    cur_n += kBlockN;
    while (cur_n >= N) {
      cur_n -= N;
      cur_slot = (cur_slot + 1 == W) ? 0 : cur_slot + 1;
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* Kl = lds + buf * kStage;
    uint16_t* Vl = Kl + kKTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(Kl + (k_r0 + 16 * i) * kKRow + 8 * k_c) = kst[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(Vl + (v_d0 + 32 * i) * kVRow + 8 * v_kc) = vst[i];
  };

  // ---- running state -----------------------------------------------------------
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m_run = -1.0e30f;  // running row max of scaled scores (log2 units), maybe stale by < 8
  float l_run = 0.0f;      // this lane's partial row sum of the bf16 weights
  const float cl = a.c_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16 zero16 = {};

  // A-operand row m of the score MFMA reads key kappa(m): lane half hf of
  // output register i then holds key 16*hf + i of each 32-key block.
  const int krow = 16 * ((lr >> 2) & 1) + 4 * (lr >> 3) + (lr & 3);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);

    const uint16_t* Kl = lds + buf * kStage;
    const uint16_t* Vl = Kl + kKTile;

    // S^T = K Q^T for keys [0,32) and [32,64) of the tile
    f32x16 s0 = zero16, s1 = zero16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 k0 = *(const bf16x8*)(Kl + krow * kKRow + 16 * s + 8 * hf);
      const bf16x8 k1 = *(const bf16x8*)(Kl + (32 + krow) * kKRow + 16 * s + 8 * hf);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
    }

    // mask keys past the end (last tile only)
    const int key_lim = nkeys - kt * kBlockN;
    if (key_lim < kBlockN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * hf + i >= key_lim) s0[i] = -INFINITY;
        if (32 + 16 * hf + i >= key_lim) s1[i] = -INFINITY;
      }
    }

    // online softmax (log2 domain); O and l are rescaled only when some row max
    // grows past the stale one by more than 2^8 (wave-uniform decision)
    float mx = __builtin_elementwise_maximum(s0[0], s0[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[i], s0[i + 1]));
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s1[i], s1[i + 1]));
    const float mt = xhalf_max(mx) * cl;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleLog2) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    const float neg_m = -m_run;
    u32x4 pw[4];  // P^T operands: block b, half-step u -> keys 32b + 16hf + 8u + 0..7
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a0 = __builtin_amdgcn_exp2f(fmaf(s0[2 * e], cl, neg_m));
      const float a1 = __builtin_amdgcn_exp2f(fmaf(s0[2 * e + 1], cl, neg_m));
      const float b0 = __builtin_amdgcn_exp2f(fmaf(s1[2 * e], cl, neg_m));
      const float b1 = __builtin_amdgcn_exp2f(fmaf(s1[2 * e + 1], cl, neg_m));
      const uint32_t pa = pack2(a0, a1), pb = pack2(b0, b1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pa), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb), ones, l_run, false);
      pw[e >> 2][e & 3] = pa;
      pw[2 + (e >> 2)][e & 3] = pb;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 vf =
              *(const bf16x8*)(Vl + (32 * dt + lr) * kVRow + 32 * b + 16 * hf + 8 * u);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pw[2 * b + u]), o[dt], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16, token-major -----------------------------------
  const float inv = 1.0f / xhalf_sum(l_run);
  if (qvalid) {
    uint16_t* orow = sg.o + (int64_t)qi * sg.o_ld + h * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // registers 4*g4 .. 4*g4+3 hold dims 32dt + 8g4 + 4hf + 0..3
        u32x2 w;
        w[0] = pack2(o[dt][4 * g4 + 0] * inv, o[dt][4 * g4 + 1] * inv);
        w[1] = pack2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * g4 + 4 * hf) = w;
      }
    }
  }
}

hipError_t prepare_window_attn() {
  hipError_t e = hipFuncSetAttribute((const void*)window_attn_kernel<false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)window_attn_kernel<true>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
}

hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s) {
  if (a.N < kBlockN)
    hipLaunchKernelGGL(window_attn_kernel<true>, dim3((unsigned)a.total_tiles), dim3(kThreads), kLdsBytes, s, a);
  else
    hipLaunchKernelGGL(window_attn_kernel<false>, dim3((unsigned)a.total_tiles), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace rfattn
