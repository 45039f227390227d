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

int window_attn_block_m() { return kBlockM; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__global__ __launch_bounds__(kThreads, 2) void window_attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // query column of this lane in the 32x32 tiles
  const int hf = lane >> 5;  // lane half: selects k-slots 0-7 / 8-15 of an MFMA step

  // ---- work-group -> (segment, head, query tile) ---------------------------
  const int bid = blockIdx.x;
  int si = 0;
#pragma unroll
  for (int s = 1; s < kMaxSegments; ++s)
    if (s < a.n_segs && bid >= a.seg[s].tile_begin) si = s;
  const SegDev& sg = a.seg[si];
  const int local = bid - sg.tile_begin;
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

  // ---- tile loaders ----------------------------------------------------------
  const int nkeys = sg.ctx_keys;
  const int ntiles = (nkeys + kBlockN - 1) / kBlockN;
  const int N = a.N;
  const int W = a.W;
  const uint16_t* kbase = a.k_ring + (int64_t)h * N * kHeadDim;
  const uint16_t* vbase = a.v_ring + (int64_t)h * kHeadDim * N;
  // K: rows (tid>>4) + 16i, 16-byte chunk tid&15.  V^T: dims (tid>>3) + 32i, key chunk tid&7.
  const int k_r0 = tid >> 4, k_c = tid & 15;
  const int v_d0 = tid >> 3, v_kc = tid & 7;
  u32x4 kst[4], vst[4];

  // Cursor of the tile start in the key stream: slot and token offset.
  int cur_slot = sg.ctx_slot0;
  int cur_n = 0;

  auto locate = [&](int off, int& slot, int& n) {
    n = cur_n + off;
    slot = cur_slot;
    while (n >= N) {
      n -= N;
      slot = (slot + 1 == W) ? 0 : slot + 1;
    }
  };

  auto load_tile = [&](int kt) {
    const int key0 = kt * kBlockN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = k_r0 + 16 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key0 + r < nkeys) {
        int slot, n;
        locate(r, slot, n);
        v = *(const u32x4*)(kbase + slot * a.slot_elems + (int64_t)n * kHeadDim + 8 * k_c);
      }
      kst[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = v_d0 + 32 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key0 + 8 * v_kc < nkeys) {
        int slot, n;
        locate(8 * v_kc, slot, n);
        v = *(const u32x4*)(vbase + slot * a.slot_elems + (int64_t)d * N + n);
      }
      vst[i] = v;
    }
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
  float m_run = -1.0e30f;  // running max of scaled scores (log2 units)
  float l_run = 0.0f;      // this lane's partial row sum (its 16-key halves)
  const float cl = a.c_log2;

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
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) { s0[i] = 0.0f; s1[i] = 0.0f; }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 k0 = *(const bf16x8*)(Kl + krow * kKRow + 16 * s + 8 * hf);
      const bf16x8 k1 = *(const bf16x8*)(Kl + (32 + krow) * kKRow + 16 * s + 8 * hf);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
    }

    // mask keys past the end (last tile only)
    const int key_lim = nkeys - kt * kBlockN;  // valid keys in this tile
    if (key_lim < kBlockN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * hf + i >= key_lim) s0[i] = -INFINITY;
        if (32 + 16 * hf + i >= key_lim) s1[i] = -INFINITY;
      }
    }

    // online softmax (log2 domain)
    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * cl);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], cl, -m_new));
      s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], cl, -m_new));
      ls += s0[i] + s1[i];
    }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;

    // P^T operands: block b, half-step u -> keys 32b + 16hf + 8u + 0..7
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16x2(s0[8 * u + 2 * e], s0[8 * u + 2 * e + 1]);
        w1[e] = pack_bf16x2(s1[8 * u + 2 * e], s1[8 * u + 2 * e + 1]);
      }
      pb[u] = as_bf16x8(w0);
      pb[2 + u] = as_bf16x8(w1);
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
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[2 * b + u], o[dt], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16, token-major -----------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* orow = sg.o + (int64_t)qi * sg.o_ld + h * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // registers 4*g4 .. 4*g4+3 hold dims 32dt + 8g4 + 4hf + 0..3
        u32x2 w;
        w[0] = pack_bf16x2(o[dt][4 * g4 + 0] * inv, o[dt][4 * g4 + 1] * inv);
        w[1] = pack_bf16x2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * g4 + 4 * hf) = w;
      }
    }
  }
}

hipError_t prepare_window_attn() {
  return hipFuncSetAttribute((const void*)window_attn_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
}

hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(window_attn_kernel, dim3((unsigned)a.total_tiles), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace rfattn
