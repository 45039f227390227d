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
// Work decomposition.  One work-group = (segment, head, 256 query rows):
// four waves (one per SIMD), each owning two groups of 32 query rows.  Per
// 64-key tile and group:
//   S^T[key][q] = K_tile . Q^T    2 key blocks x 8 k-steps of v_mfma_f32_32x32x16_bf16
//   online softmax in float32, exp2 with scale*log2(e) folded into one FMA
//   O^T[d][q]  += V^T_tile . P^T  4 dim blocks x 4 k-steps
// Every K and V fragment read from LDS feeds the MFMAs of both groups.
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators, so a row max needs one cross-half exchange, the row sum
// none until the end, and the rescale is a per-lane scalar.  The key order
// inside a tile is permuted (kappa below) so that each lane's 16 softmax
// values per key block are 16 consecutive keys, which is what the P^T
// operand of the value product needs; the softmax is order-free over keys.
//
// Software pipeline per wave, iteration j: the score MFMAs of tile j are
// issued alongside the softmax of tile j-1, then the value MFMAs of tile j-1
// alongside staging the next K/V tiles.  K/V tiles are gathered from the
// ring slots (a tile may straddle two frames) with raw buffer loads into
// registers and written to LDS one iteration later; the K pipeline runs one
// tile ahead of the V pipeline.  Q is loaded once with 3D-RoPE applied on
// the fly (bit-identical to rf_rope3d_apply); keys are stored rotated.
#include "device_common.h"
#include "kernels.h"

namespace rfattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroups = 2;                 // 32-query groups per wave (share every K/V fragment)
constexpr int kWaves = 4;                  // one wave per SIMD
constexpr int kBlockM = kWaves * kGroups * 32;  // query rows per work-group (256)
constexpr int kBlockN = 64;                // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr int kKRow = kHeadDim + 8;        // LDS row stride of K tile (272 B: conflict-free 16 B reads)
constexpr int kVRow = kBlockN + 8;         // LDS row stride of V^T tile (144 B)
constexpr int kKTile = kBlockN * kKRow;    // elements
constexpr int kVTile = kHeadDim * kVRow;   // elements
constexpr size_t kLdsBytes = 2 * (kKTile + kVTile) * sizeof(uint16_t);  // K and V, two each
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
__global__ __launch_bounds__(kThreads, 1) void window_attn_kernel(AttnArgs a) {
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

  // ---- Q fragments, RoPE'd on load: group g of this wave holds query rows
  // q0 + 32g + lr; lane half hf holds dims 16s + 8hf .. +7 of k-step s ------
  const int q0 = qt * kBlockM + wave * (kGroups * 32);
  bf16x8 qf[kGroups][8];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int qi = q0 + 32 * g + lr;
    if (qi < sg.q_tokens) {
      const int f = qi / a.N;
      const int pin = qi - f * a.N;
      const int row = pin / a.gw;
      const int col = pin - row * a.gw;
      const uint16_t* qrow = sg.q + (int64_t)qi * sg.q_ld + h * kHeadDim;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 2 * s + hf;
        u32x4 x = *(const u32x4*)(qrow + 8 * c);
        qf[g][s] = as_bf16x8(rope_chunk(x, 4 * c, sg.q_t0 + f, row, col, a.tab));
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[g][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  // ---- tile loaders (byte offsets into the rings, raw buffer loads) ------------
  // The K pipeline runs one tile ahead of the V pipeline: tile j's keys are
  // needed in iteration j (scores), its values in iteration j+1 (after the
  // softmax), so two LDS buffers per operand suffice.
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

  // Cursors of the next tile to load (uniform): slot and token offset of its first key.
  int kslot = sg.ctx_slot0, kn = 0, kload = 0;
  int vslot = sg.ctx_slot0, vn = 0, vload = 0;
  auto advance = [&](int& slot, int& n) {
    n += kBlockN;
    while (n >= N) {
      n -= N;
      slot = (slot + 1 == W) ? 0 : slot + 1;
    }
  };

  auto load_k = [&]() {
    const int key_lim = nkeys - kload * kBlockN;  // valid keys in this tile (may be <= 0)
    uint32_t off[4];
    if constexpr (!kSmallN) {
      const int b = N - kn;  // keys of this tile still in the current frame
      const int nxt = (kslot + 1 == W) ? 0 : kslot + 1;
      const uint32_t ka = (uint32_t)kslot * slot_b + k_head + (uint32_t)kn * (kHeadDim * 2u);
      const uint32_t kb = (uint32_t)nxt * slot_b + k_head - (uint32_t)b * (kHeadDim * 2u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = k_r0 + 16 * i;
        off[i] = (uint32_t)r * (kHeadDim * 2u) + 16u * k_c + (r < b ? ka : kb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int n = kn + k_r0 + 16 * i, slot = kslot;
        while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
        off[i] = (uint32_t)slot * slot_b + k_head + (uint32_t)n * (kHeadDim * 2u) + 16u * k_c;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (k_r0 + 16 * i >= key_lim) off[i] = kOutOfRange;  // past the end: zeros
      kst[i] = bload(krs, off[i]);
    }
    advance(kslot, kn);
    ++kload;
  };

  auto load_v = [&]() {
    const int key_lim = nkeys - vload * kBlockN;
    uint32_t base;
    if constexpr (!kSmallN) {
      const int b = N - vn;
      const int nxt = (vslot + 1 == W) ? 0 : vslot + 1;
      base = (8 * v_kc < b) ? (uint32_t)vslot * slot_b + v_head + (uint32_t)vn * 2u
                            : (uint32_t)nxt * slot_b + v_head - (uint32_t)b * 2u;
    } else {
      int n = vn + 8 * v_kc, slot = vslot;
      while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
      base = (uint32_t)slot * slot_b + v_head + (uint32_t)n * 2u - 16u * v_kc;
    }
    const bool valid = 8 * v_kc < key_lim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = base + (uint32_t)(v_d0 + 32 * i) * (uint32_t)N * 2u + 16u * v_kc;
      vst[i] = bload(vrs, valid ? off : kOutOfRange);
    }
    advance(vslot, vn);
    ++vload;
  };

  auto store_k = [&](int buf) {
    uint16_t* Kl = lds + buf * kKTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(Kl + (k_r0 + 16 * i) * kKRow + 8 * k_c) = kst[i];
  };
  auto store_v = [&](int buf) {
    uint16_t* Vl = lds + 2 * kKTile + buf * kVTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(Vl + (v_d0 + 32 * i) * kVRow + 8 * v_kc) = vst[i];
  };

  // ---- running state -----------------------------------------------------------
  f32x16 o[kGroups][4];
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[g][dt][i] = 0.0f;
  float m_run[kGroups], l_run[kGroups];  // running row max (log2 units, stale by < 8), row sum
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    m_run[g] = -1.0e30f;
    l_run[g] = 0.0f;
  }
  const float cl = a.c_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16 zero16 = {};

  // A-operand row m of the score MFMA reads key kappa(m): lane half hf of
  // output register i then holds key 16*hf + i of each 32-key block.
  const int krow = 16 * ((lr >> 2) & 1) + 4 * (lr >> 3) + (lr & 3);

  // S^T = K Q^T, keys [0,32) and [32,64) of the tile in K buffer `buf`, for
  // both query groups; every K fragment read from LDS feeds two MFMAs.
  auto scores = [&](int buf, f32x16 (&S)[kGroups][2]) {
    const uint16_t* Kl = lds + buf * kKTile;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) S[g][0] = S[g][1] = zero16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 k0 = *(const bf16x8*)(Kl + krow * kKRow + 16 * s + 8 * hf);
      const bf16x8 k1 = *(const bf16x8*)(Kl + (32 + krow) * kKRow + 16 * s + 8 * hf);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        S[g][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[g][s], S[g][0], 0, 0, 0);
        S[g][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[g][s], S[g][1], 0, 0, 0);
      }
    }
  };

  // Online softmax of one group's tile scores (log2 domain) into bf16 weights
  // pw.  The running max only moves when some row's tile max exceeds it by
  // more than 2^8 (wave-uniform decision); alpha then rescales l here and O
  // before the next value product.  The row sums are added separately.
  auto softmax = [&](int g, f32x16& s0, f32x16& s1, uint32_t (&pr)[16], bool& rescale, float& alpha) {
    float mx = __builtin_elementwise_maximum(s0[0], s0[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2)
      mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[i], s0[i + 1]));
#pragma unroll
    for (int i = 0; i < 16; i += 2)
      mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s1[i], s1[i + 1]));
    const float mt = xhalf_max(mx) * cl;
    rescale = __builtin_amdgcn_ballot_w64(mt > m_run[g] + kRescaleLog2) != 0;
    const float m_new = rescale ? fmaxf(m_run[g], mt) : m_run[g];
    alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
    m_run[g] = m_new;
    l_run[g] *= alpha;
    const float neg_m = -m_new;
    // pr[e]: keys 2e, 2e+1 of this lane's 16 in block 0; pr[8+e]: same in block 1
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = pack2(__builtin_amdgcn_exp2f(fmaf(s0[2 * e], cl, neg_m)),
                    __builtin_amdgcn_exp2f(fmaf(s0[2 * e + 1], cl, neg_m)));
      pr[8 + e] = pack2(__builtin_amdgcn_exp2f(fmaf(s1[2 * e], cl, neg_m)),
                        __builtin_amdgcn_exp2f(fmaf(s1[2 * e + 1], cl, neg_m)));
    }
  };

  // Row sums of the bf16 weights.  They are read from the scalar words: the
  // compiler picks wrong registers for bf16x2 bit-casts of elements of a
  // 4-word vector feeding the dot2 builtin.
  auto row_sums = [&](int g, const uint32_t (&pr)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      l_run[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr[i]), ones, l_run[g], false);
  };

  // O^T += V^T P^T with the values in V buffer `buf`, both groups per fragment.
  // P^T operand of block b, half-step u: keys 32b + 16hf + 8u + 0..7.
  auto values = [&](int buf, const uint32_t (&pr)[kGroups][16]) {
    const uint16_t* Vl = lds + 2 * kKTile + buf * kVTile;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 vf =
              *(const bf16x8*)(Vl + (32 * dt + lr) * kVRow + 32 * b + 16 * hf + 8 * u);
#pragma unroll
          for (int g = 0; g < kGroups; ++g) {
            const int w = 8 * b + 4 * u;
            const u32x4 pv = {pr[g][w], pr[g][w + 1], pr[g][w + 2], pr[g][w + 3]};
            o[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pv), o[g][dt], 0, 0, 0);
          }
        }
      }
    }
  };

  auto rescale_o = [&](int g, bool rescale, float alpha) {
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[g][dt][i] *= alpha;
    }
  };

  // Keeps values materialised at this point (no instruction is emitted): the
  // softmax stays in the phase whose MFMAs it is meant to overlap.
  auto pin = [](const uint32_t (&pr)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(pr[i]));
  };

  // ---- software pipeline over key tiles ----------------------------------------
  // iteration j, phase 1: scores of tile j   | softmax of tile j-1
  //              phase 2: values of tile j-1 | stage K_{j+1}, V_j to LDS,
  //                                            fetch K_{j+2}, V_{j+1}
  load_k();  // K_0
  load_v();  // V_0
  store_k(0);
  store_v(0);
  load_k();  // K_1
  __syncthreads();
  f32x16 sp[kGroups][2];  // scores of the previous tile
  scores(0, sp);
  store_k(1);
  load_k();  // K_2
  load_v();  // V_1
  __syncthreads();

  for (int j = 1; j < ntiles; ++j) {
    f32x16 sn[kGroups][2];
    uint32_t pw[kGroups][16];
    bool rs[kGroups];
    float alpha[kGroups];
    scores(j & 1, sn);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      softmax(g, sp[g][0], sp[g][1], pw[g], rs[g], alpha[g]);
      pin(pw[g]);
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) rescale_o(g, rs[g], alpha[g]);
    values((j - 1) & 1, pw);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) row_sums(g, pw[g]);
    store_k((j + 1) & 1);  // K_{j+1}
    store_v(j & 1);        // V_j
    load_k();              // K_{j+2}
    load_v();              // V_{j+1}
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      sp[g][0] = sn[g][0];
      sp[g][1] = sn[g][1];
    }
  }

  {  // last tile: mask keys past the end, then its softmax and values
    const int key_lim = nkeys - (ntiles - 1) * kBlockN;
    if (key_lim < kBlockN) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (16 * hf + i >= key_lim) sp[g][0][i] = -INFINITY;
          if (32 + 16 * hf + i >= key_lim) sp[g][1][i] = -INFINITY;
        }
    }
    uint32_t pw[kGroups][16];
    bool rs[kGroups];
    float alpha[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) softmax(g, sp[g][0], sp[g][1], pw[g], rs[g], alpha[g]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) rescale_o(g, rs[g], alpha[g]);
    values((ntiles - 1) & 1, pw);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) row_sums(g, pw[g]);
  }

  // ---- epilogue: O = O^T / l, bf16, token-major -----------------------------------
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const float inv = 1.0f / xhalf_sum(l_run[g]);
    const int qi = q0 + 32 * g + lr;
    if (qi < sg.q_tokens) {
      uint16_t* orow = sg.o + (int64_t)qi * sg.o_ld + h * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          // registers 4*g4 .. 4*g4+3 hold dims 32dt + 8g4 + 4hf + 0..3
          u32x2 w;
          w[0] = pack2(o[g][dt][4 * g4 + 0] * inv, o[g][dt][4 * g4 + 1] * inv);
          w[1] = pack2(o[g][dt][4 * g4 + 2] * inv, o[g][dt][4 * g4 + 3] * inv);
          *(u32x2*)(orow + 32 * dt + 8 * g4 + 4 * hf) = w;
        }
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
