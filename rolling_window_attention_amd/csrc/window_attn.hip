// Flash-style non-causal window attention for gfx950 (CDNA4), bf16 MFMA.
//
// Source: the DiT self-attention of 23,400 query tokens over 32,760 context
// tokens in 12 heads that dominates the step (ai4snews digest of "A
// kernel-centric path to real-time video generation on Trainium", second
// paragraph); attention transposes live inside the attention kernel
// (vibeleaderboard digest, key takeaways); the denoise and cache-update
// passes are batched ("Optimizing Real-Time Video Generation on Trainium
// Chips", section 8) -- here as several query segments in one launch.
//
// Work split.  A launch's query tiles -- (segment, head, 256 query rows) --
// fill whole rounds of the GPU's work-group slots (one per CU) in the
// ordinary way: one work-group per tile, numbered so that each XCD walks
// consecutive tiles of one head and its resident work-groups read the same
// K/V tiles at about the same time (L2 reuse).  The tiles left over for a
// last, partly filled round are not run one per work-group: each is cut into
// the same n_split equal ranges of its key tiles (64 keys each), one
// work-group per piece, with n_split chosen on the host so that those pieces
// end soonest; the pieces are dealt so that the work-groups of one XCD run
// the same key range of consecutive tiles of one head (L2 reuse again).  Each
// piece leaves a partial result (unnormalised O, running max, row sum) in the
// workspace, and window_attn_fixup merges a tile's pieces.  A launch with
// fewer tiles than slots (the cache-update pass alone) is split this way
// entirely.
//
// Per query tile: eight waves of 32 query rows (two per SIMD) share each K/V
// tile, which the work-group fetches and stages once (a wave whose rows all lie
// past the segment's end only stages).  Per 64-key tile:
//   T^T[key][q] = K_tile . Q'^T - m  v_mfma_f32_32x32x16_bf16, 2 key blocks x 8 k-steps
//   online softmax in float32: 2^T, bf16 weights P, row sums
//   O^T[d][q]  += V^T_tile . P^T     4 dim blocks x 4 k-steps
// Q' is Q rotated (3D-RoPE) and scaled by scale*log2(e) on load, so the score
// MFMAs deliver exponents in log2 units; the running row max m enters as the
// accumulator input of each key block's first k-step (a register block holding
// -m for this lane's query).  The softmax is then one exp2, half a pack and
// half a dot2 per score, plus the tile max.
//
// Registers (256 per lane for each of the two waves of a SIMD): the O^T
// accumulators sit in the fixed accumulation registers a[0:63] and the Q'
// fragments in 32 further accumulation registers, leaving 160 VGPRs for the
// scores, the K/V fragments, the weights and the staging.  With O^T out of the
// VGPR file, the VALU work of the other wave on the SIMD issues more freely
// next to the value MFMAs.  Those MFMAs are written as inline assembly on
// a[16dt:16dt+15]; so are the zeroing, the lazy rescale and the final reads of
// O^T.  The compiler does not see that a[0:63] hold live values, so the
// library build scans the generated assembly and fails if any instruction
// outside these statements names a0..a63.  The compiler does not see either
// that the statements are MFMAs, so they carry their own wait states: two
// before an MFMA whose operand the VALU may just have written (the weights P,
// -m), and 20 (the scores) or 24 (O^T at the end) between the last MFMA writing
// a register and the first VALU instruction reading it.  The build also scans
// the generated assembly for any instruction (its own or the compiler's) that
// touches an MFMA result with fewer than 12 wait states (what the compiler
// itself inserts for these MFMAs), or feeds an MFMA a VALU result with fewer
// than 2.
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators, so a row max needs one cross-half exchange, the row sum
// none until the end, and the rescale is a per-lane scalar.  The key order
// inside a tile is permuted (kappa below) so that each lane's 16 softmax
// values per key block are 16 consecutive keys, which is what the P^T
// operand of the value product needs; the softmax is order-free over keys.
// The K tile is staged into LDS already in that order (row m holds key
// kappa(m)), so the fragment reads walk consecutive rows.
//
// Schedule: the eight waves form two groups (waves 0-3 and 4-7, one wave of
// each per SIMD) that play ping-pong.  A key-tile step has two halves
// separated by work-group barriers: an MFMA half (value MFMAs of tile j-1,
// score MFMAs of tile j) and a softmax half (weights of tile j; staging of
// the group's share of the next K/V tiles).  Group 1 runs one half behind
// group 0, so on every SIMD one wave issues MFMAs while the other does its
// softmax.  (The compiler moves the exponentials of the softmax half down to
// the start of the next MFMA half, next to the value MFMAs that use them;
// pinning them in the softmax half measured slower, as the other wave's MFMAs
// halve a wave's VALU issue rate.)  K/V tiles are gathered from the ring slots with raw buffer loads
// into registers and written to padded LDS rows (conflict-free 16-byte
// fragment reads) one step later: a tile inside one frame takes a fixed lane
// offset plus a scalar base; a tile straddling two frames (or past the
// context's end) takes per-row offsets.  Keys are stored rotated in the ring.
#include "device_common.h"
#include "kernels.h"

namespace rfattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockM = kAttnBlockM;       // query rows per work item (256)
constexpr int kBlockN = kAttnBlockN;       // keys per tile (64)
constexpr int kThreads = 512;              // 8 waves of 32 query rows
constexpr int kKRow = kHeadDim + 8;        // LDS row stride of K tile (272 B: conflict-free 16 B reads)
constexpr int kVRow = kBlockN + 8;         // LDS row stride of V^T tile (144 B)
constexpr int kKTile = kBlockN * kKRow;    // elements
constexpr int kVTile = kHeadDim * kVRow;   // elements
constexpr size_t kLdsBytes = 2 * (kKTile + kVTile) * sizeof(uint16_t);  // K and V, two each
constexpr float kRescaleLog2 = 8.0f;       // rescale O only when a row max grows by > 2^8
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;   // buffer offset past the end: the load returns 0
constexpr int kXcds = 8;                   // MI355X: work-groups go round-robin over 8 XCDs


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
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// ---- O^T in accumulation registers a[0:63] (block dt in a[16dt:16dt+15]) --------
#define RF_O_REGS                                                                                                 \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", "a16", "a17", \
      "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", "a32", "a33", \
      "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", \
      "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63"
#define RF_FOR64(M)                                                                                                \
  M(0) M(1) M(2) M(3) M(4) M(5) M(6) M(7) M(8) M(9) M(10) M(11) M(12) M(13) M(14) M(15) M(16) M(17) M(18) M(19)    \
  M(20) M(21) M(22) M(23) M(24) M(25) M(26) M(27) M(28) M(29) M(30) M(31) M(32) M(33) M(34) M(35) M(36) M(37)    \
  M(38) M(39) M(40) M(41) M(42) M(43) M(44) M(45) M(46) M(47) M(48) M(49) M(50) M(51) M(52) M(53) M(54) M(55)    \
  M(56) M(57) M(58) M(59) M(60) M(61) M(62) M(63)
#define RF_ZERO1(n) "v_accvgpr_write_b32 a" #n ", 0\n\t"
#define RF_SCALE1(n) "v_accvgpr_read_b32 %0, a" #n "\n\tv_mul_f32 %0, %0, %1\n\tv_accvgpr_write_b32 a" #n ", %0\n\t"
#define RF_RD1(i, n) "v_accvgpr_read_b32 %" #i ", a" #n "\n\t"
#define RF_RD16(n0, n1, n2, n3, n4, n5, n6, n7, n8, n9, n10, n11, n12, n13, n14, n15)                          \
  RF_RD1(0, n0) RF_RD1(1, n1) RF_RD1(2, n2) RF_RD1(3, n3) RF_RD1(4, n4) RF_RD1(5, n5) RF_RD1(6, n6) RF_RD1(7, n7) \
      RF_RD1(8, n8) RF_RD1(9, n9) RF_RD1(10, n10) RF_RD1(11, n11) RF_RD1(12, n12) RF_RD1(13, n13) RF_RD1(14, n14) \
          RF_RD1(15, n15)
#define RF_OUT16(r)                                                                                               \
  "=v"(r[0]), "=v"(r[1]), "=v"(r[2]), "=v"(r[3]), "=v"(r[4]), "=v"(r[5]), "=v"(r[6]), "=v"(r[7]), "=v"(r[8]),     \
      "=v"(r[9]), "=v"(r[10]), "=v"(r[11]), "=v"(r[12]), "=v"(r[13]), "=v"(r[14]), "=v"(r[15])

// O^T block dt += A . B (A: 32 dims x 16 keys of V^T, B: 16 keys x 32 queries of
// P^T).  The four blocks of one 16-key group take the same B operand in the order
// dt = 0..3; the s_nop 1 before the first covers a B operand written by the VALU
// just before (the next three read it after that first MFMA has issued).
template <int DT>
__device__ __forceinline__ void mfma_o(bf16x8 a, u32x4 b);
template <>
__device__ __forceinline__ void mfma_o<0>(bf16x8 a, u32x4 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[0:15], %0, %1, a[0:15]" ::"v"(a), "v"(b)
               : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15");
}
template <>
__device__ __forceinline__ void mfma_o<1>(bf16x8 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 a[16:31], %0, %1, a[16:31]" ::"v"(a), "v"(b)
               : "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31");
}
template <>
__device__ __forceinline__ void mfma_o<2>(bf16x8 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 a[32:47], %0, %1, a[32:47]" ::"v"(a), "v"(b)
               : "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47");
}
template <>
__device__ __forceinline__ void mfma_o<3>(bf16x8 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 a[48:63], %0, %1, a[48:63]" ::"v"(a), "v"(b)
               : "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63");
}

// The context a work item attends over: the ring's buffers and capacity, the
// slot of its first frame (frame shift included) and its keys.
struct CtxView {
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  int W;
  int ctx_slot0;
  int ctx_keys;
  int key_tiles;
  int64_t ctx_t0;  // absolute frame of the first context frame (keys rotated on load only)
};

// One work item: query tile qt of head h of segment sg over context cv, key
// tiles [ka, kb).  A complete item (all key tiles) writes the normalised bf16
// output; a piece of a split tile writes its partial result to `part`.
// kRotK (a measurement variant): the ring holds un-rotated keys, and every K
// tile is rotated by 3D-RoPE in float32 as it is staged into LDS, i.e. once per
// query tile that reads it instead of once when it enters the ring.
template <bool kSmallN, bool kRotK = false>
__device__ __forceinline__ void run_item(const AttnArgs& a, uint16_t* lds, const SegDev& sg, const CtxView& cv,
                                         int h, int qt, int ka, int kb, float* part) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // query column of this lane in the 32x32 tiles
  const int hf = lane >> 5;  // lane half: selects k-slots 0-7 / 8-15 of an MFMA step

  // ---- Q fragment: RoPE'd and scaled by c = scale*log2(e) on load, rounded to
  // bf16 once; lane holds query row lr, dims 16s+8hf..+7.  The score MFMAs then
  // yield scaled scores in log2 units directly.
  const int qi = qt * kBlockM + wave * 32 + lr;
  const bool qvalid = qi < sg.q_tokens;
  bf16x8 qf[8];
  if (qvalid) {
    const int pos = qi + sg.q_tok0;  // token index counted from the start of frame q_t0
    const int f = pos / a.N;
    const int pin = pos - f * a.N;
    const int row = pin / a.gw;
    const int col = pin - row * a.gw;
    const uint16_t* qrow = sg.q + (int64_t)qi * sg.q_ld + h * kHeadDim;
    const double cl64 = (double)a.c_log2;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + hf;
      u32x4 x = *(const u32x4*)(qrow + 8 * c);
      qf[s] = as_bf16x8(rope_chunk_scaled(x, 4 * c, sg.q_t0 + frame_shift(a.fs) + f, row, col, a.tab, cl64));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  // ---- tile loaders (byte offsets into the rings, raw buffer loads) ------------
  // The K pipeline runs one tile ahead of the V pipeline: tile j's keys are
  // needed in iteration j (scores), its values in iteration j+1 (after the
  // softmax), so two LDS buffers per operand suffice.
  const int nkeys = cv.ctx_keys;
  const int ntiles = kb - ka;  // key tiles of this item: ka .. kb-1
  const int N = a.N;
  const int W = cv.W;
  const uint32_t slot_b = (uint32_t)a.slot_elems * 2u;
  const uint32_t ring_b = slot_b * (uint32_t)W;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(cv.k_ring), 0, (int)ring_b, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(cv.v_ring), 0, (int)ring_b, kBufferWord3);
  const uint32_t k_head = (uint32_t)h * (uint32_t)N * (kHeadDim * 2u);  // K: [H][N][D]
  const uint32_t v_head = (uint32_t)h * kHeadDim * (uint32_t)N * 2u;    // V: [H][N/8][D][8]
  // K: rows (tid>>4) + 32i, 16-byte chunk tid&15.  V^T: dims (tid>>3) + 64i, key chunk tid&7
  // (8 keys of one dim: one 16-byte chunk of the ring's [n/8][d][8] blocks, 2 KB per key group).
  const int k_r0 = tid >> 4, k_c = tid & 15;
  // LDS row of key k_r0 (and 32 + k_r0): the inverse of the key order kappa the
  // score MFMAs read in (below)
  const int k_lds = (k_r0 & 3) + 4 * ((k_r0 >> 4) & 1) + 8 * ((k_r0 >> 2) & 3);
  const int v_d0 = tid >> 3, v_kc = tid & 7;
  // Lane parts of the byte offsets for a tile inside one frame; row i adds a
  // uniform 32*i rows (K) or 64*i dims (V), carried in the scalar offset.
  const uint32_t k_lane = (uint32_t)k_r0 * (kHeadDim * 2u) + 16u * k_c;
  const uint32_t v_lane = (uint32_t)v_d0 * 16u + 2048u * v_kc;
  u32x4 kst[2], vst[2];
  int kst_n = 0, kst_fr = 0, kst_lim = 0;  // kRotK: position of the tile in kst (wave-uniform)

  // Cursors of the next tile to load (uniform): slot and token offset of its
  // first key, starting at key tile ka; kfr counts the K cursor's frames.
  int kslot, kn, kfr;
  {
    const int key0 = ka * kBlockN;
    const int f0 = key0 / N;
    kn = key0 - f0 * N;
    kslot = (cv.ctx_slot0 + f0) % W;
    kfr = f0;
  }
  int kload = ka;
  int vslot = kslot, vn = kn, vload = ka;
  auto advance = [&](int& slot, int& n) {
    n += kBlockN;
    while (n >= N) {
      n -= N;
      slot = (slot + 1 == W) ? 0 : slot + 1;
    }
  };

  // kRotK: rotate row i of the staged chunk in place, its key being in-frame token
  // n of context frame fr: float32 products, one rounding to bf16.
  const float2* tab_t = a.tab.t;
  const float2* tab_h = a.tab.h;
  const float2* tab_w = a.tab.w;
  const int tab_pt = a.tab.pt, tab_ph = a.tab.ph, tab_pw = a.tab.pw;
  const int gw = a.gw;
  auto rotate_row = [&](int i, int fr, int n) {
    const int row = n / gw;
    const int col = n - row * gw;
    const int64_t t = cv.ctx_t0 + fr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 4 * k_c + j;
      const float2* ptr = p < tab_pt ? tab_t + t * tab_pt + p
                          : (p < tab_pt + tab_ph ? tab_h + row * tab_ph + (p - tab_pt)
                                                 : tab_w + col * tab_pw + (p - tab_pt - tab_ph));
      const float2 cs = *ptr;
      const float x0 = bf16_to_f32(kst[i][j] & 0xFFFFu), x1 = bf16_to_f32(kst[i][j] >> 16);
      kst[i][j] = pack2(x0 * cs.x - x1 * cs.y, x0 * cs.y + x1 * cs.x);
    }
  };

  auto load_k = [&]() {
    const int key_lim = nkeys - kload * kBlockN;  // valid keys in this tile (may be <= 0)
    kst_n = kn;
    kst_fr = kfr;
    kst_lim = key_lim;
    if (!kSmallN && kn + kBlockN <= N && key_lim >= kBlockN) {
      // whole tile in one frame, all keys valid: lane offset + uniform offset
      const uint32_t base = (uint32_t)kslot * slot_b + k_head + (uint32_t)kn * (kHeadDim * 2u);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        kst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               krs, k_lane, base + (uint32_t)i * (32u * kHeadDim * 2u), 0));
    } else {
      uint32_t off[2];
      if constexpr (!kSmallN) {
        const int b = N - kn;  // keys of this tile still in the current frame
        const int nxt = (kslot + 1 == W) ? 0 : kslot + 1;
        const uint32_t ba = (uint32_t)kslot * slot_b + k_head + (uint32_t)kn * (kHeadDim * 2u);
        const uint32_t bb = (uint32_t)nxt * slot_b + k_head - (uint32_t)b * (kHeadDim * 2u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = k_r0 + 32 * i;
          off[i] = (uint32_t)r * (kHeadDim * 2u) + 16u * k_c + (r < b ? ba : bb);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          int n = kn + k_r0 + 32 * i, slot = kslot;
          while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
          off[i] = (uint32_t)slot * slot_b + k_head + (uint32_t)n * (kHeadDim * 2u) + 16u * k_c;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (k_r0 + 32 * i >= key_lim) off[i] = kOutOfRange;  // past the end: zeros
        kst[i] = bload(krs, off[i]);
      }
    }
    kn += kBlockN;
    while (kn >= N) {
      kn -= N;
      kslot = (kslot + 1 == W) ? 0 : kslot + 1;
      ++kfr;
    }
    ++kload;
  };

  auto load_v = [&]() {
    const int key_lim = nkeys - vload * kBlockN;
    if (!kSmallN && vn + kBlockN <= N && key_lim >= kBlockN) {
      const uint32_t base = (uint32_t)vslot * slot_b + v_head + (uint32_t)(vn / 8) * 2048u;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        vst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               vrs, v_lane, base + (uint32_t)i * 64u * 16u, 0));
    } else {
      uint32_t base;
      if constexpr (!kSmallN) {
        const int b = N - vn;
        const int nxt = (vslot + 1 == W) ? 0 : vslot + 1;
        // chunk c of the tile is key group vn/8 + c of this frame, or group
        // vn/8 + c - N/8 of the next one (b and N are multiples of 8)
        base = (8 * v_kc < b) ? (uint32_t)vslot * slot_b + v_head + (uint32_t)(vn / 8) * 2048u
                              : (uint32_t)nxt * slot_b + v_head + (uint32_t)(vn / 8) * 2048u -
                                    (uint32_t)(N / 8) * 2048u;
      } else {
        int n = vn + 8 * v_kc, slot = vslot;
        while (n >= N) { n -= N; slot = (slot + 1 == W) ? 0 : slot + 1; }
        base = (uint32_t)slot * slot_b + v_head + (uint32_t)(n / 8) * 2048u - 2048u * v_kc;
      }
      const bool valid = 8 * v_kc < key_lim;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t off = base + v_lane + (uint32_t)i * 64u * 16u;
        vst[i] = bload(vrs, valid ? off : kOutOfRange);
      }
    }
    advance(vslot, vn);
    ++vload;
  };

  auto store_k = [&](int buf) {
    uint16_t* Kl = lds + buf * kKTile;
    if constexpr (kRotK) {  // rows past the context's end hold zeros and stay so
      const int b = N - kst_n;  // keys of the tile in its first frame
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = k_r0 + 32 * i;
        if (r < kst_lim) {
          if (r < b) rotate_row(i, kst_fr, kst_n + r);
          else rotate_row(i, kst_fr + 1, kst_n + r - N);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4*)(Kl + (k_lds + 32 * i) * kKRow + 8 * k_c) = kst[i];
  };
  auto store_v = [&](int buf) {
    uint16_t* Vl = lds + 2 * kKTile + buf * kVTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4*)(Vl + (v_d0 + 64 * i) * kVRow + 8 * v_kc) = vst[i];
  };

  // ---- running state -----------------------------------------------------------
  asm volatile(RF_FOR64(RF_ZERO1) ::: RF_O_REGS);  // O^T = 0
  // Running row max m (log2 units).  The score MFMAs subtract it themselves:
  // the first k-step of each key block accumulates onto negm, -m in all 16
  // entries (every entry of a lane's accumulator belongs to its query).
  float m_run = 0.0f;
  float l_run = 0.0f;  // this lane's partial row sum of the bf16 weights
  f32x16 negm = {};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // A-operand row m of the score MFMA is LDS row m of the K tile, which the
  // staging filled with key kappa(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3) (k_lds is
  // the inverse): lane half hf of output register i then holds key 16*hf + i of
  // each 32-key block, and a quarter-wave's fragment reads cover 16 consecutive
  // rows, which the 272-byte row stride spreads over all LDS banks.

  // T^T = K Q'^T - m for keys [0,32) and [32,64) of the tile in K buffer `buf`
  // (Q' = c Q): the exponents of the softmax weights in log2 units.  All 16
  // K fragments are read before the first MFMA (sched_barrier keeps the
  // compiler from sinking the reads next to their MFMAs), so LDS latency is
  // paid once per block.  The Q' fragments are B operands taken from
  // accumulation registers.  Eight statements of two MFMAs each let every
  // pair start as soon as its two fragments have arrived; the last one waits
  // out the MFMA latency before the softmax reads the scores.
  // Both MFMA blocks run at raised wave priority.
  auto scores = [&](int buf, f32x16& s0, f32x16& s1) {
    const uint16_t* Kl = lds + buf * kKTile;
    __builtin_amdgcn_s_setprio(1);
    bf16x8 kf[16];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[2 * s] = *(const bf16x8*)(Kl + lr * kKRow + 16 * s + 8 * hf);
      kf[2 * s + 1] = *(const bf16x8*)(Kl + (32 + lr) * kKRow + 16 * s + 8 * hf);
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %5, %4\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %5, %4"
                 : "=&v"(s0), "=&v"(s1)
                 : "v"(kf[0]), "v"(kf[1]), "v"(negm), "a"(qf[0]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[2]), "v"(kf[3]), "a"(qf[1]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[4]), "v"(kf[5]), "a"(qf[2]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[6]), "v"(kf[7]), "a"(qf[3]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[8]), "v"(kf[9]), "a"(qf[4]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[10]), "v"(kf[11]), "a"(qf[5]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[12]), "v"(kf[13]), "a"(qf[6]));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %3, %4, %1\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(s0), "+v"(s1)
                 : "v"(kf[14]), "v"(kf[15]), "a"(qf[7]));
    __builtin_amdgcn_s_setprio(0);
  };

  // Row max of a tile's exponents (both lane halves).
  auto tile_max = [&](const f32x16& s0, const f32x16& s1) -> float {
    // two chains of 3-input maxima
    float ma = __builtin_elementwise_maximum(s0[0], s0[1]);
    float mb = __builtin_elementwise_maximum(s1[0], s1[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      ma = __builtin_elementwise_maximum(__builtin_elementwise_maximum(ma, s0[i]), s0[i + 1]);
      mb = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mb, s1[i]), s1[i + 1]);
    }
    return xhalf_max(__builtin_elementwise_maximum(ma, mb));
  };

  // Move the running max up to m_new: shift this tile's exponents, rescale l
  // and O^T (in its accumulation registers), refresh -m for the MFMAs.
  auto raise_max = [&](float m_new, f32x16& s0, f32x16& s1) {
    const float delta = m_new - m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] -= delta;
      s1[i] -= delta;
    }
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    l_run *= alpha;
    float t;
    asm volatile(RF_FOR64(RF_SCALE1) : "=&v"(t) : "v"(alpha) : RF_O_REGS);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m_new;
  };

  // Online softmax of one tile: the running max only moves when some row's
  // exponent exceeds 8 (wave-uniform decision, weights stay <= 2^8 meanwhile);
  // then bf16 weights 2^t into pw, summed into l.
  auto softmax = [&](f32x16& s0, f32x16& s1, u32x4 (&pw)[4]) {
    const float mt = tile_max(s0, s1);
    if (__builtin_amdgcn_ballot_w64(mt > kRescaleLog2) != 0)
      raise_max(m_run + fmaxf(mt, 0.0f), s0, s1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a0 = __builtin_amdgcn_exp2f(s0[2 * e]);
      const float a1 = __builtin_amdgcn_exp2f(s0[2 * e + 1]);
      const float b0 = __builtin_amdgcn_exp2f(s1[2 * e]);
      const float b1 = __builtin_amdgcn_exp2f(s1[2 * e + 1]);
      const uint32_t pa = pack2(a0, a1), pb = pack2(b0, b1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pa), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb), ones, l_run, false);
      pw[e >> 2][e & 3] = pa;
      pw[2 + (e >> 2)][e & 3] = pb;
    }
  };

  // O^T += V^T P^T with the values in V buffer `buf` (fragments read up front)
  auto values = [&](int buf, const u32x4 (&pw)[4]) {
    const uint16_t* Vl = lds + 2 * kKTile + buf * kVTile;
    __builtin_amdgcn_s_setprio(1);
    bf16x8 vf[16];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int bu = 0; bu < 4; ++bu)
        vf[4 * dt + bu] = *(const bf16x8*)(Vl + (32 * dt + lr) * kVRow + 32 * (bu >> 1) + 16 * hf + 8 * (bu & 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int bu = 0; bu < 4; ++bu) {
      mfma_o<0>(vf[bu], pw[bu]);
      mfma_o<1>(vf[4 + bu], pw[bu]);
      mfma_o<2>(vf[8 + bu], pw[bu]);
      mfma_o<3>(vf[12 + bu], pw[bu]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Keys past the end of the context (only in key tile key_tiles-1) get no weight.
  auto mask_tail = [&](int tile, f32x16& s0, f32x16& s1) {
    const int key_lim = nkeys - tile * kBlockN;
    if (key_lim < kBlockN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * hf + i >= key_lim) s0[i] = -INFINITY;
        if (32 + 16 * hf + i >= key_lim) s1[i] = -INFINITY;
      }
    }
  };

  // ---- software pipeline over key tiles: two wave groups in ping-pong --------
  // Group 0 (waves 0-3) and group 1 (waves 4-7) put one wave on each SIMD.
  // Each step has two halves separated by barriers: an MFMA half (values of
  // tile j-1, scores of tile j) and a softmax half (weights of tile j, and
  // staging this group's share of the next K/V tiles).  Group 1 runs one half
  // behind group 0, so on every SIMD one wave's MFMAs overlap the other
  // wave's softmax.  Group g stages K_{j+1+g} and V_{j+g} in the softmax half
  // of step j: both shares of K_{j+1}, V_j are in LDS before group 0's MFMA
  // half of step j+1, and no buffer is written while a group still reads it.
  const int grp = __builtin_amdgcn_readfirstlane(wave) >> 2;  // wave-uniform
  load_k();  // K_0
  store_k(0);
  load_k();  // K_1
  load_v();  // V_0
  __syncthreads();
  if (grp == 1) {  // group 1's extra first half
    store_k(1);
    store_v(0);
    load_k();  // K_2
    load_v();  // V_1
    __syncthreads();
  }
  // A wave whose 32 query rows all lie past the segment's end (the last query
  // tile of a segment that is not a multiple of 256 rows) computes nothing: it
  // only stages its share of the K/V tiles and keeps the barriers, in a loop of
  // its own (the working waves' loop is left as it is).  Its O^T, m and l stay
  // 0; no output row of it is ever written.
  const bool live = __builtin_amdgcn_readfirstlane(wave) * 32 < sg.q_tokens - qt * kBlockM;
  f32x16 x0, x1;
  u32x4 pw[4];
  if (live) {
    for (int j = 0; j < ntiles; ++j) {
      if (j > 0) values((j - 1) & 1, pw);
      scores(j & 1, x0, x1);
      __syncthreads();
      if (j == ntiles - 1) mask_tail(kb - 1, x0, x1);
      if (j == 0) {  // first tile: the running max starts at its row max
        const float m0 = tile_max(x0, x1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x0[i] -= m0;
          x1[i] -= m0;
        }
        m_run = m0;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m0;
      }
      softmax(x0, x1, pw);
      store_k((j + 1 + grp) & 1);
      store_v((j + grp) & 1);
      load_k();
      load_v();
      __syncthreads();
    }
    values((ntiles - 1) & 1, pw);
  } else {
    for (int j = 0; j < ntiles; ++j) {
      __syncthreads();
      store_k((j + 1 + grp) & 1);
      store_v((j + grp) & 1);
      load_k();
      load_v();
      __syncthreads();
    }
  }
  if (grp == 0) __syncthreads();  // the same barrier count as group 1

  // O^T out of the accumulation registers, once the last MFMAs have drained.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: RF_O_REGS);
  f32x16 o[4];
  {
    float r[4][16];
    asm volatile(RF_RD16(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15) : RF_OUT16(r[0]));
    asm volatile(RF_RD16(16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31) : RF_OUT16(r[1]));
    asm volatile(RF_RD16(32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47) : RF_OUT16(r[2]));
    asm volatile(RF_RD16(48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63) : RF_OUT16(r[3]));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = r[dt][i];
  }

  // ---- epilogue --------------------------------------------------------------------
  const float l_tot = xhalf_sum(l_run);
  if (ka == 0 && kb == cv.key_tiles) {  // whole item: O = O^T / l, bf16, token-major
    const float inv = 1.0f / l_tot;
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
  } else {  // piece of a split tile: unnormalised O [chunk][row][8], then m[row], l[row]
    // Chunk c = 4 dt + g4 holds dims 32 dt + 8 g4 + 0..7 of every row, so one store
    // instruction of a wave (32 rows x both halves) writes 1 KB contiguous.
    const int r = wave * 32 + lr;  // row inside the query tile
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 w = {o[dt][4 * g4 + 0], o[dt][4 * g4 + 1], o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]};
        *(f32x4*)(part + ((4 * dt + g4) * kPartRows + r) * 8 + 4 * hf) = w;
      }
    if (hf == 0) {
      part[kPartRows * kHeadDim + r] = m_run;
      part[kPartRows * kHeadDim + kPartRows + r] = l_tot;
    }
  }
}

// The launch's context in window mode: the ring descriptor as the device holds it
// now (capacity clamped to the validated one, at least one frame of the window).
__device__ __forceinline__ CtxView window_view(const AttnArgs& a) {
  const DevRing* r = a.ring_dev;
  const int cap = r->capacity;
  const int W = cap < 1 ? 1 : (cap > a.W ? a.W : cap);
  const int cnt = r->count < 1 ? 1 : (r->count > W ? W : r->count);
  const int keys = cnt * a.N;
  return CtxView{r->k, r->v, W, (int)mod_pos(r->first, W), keys, (keys + kBlockN - 1) / kBlockN, r->first};
}

// The context of segment sg: the window (window mode) or its own range.
__device__ __forceinline__ CtxView seg_view(const AttnArgs& a, const SegDev& sg, const CtxView& wv) {
  if (a.ring_dev) return wv;
  const int W = a.W;
  const int64_t sh = frame_shift(a.fs);
  return CtxView{a.k_ring, a.v_ring, W, (sg.ctx_slot0 + (int)(sh % W)) % W, sg.ctx_keys, sg.key_tiles,
                 sg.ctx_t0 + sh};
}

// Segment of query tile `tile` (segments are found by their first tile).
__device__ __forceinline__ int tile_segment(const AttnArgs& a, int tile) {
  int si = 0;
#pragma unroll
  for (int s = 1; s < kMaxSegments; ++s)
    if (s < a.n_segs && tile >= a.seg[s].tile_begin) si = s;
  return si;
}

// Key tiles [ka, kb) of piece c of a query tile cut into n_split equal key ranges.
__device__ __forceinline__ int piece_begin(int c, int key_tiles, int n_split) { return c * key_tiles / n_split; }

// Work-group -> (split tile, piece) of the last round(s): pieces are numbered
// piece-major (all tiles' piece 0, then piece 1, ...) and dealt XCD-contiguously,
// so the work-groups of one XCD run the same key range of consecutive query tiles
// of one head at the same time and share those keys and values in their L2.
__device__ __forceinline__ void split_piece(const AttnArgs& a, int b, int* tile, int* c) {
  const int n_pieces = a.split_tiles * a.n_split;
  const int pi = xcd_tile(b, n_pieces);
  *c = pi / a.split_tiles;
  *tile = a.dp_tiles + (pi - *c * a.split_tiles);
}

// kSmallN: frames shorter than a key tile (a tile may cover 3+ frames); the
// general per-row frame walk is used.  Otherwise a tile straddles at most one
// frame boundary and each row picks one of two bases.
template <bool kSmallN, bool kRotK>
__global__ __launch_bounds__(kThreads, 1) void window_attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  CtxView wv{};
  if (a.ring_dev) wv = window_view(a);
  int tile, c = 0;
  if ((int)blockIdx.x < a.dp_tiles) {
    tile = xcd_tile(blockIdx.x, a.dp_tiles);  // whole query tiles in XCD-contiguous order
  } else {
    split_piece(a, (int)blockIdx.x - a.dp_tiles, &tile, &c);
  }
  const SegDev& sg = a.seg[tile_segment(a, tile)];
  const CtxView cv = seg_view(a, sg, wv);
  const int tl = tile - sg.tile_begin;
  const int h = tl / sg.q_tiles;
  const int qt = tl - h * sg.q_tiles;
  if ((int)blockIdx.x < a.dp_tiles) {
    run_item<kSmallN, kRotK>(a, lds, sg, cv, h, qt, 0, cv.key_tiles, nullptr);
    return;
  }
  // one of the n_split key ranges of a split tile: a partial result for the merge
  const int ka = piece_begin(c, cv.key_tiles, a.n_split);
  const int kb = piece_begin(c + 1, cv.key_tiles, a.n_split);
  if (ka == kb) return;  // window mode: fewer key tiles at run time than pieces (the merge skips it)
  float* part = a.partial + (size_t)((tile - a.dp_tiles) * a.n_split + c) * kPartFloats;
  run_item<kSmallN, kRotK>(a, lds, sg, cv, h, qt, ka, kb, part);
}

// Merge the n_split pieces of split tile dp_tiles + blockIdx.x:
// O = sum 2^(m_i - M) O_i / sum 2^(m_i - M) l_i, M = max m_i (pieces in order).
// Thread t merges row t/2, dims 8c + 4(t%2) + 0..3 of every chunk c: the loads
// of a wave read 1 KB contiguous.  The bf16 rows are staged in LDS (16-byte
// chunk c of row r at position c ^ (r mod 16)) and written 256 bytes per row.
__global__ __launch_bounds__(2 * kPartRows) void window_attn_fixup(AttnArgs a) {
  constexpr int kChunks = kHeadDim / 8;
  __shared__ __attribute__((aligned(16))) uint16_t img[kPartRows * kHeadDim];
  CtxView wv{};
  if (a.ring_dev) wv = window_view(a);
  const int tile = a.dp_tiles + (int)blockIdx.x;
  const SegDev& sg = a.seg[tile_segment(a, tile)];
  const int kt = seg_view(a, sg, wv).key_tiles;
  const int tl = tile - sg.tile_begin;
  const int h = tl / sg.q_tiles;
  const int qt = tl - h * sg.q_tiles;
  const int r = threadIdx.x >> 1;  // row inside the query tile
  const int jh = threadIdx.x & 1;  // which four of each chunk's eight dims
  const float* base = a.partial + (size_t)blockIdx.x * a.n_split * kPartFloats;

  float M = -INFINITY;
  for (int c = 0; c < a.n_split; ++c) {
    if (piece_begin(c, kt, a.n_split) == piece_begin(c + 1, kt, a.n_split)) continue;  // no piece
    M = fmaxf(M, base[(size_t)c * kPartFloats + kPartRows * kHeadDim + r]);
  }
  f32x4 acc[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float L = 0.0f;
  for (int c = 0; c < a.n_split; ++c) {
    if (piece_begin(c, kt, a.n_split) == piece_begin(c + 1, kt, a.n_split)) continue;
    const float* p = base + (size_t)c * kPartFloats;
    const float sc = __builtin_amdgcn_exp2f(p[kPartRows * kHeadDim + r] - M);
    L += sc * p[kPartRows * kHeadDim + kPartRows + r];
    const float* src = p + r * 8 + 4 * jh;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const f32x4 x = *(const f32x4*)(src + q * kPartRows * 8);
      acc[q][0] += sc * x[0];
      acc[q][1] += sc * x[1];
      acc[q][2] += sc * x[2];
      acc[q][3] += sc * x[3];
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const u32x2 w = {pack2(acc[q][0] * inv, acc[q][1] * inv), pack2(acc[q][2] * inv, acc[q][3] * inv)};
    *(u32x2*)(img + r * kHeadDim + (q ^ (r & 15)) * 8 + 4 * jh) = w;
  }
  __syncthreads();
  const int q = threadIdx.x & (kChunks - 1);  // 16-byte chunk of the row
  for (int rr = threadIdx.x / kChunks; rr < kPartRows; rr += 2 * kPartRows / kChunks) {
    const int qi = qt * kBlockM + rr;
    if (qi < sg.q_tokens)
      *(u32x4*)(sg.o + (int64_t)qi * sg.o_ld + h * kHeadDim + q * 8) =
          *(const u32x4*)(img + rr * kHeadDim + (q ^ (rr & 15)) * 8);
  }
}

hipError_t prepare_window_attn() {
  hipError_t e = hipFuncSetAttribute((const void*)window_attn_kernel<false, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)window_attn_kernel<true, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)window_attn_kernel<false, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  return e;
}

hipError_t launch_window_attn(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.dp_tiles + a.split_tiles * a.n_split));
  if (a.rot_k)  // the host admits it for frames of at least one key tile only
    hipLaunchKernelGGL((window_attn_kernel<false, true>), grid, dim3(kThreads), kLdsBytes, s, a);
  else if (a.N < kBlockN)
    hipLaunchKernelGGL((window_attn_kernel<true, false>), grid, dim3(kThreads), kLdsBytes, s, a);
  else
    hipLaunchKernelGGL((window_attn_kernel<false, false>), grid, dim3(kThreads), kLdsBytes, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split_tiles == 0 || a.n_split == 1) return e;
  hipLaunchKernelGGL(window_attn_fixup, dim3((unsigned)a.split_tiles), dim3(2 * kPartRows), 0, s, a);
  return hipGetLastError();
}

}  // namespace rfattn
