/*
 * rfattn.h -- C ABI of librfattn: rolling-window DiT attention with 3D-RoPE
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the problem statement of the source pages (the
 * Amazon Science post "A kernel-centric path to real-time video generation
 * on Trainium" and its digests):
 *   - video RoPE rotates over three axes, time, height and width
 *     ("Amazon and Reactor tune Trainium for real-time video generation",
 *     section "Three problems for generic compilers");
 *   - every layer reads and writes a rolling KV cache, frames are generated
 *     and evicted in a sliding window, and attention lengths vary between
 *     passes (same section);
 *   - 23,400 query tokens attend to 32,760 context tokens over 12 heads
 *     (ai4snews digest, second paragraph; brifing.si "Optimizing Real-Time
 *     Video Generation on Trainium Chips", section 4);
 *   - the denoise pass and the lighter cache-update pass run batched
 *     together ("Optimizing Real-Time Video Generation on Trainium Chips",
 *     section 8; vibeleaderboard digest, key takeaways);
 *   - transposes happen inside the kernels, never as passes of their own
 *     (vibeleaderboard digest, key takeaways; ai4snews, first paragraph).
 *
 * Conventions shared by every call:
 *   - Tensors are bf16 (raw 16-bit patterns) in device memory that the
 *     CALLER owns.  The library allocates device memory only in rf_create
 *     (the RoPE tables and the attention workspace) and frees it in
 *     rf_destroy; no call allocates.
 *   - Calls are asynchronous and stream-ordered: work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream)
 *     and the call returns without synchronising.
 *   - Validation happens on the host before anything is enqueued.  On any
 *     error nothing is enqueued and no descriptor is modified.  RF_ERR_HIP
 *     reports a failed launch; rf_last_error() gives the detail.
 *   - "Token-major" means [tokens][ld] elements, heads contiguous inside a
 *     row: element (token i, head h, dim d) is at i*ld + h*head_dim + d.
 *     ld is in elements, >= n_heads*head_dim and a multiple of 8; every
 *     pointer is 16-byte aligned.
 *   - Token positions: token i of a block whose first frame is t0 is at
 *     (frame t0 + i/N, row (i%N)/grid_w, column i%grid_w), N = grid_h*grid_w.
 *     Frames are absolute latent frame indices in 0..max_frame-1.
 *
 * Notes for callers written against a plainer sketch of this interface
 * (V ring [W][H][N][D], frame counts everywhere, one ld per call):
 *   - the V ring is [W][H][N/8][D][8]: values in blocks of 8 tokens, so the
 *     value product reads 8 consecutive keys of one dim as one 16-byte chunk
 *     and the roll writes whole 1 KB runs; token n, dim d of a head sits at
 *     [n/8][d][n%8] (a caller that inspects V slots reorders the axes);
 *   - rf_rope3d_apply takes a token count (n_frames*N for whole frames) and
 *     separate input and output strides (x_ld, y_ld);
 *   - an rf_attn_segment names its queries as a token range (q_t0, q_tok0,
 *     q_tokens): whole frames are q_tok0 = 0, q_tokens = n_frames*N;
 *   - rf_geom.max_frame is the number of table rows (frames 0..max_frame-1),
 *     i.e. the largest supported frame index plus one.
 */
#ifndef RFATTN_H
#define RFATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RF_OK = 0,
  RF_ERR_NULL = 1,        /* a required pointer is NULL                          */
  RF_ERR_ALIGN = 2,       /* pointer not 16-byte aligned or ld not a multiple of 8 */
  RF_ERR_SHAPE = 3,       /* unsupported geometry or inconsistent sizes          */
  RF_ERR_RANGE = 4,       /* frames outside the ring window or the RoPE tables   */
  RF_ERR_UNSUPPORTED = 5, /* current device is not gfx950                        */
  RF_ERR_HIP = 6          /* HIP runtime error (allocation, copy or launch)      */
} rf_status;

/* Model geometry, fixed for the lifetime of a context. */
typedef struct {
  int32_t grid_h, grid_w;  /* latent frame grid; N = grid_h*grid_w tokens per frame,
                              N must be a multiple of 8                             */
  int32_t n_heads;         /* H >= 1 (query heads == key/value heads)               */
  int32_t head_dim;        /* D; this library supports 128                          */
  int32_t rope_pairs[3];   /* rotation pairs on the time, row and column axes;
                              sum == D/2.  Pair p rotates dims (2p, 2p+1); pairs
                              0..P_t-1 use the frame index, the next P_h the row,
                              the last P_w the column                               */
  double rope_base;        /* frequency base b: pair j of an axis with P pairs
                              turns by pos * b^(-j/P) radians                       */
  int64_t max_frame;       /* frame indices 0..max_frame-1 are supported            */
} rf_geom;

/* Opaque context: the geometry, the device-resident cos/sin tables (each
 * float64 libm cos/sin of pos*b^(-j/P), rounded to float32) and the
 * attention workspace (partial results of query tiles split across
 * work-groups: 2 x CUs x 130 KB, 68 MB on a 256-CU MI355X).  The tables
 * are immutable after creation; rf_rope3d_apply and rf_kvcache_roll may use
 * one context from several threads and streams.  rf_window_attention calls
 * that share a context share its workspace and must be ordered (one stream,
 * or synchronised); use one context per concurrent stream otherwise. */
typedef struct rf_ctx rf_ctx;

/* Validate `g`, check that the current HIP device is gfx950, upload the
 * RoPE tables and allocate the attention workspace.  These are the library's
 * only allocations.  *out is set only on RF_OK.  Synchronous. */
rf_status rf_create(const rf_geom* g, rf_ctx** out);

/* Free a context (NULL is ignored).  The caller must first make sure no work
 * that uses it is still queued.  It frees device memory, which is not
 * allowed while a stream of the device is being captured into a graph (the
 * capture is invalidated): destroy contexts outside captures. */
void rf_destroy(rf_ctx* ctx);

/* Human-readable name of a status code (static storage). */
const char* rf_status_string(rf_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* rf_last_error(void);

/*
 * rf_rope3d_apply -- 3D rotary embedding of a token-major bf16 tensor.
 *
 * Source: RoPE over time, height and width ("Amazon and Reactor tune
 * Trainium for real-time video generation", section "Three problems for
 * generic compilers"; the pages report a hand-written kernel for it,
 * section "Results with the Neuron Kernel Interface").
 *
 * x: [n_tokens][x_ld] bf16, heads contiguous; y: [n_tokens][y_ld].  y may
 * equal x with y_ld == x_ld (in place); other overlaps are not allowed.
 * Token i sits at (t0 + i/N, (i%N)/grid_w, i%grid_w).  For every pair p:
 *   y[2p]   = bf16_rne( fl64( x[2p]*c - x[2p+1]*s ) )
 *   y[2p+1] = bf16_rne( fl64( x[2p]*s + x[2p+1]*c ) )
 * with c, s the float32 table entries; the products are exact in float64,
 * so the result is unique and reproducible bit for bit.
 * n_tokens == 0 is a no-op (x and y are not examined).  Errors: RF_ERR_NULL, RF_ERR_ALIGN,
 * RF_ERR_SHAPE (ld too small, n_tokens < 0), RF_ERR_RANGE (t0 < 0 or the
 * last token's frame >= max_frame).
 */
rf_status rf_rope3d_apply(const rf_ctx* ctx, const void* x, int64_t x_ld, void* y,
                          int64_t y_ld, int64_t t0, int64_t n_tokens, void* stream);

/*
 * Ring-buffer KV cache of `capacity` frame slots.  Frame t lives in slot
 * t % capacity.  Valid frames: first .. first+count-1 (count <= capacity).
 *   k: bf16 [capacity][H][N][D] -- keys, already rotated by 3D-RoPE at their
 *      own positions, head-major inside a slot (rows of D contiguous);
 *   v: bf16 [capacity][H][N/8][D][8] -- values in blocks of 8 tokens: token n,
 *      dim d of head h at [slot][h][n/8][d][n%8] (8 consecutive keys of one
 *      dim are one 16-byte chunk; the 128 dims of a key group are 2 KB).
 * The caller allocates both (capacity*H*N*D*2 bytes each, 16-byte aligned)
 * and zero-fills or otherwise initialises them; a new cache has count == 0.
 * The library reads and writes the descriptor only inside rf_kvcache_roll
 * (and rf_qkv_project).
 * Size limit: the attention kernel addresses each ring buffer with 32-bit
 * byte offsets, so capacity*H*N*D*2 + 16 must not exceed 0x7FFFFFF0
 * (2 GiB - 16 bytes): at most 448 slots at 30x52 tokens, 12 heads of 128.
 * Every call that takes a ring returns RF_ERR_SHAPE for a larger one before
 * anything is enqueued; rf_kvcache_bytes checks a capacity in advance.
 */
typedef struct {
  void* k;
  void* v;
  int32_t capacity; /* W >= 1 */
  int32_t count;    /* 0..capacity */
  int64_t first;    /* oldest valid frame (any value while count == 0) */
} rf_kvcache;

/*
 * rf_kvcache_bytes -- host-only: the size in bytes of one ring buffer (K or
 * V) of `capacity` slots for geometry g, i.e. capacity*H*N*D*2.  Touches no
 * device.  Errors: RF_ERR_NULL (g or bytes NULL), RF_ERR_SHAPE (invalid
 * geometry as in rf_create, capacity < 1, or a ring beyond the size limit
 * above).  *bytes is written only on RF_OK.
 */
rf_status rf_kvcache_bytes(const rf_geom* g, int32_t capacity, int64_t* bytes);

/*
 * rf_kvcache_roll -- write n_frames new frames t0..t0+n_frames-1 into the
 * ring in one pass: keys are rotated by 3D-RoPE (bit-exact, as
 * rf_rope3d_apply) and stored head-major, values are stored in their 8-token
 * blocks (transposed); no separate transpose or copy pass.  Frames already in the window are
 * overwritten in place; later frames are appended, and appending to a full
 * ring evicts the oldest frame (its slot is the one written).  Other slots
 * are left untouched.
 *
 * Source: the rolling KV cache that every layer reads and writes, frames
 * generated and evicted in a sliding window ("Amazon and Reactor tune
 * Trainium for real-time video generation", section "Three problems for
 * generic compilers"); the pages report a hand-written cache-copy kernel
 * (section "Results with the Neuron Kernel Interface").
 *
 * k_new, v_new: token-major [n_frames*N][ld] bf16, un-rotated.
 * Requires 1 <= n_frames <= capacity and, unless the ring is empty,
 * first <= t0 <= first+count (an empty ring starts its window at t0); a ring
 * beyond the size limit gives RF_ERR_SHAPE.
 * On RF_OK, *c's first/count are updated on the host after the kernel is
 * enqueued; on error *c is unchanged.  The caller serialises calls that
 * share a descriptor.
 */
rf_status rf_kvcache_roll(const rf_ctx* ctx, rf_kvcache* c, const void* k_new, int64_t k_ld,
                          const void* v_new, int64_t v_ld, int64_t t0, int32_t n_frames,
                          void* stream);

/*
 * rf_kvcache_plan_roll -- host-only: validate a roll as rf_kvcache_roll
 * would and write the descriptor it would leave into *after (first, count;
 * k, v and capacity copied).  Touches no device.  Lets a caller that keeps
 * one descriptor per layer advance them in lockstep.
 */
rf_status rf_kvcache_plan_roll(const rf_kvcache* c, int64_t t0, int32_t n_frames,
                               rf_kvcache* after);

/*
 * One group of query tokens and the context frames they attend to.  The
 * queries are q_tokens consecutive tokens of the frame sequence, the first
 * being token q_tok0 of frame q_t0: query i sits at frame
 * q_t0 + (q_tok0 + i) / N, in-frame index (q_tok0 + i) % N (its RoPE
 * position).  Whole frames: q_tok0 = 0, q_tokens = frames * N.  A block cut
 * at any token is the sequence split of the pages' hybrid heads x sequence
 * sharding ("Optimizing Real-Time Video Generation on Trainium Chips",
 * section 7 "Hybrid sharding solution"), whose halves of 11,700 tokens cut
 * a frame.
 */
typedef struct {
  const void* q;      /* token-major [q_tokens][q_ld] bf16, un-rotated queries    */
  int64_t q_ld;
  void* o;            /* token-major [q_tokens][o_ld] bf16 output                */
  int64_t o_ld;
  int64_t q_t0;       /* frame index of the first query token                    */
  int32_t q_tok0;     /* 0 <= q_tok0 < N: the first query token's index in frame q_t0 */
  int32_t q_tokens;   /* >= 1                                                     */
  int64_t ctx_t0;     /* context frames ctx_t0 .. ctx_t0+ctx_frames-1, all inside */
  int32_t ctx_frames; /* >= 1                       the ring's valid window       */
  int32_t reserved;   /* 0                                                        */
} rf_attn_segment;

#define RF_MAX_SEGMENTS 8

/*
 * rf_window_attention -- non-causal multi-head attention of each segment's
 * query tokens over its context frames in the ring, all segments in ONE
 * launch (the denoise pass and the cache-update pass batched together).
 *
 * Source: the DiT self-attention, 23,400 queries over 32,760 context
 * tokens in 12 heads, the dominant cost (ai4snews digest, second
 * paragraph); two passes per window, denoise then cache update, with
 * attention lengths that vary ("Amazon and Reactor tune Trainium for
 * real-time video generation", section "Three problems for generic
 * compilers"); batching the two phases ("Optimizing Real-Time Video
 * Generation on Trainium Chips", section 8); transposes fused into the
 * attention kernel (vibeleaderboard digest, key takeaways).
 *
 * For each segment, head h and query token i:
 *   s_j = scale * <RoPE(q_i), k_j>  over every token j of the context frames
 *         (RoPE at the query's position, as rf_rope3d_apply; k_j as stored:
 *         already rotated),
 *   o_i = sum_j softmax(s)_j v_j, written as bf16 (round to nearest even).
 * Precision: the rotated query, times scale*log2(e), is rounded to bf16 once
 * (the same relative error as rounding the rotated query itself); scores,
 * the softmax and the accumulators are float32; the softmax weights enter
 * the value product as bf16.  scale == 0 means 1/sqrt(head_dim).
 * The context length is a runtime argument (whole frames); nothing is
 * recompiled or reallocated when it changes.
 *
 * Work split: query tiles of 256 rows run whole on the GPU's work-group
 * slots (one per CU) in full rounds; each tile of a last, partly filled round
 * is cut into the same number of equal key ranges (chosen so that these pieces
 * end soonest, at most two pieces per slot), one work-group per piece, and the
 * pieces are merged by a second kernel on the same stream (the result does not
 * depend on the split beyond float32 rounding; it is deterministic for a given
 * launch shape).
 *
 * Errors: RF_ERR_NULL, RF_ERR_ALIGN, RF_ERR_SHAPE (n_segs outside
 * 1..RF_MAX_SEGMENTS, q_tokens/ctx_frames < 1, q_tok0 outside 0..N-1,
 * reserved != 0, ld too small, a ring beyond the size limit of
 * rf_kvcache), RF_ERR_RANGE (context not inside
 * first..first+count-1, or query frames beyond the tables).  Output rows
 * must not overlap between segments.
 */
rf_status rf_window_attention(const rf_ctx* ctx, const rf_kvcache* c,
                              const rf_attn_segment* segs, int32_t n_segs, float scale,
                              void* stream);

/*
 * rf_window_attention_rawk -- a measurement variant of rf_window_attention for
 * a ring whose K buffer holds UN-rotated keys ([W][H][N][D], as the caller
 * wrote them): every K tile is rotated by 3D-RoPE as it is staged for the
 * score products (float32 products of the bf16 key and the float32 table
 * entries, one rounding to bf16), i.e. once for every query tile that reads
 * it, where the library otherwise rotates each key once when it enters the
 * ring.  It exists to measure that choice (the pages single 3D-RoPE out as a
 * cost: "Amazon and Reactor tune Trainium for real-time video generation",
 * section "Three problems for generic compilers").  Same arguments and
 * results as rf_window_attention up to the keys' rounding (the float32
 * rotation may differ from the ring's float64 one by one bf16 step); frames
 * of fewer than 64 tokens give RF_ERR_SHAPE.
 */
rf_status rf_window_attention_rawk(const rf_ctx* ctx, const rf_kvcache* c,
                                   const rf_attn_segment* segs, int32_t n_segs, float scale,
                                   void* stream);

/*
 * rf_window_attention_noalloc -- rf_window_attention for callers that cannot
 * allocate or free device memory once set up (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same validation,
 * kernels and results (bit for bit), but the partial results of split query
 * tiles go to a static device array of the library instead of the context's
 * workspace.  No allocation happens in this call.
 *
 * The array holds 512 partial results (2 x 256 x 130 KB = 68 MB): the most a
 * launch makes on a GPU of up to 256 compute units (256 on an MI355X), whose
 * split round has at most two pieces per work-group slot.  Each device keeps its own copy from the
 * library's load until the process ends; its address is looked up when the
 * first context of a device is created.  A launch that would need more
 * returns RF_ERR_SHAPE before anything is enqueued; RF_ERR_HIP if the array's
 * address could not be looked up on ctx's device.  Nothing in it needs to
 * start at zero (every partial result is written before it is read, inside the
 * call's own launches).
 * All noalloc calls on one device share the array, across contexts and
 * streams: calls that overlap in time on one device race and give wrong
 * results.  Order them (one stream, or synchronise).
 */
rf_status rf_window_attention_noalloc(const rf_ctx* ctx, const rf_kvcache* c,
                                      const rf_attn_segment* segs, int32_t n_segs, float scale,
                                      void* stream);

/*
 * Device-resident ring descriptors, for steps replayed from a captured graph
 * and for rolling several layers' rings in one launch.
 *
 * Source: every layer of the model reads and writes its own rolling KV cache,
 * and the attention length changes from pass to pass while the window fills
 * ("Amazon and Reactor tune Trainium for real-time video generation", section
 * "Three problems for generic compilers"); a real-time step has a budget of
 * tens of milliseconds for all layers ("Optimizing Real-Time Video Generation
 * on Trainium Chips", section 3).
 *
 * An rf_kvcache_dev lives in device memory (caller-owned, 16-byte aligned, 32
 * bytes) and describes one ring: its buffers and capacity, written only by
 * rf_kvcache_upload, and its window (first, count), which the kernels of
 * rf_kvcache_roll_layers advance on the device by the ring rule of
 * rf_kvcache_roll (the frame shift included) and rf_window_attention_dev reads
 * when its kernels run.  A graph that captured a step's launches therefore
 * replays it with the window the device holds at replay time -- e.g. every
 * step of a window that fills from empty, whose context grows frame by frame.
 * The host-side rf_kvcache of the same ring (the "host descriptor") is still
 * passed to every call: the host validates against it and advances it on
 * success, as for rf_kvcache_roll; replays advance only the device copy.
 * Callers keep the two describing the same buffers and capacity (write the
 * device copy only with rf_kvcache_upload); the kernels clamp what they read
 * (capacity to the host descriptor's, count to 1..capacity), so a stale device
 * window gives wrong frames, never an access outside the ring.
 */
typedef struct {
  void* k;
  void* v;
  int64_t first;
  int32_t count;
  int32_t capacity;
} rf_kvcache_dev;

/*
 * rf_kvcache_upload -- write n host descriptors (each validated as by
 * rf_kvcache_roll: buffers, alignment, capacity, size limit) into the device
 * array d_rings[0..n-1], on `stream` (a kernel: stream-ordered and capturable,
 * no host-to-device copy).  1 <= n <= 65535.  Use it to create the device
 * copies and to reset a window (upload a descriptor with count 0).
 */
rf_status rf_kvcache_upload(const rf_ctx* ctx, const rf_kvcache* rings, int32_t n,
                            rf_kvcache_dev* d_rings, void* stream);

/*
 * rf_kvcache_roll_layers -- rf_kvcache_roll of the same frames t0..t0+n_frames-1
 * into n_layers rings in ONE launch (grouped roll): layer l's keys and values
 * are token-major at k_new + l*k_layer_stride and v_new + l*v_layer_stride
 * (elements; strides >= 0, multiples of 8), its ring is d_rings[l], whose
 * window the launch advances on the device.  rings[0..n_layers-1] are the host
 * descriptors of the same rings: each is validated like rf_kvcache_roll's
 * (the roll must be legal for every layer), and advanced on success.  Layers
 * may have different capacities; they may not share a buffer.  Bit for bit the
 * same ring contents as n_layers separate rf_kvcache_roll calls.
 * 1 <= n_layers <= 65535.  Errors: those of rf_kvcache_roll, per layer.
 */
rf_status rf_kvcache_roll_layers(const rf_ctx* ctx, rf_kvcache* rings, rf_kvcache_dev* d_rings,
                                 int32_t n_layers, const void* k_new, int64_t k_layer_stride,
                                 int64_t k_ld, const void* v_new, int64_t v_layer_stride,
                                 int64_t v_ld, int64_t t0, int32_t n_frames, void* stream);

/*
 * rf_window_attention_dev -- rf_window_attention over the window of a
 * device-resident descriptor: every segment attends over all frames the ring
 * holds when the kernels run (d_ring's first .. first+count-1), so a captured
 * launch follows the window as it grows or slides.  Segments must give
 * ctx_t0 == 0 and ctx_frames == 0; queries and outputs are as in
 * rf_window_attention.  c is the ring's host descriptor (validated; the
 * launch is checked as for a window of `capacity` frames).  Results equal an
 * rf_window_attention call over the same frames up to float32 rounding (the
 * key-split work may be cut differently).  Errors: those of
 * rf_window_attention, RF_ERR_SHAPE for a segment with a context range.
 */
rf_status rf_window_attention_dev(const rf_ctx* ctx, const rf_kvcache* c,
                                  const rf_kvcache_dev* d_ring, const rf_attn_segment* segs,
                                  int32_t n_segs, float scale, void* stream);

/*
 * rf_device_copy -- a measurement aid, not a step of the path: copy `bytes`
 * (a multiple of 16) from src to dst on `stream` with one plain kernel
 * (16 bytes per thread, non-temporal loads and stores).  Its rate at a given
 * size is the bandwidth a single launch that only moves bytes reaches, the
 * practical ceiling for the RoPE and roll kernels, which move the same bytes
 * and add arithmetic.  Both pointers 16-byte aligned device memory, not
 * overlapping.  bytes == 0 is a no-op.  Errors: RF_ERR_NULL, RF_ERR_ALIGN,
 * RF_ERR_SHAPE.  Needs no context.
 */
rf_status rf_device_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * rf_set_frame_shift / rf_add_frame_shift -- replaying a captured steady-state
 * step.  A window step repeats with every frame index one higher than the
 * step before (the window slides by one frame; "Amazon and Reactor tune
 * Trainium for real-time video generation", section "Three problems for
 * generic compilers": frames generated and evicted in a sliding window, every
 * layer reading and writing its rolling KV cache).  With a shift set, every
 * later launch on ctx (rf_rope3d_apply, rf_kvcache_roll, rf_window_attention,
 * rf_qkv_project) reads the int64 at d_shift (device memory) when its kernels
 * run, clamps it to 0..max_shift, and adds it to all absolute frame indices of
 * the call: RoPE positions and ring slots (mod capacity).  A caller can thus
 * capture one step's launches in a HIP graph once (host arguments of step s)
 * and replay it for steps s+1, s+2, ... by advancing *d_shift inside the graph
 * with rf_add_frame_shift.
 *
 * rf_set_frame_shift: d_shift 8-byte aligned device memory owned by the caller
 *   (NULL turns the shift off); 0 <= max_shift < max_frame.  From then on the
 *   host validation of every call checks its frame ranges with max_shift
 *   added, so no replay within the clamp reads past the RoPE tables.  The
 *   caller orders this call after any queued work of the context.
 * rf_add_frame_shift: enqueue *d_shift += delta on `stream` (one-thread
 *   kernel; capturable).
 * Replays do not update the host-side rf_kvcache descriptors: advance them
 * with rf_kvcache_plan_roll if the caller needs them afterwards.  The shift
 * moves every frame index alike; the ring must hold the frames that the
 * shifted calls expect, which holds when each replayed step rolls its own new
 * frames (the usual step: roll, then attention).
 */
rf_status rf_set_frame_shift(rf_ctx* ctx, const int64_t* d_shift, int64_t max_shift);
rf_status rf_add_frame_shift(const rf_ctx* ctx, int64_t* d_shift, int64_t delta, void* stream);

/*
 * rf_qkv_project -- the layer's QKV projection, fused with the cache write:
 * for the layer input of frames t0..t0+n_frames-1,
 *   y = x W^T,  q = y[:, 0:C],  k = y[:, C:2C],  v = y[:, 2C:3C]   (C = H*D),
 * with q written token-major to `q` (un-rotated: rf_window_attention rotates
 * queries itself) and k, v rounded to bf16 and written into the ring exactly
 * as rf_kvcache_roll would write them (k rotated by the bit-exact 3D-RoPE,
 * v transposed), so k and v never reach memory as tensors of their own.  The
 * ring bookkeeping (overwrite in place, append, evict the oldest) and the
 * descriptor update are those of rf_kvcache_roll.
 *
 * Source: every layer reads and writes a rolling KV cache and rotates its
 * queries and keys over time, height and width ("Amazon and Reactor tune
 * Trainium for real-time video generation", section "Three problems for
 * generic compilers"), with 12 attention heads (ai4snews digest, second
 * paragraph).  The projection is not printed on the pages; this is the
 * standard multi-head self-attention projection (one [3C][C] weight: the q
 * rows, then the k rows, then the v rows; feature h*D + d of each block is
 * dimension d of head h).
 *
 * x: token-major [n_frames*N][x_ld] bf16 layer input, x_ld >= C.
 * w: [3C][w_ld] bf16 weight (row = output feature, w_ld >= C).
 * q: token-major [n_frames*N][q_ld] bf16 output, q_ld >= C; must not overlap
 *    x, w or the ring.
 * All three 16-byte aligned, ld multiples of 8 and at most 2^22.
 * Precision: bf16 products accumulated in float32 over the C input
 * features, rounded once to bf16 (round to nearest even).
 * Requirements and errors on the ring, t0 and n_frames as rf_kvcache_roll.
 */
rf_status rf_qkv_project(const rf_ctx* ctx, rf_kvcache* c, const void* x, int64_t x_ld,
                         const void* w, int64_t w_ld, void* q, int64_t q_ld, int64_t t0,
                         int32_t n_frames, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RFATTN_H */
