// Host side of librfattn: the C ABI declared in include/rfattn.h.
//
// Validation is done here, on the host, before anything is enqueued; the
// ring-buffer bookkeeping (first/count) lives only in the caller's
// descriptor; the RoPE tables are built once in float64 with the C library's
// pow/cos/sin, rounded to float32 and uploaded in rf_create.
//
// Sources for the operations: see the comments of include/rfattn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "rfattn.h"

using namespace rfattn;

struct rf_ctx {
  rf_geom g;
  int device;
  float2* d_tab;      // one allocation: [t table | h table | w table]
  RopeTables tab;
  int max_workers;    // persistent attention work-groups: kWorkersPerCu per CU
  float* d_partial;   // attention workspace: 2 * max_workers partial results
  const int64_t* d_shift;  // device frame shift added by every launch (NULL: none)
  int64_t max_shift;       // its clamp, validated against the tables
  float* d_scratch;        // this device's static attention scratch (NULL if unavailable)
  hipError_t scratch_err;  // why it is unavailable
};

// Static attention workspace for rf_window_attention_noalloc: room for the
// partial results of two pieces per work-group slot of a GPU of up to
// kScratchWorkers compute units (512 pieces, 68 MB).
// Each device holds its own copy from the library's load until the process
// ends.  In host code `scratch` is only a host-side stand-in: its device
// address comes from hipGetSymbolAddress, per device (scratch_address).
constexpr int kScratchWorkers = 256;
constexpr int64_t kScratchFloats = (int64_t)2 * kScratchWorkers * kPartFloats;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

thread_local char g_err[512] = "";

// The device address of `scratch` on the current device, looked up once per
// device (at its first rf_create) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};
bool g_scratch_done[kMaxDevices] = {};

float* scratch_address(int dev, hipError_t* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? static_cast<float*>(ptr) : nullptr;
    g_scratch_done[dev] = true;
  }
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

rf_status fail(rf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rf_status hip_fail(hipError_t e, const char* what) {
  return fail(RF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxTokens = int64_t(1) << 24;  // device index math is exact below this
constexpr int64_t kMaxProjLd = int64_t(1) << 22;  // 256 rows of the projection's operands: < 2^31 bytes
constexpr int kMaxLayers = 65535;                 // rings per grouped roll (the grid's y extent)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rf_status check_geom(const rf_geom* g) {
  if (!g) return fail(RF_ERR_NULL, "geometry is NULL");
  if (g->grid_h < 1 || g->grid_w < 1) return fail(RF_ERR_SHAPE, "grid must be at least 1x1");
  const int64_t n = (int64_t)g->grid_h * g->grid_w;
  if (n % 8 != 0) return fail(RF_ERR_SHAPE, "tokens per frame (%lld) must be a multiple of 8", (long long)n);
  if (n > (int64_t(1) << 20)) return fail(RF_ERR_SHAPE, "tokens per frame too large");
  if (g->n_heads < 1 || g->n_heads > 1024) return fail(RF_ERR_SHAPE, "n_heads must be in 1..1024");
  if (g->head_dim != kHeadDim) return fail(RF_ERR_SHAPE, "head_dim must be %d", kHeadDim);
  for (int a = 0; a < 3; ++a)
    if (g->rope_pairs[a] < 0) return fail(RF_ERR_SHAPE, "rope_pairs must be >= 0");
  if (g->rope_pairs[0] + g->rope_pairs[1] + g->rope_pairs[2] != g->head_dim / 2)
    return fail(RF_ERR_SHAPE, "rope_pairs must sum to head_dim/2");
  if (!(g->rope_base > 0.0) || !std::isfinite(g->rope_base)) return fail(RF_ERR_SHAPE, "rope_base must be > 0");
  if (g->max_frame < 1 || g->max_frame > (int64_t(1) << 20))
    return fail(RF_ERR_SHAPE, "max_frame must be in 1..2^20");
  return RF_OK;
}

// cos/sin of pos * base^(-j/P) for pos in [0, npos), j in [0, P): float64 libm, rounded to float32.
void fill_axis(std::vector<float2>& out, int64_t npos, int P, double base) {
  std::vector<double> omega(P);
  for (int j = 0; j < P; ++j) omega[j] = std::pow(base, -((double)j / (double)P));
  for (int64_t p = 0; p < npos; ++p)
    for (int j = 0; j < P; ++j) {
      const double th = (double)p * omega[j];
      out.push_back(make_float2((float)std::cos(th), (float)std::sin(th)));
    }
}

rf_status check_ctx(const rf_ctx* ctx) {
  if (!ctx) return fail(RF_ERR_NULL, "context is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != ctx->device)
    return fail(RF_ERR_UNSUPPORTED, "context belongs to device %d, current device is %d", ctx->device, dev);
  return RF_OK;
}

rf_status check_tensor(const void* p, int64_t ld, int64_t min_ld, const char* name) {
  if (!p) return fail(RF_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(RF_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (ld % 8 != 0) return fail(RF_ERR_ALIGN, "%s row stride %lld is not a multiple of 8", name, (long long)ld);
  if (ld < min_ld) return fail(RF_ERR_SHAPE, "%s row stride %lld < heads*head_dim", name, (long long)ld);
  return RF_OK;
}

rf_status check_ring(const rf_kvcache* c, bool need_memory) {
  if (!c) return fail(RF_ERR_NULL, "cache descriptor is NULL");
  if (c->capacity < 1) return fail(RF_ERR_SHAPE, "cache capacity must be >= 1");
  if (c->count < 0 || c->count > c->capacity) return fail(RF_ERR_SHAPE, "cache count outside 0..capacity");
  if (need_memory) {
    if (!c->k || !c->v) return fail(RF_ERR_NULL, "cache k/v buffer is NULL");
    if (!aligned16(c->k) || !aligned16(c->v)) return fail(RF_ERR_ALIGN, "cache buffers must be 16-byte aligned");
  }
  return RF_OK;
}

// The attention kernel addresses a ring buffer (K or V) with 32-bit byte offsets
// through one buffer resource and uses kRingOffsetLimit itself as its
// "past the end, load zeros" offset, so every byte of a ring must lie below it.
constexpr int64_t kRingOffsetLimit = 0x7FFFFFF0;

// Bytes of one ring buffer (K or V) of `capacity` slots, or an error if the ring
// cannot be addressed by the attention kernel.  Needs a validated geometry.
rf_status ring_bytes(const rf_geom& g, int64_t capacity, int64_t* bytes) {
  if (capacity < 1) return fail(RF_ERR_SHAPE, "cache capacity must be >= 1");
  const int64_t slot = (int64_t)g.n_heads * g.grid_h * g.grid_w * g.head_dim * 2;
  if (slot > kRingOffsetLimit / capacity || slot * capacity + 16 > kRingOffsetLimit)
    return fail(RF_ERR_SHAPE,
                "a ring of %lld slots of %lld bytes exceeds the attention kernel's 32-bit range "
                "(at most %lld bytes per K or V buffer: capacity <= %lld)",
                (long long)capacity, (long long)slot, (long long)(kRingOffsetLimit - 16),
                (long long)((kRingOffsetLimit - 16) / slot));
  *bytes = slot * capacity;
  return RF_OK;
}

// check_ring plus the ring's byte size against the attention kernel's range.
rf_status check_ring_geom(const rf_geom& g, const rf_kvcache* c, bool need_memory) {
  rf_status st = check_ring(c, need_memory);
  if (st != RF_OK) return st;
  int64_t bytes = 0;
  return ring_bytes(g, c->capacity, &bytes);
}

int64_t mod(int64_t a, int64_t m) {
  int64_t r = a % m;
  return r < 0 ? r + m : r;
}

}  // namespace

extern "C" {

const char* rf_status_string(rf_status s) {
  switch (s) {
    case RF_OK: return "RF_OK";
    case RF_ERR_NULL: return "RF_ERR_NULL";
    case RF_ERR_ALIGN: return "RF_ERR_ALIGN";
    case RF_ERR_SHAPE: return "RF_ERR_SHAPE";
    case RF_ERR_RANGE: return "RF_ERR_RANGE";
    case RF_ERR_UNSUPPORTED: return "RF_ERR_UNSUPPORTED";
    case RF_ERR_HIP: return "RF_ERR_HIP";
  }
  return "RF_ERR_UNKNOWN";
}

const char* rf_last_error(void) { return g_err; }

rf_status rf_create(const rf_geom* g, rf_ctx** out) {
  g_err[0] = 0;
  if (!out) return fail(RF_ERR_NULL, "out is NULL");
  rf_status st = check_geom(g);
  if (st != RF_OK) return st;

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(RF_ERR_UNSUPPORTED, "device %d is %s, librfattn is built for gfx950", dev, prop.gcnArchName);

  std::vector<float2> host;
  fill_axis(host, g->max_frame, g->rope_pairs[0], g->rope_base);
  const size_t off_h = host.size();
  fill_axis(host, g->grid_h, g->rope_pairs[1], g->rope_base);
  const size_t off_w = host.size();
  fill_axis(host, g->grid_w, g->rope_pairs[2], g->rope_base);
  if (host.empty()) host.push_back(make_float2(1.f, 0.f));

  const int max_workers = kWorkersPerCu * prop.multiProcessorCount;
  float2* d = nullptr;
  float* part = nullptr;
  e = hipMalloc((void**)&d, host.size() * sizeof(float2));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(tables)");
  e = hipMalloc((void**)&part, (size_t)2 * max_workers * kPartFloats * sizeof(float));
  if (e == hipSuccess) e = hipMemcpy(d, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = prepare_window_attn();
  if (e == hipSuccess) e = prepare_qkv_proj();
  if (e != hipSuccess) {
    (void)hipFree(d);
    if (part) (void)hipFree(part);
    return hip_fail(e, "table upload / workspace / kernel setup");
  }
  rf_ctx* c = new rf_ctx;
  c->g = *g;
  c->device = dev;
  c->d_tab = d;
  c->max_workers = max_workers;
  c->d_partial = part;
  c->d_shift = nullptr;
  c->max_shift = 0;
  c->d_scratch = scratch_address(dev, &c->scratch_err);  // its failure only disables the noalloc call
  c->tab.t = d;
  c->tab.h = d + off_h;
  c->tab.w = d + off_w;
  c->tab.pt = g->rope_pairs[0];
  c->tab.ph = g->rope_pairs[1];
  c->tab.pw = g->rope_pairs[2];
  *out = c;
  return RF_OK;
}

void rf_destroy(rf_ctx* ctx) {
  if (!ctx) return;
  (void)hipFree(ctx->d_tab);
  (void)hipFree(ctx->d_partial);
  delete ctx;
}

rf_status rf_kvcache_bytes(const rf_geom* g, int32_t capacity, int64_t* bytes) {
  g_err[0] = 0;
  rf_status st = check_geom(g);
  if (st != RF_OK) return st;
  if (!bytes) return fail(RF_ERR_NULL, "bytes is NULL");
  return ring_bytes(*g, capacity, bytes);
}

rf_status rf_rope3d_apply(const rf_ctx* ctx, const void* x, int64_t x_ld, void* y, int64_t y_ld,
                          int64_t t0, int64_t n_tokens, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  const rf_geom& g = ctx->g;
  const int64_t row = (int64_t)g.n_heads * g.head_dim;
  if (n_tokens < 0 || n_tokens >= kMaxTokens) return fail(RF_ERR_SHAPE, "n_tokens must be in 0..2^24-1");
  if (n_tokens == 0) return RF_OK;  // nothing to touch: pointers may be NULL
  if ((st = check_tensor(x, x_ld, row, "x")) != RF_OK) return st;
  if ((st = check_tensor(y, y_ld, row, "y")) != RF_OK) return st;
  if (x == y && x_ld != y_ld) return fail(RF_ERR_SHAPE, "in-place RoPE needs y_ld == x_ld");
  const int64_t N = (int64_t)g.grid_h * g.grid_w;
  if (t0 < 0 || t0 + (n_tokens - 1) / N + ctx->max_shift >= g.max_frame)
    return fail(RF_ERR_RANGE, "frames %lld..%lld outside the tables (max_frame %lld)", (long long)t0,
                (long long)(t0 + (n_tokens - 1) / N), (long long)g.max_frame);
  RopeArgs a;
  a.x = (const uint16_t*)x;
  a.y = (uint16_t*)y;
  a.x_ld = x_ld;
  a.y_ld = y_ld;
  a.t0 = t0;
  a.n_tokens = n_tokens;
  a.N = (int)N;
  a.gw = g.grid_w;
  a.H = g.n_heads;
  a.tab = ctx->tab;
  a.fs = {ctx->d_shift, ctx->max_shift};
  hipError_t e = launch_rope3d(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rope3d launch");
  return RF_OK;
}

rf_status rf_kvcache_plan_roll(const rf_kvcache* c, int64_t t0, int32_t n_frames, rf_kvcache* after) {
  g_err[0] = 0;
  rf_status st = check_ring(c, false);
  if (st != RF_OK) return st;
  if (!after) return fail(RF_ERR_NULL, "after is NULL");
  if (n_frames < 1 || n_frames > c->capacity)
    return fail(RF_ERR_SHAPE, "n_frames must be in 1..capacity (%d)", c->capacity);
  int64_t first = c->first;
  int64_t end = c->first + c->count;  // one past the newest valid frame
  if (c->count == 0) {
    first = t0;
    end = t0;
  } else if (t0 < c->first || t0 > end) {
    return fail(RF_ERR_RANGE, "roll start %lld outside %lld..%lld", (long long)t0, (long long)c->first,
                (long long)end);
  }
  const int64_t new_end = std::max(end, t0 + n_frames);
  int64_t count = new_end - first;
  if (count > c->capacity) {  // appends to a full ring evict the oldest frames
    first = new_end - c->capacity;
    count = c->capacity;
  }
  *after = *c;
  after->first = first;
  after->count = (int32_t)count;
  return RF_OK;
}

rf_status rf_kvcache_roll(const rf_ctx* ctx, rf_kvcache* c, const void* k_new, int64_t k_ld,
                          const void* v_new, int64_t v_ld, int64_t t0, int32_t n_frames, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  const rf_geom& g = ctx->g;
  if ((st = check_ring_geom(g, c, true)) != RF_OK) return st;
  const int64_t row = (int64_t)g.n_heads * g.head_dim;
  if ((st = check_tensor(k_new, k_ld, row, "k_new")) != RF_OK) return st;
  if ((st = check_tensor(v_new, v_ld, row, "v_new")) != RF_OK) return st;
  rf_kvcache after;
  if ((st = rf_kvcache_plan_roll(c, t0, n_frames, &after)) != RF_OK) return st;
  if (t0 < 0 || t0 + n_frames + ctx->max_shift > g.max_frame)
    return fail(RF_ERR_RANGE, "frames %lld..%lld outside the tables (max_frame %lld)", (long long)t0,
                (long long)(t0 + n_frames - 1), (long long)g.max_frame);
  const int64_t N = (int64_t)g.grid_h * g.grid_w;
  if ((int64_t)n_frames * N >= kMaxTokens) return fail(RF_ERR_SHAPE, "too many tokens in one roll");
  if ((int64_t)n_frames * g.n_heads > 65535) return fail(RF_ERR_SHAPE, "n_frames*n_heads must be <= 65535");

  RollArgs a;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_ld = k_ld;
  a.v_ld = v_ld;
  a.k_layer_stride = a.v_layer_stride = 0;
  a.rings = nullptr;
  a.n_layers = 1;
  a.k_ring = (uint16_t*)c->k;
  a.v_ring = (uint16_t*)c->v;
  a.slot_elems = (int64_t)g.n_heads * N * g.head_dim;
  a.t0 = t0;
  a.slot0 = (int)mod(t0, c->capacity);
  a.n_frames = n_frames;
  a.W = c->capacity;
  a.N = (int)N;
  a.gw = g.grid_w;
  a.H = g.n_heads;
  a.tab = ctx->tab;
  a.fs = {ctx->d_shift, ctx->max_shift};
  hipError_t e = launch_roll(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kvcache roll launch");
  c->first = after.first;
  c->count = after.count;
  return RF_OK;
}

rf_status rf_qkv_project(const rf_ctx* ctx, rf_kvcache* c, const void* x, int64_t x_ld, const void* w,
                         int64_t w_ld, void* q, int64_t q_ld, int64_t t0, int32_t n_frames, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  const rf_geom& g = ctx->g;
  if ((st = check_ring_geom(g, c, true)) != RF_OK) return st;
  const int64_t C = (int64_t)g.n_heads * g.head_dim;
  if ((st = check_tensor(x, x_ld, C, "x")) != RF_OK) return st;
  if ((st = check_tensor(w, w_ld, C, "w")) != RF_OK) return st;
  if ((st = check_tensor(q, q_ld, C, "q")) != RF_OK) return st;
  if (x_ld > kMaxProjLd || w_ld > kMaxProjLd || q_ld > kMaxProjLd)
    return fail(RF_ERR_SHAPE, "row strides must be at most 2^22 elements");
  rf_kvcache after;
  if ((st = rf_kvcache_plan_roll(c, t0, n_frames, &after)) != RF_OK) return st;
  if (t0 < 0 || t0 + n_frames + ctx->max_shift > g.max_frame)
    return fail(RF_ERR_RANGE, "frames %lld..%lld outside the tables (max_frame %lld)", (long long)t0,
                (long long)(t0 + n_frames - 1), (long long)g.max_frame);
  const int64_t N = (int64_t)g.grid_h * g.grid_w;
  const int64_t M = (int64_t)n_frames * N;
  if (M >= kMaxTokens) return fail(RF_ERR_SHAPE, "too many tokens in one projection");

  ProjArgs a;
  a.x = (const uint16_t*)x;
  a.w = (const uint16_t*)w;
  a.q = (uint16_t*)q;
  a.k_ring = (uint16_t*)c->k;
  a.v_ring = (uint16_t*)c->v;
  a.x_ld = x_ld;
  a.w_ld = w_ld;
  a.q_ld = q_ld;
  a.slot_elems = (int64_t)g.n_heads * N * g.head_dim;
  a.t0 = t0;
  a.M = (int)M;
  a.C = (int)C;
  a.N = (int)N;
  a.gw = g.grid_w;
  a.W = c->capacity;
  a.slot0 = (int)mod(t0, c->capacity);
  a.tiles_per_part = (int)((C + 255) / 256);
  a.f_tiles = 3 * a.tiles_per_part;
  a.n_tiles = (int)((M + 255) / 256) * a.f_tiles;
  a.n_workers = std::max(8, ctx->max_workers / kWorkersPerCu / 8 * 8);
  a.inv_n = 1.0f / (float)N;
  a.inv_gw = 1.0f / (float)g.grid_w;
  a.tab = ctx->tab;
  a.fs = {ctx->d_shift, ctx->max_shift};
  hipError_t e = launch_qkv_proj(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "qkv projection launch");
  c->first = after.first;
  c->count = after.count;
  return RF_OK;
}

rf_status rf_set_frame_shift(rf_ctx* ctx, const int64_t* d_shift, int64_t max_shift) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if (!d_shift) {
    ctx->d_shift = nullptr;
    ctx->max_shift = 0;
    return RF_OK;
  }
  if ((reinterpret_cast<uintptr_t>(d_shift) & 7u) != 0) return fail(RF_ERR_ALIGN, "d_shift is not 8-byte aligned");
  if (max_shift < 0 || max_shift >= ctx->g.max_frame)
    return fail(RF_ERR_RANGE, "max_shift must be in 0..max_frame-1");
  ctx->d_shift = d_shift;
  ctx->max_shift = max_shift;
  return RF_OK;
}

rf_status rf_add_frame_shift(const rf_ctx* ctx, int64_t* d_shift, int64_t delta, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if (!d_shift) return fail(RF_ERR_NULL, "d_shift is NULL");
  if ((reinterpret_cast<uintptr_t>(d_shift) & 7u) != 0) return fail(RF_ERR_ALIGN, "d_shift is not 8-byte aligned");
  hipError_t e = launch_add_shift(d_shift, delta, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "frame shift launch");
  return RF_OK;
}

}  // extern "C"

namespace {

// Pieces per split tile: the tiles of the last, partial round (tail < slots of
// them) are each cut into n equal key ranges, one work-group per piece, merged
// afterwards.  Choose the n that ends those rounds soonest -- ceil(n*tail/slots)
// rounds of 1/n of a tile -- with every piece at least one key tile and all
// partial results in the workspace (max_pieces); ties go to the smaller n.
int choose_split(int64_t tail, int64_t slots, int64_t min_key_tiles, int64_t max_pieces) {
  int best = 1;
  double best_t = 1.0;  // one round of whole tiles
  for (int64_t n = 2; tail > 0 && n <= min_key_tiles && n * tail <= max_pieces; ++n) {
    const double t = (double)((n * tail + slots - 1) / slots) / (double)n;
    if (t < best_t - 1e-9) {
      best = (int)n;
      best_t = t;
    }
  }
  return best;
}

// Validation and launch arguments of one rf_window_attention call (everything but
// the workspace pointer).  Enqueues nothing.
rf_status build_attn_args(const rf_ctx* ctx, const rf_kvcache* c, const rf_attn_segment* segs, int32_t n_segs,
                          float scale, AttnArgs& a) {
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if ((st = check_ring_geom(ctx->g, c, true)) != RF_OK) return st;
  if (!segs) return fail(RF_ERR_NULL, "segments is NULL");
  if (n_segs < 1 || n_segs > RF_MAX_SEGMENTS)
    return fail(RF_ERR_SHAPE, "n_segs must be in 1..%d", RF_MAX_SEGMENTS);
  if (scale == 0.0f) scale = 1.0f / std::sqrt((float)ctx->g.head_dim);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(RF_ERR_SHAPE, "scale must be > 0 and finite");
  if (c->count == 0) return fail(RF_ERR_RANGE, "the cache holds no frames");

  const rf_geom& g = ctx->g;
  const int64_t N = (int64_t)g.grid_h * g.grid_w;
  const int64_t row = (int64_t)g.n_heads * g.head_dim;
  std::memset(&a, 0, sizeof(a));
  int64_t units = 0, tiles = 0, min_key_tiles = INT64_MAX;
  for (int i = 0; i < n_segs; ++i) {
    const rf_attn_segment& s = segs[i];
    if ((st = check_tensor(s.q, s.q_ld, row, "q")) != RF_OK) return st;
    if ((st = check_tensor(s.o, s.o_ld, row, "o")) != RF_OK) return st;
    if (s.q_tokens < 1 || s.ctx_frames < 1)
      return fail(RF_ERR_SHAPE, "segment %d: q_tokens and ctx_frames must be >= 1", i);
    if (s.q_tok0 < 0 || s.q_tok0 >= N)
      return fail(RF_ERR_SHAPE, "segment %d: q_tok0 %d outside 0..%lld", i, (int)s.q_tok0, (long long)(N - 1));
    if (s.reserved != 0) return fail(RF_ERR_SHAPE, "segment %d: reserved must be 0", i);
    if ((int64_t)s.q_tokens >= kMaxTokens) return fail(RF_ERR_SHAPE, "segment %d: too many query tokens", i);
    const int64_t q_span = ((int64_t)s.q_tok0 + s.q_tokens + N - 1) / N;  // frames the queries touch
    if (s.q_t0 < 0 || s.q_t0 + q_span + ctx->max_shift > g.max_frame)
      return fail(RF_ERR_RANGE, "segment %d: query frames outside the tables", i);
    if (s.ctx_t0 < c->first || s.ctx_t0 + s.ctx_frames > c->first + c->count)
      return fail(RF_ERR_RANGE, "segment %d: context %lld..%lld outside the window %lld..%lld", i,
                  (long long)s.ctx_t0, (long long)(s.ctx_t0 + s.ctx_frames - 1), (long long)c->first,
                  (long long)(c->first + c->count - 1));
    SegDev& d = a.seg[i];
    d.q = (const uint16_t*)s.q;
    d.o = (uint16_t*)s.o;
    d.q_ld = s.q_ld;
    d.o_ld = s.o_ld;
    d.q_t0 = s.q_t0;
    d.q_tok0 = s.q_tok0;
    d.q_tokens = s.q_tokens;
    d.q_tiles = (d.q_tokens + kAttnBlockM - 1) / kAttnBlockM;
    d.ctx_keys = (int)(s.ctx_frames * N);
    d.ctx_slot0 = (int)mod(s.ctx_t0, c->capacity);
    d.ctx_t0 = s.ctx_t0;
    d.key_tiles = (d.ctx_keys + kAttnBlockN - 1) / kAttnBlockN;
    d.tile_begin = (int)tiles;
    tiles += (int64_t)d.q_tiles * g.n_heads;
    units += (int64_t)d.q_tiles * g.n_heads * d.key_tiles;
    min_key_tiles = std::min<int64_t>(min_key_tiles, d.key_tiles);
    if (units > (int64_t(1) << 31)) return fail(RF_ERR_SHAPE, "launch too large");
  }
  a.total_tiles = (int)tiles;
  // Whole rounds of tiles run one per work-group; the tiles of the last, partial
  // round are cut into equal key ranges.
  const int64_t slots = ctx->max_workers;
  a.dp_tiles = (int)(tiles / slots * slots);
  a.split_tiles = (int)(tiles - a.dp_tiles);
  a.n_split = choose_split(a.split_tiles, slots, min_key_tiles, 2 * slots);
  a.partial = nullptr;  // set by the caller
  a.n_segs = n_segs;
  a.k_ring = (const uint16_t*)c->k;
  a.v_ring = (const uint16_t*)c->v;
  a.slot_elems = (int64_t)g.n_heads * N * g.head_dim;
  a.W = c->capacity;
  a.N = (int)N;
  a.gw = g.grid_w;
  a.H = g.n_heads;
  a.c_log2 = scale * 1.4426950408889634f;
  a.tab = ctx->tab;
  a.fs = {ctx->d_shift, ctx->max_shift};
  return RF_OK;
}

}  // namespace

extern "C" {

rf_status rf_window_attention(const rf_ctx* ctx, const rf_kvcache* c, const rf_attn_segment* segs,
                              int32_t n_segs, float scale, void* stream) {
  g_err[0] = 0;
  AttnArgs a;
  rf_status st = build_attn_args(ctx, c, segs, n_segs, scale, a);
  if (st != RF_OK) return st;
  a.partial = ctx->d_partial;
  hipError_t e = launch_window_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "window attention launch");
  return RF_OK;
}

rf_status rf_window_attention_rawk(const rf_ctx* ctx, const rf_kvcache* c, const rf_attn_segment* segs,
                                   int32_t n_segs, float scale, void* stream) {
  g_err[0] = 0;
  AttnArgs a;
  rf_status st = build_attn_args(ctx, c, segs, n_segs, scale, a);
  if (st != RF_OK) return st;
  if (a.N < kAttnBlockN)
    return fail(RF_ERR_SHAPE, "keys rotated on load need frames of at least %d tokens", kAttnBlockN);
  a.rot_k = 1;
  a.partial = ctx->d_partial;
  hipError_t e = launch_window_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "window attention launch");
  return RF_OK;
}

rf_status rf_window_attention_noalloc(const rf_ctx* ctx, const rf_kvcache* c, const rf_attn_segment* segs,
                                      int32_t n_segs, float scale, void* stream) {
  g_err[0] = 0;
  AttnArgs a;
  rf_status st = build_attn_args(ctx, c, segs, n_segs, scale, a);
  if (st != RF_OK) return st;
  if (!ctx->d_scratch)
    return fail(RF_ERR_HIP, "the static attention scratch of device %d is not available: %s", ctx->device,
                hipGetErrorString(ctx->scratch_err));
  const int64_t need = (int64_t)a.split_tiles * a.n_split * kPartFloats;
  if (a.n_split > 1 && need > kScratchFloats)
    return fail(RF_ERR_SHAPE,
                "this launch needs %lld floats of attention scratch (%d partial results), the static "
                "scratch holds %lld (%d)",
                (long long)need, a.split_tiles * a.n_split, (long long)kScratchFloats, 2 * kScratchWorkers);
  a.partial = ctx->d_scratch;
  hipError_t e = launch_window_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "window attention launch");
  return RF_OK;
}

rf_status rf_device_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  g_err[0] = 0;
  if (bytes == 0) return RF_OK;
  if (!dst || !src) return fail(RF_ERR_NULL, "dst / src is NULL");
  if (bytes < 0 || bytes % 16 != 0) return fail(RF_ERR_SHAPE, "bytes must be a non-negative multiple of 16");
  if (!aligned16(dst) || !aligned16(src)) return fail(RF_ERR_ALIGN, "dst / src must be 16-byte aligned");
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) return fail(RF_ERR_SHAPE, "dst and src overlap");
  hipError_t e = launch_copy(dst, src, (uint64_t)bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "copy launch");
  return RF_OK;
}

rf_status rf_kvcache_upload(const rf_ctx* ctx, const rf_kvcache* rings, int32_t n, rf_kvcache_dev* d_rings,
                            void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if (!rings || !d_rings) return fail(RF_ERR_NULL, "rings / d_rings is NULL");
  if (n < 1 || n > kMaxLayers) return fail(RF_ERR_SHAPE, "n must be in 1..%d", kMaxLayers);
  if ((reinterpret_cast<uintptr_t>(d_rings) & 15u) != 0) return fail(RF_ERR_ALIGN, "d_rings is not 16-byte aligned");
  for (int i = 0; i < n; ++i)
    if ((st = check_ring_geom(ctx->g, &rings[i], true)) != RF_OK)
      return fail(st, "ring %d: %s", i, std::string(g_err).c_str());
  for (int i0 = 0; i0 < n; i0 += kUploadMax) {
    UploadArgs a;
    std::memset(&a, 0, sizeof(a));
    a.n = std::min(kUploadMax, n - i0);
    for (int i = 0; i < a.n; ++i) {
      const rf_kvcache& r = rings[i0 + i];
      a.d[i] = DevRing{(uint16_t*)r.k, (uint16_t*)r.v, r.first, r.count, r.capacity};
    }
    hipError_t e = launch_upload_rings(reinterpret_cast<DevRing*>(d_rings) + i0, a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ring descriptor upload");
  }
  return RF_OK;
}

rf_status rf_kvcache_roll_layers(const rf_ctx* ctx, rf_kvcache* rings, rf_kvcache_dev* d_rings, int32_t n_layers,
                                 const void* k_new, int64_t k_layer_stride, int64_t k_ld, const void* v_new,
                                 int64_t v_layer_stride, int64_t v_ld, int64_t t0, int32_t n_frames, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if (!rings || !d_rings) return fail(RF_ERR_NULL, "rings / d_rings is NULL");
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(RF_ERR_SHAPE, "n_layers must be in 1..%d", kMaxLayers);
  if ((reinterpret_cast<uintptr_t>(d_rings) & 15u) != 0) return fail(RF_ERR_ALIGN, "d_rings is not 16-byte aligned");
  const rf_geom& g = ctx->g;
  const int64_t row = (int64_t)g.n_heads * g.head_dim;
  if ((st = check_tensor(k_new, k_ld, row, "k_new")) != RF_OK) return st;
  if ((st = check_tensor(v_new, v_ld, row, "v_new")) != RF_OK) return st;
  if (k_layer_stride < 0 || v_layer_stride < 0 || k_layer_stride % 8 != 0 || v_layer_stride % 8 != 0)
    return fail(RF_ERR_ALIGN, "layer strides must be >= 0 and multiples of 8");
  std::vector<rf_kvcache> after(n_layers);
  std::vector<const void*> bufs;
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_ring_geom(g, &rings[l], true)) != RF_OK) return fail(st, "layer %d: %s", l, std::string(g_err).c_str());
    if ((st = rf_kvcache_plan_roll(&rings[l], t0, n_frames, &after[l])) != RF_OK)
      return fail(st, "layer %d: %s", l, std::string(g_err).c_str());
    bufs.push_back(rings[l].k);
    bufs.push_back(rings[l].v);
  }
  std::sort(bufs.begin(), bufs.end());
  if (std::adjacent_find(bufs.begin(), bufs.end()) != bufs.end())
    return fail(RF_ERR_SHAPE, "two layers share a ring buffer");
  if (t0 < 0 || t0 + n_frames + ctx->max_shift > g.max_frame)
    return fail(RF_ERR_RANGE, "frames %lld..%lld outside the tables (max_frame %lld)", (long long)t0,
                (long long)(t0 + n_frames - 1), (long long)g.max_frame);
  const int64_t N = (int64_t)g.grid_h * g.grid_w;
  if ((int64_t)n_frames * N >= kMaxTokens) return fail(RF_ERR_SHAPE, "too many tokens in one roll");
  if ((int64_t)n_frames * g.n_heads > 65535) return fail(RF_ERR_SHAPE, "n_frames*n_heads must be <= 65535");

  RollArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_ld = k_ld;
  a.v_ld = v_ld;
  a.k_layer_stride = k_layer_stride;
  a.v_layer_stride = v_layer_stride;
  a.rings = reinterpret_cast<DevRing*>(d_rings);
  a.n_layers = n_layers;
  a.slot_elems = (int64_t)g.n_heads * N * g.head_dim;
  a.t0 = t0;
  a.n_frames = n_frames;
  a.W = rings[0].capacity;  // per layer from its descriptor on the device
  a.N = (int)N;
  a.gw = g.grid_w;
  a.H = g.n_heads;
  a.tab = ctx->tab;
  a.fs = {ctx->d_shift, ctx->max_shift};
  hipError_t e = launch_roll(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "grouped kvcache roll launch");
  for (int l = 0; l < n_layers; ++l) {
    rings[l].first = after[l].first;
    rings[l].count = after[l].count;
  }
  return RF_OK;
}

rf_status rf_window_attention_dev(const rf_ctx* ctx, const rf_kvcache* c, const rf_kvcache_dev* d_ring,
                                  const rf_attn_segment* segs, int32_t n_segs, float scale, void* stream) {
  g_err[0] = 0;
  rf_status st = check_ctx(ctx);
  if (st != RF_OK) return st;
  if ((st = check_ring_geom(ctx->g, c, true)) != RF_OK) return st;
  if (!d_ring || !segs) return fail(RF_ERR_NULL, "d_ring / segments is NULL");
  if ((reinterpret_cast<uintptr_t>(d_ring) & 15u) != 0) return fail(RF_ERR_ALIGN, "d_ring is not 16-byte aligned");
  if (n_segs < 1 || n_segs > RF_MAX_SEGMENTS) return fail(RF_ERR_SHAPE, "n_segs must be in 1..%d", RF_MAX_SEGMENTS);
  if (c->count == 0) return fail(RF_ERR_RANGE, "the cache holds no frames");
  // Validate as a launch over the ring's largest window (capacity frames): the
  // queries, the tables and the unit count; the window itself is read by the kernels.
  std::vector<rf_attn_segment> full(segs, segs + n_segs);
  rf_kvcache whole = *c;
  whole.first = 0;
  whole.count = c->capacity;
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].ctx_t0 != 0 || segs[i].ctx_frames != 0)
      return fail(RF_ERR_SHAPE, "segment %d: ctx_t0 and ctx_frames must be 0 (the window is read on the device)", i);
    full[i].ctx_t0 = 0;
    full[i].ctx_frames = c->capacity;
  }
  AttnArgs a;
  if ((st = build_attn_args(ctx, &whole, full.data(), n_segs, scale, a)) != RF_OK) return st;
  // The split tiles are cut as a launch over the host descriptor's window would be
  // (so that such a launch gives the bits of rf_window_attention over the same
  // frames); with fewer key tiles at run time than pieces, some pieces are empty.
  AttnArgs now;
  for (int i = 0; i < n_segs; ++i) {
    full[i].ctx_t0 = c->first;
    full[i].ctx_frames = c->count;
  }
  if ((st = build_attn_args(ctx, c, full.data(), n_segs, scale, now)) != RF_OK) return st;
  a.n_split = now.n_split;
  a.ring_dev = reinterpret_cast<const DevRing*>(d_ring);
  a.partial = ctx->d_partial;
  hipError_t e = launch_window_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "window attention launch");
  return RF_OK;
}

}  // extern "C"
