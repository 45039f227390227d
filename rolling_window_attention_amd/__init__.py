"""librfattn Python binding: rolling-window DiT attention with 3D-RoPE on MI355X.

A thin ctypes layer over the C ABI in ``include/rfattn.h``.  It only marshals
arguments -- torch tensors become device pointers and row strides, the current
torch stream becomes the HIP stream -- and raises ``RfError`` on any non-OK
status.  Every step of the computation runs in the HIP kernels of
``librfattn.so``; there is no fallback.  If the library is not built, the
first call raises.

    ctx = Context()                                   # 30x52 grid, 12 heads of 128
    cache = KVCache(ctx, capacity=21)                 # ring of 21 frame slots
    cache.roll(k_new, v_new, t0)                      # RoPE(K) + V^T into the ring
    cache.project(x, w, q, t0)                        # or: q = x Wq^T, k and v straight into the ring
    window_attention(ctx, cache, [Segment(q, q_t0, o, ctx_t0, ctx_frames), ...])
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librfattn.so")

RF_OK = 0
STATUS_NAMES = {0: "RF_OK", 1: "RF_ERR_NULL", 2: "RF_ERR_ALIGN", 3: "RF_ERR_SHAPE",
                4: "RF_ERR_RANGE", 5: "RF_ERR_UNSUPPORTED", 6: "RF_ERR_HIP"}
MAX_SEGMENTS = 8

# Every entry point include/rfattn.h declares.
EXPORTS = ("rf_create", "rf_destroy", "rf_status_string", "rf_last_error", "rf_rope3d_apply",
           "rf_kvcache_bytes", "rf_kvcache_roll", "rf_kvcache_plan_roll", "rf_window_attention",
           "rf_qkv_project", "rf_set_frame_shift", "rf_add_frame_shift",
           "rf_window_attention_noalloc", "rf_kvcache_upload", "rf_kvcache_roll_layers",
           "rf_window_attention_dev", "rf_window_attention_rawk", "rf_device_copy")


class RfError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class Geom(ctypes.Structure):
    _fields_ = [("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_pairs", ctypes.c_int32 * 3), ("rope_base", ctypes.c_double),
                ("max_frame", ctypes.c_int64)]


class KVCacheDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32), ("first", ctypes.c_int64)]


class SegmentDesc(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_ld", ctypes.c_int64), ("o", ctypes.c_void_p),
                ("o_ld", ctypes.c_int64), ("q_t0", ctypes.c_int64), ("q_tok0", ctypes.c_int32),
                ("q_tokens", ctypes.c_int32), ("ctx_t0", ctypes.c_int64), ("ctx_frames", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class KVCacheDevDesc(ctypes.Structure):
    """rf_kvcache_dev: the layout of a device-resident ring descriptor (DeviceRings keeps
    them as rows of an int64 device tensor)."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("first", ctypes.c_int64),
                ("count", ctypes.c_int32), ("capacity", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded librfattn (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.rf_create.argtypes = [ctypes.POINTER(Geom), ctypes.POINTER(vp)]
        L.rf_create.restype = i32
        L.rf_destroy.argtypes = [vp]
        L.rf_destroy.restype = None
        L.rf_status_string.argtypes = [i32]
        L.rf_status_string.restype = ctypes.c_char_p
        L.rf_last_error.argtypes = []
        L.rf_last_error.restype = ctypes.c_char_p
        L.rf_rope3d_apply.argtypes = [vp, vp, i64, vp, i64, i64, i64, vp]
        L.rf_rope3d_apply.restype = i32
        L.rf_kvcache_bytes.argtypes = [ctypes.POINTER(Geom), i32, ctypes.POINTER(i64)]
        L.rf_kvcache_bytes.restype = i32
        L.rf_kvcache_roll.argtypes = [vp, ctypes.POINTER(KVCacheDesc), vp, i64, vp, i64, i64, i32, vp]
        L.rf_kvcache_roll.restype = i32
        L.rf_kvcache_plan_roll.argtypes = [ctypes.POINTER(KVCacheDesc), i64, i32,
                                           ctypes.POINTER(KVCacheDesc)]
        L.rf_kvcache_plan_roll.restype = i32
        L.rf_window_attention.argtypes = [vp, ctypes.POINTER(KVCacheDesc),
                                          ctypes.POINTER(SegmentDesc), i32, ctypes.c_float, vp]
        L.rf_window_attention.restype = i32
        L.rf_device_copy.argtypes = [vp, vp, i64, vp]
        L.rf_device_copy.restype = i32
        L.rf_window_attention_rawk.argtypes = L.rf_window_attention.argtypes
        L.rf_window_attention_rawk.restype = i32
        L.rf_window_attention_noalloc.argtypes = L.rf_window_attention.argtypes
        L.rf_window_attention_noalloc.restype = i32
        L.rf_kvcache_upload.argtypes = [vp, ctypes.POINTER(KVCacheDesc), i32, vp, vp]
        L.rf_kvcache_upload.restype = i32
        L.rf_kvcache_roll_layers.argtypes = [vp, ctypes.POINTER(KVCacheDesc), vp, i32, vp, i64, i64, vp, i64,
                                             i64, i64, i32, vp]
        L.rf_kvcache_roll_layers.restype = i32
        L.rf_window_attention_dev.argtypes = [vp, ctypes.POINTER(KVCacheDesc), vp, ctypes.POINTER(SegmentDesc),
                                              i32, ctypes.c_float, vp]
        L.rf_window_attention_dev.restype = i32
        L.rf_qkv_project.argtypes = [vp, ctypes.POINTER(KVCacheDesc), vp, i64, vp, i64, vp, i64, i64, i32, vp]
        L.rf_qkv_project.restype = i32
        L.rf_set_frame_shift.argtypes = [vp, vp, i64]
        L.rf_set_frame_shift.restype = i32
        L.rf_add_frame_shift.argtypes = [vp, vp, i64, vp]
        L.rf_add_frame_shift.restype = i32
        _lib = L
    return _lib


def _check(status):
    if status != RF_OK:
        raise RfError(status, lib().rf_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _token_major(t, name, n_heads, head_dim):
    """Pointer and row stride of a [tokens, H, D] (or [tokens, H*D]) bf16 device tensor."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values")
    if t.dim() == 3:
        if t.shape[1:] != (n_heads, head_dim) or t.stride(2) != 1 or t.stride(1) != head_dim:
            raise ValueError(f"{name} must be [tokens, {n_heads}, {head_dim}] with heads contiguous")
    elif t.dim() == 2:
        if t.shape[1] != n_heads * head_dim or t.stride(1) != 1:
            raise ValueError(f"{name} must be [tokens, {n_heads * head_dim}] with rows contiguous")
    else:
        raise ValueError(f"{name} must be token-major [tokens, H, D]")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0), t.shape[0]


def _check_shift(shift):
    if not isinstance(shift, torch.Tensor) or not shift.is_cuda or shift.dtype != torch.int64:
        raise TypeError("shift must be an int64 CUDA tensor")
    if shift.numel() < 1:
        raise ValueError("shift must hold at least one element")


_pending_destroy = []


def _destroy_pending():
    """rf_destroy the handles of closed contexts, unless a graph capture is under way on
    the current stream."""
    if not _pending_destroy or torch.cuda.is_current_stream_capturing():
        return
    while _pending_destroy:
        lib().rf_destroy(_pending_destroy.pop())


def _geom(grid_h, grid_w, n_heads, head_dim, pairs, base, max_frame):
    return Geom(grid_h, grid_w, n_heads, head_dim, (ctypes.c_int32 * 3)(*pairs), base, max_frame)


def kvcache_bytes(capacity, grid_h=30, grid_w=52, n_heads=12, head_dim=128, pairs=(22, 21, 21),
                  base=10000.0, max_frame=4096):
    """Bytes of one ring buffer (K or V) of `capacity` slots (rf_kvcache_bytes, host-only);
    raises RfError for an invalid geometry or a ring beyond the library's size limit."""
    g = _geom(grid_h, grid_w, n_heads, head_dim, pairs, base, max_frame)
    out = ctypes.c_int64()
    _check(lib().rf_kvcache_bytes(ctypes.byref(g), capacity, ctypes.byref(out)))
    return out.value


class Context:
    """Geometry + device RoPE tables (rf_create / rf_destroy)."""

    def __init__(self, grid_h=30, grid_w=52, n_heads=12, head_dim=128, pairs=(22, 21, 21),
                 base=10000.0, max_frame=4096):
        g = _geom(grid_h, grid_w, n_heads, head_dim, pairs, base, max_frame)
        _destroy_pending()
        h = ctypes.c_void_p()
        _check(lib().rf_create(ctypes.byref(g), ctypes.byref(h)))
        self._h = h
        self.grid_h, self.grid_w, self.n_heads, self.head_dim = grid_h, grid_w, n_heads, head_dim
        self.pairs, self.base, self.max_frame = tuple(pairs), base, max_frame
        self.tokens_per_frame = grid_h * grid_w

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("context is closed")
        return self._h

    def close(self):
        """Free the context (rf_destroy).  While the current stream is being captured
        into a graph, freeing device memory would invalidate the capture, so the handle
        is then kept and freed at the next close or Context creation outside a capture
        (this happens when the garbage collector runs inside a capture)."""
        if getattr(self, "_h", None) is not None:
            _pending_destroy.append(self._h)
            self._h = None
        _destroy_pending()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_frame_shift(self, shift, max_shift):
        """Every later launch on this context adds shift[0] (an int64 CUDA tensor, read
        when its kernels run, clamped to 0..max_shift) to all its frame indices; None
        turns it off.  For replaying one captured step as the following steps."""
        if shift is None:
            _check(lib().rf_set_frame_shift(self.handle, None, 0))
            self._shift = None
            return
        _check_shift(shift)
        _check(lib().rf_set_frame_shift(self.handle, ctypes.c_void_p(shift.data_ptr()), max_shift))
        self._shift = shift  # keep the memory alive while the context uses it

    def add_frame_shift(self, shift, delta, stream=None):
        """Enqueue shift[0] += delta (stream-ordered, capturable in a graph)."""
        _check_shift(shift)
        _check(lib().rf_add_frame_shift(self.handle, ctypes.c_void_p(shift.data_ptr()), delta,
                                        _stream(stream)))

    def rope3d_apply(self, x, t0, y=None, stream=None):
        """y = 3D-RoPE(x) for token-major bf16 x whose first token is in frame t0."""
        if y is None:
            y = torch.empty_like(x)
        xp, xld, n = _token_major(x, "x", self.n_heads, self.head_dim)
        yp, yld, ny = _token_major(y, "y", self.n_heads, self.head_dim)
        if ny != n:
            raise ValueError("x and y must have the same number of tokens")
        _check(lib().rf_rope3d_apply(self.handle, xp, xld, yp, yld, t0, n, _stream(stream)))
        return y


class KVCache:
    """A ring of `capacity` frame slots: k [W, H, N, D] (rotated), v [W, H, N/8, D, 8]
    (values in blocks of 8 tokens: token n, dim d at [n // 8, d, n % 8])."""

    def __init__(self, ctx, capacity, device="cuda"):
        self.ctx = ctx
        kvcache_bytes(capacity, ctx.grid_h, ctx.grid_w, ctx.n_heads, ctx.head_dim, ctx.pairs,
                      ctx.base, ctx.max_frame)  # the size limit, before allocating
        shape_k = (capacity, ctx.n_heads, ctx.tokens_per_frame, ctx.head_dim)
        shape_v = (capacity, ctx.n_heads, ctx.tokens_per_frame // 8, ctx.head_dim, 8)
        self.k = torch.zeros(shape_k, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros(shape_v, dtype=torch.bfloat16, device=device)
        self.desc = KVCacheDesc(self.k.data_ptr(), self.v.data_ptr(), capacity, 0, 0)

    @property
    def capacity(self):
        return self.desc.capacity

    @property
    def first(self):
        return self.desc.first

    @property
    def count(self):
        return self.desc.count

    def window(self):
        return list(range(self.desc.first, self.desc.first + self.desc.count))

    def roll(self, k_new, v_new, t0, stream=None):
        """Write frames t0.. of token-major k_new/v_new ([n*N, H, D]) into the ring."""
        c = self.ctx
        kp, kld, nk = _token_major(k_new, "k_new", c.n_heads, c.head_dim)
        vp, vld, nv = _token_major(v_new, "v_new", c.n_heads, c.head_dim)
        if nk != nv or nk % c.tokens_per_frame:
            raise ValueError("k_new and v_new must hold the same whole number of frames")
        n = nk // c.tokens_per_frame
        _check(lib().rf_kvcache_roll(c.handle, ctypes.byref(self.desc), kp, kld, vp, vld, t0, n,
                                     _stream(stream)))

    def project(self, x, w, q, t0, stream=None):
        """QKV projection of the layer input x ([n*N, H*D]) with weight w ([3*H*D, H*D]):
        queries into q ([n*N, H, D] or [n*N, H*D]); rotated keys and transposed values
        of frames t0.. into the ring, as roll() would write them."""
        c = self.ctx
        xp, xld, nx = _token_major(x, "x", c.n_heads, c.head_dim)
        qp, qld, nq = _token_major(q, "q", c.n_heads, c.head_dim)
        wp, wld, nw = _token_major(w, "w", c.n_heads, c.head_dim)
        if nw != 3 * c.n_heads * c.head_dim:
            raise ValueError("w must be [3*H*D, H*D]")
        if nx != nq or nx % c.tokens_per_frame:
            raise ValueError("x and q must hold the same whole number of frames")
        n = nx // c.tokens_per_frame
        _check(lib().rf_qkv_project(c.handle, ctypes.byref(self.desc), xp, xld, wp, wld, qp, qld, t0, n,
                                    _stream(stream)))

    def plan_roll(self, t0, n_frames):
        """(first, count) the ring would have after rolling frames t0..t0+n_frames-1."""
        after = KVCacheDesc()
        _check(lib().rf_kvcache_plan_roll(ctypes.byref(self.desc), t0, n_frames, ctypes.byref(after)))
        return after.first, after.count


class Segment:
    """Query tokens q attending to context frames ctx_t0..ctx_t0+ctx_frames-1.  q's first
    token is token q_tok0 of frame q_t0 (0 for whole frames); q and o hold any number
    of tokens."""

    def __init__(self, q, q_t0, o, ctx_t0, ctx_frames, q_tok0=0):
        self.q, self.q_t0, self.o, self.ctx_t0, self.ctx_frames = q, q_t0, o, ctx_t0, ctx_frames
        self.q_tok0 = q_tok0


def window_attention(ctx, cache, segments, scale=0.0, stream=None):
    """All segments in one launch; outputs are written into each segment's o."""
    _check(lib().rf_window_attention(ctx.handle, ctypes.byref(cache.desc), *_segments(ctx, segments),
                                     scale, _stream(stream)))


def window_attention_noalloc(ctx, cache, segments, scale=0.0, stream=None):
    """window_attention with the library's static per-device scratch instead of the
    context's workspace (rf_window_attention_noalloc): no allocation in the call; calls
    that overlap in time on one device race."""
    _check(lib().rf_window_attention_noalloc(ctx.handle, ctypes.byref(cache.desc), *_segments(ctx, segments),
                                             scale, _stream(stream)))


def window_attention_rawk(ctx, cache, segments, scale=0.0, stream=None):
    """Measurement variant (rf_window_attention_rawk): cache.k holds UN-rotated keys, and
    the kernel rotates every key tile as it stages it."""
    _check(lib().rf_window_attention_rawk(ctx.handle, ctypes.byref(cache.desc), *_segments(ctx, segments),
                                          scale, _stream(stream)))


def _segments(ctx, segments):
    """The rf_attn_segment array of a launch and its length."""
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError(f"1..{MAX_SEGMENTS} segments per launch")
    arr = (SegmentDesc * len(segments))()
    for i, s in enumerate(segments):
        qp, qld, nq = _token_major(s.q, "q", ctx.n_heads, ctx.head_dim)
        op, old, no = _token_major(s.o, "o", ctx.n_heads, ctx.head_dim)
        if nq != no:
            raise ValueError("q and o must hold the same number of tokens")
        arr[i] = SegmentDesc(qp, qld, op, old, s.q_t0, s.q_tok0, nq, s.ctx_t0, s.ctx_frames, 0)
    return arr, len(segments)


def plan_roll(capacity, first, count, t0, n_frames):
    """Host-only ring bookkeeping (rf_kvcache_plan_roll) without any device memory."""
    d = KVCacheDesc(None, None, capacity, count, first)
    after = KVCacheDesc()
    _check(lib().rf_kvcache_plan_roll(ctypes.byref(d), t0, n_frames, ctypes.byref(after)))
    return after.first, after.count


DEV_DESC_BYTES = ctypes.sizeof(KVCacheDevDesc)  # 32


def _layered(t, name, n_heads, head_dim):
    """Pointer, layer stride, row stride and tokens of a [layers, tokens, H, D] (or
    [layers, tokens, H*D]) bf16 device tensor; a layer stride of 0 (expand) is allowed."""
    if not isinstance(t, torch.Tensor) or t.dim() not in (3, 4):
        raise ValueError(f"{name} must be [layers, tokens, H, D] or [layers, tokens, H*D]")
    ptr, ld, tokens = _token_major(t[0], name, n_heads, head_dim)
    return ptr, t.stride(0), ld, tokens


class DeviceRings:
    """Device-resident descriptors (rf_kvcache_dev) of the rings of `caches` -- KVCache
    objects of one context, one per layer -- in one device array, written from the
    caches' host descriptors by rf_kvcache_upload."""

    def __init__(self, caches, stream=None):
        self.caches = list(caches)
        if not self.caches:
            raise ValueError("at least one cache")
        self.ctx = self.caches[0].ctx
        if any(c.ctx is not self.ctx for c in self.caches):
            raise ValueError("all caches must belong to one context")
        self.buf = torch.zeros((len(self.caches), DEV_DESC_BYTES // 8), dtype=torch.int64,
                               device=self.caches[0].k.device)
        self._descs = (KVCacheDesc * len(self.caches))()
        self.upload(stream)

    def __len__(self):
        return len(self.caches)

    def ptr(self, layer=0):
        if not 0 <= layer < len(self.caches):
            raise IndexError(layer)
        return ctypes.c_void_p(self.buf.data_ptr() + DEV_DESC_BYTES * layer)

    def _gather(self):
        for i, c in enumerate(self.caches):
            self._descs[i] = c.desc

    def _scatter(self):
        for i, c in enumerate(self.caches):
            c.desc.first, c.desc.count = self._descs[i].first, self._descs[i].count

    def upload(self, stream=None):
        """Write the caches' host descriptors to the device copies (rf_kvcache_upload)."""
        self._gather()
        _check(lib().rf_kvcache_upload(self.ctx.handle, self._descs, len(self.caches), self.ptr(0),
                                       _stream(stream)))

    def reset(self, stream=None):
        """Empty every ring's window, on the host and (stream-ordered) on the device."""
        for c in self.caches:
            c.desc.first, c.desc.count = 0, 0
        self.upload(stream)

    def roll(self, k_new, v_new, t0, stream=None):
        """Grouped roll (rf_kvcache_roll_layers): layer l's frames t0.. from k_new[l], v_new[l]
        ([layers, n*N, H, D]) into ring l, one launch; windows advance on host and device."""
        c = self.ctx
        kp, ks, kld, nk = _layered(k_new, "k_new", c.n_heads, c.head_dim)
        vp, vs, vld, nv = _layered(v_new, "v_new", c.n_heads, c.head_dim)
        if k_new.shape[0] != len(self.caches) or v_new.shape[0] != len(self.caches):
            raise ValueError("one input block per layer")
        if nk != nv or nk % c.tokens_per_frame:
            raise ValueError("k_new and v_new must hold the same whole number of frames")
        self._gather()
        _check(lib().rf_kvcache_roll_layers(c.handle, self._descs, self.ptr(0), len(self.caches), kp, ks, kld,
                                            vp, vs, vld, t0, nk // c.tokens_per_frame, _stream(stream)))
        self._scatter()


def window_attention_dev(ctx, rings, layer, segments, scale=0.0, stream=None):
    """rf_window_attention_dev: the segments (context fields 0) attend over the window of
    ring `layer` of `rings` (a DeviceRings) as the device holds it when the kernels run."""
    cache = rings.caches[layer]
    _check(lib().rf_window_attention_dev(ctx.handle, ctypes.byref(cache.desc), rings.ptr(layer),
                                         *_segments(ctx, segments), scale, _stream(stream)))


def device_copy(dst, src, stream=None):
    """rf_device_copy of src's bytes into dst (device tensors of equal byte size): the
    plain-copy bandwidth ceiling the bandwidth-bound kernels are measured against."""
    for t, name in ((dst, "dst"), (src, "src")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous CUDA tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src must have the same size in bytes")
    _check(lib().rf_device_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), nbytes,
                                _stream(stream)))
