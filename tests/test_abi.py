"""CPU-only checks of the C ABI: the library loads, exports every entry point the
header declares, and its host-side validation and ring bookkeeping behave (no GPU call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import rolling_window_attention_amd as rf
from oracle.ring import RingError, RingModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rfattn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rf.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return rf.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(rf_[a-z0-9_]+)\s*\(", src))


def test_header_and_binding_agree():
    assert _declared() == set(rf.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
    # and they are real exported functions of the shared object
    out = os.popen(f"nm -D --defined-only {rf.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings(L):
    for code, name in rf.STATUS_NAMES.items():
        assert L.rf_status_string(code).decode() == name
    assert L.rf_status_string(99).decode() == "RF_ERR_UNKNOWN"


def _geom(**kw):
    d = dict(grid_h=30, grid_w=52, n_heads=12, head_dim=128, pairs=(22, 21, 21), base=1e4,
             max_frame=4096)
    d.update(kw)
    return rf.Geom(d["grid_h"], d["grid_w"], d["n_heads"], d["head_dim"],
                   (ctypes.c_int32 * 3)(*d["pairs"]), d["base"], d["max_frame"])


@pytest.mark.parametrize("kw", [dict(head_dim=64, pairs=(11, 11, 10)), dict(pairs=(22, 21, 20)),
                                dict(pairs=(-1, 43, 22)), dict(grid_h=5, grid_w=5),
                                dict(grid_h=0), dict(n_heads=0), dict(base=0.0),
                                dict(base=float("nan")), dict(max_frame=0),
                                dict(max_frame=1 << 21)])
def test_create_rejects_bad_geometry_before_touching_a_device(L, kw):
    g = _geom(**kw)
    h = ctypes.c_void_p()
    st = L.rf_create(ctypes.byref(g), ctypes.byref(h))
    assert st == 3, rf.STATUS_NAMES.get(st)
    assert h.value is None
    assert L.rf_last_error().decode()


def test_null_arguments(L):
    h = ctypes.c_void_p()
    assert L.rf_create(None, ctypes.byref(h)) == 1
    assert L.rf_create(ctypes.byref(_geom()), None) == 1
    assert L.rf_rope3d_apply(None, None, 1536, None, 1536, 0, 1, None) == 1
    assert L.rf_window_attention(None, None, None, 1, 0.0, None) == 1
    assert L.rf_kvcache_roll(None, None, None, 1536, None, 1536, 0, 1, None) == 1
    L.rf_destroy(None)  # ignored


def test_plan_roll_matches_oracle_ring_model(L):
    rng = np.random.default_rng(0)
    for W in (1, 3, 5, 21):
        for _ in range(300):
            model = RingModel(W)
            first, count = 0, 0
            for _ in range(int(rng.integers(1, 10))):
                if model.count == 0:
                    t0 = int(rng.integers(0, 100))
                else:
                    t0 = int(rng.integers(model.first - 2, model.first + model.count + 3))
                n = int(rng.integers(0, W + 2))
                try:
                    model.check_roll(t0, n)
                    ok = True
                except RingError:
                    ok = False
                if ok:
                    model.roll(t0, n)
                    first, count = rf.plan_roll(W, first, count, t0, n)
                    assert (first, count) == (model.first, model.count)
                else:
                    with pytest.raises(rf.RfError):
                        rf.plan_roll(W, first, count, t0, n)


def test_plan_roll_rejects_bad_descriptors(L):
    with pytest.raises(rf.RfError):
        rf.plan_roll(0, 0, 0, 0, 1)
    with pytest.raises(rf.RfError):
        rf.plan_roll(5, 0, 6, 0, 1)


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes structures have the C structures' sizes and field offsets (the header
    compiled by the host C compiler)."""
    pairs = [(rf.Geom, "rf_geom"), (rf.KVCacheDesc, "rf_kvcache"), (rf.SegmentDesc, "rf_attn_segment"),
             (rf.KVCacheDevDesc, "rf_kvcache_dev")]
    lines = ["#include <stddef.h>", "#include <stdio.h>", f'#include "{HEADER}"', "int main(void) {"]
    for cls, cname in pairs:
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    assert os.system(f"gcc -std=c11 -o {exe} {src}") == 0
    got = dict(l.rsplit(" ", 1) for l in os.popen(str(exe)).read().splitlines())
    for cls, cname in pairs:
        assert int(got[f"{cname} size"]) == ctypes.sizeof(cls), cname
        for field, _ in cls._fields_:
            assert int(got[f"{cname} {field}"]) == getattr(cls, field).offset, (cname, field)


def test_binding_rejects_host_and_wrong_typed_tensors():
    """Pointers reach the kernels only from bf16 (or int16) device tensors of the right
    shape; host tensors and other dtypes are refused before any library call."""
    import torch
    with pytest.raises(TypeError):
        rf._token_major(torch.zeros((4, 12, 128), dtype=torch.bfloat16), "q", 12, 128)
    with pytest.raises(TypeError):
        rf._token_major(np.zeros((4, 12, 128), dtype=np.uint16), "q", 12, 128)
    with pytest.raises(TypeError):
        rf._check_shift(torch.zeros(1, dtype=torch.int64))
    with pytest.raises(TypeError):
        rf._check_shift(None)


SLOT_30x52x12 = 12 * 30 * 52 * 128 * 2   # bytes of one ring slot at the workload geometry


@pytest.mark.parametrize("capacity,ok", [(1, True), (21, True), (448, True), (449, False),
                                         (897, False), (0, False), (-3, False)])
def test_ring_size_limit_at_the_workload_geometry(L, capacity, ok):
    """The attention kernel addresses a ring buffer with 32-bit offsets and uses
    0x7FFFFFF0 as its past-the-end offset: 448 slots of 4,792,320 bytes fit, 449 do not
    (that sentinel would fall inside the ring), 897 would wrap the offsets."""
    if ok:
        assert rf.kvcache_bytes(capacity) == capacity * SLOT_30x52x12
        assert capacity * SLOT_30x52x12 + 16 <= 0x7FFFFFF0
    else:
        with pytest.raises(rf.RfError) as e:
            rf.kvcache_bytes(capacity)
        assert e.value.status == 3


def test_ring_size_limit_with_a_large_slot(L):
    """A legal geometry whose single slot already exceeds the 32-bit range (1024 x 1024
    tokens per frame, 12 heads: 3.2 GB per slot) is refused at any capacity; a 1-head
    slot of 256 MiB fits 7 times, not 8."""
    with pytest.raises(rf.RfError) as e:
        rf.kvcache_bytes(1, grid_h=1024, grid_w=1024)
    assert e.value.status == 3
    one_head = 1024 * 1024 * 128 * 2
    assert rf.kvcache_bytes(7, grid_h=1024, grid_w=1024, n_heads=1) == 7 * one_head
    with pytest.raises(rf.RfError):
        rf.kvcache_bytes(8, grid_h=1024, grid_w=1024, n_heads=1)


def test_ring_size_query_validates_its_arguments(L):
    out = ctypes.c_int64(-1)
    assert L.rf_kvcache_bytes(None, 21, ctypes.byref(out)) == 1
    assert L.rf_kvcache_bytes(ctypes.byref(_geom()), 21, None) == 1
    assert L.rf_kvcache_bytes(ctypes.byref(_geom(head_dim=64, pairs=(11, 11, 10))), 21,
                              ctypes.byref(out)) == 3
    assert out.value == -1  # untouched on error


def test_device_copy_validates_before_any_launch(L):
    """rf_device_copy's argument errors come from the host, before anything is enqueued
    (fake pointers are never dereferenced)."""
    assert L.rf_device_copy(None, None, 0, None) == 0          # nothing to copy
    assert L.rf_device_copy(None, ctypes.c_void_p(0x2000), 16, None) == 1
    assert L.rf_device_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2001), 16, None) == 2
    assert L.rf_device_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 17, None) == 3
    assert L.rf_device_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1010), 32, None) == 3  # overlap
