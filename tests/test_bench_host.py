"""CPU checks of bench.py's host logic: the HBM-traffic figures it reports are tied to the
kernel sources they were measured on."""
import importlib.util
import os
import shutil

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _copy_sources(b, dst):
    src = os.path.join(ROOT, "rolling_window_attention_amd")
    for name in b.KERNEL_SOURCES:
        os.makedirs(os.path.dirname(os.path.join(dst, name)), exist_ok=True)
        shutil.copy(os.path.join(src, name), os.path.join(dst, name))


def test_source_hash_ignores_comments_but_not_code(tmp_path):
    b = _bench()
    _copy_sources(b, tmp_path)
    h0 = b.kernel_source_hash(str(tmp_path))
    assert h0 == b.kernel_source_hash()
    kernel = tmp_path / "csrc" / "window_attn.hip"
    text = kernel.read_text()
    kernel.write_text("// a comment line\n\n" + text.replace("\n", "  // trailing note\n", 1))
    assert b.kernel_source_hash(str(tmp_path)) == h0
    kernel.write_text(text + "\nstatic int rf_unused_probe = 1;\n")
    assert b.kernel_source_hash(str(tmp_path)) != h0


def test_traffic_record_matches_the_current_sources_or_is_ignored():
    b = _bench()
    t = b.measured_traffic(1.0)
    # either the committed counter record was taken on these sources, or bench.py
    # reports no traffic figure at all
    import json
    with open(b.TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec["kernel_source_sha"] == b.kernel_source_hash():
        assert t == rec["hbm_bytes_per_launch"] > 0
    else:
        assert t is None
