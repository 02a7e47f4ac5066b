"""Host-side logic of bench.py (no GPU): the counter-summary lookup that
feeds the roofline's `traffic`, and the refusal of more than one GPU."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _tree(tmp_path, digest_of=None, traffic=123456):
    csrc = tmp_path / "bit_weight_kv_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f, text in (("attention.hip", "kernel A\n"), ("common.h", "helpers\n")):
        (csrc / f).write_text(text)
    h = hashlib.sha256()
    for f in ("attention.hip", "common.h"):
        h.update((csrc / f).read_bytes())
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "decode_attention_opt175b_4bit_b144.md").write_text(
        f"# summary\n\ntraffic_bytes_per_launch: {traffic}\nsource_sha256: {digest_of or h.hexdigest()}\n")
    return csrc


def test_traffic_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    b = _bench()
    csrc = _tree(tmp_path)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("decode_attention") == 123456
    assert b.measured_traffic("prefill_attention") is None  # no summary for this class
    (csrc / "common.h").write_text("helpers, edited\n")        # any source of the kernel changed
    assert b.measured_traffic("decode_attention") is None


def test_traffic_missing_summary_or_wrong_digest(tmp_path, monkeypatch):
    b = _bench()
    _tree(tmp_path, digest_of="0" * 64)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("decode_attention") is None
    monkeypatch.setattr(b, "ROOT", str(tmp_path / "nowhere"))
    assert b.measured_traffic("decode_attention") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
