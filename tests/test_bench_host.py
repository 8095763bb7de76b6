"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the hash that
ties the traffic record to the kernel sources, and the kernel-name matcher
that picks the bf16 instances out of profiler traces."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _copy_sources(tmp_path):
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)


def test_source_hash_ignores_comments_not_code(tmp_path):
    _copy_sources(tmp_path)
    base = bench.kernel_source_hash(str(tmp_path))
    assert base == bench.kernel_source_hash(ROOT)
    path = tmp_path / bench.KERNEL_SOURCES[0]
    text = path.read_text()
    path.write_text("// a new line of comment\n/* and a block\n   comment */\n" + text + "\n\n")
    assert bench.kernel_source_hash(str(tmp_path)) == base
    path.write_text(text.replace("constexpr int NST = 4;", "constexpr int NST = 8;"))
    assert "constexpr int NST = 4;" in text
    assert bench.kernel_source_hash(str(tmp_path)) != base


def test_traffic_is_reported_only_for_the_recorded_kernels(tmp_path, monkeypatch):
    """bench.py reports the record's bytes while the kernel sources hash to
    the recorded value, and null for any other sources."""
    import json
    with open(bench.TRAFFIC_RECORD) as f:
        head, body = f.read().split("\n", 1)
    rec = json.loads(body)
    want = rec["hbm_bytes_per_lbm_run"] if rec["kernel_source_hash"] == bench.kernel_source_hash() else None
    assert bench.recorded_traffic() == want
    stale = tmp_path / "record.txt"
    stale.write_text(head + "\n" + json.dumps(dict(rec, kernel_source_hash="0" * 16)))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(stale))
    assert bench.recorded_traffic() is None
    fresh = tmp_path / "fresh.txt"
    fresh.write_text(head + "\n" + json.dumps(dict(rec, kernel_source_hash=bench.kernel_source_hash())))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(fresh))
    assert bench.recorded_traffic() == rec["hbm_bytes_per_lbm_run"]


@pytest.mark.parametrize("name,base,want", [
    ("_ZN3lbm12_GLOBAL__N_115attn_d64_kernelIDF16bLb0EEEvNS_9BatchArgsE", "attn_d64_kernel", True),
    ("_ZN3lbm12_GLOBAL__N_115attn_d64_kernelIDF16_Lb0EEEvNS_9BatchArgsE", "attn_d64_kernel", False),
    ("void lbm::(anonymous namespace)::attn_d64_kernel<__bf16, false>(lbm::BatchArgs)",
     "attn_d64_kernel", True),
    ("_ZN3lbm12_GLOBAL__N_112merge_kernelIDF16bLi64EEEvNS_8AttnArgsE", "merge_kernel", True),
    ("_ZN3lbm12_GLOBAL__N_112merge_kernelIfLi64EEEvNS_8AttnArgsE", "merge_kernel", False),
])
def test_bf16_kernel_names(name, base, want):
    assert bench.bf16_kernel(name, base) is want


def test_append_traffic_follows_the_append_sources(tmp_path, monkeypatch):
    """The append's recorded bytes are reported while append.hip and
    kernels.h hash to the recorded value, and null otherwise (an attention
    change alone does not void them)."""
    import json
    rec = {"kernel_source_hash": "0" * 16, "hbm_bytes_per_lbm_run": 1,
           "append_source_hash": bench.kernel_source_hash(sources=bench.APPEND_SOURCES),
           "hbm_bytes_per_append": 11534336}
    path = tmp_path / "record.txt"
    path.write_text("header\n" + json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.recorded_append_traffic() == 11534336
    assert bench.recorded_traffic() is None
    path.write_text("header\n" + json.dumps(dict(rec, append_source_hash="1" * 16)))
    assert bench.recorded_append_traffic() is None
    assert bench.kernel_source_hash(sources=bench.APPEND_SOURCES) != bench.kernel_source_hash()


def test_host_identity_names_the_cpu_and_the_blas():
    ident = bench.host_identity()
    assert set(ident) == {"cpu_model", "blas", "host_cpus"}
    assert ident["host_cpus"] >= 1
    if ident["blas"] is not None:
        assert ident["blas"]["threads"] >= 1 and ident["blas"]["library"]


def test_window_record():
    w = {"F_first": 981, "F_last": 1000, "kv_lens": [104448, 104562], "fps": 70.0,
         "ms_per_step": 14.2857, "tflops": 1000.0, "avg_launch_ms": 0.58,
         "median_launch_ms": 0.579, "splits": 8}
    r = bench.window_record(w, 2516.6, 24)
    assert r["timed_frames"] == [981, 1000] and r["kv_len"] == [104448, 104562]
    assert r["frac"] == round(1000.0 / 2516.6, 4) and r["blocks"] == 24
