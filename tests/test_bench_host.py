"""Host-side logic of bench.py, on the CPU: the code hash that ties the
committed byte counters to the kernel sources, the counter-file parsing,
and the refusal of runs on more than one GPU."""
import importlib.util
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _copy_sources(tmp_path):
    dst = tmp_path / "combine_dispatch_layout_02_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "combine_dispatch_layout_02_amd", "csrc"), dst)
    return dst


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    b = _bench()
    ref = b.kernel_source_hash()
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.kernel_source_hash() == ref
    p = csrc / "combine.hip"
    p.write_text(p.read_text() + "\n// a comment\n/* and a\n   block comment */\n\n   \n")
    assert b.kernel_source_hash() == ref


def test_source_hash_changes_with_code(tmp_path, monkeypatch):
    b = _bench()
    ref = b.kernel_source_hash()
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    p = csrc / "dispatch.hip"
    p.write_text(p.read_text() + "\nnamespace ep { constexpr int kUnused = 1; }\n")
    assert b.kernel_source_hash() != ref


def test_measured_traffic_reads_matching_counters_only(tmp_path, monkeypatch):
    b = _bench()
    sha = b.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = ["# comment line", "workload=w1", f"kernel_sources_sha256={sha}", "fetch_scale=2.0", "write_scale=1.0",
            "kernel=ep_combine_bf16_kernel<4,8> fetch_kib=1.0 write_kib=1.0 read_bytes=2048 write_bytes=1024 "
            "traffic_bytes=3072"]
    (prof / "counters_w1.txt").write_text("\n".join(body) + "\n")
    body[2] = "kernel_sources_sha256=" + "0" * 64
    (prof / "counters_w2.txt").write_text("\n".join(body) + "\n")
    monkeypatch.setattr(b, "PROFILES", str(prof))
    assert b.measured_traffic("w1", "ep_combine_bf16_kernel") == 3072
    assert b.measured_traffic("w1", "ep_dispatch_copy_kernel") is None   # no such kernel line
    assert b.measured_traffic("w2", "ep_combine_bf16_kernel") is None    # counters of other code
    assert b.measured_traffic("w3", "ep_combine_bf16_kernel") is None    # no counter file


def test_committed_counter_files_parse():
    b = _bench()
    names = [f for f in os.listdir(b.PROFILES) if f.startswith("counters_") and f.endswith(".txt")]
    assert names
    for f in names:
        fields = {}
        for line in open(os.path.join(b.PROFILES, f)):
            if line.startswith("#") or "=" not in line:
                continue
            parts = dict(p.split("=", 1) for p in line.split())
            if "kernel" in parts:
                # each field is rounded on its own: the sum may differ by a byte
                assert abs(int(parts["traffic_bytes"]) - int(parts["read_bytes"]) - int(parts["write_bytes"])) <= 2, \
                    (f, parts["kernel"])
            else:
                fields.update(parts)
        assert len(fields.get("kernel_sources_sha256", "")) == 64, f
        assert float(fields["fetch_scale"]) > 0 and float(fields["write_scale"]) > 0, f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_mix_ceiling_weights_the_read_and_write_rates():
    b = _bench()
    ceil = {"read": {"gbs": 6000.0}, "write": {"gbs": 4000.0}}
    assert b.mix_ceiling(1e9, 0.0, ceil) == 6000.0
    assert b.mix_ceiling(0.0, 1e9, ceil) == 4000.0
    # half and half: the bus time of each share, one after the other
    mixed = b.mix_ceiling(1e9, 1e9, ceil)
    assert abs(mixed - 2e9 / (1e9 / 6000.0 + 1e9 / 4000.0)) < 1e-6
    assert 4000.0 < mixed < 6000.0
    assert b.mix_ceiling(0.0, 0.0, ceil) == 0.0


def test_host_cores_follows_the_job_share(monkeypatch):
    b = _bench()
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert b.host_cores() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.setenv("OMP_NUM_THREADS", "")
    assert b.host_cores() == len(os.sched_getaffinity(0))
