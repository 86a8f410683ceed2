"""Host-side logic of bench.py (no GPU): the command-line contract for more than one GPU and
the lookup of the committed HBM-traffic records, which must be ignored once the kernel source
they were measured on has changed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from normalisation_dilated_conv1d_amd.profiling import source_digest  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_unknown_workload_is_none():
    assert bench.measured_traffic(0) is None
    assert bench.measured_traffic(2) is None


def test_traffic_committed_records_match_sources():
    """Every committed traffic record describes the kernel source as it is now."""
    for workload in sorted(bench.TRAFFIC_FILES):
        assert bench.measured_traffic(workload) is not None, workload


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC_FILES))
def test_traffic_record_lookup(workload, tmp_path, monkeypatch):
    kernel, _ = bench.TRAFFIC_FILES[workload]
    rec = {"kernel": kernel, "source_sha256": source_digest(kernel),
           "traffic_bytes_per_launch": 123456.0}
    path = tmp_path / "t.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setitem(bench.TRAFFIC_FILES, workload, (kernel, str(path)))
    assert bench.measured_traffic(workload) == 123456.0
    # a record taken on other sources, or for another kernel, is not used
    path.write_text(json.dumps(dict(rec, source_sha256="0" * 64)))
    assert bench.measured_traffic(workload) is None
    other = "conv_bf16_kernel" if kernel == "conv_f32_kernel" else "conv_f32_kernel"
    path.write_text(json.dumps(dict(rec, kernel=other)))
    assert bench.measured_traffic(workload) is None
    # a missing or unreadable record gives None rather than an error
    path.write_text("{not json")
    assert bench.measured_traffic(workload) is None
    monkeypatch.setitem(bench.TRAFFIC_FILES, workload, (kernel, str(tmp_path / "missing.json")))
    assert bench.measured_traffic(workload) is None


def test_source_digest_ignores_comments_only():
    """Comments and layout do not change what the compiler sees; any code token does."""
    from normalisation_dilated_conv1d_amd.profiling import strip_comments
    base = 'int f(int a) {\n  // twice\n  return 2 * a; /* a */\n}\nconst char* s = "x // y";\n'
    reworded = 'int f(int a) {   // doubles a\n  return 2 * a;\n}\n/* the literal */\nconst char* s = "x // y";'
    assert strip_comments(base) == strip_comments(reworded)
    assert strip_comments(base) != strip_comments(base.replace("2 * a", "3 * a"))
    # comment markers inside string literals are code
    assert strip_comments(base) != strip_comments(base.replace('"x // y"', '"x "'))
    assert strip_comments("a/**/b") == "a b"


def test_source_digest_covers_per_file_flags(monkeypatch):
    """A compile flag given to one kernel's source changes that kernel's machine code, so it
    makes that kernel's counter records stale and leaves the others valid."""
    from normalisation_dilated_conv1d_amd import build
    before = {k: source_digest(k) for k in ("conv_f32_kernel", "conv_gn_fused_kernel")}
    flags = dict(build.FILE_FLAGS)
    flags["conv_f32.hip"] = flags.get("conv_f32.hip", []) + ["-mllvm", "-some-other-choice"]
    monkeypatch.setattr(build, "FILE_FLAGS", flags)
    assert source_digest("conv_f32_kernel") != before["conv_f32_kernel"]
    assert source_digest("conv_gn_fused_kernel") == before["conv_gn_fused_kernel"]
