"""Host-side parts of bench.py: the one-GPU rule and the profile summaries it
attaches (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_more_than_one_gpu_exits_with_a_message():
    # the check runs before anything touches a GPU
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_profile_summary_names_its_command_and_sources():
    names = sorted(f for f in os.listdir(PROFILES) if f.endswith(".txt"))
    assert names
    for f in names:
        text = open(os.path.join(PROFILES, f)).read()
        assert "rocprofv3" in text, f
        if f != "copy_calibration_256MiB.txt":
            assert any(line.startswith("source_sha256_16:") for line in text.splitlines()), f


def test_profile_fields_attach_only_to_the_sources_they_describe():
    # every configuration bench times has a kernel-trace and a traffic summary;
    # bench attaches one only while its recorded source hash is the current one
    current = bench.source_hash()
    for name, _, _ in bench.CONFIGS:
        for kind, field in (("kernels", "avg_ns"), ("traffic", "traffic_bytes_per_launch")):
            path = os.path.join(PROFILES, f"{kind}_{name}.txt")
            assert os.path.exists(path), path
            lines = open(path).read().splitlines()
            sha = [ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("source_sha256_16:")]
            kernels = [ln.split(":")[0] for ln in lines if ln and not ln.startswith("#") and "=" in ln
                       and not ln.startswith("source_sha256_16")]
            assert sha and kernels, path
            got = bench.profile_fields(name, kind, kernels[0])
            if sha[0] == current:
                assert got is not None and got[field] > 0, (path, kernels[0])
            else:
                assert got is None, path
