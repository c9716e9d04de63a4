"""Host-side pieces of bench.py (no GPU): the HBM traffic it reports next to a
roofline comes from a counter summary under profiles/ and is used only while the
measured kernels' sources hash as they did when the counters were taken."""

import hashlib
import os
import shutil

import pytest

import bench

SOURCES = "gemm_a16.hip+small_unit.h+device_common.h+lds_copy.h+host_internal.h"


def _tree(tmp_path):
    """A copy of the kernel sources and a summary whose rows carry their hashes: a
    kernel name with a comma in its template arguments, and two rows of a stage."""
    root = tmp_path / "repo"
    csrc = root / "mxfp4_weights_fp8_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "mxfp4_weights_fp8_amd", "csrc"), csrc)
    h = hashlib.sha256()
    for name in SOURCES.split("+"):
        h.update((csrc / name).read_bytes())
    sha = h.hexdigest()
    (root / "profiles").mkdir()
    (root / "profiles" / "wl_traffic.txt").write_text(
        "# comment line, ignored\n"
        "kernel,dispatches,fetch_kib,write_kib,traffic_bytes,source_files,source_sha256\n"
        f"moe::k_w13_a16<false, 4>,16,1.0,2.0,1000,{SOURCES},{sha}\n"
        f"moe::k_a,4,1.0,2.0,300,{SOURCES},{sha}\n"
        f"moe::k_b,4,1.0,2.0,40,{SOURCES},{sha}\n"
        "moe::k_plan_fused,17,9.5,2.3,21923,-,-\n")
    return root, csrc


def test_traffic_lookup(tmp_path, monkeypatch):
    root, csrc = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.measured_traffic("wl", "moe::k_w13_a16<false, 4>") == 1000
    assert bench.measured_traffic("wl", ["moe::k_a", "moe::k_b"]) == 340      # a stage: the sum
    assert bench.measured_traffic("wl", ["moe::k_a", "moe::k_missing"]) is None
    assert bench.measured_traffic("wl", "moe::k_plan_fused") is None          # no sources recorded
    assert bench.measured_traffic("no_such_workload", "moe::k_a") is None
    # a changed source makes every row that hashed it stale
    (csrc / "small_unit.h").write_text((csrc / "small_unit.h").read_text() + "\n// changed\n")
    assert bench.measured_traffic("wl", "moe::k_w13_a16<false, 4>") is None
    assert bench.measured_traffic("wl", ["moe::k_a", "moe::k_b"]) is None


def test_committed_summaries_parse():
    """Every committed counter summary has the columns the lookup expects."""
    for name in os.listdir(os.path.join(bench.ROOT, "profiles")):
        if not name.endswith("_traffic.txt"):
            continue
        rows = [l for l in open(os.path.join(bench.ROOT, "profiles", name)) if l.strip() and not l.startswith("#")]
        assert rows[0].strip() == "kernel,dispatches,fetch_kib,write_kib,traffic_bytes,source_files,source_sha256"
        for r in rows[1:]:
            f = r.strip().rsplit(",", 6)
            assert len(f) == 7 and f[0].startswith("moe::"), (name, r)
            float(f[4])


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
