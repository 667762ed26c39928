"""The benchmark's contract pieces that need no GPU: the multi-GPU refusal, the per-family source hashes behind
the traffic records, the workload flags, and the committed profile summaries (each names its command)."""

import glob
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_follows_the_kernel_family():
    tile = bench.kernel_source_hash("tile_256x256x64_mi16")
    assert tile == bench.kernel_source_hash("tile_256x256x32_mi16_nn")  # same source file
    assert tile != bench.kernel_source_hash("skinny_m16_n256_k64")
    assert tile != bench.kernel_source_hash("masked_64x64x64_vecu")
    # the workspace split covers both first passes (skinny or 256 x 256 tiles) and the reduction
    ks = bench.kernel_source_hash("ksplit_skinny_m64_n64_k64+reduce")
    assert ks == bench.kernel_source_hash("ksplit_tile_256x256x64_mi16+reduce")
    assert ks not in (tile, bench.kernel_source_hash("skinny_m16_n64_k64"))
    assert len(bench.kernel_source_hash()) == 16


def test_workload_flags_are_kept_for_the_profile_commands():
    argv = ["--steps", "5", "--workload", "ragged_f16_1000x1500x777", "--no-secondary", "--warmup", "2"]
    assert bench.workload_args(argv) == "--workload ragged_f16_1000x1500x777 --no-secondary"
    assert bench.workload_args(["--secondary", "rowsum_f32_16384x16384"]) == "--secondary rowsum_f32_16384x16384"
    assert bench.workload_args([]) == ""


def test_profile_summaries_name_their_commands():
    texts = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))
    assert texts, "no profile summaries"
    for path in texts:
        head = open(path).read()
        assert "rocprofv3 " in head and "bench.py" in head, f"{os.path.basename(path)} names no command"
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))):
        rec = json.load(open(path))
        for key in ("kernel", "workload", "source_hash", "hbm_bytes_per_launch", "commands"):
            assert key in rec, f"{os.path.basename(path)}: {key}"
        assert all("rocprofv3 --pmc" in c for c in rec["commands"])
        assert os.path.basename(path) == f"traffic_{rec['workload']}.json"


def test_cpu_model_is_named():
    assert bench.cpu_model() and "\n" not in bench.cpu_model()
