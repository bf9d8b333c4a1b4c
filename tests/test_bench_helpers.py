"""bench.py's measurement helpers on the CPU: which call each dispatched
kernel belongs to, the algorithmic byte counts of the headline workload,
the counter-traffic scaling, and the refusal of more than one GPU.  No GPU
and no profiler are needed: the counter files are synthetic."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from testgen import configs as C  # noqa: E402


@pytest.mark.parametrize("name,family", [
    ("void ssmt::commit_verify_kernel<ssmt::bf16_t, float, 8, false, false>(ssmt::CommitVerifyArgs)", "commit_verify"),
    ("void ssmt::commit_verify_kernel<ssmt::bf16_t, float, 8, true, false>(ssmt::CommitVerifyArgs)", "commit_verify"),
    ("void ssmt::commit_verify_kernel<ssmt::bf16_t, float, 8, false, true>(ssmt::CommitVerifyArgs)", "verify"),
    ("void ssmt::verify_tt_ws_kernel<ssmt::bf16_t, float, 8, 4, true>(ssmt::CommitVerifyArgs, int)", "commit_verify"),
    ("void ssmt::verify_tt_ws_kernel<ssmt::bf16_t, float, 8, 4, false>(ssmt::CommitVerifyArgs, int)", "verify"),
    ("void ssmt::verify_tt_kernel<ssmt::bf16_t, float, 8, 4, false>(ssmt::VerifyArgs, int)", "verify"),
    ("void ssmt::verify_proj_kernel<float, float, 2>(ssmt::VerifyArgs)", "verify"),
    ("void ssmt::commit_kernel<ssmt::bf16_t, float, 8>(ssmt::CommitArgs, int)", "commit"),
    ("void ssmt::verify_fifo_kernel<ssmt::bf16_t, 8>(ssmt::VerifyArgs, int, int)", "verify_fifo"),
    ("void (anonymous namespace)::probe_kernel<1, 0, 0>(float const*, float*, long, int, unsigned int*)", "copy"),
    ("void (anonymous namespace)::probe_kernel<1, 0, 1>(float const*, float*, long, int, unsigned int*)", None),
    # the options' helpers are not the round's kernel
    ("void ssmt::bc_conv_kernel<ssmt::bf16_t>(ssmt::CommitVerifyArgs)", None),
    ("void ssmt::commit_window_bc_kernel<ssmt::bf16_t>(ssmt::WindowBcArgs)", None),
    ("__amd_rocclr_copyBuffer", None),
])
def test_kernel_family(name, family):
    assert bench.kernel_family(name) == family


def test_algorithmic_bytes_of_the_headline_workload():
    """Mamba2-2.7B batch 16, 16-node trees, bf16 inputs, fp32 state: per
    (layer, sequence) the root state is 80 x 64 x 128 x 4 = 2,621,440 B, the
    conv window 3 x 5120 x 2 = 30,720 B, and each node reads x (10,240 B),
    B and C (512 B), dt_raw (160 B) and writes y (20,480 B)."""
    cfg = C.CONFIGS[3]
    units, T = cfg.L * cfg.Bsz, cfg.T
    state, window, node_in, node_y = 2_621_440, 30_720, 10_240 + 512 + 160, 20_480
    parent = cfg.Bsz * T * 4
    no_path = [0] * cfg.Bsz
    ab = bench.algorithmic_bytes(cfg, no_path)
    assert ab["verify"] == units * (state + window + T * (node_in + node_y)) + parent == 3_230_139_392
    # nothing accepted: the commit reads and writes state and window only
    assert ab["commit"] == units * 2 * (state + window) + cfg.Bsz * (T + 1) * 4
    # every accepted node adds its x, B and dt_raw once per layer
    one = [1] * cfg.Bsz
    ab1 = bench.algorithmic_bytes(cfg, one)
    assert ab1["commit"] - ab["commit"] == cfg.L * cfg.Bsz * (10_240 + 256 + 160)
    # the fused round: the commit's bytes plus the next tree's inputs, y and parent[]
    assert ab1["commit_verify"] - ab1["commit"] == units * T * (node_in + node_y) + parent


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kn, cn, v in rows:
            w.writerow({"Kernel_Name": kn, "Counter_Name": cn, "Counter_Value": v})


def test_record_traffic_scales_counters_by_the_copy_probe(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are averaged per kernel
    family and scaled by bytes / reading of the plain 4 GiB copy probe."""
    rnd = "void ssmt::commit_verify_kernel<ssmt::bf16_t, float, 8, false, false>(ssmt::CommitVerifyArgs)"
    ver = "void ssmt::commit_verify_kernel<ssmt::bf16_t, float, 8, false, true>(ssmt::CommitVerifyArgs)"
    copy = "void (anonymous namespace)::probe_kernel<1, 0, 0>(float const*, float*, long, int, unsigned int*)"
    prof = tmp_path / "pmc"
    # the round: 900 and 1100 KiB fetched (mean 1000), 500 KiB written; verify 300 / 40
    _counter_csv(str(prof / "fetch"), [(rnd, "FETCH_SIZE", 900), (rnd, "FETCH_SIZE", 1100), (ver, "FETCH_SIZE", 300)])
    _counter_csv(str(prof / "write"), [(rnd, "WRITE_SIZE", 500), (ver, "WRITE_SIZE", 40)])
    # the copy probe moves 4 GiB each way: a fetch reading of 2 GiB-worth
    # (scale 2) and a write reading of 4 GiB-worth (scale 1)
    _counter_csv(str(prof / "copy_fetch"), [(copy, "FETCH_SIZE", 2 * 1024 * 1024)])
    _counter_csv(str(prof / "copy_write"), [(copy, "WRITE_SIZE", 4 * 1024 * 1024)])
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda paths: "sha")
    cfg = C.CONFIGS[3]
    assert bench.record_traffic(str(prof), cfg) == 0
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert rec["scale"]["fetch"] == 2.0 and rec["scale"]["write"] == 1.0
    ent = rec["workloads"][cfg.name]
    assert ent["commit_verify"]["bytes_per_launch"] == 1000 * 1024 * 2 + 500 * 1024
    assert ent["verify"]["bytes_per_launch"] == 300 * 1024 * 2 + 40 * 1024
    assert "commit" not in ent  # no dispatch of it in these runs
    # and the bench reads it back for the same source only
    assert bench.load_traffic("commit_verify", cfg) == 1000 * 1024 * 2 + 500 * 1024
    monkeypatch.setattr(bench, "source_sha", lambda paths: "other")
    assert bench.load_traffic("commit_verify", cfg) is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
