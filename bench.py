#!/usr/bin/env python3
"""Throughput of the tree-verification hot path on one MI355X.

One step = ssm_tree_verify over every (layer, sequence) of the workload,
then ssm_tree_commit of each sequence's accepted path (in place), i.e. one
pass of the whole hot path.  Inputs are generated on the host, copied to
HBM before timing, and stay resident.

The JSON line reports verified tree-node-layers/s (layers x sequences x
nodes per step), the roofline of the dominant kernel (algorithmic bytes per
launch over its HIP-event duration, against 8 TB/s), per-kernel figures,
and the float64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verified tree-node-layers/sec (Mamba2-2.7B SSM, 16-node tree); % HBM peak"
KERNEL_SOURCES = {"verify": "mamba2_tree_verification_amd/csrc/verify_mfma.hip",
                  "commit": "mamba2_tree_verification_amd/csrc/commit.hip"}


def algorithmic_bytes(cfg, path_len):
    """Minimal HBM traffic per launch.

    verify: root state + conv window per (layer, sequence); x, B, C, dt_raw
    and the fp32 y per node; parent[] once.  commit: root state read and
    written, window read and written, and x, B, dt_raw of each accepted
    node; path and lengths once.  Parameters are excluded (reported apart).
    """
    e = cfg.e
    L, Bsz, T, H, P, N, G, W, d = cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.d_in
    state = H * P * N * 4
    window = (W - 1) * d * e
    node_in = d * e + 2 * G * N * e + H * e
    verify = L * Bsz * (state + window + T * (node_in + d * 4)) + Bsz * T * 4
    acc = int(sum(int(n) for n in path_len))
    commit = L * (Bsz * (2 * state + 2 * window) + acc * (d * e + G * N * e + H * e)) + Bsz * (T + 1) * 4
    params = L * (3 * H * 4 + d * W * 4)
    return verify, commit, params


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if recorded for
    the current kernel source (see profiles/)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha([KERNEL_SOURCES[kernel], "mamba2_tree_verification_amd/csrc/common.h"]):
        return None
    return rec.get("bytes_per_launch")


PROBE_BYTES = 4 << 30  # the plain copy of hbm_probe: reads and writes this many bytes per dispatch
KERNEL_MATCH = {"verify": ("verify_mfma_kernel", "verify_proj_kernel"), "commit": ("commit_kernel",),
                "copy": ("copyBuffer",)}


def _pmc_per_dispatch(run_dir, counter):
    """Mean value of `counter` per dispatch, by kernel family, from a
    rocprofv3 --pmc run written with --output-format csv."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                for fam, keys in KERNEL_MATCH.items():
                    if any(k in row["Kernel_Name"] for k in keys):
                        acc.setdefault(fam, []).append(float(row["Counter_Value"]))
    return {fam: sum(v) / len(v) for fam, v in acc.items()}


def record_traffic(prof_dir):
    """Write profiles/traffic.json from four rocprofv3 --pmc runs under
    prof_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of this bench),
    copy_fetch/ and copy_write/ (the same counters over `bench.py --probe`).
    Each counter is scaled by bytes-moved / counter-reading of the plain
    4 GiB device copy, so traffic is in bytes per launch."""
    fetch = _pmc_per_dispatch(os.path.join(prof_dir, "fetch"), "FETCH_SIZE")
    write = _pmc_per_dispatch(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    cf = _pmc_per_dispatch(os.path.join(prof_dir, "copy_fetch"), "FETCH_SIZE")["copy"]
    cw = _pmc_per_dispatch(os.path.join(prof_dir, "copy_write"), "WRITE_SIZE")["copy"]
    sf, sw = PROBE_BYTES / (cf * 1024), PROBE_BYTES / (cw * 1024)
    out = {"scale": {"fetch": round(sf, 4), "write": round(sw, 4), "copy_bytes": PROBE_BYTES,
                     "copy_fetch_kib": cf, "copy_write_kib": cw}}
    for k in ("verify", "commit"):
        out[k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                  "bytes_per_launch": int(round(fetch[k] * 1024 * sf + write[k] * 1024 * sw)),
                  "source_sha": source_sha([KERNEL_SOURCES[k], "mamba2_tree_verification_amd/csrc/common.h"])}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(cfg, inp, target_s=12.0, threads=16):
    """Time the float64 oracle (verify + commit) on whole layers of the
    workload until about target_s of wall time is covered."""
    import numpy as np  # noqa: F401
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from testgen.configs import unit_f64

    o = oracle.get()
    # calibrate on one unit, single thread
    u0 = unit_f64(cfg, 0, 0, inp)
    t0 = time.perf_counter()
    o.verify(inp.parent[0], u0, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)
    n0 = int(inp.path_len[0])
    o.commit(inp.parent[0], inp.path[0, :n0], n0, u0, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)
    per_unit = time.perf_counter() - t0
    layers = max(1, min(cfg.L, int(target_s * threads / max(per_unit, 1e-6) / cfg.Bsz)))
    units = [(l, b) for l in range(layers) for b in range(cfg.Bsz)]
    prepared = {lb: unit_f64(cfg, lb[0], lb[1], inp) for lb in units}

    def one(lb):
        l, b = lb
        u = prepared[lb]
        n = int(inp.path_len[b])
        o.verify(inp.parent[b], u, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)
        o.commit(inp.parent[b], inp.path[b, :n], n, u, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)

    # whole passes over the sample until about target_s / threads of wall time
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(one, units))
            passes += 1
            if time.perf_counter() - t0 >= target_s / threads * 4 or passes >= 100:
                break
    wall = time.perf_counter() - t0
    node_layers = passes * len(units) * cfg.T
    return {"value": node_layers / wall, "unit": "tree-node-layers/s", "cores": threads, "kind": "oracle",
            "sample": "verify+commit of layers 0..%d x %d sequences (%d of %d (layer, sequence) units), "
                      "%d pass(es), float64, %.1f s wall" % (layers - 1, cfg.Bsz, len(units), cfg.L * cfg.Bsz, passes,
                                                              wall)}


def hbm_probe(torch, nbytes=4 << 30, reps=10):
    """Plain device copy (torch copy_) and read (torch sum) bandwidth over
    buffers far larger than the 256 MB last-level cache."""
    n = nbytes // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * nbytes), ("read", lambda: a.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"GB/s": round(moved / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4), "bytes": moved}
    return {"probe": "hbm", "buffer_bytes": nbytes, **out}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = Mamba2-2.7B batch 16 x tree 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR and exit")
    ap.add_argument("--probe", action="store_true",
                    help="only measure plain HBM copy and read bandwidth (practical ceilings) and exit")
    args = ap.parse_args(argv)

    if args.record_traffic:
        return record_traffic(args.record_traffic)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the verify and commit "
              "kernels shard by sequence or head with no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    import mamba2_tree_verification_amd as m
    from testgen import configs as C
    from testgen.device import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.probe:
        print(json.dumps(hbm_probe(torch)), flush=True)
        return 0
    m.load()
    cfg = C.CONFIGS[args.config]
    t_gen = time.perf_counter()
    inp = C.make_inputs(cfg, nthreads=args.threads)
    g = upload(inp)
    t_gen = time.perf_counter() - t_gen
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    st_v = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    st_c = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    state = g.state  # committed in place, step after step
    window = g.window

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        m.verify(dims, prm, g.parent, g.x, g.B, g.C, g.dt_raw, window, state, y, st_v)
        if ev is not None:
            ev[1].record()
        m.commit(dims, prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, window, state, window, state, st_c)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not (st_v.cpu() == 0).all() or not (st_c.cpu() == 0).all():
        print("bench: nonzero sequence status", file=sys.stderr)
        return 1

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ver_ms = [e[0].elapsed_time(e[1]) for e in evs]
    com_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    if torch.isnan(y).any():
        print("bench: NaN in y", file=sys.stderr)
        return 1

    # the page's own form (explicit FIFO walk, every child state materialised),
    # timed apart for comparison; not part of the step
    dims_fifo = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, fifo=True)
    fifo_ms = []
    for k in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        m.verify(dims_fifo, prm, g.parent, g.x, g.B, g.C, g.dt_raw, window, state, y, st_v)
        e1.record()
        torch.cuda.synchronize()
        if k:
            fifo_ms.append(e0.elapsed_time(e1))

    vb, cb, pb = algorithmic_bytes(cfg, inp.path_len)
    v_avg = sum(ver_ms) / len(ver_ms)
    c_avg = sum(com_ms) / len(com_ms)
    node_layers = cfg.L * cfg.Bsz * cfg.T

    def roof(kernel, nbytes, ms):
        ach = nbytes / (ms * 1e-3) / 1e9
        tr = load_traffic(kernel)
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr}

    kern = {"verify": dict(ms=round(v_avg, 4), ms_min=round(min(ver_ms), 4), bytes=vb,
                           node_layers_per_s=round(node_layers / (v_avg * 1e-3), 1),
                           roofline=roof("verify", vb, v_avg)),
            "commit": dict(ms=round(c_avg, 4), ms_min=round(min(com_ms), 4), bytes=cb,
                           roofline=roof("commit", cb, c_avg)),
            "verify_fifo_walk": dict(ms=round(sum(fifo_ms) / len(fifo_ms), 4), bytes=vb,
                                     note="SSM_TREE_VERIFY_FIFO, not in the step")}
    dominant = "verify" if v_avg >= c_avg else "commit"
    rec = {
        "metric": METRIC,
        "value": round(node_layers / (ms_per_step * 1e-3), 1),
        "unit": "tree-node-layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.L, "batch": cfg.Bsz, "tree_nodes": cfg.T,
                   "nheads": cfg.H, "headdim": cfg.P, "d_state": cfg.N, "ngroups": cfg.G, "conv_width": cfg.W,
                   "inputs": "bf16" if cfg.bf16 else "f32", "state": "f32",
                   "step": "ssm_tree_verify + in-place ssm_tree_commit", "parallelism": "single-gpu"},
        "roofline": dict(kern[dominant]["roofline"], kernel=dominant),
        "kernels": kern,
        "param_bytes_per_call": pb,
        "verify_hbm_frac": kern["verify"]["roofline"]["frac"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds, args.threads)
    rec["setup_s"] = round(t_gen, 1)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
