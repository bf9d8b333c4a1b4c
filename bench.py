#!/usr/bin/env python3
"""Throughput of the tree-verification hot path on one MI355X.

One step = one round of speculative decoding over every (layer, sequence)
of the workload: the previous tree's accepted path is committed into the
root state and conv window (in place) and the next tree is verified from
the committed state, by one ssm_tree_commit_verify call, i.e. one pass of
the whole hot path.  Two trees of the workload's shape alternate as
previous and next.  Inputs are generated on the host, copied to HBM before
timing, and stay resident.

The JSON line reports verified tree-node-layers/s (layers x sequences x
nodes per step), the roofline of the step's kernel (algorithmic bytes per
launch over its HIP-event duration, against 8 TB/s), the same figures for
the separate ssm_tree_verify and ssm_tree_commit kernels and for the
explicit FIFO walk (timed apart, outside the step), and the float64 oracle
timed on a bounded sample on the host cores.
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
CSRC = "mamba2_tree_verification_amd/csrc/"
KERNELS = ("verify", "commit", "commit_verify", "verify_fifo")


def verify_source(cfg):
    """The verify kernel a workload's shape dispatches to (plain flags)."""
    if cfg.T <= 16 and cfg.P % 16 == 0:
        return CSRC + "commit_verify.hip"  # the round's kernel with nothing to commit
    if cfg.T <= 64 and cfg.P % 16 == 0 and (cfg.d_in // cfg.G) % 64 == 0:
        return CSRC + "verify_tt.hip"
    return CSRC + "verify.hip"


def tt_round(cfg):
    """Whether a workload's round of 17-64-node trees runs as one launch of
    the role-split verify (else as commit, then verify)."""
    return (cfg.bf16 and 16 < cfg.T <= 64 and cfg.N <= 128 and cfg.P % 64 == 0
            and (cfg.d_in // cfg.G) % 512 == 0)


def kernel_sources(kernel, cfg):
    """Source files whose change invalidates a recorded traffic figure."""
    if kernel == "verify":
        files = [verify_source(cfg)]
    elif kernel == "verify_fifo":
        files = [CSRC + "verify_fifo.hip"]
    elif kernel == "commit":
        files = [CSRC + "commit.hip"]
    elif cfg.T <= 16 and cfg.P % 16 == 0:
        files = [CSRC + "commit_verify.hip"]
    elif tt_round(cfg):
        files = [CSRC + "verify_tt.hip"]
    else:  # the round runs as a commit followed by a verify
        files = [CSRC + "commit.hip", verify_source(cfg)]
    return files + [CSRC + "common.h"]


def _last_template_arg(name):
    head = name.split("(")[0]
    return head[head.rfind(",") + 1:].strip(" >") if "<" in head else ""


def kernel_family(name):
    """Which call a dispatched kernel belongs to: verify, commit,
    commit_verify (the round), verify_fifo (the FIFO walk), copy (the plain
    coalesced copy probe), or None.  The round's kernel with nothing to commit (last template argument
    true) serves ssm_tree_verify on trees of at most 16 nodes; the
    role-split verify with the commit (last argument true) is the round of
    17-64-node trees."""
    if "probe_kernel<1, 0, 0>" in name:
        return "copy"
    if "commit_verify_kernel<" in name:
        return "verify" if _last_template_arg(name) == "true" else "commit_verify"
    if "verify_tt_ws_kernel<" in name:
        return "commit_verify" if _last_template_arg(name) == "true" else "verify"
    if any(k in name for k in ("verify_tt_kernel", "verify_proj_kernel")):
        return "verify"
    if "::commit_kernel" in name:
        return "commit"
    if "verify_fifo_kernel<" in name:
        return "verify_fifo"
    return None


def algorithmic_bytes(cfg, path_len):
    """Minimal HBM traffic per launch.

    verify: root state + conv window per (layer, sequence); x, B, C, dt_raw
    and the fp32 y per node; parent[] once.  commit: root state read and
    written, window read and written, and x, B, dt_raw of each accepted
    node; path and lengths once.  commit_verify: the commit's bytes plus the
    next tree's per-node inputs and y and its parent[] (the root state and
    window are read once, by the commit).  Parameters are excluded (reported
    apart).
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
    fused = commit + L * Bsz * T * (node_in + d * 4) + Bsz * T * 4
    return {"verify": verify, "commit": commit, "commit_verify": fused, "params": params}


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, cfg):
    """HBM bytes per launch measured with rocprofv3 counters on this
    workload, if recorded for the current kernel source (see profiles/)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get("workloads", {}).get(cfg.name, {}).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel_sources(kernel, cfg)):
        return None
    return rec.get("bytes_per_launch")


PROBE_BYTES = 4 << 30  # hbm_probe's buffer: the copy probe reads and writes this many bytes per dispatch


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
                fam = kernel_family(row["Kernel_Name"])
                if fam:
                    acc.setdefault(fam, []).append(float(row["Counter_Value"]))
    return {fam: sum(v) / len(v) for fam, v in acc.items()}


def record_traffic(prof_dir, cfg):
    """Add this workload's entry to profiles/traffic.json from four
    rocprofv3 --pmc runs under prof_dir: fetch/ and write/ (FETCH_SIZE,
    WRITE_SIZE of this bench on the workload), copy_fetch/ and copy_write/
    (the same counters over `bench.py --probe --copy-only`).  Each counter is
    scaled by bytes-moved / counter-reading of the plain 4 GiB copy probe,
    so traffic is in bytes per launch.  A kernel the workload runs as several launches
    (the round of a tree too deep for the fused kernel) is not recorded."""
    fetch = _pmc_per_dispatch(os.path.join(prof_dir, "fetch"), "FETCH_SIZE")
    write = _pmc_per_dispatch(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    cf = _pmc_per_dispatch(os.path.join(prof_dir, "copy_fetch"), "FETCH_SIZE")["copy"]
    cw = _pmc_per_dispatch(os.path.join(prof_dir, "copy_write"), "WRITE_SIZE")["copy"]
    sf, sw = PROBE_BYTES / (cf * 1024), PROBE_BYTES / (cw * 1024)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out.setdefault("workloads", {})
    out = {"scale": {"fetch": round(sf, 4), "write": round(sw, 4), "copy_bytes": PROBE_BYTES,
                     "copy_fetch_kib": cf, "copy_write_kib": cw}, "workloads": out["workloads"]}
    ent = {}
    for k in KERNELS:
        if k not in fetch or k not in write:
            continue
        ent[k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                  "bytes_per_launch": int(round(fetch[k] * 1024 * sf + write[k] * 1024 * sw)),
                  "source_sha": source_sha(kernel_sources(k, cfg))}
    out["workloads"][cfg.name] = ent
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out), flush=True)
    return 0


def host_cpu():
    """CPU model and counts of the host this runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(cfg, inp, target_s=12.0, threads=16, per_core_cfg=None):
    """Time the float64 oracle (verify + commit) on whole layers of the
    workload until about target_s of CPU time is covered, on `threads`
    worker threads (at most the CPUs this process may use); then one thread
    on the per-core workload for a per-core rate."""
    import numpy as np  # noqa: F401
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from testgen.configs import unit_f64

    o = oracle.get()
    host = host_cpu()
    threads = max(1, min(threads, host["usable_cpus"]))
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

    def one(ci, pin, lb, u):
        l, b = lb
        n = int(pin.path_len[b])
        o.verify(pin.parent[b], u, ci.H, ci.P, ci.N, ci.G, ci.W, ci.silu)
        o.commit(pin.parent[b], pin.path[b, :n], n, u, ci.H, ci.P, ci.N, ci.G, ci.W, ci.silu)

    # whole passes over the sample until about target_s / threads of wall time
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(lambda lb: one(cfg, inp, lb, prepared[lb]), units))
            passes += 1
            if time.perf_counter() - t0 >= target_s / threads * 4 or passes >= 100:
                break
    wall = time.perf_counter() - t0
    node_layers = passes * len(units) * cfg.T
    out = {"value": node_layers / wall, "unit": "tree-node-layers/s", "cores": threads, "kind": "oracle",
           "sample": "verify+commit of layers 0..%d x %d sequences (%d of %d (layer, sequence) units), "
                     "%d pass(es), float64, %.1f s wall on %d threads" % (
                         layers - 1, cfg.Bsz, len(units), cfg.L * cfg.Bsz, passes, wall, threads), **host}
    if per_core_cfg is not None:
        from testgen import configs as C
        pc = per_core_cfg
        pin = C.make_inputs(pc, nthreads=threads)
        punits = [(l, b) for l in range(pc.L) for b in range(pc.Bsz)]
        pprep = {lb: unit_f64(pc, lb[0], lb[1], pin) for lb in punits}
        done = 0
        t0 = time.perf_counter()
        while True:
            for lb in punits:
                one(pc, pin, lb, pprep[lb])
            done += 1
            if time.perf_counter() - t0 >= 2.0:
                break
        w1 = time.perf_counter() - t0
        out["per_core"] = {"workload": pc.name, "threads": 1,
                           "value": round(done * len(punits) * pc.T / w1, 1), "unit": "tree-node-layers/s",
                           "sample": "verify+commit of all %d units, %d pass(es), %.1f s" % (len(punits), done, w1)}
    return out


def rotated_rates(torch, m, C, cid, threads, min_bytes=1 << 30, reps=3):
    """Verify alone and the fused round on a workload small enough to sit in
    the 256 MB last-level cache, with enough independent input sets (each
    with its own trees, inputs, root state and window) that consecutive
    calls never find their bytes in that cache: the sets are cycled in
    turn, every call timed with HIP events on the launch stream."""
    from testgen.device import upload
    cfg = C.CONFIGS[cid]
    ab = algorithmic_bytes(cfg, np_zeros(cfg.Bsz))
    per_set = ab["verify"] + ab["commit_verify"]
    K = max(3, -(-min_bytes // per_set))
    sets = []
    for k in range(K):
        ck = cfg.replace(cid=cfg.cid + 1000 + k)
        inp = C.make_inputs(ck, nthreads=threads)
        nx = C.make_inputs(ck.replace(cid=ck.cid + 500), nthreads=threads,
                           skip=("state", "window", "A", "D", "dt_bias", "conv_w", "conv_b"))
        g, g2 = upload(inp), upload(nx)
        sets.append((g, g2, inp.path_len, nx.path_len))
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prms = [m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b) for g, _, _, _ in sets]
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    st_c = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    st_v = torch.empty_like(st_c)
    flips = [0] * K

    def verify(i):
        g = sets[i][0]
        m.verify(dims, prms[i], g.parent, g.x, g.B, g.C, g.dt_raw, g.window, g.state, y, st_v)

    def round_(i):
        g, g2 = sets[i][0], sets[i][1]
        prev, nxt = (g, g2) if flips[i] % 2 == 0 else (g2, g)
        flips[i] += 1
        m.commit_verify(dims, prms[i], prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, g.window,
                        g.state, g.window, g.state, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, y, st_c, st_v)

    def timed_cycle(fn):
        for i in range(K):  # one untimed pass
            fn(i)
        torch.cuda.synchronize()
        evs = []
        for r in range(reps):
            for i in range(K):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn(i)
                e1.record()
                evs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    vms, rms = timed_cycle(verify), timed_cycle(round_)
    if not (st_v.cpu() == 0).all() or not (st_c.cpu() == 0).all() or torch.isnan(y).any():
        raise SystemExit("bench: bad status or NaN on workload %d" % cid)
    nl = cfg.L * cfg.Bsz * cfg.T
    rb = sum((algorithmic_bytes(cfg, a)["commit_verify"] + algorithmic_bytes(cfg, b)["commit_verify"]) // 2
             for _, _, a, b in sets) // K

    def rate(ms, nbytes):
        a = sum(ms) / len(ms)
        gbs = nbytes / (a * 1e-3) / 1e9
        return {"ms": round(a, 4), "ms_min": round(min(ms), 4), "bytes": nbytes,
                "node_layers_per_s": round(nl / (a * 1e-3), 1), "GBps": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4)}

    out = {"workload": cfg.name, "input_sets": K, "bytes_per_set": per_set,
           "verify": rate(vms, ab["verify"]), "round": rate(rms, rb),
           "note": "sets cycled so that no call finds its inputs in the last-level cache; not in the step"}
    del sets, prms
    torch.cuda.empty_cache()
    return out


def stress_workload(torch, m, C, threads, reps=4):
    """The batch-64 tree-64 stress workload (64-node trees, 10.7 GB of root
    state, far past the last-level cache): the one-launch round in place,
    verify alone, and the same round as the two calls (commit in place, then
    verify), each timed with HIP events; inputs resident before timing."""
    from testgen.device import upload
    cfg = C.CONFIGS[4]
    inp = C.make_inputs(cfg, nthreads=threads)
    nx = C.make_inputs(cfg.replace(cid=cfg.cid + 500), nthreads=threads,
                       skip=("state", "window", "A", "D", "dt_bias", "conv_w", "conv_b"))
    g, g2 = upload(inp), upload(nx)
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    st_c = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    st_v = torch.empty_like(st_c)
    flip = [0]

    def round_():
        prev, nxt = (g, g2) if flip[0] % 2 == 0 else (g2, g)
        flip[0] += 1
        m.commit_verify(dims, prm, prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, g.window,
                        g.state, g.window, g.state, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, y, st_c, st_v)

    def verify():
        m.verify(dims, prm, g2.parent, g2.x, g2.B, g2.C, g2.dt_raw, g.window, g.state, y, st_v)

    def two_calls():
        prev, nxt = (g, g2) if flip[0] % 2 == 0 else (g2, g)
        flip[0] += 1
        m.commit(dims, prm, prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, g.window, g.state,
                 g.window, g.state, st_c)
        m.verify(dims, prm, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, g.window, g.state, y, st_v)

    def timed(fn):
        for _ in range(WARM_EXTRA // 2):  # the ramp to the steady rate (10 calls of 64-node trees)
            fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return out

    rms, vms, tms = timed(round_), timed(verify), timed(two_calls)
    if not (st_v.cpu() == 0).all() or not (st_c.cpu() == 0).all() or torch.isnan(y).any():
        raise SystemExit("bench: bad status or NaN on the stress workload")
    a1, a2 = algorithmic_bytes(cfg, inp.path_len), algorithmic_bytes(cfg, nx.path_len)
    rb = (a1["commit_verify"] + a2["commit_verify"]) // 2
    nl = cfg.L * cfg.Bsz * cfg.T

    def rate(ms, nbytes):
        a = sum(ms) / len(ms)
        gbs = nbytes / (a * 1e-3) / 1e9
        return {"ms": round(a, 4), "ms_min": round(min(ms), 4), "bytes": nbytes,
                "node_layers_per_s": round(nl / (a * 1e-3), 1), "GBps": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4)}

    out = {"workload": cfg.name, "round": dict(rate(rms, rb), kernel="verify_tt_ws_kernel (one launch)"),
           "verify": dict(rate(vms, a2["verify"]), kernel="verify_tt_ws_kernel"),
           "two_call_round": dict(rate(tms, rb), kernels="commit_kernel + verify_tt_ws_kernel"),
           "note": "not in the step"}
    del g, g2, y
    torch.cuda.empty_cache()
    return out


def np_zeros(n):
    import numpy as np
    return np.zeros(n, np.int32)


def per_layer_round(torch, m, cfg, g, g2, state, window, y, st_c, st_v, timed):
    """The decode round as a model issues it: one ssm_tree_commit_verify call
    per layer (L launches, each with L = 1), through the raw C entry point
    with precomputed addresses, plain and replayed from a HIP graph captured
    on a side stream.  Not part of the step; reported apart."""
    dims1 = m.make_dims(1, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prms = [m.make_params(g.A[l], g.D[l], g.dt_bias[l], g.conv_w[l], None if g.conv_b is None else g.conv_b[l])
            for l in range(cfg.L)]

    def addr(t):
        return None if t is None else t.data_ptr()

    calls = [(prms[l], addr(g.parent), addr(g.path), addr(g.path_len), addr(g.x[l]), addr(g.B[l]), None,
              addr(g.dt_raw[l]), addr(window[l]), addr(state[l]), addr(window[l]), addr(state[l]),
              addr(g2.parent), addr(g2.x[l]), addr(g2.B[l]), addr(g2.C[l]), addr(g2.dt_raw[l]), None, addr(y[l]),
              addr(st_c), addr(st_v)) for l in range(cfg.L)]

    def round_():
        hs = torch.cuda.current_stream().cuda_stream
        for c in calls:
            rc = m.ssm_tree_commit_verify(dims1, *c, hs)
            if rc != m.OK:
                raise m.SsmTreeError(rc, "ssm_tree_commit_verify")

    plain = timed(round_)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        round_()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        round_()
    torch.cuda.synchronize()
    replay = timed(graph.replay)
    node_layers = cfg.L * cfg.Bsz * cfg.T

    def avg(v):
        return sum(v) / len(v)

    return {"launches": cfg.L, "plain_ms": round(avg(plain), 4), "graph_ms": round(avg(replay), 4),
            "graph_node_layers_per_s": round(node_layers / (avg(replay) * 1e-3), 1),
            "note": "one call per layer (L = 1 each); not in the step"}


def draft_decode(torch, m, C, upload, threads, timed, steps=15):
    """The draft side (SpecMamba page sec. 3.1) on the Mamba2-370M draft
    shape (48 layers, batch 1): tokens decoded one at a time, each a
    one-node ssm_tree_commit_verify round that commits the previous token
    into the working state (in place) and emits the new token's y.  A chain
    of steps + 1 tokens is the per-token log.  Plain launches through the
    raw entry point, and the whole chain replayed from a HIP graph."""
    cfg = C.CONFIGS[1]
    inp = C.make_inputs(cfg, nthreads=threads)
    g = upload(inp)
    dims1 = m.make_dims(cfg.L, cfg.Bsz, 1, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)
    one = torch.full((cfg.Bsz, 1), -1, dtype=torch.int32, device="cuda")
    path0 = torch.zeros((cfg.Bsz, 1), dtype=torch.int32, device="cuda")
    plen = torch.ones((cfg.Bsz,), dtype=torch.int32, device="cuda")
    tok = {k: [t[:, :, i:i + 1].contiguous() for i in range(cfg.T)] for k, t in
           (("x", g.x), ("B", g.B), ("C", g.C), ("dt", g.dt_raw))}
    y = torch.empty((cfg.L, cfg.Bsz, 1, cfg.d_in), dtype=torch.float32, device="cuda")
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    st, win = g.state, g.window
    calls = [(prm, one.data_ptr(), path0.data_ptr(), plen.data_ptr(), tok["x"][k - 1].data_ptr(),
              tok["B"][k - 1].data_ptr(), None, tok["dt"][k - 1].data_ptr(), win.data_ptr(), st.data_ptr(),
              win.data_ptr(), st.data_ptr(), one.data_ptr(), tok["x"][k].data_ptr(), tok["B"][k].data_ptr(),
              tok["C"][k].data_ptr(), tok["dt"][k].data_ptr(), None, y.data_ptr(), cst.data_ptr(),
              vst.data_ptr()) for k in range(1, steps + 1)]

    def chain():
        hs = torch.cuda.current_stream().cuda_stream
        for c in calls:
            rc = m.ssm_tree_commit_verify(dims1, *c, hs)
            if rc != m.OK:
                raise m.SsmTreeError(rc, "ssm_tree_commit_verify")

    plain = timed(chain)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        chain()
    torch.cuda.synchronize()
    replay = timed(graph.replay)
    torch.cuda.synchronize()
    if not (cst.cpu() == 0).all() or not (vst.cpu() == 0).all() or torch.isnan(y).any():
        raise SystemExit("bench: draft decode produced a bad status or NaN")
    e = cfg.e
    per_layer = (2 * cfg.H * cfg.P * cfg.N * 4 + 2 * (cfg.W - 1) * cfg.d_in * e +
                 (cfg.d_in * e + cfg.G * cfg.N * e + cfg.H * e) +
                 (cfg.d_in * e + 2 * cfg.G * cfg.N * e + cfg.H * e + cfg.d_in * 4))
    token_bytes = cfg.L * cfg.Bsz * per_layer

    def avg(v):
        return sum(v) / len(v)

    tp, tg = avg(plain) / steps, avg(replay) / steps
    return {"workload": cfg.name, "layers": cfg.L, "batch": cfg.Bsz, "bytes_per_token": token_bytes,
            "plain_us_per_token": round(tp * 1e3, 2), "graph_us_per_token": round(tg * 1e3, 2),
            "graph_tokens_per_s": round(1e3 / tg, 1), "graph_GBps": round(token_bytes / (tg * 1e-3) / 1e9, 1),
            "note": "one-node ssm_tree_commit_verify per draft token (all layers in one call); not in the step"}


# untimed rounds before an extra round is timed: a fresh process or workload
# takes about 20 rounds to reach its steady rate
WARM_EXTRA = 20


def options_round(torch, m, C, cfg, g, g2, state, timed, threads, path_lens):
    """The same decode round with the Mamba2-convention options: SiLU over
    the conv of x, B and C (SSM_TREE_CONV_XBC) and the output gate
    y * silu(z).  The window, conv weights and gate inputs of the option
    shapes are drawn for the workload; trees, state and the other inputs are
    the bench's own.  Not part of the step; reported apart."""
    from testgen.device import tensor
    co = cfg.replace(cid=cfg.cid + 600, silu=True, xbc=True, gate=True)
    win = tensor(C.draw(co, "window", nthreads=threads), cfg.bf16)
    cw = tensor(C.draw(co, "conv_w", nthreads=threads), False)
    zs = [tensor(C.draw(co.replace(cid=co.cid + i), "z", nthreads=threads), cfg.bf16) for i in range(2)]
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, True, xbc=True)
    prm = m.make_params(g.A, g.D, g.dt_bias, cw, None)
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    trees = (g, g2)
    k = [0]

    def step():
        prev, nxt = trees[k[0] % 2], trees[(k[0] + 1) % 2]
        m.commit_verify(dims, prm, prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, win, state,
                        win, state, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, y, cst, vst, C_prev=prev.C,
                        z=zs[(k[0] + 1) % 2])
        k[0] += 1

    for _ in range(WARM_EXTRA):  # a fresh workload's ramp to its steady rate, as for the step
        step()
    ms = timed(step, reps=9)
    torch.cuda.synchronize()
    if not (cst.cpu() == 0).all() or not (vst.cpu() == 0).all() or torch.isnan(y).any():
        raise SystemExit("bench: the option round produced a bad status or NaN")
    e = cfg.e
    gn = cfg.G * cfg.N
    plain = [algorithmic_bytes(cfg, pl)["commit_verify"] for pl in path_lens]
    acc = [int(sum(int(n) for n in pl)) for pl in path_lens]
    # extra: the window's B and C rows read and written, the gate input, and
    # the C row of every accepted node
    extra = [cfg.L * (cfg.Bsz * (2 * (cfg.W - 1) * 2 * gn * e + cfg.T * cfg.d_in * e) + a * gn * e) for a in acc]
    nbytes = (sum(plain) + sum(extra)) // 2
    avg = sum(ms) / len(ms)
    ach = nbytes / (avg * 1e-3) / 1e9
    return {"options": "SiLU over the conv of x, B and C; y * silu(z)", "ms": round(avg, 4),
            "ms_min": round(min(ms), 4), "bytes": nbytes, "GBps": round(ach, 1),
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "node_layers_per_s": round(cfg.L * cfg.Bsz * cfg.T / (avg * 1e-3), 1), "note": "not in the step"}


def state_bf16_round(torch, m, cfg, g, g2, state, window, timed, path_lens):
    """The same decode round with the root state stored as bfloat16
    (SSM_TREE_STATE_BF16): the bench's state rounded to bf16, committed and
    verified in place.  Not part of the step; reported apart."""
    sb = state.to(torch.bfloat16)
    win = None if window is None else window.clone()
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu,
                       state_bf16=True)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    trees = (g, g2)
    k = [0]

    def step():
        prev, nxt = trees[k[0] % 2], trees[(k[0] + 1) % 2]
        m.commit_verify(dims, prm, prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, win, sb,
                        win, sb, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, y, cst, vst)
        k[0] += 1

    try:
        for _ in range(WARM_EXTRA):
            step()
        ms = timed(step, reps=9)
    except m.SsmTreeError as e:  # shapes no kernel takes with a bf16 state
        return {"skipped": str(e)}
    torch.cuda.synchronize()
    if not (cst.cpu() == 0).all() or not (vst.cpu() == 0).all() or torch.isnan(y).any():
        raise SystemExit("bench: the bf16-state round produced a bad status or NaN")
    # the root state is read and written once per round, 2 bytes per element instead of 4
    half = cfg.L * cfg.Bsz * cfg.H * cfg.P * cfg.N * 2
    nbytes = sum(algorithmic_bytes(cfg, pl)["commit_verify"] for pl in path_lens) // len(path_lens) - 2 * half
    avg = sum(ms) / len(ms)
    ach = nbytes / (avg * 1e-3) / 1e9
    out = {"state": "bf16 (rounded to nearest even on store)", "ms": round(avg, 4), "ms_min": round(min(ms), 4),
           "bytes": nbytes, "GBps": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4),
           "node_layers_per_s": round(cfg.L * cfg.Bsz * cfg.T / (avg * 1e-3), 1), "note": "not in the step"}
    # the two calls apart (verify reads the state once, commit reads and writes it)
    ab = algorithmic_bytes(cfg, path_lens[0])
    vms = timed(lambda: m.verify(dims, prm, g.parent, g.x, g.B, g.C, g.dt_raw, win, sb, y, vst))
    cms = timed(lambda: m.commit(dims, prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, win, sb, win, sb, cst))
    for name, v, nb in (("verify", vms, ab["verify"] - half), ("commit", cms, ab["commit"] - 2 * half)):
        a = sum(v) / len(v)
        out[name] = {"ms": round(a, 4), "bytes": nb, "GBps": round(nb / (a * 1e-3) / 1e9, 1),
                     "frac": round(nb / (a * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


PROBE_KINDS = {0: "read", 1: "copy", 2: "read+1/8 write"}
PROBE_LAYOUTS = {0: "coalesced", 1: "mfma"}


def load_probe():
    """libssm_tree_probe.so: hand-written streaming kernels in the root
    state's tiles and access patterns (csrc/probe.hip)."""
    import ctypes
    from mamba2_tree_verification_amd import build as hb
    if not os.path.exists(hb.PROBE_LIB):
        raise SystemExit("libssm_tree_probe.so is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(hb.PROBE_LIB)
    p, i = ctypes.c_void_p, ctypes.c_int
    L.ssm_probe_stream.argtypes = [i, i, i, i, p, p, ctypes.c_int64, p, p]
    L.ssm_probe_stream.restype = i
    L.ssm_probe_dst_bytes.argtypes = [i, ctypes.c_int64]
    L.ssm_probe_dst_bytes.restype = ctypes.c_int64
    return L


def hbm_probe(torch, nbytes=PROBE_BYTES, reps=8, variants=None):
    """Bandwidth of the hand-written probe kernels over a buffer far larger
    than the 256 MB last-level cache: read only, copy, and read with one
    row written per eight read, in the coalesced and the matrix-core
    operand layouts, plain and non-temporal, one workgroup per 32 KiB tile
    or a persistent grid of 4 workgroups per CU.  Bytes moved per launch
    over the HIP-event time of the launch."""
    L = load_probe()
    tiles = nbytes // (64 * 512)
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty(L.ssm_probe_dst_bytes(1, tiles) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if variants is None:  # nt: bit 0 non-temporal loads, bit 1 non-temporal stores
        variants = [(k, lay, nt, grid) for k in (0, 1, 2) for lay in (0, 1) for nt in ((0, 1) if k == 0 else (0, 1, 2, 3))
                    for grid in (0, 4 * cus)]
    hs = torch.cuda.current_stream().cuda_stream
    out = []
    for kind, lay, nt, grid in variants:
        def run():
            rc = L.ssm_probe_stream(kind, lay, nt, grid, src.data_ptr(), dst.data_ptr(), tiles, sink.data_ptr(), hs)
            if rc:
                raise SystemExit("probe launch failed: %d" % rc)
        run()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        moved = nbytes + L.ssm_probe_dst_bytes(kind, tiles)
        a = sum(ms) / len(ms)
        out.append({"kind": PROBE_KINDS[kind], "layout": PROBE_LAYOUTS[lay],
                    "nt": ("loads " if nt & 1 else "") + ("stores" if nt & 2 else "") or "none",
                    "grid": "per tile" if grid == 0 else "persistent %d" % grid, "bytes": moved,
                    "ms": round(a, 4), "GBps": round(moved / (a * 1e-3) / 1e9, 1)})
    del src, dst
    torch.cuda.empty_cache()
    best = {}
    for r in out:
        if r["GBps"] > best.get(r["kind"], {}).get("GBps", 0):
            best[r["kind"]] = r
    return {"probe": "hbm", "buffer_bytes": nbytes, "variants": out,
            "best": {k: {"GBps": v["GBps"], "frac": round(v["GBps"] / HBM_PEAK_GBS, 4),
                         "variant": "%s %s, non-temporal %s, %s" % (v["layout"], k, v["nt"], v["grid"])}
                     for k, v in best.items()}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=3, help="workload id (3 = Mamba2-2.7B batch 16 x tree 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-layer, draft and option rounds (their dispatches share the step kernel's "
                         "name; profiler runs of the step use this)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR and exit")
    ap.add_argument("--probe", action="store_true",
                    help="only run the hand-written HBM probe kernels (practical ceilings) and exit")
    ap.add_argument("--copy-only", action="store_true",
                    help="with --probe: only the coalesced plain copy probe (the counter scale of --record-traffic)")
    args = ap.parse_args(argv)

    if args.record_traffic:
        from testgen import configs as C
        return record_traffic(args.record_traffic, C.CONFIGS[args.config])
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
        print(json.dumps(hbm_probe(torch, variants=[(1, 0, 0, 0)] if args.copy_only else None)), flush=True)
        return 0
    m.load()
    cfg = C.CONFIGS[args.config]
    t_gen = time.perf_counter()
    inp = C.make_inputs(cfg, nthreads=args.threads)
    g = upload(inp)
    # a second tree per sequence (own nodes and accepted path, same layers)
    inp2 = C.make_inputs(cfg.replace(cid=cfg.cid + 500), nthreads=args.threads,
                         skip=("state", "window", "A", "D", "dt_bias", "conv_w", "conv_b"))
    g2 = upload(inp2)
    t_gen = time.perf_counter() - t_gen
    dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    st_v = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    st_c = torch.empty(cfg.Bsz, dtype=torch.int32, device="cuda")
    state = g.state  # committed in place, step after step
    window = g.window
    trees = (g, g2)

    def step(k, ev=None):
        prev, nxt = trees[k % 2], trees[(k + 1) % 2]
        if ev is not None:
            ev[0].record()
        m.commit_verify(dims, prm, prev.parent, prev.path, prev.path_len, prev.x, prev.B, prev.dt_raw, window, state,
                        window, state, nxt.parent, nxt.x, nxt.B, nxt.C, nxt.dt_raw, y, st_c, st_v)
        if ev is not None:
            ev[1].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # (the statuses are checked after the timed steps: with the process's
    # first device-to-host copy just before them, the timed steps of a first
    # run on a box measured 3-5% slower, with slow steps throughout)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cv_ms = [e[0].elapsed_time(e[1]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    # the round's statuses and NaN check stay on the device (stream order)
    # until the separate calls below have been timed too
    round_st = torch.stack([st_v, st_c])
    round_nan = torch.isnan(y).any()

    # not part of the step, timed apart for comparison: the same round as two
    # calls (verify from the state, then the in-place commit), and the page's
    # own form of verification (explicit FIFO walk, every child state
    # materialised)
    def timed(fn, reps=5, warm=0):
        for _ in range(warm):  # the ramp of a call not yet run in this process
            fn()
        out = []
        for k in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if k:
                out.append(e0.elapsed_time(e1))
        return out

    ver_ms = timed(lambda: m.verify(dims, prm, g.parent, g.x, g.B, g.C, g.dt_raw, window, state, y, st_v), reps=11,
                   warm=WARM_EXTRA // 2)
    com_ms = timed(lambda: m.commit(dims, prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, window, state,
                                    window, state, st_c), reps=11, warm=WARM_EXTRA // 2)
    dims_fifo = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, fifo=True)
    fifo_ms = timed(lambda: m.verify(dims_fifo, prm, g.parent, g.x, g.B, g.C, g.dt_raw, window, state, y, st_v),
                    reps=3)

    if not (round_st.cpu() == 0).all():
        print("bench: nonzero sequence status", file=sys.stderr)
        return 1
    if bool(round_nan):
        print("bench: NaN in y", file=sys.stderr)
        return 1

    per_layer = draft = opts = sbf = ceiling = stress = None
    small = {}
    if not args.no_extras:
        # practical ceilings of the same GPU, by the hand-written probes
        ceiling = hbm_probe(torch, nbytes=2 << 30, reps=4,
                            variants=[(0, 0, 1, 0), (0, 1, 0, 0), (1, 0, 0, 0), (1, 0, 1, 0), (1, 1, 0, 0),
                                      (2, 0, 1, 0), (2, 1, 0, 0)])
        for cid in (1, 2):
            small[C.CONFIGS[cid].name] = rotated_rates(torch, m, C, cid, args.threads)
        if args.config != 4:
            stress = stress_workload(torch, m, C, args.threads)
        sbf = state_bf16_round(torch, m, cfg, g, g2, state, window, timed, (inp.path_len, inp2.path_len))
        per_layer = per_layer_round(torch, m, cfg, g, g2, state, window, y, st_c, st_v, timed)
        draft = draft_decode(torch, m, C, upload, args.threads, timed)
        if 1 <= cfg.T <= 16 and cfg.P % 16 == 0:  # the shapes the options run on
            opts = options_round(torch, m, C, cfg, g, g2, state, timed, args.threads, (inp.path_len, inp2.path_len))

    ab = algorithmic_bytes(cfg, inp.path_len)
    ab2 = algorithmic_bytes(cfg, inp2.path_len)
    # the step alternates which tree's path is committed: average the two
    cvb = (ab["commit_verify"] + ab2["commit_verify"]) // 2
    node_layers = cfg.L * cfg.Bsz * cfg.T

    def avg(v):
        return sum(v) / len(v)

    def roof(kernel, nbytes, ms):
        ach = nbytes / (ms * 1e-3) / 1e9
        tr = load_traffic(kernel, cfg)
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr}

    # verify's arithmetic: C . h0 is 2 T flops per root-state element (the
    # path terms are O(T^2) per channel and left out).  Trees of at most 16
    # nodes: fp32 matrix-core products (157.3 TFLOP/s); 17-64 nodes with bf16
    # inputs: bf16 products against the state split into three bf16 terms,
    # counted as executed (3 x, nodes padded to 16-node tiles) against the
    # bf16 peak (2500 TFLOP/s); other shapes: vector ALU without packed fp32
    # (78.6 TFLOP/s = 256 CUs x 64 FMA lanes x 2 x 2.4 GHz)
    vsrc = os.path.basename(verify_source(cfg))
    vflops = 2 * cfg.L * cfg.Bsz * cfg.T * cfg.H * cfg.P * cfg.N
    if vsrc == "verify_tt.hip" and cfg.bf16:
        engine, vpeak = "mfma bf16 (state split in 3 bf16 terms)", 2500.0
        xflops = 3 * 2 * cfg.L * cfg.Bsz * (16 * ((cfg.T + 15) // 16)) * cfg.H * cfg.P * cfg.N
    elif vsrc in ("verify_tt.hip", "commit_verify.hip"):
        engine, vpeak, xflops = "mfma fp32", 157.3, vflops
    else:
        engine, vpeak, xflops = "valu fp32", 78.6, vflops
    vach = xflops / (avg(ver_ms) * 1e-3) / 1e12
    # the FIFO walk forms every child state: per (state element, node) the
    # update dA h_parent + (dt x~) B (a multiply and a fused multiply-add)
    # and the term of C . h (a fused multiply-add), 5 flop, on the vector ALU
    # without packed fp32 (78.6 TFLOP/s)
    fflops = 5 * cfg.L * cfg.Bsz * cfg.T * cfg.H * cfg.P * cfg.N
    fach = fflops / (avg(fifo_ms) * 1e-3) / 1e12
    fcompute = {"engine": "valu fp32", "flops": fflops, "achieved": round(fach, 2), "peak": 78.6,
                "unit": "TFLOP/s", "frac": round(fach / 78.6, 4)}
    vcompute = {"engine": engine, "flops": xflops, "achieved": round(vach, 2),
                "peak": vpeak, "unit": "TFLOP/s", "frac": round(vach / vpeak, 4)}

    kern = {"commit_verify": dict(ms=round(avg(cv_ms), 4), ms_min=round(min(cv_ms), 4),
                                  ms_median=round(sorted(cv_ms)[len(cv_ms) // 2], 4),
                                  ms_max=round(max(cv_ms), 4), bytes=cvb,
                                  node_layers_per_s=round(node_layers / (avg(cv_ms) * 1e-3), 1),
                                  roofline=roof("commit_verify", cvb, avg(cv_ms))),
            "verify": dict(ms=round(avg(ver_ms), 4), ms_min=round(min(ver_ms), 4), bytes=ab["verify"],
                           node_layers_per_s=round(node_layers / (avg(ver_ms) * 1e-3), 1),
                           roofline=roof("verify", ab["verify"], avg(ver_ms)), compute=vcompute,
                           note="not in the step"),
            "commit": dict(ms=round(avg(com_ms), 4), ms_min=round(min(com_ms), 4), bytes=ab["commit"],
                           roofline=roof("commit", ab["commit"], avg(com_ms)), note="not in the step"),
            "verify_fifo_walk": dict(ms=round(avg(fifo_ms), 4), bytes=ab["verify"],
                                     roofline=roof("verify_fifo", ab["verify"], avg(fifo_ms)), compute=fcompute,
                                     note="SSM_TREE_VERIFY_FIFO: the page's breadth-first walk with a FIFO of "
                                          "live states, every child state formed on the vector ALU; not in the "
                                          "step")}
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
                   "step": "ssm_tree_commit_verify: in-place commit of the previous tree's accepted path, "
                           "verify of the next tree", "parallelism": "single-gpu"},
        "roofline": dict(kern["commit_verify"]["roofline"], kernel="commit_verify"),
        "kernels": kern,
        "two_call_step_ms": round(avg(ver_ms) + avg(com_ms), 4),
        "per_layer": per_layer,
        "draft_decode": draft,
        "options_round": opts,
        "state_bf16_round": sbf,
        "small_workloads": small or None,
        "stress_workload": stress,
        "ceiling": ceiling,
        "param_bytes_per_call": ab["params"],
        "verify_hbm_frac": kern["verify"]["roofline"]["frac"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds, args.threads,
                                           per_core_cfg=C.CONFIGS[2])
    rec["setup_s"] = round(t_gen, 1)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
