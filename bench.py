"""Throughput of the SchNet CFConv energy + force path on one MI355X.

A step is one pass of the whole hot path over one batch: the Langevin (BAOAB)
update of every replica, a neighbour-list rebuild (receiver-sorted CSR), the
fused CFConv energy evaluation, and the analytic backward for the forces.
The workload is 64 replicas of a 269-bead coarse-grained chain (D 128,
50 Gaussians on 0-12 A, cosine cutoff 12 A, 3 interaction blocks, fp32), with
synthetic seeded positions and random-init weights. The list is rebuilt every
step at the cutoff radius, so every listed edge contributes.

Prints one JSON line: directed edges through energy+forces per second (value),
replica-steps per second, the roofline of the dominant kernel (backward
CFConv, timed with HIP events around every launch inside the timed region)
and the fp64 oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from schnet_continuous_filter_amd import profiling  # noqa: E402  (no GPU work at import)

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PREC_TAGS = {0: "f32", 1: "bf16", 2: "w16a16", 3: "f16x2"}
DTYPE_TAGS = {0: "f32", 1: "bf16-filter/f16x2-atomwise/f32", 2: "f16-mlps/f32", 3: "f16x2-filter/f32"}
PROFILES = os.path.join(ROOT, "profiles")


def bwd_traffic(workload, m):
    """Counter-measured bytes per k_cf_bwd launch for this workload and filter
    precision (profiles/cfconv_bwd_<workload>[_f16x2]_counters.txt), or None
    when no such record exists or the kernels changed since it was taken."""
    for name in (f"cfconv_bwd_{workload}_counters.txt", f"cfconv_bwd_{workload}_f16x2_counters.txt"):
        path = os.path.join(PROFILES, name)
        if not os.path.exists(path):
            continue
        rec = json.load(open(path))
        kern = rec.get("kernel", "")   # "void sn::k_cf_bwd<D, KP, precision>(sn::CfParams)"
        if (rec.get("kernel_hash") == profiling.kernel_hash() and kern.startswith(f"void sn::k_cf_bwd<{m.D}, ")
                and f", {m.filter_dtype}>(" in kern and rec.get("workload", "").split("_")[0] == workload):
            return rec.get("bytes_per_launch")
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cg269x64",
                    choices=["cg269x64", "cg32", "bulk4k", "bulk64k", "md1024"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--precision", choices=["f32", "bf16", "w16a16", "f16x2"], default=None,
                    help="override the workload's network operand precision")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-alt", action="store_true",
                    help="fp32 workloads: skip the extra timing with the filter on fp16 pairs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device copy of known size (for counter scaling)")
    ap.add_argument("--sweep-replicas", default="",
                    help="comma-separated replica counts: MD throughput and memory of the "
                         "269-bead chain model (bf16 filter, 1 A skin, rebuild every 10) per count")
    ap.add_argument("--topology", default="",
                    help="comma-separated compaction factors: energy+force time of the fused and "
                         "unfused pipelines on 64 chains rescaled about their centroids")
    ap.add_argument("--ablation", action="store_true",
                    help="time one energy+force evaluation on a prebuilt list: fused vs the "
                         "unfused pipeline (segment sums, atomic scatter), fp32 vs bf16 filters")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 256 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 5}))


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands, on a bounded sample of the same workload:
    8 replicas, MD steps (rebuild + energy/forces + BAOAB) until the budget."""
    import numpy as np
    import oracle
    from gen.configs import make_config
    from threadpoolctl import threadpool_info

    R = 8
    c, pos, types, w = make_config(cfg.name, n_replicas=R)
    m = c.model
    desc = oracle.ModelDesc(m.n_types, m.D, m.Dr, m.T, m.rbf_min, m.rbf_max, m.r_cut, m.H,
                            m.filter_dtype)
    W = oracle.unpack_weights(desc, w)
    N = c.system.atoms_per_replica
    per = c.system.periodic
    box = c.system.box
    state = {}

    def rebuild(p):
        state["nl"] = oracle.neighbor_list(np.asarray(p, np.float32), R, N, per, box, m.r_cut)

    def forces(p):
        return oracle.energy_forces(desc, None, p, types, *state["nl"], n_replicas=R,
                                    periodic=per, box=box, weights=W)

    rebuild(pos)
    E0, F0 = forces(pos.astype(np.float64))
    vel = oracle.init_velocities(0, len(pos), 300.0, 100.0)
    p, v, F = pos.astype(np.float64), vel, F0
    steps, edges = 0, 0
    t0 = time.perf_counter()
    while True:
        p, v, F, E, _ = oracle.baoab_run(forces, rebuild, p, v, F, dt_fs=2.0, temperature_K=300.0,
                                         gamma_per_ps=1.0, mass_amu=100.0, skin=0.0,
                                         rebuild_every=1, seed=0, step0=steps, n_steps=1,
                                         periodic=per, box=box)
        steps += 1
        edges += len(state["nl"][1])
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": edges / dt, "unit": "edges/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{R} of {c.system.n_replicas} replicas x {N} beads, {steps} MD steps "
                      f"(rebuild + fp64 energy/forces + BAOAB) in {dt:.1f} s; "
                      f"{R * steps / dt:.3g} replica-steps/s",
            "replica_steps_per_s": R * steps / dt}


def ablation(args):
    """The switches FlashSchNet ablates (fusion, segmented reduction, 16-bit
    filters; §4.5 "End-to-end integration") on one MI355X: one energy+force
    evaluation on a prebuilt list, per variant, with the workspace it needs."""
    import numpy as np
    import torch
    from gen.configs import CONFIGS, make_config
    from schnet_continuous_filter_amd import _lib as L

    cfg = CONFIGS[args.workload]
    c, pos, types, w = make_config(cfg.name)
    m, s = c.model, c.system
    R, N = s.n_replicas, s.atoms_per_replica
    system = L.make_system(R, N, s.periodic, s.box)
    dev = torch.device("cuda")
    p = torch.from_numpy(pos).to(dev).reshape(-1)
    t = torch.from_numpy(types).to(dev)
    n = R * N
    ws_nbr = L.Workspace(L.sn_workspace_size(None, system))
    rowptr = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    ne = L.sn_build_neighbors(system, p, m.r_cut, rowptr, None, 0, ws_nbr)
    col = torch.empty(max(ne, 1), dtype=torch.int32, device=dev)
    L.sn_reset_device_status(ws_nbr)
    L.sn_build_neighbors(system, p, m.r_cut, rowptr, col, ne, ws_nbr)
    energy = torch.empty(R, dtype=torch.float32, device=dev)
    forces = torch.empty(3 * n, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    variants = {}
    energies = {}
    dtypes = [m.filter_dtype] + [fd for fd in (0, 1, 2, 3) if fd != m.filter_dtype]
    for fd in dtypes:
        tag = PREC_TAGS[fd]
        desc = L.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut, fd)
        model = L.sn_model_create(desc, w)
        runs = [("fused", L.sn_workspace_size(desc, system), None)]
        if fd == m.filter_dtype and fd in (0, 1):
            ub = L.sn_unfused_workspace_size(desc, system, ne)
            runs += [("unfused_segmented", ub, 0), ("unfused_atomic", ub, L.SN_UNFUSED_ATOMIC)]
        for name, nbytes, flags in runs:
            ws = L.Workspace(nbytes)
            if flags is None:
                fn = lambda: L.sn_energy_forces(model, system, p, t, rowptr, col, energy, forces,
                                                ws)
            else:
                fn = lambda: L.sn_energy_forces_unfused(model, system, p, t, rowptr, col, ne,
                                                        flags, energy, forces, ws)
            ms = timed(fn)
            st = L.sn_get_device_status(ws)
            if st[0] != 0:
                print(f"{name} {tag}: device status {st}", file=sys.stderr)
                sys.exit(1)
            key = f"{name}_{tag}"
            variants[key] = {"ms": ms, "edges_per_s": ne / (ms * 1e-3),
                             "workspace_bytes": nbytes}
            energies[key] = energy.double().cpu().numpy().copy()
            del ws
            torch.cuda.empty_cache()
        L.sn_model_destroy(model)
    base = f"_{PREC_TAGS[m.filter_dtype]}"
    ref = energies["fused" + base]
    for k, e in energies.items():
        variants[k]["energy_rel_diff_vs_fused"] = float(np.max(np.abs(e - ref) / np.abs(ref)))
    ms = {k: v["ms"] for k, v in variants.items()}
    line = {
        "metric": "energy+force evaluation time per variant (same GPU, prebuilt list)",
        "unit": "ms",
        "higher_is_better": False,
        "config": {"workload": cfg.name, "replicas": R, "atoms_per_replica": N,
                   "directed_edges": ne, "D": m.D, "Dr": m.Dr, "T": m.T,
                   "filter": PREC_TAGS[m.filter_dtype]},
        "steps": args.steps, "warmup": args.warmup,
        "variants": variants,
        "speedup": {
            "segmented_vs_atomic (unfused)": ms["unfused_atomic" + base] / ms["unfused_segmented" + base],
            "fusion (fused vs unfused, segmented)": ms["unfused_segmented" + base] / ms["fused" + base],
            "fused vs unfused_atomic": ms["unfused_atomic" + base] / ms["fused" + base],
            "bf16 vs f32 filter (fused)": ms["fused_f32"] / ms["fused_bf16"],
            "w16a16 vs f32 (fused)": ms["fused_f32"] / ms["fused_w16a16"],
            "f16x2 vs f32 (fused)": ms["fused_f32"] / ms["fused_f16x2"],
        },
    }
    print(json.dumps(line))


def sweep_replicas(args):
    """Replica-count scaling (§5.2 "Memory reduction enables better
    scalability", Figure 7): MD replica-steps/s and device memory per count,
    with the workspace the unfused pipeline would need for the same list."""
    import torch
    from gen.configs import make_config
    from schnet_continuous_filter_amd import _lib as L

    rows = []
    for R in [int(v) for v in args.sweep_replicas.split(",")]:
        c, pos, types, w = make_config("md1024", n_replicas=R)
        m, s, md = c.model, c.system, c.md
        N = s.atoms_per_replica
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        desc = L.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut,
                           m.filter_dtype)
        system = L.make_system(R, N, s.periodic, s.box)
        model = L.sn_model_create(desc, w)
        wsb = L.sn_workspace_size(desc, system)
        ws = L.Workspace(wsb)
        p = torch.from_numpy(pos).cuda().reshape(-1)
        t = torch.from_numpy(types).cuda()
        prm = L.make_md_params(md.dt_fs, md.temperature_K, md.gamma_per_ps, md.mass_amu, md.skin,
                               md.rebuild_every, 0)
        rowptr0 = torch.zeros(R * N + 1, dtype=torch.int32, device="cuda")
        ne0 = L.sn_build_neighbors(system, p, m.r_cut + md.skin, rowptr0, None, 0, ws)
        L.sn_reset_device_status(ws)
        cap = int(ne0 * 1.5) + 1024
        state = L.MdState(p, cap)
        energy = torch.empty(R, dtype=torch.float32, device="cuda")
        L.sn_md_init(model, system, t, prm, state, energy, ws)
        L.sn_md_step(model, system, t, prm, state, args.warmup, energy, ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        L.sn_md_step(model, system, t, prm, state, args.steps, energy, ws)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st = L.sn_get_device_status(ws)
        if st[0] != 0:
            print(f"R={R}: device status {st}", file=sys.stderr)
            sys.exit(1)
        rows.append({"replicas": R, "edges_at_start": ne0, "ms_per_step": 1000 * dt / args.steps,
                     "replica_steps_per_s": R * args.steps / dt,
                     "peak_device_bytes": torch.cuda.max_memory_allocated(),
                     "workspace_bytes": wsb,
                     "unfused_workspace_bytes": L.sn_unfused_workspace_size(desc, system, cap)})
        del state, ws
        L.sn_model_destroy(model)
    print(json.dumps({"metric": "replica-steps/s vs replica count (269-bead chain, bf16 filter)",
                      "unit": "replica-steps/s", "higher_is_better": True, "steps": args.steps,
                      "warmup": args.warmup, "rows": rows}))


def topology(args):
    """Dynamic-topology robustness (§5.2 "Robustness to dynamic graph
    topology", Figures 5 and 6): the same 64 chains rescaled about their
    centroids, so that the edge count and the share of long-range
    (sequence-distant) contacts change; one energy+force evaluation per
    pipeline on each list."""
    import numpy as np
    import torch
    from gen.configs import make_config
    from gen.systems import rescale_replicas
    from schnet_continuous_filter_amd import _lib as L

    c, pos0, types, w = make_config("cg269x64")
    m, s = c.model, c.system
    R, N = s.n_replicas, s.atoms_per_replica
    n = R * N
    system = L.make_system(R, N, s.periodic, s.box)
    desc = L.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut,
                       m.filter_dtype)
    model = L.sn_model_create(desc, w)
    t = torch.from_numpy(types).cuda()
    energy = torch.empty(R, dtype=torch.float32, device="cuda")
    forces = torch.empty(3 * n, dtype=torch.float32, device="cuda")
    rows = []
    for f in [float(v) for v in args.topology.split(",")]:
        p = torch.from_numpy(rescale_replicas(pos0, N, f)).cuda().reshape(-1)
        ws_nbr = L.Workspace(L.sn_workspace_size(desc, system))
        rowptr = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
        ne = L.sn_build_neighbors(system, p, m.r_cut, rowptr, None, 0, ws_nbr)
        col = torch.empty(max(ne, 1), dtype=torch.int32, device="cuda")
        L.sn_reset_device_status(ws_nbr)
        L.sn_build_neighbors(system, p, m.r_cut, rowptr, col, ne, ws_nbr)
        rp = rowptr.cpu().numpy()
        cl = col[:ne].cpu().numpy()
        recv = np.repeat(np.arange(n), np.diff(rp))
        long_range = float(np.mean(np.abs(recv - cl) > 16)) if ne else 0.0
        row = {"factor": f, "edges": ne, "edges_per_bead": ne / n,
               "max_row": int(np.diff(rp).max()), "share_seq_sep_gt16": long_range}
        uws = L.Workspace(L.sn_unfused_workspace_size(desc, system, ne))
        for name, fn in (
                ("fused", lambda: L.sn_energy_forces(model, system, p, t, rowptr, col, energy,
                                                     forces, ws_nbr)),
                ("unfused_segmented", lambda: L.sn_energy_forces_unfused(
                    model, system, p, t, rowptr, col, ne, 0, energy, forces, uws)),
                ("unfused_atomic", lambda: L.sn_energy_forces_unfused(
                    model, system, p, t, rowptr, col, ne, L.SN_UNFUSED_ATOMIC, energy, forces,
                    uws))):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.steps
            row[name] = {"ms": ms, "edges_per_s": ne / (ms * 1e-3)}
        for wsx in (ws_nbr, uws):
            st = L.sn_get_device_status(wsx)
            if st[0] != 0:
                print(f"factor {f}: device status {st}", file=sys.stderr)
                sys.exit(1)
        rows.append(row)
        del uws
        torch.cuda.empty_cache()
    L.sn_model_destroy(model)
    print(json.dumps({"metric": "energy+force edges/s vs conformation (64 x 269-bead chains)",
                      "unit": "edges/s", "higher_is_better": True, "steps": args.steps,
                      "warmup": args.warmup, "rows": rows}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch  # noqa: F401  (initialises the device before any library call)
    if args.ablation:
        ablation(args)
        return
    if args.sweep_replicas:
        sweep_replicas(args)
        return
    if args.topology:
        topology(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    from gen.configs import CONFIGS, make_config

    cfg = CONFIGS[args.workload]
    c, pos, types, w = make_config(cfg.name)
    m = c.model
    if args.precision is not None:
        import dataclasses
        m = dataclasses.replace(m, filter_dtype={v: k for k, v in PREC_TAGS.items()}[args.precision])
    r = md_timing(cfg, c, m, pos, types, w, args.steps, args.warmup)
    R = c.system.n_replicas
    flops_bwd = 4.0 * m.D * (m.Dr + m.D) * r["ne"]    # recompute (2D(Dr+D)) + dgrad (2D(Dr+D))
    avg_bwd_s = r["bwd_ms"] / 1000.0 / max(r["bwd_n"], 1)
    achieved = flops_bwd / avg_bwd_s / 1e12
    half = m.filter_dtype != 0          # 16-bit operands: the dense fp16/bf16 MFMA peak
    peak = PEAK_BF16_MFMA_TFLOPS if half else PEAK_FP32_MFMA_TFLOPS
    traffic = bwd_traffic(cfg.name, m)
    line = {
        "metric": "CFConv energy+force edges/sec and replica-MD-steps/sec at 1 GPU; % HBM roofline",
        "value": r["edges_per_s"],
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAGS[m.filter_dtype],
        "data": "synthetic (seeded chains/boxes, random-init weights)",
        "config": {"workload": cfg.name, "replicas": R,
                   "atoms_per_replica": c.system.atoms_per_replica,
                   "directed_edges": r["ne"], "list_radius_A": r["r_list"],
                   "list_edges": r["ne_list"], "D": m.D, "Dr": m.Dr,
                   "T": m.T, "r_cut_A": m.r_cut,
                   "step": "BAOAB + neighbour rebuild + energy/forces"},
        "replica_steps_per_s": r["replica_steps_per_s"],
        "roofline": {"kernel": "k_cf_bwd (fused CFConv backward, one interaction block)",
                     "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "flops_per_launch": flops_bwd, "avg_launch_us": avg_bwd_s * 1e6,
                     "launches": r["bwd_n"],
                     "fwd_avg_launch_us": r["fwd_ms"] * 1000.0 / max(r["fwd_n"], 1)},
        "n_rebuilds": r["n_rebuilds"],
    }
    if m.filter_dtype == 0 and args.precision is None and not args.no_alt:
        # the same fp32 model with the filter products on fp16 pairs (held to
        # the fp32 parity bars), timed the same way
        import dataclasses
        m2 = dataclasses.replace(m, filter_dtype=3)
        r2 = md_timing(cfg, c, m2, pos, types, w, args.steps, args.warmup)
        line["f16x2_filter"] = {
            "value": r2["edges_per_s"], "unit": "edges/s", "ms_per_step": r2["ms_per_step"],
            "replica_steps_per_s": r2["replica_steps_per_s"], "dtype": DTYPE_TAGS[3],
            "bwd_avg_launch_us": r2["bwd_ms"] * 1000.0 / max(r2["bwd_n"], 1),
            "fwd_avg_launch_us": r2["fwd_ms"] * 1000.0 / max(r2["fwd_n"], 1),
            # counter-measured bytes per backward launch of this path (or None)
            "bwd_traffic": bwd_traffic(cfg.name, m2),
            "parity": "fp32 bars (energy 1e-5 relative, forces 1e-4 of the force RMS)"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line))


def md_timing(cfg, c, m, pos, types, w, steps, warmup):
    """MD steps of one model on the workload: warm-up, then `steps` timed
    steps with the CFConv kernels' launch times recorded by the library."""
    import torch
    from schnet_continuous_filter_amd import _lib as L
    s = c.system
    R, N = s.n_replicas, s.atoms_per_replica
    desc = L.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut,
                       m.filter_dtype)
    system = L.make_system(R, N, s.periodic, s.box)
    model = L.sn_model_create(desc, w)
    ws = L.Workspace(L.sn_workspace_size(desc, system))
    dev = torch.device("cuda")
    p = torch.from_numpy(pos).to(dev).reshape(-1)
    t = torch.from_numpy(types).to(dev)
    if c.md is not None:          # the MD workload keeps its own skin and cadence
        md = L.make_md_params(c.md.dt_fs, c.md.temperature_K, c.md.gamma_per_ps, c.md.mass_amu,
                              c.md.skin, c.md.rebuild_every, 0)
        r_list = m.r_cut + c.md.skin
    else:                         # rebuild every step at the cutoff
        md = L.make_md_params(2.0, 300.0, 1.0, 100.0, 0.0, 1, 0)
        r_list = m.r_cut
    rowptr0 = torch.zeros(R * N + 1, dtype=torch.int32, device=dev)
    ne0 = L.sn_build_neighbors(system, p, r_list, rowptr0, None, 0, ws)
    L.sn_reset_device_status(ws)
    capacity = int(ne0 * 1.5) + 1024
    state = L.MdState(p, capacity)
    energy = torch.empty(R, dtype=torch.float32, device=dev)
    L.sn_md_init(model, system, t, md, state, energy, ws)
    L.sn_md_step(model, system, t, md, state, warmup, energy, ws)
    torch.cuda.synchronize()
    L.sn_profile_read(0)
    L.sn_profile_read(1)

    L.sn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    L.sn_md_step(model, system, t, md, state, steps, energy, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    L.sn_profile_enable(False)
    bwd_ms, bwd_n = L.sn_profile_read(1)
    fwd_ms, fwd_n = L.sn_profile_read(0)
    status, detail, n_rebuilds = L.sn_get_device_status(ws)
    if status != 0:
        print(f"device status {status} ({L.status_string(status)}), detail {detail}",
              file=sys.stderr)
        sys.exit(1)
    # edge counts on the final positions (untimed): the pairs inside the
    # cutoff are the work (the MD evaluates only those); the list's own size
    ne_list = L.sn_build_neighbors(system, state.pos, r_list, state.rowptr, state.col, capacity,
                                   ws)
    ne = L.sn_build_neighbors(system, state.pos, m.r_cut, state.rowptr, state.col, capacity, ws)
    L.sn_model_destroy(model)
    return {"edges_per_s": ne * steps / elapsed, "ms_per_step": 1000.0 * elapsed / steps,
            "replica_steps_per_s": R * steps / elapsed, "ne": ne, "ne_list": ne_list,
            "r_list": r_list,
            "bwd_ms": bwd_ms, "bwd_n": bwd_n, "fwd_ms": fwd_ms, "fwd_n": fwd_n,
            "n_rebuilds": n_rebuilds}


if __name__ == "__main__":
    main()
