"""Throughput of the SchNet CFConv energy + force path on one MI355X.

Headline (no flags): the 1024-replica MD workload. A step is one pass of the
whole hot path over the batch: the Langevin (BAOAB) update of every bead, the
neighbour-list rebuild every 10 steps at r_cut + 1 A (and on the skin guard),
the per-step active list, the fused CFConv energy evaluation and the analytic
backward for the forces. 1024 replicas of a 269-bead chain, D 128, 50
Gaussians on 0-12 A, cosine cutoff 12 A, 3 interaction blocks, bf16 filter
network with fp32 accumulation; synthetic seeded chains and random-init
weights. `value` is replica-steps per second (the pages' timestep.mol/s),
the median of `--repeats` runs of exactly `--steps` steps each.

Beside it, the energy + force evaluation of the other workloads on a prebuilt
list (median of 5 runs x N iterations after 20 warm-ups): the 32-bead chain
(launch latency), 64 x 269-bead chains, and the 4096- and 65,536-atom
periodic boxes (fp32), each with the roofline of its dominant kernel (the
fused CFConv backward, timed with HIP events around every launch inside the
timed region) and its counter-measured HBM traffic; and the fp64 oracle timed
on the host cores on bounded samples.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from schnet_continuous_filter_amd import profiling  # noqa: E402  (no GPU work at import)

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0    # dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0
PREC_TAGS = {0: "f32", 1: "bf16", 2: "w16a16", 3: "f16x2"}
DTYPE_TAGS = {0: "f32", 1: "bf16-filter/f16x2-atomwise/f32", 2: "f16-mlps/f32", 3: "f16x2-filter/f32"}
PROFILES = os.path.join(ROOT, "profiles")
SUB_WORKLOADS = ("cg32", "cg269x64", "bulk4k", "bulk64k")


def counter_record(kind, workload, m):
    """The committed counter record (profiles/cfconv_<kind>_<workload>[_tag]_counters.txt)
    of the kernel of this workload and precision, or None when there is none
    or the kernels changed since it was taken. kind: 'bwd' or 'fwd'."""
    for name in (f"cfconv_{kind}_{workload}_{PREC_TAGS[m.filter_dtype]}_counters.txt",):
        path = os.path.join(PROFILES, name)
        if not os.path.exists(path):
            continue
        rec = json.load(open(path))
        if (rec.get("kernel_hash") == profiling.kernel_hash()
                and kernel_args(rec.get("kernel", ""), kind)[:3:2] == [str(m.D), str(m.filter_dtype)]
                and rec.get("workload", "").split("_")[0] == workload):
            return rec
    return None


def kernel_args(name, kind):
    """Template arguments of a CFConv kernel name as rocprofv3 reports it,
    "void sn::k_cf_bwd<D, KP, precision, q>(sn::CfParams)" (the forward has
    no q), as strings; [] for another kernel."""
    head = f"void sn::k_cf_{kind}<"
    if not name.startswith(head) or ">(" not in name:
        return []
    return [a.strip() for a in name[len(head):name.index(">(")].split(",")]


def utilisation_record(kind, workload, m):
    """MFMA-busy and VALU-busy fractions of the kernel from the committed
    counter record (profiles/cfconv_<kind>_<workload>_<prec>_util.txt), or
    None (missing, or the kernels changed since)."""
    path = os.path.join(PROFILES, f"cfconv_{kind}_{workload}_{PREC_TAGS[m.filter_dtype]}_util.txt")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != profiling.kernel_hash():
        return None
    return {k: rec[k] for k in ("mfma_busy", "valu_busy") if k in rec}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000,
                    help="MD steps per timed run of the headline workload")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--repeats", type=int, default=3,
                    help="timed runs of the headline; value is their median")
    ap.add_argument("--workload", default="md1024",
                    choices=["cg269x64", "cg32", "bulk4k", "bulk64k", "md1024"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subs", action="store_true",
                    help="skip the energy+force lines of the other workloads")
    ap.add_argument("--subs", default=",".join(SUB_WORKLOADS),
                    help="comma-separated workloads timed as energy+force evaluations")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle on the whole 65,536-atom box (about a minute "
                         "or more of host time)")
    ap.add_argument("--precision", choices=["f32", "bf16", "w16a16", "f16x2"], default=None,
                    help="override the workload's network operand precision")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device copy of known size (for counter scaling)")
    ap.add_argument("--ef-only", default="",
                    help="only time the energy+force evaluation of this workload (for "
                         "profiler runs); with --precision and --order")
    ap.add_argument("--order", choices=["given", "cell"], default="given",
                    help="with --ef-only on a periodic box: atoms as generated, or relabelled "
                         "in the order of 5 A cells (the same system)")
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


# ---------------------------------------------------------------- the oracle on the host
def host_info():
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def _oracle_model(m):
    import oracle
    return oracle.ModelDesc(m.n_types, m.D, m.Dr, m.T, m.rbf_min, m.rbf_max, m.r_cut, m.H,
                            m.filter_dtype)


def cpu_md_subset(R=8, steps=10):
    """The oracle as it stands on the MD workload's subset: R replicas of the
    269-bead chain, `steps` BAOAB steps (list at r_cut + 1 A rebuilt every 10
    steps, fp64 energy and forces with the bf16-rounded filter weights)."""
    import numpy as np
    import oracle
    from gen.configs import make_config

    c, pos, types, w = make_config("md1024", n_replicas=R)
    m, md = c.model, c.md
    desc = _oracle_model(m)
    W = oracle.unpack_weights(desc, w)
    N = c.system.atoms_per_replica
    state = {}

    def rebuild(p):
        state["nl"] = oracle.neighbor_list(np.asarray(p, np.float32), R, N, False, 0.0,
                                           m.r_cut + md.skin)

    def forces(p):
        return oracle.energy_forces(desc, None, p, types, *state["nl"], n_replicas=R,
                                    weights=W)

    t0 = time.perf_counter()
    rebuild(pos)
    E0, F0 = forces(pos.astype(np.float64))
    vel = oracle.init_velocities(0, len(pos), md.temperature_K, md.mass_amu)
    oracle.baoab_run(forces, rebuild, pos, vel, F0, dt_fs=md.dt_fs,
                     temperature_K=md.temperature_K, gamma_per_ps=md.gamma_per_ps,
                     mass_amu=md.mass_amu, skin=md.skin, rebuild_every=md.rebuild_every,
                     seed=0, step0=0, n_steps=steps)
    dt = time.perf_counter() - t0
    return R * steps / dt, dt


def cpu_ef(name, reps):
    """The oracle's energy + forces of a whole workload on its own list
    (median of `reps` runs), in edges/s."""
    import numpy as np
    import oracle
    from gen.configs import make_config

    c, pos, types, w = make_config(name)
    m, s = c.model, c.system
    desc = _oracle_model(m)
    W = oracle.unpack_weights(desc, w)
    rp, col = oracle.neighbor_list(pos, s.n_replicas, s.atoms_per_replica, s.periodic, s.box,
                                   m.r_cut)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.energy_forces(desc, None, pos, types, rp, col, n_replicas=s.n_replicas,
                             periodic=s.periodic, box=s.box, weights=W)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return len(col) / t, t


def cpu_baseline(subs, full):
    """The oracle on the host cores: the MD subset for the headline (8 of the
    1024 replicas, 10 steps), and whole energy + force evaluations of the
    other workloads, with every core the process may use and with one."""
    from threadpoolctl import threadpool_info, threadpool_limits

    cores, model = host_info()
    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        rs, dt = cpu_md_subset()
        out = {"value": rs, "unit": "replica-steps/s", "cores": cores, "kind": "oracle",
               "sample": f"8 of 1024 replicas x 269 beads, 10 BAOAB steps (list at 13 A, fp64 "
                         f"energy/forces, bf16-rounded filter weights) in {dt:.1f} s",
               "cpu_model": model, "blas_threads": blas, "workloads": {}}
        for name in subs:
            if name == "bulk64k" and not full:
                continue
            eps, t = cpu_ef(name, 1 if name in ("bulk64k", "cg269x64", "bulk4k") else 3)
            out["workloads"][name] = {"edges_per_s": eps, "s_per_ef": t, "threads": blas}
    with threadpool_limits(limits=1):
        for name in ("cg32", "bulk4k"):
            if name in subs:
                eps, t = cpu_ef(name, 1 if name == "bulk4k" else 3)
                out["workloads"][name]["edges_per_s_1thread"] = eps
    return out


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


def cf_flops(m, edges):
    """Algorithmic work of the fused CFConv kernels per launch: the two filter
    products per directed edge, 2 D (Dr + D) flops forward. The backward of a
    block whose source sums are wanted recomputes both products and runs
    their derivative along d through both, 4 D (Dr + D); the first block's
    backward (no source sums: its input is the embedding) needs the first
    product's values and tangents and the second's tangents only,
    2 D (2 Dr + D). Returned: forward, and the backward averaged over the T
    launches of one evaluation (what the mean launch time is taken over)."""
    fwd = 2.0 * m.D * (m.Dr + m.D) * edges
    bwd_q = 4.0 * m.D * (m.Dr + m.D) * edges
    bwd_0 = 2.0 * m.D * (2 * m.Dr + m.D) * edges
    return fwd, ((m.T - 1) * bwd_q + bwd_0) / m.T


def roofline(m, edges, bwd_us, fwd_us, workload):
    """Roofline object of the dominant kernel (the fused backward): achieved
    matrix throughput against the peak of its operand type, its
    counter-measured traffic (bytes per launch, None when no record of the
    current kernel exists) and the HBM fraction that traffic makes at the
    launch time."""
    _, fl_b = cf_flops(m, edges)
    half = m.filter_dtype != 0
    peak = PEAK_BF16_MFMA_TFLOPS if half else PEAK_FP32_MFMA_TFLOPS
    achieved = fl_b / (bwd_us * 1e-6) / 1e12
    rec = counter_record("bwd", workload, m)
    traffic = rec["bytes_per_launch"] if rec else None
    out = {"kernel": "k_cf_bwd (fused CFConv backward; mean over the T launches of an evaluation)",
           "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
           "frac": achieved / peak, "traffic": traffic,
           "flops_per_launch": fl_b, "avg_launch_us": bwd_us, "fwd_avg_launch_us": fwd_us,
           "hbm_gbs_at_traffic": (traffic / (bwd_us * 1e-6) / 1e9) if traffic else None,
           "hbm_frac_at_traffic": (traffic / (bwd_us * 1e-6) / 1e9 / PEAK_HBM_GBS)
           if traffic else None}
    util = utilisation_record("bwd", workload, m)
    if util:
        out["counters"] = util
    return out


def model_for(name, precision, order="given"):
    from gen.configs import make_config
    c, pos, types, w = make_config(name)
    if order == "cell":
        from gen.systems import cell_order
        if not c.system.periodic or c.system.n_replicas != 1:
            raise SystemExit("--order cell applies to a single periodic box")
        k = cell_order(pos, c.system.box)
        pos, types = pos[k].copy(), types[k].copy()
    m = c.model
    if precision is not None:
        import dataclasses
        m = dataclasses.replace(m, filter_dtype={v: k for k, v in PREC_TAGS.items()}[precision])
    return c, m, pos, types, w


def ef_timing(name, precision=None, runs=5, warmup=20, order="given"):
    """One energy + force evaluation of a workload on a prebuilt list (the
    list at r_cut, built and timed separately): median over `runs` runs of
    `iters` evaluations after `warmup`, with the CFConv launches timed by the
    library's event hook."""
    import torch
    from schnet_continuous_filter_amd import _lib as L
    c, m, pos, types, w = model_for(name, precision, order)
    s = c.system
    R, N = s.n_replicas, s.atoms_per_replica
    n = R * N
    iters = 100 if n <= 20000 else 20
    desc = L.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut,
                       m.filter_dtype)
    system = L.make_system(R, N, s.periodic, s.box)
    model = L.sn_model_create(desc, w)
    ws = L.Workspace(L.sn_workspace_size(desc, system))
    dev = torch.device("cuda")
    p = torch.from_numpy(pos).to(dev).reshape(-1)
    t = torch.from_numpy(types).to(dev)
    rowptr = torch.zeros(n + 1, dtype=torch.int32, device=dev)
    ne = L.sn_build_neighbors(system, p, m.r_cut, rowptr, None, 0, ws)
    col = torch.empty(max(ne, 1), dtype=torch.int32, device=dev)
    L.sn_reset_device_status(ws)
    L.sn_build_neighbors(system, p, m.r_cut, rowptr, col, ne, ws)
    energy = torch.empty(R, dtype=torch.float32, device=dev)
    forces = torch.empty(3 * n, dtype=torch.float32, device=dev)

    def timed(fn, k):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(k):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    build = lambda: L.sn_build_neighbors(system, p, m.r_cut, rowptr, col, ne, ws,
                                         return_count=False)
    ef = lambda: L.sn_energy_forces(model, system, p, t, rowptr, col, energy, forces, ws)
    for _ in range(warmup):
        build()
        ef()
    torch.cuda.synchronize()
    build_ms = statistics.median(timed(build, iters) for _ in range(runs))
    L.sn_profile_read(0)
    L.sn_profile_read(1)
    L.sn_profile_enable(True)
    ms = [timed(ef, iters) for _ in range(runs)]
    L.sn_profile_enable(False)
    bwd_ms, bwd_n = L.sn_profile_read(1)
    fwd_ms, fwd_n = L.sn_profile_read(0)
    status, detail, _ = L.sn_get_device_status(ws)
    L.sn_model_destroy(model)
    if status != 0:
        print(f"{name}: device status {status} ({L.status_string(status)}), detail {detail}",
              file=sys.stderr)
        sys.exit(1)
    med = statistics.median(ms)
    bwd_us = 1000.0 * bwd_ms / max(bwd_n, 1)
    fwd_us = 1000.0 * fwd_ms / max(fwd_n, 1)
    return {"workload": name, "replicas": R, "atoms_per_replica": N, "directed_edges": ne,
            "dtype": DTYPE_TAGS[m.filter_dtype], "ms_per_ef": med,
            "ms_per_ef_runs": ms, "runs": runs, "iters": iters, "warmup": warmup,
            "edges_per_s": ne / (med * 1e-3),
            "list_build_ms": build_ms,
            "edges_per_s_build_and_ef": ne / ((med + build_ms) * 1e-3),
            "roofline": roofline(m, ne, bwd_us, fwd_us, name)}


def ef_only(args):
    """Energy + force evaluations of one workload, nothing else (for profiler
    runs whose kernel statistics must cover exactly those launches)."""
    r = ef_timing(args.ef_only, args.precision, runs=max(1, args.repeats), warmup=args.warmup,
                  order=args.order)
    r["order"] = args.order
    r.pop("ms_per_ef_runs")
    print(json.dumps(r))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch  # (initialises the device before any library call)
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
    if args.ef_only:
        ef_only(args)
        return
    name = args.workload
    c, m, pos, types, w = model_for(name, args.precision)
    torch.cuda.reset_peak_memory_stats()
    r = md_timing(c, m, pos, types, w, args.steps, args.warmup, args.repeats)
    peak_mem = torch.cuda.max_memory_allocated()
    R = c.system.n_replicas
    line = {
        "metric": "CFConv energy+force edges/sec and replica-MD-steps/sec at 1 GPU; % HBM roofline",
        "value": r["replica_steps_per_s"],
        "unit": "replica-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "repeats": args.repeats,
        "ms_per_step": r["ms_per_step"],
        "ms_per_step_runs": r["ms_per_step_runs"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAGS[m.filter_dtype],
        "data": "synthetic (seeded chains/boxes, random-init weights)",
        "config": {"workload": name, "replicas": R,
                   "atoms_per_replica": c.system.atoms_per_replica,
                   "directed_edges_per_step": r["ne"], "list_radius_A": r["r_list"],
                   "list_edges_at_end": r["ne_list"], "D": m.D, "Dr": m.Dr,
                   "T": m.T, "r_cut_A": m.r_cut,
                   "rebuild_every": r["rebuild_every"],
                   "step": "BAOAB + scheduled neighbour rebuild + active list + energy/forces"},
        "edges_per_s": r["edges_per_s"],
        "peak_device_bytes": peak_mem,
        "roofline": roofline(m, r["ne"], r["bwd_us"], r["fwd_us"], name),
        "n_rebuilds": r["n_rebuilds"],
    }
    subs = [] if args.no_subs else [v for v in args.subs.split(",") if v]
    if subs:
        line["energy_forces"] = {}
        for sub in subs:
            e = ef_timing(sub)
            e.pop("ms_per_ef_runs")
            line["energy_forces"][sub] = e
        # the same fp32 models with their filter and atom-wise products on
        # fp16 hi/lo pairs (fp32-grade: held to the fp32 parity bars)
        line["energy_forces_f16x2"] = {}
        for sub in subs:
            e = ef_timing(sub, "f16x2")
            e.pop("ms_per_ef_runs")
            line["energy_forces_f16x2"][sub] = e
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(subs, args.cpu_full)
    print(json.dumps(line))


def md_timing(c, m, pos, types, w, steps, warmup, repeats):
    """MD steps of one model on the workload. Every repeat starts the same
    trajectory from the same state (initial velocities, list build and forces,
    then `warmup` steps, untimed) and times `steps` steps bracketed by device
    synchronisations, so that the repeats do the same work; the CFConv
    kernels' launch times are recorded by the library and the edges each
    evaluation ran on are counted on the device."""
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
    p0 = torch.from_numpy(pos).to(dev).reshape(-1)
    t = torch.from_numpy(types).to(dev)
    if c.md is not None:          # the MD workload keeps its own skin and cadence
        md = L.make_md_params(c.md.dt_fs, c.md.temperature_K, c.md.gamma_per_ps, c.md.mass_amu,
                              c.md.skin, c.md.rebuild_every, 0)
        r_list = m.r_cut + c.md.skin
        every = c.md.rebuild_every
    else:                         # rebuild every step at the cutoff
        md = L.make_md_params(2.0, 300.0, 1.0, 100.0, 0.0, 1, 0)
        r_list = m.r_cut
        every = 1
    rowptr0 = torch.zeros(R * N + 1, dtype=torch.int32, device=dev)
    ne0 = L.sn_build_neighbors(system, p0, r_list, rowptr0, None, 0, ws)
    L.sn_reset_device_status(ws)
    capacity = int(ne0 * 1.5) + 1024
    state = L.MdState(p0, capacity)
    energy = torch.empty(R, dtype=torch.float32, device=dev)
    runs, edges, rebuilds = [], [], []
    bwd_ms = fwd_ms = 0.0
    bwd_n = fwd_n = 0
    for _ in range(repeats):
        state.pos.copy_(p0)
        state.step = 0
        L.sn_md_init(model, system, t, md, state, energy, ws)
        L.sn_md_step(model, system, t, md, state, warmup, energy, ws)
        torch.cuda.synchronize()
        L.sn_reset_device_status(ws)
        L.sn_profile_read(0)
        L.sn_profile_read(1)
        L.sn_profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        L.sn_md_step(model, system, t, md, state, steps, energy, ws)
        torch.cuda.synchronize()
        runs.append(time.perf_counter() - t0)
        L.sn_profile_enable(False)
        b = L.sn_profile_read(1)
        f = L.sn_profile_read(0)
        bwd_ms, bwd_n, fwd_ms, fwd_n = bwd_ms + b[0], bwd_n + b[1], fwd_ms + f[0], fwd_n + f[1]
        status, detail, n_rebuilds = L.sn_get_device_status(ws)
        if status != 0:
            print(f"device status {status} ({L.status_string(status)}), detail {detail}",
                  file=sys.stderr)
            sys.exit(1)
        n_eval, n_edges = L.sn_get_device_counters(ws)
        assert n_eval == steps
        edges.append(n_edges)
        rebuilds.append(n_rebuilds)
        print(f"timed run: {steps} steps in {runs[-1]:.3f} s, {n_edges / steps:.0f} edges "
              f"per evaluation, {n_rebuilds} list builds", file=sys.stderr, flush=True)
    k = sorted(range(repeats), key=lambda i: runs[i])[repeats // 2]   # the median run
    elapsed = runs[k]
    ne_mean = edges[k] / steps
    # the list's size at the end of the last run (untimed)
    ne_list = L.sn_build_neighbors(system, state.pos, r_list, state.rowptr, state.col, capacity,
                                   ws)
    L.sn_model_destroy(model)
    return {"edges_per_s": edges[k] / elapsed, "ms_per_step": 1000.0 * elapsed / steps,
            "ms_per_step_runs": [1000.0 * v / steps for v in runs],
            "replica_steps_per_s": R * steps / elapsed, "ne": ne_mean, "ne_list": ne_list,
            "r_list": r_list, "rebuild_every": every,
            "bwd_us": 1000.0 * bwd_ms / max(bwd_n, 1), "fwd_us": 1000.0 * fwd_ms / max(fwd_n, 1),
            "bwd_n": bwd_n, "fwd_n": fwd_n, "n_rebuilds": rebuilds[k]}


if __name__ == "__main__":
    main()
