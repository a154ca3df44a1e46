"""Benchmark of the WISE working-set attention path on one MI355X.

One timed step is one whole recurrent-attention trajectory of the 4K
workload (batch 1, 32 heads, head_dim 128, seq 4096, block 64, T = 32
recurrent steps, td = 8, eta = 0.9): td discovery steps (dense attention +
fused block mass, in whichever of its two forms - partials on chip or in a
workspace - is faster on the workload), one support selection, and T - td
reuse steps of
block-sparse attention, each step on its own synthetic Q/K/V already resident
in HBM.  The headline value is the late-step block-sparse kernel's throughput
on its executed MFMA FLOPs; the same run reports the late-step speedup over
the library's own dense kernel, the realised support density, a roofline
record for the sparse kernel and the fp64 CPU oracle timed on a sample
(discovery, selection and late phases, plus a single-thread sample).

A sweep over the other workloads (8K, 16K and 32K context, the wide-head
batched workload, the long block-128 workload, and the 4K inputs selected at
eta = 0.6, about 15% of the full block grid) follows, each with its own
discovery steps, selection and a few reuse steps: late-step TFLOP/s, the
fraction of the bf16 peak, speedup over the dense kernel next to
1/density, and the same-backend comparison, every timing as median and
interquartile range.

    python bench.py [--steps K] [--warmup W] [--config ctx4k] [--no-cpu-baseline] [--no-sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "late-step sparse-attn TFLOP/s (% bf16 MFMA peak) + speedup vs dense, 4K ctx"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="ctx4k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4, help="most heads in the CPU-oracle sample")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of timed CPU-oracle work")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-workload sweep (8K, 16K, 32K, wide, long)")
    ap.add_argument("--sweep", default="ctx8k,ctx16k,ctx32k,wide,long,ctx4k_eta06",
                    help="workloads of the sweep (comma-separated)")
    ap.add_argument("--sweep-passes", type=int, default=7)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB first (HBM counter calibration)")
    ap.add_argument("--no-block-study", action="store_true",
                    help="skip the block-size study (the same inputs at block 16, 32, 64, 128)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the selection-variant figures (temporal union and the early-static controls)")
    ap.add_argument("--no-same-backend", action="store_true",
                    help="skip timing the sparse kernel on a full causal CSR (the same-backend comparison)")
    return ap.parse_args(argv)


def flop_counts(cfg, row_ptr_h):
    """Executed and algorithmic FLOPs of one sparse launch and one dense launch."""
    B, D, nb = cfg.block, cfg.head_dim, cfg.n_blocks
    heads = cfg.batch * cfg.heads
    n_rows = heads * nb
    nnz = int(row_ptr_h[-1])
    sparse_exec = 4.0 * D * B * B * nnz
    # every row holds its diagonal block, of which B(B+1)/2 query-key pairs are admissible
    sparse_alg = 4.0 * D * (B * B * (nnz - n_rows) + n_rows * B * (B + 1) / 2)
    dense_blocks = heads * nb * (nb + 1) // 2
    dense_exec = 4.0 * D * B * B * dense_blocks
    dense_alg = 4.0 * D * heads * cfg.seq_len * (cfg.seq_len + 1) / 2
    return dict(nnz=nnz, n_rows=n_rows, sparse_exec=sparse_exec, sparse_alg=sparse_alg,
                dense_exec=dense_exec, dense_alg=dense_alg, dense_blocks=dense_blocks,
                density_adm=nnz / dense_blocks, density_full=nnz / (heads * nb * nb))


def sparse_bytes(cfg, nnz, n_rows):
    """Compulsory HBM bytes of one sparse launch: Q, K, V read once, O written
    once (8 * S * D bytes per head), plus the CSR.  Re-reads of a K/V block by
    several rows are meant to hit L2/MALL."""
    D = cfg.head_dim
    heads = cfg.batch * cfg.heads
    qkvo = 4 * 2.0 * heads * cfg.seq_len * D
    csr = 4.0 * (n_rows + 1 + nnz)
    return qkvo + csr


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"sparse_attn_{name}_hbm_traffic.md")
KERNEL_SOURCES = ["block_sparse_attention_wise_amd/csrc/wise_attn_kernel.h",
                  "block_sparse_attention_wise_amd/csrc/wise_attn_d128.hip"]


def kernel_source_hash() -> str:
    """Hash of the attention kernel's code: line comments and blank lines are
    left out, so that editing a comment does not retire the counter record."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(name: str = "ctx4k"):
    """HBM bytes per sparse launch of workload ``name`` from the committed
    rocprofv3 counter runs (FETCH_SIZE / WRITE_SIZE, copy-calibrated), or
    None when there is no record or the attention kernel source changed
    since it was taken."""
    try:
        kv = {}
        with open(traffic_file(name)) as fh:
            for line in fh:
                if ":" in line and line.split(":")[0].strip() in (
                        "kernel_source_hash", "sparse_read_bytes_per_launch",
                        "sparse_write_bytes_per_launch"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_hash") != kernel_source_hash():
            return None
        return int(kv["sparse_read_bytes_per_launch"]) + int(kv["sparse_write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, max_heads: int, budget_s: float = 20.0):
    """The fp64 oracle, as it stands, timed on a bounded sample of the
    workload: heads 0, 1, ... of batch 0, each through its td discovery steps
    (dense attention, Eq. 2, with the block mass of Eq. 5), the selection
    (Eq. 6 on the mean mass) and its T - td late steps (masked attention,
    Eq. 8), until ``max_heads`` heads or about ``budget_s`` seconds of timed
    work.  Each phase is timed on its own.  The headline rate is the late
    phase's, on the same algorithmic FLOP count as the GPU figure; one
    discovery and one late head-step are also timed on a single thread."""
    import oracle
    from wise_inputs import Workload
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:                                          # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    wl = Workload(cfg, threads=1)
    B, td, D, S, nb = cfg.block, cfg.td, cfg.head_dim, cfg.seq_len, cfg.n_blocks
    sc = oracle.default_scale(D)
    dense_flops = 4.0 * D * S * (S + 1) / 2                    # one head, one step, algorithmic

    def discovery(Q, K, V):
        a = oracle.attention_weights(Q, K, sc)
        oracle.attention_output(a, V)
        return np.array([oracle.block_mass_rows(a[oracle.block_rows(qb, B, S)], B) for qb in range(nb)])

    def late_flops(supports):
        n_pairs = 0
        for qb, sup in supports.items():
            n_pairs += B * B * (len(sup) - 1) + B * (B + 1) // 2
        return 4.0 * D * n_pairs

    t_disc = t_sel = t_late = 0.0
    n_disc = n_sel = n_late = 0
    f_late = 0.0
    first = None
    for h in range(max_heads):
        masses, supports = [], {}
        for t, (q, k, v) in wl.head_steps(0, h):
            Q, K, V = (oracle.bf16_to_f64(x) for x in (q, k, v))
            if t < td:
                t0 = time.perf_counter()
                masses.append(discovery(Q, K, V))
                t_disc += time.perf_counter() - t0
                n_disc += 1
                continue
            if not supports:
                t0 = time.perf_counter()
                mbar = oracle.mean_block_mass(masses)
                supports = {qb: oracle.select_support(mbar[qb], qb, cfg.eta, cfg.cap) for qb in range(nb)}
                t_sel += time.perf_counter() - t0
                n_sel += 1
            if first is None:
                first = (Q, K, V, supports, masses[-1])
            t0 = time.perf_counter()
            oracle.masked_attention(Q, K, V, supports, B, sc)
            t_late += time.perf_counter() - t0
            n_late += 1
            f_late += late_flops(supports)
            if t_disc + t_sel + t_late > budget_s:
                break
        if t_disc + t_sel + t_late > budget_s:
            break
    single = None
    if threadpool_limits is not None and first is not None:
        Q, K, V, supports, _ = first
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            discovery(Q, K, V)
            t1 = time.perf_counter()
            oracle.masked_attention(Q, K, V, supports, B, sc)
            t2 = time.perf_counter()
        single = {"threads": 1, "discovery_tflops": round(dense_flops / (t1 - t0) / 1e12, 5),
                  "late_tflops": round(late_flops(supports) / (t2 - t1) / 1e12, 5),
                  "discovery_s_per_head_step": round(t1 - t0, 3), "late_s_per_head_step": round(t2 - t1, 3)}
    return {"value": f_late / t_late / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"batch 0, heads 0..{n_sel - 1} of {cfg.name} (of {cfg.batch * cfg.heads}): "
                       f"{n_disc} discovery head-steps, {n_sel} selections, {n_late} late head-steps, "
                       f"each phase timed ({t_disc:.1f} + {t_sel:.2f} + {t_late:.1f} s); value = late "
                       f"phase on the algorithmic FLOPs of the sample's supports"),
            "phases": {"discovery_tflops": round(n_disc * dense_flops / t_disc / 1e12, 5) if n_disc else None,
                       "discovery_s_per_head_step": round(t_disc / max(n_disc, 1), 3),
                       "select_ms_per_head": round(1e3 * t_sel / max(n_sel, 1), 2),
                       "late_tflops": round(f_late / t_late / 1e12, 5),
                       "late_s_per_head_step": round(t_late / max(n_late, 1), 3)},
            "single_thread": single,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "threads_note": "BLAS calls use `cores` threads; numpy's elementwise steps run on one"}


def discovery_forms(wise, torch, cfg, qs, ks, vs, mass, ws, o, reps=3):
    """Both forms of the discovery step (dense attention + fused block mass,
    Eq. 2 and 5) on the workload's td discovery inputs: the one with the
    per-(query, key block) partials on chip (wise_full_attn_accum: LDS, or a
    second pass over the keys for long rows) and the one with them in a
    device workspace (wise_full_attn_accum_ws).  Returns per-launch ms of
    each (median over ``reps`` passes) and the faster form's name."""
    td, B = cfg.td, cfg.block
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    forms = {
        "on_chip": lambda t: wise.wise_full_attn_accum(qs[t], ks[t], vs[t], mass, B, o=o),
        "workspace": lambda t: wise.wise_full_attn_accum_ws(qs[t], ks[t], vs[t], mass, B, o=o, workspace=ws),
    }
    xs = {name: [] for name in forms}
    for r in range(reps + 1):            # the forms alternate, pass by pass; pass 0 warms up
        for name, fn in forms.items():
            mass.zero_()
            e0.record(stream)
            for t in range(td):
                fn(t)
            e1.record(stream)
            e1.synchronize()
            if r > 0:
                xs[name].append(e0.elapsed_time(e1) / td)
    mass.zero_()
    out = {name: float(np.median(v)) for name, v in xs.items()}
    return out, min(out, key=out.get)


def quartiles(xs):
    """Median and interquartile range of a list of timings."""
    q25, q50, q75 = np.percentile(np.asarray(xs, dtype=np.float64), [25, 50, 75])
    return {"median": round(float(q50), 4), "iqr": [round(float(q25), 4), round(float(q75), 4)]}


def run_sweep(names, passes, wise, torch, dev, n_late=4):
    """Per-workload figures on one GPU: for each workload, its td discovery
    steps (dense attention + fused block mass, workspace partials), the
    selection, and n_late reuse steps on their own drifted inputs; the
    sparse launch is timed against the library's dense launch on the same
    late-step inputs and against itself on a full causal CSR (the
    same-backend comparison).  Every timing is the per-launch average of one
    pass of back-to-back launches, over ``passes`` passes (median and IQR)."""
    from wise_inputs import CONFIGS, Workload
    out = {}
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n_launch, reps):
        fn()                                   # warm-up pass
        xs = []
        for _ in range(reps):
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            xs.append(e0.elapsed_time(e1) / n_launch)
        return xs

    for name in names:
        cfg = CONFIGS[name]
        td, T, B, D, nb = cfg.td, cfg.steps, cfg.block, cfg.head_dim, cfg.n_blocks
        n_steps = td + n_late
        log(f"sweep {name}: generating {n_steps} steps")
        t0 = time.time()
        qs, ks, vs = [], [], []
        for t, q, k, v in Workload(cfg, threads=min(16, os.cpu_count() or 1)).steps(n_steps):
            for src, dst in ((q, qs), (k, ks), (v, vs)):
                dst.append(torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).to(dev))
        log(f"sweep {name}: inputs ready in {time.time() - t0:.1f} s")
        mass = torch.zeros(cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device=dev)
        o = torch.empty_like(qs[0])
        ws = torch.empty(max(wise.wise_accum_workspace_bytes(cfg.batch, cfg.heads, cfg.seq_len, D, B), 16),
                         dtype=torch.uint8, device=dev)
        n_rows = cfg.batch * cfg.heads * nb
        row_ptr = torch.empty(n_rows + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(wise.wise_select_max_nnz(cfg.batch, cfg.heads, cfg.seq_len, D, B, cfg.cap),
                              dtype=torch.int32, device=dev)

        forms, used = discovery_forms(wise, torch, cfg, qs, ks, vs, mass, ws, o)

        def discover():
            mass.zero_()
            for t in range(td):
                if used == "on_chip":
                    wise.wise_full_attn_accum(qs[t], ks[t], vs[t], mass, B, o=o)
                else:
                    wise.wise_full_attn_accum_ws(qs[t], ks[t], vs[t], mass, B, o=o, workspace=ws)

        def select():
            wise.wise_select_support(mass, td, cfg.eta, D, B, cfg.cap, row_ptr=row_ptr, col_idx=col_idx)

        k1 = timed(discover, td, passes)
        discover()
        k3 = timed(select, 1, passes)
        rp_h = row_ptr.cpu().numpy()
        fc = flop_counts(cfg, rp_h)

        def late():
            for t in range(td, n_steps):
                wise.wise_sparse_attn(qs[t], ks[t], vs[t], row_ptr, col_idx, B, o=o)

        def dense():
            for t in range(td, n_steps):
                wise.wise_full_attn(qs[t], ks[t], vs[t], B, o=o)
        full_rp = torch.from_numpy(np.concatenate([[0], np.cumsum(
            np.tile(np.arange(1, nb + 1), cfg.batch * cfg.heads))]).astype(np.int32)).to(dev)
        full_ci = torch.from_numpy(np.tile(np.concatenate([np.arange(q + 1) for q in range(nb)]),
                                           cfg.batch * cfg.heads).astype(np.int32)).to(dev)

        def full():
            for t in range(td, n_steps):
                wise.wise_sparse_attn(qs[t], ks[t], vs[t], full_rp, full_ci, B, o=o)
        k4 = timed(late, n_late, passes)
        k2 = timed(dense, n_late, passes)
        kf = timed(full, n_late, max(3, passes // 2))
        m = lambda xs: float(np.median(xs))
        t4, t2, t1, t3, tf = m(k4), m(k2), m(k1), m(k3), m(kf)
        ideal = 1.0 / fc["density_adm"]
        traffic = measured_traffic(name)
        out[name] = {
            "workload": (f"batch {cfg.batch}, {cfg.heads} heads, head_dim {D}, seq {cfg.seq_len}, block {B}, "
                         f"T {T}, td {td}, eta {cfg.eta}, cap {cfg.cap}"),
            "density_admissible": round(fc["density_adm"], 4),
            "density_full_grid": round(fc["density_full"], 4),
            "sparse_tflops_exec": round(fc["sparse_exec"] / (t4 * 1e-3) / 1e12, 2),
            "frac_bf16_peak_algorithmic": round(fc["sparse_alg"] / (t4 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_traffic_bytes_per_launch": traffic,
            "hbm_GBps": round(traffic / (t4 * 1e-3) / 1e9, 1) if traffic else None,
            "late_step_speedup_vs_dense": round(t2 / t4, 3),
            "ideal_speedup_1_over_density": round(ideal, 3),
            "speedup_over_ideal": round(t2 / t4 / ideal, 3),
            "same_backend_full_vs_support": round(tf / t4, 3),
            "setup_inclusive_speedup": round((T - td) * t2 / (t3 + (T - td) * t4), 3),
            "trajectory_speedup": round(T * t2 / (td * t1 + t3 + (T - td) * t4), 3),
            "dense_tflops_exec": round(fc["dense_exec"] / (t2 * 1e-3) / 1e12, 2),
            "accum_tflops_exec": round(fc["dense_exec"] / (t1 * 1e-3) / 1e12, 2),
            "discovery_forms": {n: {"ms": round(v, 4), "tflops_exec": round(fc["dense_exec"] / (v * 1e-3) / 1e12, 2)}
                                for n, v in forms.items()} | {"used": used},
            "kernel_ms": {"sparse_attn": quartiles(k4), "full_attn": quartiles(k2),
                          "full_attn_accum": quartiles(k1), "select_support": quartiles(k3),
                          "sparse_attn_full_csr": quartiles(kf)},
            "timed": f"{passes} passes of {n_late} late / {td} discovery launches; trajectory figures "
                     f"use the workload's T {T} and td {td} with these per-launch times",
        }
        log(f"sweep {name}: sparse {out[name]['sparse_tflops_exec']} TFLOP/s, speedup "
            f"{out[name]['late_step_speedup_vs_dense']} (ideal {out[name]['ideal_speedup_1_over_density']})")
        del qs, ks, vs, mass, o, ws, row_ptr, col_idx, full_rp, full_ci
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the WISE path here runs on a single MI355X "
              "(per-(batch, head) sharding across GPUs is a design note, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_wise_amd as wise
    from wise_inputs import CONFIGS, Workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wise.load_library()
    cfg = CONFIGS[args.config]
    T, td, B, D = cfg.steps, cfg.td, cfg.block, cfg.head_dim
    dev = torch.device("cuda:0")

    log(f"generating {T} steps of {cfg.name} inputs")
    t0 = time.time()
    qs, ks, vs = [], [], []
    for t, q, k, v in Workload(cfg, threads=min(16, os.cpu_count() or 1)).steps():
        for src, dst in ((q, qs), (k, ks), (v, vs)):
            dst.append(torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).to(dev))
    log(f"inputs ready in {time.time() - t0:.1f} s")

    nb = cfg.n_blocks
    mass = torch.zeros(cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device=dev)
    outs = [torch.empty_like(qs[0]) for _ in range(T)]
    n_rows = cfg.batch * cfg.heads * nb
    row_ptr = torch.empty(n_rows + 1, dtype=torch.int32, device=dev)
    cap = wise.wise_select_max_nnz(cfg.batch, cfg.heads, cfg.seq_len, D, B, cfg.cap)
    col_idx = torch.empty(cap, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    # Workspace of the discovery step's workspace form (allocated once,
    # outside the timed region).
    ws = torch.empty(max(wise.wise_accum_workspace_bytes(cfg.batch, cfg.heads, cfg.seq_len, D, B), 16),
                     dtype=torch.uint8, device=dev)

    # The discovery step runs in whichever of its two forms is faster on this
    # workload (on-chip partials, or partials in the workspace); chosen after
    # the warm-up trajectories below.
    used_form = "workspace"

    def accum(t, m):
        if used_form == "on_chip":
            wise.wise_full_attn_accum(qs[t], ks[t], vs[t], m, B, o=outs[t])
        else:
            wise.wise_full_attn_accum_ws(qs[t], ks[t], vs[t], m, B, o=outs[t], workspace=ws)

    def trajectory(record=False):
        if record:
            ev[0].record(stream)
        mass.zero_()
        for t in range(td):
            accum(t, mass)
        if record:
            ev[1].record(stream)
        wise.wise_select_support(mass, td, cfg.eta, D, B, cfg.cap, row_ptr=row_ptr, col_idx=col_idx)
        if record:
            ev[2].record(stream)
        for t in range(td, T):
            wise.wise_sparse_attn(qs[t], ks[t], vs[t], row_ptr, col_idx, B, o=outs[t])
        if record:
            ev[3].record(stream)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy} MiB read + {args.calibrate_copy} MiB written, x3")
        del src, dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        trajectory()
    torch.cuda.synchronize()
    forms, used_form = discovery_forms(wise, torch, cfg, qs, ks, vs, mass, ws, outs[0], reps=5)
    log(f"discovery forms (ms per launch): {forms}; trajectory uses {used_form}")
    for _ in range(args.warmup):
        trajectory()
    torch.cuda.synchronize()

    per = {"k1": [], "k3": [], "k4": []}
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        trajectory(record=True)
        ev[3].synchronize()
        per["k1"].append(ev[0].elapsed_time(ev[1]))
        per["k3"].append(ev[1].elapsed_time(ev[2]))
        per["k4"].append(ev[2].elapsed_time(ev[3]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    log(f"timed {args.steps} trajectories in {wall:.3f} s")

    rp_h = row_ptr.cpu().numpy()
    fc = flop_counts(cfg, rp_h)

    # Dense baseline on the same late-step inputs (the speedup denominator).
    def dense_late():
        for t in range(td, T):
            wise.wise_full_attn(qs[t], ks[t], vs[t], B, o=outs[t])
    for _ in range(args.warmup):
        dense_late()
    dts = []
    for _ in range(args.steps):
        ev[0].record(stream)
        dense_late()
        ev[1].record(stream)
        ev[1].synchronize()
        dts.append(ev[0].elapsed_time(ev[1]))

    # Same backend on every causal block (full-support CSR), on request.
    fts = []
    full_rp = torch.from_numpy(np.concatenate([[0], np.cumsum(
        np.tile(np.arange(1, nb + 1), cfg.batch * cfg.heads))]).astype(np.int32)).to(dev)
    full_ci = torch.from_numpy(np.tile(np.concatenate([np.arange(q + 1) for q in range(nb)]),
                                       cfg.batch * cfg.heads).astype(np.int32)).to(dev)

    def full_sparse():
        for t in range(td, T):
            wise.wise_sparse_attn(qs[t], ks[t], vs[t], full_rp, full_ci, B, o=outs[t])
    if not args.no_same_backend:
        for _ in range(args.warmup):
            full_sparse()
        for _ in range(max(3, args.steps // 4)):
            ev[0].record(stream)
            full_sparse()
            ev[1].record(stream)
            ev[1].synchronize()
            fts.append(ev[0].elapsed_time(ev[1]))

    med = lambda xs: float(np.median(xs))
    n_late = T - td

    def timed_ms(fn, reps):
        for _ in range(2):
            fn()
        out = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            ev[1].synchronize()
            out.append(ev[0].elapsed_time(ev[1]))
        return med(out)

    # Selection variants on the same discovery steps: per-step masses (one
    # zeroed buffer per step), the union over the last four discovery steps,
    # and the early-static controls with the first step; then the late
    # sparse launch on each variant's support.
    variants = None
    diagnostics = None
    if not args.no_variants:
        step_mass = torch.zeros(td, cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device=dev)
        for t in range(td):
            accum(t, step_mass[t])
        win = step_mass[td - min(4, td):td].contiguous()
        first = step_mass[:1].contiguous()
        ctrl = torch.cat([first, win]).contiguous()
        vcap = wise.wise_select_max_nnz(cfg.batch, cfg.heads, cfg.seq_len, D, B, 0)
        variants = {}
        for name, kind, sm in (("union", wise.SELECT_UNION, win), ("static", wise.SELECT_STATIC, first),
                               ("mass_matched", wise.SELECT_MASS_MATCHED, ctrl),
                               ("size_matched", wise.SELECT_SIZE_MATCHED, ctrl)):
            rp_v = torch.empty_like(row_ptr)
            ci_v = torch.empty(max(vcap, 1), dtype=torch.int32, device=dev)
            sel_ms = timed_ms(lambda: wise.wise_select_variant(kind, sm, cfg.eta, D, B, row_ptr=rp_v,
                                                               col_idx=ci_v), 5)
            fcv = flop_counts(cfg, rp_v.cpu().numpy())

            def late_v():
                for t in range(td, T):
                    wise.wise_sparse_attn(qs[t], ks[t], vs[t], rp_v, ci_v, B, o=outs[t])
            sp_ms = timed_ms(late_v, 3) / n_late
            variants[name] = {"select_ms": round(sel_ms, 4),
                              "density_admissible": round(fcv["density_adm"], 4),
                              "sparse_ms": round(sp_ms, 4),
                              "sparse_tflops_exec": round(fcv["sparse_exec"] / (sp_ms * 1e-3) / 1e12, 2),
                              "steps": "union of steps %d..%d" % (td - min(4, td), td - 1) if name == "union"
                              else ("step 0" if name == "static" else
                                    "step 0 ranking; union of steps %d..%d" % (td - min(4, td), td - 1))}
        # Diagnostics (Section 7; Appendix C.2): unrestricted block masses
        # at the late steps too, then the retained future attention mass of
        # the frozen supports, the adjacent rolling-set Jaccard at the
        # switch (Eq. 24) and the switch-vs-final Jaccard (Eq. 25).
        late_mass = torch.zeros(T - td, cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device=dev)
        for t in range(td, T):
            accum(t, late_mass[t - td])
        sel_union = wise.wise_select_variant(wise.SELECT_UNION, win, cfg.eta, D, B)

        def retained(csr):
            vals = [wise.wise_support_mass(late_mass[i], csr[0], csr[1], D, B) for i in range(T - td)]
            return float(torch.stack(vals).double().mean().item())

        def jacc(a, bb):
            inter, uni = wise.wise_support_overlap(a, bb, cfg.batch, cfg.heads, nb, D, B)
            per_b = inter.view(cfg.batch, -1).double().sum(1) / uni.view(cfg.batch, -1).double().sum(1)
            return float(per_b.mean().item())
        w = min(4, td)
        prev = step_mass[max(0, td - 1 - w):td - 1].contiguous() if td >= 2 else win
        fin = late_mass[T - td - min(4, T - td):].contiguous()
        w_prev = wise.wise_select_variant(wise.SELECT_UNION, prev, cfg.eta, D, B)
        w_fin = wise.wise_select_variant(wise.SELECT_UNION, fin, cfg.eta, D, B)
        diagnostics = {
            "retained_future_mass": round(retained((row_ptr, col_idx)), 4),
            "retained_future_mass_union": round(retained(sel_union), 4),
            "rolling_jaccard_at_switch": round(jacc(sel_union, w_prev), 4),
            "jaccard_switch_vs_final": round(jacc(sel_union, w_fin), 4),
            "note": (f"unrestricted masses of late steps {td}..{T - 1}; frozen supports: the main selection "
                     f"and the union of steps {td - w}..{td - 1}; rolling sets of Eq. 23 at steps "
                     f"{td - 2} and {T - 1}"),
        }
        del step_mass, win, first, ctrl, late_mass
    k4_ms = med(per["k4"]) / n_late            # one sparse launch
    k1_ms = med(per["k1"]) / td                # one discovery launch (incl. the mass memset share)
    k3_ms = med(per["k3"])
    k2_ms = med(dts) / n_late                  # one dense launch
    kfull_ms = med(fts) / n_late if fts else None
    value = fc["sparse_exec"] / (k4_ms * 1e-3) / 1e12
    alg_tflops = fc["sparse_alg"] / (k4_ms * 1e-3) / 1e12
    step_ms = wall / args.steps * 1e3
    traffic = measured_traffic(args.config)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: recurrent attention trajectory, batch {cfg.batch}, "
                                f"{cfg.heads} heads, head_dim {D}, seq {cfg.seq_len}, block {B}, "
                                f"T {T}, td {td}, eta {cfg.eta}, cap {cfg.cap}"),
                   "batch": cfg.batch, "heads": cfg.heads, "seq_len": cfg.seq_len,
                   "head_dim": D, "block": B, "recurrent_steps": T, "td": td, "eta": cfg.eta,
                   "parallelism": "single-gpu"},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "late_step_speedup_vs_dense": round(k2_ms / k4_ms, 3),
        "ideal_speedup_1_over_density": round(1.0 / fc["density_adm"], 3),
        "setup_inclusive_speedup": round(n_late * k2_ms / (k3_ms + n_late * k4_ms), 3),
        "trajectory_speedup": round(T * k2_ms / (td * k1_ms + k3_ms + n_late * k4_ms), 3),
        "same_backend_full_vs_support": round(kfull_ms / k4_ms, 3) if kfull_ms else None,
        "density_admissible": round(fc["density_adm"], 4),
        "density_full_grid": round(fc["density_full"], 4),
        "kernel_ms": {"sparse_attn": round(k4_ms, 4), "full_attn_accum": round(k1_ms, 4),
                      "select_support": round(k3_ms, 4), "full_attn": round(k2_ms, 4),
                      "sparse_attn_full_csr": round(kfull_ms, 4) if kfull_ms else None},
        "kernel_ms_quartiles": {"sparse_attn": quartiles([x / n_late for x in per["k4"]]),
                                "full_attn_accum": quartiles([x / td for x in per["k1"]]),
                                "select_support": quartiles(per["k3"]),
                                "full_attn": quartiles([x / n_late for x in dts]),
                                "sparse_attn_full_csr": quartiles([x / n_late for x in fts]) if fts else None,
                                "note": "per launch: each timed trajectory's launches back to back, "
                                        "median and interquartile range over the timed trajectories"},
        "dense_tflops_exec": round(fc["dense_exec"] / (k2_ms * 1e-3) / 1e12, 2),
        "accum_tflops_exec": round(fc["dense_exec"] / (k1_ms * 1e-3) / 1e12, 2),
        "discovery_forms": {n: {"ms": round(v, 4), "tflops_exec": round(fc["dense_exec"] / (v * 1e-3) / 1e12, 2)}
                            for n, v in forms.items()} | {"used": used_form},
        "sparse_tflops_algorithmic": round(alg_tflops, 2),
        "roofline": {"bound": "mfma", "kernel": f"wise_attn_kernel (sparse, head_dim {D}, block {B})",
                     "achieved": round(alg_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(alg_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 counters)",
                     "traffic_GBps": round(traffic / (k4_ms * 1e-3) / 1e9, 1) if traffic else None,
                     "compulsory_GBps": round(sparse_bytes(cfg, fc["nnz"], fc["n_rows"]) /
                                              (k4_ms * 1e-3) / 1e9, 1)},
    }
    # Block-size study (the pages' B in {16, 32, 64, 128} ablation): the
    # same inputs, discovery masses, selection and late sparse launches at
    # every block size; the dense denominator is the workload's own dense
    # launch (its cost does not depend on the block size).
    block_study = None
    if not args.no_block_study:
        block_study = {}
        k2_ms_ref = med(dts) / n_late
        for Bs in (16, 32, 64, 128):
            if cfg.seq_len % max(Bs, 32) != 0:
                continue
            cfg_b = cfg.with_(block=Bs)
            nb_b = cfg.seq_len // Bs
            m_b = torch.zeros(cfg.batch, cfg.heads, nb_b, nb_b, dtype=torch.float32, device=dev)
            ws_b = torch.empty(max(wise.wise_accum_workspace_bytes(cfg.batch, cfg.heads, cfg.seq_len, D, Bs), 16),
                               dtype=torch.uint8, device=dev)
            forms_b, _ = discovery_forms(wise, torch, cfg_b, qs, ks, vs, m_b, ws_b, outs[0])
            for t in range(td):
                wise.wise_full_attn_accum_ws(qs[t], ks[t], vs[t], m_b, Bs, o=outs[t], workspace=ws_b)
            rp_b, ci_b = wise.wise_select_support(m_b, td, cfg.eta, D, Bs, cfg.cap)
            fcb = flop_counts(cfg_b, rp_b.cpu().numpy())

            def late_b():
                for t in range(td, T):
                    wise.wise_sparse_attn(qs[t], ks[t], vs[t], rp_b, ci_b, Bs, o=outs[t])
            sp = timed_ms(late_b, 3) / n_late
            block_study[str(Bs)] = {"density_admissible": round(fcb["density_adm"], 4),
                                    "sparse_ms": round(sp, 4),
                                    "sparse_tflops_exec": round(fcb["sparse_exec"] / (sp * 1e-3) / 1e12, 2),
                                    "late_step_speedup_vs_dense": round(k2_ms_ref / sp, 3),
                                    "ideal_speedup_1_over_density": round(1.0 / fcb["density_adm"], 3),
                                    "discovery_ms": {n: round(v, 4) for n, v in forms_b.items()}}
            del m_b, rp_b, ci_b, ws_b

    if variants is not None:
        k2 = med(dts) / n_late
        for vv in variants.values():
            vv["late_step_speedup_vs_dense"] = round(k2 / vv["sparse_ms"], 3)
        result["selection_variants"] = variants
    if diagnostics is not None:
        result["diagnostics"] = diagnostics
    if block_study is not None:
        result["block_size_study"] = block_study
    if not args.no_sweep:
        del qs, ks, vs, outs
        torch.cuda.empty_cache()
        names = [n for n in args.sweep.split(",") if n and n != args.config]
        result["sweep"] = run_sweep(names, args.sweep_passes, wise, torch, dev)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_heads, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
