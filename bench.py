"""Benchmark: E2Former-V2 on-the-fly equivariant attention on one MI355X.

One step = one pass of the whole hot path over the workload: step 1 (EAAS
pre-coupling of every atom into the workspace) and steps 2-3 (the fused
neighbour stream with online softmax and the target-side EAAS), i.e.
e2f_attn_precouple + e2f_attn_aggregate, exactly what e2f_attn_forward runs.
Inputs are synthetic (seeded generator), resident in HBM before timing.

Prints one JSON line.  ``value`` is valid edges per second for the whole
step; ``roofline`` reports the dominant kernel (the aggregate) against
MI355X's 8 TB/s HBM peak using its algorithmic bytes; ``cpu_baseline`` times
the CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALIB_COPY_MIB = 1024

WORKLOADS = {
    # name -> (generator config, description)
    "large": "N=32768 uniform atoms at 0.1/A^3, r_c 8.4 A, K=256 padded with mask, lmax=2, "
             "C=128, H=16, fp32",
    "scaleout": "N=100000 uniform atoms at 0.1/A^3, r_c 5.0 A, K=64 padded with mask, lmax=2, "
                "C=128, H=16, bf16 storage / fp32 arithmetic",
    "water": "216 rigid H2O (648 atoms), r_c 5.0 A, K=64, lmax=2, C=128, H=16, fp32",
    "tiny": "N=64 uniform atoms, r_c 5.0 A, K=32, lmax=1, C=16, H=2, fp32",
    "eaas": "EAAS tensor product alone: 2^20 unit vectors (uniform on S^2), h [2^20, 9, 128], "
            "all 15 paths of lmax=2, fp32",
}

# Per-CU vector-memory path of gfx950: one 64-lane 16-byte-per-lane load per
# 16 cycles through the texture addresser / data return units, i.e. 64 B/clk
# per CU; 256 CUs at 2.4 GHz.  The aggregate kernel's counters show these
# units >90% busy, so this is the ceiling it runs against once the gathered
# rows hit in L2.
VMEM_PATH_PEAK_GBS = 64 * 256 * 2.4



def algorithmic_bytes(N, K, E, S, C, b):
    """Bytes the method must move (each neighbour's k and h' rows once per edge; no edge tensors)."""
    per_edge = (S + 1) * C * b                      # k_j row + S rows of h'_j
    per_target = K * 5 + C * b + S * C * b + 12     # idx + mask row, q_i, out_i, pos_i
    k2 = E * per_edge + N * per_target
    k1 = N * (S * C * b + (S + 2) * C * b + 12)     # read h, write k + h' + q, read pos
    return k1, k2, per_edge, per_target


def cpu_baseline(cfg, budget_s=15.0, seed=0):
    """Time the CPU oracle (single-threaded numpy, fp64) on a bounded target sample."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.attn import attn_forward as oracle_forward

    s = cfg.spec
    rng = np.random.default_rng(seed)
    order = rng.permutation(cfg.N)
    n_t, done_t, done_e, elapsed = 16, 0, 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < budget_s and done_t < cfg.N:
            tg = np.sort(order[done_t:done_t + n_t])
            t0 = time.perf_counter()
            oracle_forward(cfg.pos, cfg.h, cfg.idx, cfg.mask, s.H, s.lmax, targets=tg,
                           chunk_edges=4096)
            elapsed += time.perf_counter() - t0
            done_e += int(cfg.mask[tg].sum())
            done_t += tg.size
            n_t = min(n_t * 2, 1024)
    return {
        "value": done_e / elapsed,
        "unit": "edges/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_t} random targets of the {cfg.N}-atom workload ({done_e} edges), "
                  f"{elapsed:.1f} s, fp64 numpy with every edge materialised, BLAS limited to 1 "
                  "thread",
        "atoms_per_s": done_t / elapsed,
    }


KERNEL_SOURCES = ["interatomic_potentials_amd/csrc/e2f_kernels.hip",
                  "interatomic_potentials_amd/csrc/e2f_backward.hip",
                  "interatomic_potentials_amd/csrc/e2f_project.hip",
                  "interatomic_potentials_amd/csrc/e2f_device.hpp",
                  "interatomic_potentials_amd/csrc/e2f_internal.hpp"]


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and whitespace do not count."""
    import hashlib
    import re
    hsh = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        hsh.update(" ".join(text.split()).encode())
    return hsh.hexdigest()[:16]


def _counter_means(path):
    """Mean counter value per (kernel, counter) from a rocprofv3 counter_collection.csv."""
    import collections
    import csv
    acc = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            # the kernel with its template arguments, without its parameter list
            name = row["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "")
            name = name.strip()
            depth, cut = 0, len(name)
            for n, ch in enumerate(name):
                depth += ch == "<"
                depth -= ch == ">"
                if ch == "(" and depth == 0:
                    cut = n
                    break
            acc[(name[:cut].strip(), row["Counter_Name"])].append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_profile(pmc_dir, workload, out_path):
    """Write the committed counter summary from a directory of rocprofv3 csv runs.

    Expects sub-directories trace_<w>, fetch_<w>, write_<w>, hit_<w>, fetch_copy, write_copy
    (each holding run_*.csv) as produced by the commands listed in the summary.
    """
    import csv
    w = workload
    d = os.path.relpath(pmc_dir, ROOT) if os.path.isabs(pmc_dir) else pmc_dir   # as the runs named it
    stats = list(csv.DictReader(open(os.path.join(pmc_dir, f"trace_{w}", "run_kernel_stats.csv"))))
    fetch, nf = _counter_means(os.path.join(pmc_dir, f"fetch_{w}", "run_counter_collection.csv"))
    write, _ = _counter_means(os.path.join(pmc_dir, f"write_{w}", "run_counter_collection.csv"))
    hit_path = os.path.join(pmc_dir, f"hit_{w}", "run_counter_collection.csv")
    hit = _counter_means(hit_path)[0] if os.path.exists(hit_path) else {}
    cf, _ = _counter_means(os.path.join(pmc_dir, "fetch_copy", "run_counter_collection.csv"))
    cw, _ = _counter_means(os.path.join(pmc_dir, "write_copy", "run_counter_collection.csv"))
    copy_bytes = CALIB_COPY_MIB << 20
    kf = copy_bytes / (cf[("__amd_rocclr_copyBuffer", "FETCH_SIZE")] * 1024)
    kw = copy_bytes / (cw[("__amd_rocclr_copyBuffer", "WRITE_SIZE")] * 1024)
    lines = [f"# rocprofv3 summary: {w} workload ({WORKLOADS[w]})", "",
             f"kernel source hash: {kernel_source_hash()}", "",
             "Commands (run from the repository root on an MI355X, TMPDIR=/tmp):", "```"]
    extra = ""
    bench_cmd = ("python -u bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline"
                 "{x}").format(w=w, x=extra)
    lines += [f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_{w} "
              f"-o run -- {bench_cmd}",
              f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch_{w} -o run "
              f"-- {bench_cmd}",
              f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write_{w} -o run "
              f"-- {bench_cmd}",
              f"rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d "
              f"{d}/hit_{w} -o run -- {bench_cmd}",
              f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/fetch_copy -o run "
              f"-- python -u bench.py --calib-copy-mib {CALIB_COPY_MIB} --steps 3",
              f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/write_copy -o run "
              f"-- python -u bench.py --calib-copy-mib {CALIB_COPY_MIB} --steps 3",
              f"python bench.py --summarize-profile {d} --workload {w}", "```", "",
              "## Kernel trace (--kernel-trace --stats)", "",
              "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        if len(name) > 200:     # library kernels with long template argument lists
            name = name.split("<")[0].replace("void ", "").strip() + "<...>"
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |")
    lines += ["", "## Counter calibration (plain device copy of "
              f"{CALIB_COPY_MIB} MiB, `__amd_rocclr_copyBuffer`)", "",
              f"- FETCH_SIZE reads {cf[('__amd_rocclr_copyBuffer', 'FETCH_SIZE')]:.0f} KiB per copy "
              f"of {copy_bytes} B read: read factor {kf:.4f} bytes per counted byte",
              f"- WRITE_SIZE reads {cw[('__amd_rocclr_copyBuffer', 'WRITE_SIZE')]:.0f} KiB per copy "
              f"of {copy_bytes} B written: write factor {kw:.4f}", "",
              "## Per-dispatch counters (mean over dispatches) and calibrated traffic", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | TCC_HIT | TCC_MISS | L2 hit rate | "
              "traffic bytes per launch |", "|---|---|---|---|---|---|---|"]
    for k in sorted({k for (k, c) in fetch}):
        fb = fetch.get((k, "FETCH_SIZE"), 0.0)
        wb = write.get((k, "WRITE_SIZE"), 0.0)
        th = hit.get((k, "TCC_HIT_sum"), 0.0)
        tm = hit.get((k, "TCC_MISS_sum"), 0.0)
        traffic = fb * 1024 * kf + wb * 1024 * kw
        kn = k if len(k) <= 200 else k.split("<")[0].strip() + "<...>"
        lines.append(f"| `{kn}` | {fb:.0f} | {wb:.0f} | {th:.4g} | {tm:.4g} | "
                     f"{th / max(th + tm, 1):.3f} | {traffic:.6g} |")
        lines.append(f"<!-- traffic {kn} {traffic:.0f} -->")
    mfma_path = os.path.join(pmc_dir, f"mfma_{w}", "run_counter_collection.csv")
    if os.path.exists(mfma_path):
        mf, nm = _counter_means(mfma_path)
        lines += ["", "## MFMA counters of the learned projections (`k_proj_eaas`)", "",
                  "```",
                  f"rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                  f"SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d "
                  f"{d}/mfma_{w} -o run -- {bench_cmd} --no-extras --no-backward",
                  "```", "",
                  "- MOPS count 512 flops each; the projections' algorithmic count is "
                  "2 (S + 2) C^2 flops per atom.",
                  "- busy share = SQ_VALU_MFMA_BUSY_CYCLES (summed over 1024 SIMDs) / "
                  "(1024 x GRBM_GUI_ACTIVE / 8), GRBM_GUI_ACTIVE being summed over the 8 XCDs.", "",
                  "| kernel | dispatches | MFMA flops per dispatch | busy share |",
                  "|---|---|---|---|"]
        for k in sorted({k for (k, c) in mf if "k_proj_eaas" in k}):
            flops = 512.0 * (mf.get((k, "SQ_INSTS_VALU_MFMA_MOPS_F32"), 0.0)
                             + mf.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0))
            busy = mf.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0)
            active = mf.get((k, "GRBM_GUI_ACTIVE"), 0.0)
            share = busy / (1024.0 * active / 8.0) if active > 0 else float("nan")
            lines.append(f"| `{k}` | {nm.get((k, 'GRBM_GUI_ACTIVE'), 0)} | {flops:.4g} | "
                         f"{share:.2f} |")
    if os.path.exists(os.path.join(pmc_dir, "trace_default", "run_kernel_trace.csv")) and \
            os.path.exists(os.path.join(pmc_dir, "default.json")) and w == "large":
        lines += _default_trace_section(pmc_dir, d)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out_path)


def _default_trace_section(pmc_dir, d):
    """The timed steps of the default command under --kernel-trace, beside the bench's own
    HIP-event timing of the same steps in the same run."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(pmc_dir, "trace_default",
                                                 "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    with open(os.path.join(pmc_dir, "default.json")) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    warmup, steps = line["warmup"], line["steps"]
    # the plain (no envelope) instance of the shared-row aggregate
    is_plain = lambda n: "k_aggregate_mt<" in n and n.split(">(")[0].endswith("false")
    plain = next((r["Kernel_Name"].split("(")[0].replace("void ", "") for r in rows
                  if is_plain(r["Kernel_Name"])), "k_aggregate_mt")
    kern, span, sched_start = [], [], None
    for r in rows:
        name = r["Kernel_Name"]
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if "k_sched_" in name and sched_start is None:
            sched_start = t0
        elif is_plain(name):
            kern.append((t1 - t0) * 1e-6)
            span.append((t1 - (sched_start if sched_start is not None else t0)) * 1e-6)
            sched_start = None
        elif "k_eaas" in name or "k_proj_eaas" in name:
            sched_start = None
    timed_k = kern[warmup:warmup + steps]
    timed_s = span[warmup:warmup + steps]
    mean = lambda v: sum(v) / max(len(v), 1)
    return ["", "## The default command under the kernel trace", "", "```",
            f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_default "
            f"-o run -- python -u bench.py > {d}/default.json", "```", "",
            f"The bench's own timing of its {steps} timed steps in this run (HIP events around "
            f"the aggregate call, schedule kernels included): "
            f"{line['kernels_ms']['aggregate']:.4f} ms.", "",
            f"- `{plain}` dispatches {warmup + 1}-{warmup + steps} (the timed steps, after "
            f"{warmup} warm-up steps): mean {mean(timed_k):.4f} ms, "
            f"min {min(timed_k):.4f}, max {max(timed_k):.4f}",
            f"- the same steps from the first schedule kernel's start to the aggregate's end: "
            f"mean {mean(timed_s):.4f} ms",
            f"- all {len(kern)} dispatches of `{plain}` in the run: mean {mean(kern):.4f} ms"]


def aggregate_kernel(spec):
    """The aggregate kernel the library launches for this workload (mirrors its selection rule)."""
    C, H = spec.C, spec.H
    d = C // H
    shared = (spec.dtype == "f32" and spec.K <= 256 and d % 4 == 0 and d // 4 in (1, 2, 4)
              and C // 4 <= 64)
    return "e2f::k_aggregate_mt" if shared else "e2f::k_aggregate"


def committed_traffic(workload, kernel="e2f::k_aggregate"):
    """Calibrated HBM bytes per launch from the committed summary, if the kernel is unchanged."""
    base = "k_eaas" if workload == "eaas" else "k_aggregate"
    path = os.path.join(ROOT, "profiles", f"{base}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"kernel source hash: {kernel_source_hash()}" not in text:
        return None
    import re
    # the plain instance: the envelope flag (the workspace flag of k_eaas) is false
    flag = {"e2f::k_aggregate": 6, "e2f::k_aggregate_mt": 4, "e2f::k_eaas": 3}[kernel]
    for args, val in re.findall(r"<!-- traffic %s<([^>]*)> (\d+) -->" % re.escape(kernel), text):
        if [x.strip() for x in args.split(",")][flag] == "false":
            return float(val)
    return None


def bench_backward(args, e2f, cfg, pos, h, idx, mask, ws, out, stream):
    """Time e2f_attn_backward (dL/dh, dL/dpos) after a forward that saves m and the lse."""
    import numpy as np
    import torch

    s = cfg.spec
    N, K, S, C, H, E = cfg.N, s.K, cfg.S, s.C, s.H, cfg.nl.n_edges
    if h.dtype != torch.float32:
        return {"skipped": "backward is fp32-only"}
    g = torch.randn_like(out)
    bws = torch.empty(e2f.attn_backward_workspace_bytes(N, K, s.lmax, C, H), dtype=torch.uint8,
                      device=h.device)
    gh = torch.empty_like(h)
    gp = torch.empty_like(pos)

    def timed(env_cutoff):
        _, msg, lse = e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, torch.float32,
                                         out=out, return_msg=True, return_lse=True,
                                         env_cutoff=env_cutoff)

        def run():
            e2f.attn_backward(pos, h, idx, mask, H, ws, msg, lse, g, bwd_ws=bws, grad_h=gh,
                              grad_pos=gp, env_cutoff=env_cutoff)

        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record(stream)
            run()
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    ms = timed(None)
    env_ms = timed(float(s.cutoff))      # the envelope-weighted softmax, radius = list cutoff
    row = (S + 1) * C * 4
    # prep reads G, m, h row 0 and writes q + dm rows; each stream reads one row block per edge
    # (k + h' for the target pass; q + dm plus lse and D for the source pass) and per atom
    # its own rows; the source pass also writes grad_h and reads h
    b_prep = N * (2 * S * C * 4 + C * 4 + row + H * 4 + 12 + 12)
    b_q = E * row + N * (K * 5 + row + C * 4 + 2 * H * 4)
    b_src = E * (row + 2 * 4) + N * (row + S * C * 4 + S * C * 4 + C * 4 + 12 + 12)
    total = b_prep + b_q + b_src
    print(f"[bench] backward: {ms:.3f} ms, {total / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic; "
          f"with the envelope {env_ms:.3f} ms", file=sys.stderr, flush=True)
    return {"ms": ms, "edges_per_s": E / (ms * 1e-3), "algorithmic_bytes": total,
            "algorithmic_GBps": total / (ms * 1e-3) / 1e9,
            "bytes_per_edge": 2 * row + 8, "envelope_ms": env_ms}


# published dense peaks of MI355X (TFLOP/s) for the matrix-core dtypes used here
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}


def bench_proj(args, e2f, cfg, pos, h, idx, mask, ws, out, stream):
    """Learned projections on the matrix cores, fused with the pre-coupling (and the full step)."""
    import numpy as np
    import torch

    from gen import proj_weights

    s = cfg.spec
    N, S, C, H, E = cfg.N, cfg.S, s.C, s.H, cfg.nl.n_edges
    bf16 = s.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    b = 2 if bf16 else 4
    w = tuple(torch.from_numpy(x).to(h.device).to(tdt)
              for x in proj_weights(s.lmax, C, seed=13, dtype=s.dtype))

    def pre():
        e2f.attn_precouple(pos, h, ws, proj=w)

    for _ in range(args.warmup):
        pre()
        e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, tdt, out=out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        pre()
        e[1].record(stream)
        e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, tdt, out=out)
        e[2].record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    step_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
    flops = 2.0 * N * (S + 2) * C * C                 # S value rows + q + k per atom
    nbytes = N * (S * C * b + 12 + (S + 2) * C * b) + (s.lmax + 3) * C * C * b  # + weights
    tflops = flops / (k_ms * 1e-3) / 1e12
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    peak = MFMA_PEAK_TFLOPS["bf16" if bf16 else "f32"]
    mfma_frac, hbm_frac = tflops / peak, gbs / HBM_PEAK_GBS
    bound = "mfma" if flops / nbytes > peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
    print(f"[bench] projected: precouple+projections {k_ms:.3f} ms ({tflops:.1f} TFLOP/s = "
          f"{mfma_frac:.2f} of MFMA peak, {gbs:.0f} GB/s), step {step_ms:.3f} ms",
          file=sys.stderr, flush=True)
    return {"kernel": "k_proj_eaas (projections on MFMA fused with the pre-coupling)",
            "ms_per_step": step_ms, "edges_per_s": E / (step_ms * 1e-3), "kernel_ms": k_ms,
            "bound": bound, "flops": flops, "achieved_tflops": tflops, "mfma_peak_tflops": peak,
            "mfma_frac": mfma_frac, "algorithmic_bytes": nbytes, "achieved_GBps": gbs,
            "hbm_frac": hbm_frac, "weights": "seeded N(0, 1/C), proj_weights(seed=13)"}


def _time(stream, steps, fn):
    """Mean milliseconds of fn() over `steps` launches, HIP events on `stream`."""
    import numpy as np
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))


def bench_neighbours(args, e2f, cfg, pos, stream):
    """The GPU neighbour-list builder on the same positions, cutoff and K (not part of a step)."""
    import numpy as np
    import torch

    s = cfg.spec
    N, K = cfg.N, s.K
    nws = torch.empty(e2f.neighbour_workspace_bytes(N), dtype=torch.uint8, device=pos.device)
    for _ in range(args.warmup):
        idx, mask = e2f.neighbour_list(pos, s.cutoff, K, ws=nws)
    torch.cuda.synchronize()
    same = bool(np.array_equal(idx.cpu().numpy(), cfg.idx)
                and np.array_equal(mask.cpu().numpy(), cfg.mask))
    ms = _time(stream, args.steps, lambda: e2f.neighbour_list(pos, s.cutoff, K, ws=nws))
    # per target: its 27 cells' grouped positions and indices are read (mostly from cache);
    # the algorithmic floor is reading the positions once and writing the rows
    nbytes = N * (12 + 16 + 4 + 4) + N * K * 5
    print(f"[bench] neighbour list: {ms:.3f} ms ({N / (ms * 1e-3) / 1e6:.1f} M atoms/s), rows equal "
          f"to the generator's: {same}", file=sys.stderr, flush=True)
    return {"kernel": "e2f_neighbour_list (cell list, Morton-ordered cells, one wave per target)",
            "ms": ms, "atoms_per_s": N / (ms * 1e-3), "rows_equal_generator": same,
            "output_bytes": N * K * 5, "min_bytes": nbytes,
            "note": "builds the padded list the step consumes; not inside the timed step"}


def bench_envelope(args, e2f, cfg, pos, h, idx, mask, ws, out, stream, k2_ms):
    """The same step with the smooth distance envelope on the softmax weights (r_env = cutoff)."""
    import torch
    s = cfg.spec
    tdt = h.dtype

    def agg():
        e2f.attn_aggregate(pos, idx, mask, ws, s.H, s.lmax, s.C, tdt, out=out,
                           env_cutoff=s.cutoff)

    e2f.attn_precouple(pos, h, ws)
    for _ in range(args.warmup):
        agg()
    torch.cuda.synchronize()
    ms = _time(stream, args.steps, agg)
    print(f"[bench] envelope: aggregate {ms:.3f} ms (plain {k2_ms:.3f} ms)", file=sys.stderr,
          flush=True)
    return {"kernel": "k_aggregate with the distance envelope (r_env = list cutoff)",
            "aggregate_ms": ms, "edges_per_s_aggregate": cfg.nl.n_edges / (ms * 1e-3),
            "overhead_vs_plain": ms / k2_ms - 1.0}


def bench_eaas(args, e2f, dev):
    """The EAAS tensor product on its own (e2f_eaas_couple over 2^20 vectors)."""
    import numpy as np
    import torch

    from gen import make_micro

    r_np, h_np, _ = make_micro()
    B, S, C = h_np.shape
    r = torch.from_numpy(r_np).to(dev)
    h = torch.from_numpy(h_np).to(dev)
    out = torch.empty_like(h)
    del h_np
    for _ in range(args.warmup):
        e2f.eaas_couple(r, h, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        e2f.eaas_couple(r, h, out=out)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    per_vec = 2 * S * C * 4 + 12
    gbs = B * per_vec / (ms * 1e-3) / 1e9
    print(f"[bench] eaas: {B} vectors, {ms:.3f} ms, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    result = {
        "metric": "EAAS tensor-product vectors/s (lmax=2, C=128, all 15 paths)",
        "value": B / (ms * 1e-3), "unit": "vectors/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded generator)",
        "config": {"workload": WORKLOADS["eaas"], "vectors": B, "lmax": 2, "channels": C},
        "roofline": {"kernel": "k_eaas", "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": committed_traffic("eaas", "e2f::k_eaas"),
                     "algorithmic_bytes_per_launch": B * per_vec, "bytes_per_vector": per_vec},
    }
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-proj", action="store_true",
                    help="skip the learned-projection variant (MFMA) timed after the main step")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the envelope variant and the neighbour-list build timed after it")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward pass (dL/dh, dL/dpos) timed after the forward")
    ap.add_argument("--index-order-reference", action="store_true",
                    help="also time the aggregate visiting targets in index order (no schedule)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="write profiles/k_aggregate_<workload>.md from rocprofv3 csv runs in DIR")
    args = ap.parse_args(argv)

    if args.summarize_profile:
        kernel = "k_eaas" if args.workload == "eaas" else "k_aggregate"
        summarize_profile(args.summarize_profile, args.workload,
                          os.path.join(ROOT, "profiles", f"{kernel}_{args.workload}.md"))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18           # float32 elements
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
              for _ in range(max(args.steps, 1))]
        for e in ev:
            e[0].record(stream)
            b.copy_(a)
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        # a plain device copy: the HBM rate a streaming kernel can reach in practice
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4,
                          "launches": len(ev) + 1, "copy_ms": ms,
                          "copy_GBps": 2 * n * 4 / (ms * 1e-3) / 1e9}))
        return 0

    import interatomic_potentials_amd as e2f
    from gen import make_config

    if args.workload == "eaas":
        return bench_eaas(args, e2f, dev)

    t_gen = time.perf_counter()
    cfg = make_config(args.workload)
    s = cfg.spec
    N, K, S, C, H = cfg.N, s.K, cfg.S, s.C, s.H
    E = cfg.nl.n_edges
    bf16 = s.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    b = 2 if bf16 else 4
    print(f"[bench] workload {args.workload}: N={N} K={K} lmax={s.lmax} C={C} H={H} "
          f"dtype={s.dtype} E={E} (inputs generated in {time.perf_counter() - t_gen:.1f} s)",
          file=sys.stderr, flush=True)

    pos = torch.from_numpy(cfg.pos).to(dev)
    h = torch.from_numpy(cfg.h).to(dev).to(tdt)
    idx = torch.from_numpy(cfg.idx).to(dev)
    mask = torch.from_numpy(cfg.mask).to(dev)
    ws = torch.empty(e2f.attn_workspace_bytes(N, s.lmax, C, e2f.BF16 if bf16 else e2f.F32),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(h)
    torch.cuda.synchronize()

    def step():
        e2f.attn_precouple(pos, h, ws)
        e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, tdt, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        e2f.attn_precouple(pos, h, ws)
        ev[k][1].record(stream)
        e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, tdt, out=out)
        ev[k][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    k2_ms_min = float(np.min([e[1].elapsed_time(e[2]) for e in ev]))

    k2_unsched_ms = None
    if args.index_order_reference:
        # reference only: the same aggregate visiting targets in index order (no schedule)
        ev_u = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
        for e in ev_u:
            e[0].record(stream)
            e2f.attn_aggregate(pos, idx, mask, ws, H, s.lmax, C, tdt, out=out,
                               targets_in_order=True)
            e[1].record(stream)
        torch.cuda.synchronize()
        k2_unsched_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev_u]))

    k1_bytes, k2_bytes, per_edge, per_target = algorithmic_bytes(N, K, E, S, C, b)
    k2_gbs = k2_bytes / (k2_ms * 1e-3) / 1e9
    step_gbs = (k1_bytes + k2_bytes) / (ms_step * 1e-3) / 1e9
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; precouple {k1_ms:.3f} ms "
          f"({k1_bytes / (k1_ms * 1e-3) / 1e9:.0f} GB/s), aggregate {k2_ms:.3f} ms "
          f"(min {k2_ms_min:.3f}) = {k2_gbs:.0f} GB/s algorithmic", file=sys.stderr, flush=True)

    traffic = committed_traffic(args.workload, aggregate_kernel(s))
    result = {
        "metric": "edges/s + achieved HBM GB/s, fused on-the-fly attention, N=32768 K=256",
        "value": E / (ms_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded generator; uniform-random atoms, N(0,1) features)",
        "config": {
            "workload": WORKLOADS[args.workload],
            "atoms": N, "padded_K": K, "valid_edges": E, "lmax": s.lmax, "channels": C,
            "heads": H, "cutoff_A": s.cutoff, "seed": s.seed,
        },
        "atoms_per_s": N / (ms_step * 1e-3),
        "step_algorithmic_GBps": step_gbs,
        "kernels_ms": {"precouple": k1_ms, "aggregate": k2_ms,
                       "aggregate_index_order_reference": k2_unsched_ms},
        "roofline": {
            "kernel": (aggregate_kernel(s).split("::")[1]
                       + (" (steps 2-3, three targets per wave sharing the rows they read)"
                          if aggregate_kernel(s).endswith("_mt") else " (steps 2-3)")
                       + ", timed with its target-schedule kernels"),
            "bound": "hbm",
            "achieved": k2_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": k2_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            # calibrated HBM/fabric bytes of the committed profile over this run's duration
            "traffic_GBps": traffic / (k2_ms * 1e-3) / 1e9 if traffic else None,
            "traffic_frac": traffic / (k2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS if traffic else None,
            "algorithmic_bytes_per_launch": k2_bytes,
            "bytes_per_edge": per_edge,
            "bytes_per_target": per_target,
            "vmem_path_peak": VMEM_PATH_PEAK_GBS,
            "vmem_path_frac": k2_gbs / VMEM_PATH_PEAK_GBS,
        },
    }
    if not args.no_proj:
        result["projected"] = bench_proj(args, e2f, cfg, pos, h, idx, mask, ws, out, stream)
    if not args.no_extras:
        result["envelope"] = bench_envelope(args, e2f, cfg, pos, h, idx, mask, ws, out, stream,
                                            k2_ms)
        result["neighbour_list"] = bench_neighbours(args, e2f, cfg, pos, stream)
    if not args.no_backward:
        result["backward"] = bench_backward(args, e2f, cfg, pos, h, idx, mask, ws, out, stream)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, budget_s=args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
