"""Benchmark: GEMM TFLOP/s and fraction of the MFMA peak on one MI355X.

Default workload: 8192^3 bf16 (A, B K-major, D bf16), one persistent-GEMM launch per step.
Inputs are seeded synthetic data already resident in HBM when the timed region starts.
Timing: HIP events on the stream the kernel is launched on (torch's current stream), around
exactly --steps launches after --warmup untimed ones, bracketed by device synchronisation.
The same line also reports the fp8 (e4m3 x e5m2) 8192^3 and varlen-M grouped workloads,
the roofline of the dominant kernel and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]
                    [--cold N]

`roofline.attainable_us` is the time at the roofline, max(FLOPs / MFMA peak, algorithmic
bytes / 8 TB/s), summed per group for grouped workloads (small groups can be HBM-bound on
their B read); `frac_of_attainable` compares the measured time with it. `--cold N` times the
primary workload rotating N input sets (the pages' cold-L2 option; N = 4 holds over 1 GB for
8192^3 bf16, more than the 256 MB MALL); the default is warm.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOPS and % of MFMA peak at 8192^3 bf16/fp8; varlen-M grouped TFLOPS"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "e5m2": 5000.0}
HBM_PEAK_GBS = 8000.0
PRIMARY = "square_8192_bf16"
SECONDARY = ["fp8_8192", "varlen_moe", "square_8192_f16", "act_4096", "batched_2048", "dact_4096",
             "varlen_k_moe", "varlen_moe_gather", "varlen_k_moe_gather"]


def code_text(src):
    """C++ source without its comments, one token run per line: what a comment or layout edit
    leaves unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return "\n".join(" ".join(line.split()) for line in "".join(out).splitlines() if line.strip())


def source_hash():
    """Hash of the kernel sources' code (comments and layout excluded): traffic counters are
    only reported for the same code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_epilogue_persistent_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(f.encode() + b"\0")
            h.update(code_text(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(inp):
    """Minimum HBM bytes: read A, B (and C) once, write the outputs once."""
    es = {"f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e5m2": 1, "none": 0}
    if inp.varlen:
        a = (inp.A.shape[0] if inp.a_idx is not None else inp.M) * inp.K * es[inp.a_dt]
        b = inp.L * inp.N * inp.K * es[inp.b_dt]
        mn = inp.M * inp.N
    elif inp.cu_seqlens_k is not None:
        a = inp.M * (inp.A.shape[1] if inp.a_idx is not None else inp.K) * es[inp.a_dt]
        b = inp.N * inp.K * es[inp.b_dt]
        mn = inp.L * inp.M * inp.N
    else:
        a = inp.L * inp.M * inp.K * es[inp.a_dt]
        b = inp.L * inp.N * inp.K * es[inp.b_dt]
        mn = inp.L * inp.M * inp.N
    return a + b + mn * (es[inp.c_dt] + es[inp.d_dt] + es[inp.post_dt])


def attainable_s(inp):
    """Seconds at the roofline: max(FLOPs / MFMA peak, algorithmic bytes / HBM peak), summed
    over the groups of a grouped problem (a small group can be HBM-bound on its B read while
    the whole problem is not)."""
    es = {"f16": 2, "bf16": 2, "f32": 4, "e4m3": 1, "e5m2": 1, "none": 0}
    peak = PEAK_TFLOPS[inp.a_dt] * 1e12
    hbm = HBM_PEAK_GBS * 1e9
    out_b = es[inp.c_dt] + es[inp.d_dt] + es[inp.post_dt]

    def roof(fl, by):
        return max(fl / peak, by / hbm)
    if inp.varlen:
        ms = [int(x) for x in (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1])]
        return sum(roof(2.0 * m * inp.N * inp.K,
                        m * inp.K * es[inp.a_dt] + inp.N * inp.K * es[inp.b_dt] + m * inp.N * out_b)
                   for m in ms)
    if inp.cu_seqlens_k is not None:
        ks = [int(x) for x in (inp.cu_seqlens_k[1:] - inp.cu_seqlens_k[:-1])]
        return sum(roof(2.0 * inp.M * inp.N * k,
                        (inp.M * es[inp.a_dt] + inp.N * es[inp.b_dt]) * k + inp.M * inp.N * out_b)
                   for k in ks)
    return roof(inp.flops(), algorithmic_bytes(inp))


def setup(name, **tuning):
    import torch
    import workloads as W
    from gemm_epilogue_persistent_amd import Plan
    from workloads import to_dev, out_like
    inp = W.WORKLOADS[name]()
    A, B, C = to_dev(inp.A), to_dev(inp.B), to_dev(inp.C)
    D = out_like(inp, inp.d_dt) if inp.d_dt != "none" else None
    P = out_like(inp, inp.post_dt) if inp.post_dt != "none" else None
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda") if inp.varlen else None
    cuk = torch.from_numpy(inp.cu_seqlens_k).to("cuda") if inp.cu_seqlens_k is not None else None
    idx = torch.from_numpy(inp.a_idx).to("cuda") if inp.a_idx is not None else None
    if inp.dact:
        tuning = dict(tuning, dact=True)
    plan = Plan(A, B, C, D, P, inp.alpha, inp.beta, inp.act, cu, cuk, idx, **tuning)
    args = (A, B, C, D, P, None, None, cu)
    if cuk is not None or idx is not None:
        plan = _Bound(plan, cu_seqlens_k=cuk, a_idx=idx)
    return inp, plan, args


class _Rotating:
    """Runs the plan on input set i % n at call i (--cold: more input bytes than the 256 MB
    MALL, so that every launch reads its operands from HBM)."""

    def __init__(self, plan, sets):
        self.plan, self.sets, self.i = plan, sets, 0

    def run(self, *_):
        self.plan.run(*self.sets[self.i % len(self.sets)])
        self.i += 1


def cold_sets(args, n):
    """n input sets: the given one and n - 1 copies of its A, B and C (outputs shared)."""
    sets = [args]
    for _ in range(n - 1):
        A, B, C = (None if x is None else x.clone() for x in args[:3])
        sets.append((A, B, C) + tuple(args[3:]))
    return sets


class _Bound:
    """A plan whose run() carries the varlen-K / gather device arrays."""

    def __init__(self, plan, **extra):
        self.plan, self.extra = plan, extra

    def run(self, *args):
        self.plan.run(*args, **self.extra)

    def grid(self):
        return self.plan.grid()

    def raster_along_n(self):
        return self.plan.raster_along_n()


SETTLE_S = 0.3  # untimed running before the warmup steps: the clock ramps up over ~0.1 s


def settle(plan, args, seconds=SETTLE_S):
    """Run the hot path untimed for `seconds`: straight after setup (host-side input
    generation leaves the GPU idle) the first ~0.1 s run at a lower clock, which measured
    7% (8192^3) to 20% (short workloads) below the steady rate."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            plan.run(*args)
        torch.cuda.synchronize()


def time_plan(plan, args, steps, warmup, settle_s=0.0):
    import torch
    stream = torch.cuda.current_stream()
    if settle_s > 0:
        settle(plan, args, settle_s)
    for _ in range(warmup):
        plan.run(*args)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        plan.run(*args)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per launch


def mfma_ceiling(dtype, peak, reps=3):
    """The MFMA rate probe (gemm_epilogue_persistent_amd.measure): pure MFMA loops on uniform
    [-1, 1) operands held in registers, one workgroup per CU (4 waves; 8 for the 16x16 forms),
    no memory traffic. Returns the sustained rate and the shader clock it ran at (cycles over
    the 100 MHz real-time counter)."""
    import statistics
    import torch
    from gemm_epilogue_persistent_amd.measure import probe_mfma
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")
    iters = 10000 if dtype.startswith("e4m3") else 20000
    # FLOPs per wave per iteration, waves per workgroup
    if dtype == "bf16_16x16":
        flop_iter, waves = 32 * 2 * 16 * 16 * 32, 8
    elif dtype == "e4m3_16x16":
        flop_iter, waves = 32 * 2 * 16 * 16 * 128, 8
    else:
        flop_iter, waves = 16 * 2 * 32 * 32 * (16 if dtype == "bf16" else 64), 4
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        probe_mfma(dtype, iters, 1111, cus, out)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        h = out.view(cus, 2).cpu().tolist()
        mhz = statistics.median(c / (r / 100.0) for c, r in h if r > 0)
        tflops = flop_iter * iters * waves * cus / (ms * 1e-3) / 1e12
        if best is None or tflops > best["tflops"]:
            best = {"tflops": round(tflops, 1), "clock_mhz": round(mhz), "frac_of_peak": round(tflops / peak, 4)}
    return best


def cpu_baseline(inp, budget_s=15.0):
    """The oracle, as is, on whole output rows of the workload (bounded sample)."""
    import numpy as np
    import oracle
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    prob = oracle.problem_from(inp)
    codes = (W.codes_of(inp.A), W.codes_of(inp.B), W.codes_of(inp.C) if inp.C is not None else None)
    # calibrate on one row per thread, then size the sample to the budget
    rows = np.stack([np.zeros(cores, np.int64), np.arange(cores, dtype=np.int64) * 7 % inp.M], 1)
    t0 = time.perf_counter()
    prob.rows(*codes, rows, nthreads=cores)
    t1 = time.perf_counter() - t0
    nrows = max(cores, int(cores * budget_s / max(t1, 1e-3)) // cores * cores)
    rows = np.stack([np.zeros(nrows, np.int64), (np.arange(nrows, dtype=np.int64) * 1031) % inp.M], 1)
    t0 = time.perf_counter()
    prob.rows(*codes, rows, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = 2.0 * nrows * inp.N * inp.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{nrows} whole output rows of {inp.name} ({nrows * inp.N} outputs, "
                      f"{flops / 1e9:.1f} GFLOP) in {dt:.1f} s, fp64 k-ascending dot products"}


def traffic_for(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/gemm_persistent_kernel_<workload>_traffic.md), if it was taken on the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"gemm_persistent_kernel_{name}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if " = " in line:
            k, v = line.split(" = ", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_hash") != source_hash():
        return None
    return int(rec["hbm_bytes_per_launch"])


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=PRIMARY)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA rate probe")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cold", type=int, default=0, metavar="N",
                    help="rotate N copies of the primary workload's inputs (cold MALL / L2); 0: warm")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (reference for traffic counters)")
    a = ap.parse_args()
    if a.copy_calibration:
        import torch
        n = a.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the GEMM shards without communication; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    inp, plan, args = setup(a.workload)
    tm, tn, G, xcd, T, P = plan.grid()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    if a.cold > 1:
        timed = _Rotating(plan, cold_sets(args, a.cold))
        ms = time_plan(timed, args, a.steps, a.warmup, SETTLE_S)
        del timed
    else:
        ms = time_plan(plan, args, a.steps, a.warmup, SETTLE_S)
    flops = inp.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    progress(f"{a.workload}: {ms * 1e3:.1f} us per step, {tflops:.1f} TFLOP/s")
    peak = PEAK_TFLOPS[inp.a_dt]
    traffic = traffic_for(a.workload)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4), "traffic": traffic,
            "kernel": "gemm_persistent_kernel", "algorithmic_bytes": algorithmic_bytes(inp),
            "hbm_gbs_algorithmic": round(algorithmic_bytes(inp) / (ms * 1e-3) / 1e9, 1),
            "attainable_us": round(attainable_s(inp) * 1e6, 1),
            "frac_of_attainable": round(attainable_s(inp) / (ms * 1e-3), 4)}
    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": inp.a_dt, "data": "synthetic",
           "config": {"workload": inp.name, "M": inp.M, "N": inp.N, "K": inp.K, "L": inp.L,
                      "tile": [tm, tn], "group_m": G, "xcd_remap": xcd,
                      "raster": "n" if plan.raster_along_n() else "m", "tiles": T, "grid": P,
                      "settle_s": SETTLE_S, "cold_sets": max(a.cold, 0) if a.cold > 1 else 0,
                      "pct_of_peak": round(100 * tflops / peak, 2)},
           "roofline": roof}
    del args, plan
    if not a.no_ceiling:
        # the practical MFMA ceiling on full-entropy data at the clock the part sustains
        ceil = {d: mfma_ceiling(d, PEAK_TFLOPS["e4m3" if d.startswith("e4m3") else "bf16"])
                for d in ("bf16", "bf16_16x16", "e4m3", "e4m3_16x16")}
        progress(f"MFMA ceiling probe: {ceil['bf16']['tflops']} (bf16 32x32), {ceil['bf16_16x16']['tflops']} "
                 f"(bf16 16x16), {ceil['e4m3']['tflops']} (fp8 32x32), {ceil['e4m3_16x16']['tflops']} "
                 f"(fp8 16x16) TFLOP/s")
        out["mfma_ceiling"] = ceil
        # the form the workload's kernel issues: 16x16 in the 8-wave kernels (256x256 tiles,
        # both operands K-major), 32x32 elsewhere
        kmajor = inp.A.stride(-1) == 1 and inp.B.stride(-1) == 1
        w8 = tm == 256 and kmajor
        form = (("e4m3_16x16" if w8 else "e4m3") if inp.a_dt in ("e4m3", "e5m2")
                else ("bf16_16x16" if w8 else "bf16"))
        c = ceil[form]
        roof["mfma_form"] = form
        roof["frac_of_mfma_ceiling"] = round(tflops / c["tflops"], 4)
    if not a.no_secondary:
        sec = {}
        for name in SECONDARY:
            if name == a.workload:
                continue
            i2, p2, a2 = setup(name)
            ms2 = time_plan(p2, a2, max(10, a.steps // 3), max(2, a.warmup // 2), SETTLE_S)
            t2 = i2.flops() / (ms2 * 1e-3) / 1e12
            progress(f"{name}: {ms2 * 1e3:.1f} us per step, {t2:.1f} TFLOP/s")
            sec[name] = {"tflops": round(t2, 2), "ms": round(ms2, 4),
                         "pct_of_peak": round(100 * t2 / PEAK_TFLOPS[i2.a_dt], 2),
                         "peak": PEAK_TFLOPS[i2.a_dt], "dtype": i2.a_dt,
                         "frac_of_attainable": round(attainable_s(i2) / (ms2 * 1e-3), 4)}
            del p2, a2, i2
            torch.cuda.empty_cache()
        out["secondary"] = sec
    if not a.no_cpu_baseline:
        progress(f"CPU oracle on a sample of {a.workload} (~{a.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(inp, a.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
