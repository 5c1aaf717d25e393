"""Benchmark of the Uno block draft-and-verify hot path on one MI355X.

One step is one pass of the whole hot path over the Qwen3-8B-shaped workload
(64 sequences x block 16, vocabulary 151936, bf16): the row-gated LoRA linear on
the 4096->4096 and 4096->12288 projections over the block's 1024 rows (noise
rows = slots 1..15), then lossless verification of the block. The metric is
verified draft positions per second (S * b / step time). Inputs are synthetic
(seeded, see workloads.py) and resident in HBM before timing starts; draft tokens
come from the library's draft sampler before the timed region.

Also reported: per-kernel average durations from HIP events on the launch
stream (back-to-back calls) and medians of single calls after a 512 MB cache flush,
the roofline fraction of the dominant kernel, near-tie counts of the verify
decisions, the TV loss kernel on the self-distillation workload (8 x 4096 rows,
vocabulary 151936) as a separate leg, verification alone at block 16 and block 8
with sampled and greedy decoding, the gated-LoRA backward on both projections, the
looped-model (64 x 8, V = 166144; seven rank-64 projections at M = 512) and
large-batch stress (256 x 16; seven rank-128 projections at M = 4096) workloads
with their HBM and MFMA fractions, the tiny workload's latencies, the decode step
on full-size synthetic stacks (Qwen3-8B shapes and the looped 3B-class stack, 4
sequences: AR step against Uno step, eager and as a HIP graph, and the looped
stack's one-loop draft), a plain copy's bandwidth, and the CPU oracle timed on a
bounded sample of the verify workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-tv] [--no-sweep]
                       [--no-legs] [--no-step]

Counter runs (rocprofv3 --pmc) time one kernel alone:
  python bench.py --only {verify,gemm_attn,gemm_mlp,tv,copy} --steps K
where `copy` is a plain 1 GiB elementwise copy (torch.neg) that calibrates the
FETCH_SIZE / WRITE_SIZE counters. `--summarize-pmc DIR --kernel NAME` turns the
four counter CSVs of such runs (DIR/{fetch,write,copy_fetch,copy_write}) into the
text summary profiles/NAME_traffic.md, which the benchmark line then reads for
its `traffic` figure as long as the kernel's source is unchanged.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
COPY_BYTES = 1 << 30            # size of the calibration copy

# Device functions launched by each timed entry point: the traffic summary counts
# only these (a counter run also holds the setup's other kernels, such as the draft
# sampler that makes the verifier's draft tokens).
KERNEL_FUNCTIONS = {
    "verify": ("verify_kernel",),
    "gated_lora_attn_4096x4096": ("gemm_kernel", "lora_down_kernel", "skinny_kernel", "skinny2_kernel"),
    "gated_lora_mlp_4096x12288": ("gemm_kernel", "lora_down_kernel", "skinny_kernel", "skinny2_kernel"),
    "tv": ("tv_kernel", "tv_pipe_kernel", "tv_count_kernel"),
}

# Source file of each timed entry point (the traffic summary is tied to its hash).
KERNEL_SOURCES = {
    "verify": "lossless_diffusion_drafted_amd/csrc/verify.hip",
    "gated_lora_attn_4096x4096": "lossless_diffusion_drafted_amd/csrc/gemm.hip",
    "gated_lora_mlp_4096x12288": "lossless_diffusion_drafted_amd/csrc/gemm.hip",
    "tv": "lossless_diffusion_drafted_amd/csrc/tv.hip",
}
ONLY = {"verify": "verify", "gemm_attn": "gated_lora_attn_4096x4096",
        "gemm_mlp": "gated_lora_mlp_4096x12288", "tv": "tv"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-tv", action="store_true", help="skip the TV-loss leg")
    ap.add_argument("--no-step", action="store_true",
                    help="skip the decode-step leg (full-size synthetic stacks, AR vs Uno step)")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the looped, stress and tiny workload legs")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the verify block-size / greedy sweep and the gated-LoRA backward leg")
    ap.add_argument("--only", choices=sorted(list(ONLY) + ["copy"]),
                    help="run one kernel alone (for counter runs) and print its timing")
    ap.add_argument("--summarize-pmc", metavar="DIR", help="write profiles/KERNEL_traffic.md from counter CSVs")
    ap.add_argument("--kernel", help="timed entry point the counter CSVs belong to (with --summarize-pmc)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("CSV", "NAME", "COMMAND"),
                    help="write profiles/NAME_kernel_trace.md from a rocprofv3 kernel_trace.csv made by COMMAND")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="run the step back to back this long before the warm-up steps (clock ramp)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="minimum CPU time spent on the oracle sample")
    return ap.parse_args()


def dev_tensor(a, device):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


class KernelTimer:
    """HIP events on the current (launch) stream around a run of n back-to-back calls
    of one entry point; the average is the steady-state time per call (an event pair
    around every single call would add the gap before each launch to it)."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn, n=1):
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        out = None
        for _ in range(n):
            out = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e, n))
        return out

    def avg_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(s.elapsed_time(e) for s, e, _ in p) / max(1, sum(n for _, _, n in p))

    def clear(self):
        self.pairs = {}


def settle(fn, ms=30.0):
    """Run fn back to back for about ms milliseconds: the measurement that follows
    sees the clock of a busy GPU (from idle the clock takes about 25 ms to ramp)."""
    import torch
    t_end = time.perf_counter() + ms / 1000.0
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def median_us_flushed(fn, n, flush):
    """Median time of n single calls, each with its own HIP event pair on the launch
    stream, after a write of the whole `flush` buffer (512 MB: larger than L2 and the
    256 MB MALL together) so that every call starts with cold caches."""
    import statistics
    import torch
    times = []
    for _ in range(n):
        flush.zero_()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        times.append((s, e))
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in times) * 1000.0


def near_tie_counts(diag, accept_len, b):
    """Slots whose decision either side may take differently in fp32 and fp64 (the HIP
    verifier flags |u - p~/q~| < 1e-6, a top-p boundary within 1e-6 of top_p, or an
    inverse-CDF draw within 1e-6 Z of a boundary), over all slots and over the
    decisive ones (slot 0, the kept slots and the first rejected slot)."""
    import torch
    flags = diag[..., 3].to(torch.int64)
    tie = (flags & 15) != 0
    slot = torch.arange(b, device=diag.device).unsqueeze(0)
    decisive = slot <= torch.clamp(accept_len.to(torch.int64), max=b - 1).unsqueeze(1)
    return {"slots": int(tie.sum().item()), "decisive_slots": int((tie & decisive).sum().item()),
            "of_slots": int(tie.numel())}


def copy_bandwidth(dev, iters=20):
    """Read+write rate of a plain 1 GiB elementwise copy (torch.neg), as context for
    the HBM roofline."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    t = KernelTimer()
    t.run("copy", lambda: torch.neg(src, out=dst), iters)
    torch.cuda.synchronize()
    ms = t.avg_ms("copy")
    del src, dst
    return 2.0 * COPY_BYTES / (ms * 1e6)


def gemm_bytes(M, N, K, r):
    # X, W, A, B read once, Y written once, the row mask read once
    return 2.0 * (M * K + N * K + r * K + N * r + M * N) + M


def verify_bytes(S, b, V, esize=2):
    # p rows for every slot, q rows for slots 1..b-1; plus drafts, ids, outputs
    return (S * b + S * (b - 1)) * V * esize + S * b * 4 * 2 + S * 16 + S * 8


def source_sha256(name):
    path = os.path.join(ROOT, KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profile(name):
    """HBM bytes per call from profiles/NAME_traffic.md, or None when the summary is
    missing or was taken on a different version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                vals[k.strip("`")] = v.strip().strip("`")
    if vals.get("source_sha256") != source_sha256(name):
        return None
    try:
        return float(vals["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def setup_verify(uno, workloads, dev):
    import numpy as np
    import torch
    sp = workloads.SAMPLING
    cfg = workloads.VERIFY_CONFIGS["qwen"]
    S, b = cfg["S"], cfg["b"]
    p_np, q_np = workloads.verify_logits("qwen")
    p, q = dev_tensor(p_np, dev), dev_tensor(q_np, dev)
    seq = dev_tensor(np.arange(S, dtype=np.int64), dev)
    pos = dev_tensor(np.zeros(S, dtype=np.int64), dev)
    draft, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    outs = dict(out_tokens=torch.empty((S, b), dtype=torch.int32, device=dev),
                accept_len=torch.empty((S,), dtype=torch.int32, device=dev),
                resampled=torch.empty((S,), dtype=torch.int32, device=dev))

    def run():
        return uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False, want_diag=False,
                                    out=outs, **sp)
    return run, outs, (p_np, q_np), (p, q, draft, seq, pos)


def setup_gemms(uno, workloads, dev):
    import torch
    gcfg = workloads.GEMM_CONFIGS["qwen"]
    M, r = gcfg["M"], gcfg["r"]
    mask = dev_tensor(workloads.noise_row_mask(M // gcfg["b"], gcfg["b"]), dev)
    runs = {}
    for gi, (name, K, N) in enumerate(gcfg["projections"]):
        X, W, A, B = workloads.gemm_inputs(M, K, N, r, tag=gi)
        X, W, A, B = (dev_tensor(a, dev) for a in (X, W, A, B))
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        runs[f"gated_lora_{name}"] = (
            lambda X=X, W=W, A=A, B=B, Y=Y: uno.uno_gated_lora_linear(X, W, A, B, mask, 1.0, out=Y),
            2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * r * N)
    return runs


def run_only(args, uno, workloads, dev):
    """One kernel alone, for counter runs: prints its average time per call."""
    import torch
    timer = KernelTimer()
    if args.only == "copy":
        # an elementwise kernel that reads and writes COPY_BYTES once each
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: torch.neg(src, out=dst)
    elif args.only == "verify":
        fn, _, _, _ = setup_verify(uno, workloads, dev)
    elif args.only == "tv":
        c = workloads.TV_CONFIG
        R, V = c["n_seq"] * c["seq_len"], c["V"]
        t, s = workloads.tv_inputs_torch(R, V, dev)
        mask = torch.from_numpy(workloads.tv_response_mask(c["n_seq"], c["seq_len"], c["resp_len"])).to(dev)
        fn = lambda: uno.uno_tv_loss_fwd_bwd(t, s, mask, c["temperature"], want_rows=False)
    else:
        fn = setup_gemms(uno, workloads, dev)[ONLY[args.only]][0]
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    timer.run(args.only, fn, args.steps)
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "calls": args.steps, "avg_us": timer.avg_ms(args.only) * 1000}))


def summarize_pmc(directory, name):
    """profiles/NAME_traffic.md from four counter runs under DIRECTORY: the kernel's
    FETCH_SIZE and WRITE_SIZE runs (pmc_ONLY/fetch, pmc_ONLY/write) and the copy's
    (pmc_copy/copy_fetch, pmc_copy/copy_write), each a rocprofv3 --pmc CSV."""
    only = [k for k, v in ONLY.items() if v == name][0]

    def function_of(kname):
        # "void uno::(anonymous namespace)::verify_kernel<unsigned short, true>(uno::VerifyArgs)"
        head = kname.split("(uno::")[0] if "(uno::" in kname else kname
        return head.replace("void ", "").replace("uno::(anonymous namespace)::", "").replace("uno::", "")

    def per_call(sub, counter, copy):
        files = glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(directory, sub)}")
        total, dispatches, kernels = 0.0, set(), {}
        for fpath in files:
            with open(fpath) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    kname = row.get("Kernel_Name", "")
                    if copy != ("uno::" not in kname):
                        continue
                    if copy and "neg" not in kname:
                        continue
                    v = float(row["Counter_Value"])
                    short = function_of(kname)
                    kernels[short] = kernels.get(short, 0.0) + v
                    if not copy and not any(short.startswith(fn) for fn in KERNEL_FUNCTIONS[name]):
                        continue                # a setup kernel of the run, not the timed entry point
                    total += v
                    dispatches.add(row.get("Dispatch_Id"))
        return total, len(dispatches), kernels

    calls = int(os.environ.get("PMC_CALLS", "0"))
    if calls <= 0:
        raise SystemExit("set PMC_CALLS to the number of timed calls in the kernel runs (warmup + steps)")
    copy_calls = int(os.environ.get("PMC_COPY_CALLS", str(calls)))
    f_kib, f_n, f_k = per_call(f"pmc_{only}/fetch", "FETCH_SIZE", False)
    w_kib, w_n, w_k = per_call(f"pmc_{only}/write", "WRITE_SIZE", False)
    cf_kib, _, _ = per_call("pmc_copy/copy_fetch", "FETCH_SIZE", True)
    cw_kib, _, _ = per_call("pmc_copy/copy_write", "WRITE_SIZE", True)
    # bytes per KiB-count, from the copy of known size (each copy reads and writes COPY_BYTES)
    f_scale = COPY_BYTES * copy_calls / cf_kib
    w_scale = COPY_BYTES * copy_calls / cw_kib
    fetch = f_kib * f_scale / calls
    write = w_kib * w_scale / calls
    out = os.path.join(ROOT, "profiles", f"{name}_traffic.md")
    with open(out, "w") as f:
        f.write(f"# HBM traffic of `{name}` (rocprofv3 counters)\n\n")
        f.write("Commands (from the repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first,\n"
                "R = the repository path):\n\n")
        for sub, ctr, what in (("fetch", "FETCH_SIZE", only), ("write", "WRITE_SIZE", only),
                               ("copy_fetch", "FETCH_SIZE", "copy"), ("copy_write", "WRITE_SIZE", "copy")):
            f.write(f"    timeout -s KILL 120 rocprofv3 --pmc {ctr} --output-format csv "
                    f"-d $R/gpurun_out/pmc_{what}/{sub} -o {sub} -- "
                    f"python3 $R/bench.py --only {what} --steps {calls - 1 if what != 'copy' else copy_calls - 1} "
                    f"--warmup 1\n")
        f.write(f"    PMC_CALLS={calls} PMC_COPY_CALLS={copy_calls} python3 bench.py --summarize-pmc gpurun_out "
                f"--kernel {name}\n\n")
        f.write("Counters are summed over the dispatches of the entry point's own kernels "
                f"({', '.join(KERNEL_FUNCTIONS[name])}) and divided by\n"
                "the number of calls; the run's setup kernels are listed below but not counted. The KiB\n"
                "counts are scaled by the copy calibration: a plain elementwise copy (torch.neg) of\n"
                f"{COPY_BYTES} B reads and writes exactly that many bytes.\n\n")
        f.write(f"- source: `{KERNEL_SOURCES[name]}`\n")
        f.write(f"- source_sha256: `{source_sha256(name)}`\n")
        f.write(f"- calls: {calls}\n")
        f.write(f"- fetch_kib_per_call: {f_kib / calls:.1f}\n")
        f.write(f"- write_kib_per_call: {w_kib / calls:.1f}\n")
        f.write(f"- copy_fetch_kib_per_copy: {cf_kib / copy_calls:.1f}\n")
        f.write(f"- copy_write_kib_per_copy: {cw_kib / copy_calls:.1f}\n")
        f.write(f"- fetch_scale_bytes_per_kib: {f_scale:.2f}\n")
        f.write(f"- write_scale_bytes_per_kib: {w_scale:.2f}\n")
        f.write(f"- hbm_fetch_bytes_per_call: {fetch:.0f}\n")
        f.write(f"- hbm_write_bytes_per_call: {write:.0f}\n")
        f.write(f"- hbm_bytes_per_call: {fetch + write:.0f}\n\n")
        f.write("Every kernel of the runs, FETCH_SIZE / WRITE_SIZE (KiB per timed call):\n\n")
        for k in sorted(set(f_k) | set(w_k)):
            f.write(f"    {k}: fetch {f_k.get(k, 0.0) / calls:.1f}  write {w_k.get(k, 0.0) / calls:.1f}\n")
    print(out)


def summarize_trace(csv_path, name, command):
    """profiles/NAME_kernel_trace.md from a rocprofv3 --kernel-trace CSV: per kernel and
    grid, the dispatch count and the mean, median, min and max duration."""
    import statistics
    groups = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            kname = row["Kernel_Name"]
            if "uno::" not in kname:
                continue                        # PyTorch's kernels that make the inputs
            head = kname.split("(uno::")[0] if "(uno::" in kname else kname
            short = head.replace("void ", "").replace("uno::(anonymous namespace)::", "").replace("uno::", "")
            wgs = int(row["Grid_Size_X"]) // max(1, int(row["Workgroup_Size_X"]))
            key = (short, f"{wgs} x {row['Grid_Size_Y']}")
            groups.setdefault(key, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"{name}_kernel_trace.md")
    with open(out, "w") as f:
        f.write(f"# Kernel durations: {name} (rocprofv3 kernel trace)\n\n")
        f.write("Command (repository root R on the GPU box; `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        f.write(f"    {command}\n")
        f.write(f"    python3 bench.py --summarize-trace <kernel_trace.csv> {name} '<the command above>'\n\n")
        f.write("Library kernels only (PyTorch's input generation left out), by kernel and grid\n"
                "(workgroups x grid y); durations in microseconds.\n\n")
        f.write("| Kernel | Grid | Dispatches | Mean | Median | Min | Max |\n|---|---|---|---|---|---|---|\n")
        for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            f.write(f"| `{k}` | {g} | {len(v)} | {statistics.fmean(v):.1f} | {statistics.median(v):.1f} | "
                    f"{min(v):.1f} | {max(v):.1f} |\n")
    print(out)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_pmc:
        if args.kernel not in KERNEL_SOURCES:
            raise SystemExit(f"--kernel must be one of {sorted(KERNEL_SOURCES)}")
        summarize_pmc(args.summarize_pmc, args.kernel)
        return
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(run with --gpus 1)\n")
        sys.exit(2)

    import torch

    import lossless_diffusion_drafted_amd as uno
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    uno.load()
    if args.only:
        run_only(args, uno, workloads, dev)
        return

    sp = workloads.SAMPLING
    cfg = workloads.VERIFY_CONFIGS["qwen"]
    S, b, V = cfg["S"], cfg["b"], cfg["V"]
    gcfg = workloads.GEMM_CONFIGS["qwen"]
    M, r = gcfg["M"], gcfg["r"]

    # --- inputs resident in HBM -------------------------------------------------
    verify_run, outs, (p_np, q_np), verify_inputs = setup_verify(uno, workloads, dev)
    gemms = setup_gemms(uno, workloads, dev)
    torch.cuda.synchronize()

    timer = KernelTimer()

    def step():
        for fn, _ in gemms.values():
            fn()
        verify_run()

    # Clock settle: from an idle GPU the first steps run slow while the clock
    # ramps (measured: 453 us per step over the first 10 steps, 297 us by the
    # 30th, 270 us from about 25 ms on). The step runs back to back for
    # --settle-ms before the warm-up steps, so the timed steps see the clock of a
    # GPU kept busy, as in a serving loop. Reported in the JSON line.
    settle_steps = 0
    t_settle = time.perf_counter() + args.settle_ms / 1000.0
    while time.perf_counter() < t_settle:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        settle_steps += 20
    # Headline: the step as a caller runs it, timed only at its boundaries (events
    # between the calls would each add a fence to the stream).
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    positions = S * b
    value = positions / (ms_per_step / 1000.0)
    # Per-call durations: each entry point of the step run args.steps times back to
    # back between one pair of HIP events.
    for name, (fn, _) in gemms.items():
        timer.run(name, fn, args.steps)
    timer.run("verify", verify_run, args.steps)
    torch.cuda.synchronize()

    kernels = {}
    vb = verify_bytes(S, b, V)
    t_ver = timer.avg_ms("verify")
    kernels["verify"] = dict(avg_us=t_ver * 1000, bytes=vb, GBps=vb / (t_ver * 1e6),
                             hbm_frac=vb / (t_ver * 1e6) / HBM_PEAK_GBS,
                             positions_per_s=positions / (t_ver / 1000))
    for name, (_, flops) in gemms.items():
        t = timer.avg_ms(name)
        kernels[name] = dict(avg_us=t * 1000, flops=flops, TFLOPs=flops / (t * 1e9),
                             mfma_frac=flops / (t * 1e9) / BF16_PEAK_TFLOPS)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    kernels["verify"]["median_us_flushed"] = median_us_flushed(verify_run, 100, flush)
    for name, (fn, _) in gemms.items():
        kernels[name]["median_us_flushed"] = median_us_flushed(fn, 100, flush)
    acc = outs["accept_len"].float()
    diag_run = uno.uno_verify_block(*verify_inputs, want_slot_accept=False, want_diag=True, **sp)
    ties = near_tie_counts(diag_run["diag"], diag_run["accept_len"], b)
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    traffic = traffic_from_profile(dominant)
    if dominant == "verify":
        roof = dict(bound="hbm", achieved=kernels["verify"]["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=kernels["verify"]["hbm_frac"], traffic=traffic, kernel="verify")
    else:
        k = kernels[dominant]
        roof = dict(bound="mfma", achieved=k["TFLOPs"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=k["mfma_frac"], traffic=traffic, kernel=dominant)

    bwd = None
    if not args.no_sweep:
        bwd = lora_bwd_benchmark(uno, workloads, dev, max(10, args.steps))

    sweep = None
    if not args.no_sweep:
        sweep = verify_sweep(uno, workloads, p_np, q_np, dev, max(10, args.steps))

    tv_leg = None
    if not args.no_tv:
        tv_leg = tv_benchmark(uno, workloads, dev, max(10, args.steps // 4))

    legs = None
    if not args.no_legs:
        legs = {"looped": workload_leg(uno, workloads, "looped", dev, max(10, args.steps), flush),
                "stress": workload_leg(uno, workloads, "stress", dev, max(10, args.steps), flush),
                "tiny": tiny_leg(uno, workloads, dev, max(10, args.steps))}
    del flush
    steps_leg = None
    if not args.no_step:
        steps_leg = step_leg(uno, workloads, dev, max(5, args.steps // 10))
    copy_gbps = copy_bandwidth(dev)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(p_np, q_np, sp, S, b, args.cpu_seconds)

    line = {
        "metric": "verified draft positions/sec at Qwen3-8B shape (B=64, block 16); HBM % / MFMA %",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped verify step: 64 seq x block 16, V=151936 bf16 logits, "
                               "T=1.0 top-k 50 top-p 0.95; gated LoRA r=128 on 4096x4096 and "
                               "4096x12288 over 1024 rows",
                   "S": S, "block": b, "vocab": V, "gemm_rows": M, "rank": r,
                   "step": list(gemms) + ["verify"]},
        "roofline": roof,
        "kernels": kernels,
        "mean_accept_len": acc.mean().item(),
        "near_ties": ties,
        "copy_GBps": copy_gbps,
        "cpu_baseline": cpu,
    }
    if legs is not None:
        line["workloads"] = legs
    if steps_leg is not None:
        line["decode_step"] = steps_leg
    if sweep is not None:
        line["verify_sweep"] = sweep
    if bwd is not None:
        line["gated_lora_bwd"] = bwd
    if tv_leg is not None:
        line["tv_loss"] = tv_leg
    print(json.dumps(line), flush=True)
    release(uno, dev)


def release(uno, dev):
    """Free every device buffer and the library's cached workspaces, then wait for the
    device, before the interpreter's own teardown: objects that outlive main() would
    otherwise be released by garbage collection at exit, after a profiler attached to
    the process may already have finalised."""
    import gc
    import torch
    from lossless_diffusion_drafted_amd import _lib
    torch.cuda.synchronize(dev)
    _lib.WORKSPACES._bufs.clear()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize(dev)


def tv_benchmark(uno, workloads, dev, iters):
    import torch
    c = workloads.TV_CONFIG
    R, V = c["n_seq"] * c["seq_len"], c["V"]
    try:
        t, s = workloads.tv_inputs_torch(R, V, dev)
        mask = torch.from_numpy(workloads.tv_response_mask(c["n_seq"], c["seq_len"], c["resp_len"])).to(dev)
        loss, rows, grad = uno.uno_tv_loss_fwd_bwd(t, s, mask, c["temperature"], want_rows=False)
    except uno.UnoError as e:
        if e.status != "UNO_ERR_UNSUPPORTED":
            raise
        return {"status": "not built"}
    settle(lambda: uno.uno_tv_loss_fwd_bwd(t, s, mask, c["temperature"], want_rows=False), 40.0)
    n_resp = int(mask.sum().item())
    timer = KernelTimer()
    timer.run("tv", lambda: uno.uno_tv_loss_fwd_bwd(t, s, mask, c["temperature"], want_rows=False), iters)
    torch.cuda.synchronize()
    ms = timer.avg_ms("tv")
    # teacher + student rows of response rows read once; gradient written for every row
    byts = 2 * n_resp * V * 2 + R * V * 2 + R
    out = dict(workload="self-distillation 8 x 4096 rows (3072 response), V=151936 bf16",
               avg_us=ms * 1000, bytes=byts, GBps=byts / (ms * 1e6), hbm_frac=byts / (ms * 1e6) / HBM_PEAK_GBS,
               loss=loss.item())
    del t, s, grad
    torch.cuda.empty_cache()
    return out


def lora_bwd_benchmark(uno, workloads, dev, iters):
    """The gated-LoRA backward (dX, dA, dB) on both Qwen-shaped projections, with the
    frozen weight's transpose made once (and, for reference, made on every call)."""
    import torch
    gcfg = workloads.GEMM_CONFIGS["qwen"]
    M, r = gcfg["M"], gcfg["r"]
    mask = dev_tensor(workloads.noise_row_mask(M // gcfg["b"], gcfg["b"]), dev)
    out = {}
    for gi, (name, K, N) in enumerate(gcfg["projections"]):
        X, W, A, B = (dev_tensor(a, dev) for a in workloads.gemm_inputs(M, K, N, r, tag=gi))
        G = dev_tensor(workloads.gemm_grad(M, N, tag=gi), dev)
        Wt = W.t().contiguous()          # the frozen weight, transposed once (setup, not timed)
        f_w = lambda: uno.uno_gated_lora_linear_bwd(G, X, W, A, B, mask, 1.0)
        f_wt = lambda: uno.uno_gated_lora_linear_bwd(G, X, W, A, B, mask, 1.0, W_t=Wt)
        settle(f_w)
        timer = KernelTimer()
        timer.run("w", f_w, iters)
        settle(f_wt)
        timer.run("b", f_wt, iters)
        torch.cuda.synchronize()
        ms = timer.avg_ms("b")
        ms_w = timer.avg_ms("w")
        # dX = dY W + U A, U = dY B, T = X A^T, dA = U^T X, dB = dY^T T
        flops = 2.0 * M * N * K + 2.0 * M * r * K + 2.0 * M * N * r + 2.0 * M * K * r + 2.0 * r * M * K + \
            2.0 * N * M * r
        out[f"gated_lora_bwd_{name}"] = dict(avg_us=ms * 1000, flops=flops, TFLOPs=flops / (ms * 1e9),
                                                    mfma_frac=flops / (ms * 1e9) / BF16_PEAK_TFLOPS,
                                                    avg_us_transposing_W=ms_w * 1000)
        del X, W, A, B, G, Wt
    torch.cuda.empty_cache()
    return out


def verify_sweep(uno, workloads, p_np, q_np, dev, iters):
    """Verify at the metric's shape (64 sequences, V = 151936) for block 16 and block 8
    (the first 8 slots of each block) and for sampled (T = 1, top-k 50, top-p 0.95)
    and greedy (T = 0) decoding."""
    import numpy as np
    import torch
    S, V = p_np.shape[0], p_np.shape[2]
    seq = dev_tensor(np.arange(S, dtype=np.int64), dev)
    pos = dev_tensor(np.zeros(S, dtype=np.int64), dev)
    out = {}
    for b in (16, 8):
        p = dev_tensor(np.ascontiguousarray(p_np[:, :b]), dev)
        q = dev_tensor(np.ascontiguousarray(q_np[:, :b]), dev)
        for label, sp in (("sampled", workloads.SAMPLING), ("greedy", dict(workloads.SAMPLING, temperature=0.0))):
            draft, _ = uno.uno_draft_sample(q, seq, pos, **sp)
            outs = dict(out_tokens=torch.empty((S, b), dtype=torch.int32, device=dev),
                        accept_len=torch.empty((S,), dtype=torch.int32, device=dev),
                        resampled=torch.empty((S,), dtype=torch.int32, device=dev))
            fn = lambda: uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False, want_diag=False,
                                              out=outs, **sp)
            timer = KernelTimer()
            settle(fn)
            timer.run("v", fn, iters)
            torch.cuda.synchronize()
            ms = timer.avg_ms("v")
            byts = verify_bytes(S, b, V)
            out[f"b{b}_{label}"] = dict(avg_us=ms * 1000, positions_per_s=S * b / (ms / 1000),
                                        GBps=byts / (ms * 1e6), hbm_frac=byts / (ms * 1e6) / HBM_PEAK_GBS,
                                        mean_accept_len=outs["accept_len"].float().mean().item())
        del p, q
    torch.cuda.empty_cache()
    return out


def verify_leg(uno, workloads, name, dev, iters, flush):
    """uno_verify_block on a whole verify workload: time per call (back to back, and the
    median of single calls after a cache flush), HBM fraction, mean accept length and
    near-tie counts."""
    import numpy as np
    import torch
    sp = workloads.SAMPLING
    c = workloads.VERIFY_CONFIGS[name]
    S, b, V = c["S"], c["b"], c["V"]
    p_np, q_np = workloads.verify_logits(name)
    p, q = dev_tensor(p_np, dev), dev_tensor(q_np, dev)
    del p_np, q_np
    seq = dev_tensor(np.arange(S, dtype=np.int64), dev)
    pos = dev_tensor(np.zeros(S, dtype=np.int64), dev)
    draft, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    outs = dict(out_tokens=torch.empty((S, b), dtype=torch.int32, device=dev),
                accept_len=torch.empty((S,), dtype=torch.int32, device=dev),
                resampled=torch.empty((S,), dtype=torch.int32, device=dev))
    fn = lambda: uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False, want_diag=False,
                                      out=outs, **sp)
    settle(fn)
    timer = KernelTimer()
    timer.run("v", fn, iters)
    torch.cuda.synchronize()
    ms = timer.avg_ms("v")
    byts = verify_bytes(S, b, V)
    d = uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False, want_diag=True, **sp)
    out = dict(shape=f"{S} x {b} x {V} bf16", avg_us=ms * 1000,
               median_us_flushed=median_us_flushed(fn, 50, flush), bytes=byts,
               GBps=byts / (ms * 1e6), hbm_frac=byts / (ms * 1e6) / HBM_PEAK_GBS,
               positions_per_s=S * b / (ms / 1000), mean_accept_len=outs["accept_len"].float().mean().item(),
               near_ties=near_tie_counts(d["diag"], d["accept_len"], b))
    del p, q, d
    torch.cuda.empty_cache()
    return out


def gemm_leg(uno, workloads, name, dev, iters, flush):
    """The workload's gated-LoRA projections at full shape, each timed back to back and
    as the median of flushed single calls, with its MFMA and HBM fractions (the
    looped and stress shapes sit near the bf16 ridge, so both are reported)."""
    import torch
    gcfg = workloads.GEMM_CONFIGS[name]
    M, r = gcfg["M"], gcfg["r"]
    mask = dev_tensor(workloads.noise_row_mask(M // gcfg["b"], gcfg["b"]), dev)
    out, total_us, total_flops = {}, 0.0, 0.0
    for gi, (pname, K, N) in enumerate(gcfg["projections"]):
        X, W, A, B = (dev_tensor(a, dev) for a in workloads.gemm_inputs(M, K, N, r, tag=gi))
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fn = lambda: uno.uno_gated_lora_linear(X, W, A, B, mask, 1.0, out=Y)
        settle(fn)
        timer = KernelTimer()
        timer.run("g", fn, iters)
        torch.cuda.synchronize()
        ms = timer.avg_ms("g")
        flops = 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * r * N
        byts = gemm_bytes(M, N, K, r)
        out[pname] = dict(K=K, N=N, avg_us=ms * 1000, median_us_flushed=median_us_flushed(fn, 50, flush),
                          flops=flops, TFLOPs=flops / (ms * 1e9),
                          mfma_frac=flops / (ms * 1e9) / BF16_PEAK_TFLOPS, bytes=byts,
                          GBps=byts / (ms * 1e6), hbm_frac=byts / (ms * 1e6) / HBM_PEAK_GBS)
        total_us += ms * 1000
        total_flops += flops
        del X, W, A, B, Y
    torch.cuda.empty_cache()
    out["all_projections"] = dict(M=M, r=r, avg_us=total_us, TFLOPs=total_flops / (total_us * 1e6),
                                  mfma_frac=total_flops / (total_us * 1e6) / BF16_PEAK_TFLOPS)
    return out


def workload_leg(uno, workloads, name, dev, iters, flush):
    leg = {"verify": verify_leg(uno, workloads, name, dev, iters, flush),
           "gated_lora": gemm_leg(uno, workloads, name, dev, iters, flush)}
    if name == "looped":
        # every gated projection runs on each of 22 layers, twice (two loops) per forward
        leg["gated_lora"]["per_forward_us"] = 44 * leg["gated_lora"]["all_projections"]["avg_us"]
    return leg


def tiny_leg(uno, workloads, dev, iters):
    """Latency of each entry point on the tiny workload (one sequence, block 8, V = 1024
    fp32; an 8 x 256 -> 256 gated LoRA of rank 16): back-to-back calls, so the figure
    is launch and on-chip latency, not bandwidth."""
    import numpy as np
    import torch
    sp = workloads.SAMPLING
    p_np, q_np = workloads.verify_logits("tiny")
    S = p_np.shape[0]
    p, q = dev_tensor(p_np, dev), dev_tensor(q_np, dev)
    seq = dev_tensor(np.arange(S, dtype=np.int64), dev)
    pos = dev_tensor(np.zeros(S, dtype=np.int64), dev)
    draft, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    c = workloads.GEMM_CONFIGS["tiny"]
    (_, K, N), = c["projections"]
    X, W, A, B = (dev_tensor(a, dev) for a in workloads.gemm_inputs(c["M"], K, N, c["r"]))
    mask = dev_tensor(workloads.noise_row_mask(c["M"] // c["b"], c["b"]), dev)
    fns = {"verify": lambda: uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False,
                                                  want_diag=False, **sp),
           "draft_sample": lambda: uno.uno_draft_sample(q, seq, pos, want_flags=False, **sp),
           "gated_lora": lambda: uno.uno_gated_lora_linear(X, W, A, B, mask, 1.0)}
    out = {}
    for k, fn in fns.items():
        fn()
        torch.cuda.synchronize()
        timer = KernelTimer()
        timer.run(k, fn, iters)
        torch.cuda.synchronize()
        out[k] = dict(avg_us=timer.avg_ms(k) * 1000)
    return out


def _graph_ms(fn, iters):
    """Average time of `iters` replays of a HIP graph of one call of fn (workspaces
    are made by a warm-up call on the capture stream first)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    t = KernelTimer()
    t.run("g", g.replay, iters)
    torch.cuda.synchronize()
    ms = t.avg_ms("g")
    del g
    return ms


def step_leg(uno, workloads, dev, iters):
    """The decode step on full-size synthetic stacks at 4 sequences: an AR step (one
    frozen forward of 4 rows and the AR draw) against an Uno step (a gated draft
    forward of the 4 blocks, the draft sampler, a frozen verify forward, verify),
    eager (every kernel launched from the host per step) and replayed from a HIP
    graph. The looped stack also drafts with one loop instead of two. Weight bytes
    per forward: every projection and the LM head read once per loop."""
    import torch
    sp = workloads.SAMPLING
    out = {}
    for name in ("qwen", "looped"):
        c = workloads.STEP_CONFIGS[name]
        m = workloads.step_model_torch(name, dev)
        model = uno.Model(m["embed"], m["lm_head"], m["weights"], m["lora_a"], m["lora_b"], kv_width=c["kv_width"],
                          head_dim=c["head_dim"], lora_scale=m["lora_scale"])
        S, b, L, V, H = c["S"], c["b"], c["loops"], c["vocab"], c["hidden"]
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        seed_tok = torch.randint(0, V, (S,), generator=g, device=dev, dtype=torch.int32)
        seq = torch.arange(S, dtype=torch.int64, device=dev)
        pos = torch.full((S,), 100, dtype=torch.int64, device=dev)
        ar_out = {"out_tokens": torch.empty((S,), dtype=torch.int32, device=dev)}
        st_out = {k: torch.empty((S, b) if k in ("out_tokens", "draft_tokens") else (S,), dtype=torch.int32,
                                 device=dev) for k in ("out_tokens", "accept_len", "resampled", "draft_tokens")}
        variants = {"ar": lambda: uno.uno_ar_step(model, seed_tok, seq, pos, loops=L, out=ar_out, **sp),
                    "uno": lambda: uno.uno_decode_step(model, b, seed_tok, seq, pos, draft_loops=L,
                                                       verify_loops=L, out=st_out, **sp)}
        if L > 1:
            variants["uno_one_loop_draft"] = lambda: uno.uno_decode_step(model, b, seed_tok, seq, pos, draft_loops=1,
                                                                         verify_loops=L, out=st_out, **sp)
        res = {}
        for k, fn in variants.items():
            fn()
            torch.cuda.synchronize()
            t = KernelTimer()
            t.run(k, fn, iters)
            torch.cuda.synchronize()
            res[k] = dict(eager_ms=t.avg_ms(k), graph_ms=_graph_ms(fn, iters))
        per_layer = sum(o * i for o, i in workloads.step_proj_dims(c))
        wbytes = 2.0 * (L * c["layers"] * per_layer + V * H)
        ar_ms = res["ar"]["graph_ms"]
        leg = dict(shape=f"{c['layers']} layers x {L} loop(s), hidden {H}, FFN {c['ffn']}, V {V}, rank {c['rank']}, "
                         f"{S} sequences, block {b}",
                   weight_bytes_per_forward=wbytes, steps=res,
                   uno_over_ar_graph=res["uno"]["graph_ms"] / ar_ms,
                   uno_over_ar_eager=res["uno"]["eager_ms"] / res["ar"]["eager_ms"],
                   ar_forward_GBps=wbytes / (ar_ms * 1e6), ar_forward_hbm_frac=wbytes / (ar_ms * 1e6) / HBM_PEAK_GBS,
                   mean_accept_len=st_out["accept_len"].float().mean().item())
        if L > 1:
            leg["one_loop_draft_over_ar_graph"] = res["uno_one_loop_draft"]["graph_ms"] / ar_ms
        out[name] = leg
        del model, m
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def cpu_baseline(p_np, q_np, sp, S, b, min_seconds):
    """The fp64 CPU oracle on the same verify workload (the whole 64-sequence block,
    repeated until min_seconds of CPU time), in positions per second."""
    import numpy as np
    import oracle
    seq = np.arange(S, dtype=np.int64)
    pos = np.zeros(S, dtype=np.int64)
    d, _ = oracle.draft_sample(q_np, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], "bf16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.verify_block(p_np, q_np, d, seq, pos, sp["temperature"], sp["top_k"], sp["top_p"], sp["seed"], "bf16")
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    blas = None
    try:
        import threadpoolctl
        blas = [dict(api=i.get("internal_api"), threads=i.get("num_threads"))
                for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    except ImportError:
        pass
    return {"value": reps * S * b / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"full verify workload (64 x 16 slots, V=151936) x {reps} repeats, "
                      f"{el:.1f} s, single-threaded numpy fp64",
            "host_cpu_count": os.cpu_count(), "blas_threads": blas}


if __name__ == "__main__":
    main()
