"""Benchmark of the Uno block draft-and-verify hot path on one MI355X.

One step is one pass of the whole hot path over the Qwen3-8B-shaped workload
(64 sequences x block 16, vocabulary 151936, bf16): the row-gated LoRA linear on
the 4096->4096 and 4096->12288 projections over the block's 1024 rows (noise
rows = slots 1..15), then lossless verification of the block. The metric is
verified draft positions per second (S * b / step time). Inputs are synthetic
(seeded, see workloads.py) and resident in HBM before timing starts; draft tokens
come from the library's draft sampler before the timed region.

Also reported: per-kernel average durations from HIP events on the launch
stream, the roofline fraction of the dominant kernel, the TV loss kernel on the
self-distillation workload (8 x 4096 rows, vocabulary 151936) as a separate leg,
and the CPU oracle timed on a bounded sample of the same verify workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-tv]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-tv", action="store_true", help="skip the TV-loss leg")
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
    """Per-kernel HIP events on the current (launch) stream."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return out

    def avg_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(s.elapsed_time(e) for s, e in p) / max(1, len(p))

    def clear(self):
        self.pairs = {}


def verify_bytes(S, b, V, esize=2):
    # p rows for every slot, q rows for slots 1..b-1; plus drafts, ids, outputs
    return (S * b + S * (b - 1)) * V * esize + S * b * 4 * 2 + S * 16 + S * 8


def main():
    args = parse()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(run with --gpus 1)\n")
        sys.exit(2)

    import numpy as np
    import torch

    import lossless_diffusion_drafted_amd as uno
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    uno.load()
    sp = workloads.SAMPLING
    cfg = workloads.VERIFY_CONFIGS["qwen"]
    S, b, V = cfg["S"], cfg["b"], cfg["V"]

    # --- inputs resident in HBM -------------------------------------------------
    p_np, q_np = workloads.verify_logits("qwen")
    p, q = dev_tensor(p_np, dev), dev_tensor(q_np, dev)
    seq = dev_tensor(np.arange(S, dtype=np.int64), dev)
    pos = dev_tensor(np.zeros(S, dtype=np.int64), dev)
    draft, _ = uno.uno_draft_sample(q, seq, pos, **sp)
    outs = dict(out_tokens=torch.empty((S, b), dtype=torch.int32, device=dev),
                accept_len=torch.empty((S,), dtype=torch.int32, device=dev),
                resampled=torch.empty((S,), dtype=torch.int32, device=dev))

    gcfg = workloads.GEMM_CONFIGS["qwen"]
    M, r = gcfg["M"], gcfg["r"]
    mask = dev_tensor(workloads.noise_row_mask(S, b), dev)
    gemms = []
    for gi, (name, K, N) in enumerate(gcfg["projections"]):
        X, W, A, B = workloads.gemm_inputs(M, K, N, r, tag=gi)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gemms.append((name, K, N, dev_tensor(X, dev), dev_tensor(W, dev), dev_tensor(A, dev),
                      dev_tensor(B, dev), Y))
    gemm_ok = True
    try:
        g = gemms[0]
        uno.uno_gated_lora_linear(g[3], g[4], g[5], g[6], mask, 1.0, out=g[7])
    except uno.UnoError as e:
        if e.status != "UNO_ERR_UNSUPPORTED":
            raise
        gemm_ok = False
    torch.cuda.synchronize()

    timer = KernelTimer()

    def step():
        if gemm_ok:
            for (name, K, N, X, W, A, B, Y) in gemms:
                timer.run(f"gated_lora_{name}",
                          lambda X=X, W=W, A=A, B=B, Y=Y: uno.uno_gated_lora_linear(X, W, A, B, mask, 1.0, out=Y))
        timer.run("verify", lambda: uno.uno_verify_block(p, q, draft, seq, pos, want_slot_accept=False,
                                                          want_diag=False, out=outs, **sp))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    positions = S * b
    value = positions / (ms_per_step / 1000.0)

    kernels = {}
    vb = verify_bytes(S, b, V)
    t_ver = timer.avg_ms("verify")
    kernels["verify"] = dict(avg_us=t_ver * 1000, bytes=vb, GBps=vb / (t_ver * 1e6),
                             hbm_frac=vb / (t_ver * 1e6) / HBM_PEAK_GBS,
                             positions_per_s=positions / (t_ver / 1000))
    if gemm_ok:
        for (name, K, N, *_rest) in gemms:
            t = timer.avg_ms(f"gated_lora_{name}")
            flops = 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * r * N
            kernels[f"gated_lora_{name}"] = dict(avg_us=t * 1000, flops=flops,
                                                 TFLOPs=flops / (t * 1e9),
                                                 mfma_frac=flops / (t * 1e9) / BF16_PEAK_TFLOPS)
    acc = outs["accept_len"].float()
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    if dominant == "verify":
        roof = dict(bound="hbm", achieved=kernels["verify"]["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=kernels["verify"]["hbm_frac"], traffic=None, kernel="verify")
    else:
        k = kernels[dominant]
        roof = dict(bound="mfma", achieved=k["TFLOPs"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=k["mfma_frac"], traffic=None, kernel=dominant)

    tv_leg = None
    if not args.no_tv:
        tv_leg = tv_benchmark(uno, workloads, dev, max(3, args.steps // 4))

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
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped verify step: 64 seq x block 16, V=151936 bf16 logits, "
                               "T=1.0 top-k 50 top-p 0.95; gated LoRA r=128 on 4096x4096 and "
                               "4096x12288 over 1024 rows" + ("" if gemm_ok else " (gated LoRA not built: verify only)"),
                   "S": S, "block": b, "vocab": V, "gemm_rows": M, "rank": r,
                   "step": (["gated_lora_attn_4096x4096", "gated_lora_mlp_4096x12288"] if gemm_ok else []) + ["verify"]},
        "roofline": roof,
        "kernels": kernels,
        "mean_accept_len": acc.mean().item(),
        "cpu_baseline": cpu,
    }
    if tv_leg is not None:
        line["tv_loss"] = tv_leg
    print(json.dumps(line))


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
    torch.cuda.synchronize()
    n_resp = int(mask.sum().item())
    timer = KernelTimer()
    for _ in range(iters):
        timer.run("tv", lambda: uno.uno_tv_loss_fwd_bwd(t, s, mask, c["temperature"], want_rows=False))
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
    return {"value": reps * S * b / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"full verify workload (64 x 16 slots, V=151936) x {reps} repeats, "
                      f"{el:.1f} s, single-threaded numpy fp64"}


if __name__ == "__main__":
    main()
