"""Benchmark of the batch-invariant selected-token logprob hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over resident synthetic inputs:

  logits_fwd  selected logprob from bf16 logits, N=16384 rows (2458 masked),
              V=151936                                    (kernel logp_fwd_rows)
  logits_bwd  its backward, fp32 dlogits [16384, 151936]  (logp_bwd_rows)
  fused_fwd   lm_head + selected logprob, hidden [8192, 4096], W [128256, 4096]
                                                          (linear_tiles_fwd + lse_chunk_combine)
  fused_fb    fused forward + backward, hidden [2048, 5120], W [151936, 5120]
                                                          (linear_tiles_fwd, lse_chunk_combine,
                                                           linear_tiles_bwd)

The headline value is the selected-logprob throughput at V=151936: active
tokens per second of the logits forward.  Each leg is timed with HIP events
on the stream its kernels run on (torch's current stream), and every leg's
rate is reported beside it.  The CPU baseline is the fp64 oracle on a bounded
sample of the same logits workload.
"""

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "tokens/s + HBM GB/s, selected-logp V=152k; fused linear_logp TFLOP/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--legs", default="logits_fwd,logits_bwd,fused_fwd,fused_fb")
    p.add_argument("--extra-legs",
                   default="logits_entropy,log_softmax,token_losses,fused_param_grads,"
                           "fused_fb_kept_logits,fused_param_grads_kept_logits,fused_fwd_n1,"
                           "logits_small,logits_varlen",
                   help="rows beyond the hot path, timed after the steps (not part of a step)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="instead of the hot path, run a plain 1 GiB device copy 5 times "
                        "(reference for hardware traffic counters)")
    p.add_argument("--yardsticks", action="store_true",
                   help="instead of the hot path, time attainable-rate yardsticks with torch "
                        "kernels: a streaming read, a fill, and the bf16 GEMMs of the fused "
                        "shapes (comparison only; nothing of the library runs)")
    return p.parse_args()


def source_hash():
    """Hash of the kernel sources and the C header (identifies a kernel build)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "invariant_logprob_amd", "csrc", "*"))) + \
            [os.path.join(ROOT, "include", "rlk.h")]:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    {} when the kernels have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hot_path_kernels_hbm_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return {}
    if rec.get("source_hash") != source_hash():
        return {}
    return {k: v["read_bytes"] + v["write_bytes"] for k, v in rec.get("per_launch", {}).items()}


def _device_desc(torch, dev):
    """Name, architecture and size of the device (the marketing name can be
    empty on some driver stacks)."""
    p = torch.cuda.get_device_properties(dev)
    arch = getattr(p, "gcnArchName", "")
    return (f"{p.name or 'AMD GPU'} ({arch}, {p.multi_processor_count} CUs, "
            f"{p.total_memory / 2**30:.0f} GiB)")


def yardsticks(torch):
    """Attainable rates of torch's own kernels on the step's shapes, as a
    comparison for the library's roofline fractions (prints one JSON line)."""
    dev = torch.device("cuda:0")

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    x = torch.ones((16384, 151936), dtype=torch.bfloat16, device=dev)
    nbytes = x.numel() * 2
    ms = timed(lambda: torch.amax(x, dim=1))
    out["read_rowmax_bf16"] = {"ms": ms, "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
    y = torch.empty((16384, 151936), dtype=torch.float32, device=dev)
    ms = timed(lambda: y.fill_(1.0))
    out["fill_fp32"] = {"ms": ms, "GB_per_s": y.numel() * 4 / (ms * 1e-3) / 1e9}
    ms = timed(lambda: y.copy_(x))
    out["convert_bf16_to_fp32"] = {"ms": ms, "GB_per_s": (nbytes + y.numel() * 4) / (ms * 1e-3) / 1e9}
    del x, y
    for n, v, h in ((8192, 128256, 4096), (2048, 151936, 5120)):
        a = torch.randn((n, h), device=dev).to(torch.bfloat16)
        w = torch.randn((v, h), device=dev).to(torch.bfloat16)
        for odt in (torch.bfloat16, torch.float32):
            if odt == torch.float32:
                fn = lambda: torch.mm(a, w.t(), out_dtype=torch.float32)
                try:
                    fn()
                except (TypeError, RuntimeError):
                    continue
            else:
                fn = lambda: a @ w.t()
            ms = timed(fn, 5)
            out[f"gemm_{n}x{v}x{h}_{str(odt).split('.')[-1]}_out"] = {
                "ms": ms, "TFLOP_per_s": 2.0 * n * v * h / (ms * 1e-3) / 1e12}
        del a, w
    print(json.dumps({"yardsticks": out, "torch": torch.__version__}))


def calibrate_copy(torch):
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                      "bytes_written_per_copy": nbytes, "copies": 5}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path is data-parallel over rows and needs no "
              "collective; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.yardsticks:
        yardsticks(torch)
        return

    import invariant_logprob_amd as ilp
    from invariant_logprob_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ilp.load_library()
    legs = [l for l in args.legs.split(",") if l]
    t_gen = time.perf_counter()

    # ---- resident inputs and outputs ------------------------------------
    c3 = wl.logits_large(seed=0, device=dev)
    n3, v3 = c3.logits.shape
    act3 = int(c3.mask.sum())
    logp3 = torch.empty(n3, dtype=torch.float32, device=dev)
    lse3 = torch.empty(n3, dtype=torch.float32, device=dev)
    d3 = torch.empty((n3, v3), dtype=torch.float32, device=dev) if "logits_bwd" in legs else None
    c4 = wl.fused_large(seed=0, device=dev) if "fused_fwd" in legs else None
    c5 = wl.fused_bwd(seed=0, device=dev) if "fused_fb" in legs else None
    if c4 is not None:
        n4, h4 = c4.hidden.shape
        v4 = c4.weight.shape[0]
        ws4 = torch.empty(ilp.linear_logp_workspace_size(n4, v4, h4), dtype=torch.uint8, device=dev)
        logp4 = torch.empty(n4, dtype=torch.float32, device=dev)
        lse4 = torch.empty(n4, dtype=torch.float32, device=dev)
    if c5 is not None:
        n5, h5 = c5.hidden.shape
        v5 = c5.weight.shape[0]
        ws5 = torch.empty(ilp.linear_logp_workspace_size(n5, v5, h5), dtype=torch.uint8, device=dev)
        logp5 = torch.empty(n5, dtype=torch.float32, device=dev)
        lse5 = torch.empty(n5, dtype=torch.float32, device=dev)
        d5 = torch.empty((n5, v5), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    def leg_logits_fwd():
        ilp.logp_selected(c3.logits, c3.targets, c3.mask, logp=logp3, lse=lse3)

    def leg_logits_bwd():
        ilp.logp_backward(c3.logits, c3.targets, lse3, c3.grad, c3.mask, out=d3)

    def leg_fused_fwd():
        ilp.linear_logp(c4.hidden, c4.weight, c4.targets, c4.mask, workspace=ws4, logp=logp4,
                        lse=lse4)

    def leg_fused_fb():
        ilp.linear_logp(c5.hidden, c5.weight, c5.targets, c5.mask, workspace=ws5, logp=logp5,
                        lse=lse5)
        ilp.linear_logp_backward(c5.hidden, c5.weight, c5.targets, lse5, c5.grad, c5.mask, out=d5)

    fns = {"logits_fwd": leg_logits_fwd, "logits_bwd": leg_logits_bwd,
           "fused_fwd": leg_fused_fwd, "fused_fb": leg_fused_fb}
    if "logits_bwd" in legs and "logits_fwd" not in legs:
        leg_logits_fwd()   # the backward needs lse

    for _ in range(args.warmup):
        for l in legs:
            fns[l]()
    torch.cuda.synchronize()

    events = {l: [] for l in legs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for l in legs:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fns[l]()
            e1.record()
            events[l].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {l: sum(a.elapsed_time(b) for a, b in events[l]) / args.steps for l in legs}
    # per-launch spread of each leg over the timed steps: median, min, p90
    spread = {}
    for l in legs:
        ts = sorted(a.elapsed_time(b) for a, b in events[l])
        spread[l] = {"ms_median": ts[len(ts) // 2], "ms_min": ts[0],
                     "ms_p90": ts[min(len(ts) - 1, int(0.9 * len(ts)))]}
    ms_per_step = wall * 1e3 / args.steps

    out_legs = {}
    roofline = None
    traffic = measured_traffic()
    if "logits_fwd" in legs:
        bytes_fwd = act3 * v3 * 2 + n3 * (8 + 1 + 8)
        gbs = bytes_fwd / (ms["logits_fwd"] * 1e-3) / 1e9
        out_legs["logits_fwd"] = {"ms": ms["logits_fwd"], "active_tokens": act3,
                                  "tokens_per_s": act3 / (ms["logits_fwd"] * 1e-3),
                                  "algorithmic_bytes": bytes_fwd, "GB_per_s": gbs,
                                  "hbm_frac": gbs / HBM_PEAK_GBS}
        roofline = {"kernel": "logp_fwd_rows", "bound": "hbm", "achieved": gbs,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                    "traffic": traffic.get("logp_fwd_rows"), "traffic_unit": "bytes per launch",
                    "algorithmic_bytes": bytes_fwd}
    if "logits_bwd" in legs:
        bytes_bwd = act3 * v3 * 2 + n3 * v3 * 4 + n3 * (8 + 1 + 4 + 4)
        gbs = bytes_bwd / (ms["logits_bwd"] * 1e-3) / 1e9
        out_legs["logits_bwd"] = {"ms": ms["logits_bwd"], "algorithmic_bytes": bytes_bwd,
                                  "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    if "fused_fwd" in legs:
        fl = 2.0 * n4 * v4 * h4
        tf = fl / (ms["fused_fwd"] * 1e-3) / 1e12
        out_legs["fused_fwd"] = {"ms": ms["fused_fwd"], "flops": fl, "TFLOP_per_s": tf,
                                 "mfma_frac": tf / BF16_PEAK_TFLOPS,
                                 "tokens_per_s": n4 / (ms["fused_fwd"] * 1e-3)}
    if "fused_fb" in legs:
        fl = 2 * 2.0 * n5 * v5 * h5
        tf = fl / (ms["fused_fb"] * 1e-3) / 1e12
        out_legs["fused_fb"] = {"ms": ms["fused_fb"], "flops": fl, "TFLOP_per_s": tf,
                                "mfma_frac": tf / BF16_PEAK_TFLOPS,
                                "dlogits_bytes": n5 * v5 * 4}
    if roofline is None and "fused_fwd" in legs:
        f = out_legs["fused_fwd"]
        roofline = {"kernel": "linear_tiles_fwd", "bound": "mfma", "achieved": f["TFLOP_per_s"],
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": f["mfma_frac"],
                    "traffic": None}

    # rows beyond the hot path, on the same logits workload, timed separately
    extra = {}
    ent3 = torch.empty(n3, dtype=torch.float32, device=dev)
    xfns = {
        "logits_entropy": (lambda: ilp.logp_entropy(c3.logits, c3.targets, c3.mask, logp=logp3,
                                                    lse=lse3, entropy=ent3),
                           act3 * v3 * 2 + n3 * (8 + 1 + 12)),
    }
    g5 = torch.Generator(device=dev).manual_seed(5)
    old3 = logp3 + 0.2 * torch.randn(n3, generator=g5, device=dev)
    ref3 = logp3 + 0.2 * torch.randn(n3, generator=g5, device=dev)
    adv3 = torch.randn(n3, generator=g5, device=dev)
    xfns["token_losses"] = (lambda: ilp.token_losses(logp3, old3, adv3, c3.mask, ref3, 0.2, 0.28,
                                                     0.04), n3 * (5 * 4 + 1 + 4 * 4))
    if d3 is not None:
        xfns["log_softmax"] = (lambda: ilp.log_softmax(c3.logits, lse3, c3.mask, out=d3),
                               act3 * v3 * 2 + n3 * v3 * 4 + n3 * 5)
    xflops = {}
    if c5 is not None and "fused_param_grads" in args.extra_legs.split(","):
        # parameter gradients of the fused path on the fwd+bwd workload: the
        # logits recompute plus the two products, 3 x 2 N V H flops
        gh5 = torch.empty((n5, h5), dtype=torch.float32, device=dev)
        gw5 = torch.empty((v5, h5), dtype=torch.float32, device=dev)
        wsg5 = torch.empty(ilp.linear_logp_param_grads_workspace_size(n5, v5, h5),
                           dtype=torch.uint8, device=dev)
        xfns["fused_param_grads"] = (
            lambda: ilp.linear_logp_param_grads(c5.hidden, c5.weight, c5.targets, lse5, c5.grad,
                                                c5.mask, grad_hidden=gh5, grad_weight=gw5,
                                                workspace=wsg5),
            n5 * h5 * 2 + v5 * h5 * 2 + n5 * h5 * 4 + v5 * h5 * 4)
        xflops["fused_param_grads"] = 3 * 2.0 * n5 * v5 * h5
        if "fused_param_grads_kept_logits" in args.extra_legs.split(","):
            # the same gradients from logits the forward kept (computed once,
            # outside the timing): the two products only, 2 x 2 N V H flops
            zk5 = torch.empty((n5, v5), dtype=torch.float32, device=dev)
            ilp.linear_logp_with_logits(c5.hidden, c5.weight, c5.targets, c5.mask, workspace=ws5,
                                        logp=logp5, lse=lse5, logits=zk5)
            xfns["fused_param_grads_kept_logits"] = (
                lambda: ilp.linear_logp_param_grads(c5.hidden, c5.weight, c5.targets, lse5,
                                                    c5.grad, c5.mask, grad_hidden=gh5,
                                                    grad_weight=gw5, workspace=wsg5, logits=zk5),
                n5 * h5 * 2 + v5 * h5 * 2 + n5 * v5 * 4 + n5 * h5 * 4 + v5 * h5 * 4)
            xflops["fused_param_grads_kept_logits"] = 2 * 2.0 * n5 * v5 * h5
    if c5 is not None and "fused_fb_kept_logits" in args.extra_legs.split(","):
        # the fwd+bwd workload with the forward keeping its fp32 logits and the
        # backward computed from them in place (one projection, 2 N V H flops)
        def kept():
            ilp.linear_logp_with_logits(c5.hidden, c5.weight, c5.targets, c5.mask, workspace=ws5,
                                        logp=logp5, lse=lse5, logits=d5)
            ilp.logp_backward(d5, c5.targets, lse5, c5.grad, c5.mask, out=d5)
        xfns["fused_fb_kept_logits"] = (kept, n5 * h5 * 2 + v5 * h5 * 2 + 2 * n5 * v5 * 4 * 2)
        xflops["fused_fb_kept_logits"] = 2.0 * n5 * v5 * h5
    if c4 is not None and "fused_fwd_n1" in args.extra_legs.split(","):
        # one row of the fused forward workload: the kernel and schedule are
        # those of any N, and the W stream (V x H bf16) is the algorithmic
        # traffic that bounds it
        h41, t41, m41 = c4.hidden[:1], c4.targets[:1], c4.mask[:1]
        lp41 = torch.empty(1, dtype=torch.float32, device=dev)
        ls41 = torch.empty(1, dtype=torch.float32, device=dev)
        xfns["fused_fwd_n1"] = (
            lambda: ilp.linear_logp(h41, c4.weight, t41, m41, workspace=ws4, logp=lp41, lse=ls41),
            v4 * h4 * 2 + h4 * 2 + 8 + 1 + 8)
    for name in [x for x in args.extra_legs.split(",") if x in xfns]:
        fn, nbytes = xfns[name]
        for _ in range(max(1, args.warmup)):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        xms = e0.elapsed_time(e1) / args.steps
        xgbs = nbytes / (xms * 1e-3) / 1e9
        if name in xflops:
            tf = xflops[name] / (xms * 1e-3) / 1e12
            extra[name] = {"ms": xms, "flops": xflops[name], "TFLOP_per_s": tf,
                           "mfma_frac": tf / BF16_PEAK_TFLOPS}
        else:
            extra[name] = {"ms": xms, "algorithmic_bytes": nbytes, "GB_per_s": xgbs,
                           "hbm_frac": xgbs / HBM_PEAK_GBS}

    # the two small logits configurations, per launch: N=8, V=1024 (latency)
    # and 8 varlen sequences packed to N~4096, V=32000.  Warm: 20 launches
    # queued back to back between one pair of events, averaged.  Cold: the
    # median of 20 launches, each queued behind a 512 MB read that evicts the
    # inputs from the MALL (a read leaves clean lines, so no write-back of the
    # flush competes with the timed launch; the read keeps the GPU busy, so no
    # submission gap is timed either).
    small = [x for x in ("logits_small", "logits_varlen") if x in args.extra_legs.split(",")]
    if small:
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        for name in small:
            cb = (wl.logits_small if name == "logits_small" else wl.logits_varlen)(seed=0, device=dev)
            nb_, vb_ = cb.logits.shape
            actb = int(cb.mask.sum())
            lpb = torch.empty(nb_, dtype=torch.float32, device=dev)
            lsb = torch.empty(nb_, dtype=torch.float32, device=dev)
            fn = (lambda cb=cb, lpb=lpb, lsb=lsb:
                  ilp.logp_selected(cb.logits, cb.targets, cb.mask, logp=lpb, lse=lsb))
            times = {}
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            e1.synchronize()
            times["warm"] = e0.elapsed_time(e1) / 20
            ts = []
            for _ in range(20):
                flush.max()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            times["cold"] = sorted(ts)[len(ts) // 2]
            nbytes = actb * vb_ * 2 + nb_ * (8 + 1 + 8)
            gbs = nbytes / (times["cold"] * 1e-3) / 1e9
            extra[name] = {"ms": times["warm"], "cold_ms": times["cold"], "rows": nb_,
                           "active_rows": actb, "V": vb_, "algorithmic_bytes": nbytes,
                           "GB_per_s_cold": gbs, "hbm_frac_cold": gbs / HBM_PEAK_GBS}
        del flush

    cpu = None
    if not args.no_cpu_baseline and "logits_fwd" in legs:
        cpu = cpu_baseline(c3, torch)

    for l in out_legs:
        out_legs[l].update(spread.get(l, {}))
    value = out_legs["logits_fwd"]["tokens_per_s"] if "logits_fwd" in legs else None
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "selected logprob from bf16 logits N=16384 (2458 masked) V=151936; "
                        "fused lm_head N=8192 H=4096 V=128256; fused fwd+bwd N=2048 H=5120 "
                        "V=151936",
            "legs": legs,
            "global_batch": n3,
            "seed": 0,
            "parallelism": "none (1 GPU)",
        },
        "legs": out_legs,
        "extra_legs": extra,
        "roofline": roofline,
        "fused_roofline": ({"kernel": "linear_tiles_fwd", "bound": "mfma",
                            "achieved": out_legs["fused_fwd"]["TFLOP_per_s"],
                            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": out_legs["fused_fwd"]["mfma_frac"],
                            "traffic": traffic.get("linear_tiles_fwd_8192x128256x4096"),
                            "traffic_unit": "bytes per launch"}
                           if "fused_fwd" in out_legs else None),
        "cpu_baseline": cpu,
        "build": ilp.build_info(),
        "device": _device_desc(torch, dev),
        "input_generation_s": t_gen,
    }
    print(json.dumps(rec))


def cpu_baseline(c3, torch, budget_s=15.0, block=256):
    """The fp64 oracle, as it stands, on a bounded sample of the same logits
    workload: consecutive 256-row blocks from the first row until about
    ``budget_s`` seconds of CPU work; tokens/s over the sample's active rows."""
    import numpy as np

    import oracle
    n = c3.logits.shape[0]
    done_rows = 0
    active = 0
    spent = 0.0
    while done_rows < n and spent < budget_s:
        r1 = min(n, done_rows + block)
        bits = c3.logits[done_rows:r1].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        t = c3.targets[done_rows:r1].cpu().numpy()
        m = c3.mask[done_rows:r1].cpu().numpy()
        t0 = time.perf_counter()
        oracle.logp_selected(bits, t, m)
        spent += time.perf_counter() - t0
        active += int(m.astype(bool).sum())
        done_rows = r1
    return {"value": active / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done_rows} rows ({active} active) of the N=16384 V=151936 logits "
                      f"workload, {spent:.1f} s of oracle time (numpy float64, one thread)",
            "host_cpus": os.cpu_count(), "host": platform.processor() or platform.machine()}


if __name__ == "__main__":
    main()
