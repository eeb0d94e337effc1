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
rate is reported beside it, with the attainable rates measured in the same
run (a plain streaming read, a bf16 MFMA loop with the shader clock it
sustains, torch's GEMM on the fused shapes).  The CPU baseline is the fp64
oracle on the host's cores, on a bounded sample of every configuration.
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
                           "fused_bwd_n1,logits_small,logits_varlen",
                   help="rows beyond the hot path, timed after the steps (not part of a step)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="instead of the hot path, run a plain 1 GiB device copy 5 times "
                        "(reference for hardware traffic counters)")
    p.add_argument("--no-yardsticks", action="store_true",
                   help="skip the attainable-rate yardsticks (a plain streaming read, a bf16 "
                        "MFMA loop with its shader clock, torch's GEMM on the fused shapes)")
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


def _hip_clock_mhz(dev_index):
    """The device's peak shader clock (hipDeviceAttributeClockRate, kHz)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, dev_index) == 0:
            return v.value / 1000.0
    except OSError:
        pass
    return None


def measure_yardsticks(torch, dev, read_buf, write_buf=None):
    """Attainable rates on this device, as yardsticks for the roofline
    fractions (comparison only: nothing of the library runs here).
      stream_read    a plain 16-byte nontemporal read of ``read_buf``
                     (yardstick/yardstick.hip), GB/s;
      stream_widen   ``read_buf``'s bf16 elements written as fp32 into
                     ``write_buf`` (read 2, write 4 bytes per element), GB/s
                     of bytes read + written;
      mfma_loop      back-to-back bf16 MFMAs on registers, TFLOP/s, and the
                     shader clock it sustains (s_memtime against the 100 MHz
                     real-time counter), MHz;
      gemm           torch's bf16 GEMM (hipBLASLt) on the two fused shapes,
                     fp32 output where torch offers it, and with bf16 output
                     and W as the row side (``bf16_out_w_rows``), TFLOP/s."""
    import ctypes

    import numpy as np
    out = {"clock_max_mhz": _hip_clock_mhz(dev.index or 0)}
    stream = torch.cuda.current_stream(dev)
    path = os.path.join(ROOT, "yardstick", "libyardstick.so")

    def ev_ms(fn, reps):
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

    if os.path.exists(path):
        ys = ctypes.CDLL(path)
        ys.yardstick_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
        ys.yardstick_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
        ys.yardstick_stream_widen.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_void_p]
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        nbytes = read_buf.numel() * read_buf.element_size()
        grid = cus * 16
        sink = torch.zeros(grid, dtype=torch.int32, device=dev)
        ms = ev_ms(lambda: ys.yardstick_stream_read(read_buf.data_ptr(), nbytes // 16, grid,
                                                    sink.data_ptr(), stream.cuda_stream), 5)
        out["stream_read"] = {"bytes": nbytes, "ms": ms, "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
        if write_buf is not None and read_buf.dtype == torch.bfloat16:
            n4 = min(read_buf.numel(), write_buf.numel()) // 4
            ms = ev_ms(lambda: ys.yardstick_stream_widen(read_buf.data_ptr(), n4, write_buf.data_ptr(),
                                                         stream.cuda_stream), 3)
            moved = n4 * 4 * (2 + 4)
            out["stream_widen"] = {"bytes": moved, "ms": ms, "GB_per_s": moved / (ms * 1e-3) / 1e9}
        mgrid, iters = 2 * cus, 20000
        clocks = torch.zeros(4 * mgrid, dtype=torch.int64, device=dev)
        msink = torch.zeros(mgrid * 256, dtype=torch.float32, device=dev)
        ms = ev_ms(lambda: ys.yardstick_mfma_loop(mgrid, iters, clocks.data_ptr(),
                                                  msink.data_ptr(), stream.cuda_stream), 3)
        c = clocks.view(mgrid, 4).cpu().numpy().astype(np.float64)
        mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1.0) * 100.0))
        flops = mgrid * 4 * 4 * iters * 32768.0
        out["mfma_loop"] = {"ms": ms, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                            "clock_mhz": mhz}
    else:
        out["missing"] = "yardstick/libyardstick.so not built"
    out["gemm"] = {}
    for n, v, h in ((8192, 128256, 4096), (2048, 151936, 5120)):
        g = torch.Generator(device=dev).manual_seed(7)
        a = torch.randn((n, h), generator=g, device=dev).to(torch.bfloat16)
        w = torch.randn((v, h), generator=g, device=dev).to(torch.bfloat16)
        try:
            fn = lambda: torch.mm(a, w.t(), out_dtype=torch.float32)
            fn()
            odt = "fp32"
        except (TypeError, RuntimeError):
            fn = lambda: a @ w.t()
            odt = "bf16"
        ms = ev_ms(fn, 3)
        rec = {"ms": ms, "out": odt, "TFLOP_per_s": 2.0 * n * v * h / (ms * 1e-3) / 1e12}
        # the same product with bf16 output and W as the row side (z^T = W h^T), the
        # fastest form hipBLASLt offers for these shapes: the least output traffic
        ms = ev_ms(lambda: w @ a.t(), 3)
        rec["bf16_out_w_rows"] = {"ms": ms, "TFLOP_per_s": 2.0 * n * v * h / (ms * 1e-3) / 1e12}
        out["gemm"][f"{n}x{v}x{h}"] = rec
        del a, w
    torch.cuda.synchronize()
    return out


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
    xexec = {}  # MFMA flops executed, where they differ from the algorithmic count
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
        # the MFMAs run each product twice, over D's bf16 parts D_hi and D_lo
        xexec["fused_param_grads"] = 5 * 2.0 * n5 * v5 * h5
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
            xexec["fused_param_grads_kept_logits"] = 4 * 2.0 * n5 * v5 * h5
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
        # one row of the fused forward workload: the row's reduction schedule
        # is that of any N (batches of at most 128 rows take a smaller launch),
        # and the W stream (V x H bf16) is the algorithmic traffic that bounds it
        h41, t41, m41 = c4.hidden[:1], c4.targets[:1], c4.mask[:1]
        lp41 = torch.empty(1, dtype=torch.float32, device=dev)
        ls41 = torch.empty(1, dtype=torch.float32, device=dev)
        xfns["fused_fwd_n1"] = (
            lambda: ilp.linear_logp(h41, c4.weight, t41, m41, workspace=ws4, logp=lp41, lse=ls41),
            v4 * h4 * 2 + h4 * 2 + 8 + 1 + 8)
    if c5 is not None and "fused_bwd_n1" in args.extra_legs.split(","):
        # one row of the fused backward workload (a decode step's gradient):
        # the W stream plus the row's V fp32 gradients
        h51, t51, m51, g51 = c5.hidden[:1], c5.targets[:1], c5.mask[:1], c5.grad[:1]
        ls51 = lse5[:1].clone()
        d51 = torch.empty((1, v5), dtype=torch.float32, device=dev)
        xfns["fused_bwd_n1"] = (
            lambda: ilp.linear_logp_backward(h51, c5.weight, t51, ls51, g51, m51, out=d51),
            v5 * h5 * 2 + h5 * 2 + 8 + 1 + 4 + 4 + v5 * 4)
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
            if name in xexec:
                te = xexec[name] / (xms * 1e-3) / 1e12
                extra[name].update({"executed_flops": xexec[name], "executed_TFLOP_per_s": te,
                                    "executed_mfma_frac": te / BF16_PEAK_TFLOPS})
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

    ys = None if args.no_yardsticks else measure_yardsticks(
        torch, dev, c3.logits, d3 if "logits_bwd" in legs else None)
    clock = None
    if ys is not None:
        clock = {"max_mhz": ys.get("clock_max_mhz"),
                 "under_mfma_load_mhz": ys.get("mfma_loop", {}).get("clock_mhz")}
        if roofline is not None and "stream_read" in ys and roofline["unit"] == "GB/s":
            att = ys["stream_read"]["GB_per_s"]
            roofline.update({"attainable": att, "attainable_kind": "plain streaming read",
                             "frac_attainable": roofline["achieved"] / att})
        if "stream_widen" in ys:
            # read-2 / write-4 bytes per element passes against the widening copy
            att = ys["stream_widen"]["GB_per_s"]
            for rec in (out_legs.get("logits_bwd"), extra.get("log_softmax")):
                if isinstance(rec, dict) and "GB_per_s" in rec:
                    rec["attainable_stream_widen"] = att
                    rec["frac_attainable_stream_widen"] = rec["GB_per_s"] / att
    fused_roof = None
    if "fused_fwd" in out_legs:
        tf = out_legs["fused_fwd"]["TFLOP_per_s"]
        fused_roof = {"kernel": "linear_tiles_fwd", "bound": "mfma", "achieved": tf,
                      "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                      "traffic": traffic.get("linear_tiles_fwd_8192x128256x4096"),
                      "traffic_unit": "bytes per launch"}
        if ys is not None:
            mhz = ys.get("mfma_loop", {}).get("clock_mhz")
            if mhz:
                fused_roof["peak_at_measured_clock"] = BF16_PEAK_TFLOPS * mhz / 2400.0
                fused_roof["frac_at_measured_clock"] = tf / fused_roof["peak_at_measured_clock"]
            if "mfma_loop" in ys:
                fused_roof["attainable_mfma_loop"] = ys["mfma_loop"]["TFLOP_per_s"]
                fused_roof["frac_attainable_mfma_loop"] = tf / ys["mfma_loop"]["TFLOP_per_s"]
            gemm = ys["gemm"].get("8192x128256x4096")
            if gemm:
                fused_roof["gemm_yardstick"] = gemm["TFLOP_per_s"]
                fused_roof["frac_gemm_yardstick"] = tf / gemm["TFLOP_per_s"]
                fused_roof["gemm_yardstick_bf16_out"] = gemm["bf16_out_w_rows"]["TFLOP_per_s"]
                fused_roof["frac_gemm_yardstick_bf16_out"] = tf / gemm["bf16_out_w_rows"]["TFLOP_per_s"]

    cpu = None
    if not args.no_cpu_baseline and "logits_fwd" in legs:
        cpu = cpu_baseline(torch, dev, c3)

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
        "fused_roofline": fused_roof,
        "clock": clock,
        "yardsticks": ys,
        "cpu_baseline": cpu,
        "build": ilp.build_info(),
        "device": _device_desc(torch, dev),
        "input_generation_s": t_gen,
    }
    print(json.dumps(rec))


def _host_cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(torch, dev, c3):
    """The fp64 oracle, as it stands, timed on the host's cores, one entry per
    configuration on a bounded sample of its workload (about 10-20 s of CPU
    work in all).  Row-wise oracle functions run over row blocks in a thread
    pool with one thread per CPU this process may use (rows are independent);
    the fused ones are called once on their sample, their fp64 products
    running on the BLAS library's threads (one per CPU).  Rates count the
    sample's active tokens, its algorithmic bytes (as the GPU legs count them)
    and, for the fused configurations, 2 N V H flops per projection."""
    import numpy as np

    import oracle
    from oracle.parallel import host_threads, map_row_blocks
    from invariant_logprob_amd import workloads as wl

    threads = host_threads()

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def pool(fn, n):
        return map_row_blocks(fn, n, block_rows=64, workers=threads)

    per = {}
    # N=8, V=1024: whole, repeated for a stable time
    b1 = wl.logits_small(seed=0, device=dev)
    x1, t1 = bits(b1.logits), b1.targets.cpu().numpy()
    oracle.logp_selected(x1, t1)
    reps = 200
    s = timed(lambda: [oracle.logp_selected(x1, t1) for _ in range(reps)]) / reps
    per["logits_small"] = {"sample": "all 8 rows (x200)", "s": s, "tokens_per_s": 8 / s,
                           "GB_per_s": 8 * 1024 * 2 / s / 1e9}
    # packed varlen batch, V=32000: every row
    b2 = wl.logits_varlen(seed=0, device=dev)
    x2, t2, m2 = bits(b2.logits), b2.targets.cpu().numpy(), b2.mask.cpu().numpy()
    n2 = x2.shape[0]
    a2 = int(m2.astype(bool).sum())
    pool(lambda r0, r1: oracle.logp_selected(x2[r0:r0 + 1], t2[r0:r0 + 1], m2[r0:r0 + 1]), 64)
    s = timed(lambda: pool(lambda r0, r1: oracle.logp_selected(x2[r0:r1], t2[r0:r1], m2[r0:r1]), n2))
    per["logits_varlen"] = {"sample": f"all {n2} rows ({a2} active)", "s": s,
                            "tokens_per_s": a2 / s, "GB_per_s": a2 * 32000 * 2 / s / 1e9}
    del x2
    # N=16384, V=151936: every row forward; the backward on 512 active rows
    x3, t3, m3 = bits(c3.logits), c3.targets.cpu().numpy(), c3.mask.cpu().numpy()
    n3, v3 = x3.shape
    a3 = int(m3.astype(bool).sum())
    s = timed(lambda: pool(lambda r0, r1: oracle.logp_selected(x3[r0:r1], t3[r0:r1], m3[r0:r1]), n3))
    per["logits_fwd"] = {"sample": f"all {n3} rows ({a3} active)", "s": s, "tokens_per_s": a3 / s,
                         "GB_per_s": a3 * v3 * 2 / s / 1e9}
    rows = np.nonzero(m3)[0][:512]
    xb, tb, gb = x3[rows], t3[rows], c3.grad.cpu().numpy()[rows]
    s = timed(lambda: pool(lambda r0, r1: oracle.logp_backward(xb[r0:r1], tb[r0:r1], None, None,
                                                               gb[r0:r1]), rows.size))
    per["logits_bwd"] = {"sample": "512 active rows (their own lse)", "s": s,
                         "tokens_per_s": rows.size / s,
                         "GB_per_s": rows.size * v3 * (2 + 4) / s / 1e9}
    del x3, xb
    # fused configurations: a 256-row forward and a 64-row backward sample
    for name, gen, nf, nb in (("fused_fwd", wl.fused_large, 256, 0),
                              ("fused_fb", wl.fused_bwd, 256, 64)):
        c = gen(seed=0, device=dev)
        hb, wb = bits(c.hidden[:nf]), bits(c.weight)
        t = c.targets[:nf].cpu().numpy()
        v, h = wb.shape
        s = timed(lambda: oracle.linear_logp(hb, wb, t))
        per[name] = {"sample": f"{nf} rows forward (the fp64 weight decoded in the call)", "s": s,
                     "tokens_per_s": nf / s, "GFLOP_per_s": 2.0 * nf * v * h / s / 1e9}
        if nb:
            g = c.grad[:nb].cpu().numpy()
            s = timed(lambda: oracle.linear_logp_backward(hb[:nb], wb, t[:nb], None, None, g))
            per[name + "_bwd"] = {"sample": f"{nb} rows backward (their own lse)", "s": s,
                                  "tokens_per_s": nb / s, "GFLOP_per_s": 2 * 2.0 * nb * v * h / s / 1e9}
        del c, hb, wb
    head = per["logits_fwd"]
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"selected logprob from bf16 logits N=16384 V=151936: {head['sample']}, "
                      f"{head['s']:.2f} s of numpy float64 oracle time on {threads} threads",
            "host_cpus": os.cpu_count(), "host_cpu_model": _host_cpu_model(),
            "blas_threads": os.environ.get("OMP_NUM_THREADS", "library default"),
            "per_config": per}


if __name__ == "__main__":
    main()
