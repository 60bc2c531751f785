"""Throughput of the FLUX-class VAE decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode1024|decode256]
                    [--no-cpu-baseline]

A step is one whole decode (conv_in ... conv_out, every kernel of the chain)
of a seeded synthetic latent, with seeded synthetic weights already packed on
the device and the latent already resident in HBM.  Default workload: latent
[16,128,128] -> RGB [3,1024,1024].  Prints ONE JSON line:

  value        the decode's direct-conv-equivalent rate: algorithmic FLOPs
               of the decode (2 Cin Cout k^2 H W per conv, no credit for the
               Winograd form's fewer multiplies, plus the attention's
               8 N c^2 + 4 N^2 c) / wall time per decode; `value_is` says so
  ms_per_step  wall time of one decode (HIP-event/host timing around K steps)
  roofline     the dominant kernel (largest share of device time) against the
               FP32 MFMA peak: `achieved` is the MFMA work it executes per
               launch (for the F(4x4) Winograd conv 36 of every 144
               direct-conv multiplies, 25 on a nearest-x2 input) / its average
               launch duration measured with HIP events on the decode stream;
               `direct_equivalent_tflops` is the direct-conv rate of the same
               launches
  cpu_baseline the float64 oracle timed on this host's cores on the whole
               256x256 decode (latent [16,32,32], the pages' render size),
               with the CPU model and thread count; `secondary_sample` times
               conv_in + the first mid resnet of the 1024x1024 decode
  secondary    the 256x256 decode (latent [16,32,32])
  tiled        the main latent decoded in 256-pixel tiles with overlaps of at
               least 64 (vae_decode_tiled), with its workspace beside the
               whole-image decode's
  sweep        the single-layer sweep at full size (3x3 and 1x1 convs,
               GroupNorm+SiLU) and a standalone nearest-x2 upsample
  stack3d      the causal 3-D conv stack on [128,17,256,256]
  decode3d     the causal 3-D decoder on a latent [16,17,32,32]
  measured_peaks  the GPU's own FP32 MFMA and HBM ceilings from the library's
               probes, and the roofline kernel's and the 3x3 convs' executed
               MFMA rates as fractions of the measured MFMA ceiling (the
               `roofline` object keeps the published peak)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import vaegen  # noqa: E402

PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
WORKLOADS = {"decode1024": 128, "decode256": 32}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the second decode size and the tiled decode (keeps profiler summaries to one workload)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the single-layer sweep")
    ap.add_argument("--no-3d", action="store_true", help="skip the causal 3-D stack and decode")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timings")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA and HBM ceilings")
    ap.add_argument("--conv3x3", default=None,
                    help="form of the 3x3 convs (winograd_2x2, implicit_gemm, winograd_4x4); default: the library's")
    ap.add_argument("--attention", default=None, choices=["split_softmax", "streaming"],
                    help="form of the decoder's mid-block attention; default: the library's")
    ap.add_argument("--layer-table", default=None,
                    help="write the timed decodes' per-layer average launch times (JSON) to this file")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the decodes, run one plain device copy of this many MiB "
                         "(reference dispatch for calibrating HBM byte counters)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "diffusion_vae_decoder_amd", "csrc")


CONV_SOURCES = {"conv3x3_wino4": "conv_wino4.hip", "conv3x3_wino": "conv_wino.hip", "conv3x3_mfma": "conv.hip"}


def conv_family(kernel: str) -> str:
    """'conv3x3_wino4', 'conv3x3_wino' or 'conv3x3_mfma' for the 3x3 conv kernels, else ''."""
    for f in CONV_SOURCES:
        if kernel.startswith(f + "<"):
            return f
    return ""


def is_conv3x3(kernel: str) -> bool:
    return conv_family(kernel) != ""


def mfma_fraction(kernel: str) -> float:
    """MFMA multiplies the kernel executes per direct-conv multiply: the
    Winograd F(2x2,3x3) form does 16 of 36 (9 of 36 on an upsampled input),
    F(4x4,3x3) 36 of 144 (25 of 144)."""
    fam = conv_family(kernel)
    if fam == "conv3x3_wino":
        return 9.0 / 36.0 if "up2x" in kernel else 16.0 / 36.0
    if fam == "conv3x3_wino4":
        return 25.0 / 144.0 if "up2x" in kernel else 36.0 / 144.0
    return 1.0


def form_fraction(form: str, upsample: bool = False) -> float:
    """mfma_fraction of the 3x3 conv kernels a form runs (the per-layer calls
    and decoders created under it)."""
    name = {"winograd_4x4": "conv3x3_wino4", "winograd_2x2": "conv3x3_wino"}.get(form, "conv3x3_mfma")
    return mfma_fraction(f"{name}<16,{'up2x' if upsample else 'plain'}>")


def conv_rates(recs) -> dict:
    """Direct-conv-equivalent and executed-MFMA rates of the 3x3 conv records."""
    conv = [r for r in recs if is_conv3x3(r["kernel"])]
    ms = sum(r["ms"] for r in conv)
    direct = sum(r["flops"] for r in conv)
    executed = sum(mfma_fraction(r["kernel"]) * r["flops"] for r in conv)
    return {"ms": ms, "direct_equivalent_tflops": direct / (ms / 1e3) / 1e12 if ms else 0.0,
            "mfma_executed_tflops": executed / (ms / 1e3) / 1e12 if ms else 0.0,
            "frac_fp32_mfma_peak": executed / (ms / 1e3) / 1e12 / PEAK_FP32_MFMA_TFLOPS if ms else 0.0}


def roofline(name: str, k: dict, steps: int, workload: str) -> dict:
    """The roofline object of kernel `name` from its records summed over the
    timed steps (k: ms, flops, bytes, n launches).  A contraction is placed
    against the FP32 MFMA peak with the MFMA work it executes (the Winograd
    forms run a fixed fraction of the direct conv's multiplies: that fraction
    of its FLOPs is the algorithm's own count); others against HBM bandwidth
    with their algorithmic bytes."""
    launch_ms = k["ms"] / k["n"]
    out = {"kernel": name, "launches_per_step": k["n"] // steps, "avg_launch_ms": launch_ms}
    if k["flops"] > 0:
        f = mfma_fraction(name)
        direct = k["flops"] / k["n"]
        achieved = f * direct / (launch_ms / 1e3) / 1e12
        out.update({"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / PEAK_FP32_MFMA_TFLOPS, "traffic": counter_traffic(name, workload),
                    "bound_is": "FP32 MFMA (v_mfma_f32_16x16x4_f32 / 32x32x2) on the products the kernel executes",
                    "flops_per_launch": f * direct, "direct_flops_per_launch": direct,
                    "executed_fraction_of_direct": f,
                    "direct_equivalent_tflops": direct / (launch_ms / 1e3) / 1e12,
                    "algorithmic_bytes_per_launch": k["bytes"] / k["n"]})
    else:
        achieved = k["bytes"] / k["n"] / (launch_ms / 1e3) / 1e9
        out.update({"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": None, "bytes_per_launch": k["bytes"] / k["n"]})
    return out


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when that summary was taken on another kernel,
    another workload, or a kernel source that has changed since."""
    fam = conv_family(kernel)
    if workload != "decode1024" or not fam:
        return None
    src_file = CONV_SOURCES[fam]
    try:
        text = open(os.path.join(ROOT, "profiles", f"{fam}_decode1024_hbm_counters.md")).read()
        src = open(os.path.join(CSRC, src_file), "rb").read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        key, _, val = line.partition(": ")
        if key in ("traffic_bytes_per_launch", "kernel", "kernel_source_sha256"):
            vals[key] = val.strip()
    if vals.get("kernel") != kernel or vals.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return float(vals["traffic_bytes_per_launch"])


def decode_flops(p: dict, h: int, w: int) -> float:
    """Algorithmic FLOPs of one decode of a latent [c, h, w] with the
    architecture in `p` (diffusers names): 2 Cin Cout k^2 H W per conv and
    8 N c^2 + 4 N^2 c for the attention over N = H W tokens."""
    fl = 0.0

    def conv(name, H, W):
        wt = p[name + ".weight"]
        k = wt.shape[-1] if wt.ndim == 4 else 1
        return 2.0 * wt.shape[0] * wt.shape[1] * k * k * H * W

    def resnet(name, H, W):
        f = conv(name + ".conv1", H, W) + conv(name + ".conv2", H, W)
        if name + ".conv_shortcut.weight" in p:
            f += conv(name + ".conv_shortcut", H, W)
        return f

    H, W = h, w
    fl += conv("conv_in", H, W) + resnet("mid_block.resnets.0", H, W) + resnet("mid_block.resnets.1", H, W)
    n, c = H * W, p["mid_block.attentions.0.to_q.weight"].shape[0]
    fl += 8.0 * n * c * c + 4.0 * n * n * c
    i = 0
    while f"up_blocks.{i}.resnets.0.conv1.weight" in p:
        j = 0
        while f"up_blocks.{i}.resnets.{j}.conv1.weight" in p:
            fl += resnet(f"up_blocks.{i}.resnets.{j}", H, W)
            j += 1
        if f"up_blocks.{i}.upsamplers.0.conv.weight" in p:
            H, W = 2 * H, 2 * W
            fl += conv(f"up_blocks.{i}.upsamplers.0.conv", H, W)
        i += 1
    return fl + conv("conv_out", H, W)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seed: int, h_sample: int) -> dict:
    """The oracle, untuned, timed on this host: the whole decode of a latent
    [16,32,32] (-> RGB [3,256,256], the pages' 256px render), then a bounded
    sample of the 1024x1024 decode (conv_in + the first mid-block resnet)."""
    import ctypes

    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-4, 0)
        libc.mallopt(-1, 1 << 30)
    except OSError:
        pass
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        blas_threads = os.cpu_count()
    p = vaegen.decoder_params(seed)
    z = vaegen.latent(seed, 32, 32)
    fl = decode_flops(p, 32, 32)
    times = []
    while sum(times) < 10.0:
        t = time.perf_counter()
        oracle.decode(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
        times.append(time.perf_counter() - t)
    dt = statistics.median(times)

    zs = vaegen.latent(seed, h_sample, h_sample)
    c = p["conv_in.weight"].shape[0]
    n = h_sample * h_sample
    sfl = 2.0 * c * 16 * 9 * n + 2 * (2.0 * c * c * 9 * n)   # conv_in + two 3x3 convs
    t = time.perf_counter()
    x = oracle.conv2d(oracle.denormalize(zs, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR),
                      p["conv_in.weight"], p["conv_in.bias"])
    oracle.resnet(x, p, "mid_block.resnets.0")
    sdt = time.perf_counter() - t
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "decode_ms": dt * 1e3, "decodes": len(times), "flops": fl, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"float64 oracle, whole decodes of latent [16,32,32] -> RGB [3,256,256] "
                      f"({fl / 1e9:.1f} GFLOP algorithmic each), repeated for >= 10 s, median; `cores` = "
                      f"the BLAS threads its matrix products used (its elementwise steps run on one thread)",
            "secondary_sample": {"value": sfl / sdt / 1e12, "unit": "TFLOP/s", "seconds": sdt,
                                 "sample": f"conv_in + mid_block.resnets.0 of the latent [16,{h_sample},"
                                           f"{h_sample}] decode ({sfl / 1e9:.1f} GFLOP)"}}


def sweep(args) -> dict:
    """The single-layer sweep at its full sizes through the per-layer entry
    points (each call includes its weight repack), plus a standalone nearest-x2
    upsample.  W warm-ups, then K timed calls bracketed by events."""
    import torch
    from diffusion_vae_decoder_amd import api

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    out = {}
    for cin, cout, k, h in [(512, 512, 3, 128), (256, 256, 3, 256), (128, 128, 3, 512), (256, 128, 3, 512),
                            (256, 128, 1, 512)]:
        x = torch.from_numpy(vaegen.activation(args.seed, f"sweep.x{cin}_{h}", (cin, h, h))).cuda()
        prm = vaegen.conv_params(args.seed, "sweep.c", cin, cout, k)
        w, b = (torch.from_numpy(prm["sweep.c." + n]).cuda() for n in ("weight", "bias"))
        y = torch.empty((cout, h, h), device="cuda")
        ms = timed(lambda: api.conv2d(x, w, b, out=y))
        fl = 2.0 * cin * cout * k * k * h * h
        f = form_fraction(api.get_conv3x3_algorithm()) if k == 3 else 1.0
        out[f"conv{k}x{k} {cin}->{cout} @{h}x{h}"] = {
            "ms": ms, "direct_equivalent_tflops": fl / ms / 1e9, "mfma_executed_tflops": f * fl / ms / 1e9,
            "frac_fp32_mfma_peak": f * fl / ms / 1e9 / PEAK_FP32_MFMA_TFLOPS}
        del x, y
    c, h = 128, 512
    x = torch.from_numpy(vaegen.activation(args.seed, "sweep.gn", (c, h, h))).cuda()
    nrm = vaegen.norm_params(args.seed, "sweep.n", c)
    g, bt = (torch.from_numpy(nrm["sweep.n." + n]).cuda() for n in ("weight", "bias"))
    y = torch.empty_like(x)
    ms = timed(lambda: api.groupnorm_silu(x, g, bt, out=y))
    by = 2.0 * c * h * h * 4
    out[f"groupnorm_silu [{c},{h},{h}]"] = {"ms": ms, "gbs": by / ms / 1e6, "frac_hbm": by / ms / 1e6 / PEAK_HBM_GBS,
                                            "note": "statistics pass + apply pass; 2 algorithmic units of traffic"}
    c, h = 256, 512
    x = torch.from_numpy(vaegen.activation(args.seed, "sweep.up", (c, h, h))).cuda()
    y = torch.empty((c, 2 * h, 2 * h), device="cuda")
    ms = timed(lambda: api.upsample_nearest2x(x, out=y))
    by = 5.0 * c * h * h * 4
    out[f"upsample_nearest2x [{c},{h},{h}]"] = {"ms": ms, "gbs": by / ms / 1e6, "frac_hbm": by / ms / 1e6 / PEAK_HBM_GBS}
    return out


def stack3d(args) -> dict:
    """The causal 3-D conv stack at full size: x [128,17,256,256], four
    (3x3x3 causal conv -> GroupNorm32+SiLU) layers with the residual added
    after every second layer, through vae_conv3d_causal_groupnorm_silu (the
    group statistics come from the conv's epilogue); the four convs are then
    timed alone through vae_conv3d_causal for their MFMA rate."""
    import torch
    from diffusion_vae_decoder_amd import api
    c, t, h = 128, 17, 256
    p = {k: torch.from_numpy(v).cuda() for k, v in vaegen.causal_stack_params(args.seed, c=c).items()}
    x0 = torch.from_numpy(vaegen.activation(args.seed, "stack3d.x", (c, t, h, h))).cuda()
    bufs = [torch.empty_like(x0) for _ in range(3)]

    def step():
        # x1 = x0 + L1(L0(x0)) in B, then x2 = x1 + L3(L2(x1)) in C; A holds the first layer of a pair
        A, B, C = bufs
        plan = [(x0, A, None, 0), (A, B, x0, 1), (B, A, None, 2), (A, C, B, 3)]
        for src, dst, res, j in plan:
            api.conv3d_causal_groupnorm_silu(src, p[f"stack.{j}.conv.weight"], p[f"stack.{j}.conv.bias"],
                                             p[f"stack.{j}.norm.weight"], p[f"stack.{j}.norm.bias"], residual=res,
                                             out=dst, out_norm=dst)
        return C

    def convs():
        A, B, C = bufs
        for j, (src, dst) in enumerate([(x0, A), (A, B), (B, A), (A, C)]):
            api.conv3d_causal(src, p[f"stack.{j}.conv.weight"], p[f"stack.{j}.conv.bias"], out=dst)

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms = timed(step)
    conv_ms = timed(convs)
    fl = 4 * 2.0 * c * c * 27 * t * h * h
    f = form_fraction(api.get_conv3x3_algorithm())
    gn_bytes = 4 * 2.0 * 4 * c * t * h * h + 2 * 4.0 * c * t * h * h   # 4 x (read + write), 2 residual reads
    return {"workload": f"causal 3-D conv stack, x [{c},{t},{h},{h}], 4 x (3x3x3 conv + GroupNorm32+SiLU)",
            "ms_per_step": ms, "direct_equivalent_tflops": fl / ms / 1e9, "conv_ms": conv_ms,
            "conv_direct_equivalent_tflops": fl / conv_ms / 1e9, "conv_mfma_executed_tflops": f * fl / conv_ms / 1e9,
            "conv_frac_fp32_mfma_peak": f * fl / conv_ms / 1e9 / PEAK_FP32_MFMA_TFLOPS,
            "groupnorm_ms_estimate": ms - conv_ms,
            "groupnorm_gbs_estimate": gn_bytes / max(ms - conv_ms, 1e-9) / 1e6,
            "note": "each call includes its weight repack; GroupNorm statistics from the conv epilogue; the "
                    "GroupNorm estimate is the stack's time minus its convs' time alone"}


def decode3d(args, t: int = 17, h: int = 32) -> dict:
    """The causal 3-D decoder on a latent [16, t, h, h] -> RGB [3, t, 8h, 8h]."""
    import torch
    from diffusion_vae_decoder_amd import api
    prm = vaegen.decoder_params(args.seed, dims=3)
    dec = api.Decoder({k: torch.from_numpy(v).cuda() for k, v in prm.items()}, vaegen.SCALING_FACTOR,
                      vaegen.SHIFT_FACTOR, causal3d=True)
    z = torch.from_numpy(vaegen.latent3d(args.seed, t, h, h)).cuda()
    rgb = torch.empty((3, t, 8 * h, 8 * h), device="cuda")
    for _ in range(max(args.warmup, 1)):
        dec.decode(z, out=rgb)
    dec.set_profiling(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.decode(z, out=rgb)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    recs = dec.profile()
    dec.set_profiling(False)
    dec.close()
    cr = conv_rates(recs)
    return {"workload": f"causal 3-D decode, latent [16,{t},{h},{h}] -> RGB [3,{t},{8 * h},{8 * h}]",
            "ms_per_step": ms,
            "direct_equivalent_tflops": sum(r["flops"] for r in recs) / args.steps / (ms / 1e3) / 1e12,
            "conv3x3x3_direct_equivalent_tflops": cr["direct_equivalent_tflops"],
            "conv3x3x3_mfma_executed_tflops": cr["mfma_executed_tflops"],
            "conv3x3x3_frac_fp32_mfma_peak": cr["frac_fp32_mfma_peak"]}


def graph_replay_ms(dec, z, steps: int, warmup: int) -> float:
    """Wall ms per decode with the decoder's HIP-graph replay on (no events)."""
    import torch
    out = torch.empty(dec.output_shape(z.shape[-2], z.shape[-1]), device="cuda") if z.dim() == 3 else None
    dec.set_graph(True)
    try:
        for _ in range(max(warmup, 1)):
            out = dec.decode(z, out=out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dec.decode(z, out=out)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps
    finally:
        dec.set_graph(False)


def latency(dec, z_dev, steps: int) -> dict:
    """Per-decode latency after the timed region: device time from a torch event
    pair around each decode on the current stream (the stream the decoder
    launches on; no per-launch events), and host-to-host time from a pinned host
    latent to a pinned host RGB (H2D copy, decode, D2H copy, synchronize).
    Median and min over `steps` decodes of each kind."""
    import torch
    c, hh, ww = z_dev.shape
    z_host = torch.empty((c, hh, ww), dtype=torch.float32, pin_memory=True)
    z_host.copy_(z_dev.cpu())
    zd = torch.empty_like(z_dev)
    rgb = torch.empty(dec.output_shape(hh, ww), dtype=torch.float32, device="cuda")
    rgb_host = torch.empty(rgb.shape, dtype=torch.float32, pin_memory=True)
    dec.decode(z_dev, out=rgb)
    torch.cuda.synchronize()
    dev = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dec.decode(z_dev, out=rgb)
        e1.record()
        e1.synchronize()
        dev.append(e0.elapsed_time(e1))
    h2h = []
    for _ in range(steps):
        t0 = time.perf_counter()
        zd.copy_(z_host, non_blocking=True)
        dec.decode(zd, out=rgb)
        rgb_host.copy_(rgb, non_blocking=True)
        torch.cuda.synchronize()
        h2h.append((time.perf_counter() - t0) * 1e3)
    return {"device_ms_median": statistics.median(dev), "device_ms_min": min(dev),
            "host_to_host_ms_median": statistics.median(h2h), "host_to_host_ms_min": min(h2h),
            "h2d_bytes": z_host.numel() * 4, "d2h_bytes": rgb_host.numel() * 4, "decodes": steps}


def secondary(dec, args, h2: int) -> dict:
    """W warm-ups then K timed decodes of a latent [16,h2,h2], per-launch events on."""
    import torch
    z2 = torch.from_numpy(vaegen.latent(args.seed, h2, h2)).cuda()
    for _ in range(max(args.warmup, 1)):
        dec.decode(z2)
    dec.set_profiling(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.decode(z2)
    torch.cuda.synchronize()
    ms2 = (time.perf_counter() - t0) * 1e3 / args.steps
    recs2 = dec.profile()
    dec.set_profiling(False)
    cr = conv_rates(recs2)
    return {"workload": f"decode latent [16,{h2},{h2}] -> RGB [3,{8 * h2},{8 * h2}]",
            "ms_per_step": ms2, "latency": latency(dec, z2, max(args.steps, 20)),
            "ms_per_step_graph_replay": None if args.no_graph else graph_replay_ms(dec, z2, args.steps, args.warmup),
            "direct_equivalent_tflops": sum(r["flops"] for r in recs2) / args.steps / (ms2 / 1e3) / 1e12,
            "conv3x3_ms_per_step": cr["ms"] / args.steps,
            "conv3x3_direct_equivalent_tflops": cr["direct_equivalent_tflops"],
            "conv3x3_mfma_executed_tflops": cr["mfma_executed_tflops"],
            "conv3x3_frac_fp32_mfma_peak": cr["frac_fp32_mfma_peak"]}


def tiled(dec, args, h: int, tile: int = 256, overlap: int = 64) -> dict:
    """The same latent decoded in tiles (vae_decode_tiled: the pages' 256-pixel
    tiles with overlaps of at least 64): W warm-ups, then K timed tiled decodes
    (events around the whole call on the current stream), and the workspace
    the tiled and the whole-image decode need."""
    import torch
    z = torch.from_numpy(vaegen.latent(args.seed, h, h)).cuda()
    rgb = torch.empty(dec.output_shape(h, h), dtype=torch.float32, device="cuda")
    for _ in range(max(args.warmup, 1)):
        dec.decode_tiled(z, tile, overlap, out=rgb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dec.decode_tiled(z, tile, overlap, out=rgb)
    e1.record()
    torch.cuda.synchronize()
    return {"workload": f"decode latent [16,{h},{h}] -> RGB [3,{8 * h},{8 * h}] in {tile}-pixel tiles, "
                        f"overlap >= {overlap}",
            "ms_per_step": e0.elapsed_time(e1) / args.steps,
            "workspace_bytes": dec.tiled_workspace_bytes(h, h, tile, overlap),
            "whole_image_workspace_bytes": dec.workspace_bytes(h, h)}


def measured_peaks(reps: int = 5) -> dict:
    """The GPU's own ceilings from the library's probes (vae_probe_mfma_f32,
    vae_probe_hbm), timed with HIP events on the stream they run on: the best
    of `reps` launches of each."""
    import torch
    from diffusion_vae_decoder_amd import api

    def best(fn):
        ts = []
        for _ in range(reps + 1):   # the first launch warms up
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return min(ts[1:])

    # one workgroup per CU: the probe's 8 accumulator chains need all of a
    # SIMD's registers, so each SIMD holds one wave
    blocks, iters = torch.cuda.get_device_properties(0).multi_processor_count, 65536
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = api.probe_mfma_f32(blocks, iters, out)[1]
    t_mfma = best(lambda: api.probe_mfma_f32(blocks, iters, out))
    n = 1 << 28   # 1 GiB of float32, four times the Infinity Cache
    grids = (1024, 4096, 16384)
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    part = torch.empty(max(grids) * 256, dtype=torch.float32, device="cuda")
    t_read = min(best(lambda: api.probe_hbm(x, blocks=g, out=part[:g * 256])) for g in grids)
    t_copy = min(best(lambda: api.probe_hbm(x, y, blocks=g)) for g in grids)
    del x, y
    torch.cuda.synchronize()
    return {"mfma_f32_tflops": flops / t_mfma / 1e12, "mfma_probe": f"{blocks} workgroups x 4 waves x {iters} rounds "
            "of 8 independent v_mfma_f32_32x32x2_f32 on register operands",
            "hbm_read_gbs": n * 4 / t_read / 1e9, "hbm_copy_gbs": 2 * n * 4 / t_copy / 1e9,
            "hbm_probe": "1 GiB read once (per-thread sums) and copied (read + write counted), the best of "
                         f"{list(grids)} workgroups of 256 threads streaming 16 KB chunks"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode of one image runs on one MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    from diffusion_vae_decoder_amd import api

    h = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.conv3x3:
        api.set_conv3x3_algorithm(args.conv3x3)
    params = vaegen.decoder_params(args.seed)
    dev_params = {k: torch.from_numpy(v).cuda() for k, v in params.items()}
    torch.cuda.synchronize()
    # first call: weight packing (weights already on the device), then the first decode
    t0 = time.perf_counter()
    dec = api.Decoder(dev_params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    if args.attention:
        dec.set_attention(args.attention)
    torch.cuda.synchronize()
    create_ms = (time.perf_counter() - t0) * 1e3
    z = torch.from_numpy(vaegen.latent(args.seed, h, h)).cuda()
    co, ho, wo = dec.output_shape(h, h)
    rgb = torch.empty((co, ho, wo), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec.decode(z, out=rgb)
    torch.cuda.synchronize()
    first_decode_ms = (time.perf_counter() - t0) * 1e3

    for _ in range(args.warmup):
        dec.decode(z, out=rgb)
    torch.cuda.synchronize()

    # timed region: exactly K decodes, every launch bracketed by HIP events on the stream
    dec.set_profiling(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.decode(z, out=rgb)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    recs = dec.profile()
    dec.set_profiling(False)
    ms_per_step = wall * 1e3 / args.steps

    if args.layer_table:
        layers = {}
        for r in recs:
            e = layers.setdefault((r["layer"], r["kernel"]), {"ms": 0.0, "flops": r["flops"], "bytes": r["bytes"]})
            e["ms"] += r["ms"] / args.steps
        with open(args.layer_table, "w") as f:
            json.dump([{"layer": l, "kernel": k, **v} for (l, k), v in layers.items()], f, indent=0)
    flops_per_step = sum(r["flops"] for r in recs) / args.steps
    by_kernel = {}
    for r in recs:
        k = by_kernel.setdefault(r["kernel"], {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "n": 0})
        k["ms"] += r["ms"]
        k["flops"] += r["flops"]
        k["bytes"] += r["bytes"]
        k["n"] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    conv_recs = [r for r in recs if is_conv3x3(r["kernel"])]
    conv_ms = sum(r["ms"] for r in conv_recs)
    conv_fl = sum(r["flops"] for r in conv_recs)
    cr = conv_rates(recs)
    roof = roofline(dom_name, dom, args.steps, args.workload)
    def rates(k, v):
        if not v["flops"]:
            return {"gbs": v["bytes"] / (v["ms"] / 1e3) / 1e9}
        direct = v["flops"] / (v["ms"] / 1e3) / 1e12
        return {"direct_equivalent_tflops": direct, "mfma_executed_tflops": mfma_fraction(k) * direct}

    breakdown = {k: {"ms_per_step": v["ms"] / args.steps, "launches_per_step": v["n"] // args.steps, **rates(k, v)}
                 for k, v in sorted(by_kernel.items(), key=lambda kv: -kv[1]["ms"])}

    out = {
        "metric": "VAE decode ms + conv TFLOP/s f32 (% FP32-MFMA peak) at 256² and 1024²",
        "value": flops_per_step / (ms_per_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "value_is": "direct-conv-equivalent TFLOP/s of the whole decode: its algorithmic FLOPs (every conv "
                    "counted as 2 Cin Cout k^2 H W, no Winograd credit; attention 8 N c^2 + 4 N^2 c) / ms_per_step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64 latent N(0,1) and weights at the stated init; no trained weights)",
        "config": {"workload": f"FLUX-class AutoencoderKL decode, latent [16,{h},{h}] -> RGB [3,{ho},{wo}], "
                               "batch 1, f32 NCHW", "latent": [16, h, h], "rgb": [co, ho, wo],
                   "flops_per_decode": flops_per_step, "conv3x3_form": api.get_conv3x3_algorithm(),
                   "attention_form": dec.get_attention()},
        "conv3x3": {"ms_per_step": conv_ms / args.steps, "direct_equivalent_tflops": conv_fl / (conv_ms / 1e3) / 1e12,
                    "mfma_executed_tflops": cr["mfma_executed_tflops"], "frac_fp32_mfma_peak": cr["frac_fp32_mfma_peak"]},
        "roofline": roof,
        "kernels": breakdown,
    }
    out["first_call"] = {"create_ms": create_ms, "first_decode_ms": first_decode_ms,
                         "note": "decoder creation packs the weights (already on the device); the first "
                                 "decode includes one-time workspace allocation"}
    out["latency"] = latency(dec, z, args.steps)
    if not args.no_graph:
        out["ms_per_step_graph_replay"] = graph_replay_ms(dec, z, args.steps, args.warmup)
    # secondary: the other decode size the metric names (after the timed region)
    if not args.no_secondary:
        out["secondary"] = secondary(dec, args, 32 if h != 32 else 128)
        out["tiled"] = tiled(dec, args, h)
    if not args.no_sweep:
        out["sweep"] = sweep(args)
    if not args.no_3d:
        out["stack3d"] = stack3d(args)
        out["decode3d"] = decode3d(args)
    if not args.no_peaks:
        pk = measured_peaks()
        pk["roofline_frac_of_measured_mfma"] = roof["achieved"] / pk["mfma_f32_tflops"] if roof["unit"] == "TFLOP/s" \
            else roof["achieved"] / pk["hbm_copy_gbs"]
        pk["conv3x3_frac_of_measured_mfma"] = cr["mfma_executed_tflops"] / pk["mfma_f32_tflops"]
        out["measured_peaks"] = pk
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = n * 4
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.seed, h)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
