"""Throughput of the tokenizer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole path over one synthetic clip of the
DV8x16x16-720p shape (1 x 3 x 49 x 720 x 1280 bf16), every stage a HIP kernel
behind the C ABI:

  Haar patcher (causal first frame, 2 levels)  ->  spatial 1x3x3 conv 192->256
  ->  causal temporal 3x1x1 conv 256->256 with the 1x1 projection 256->6 in its
  epilogue  ->  FSQ indices;  FSQ of a separate N(0, 1.5) 6-channel latent  ->
  dequantize;  inverse Haar of the coefficients back to pixels.

Inputs are resident in HBM before timing.  `value` is frames per second of the
whole step (49 frames per step), timed over K steps that carry only one pair of
HIP events, around the dominant kernel; K further steps with an event between
every stage give the per-stage breakdown.  The roofline object reports the
dominant kernel, the spatial convolution's MFMA implicit GEMM: algorithmic FLOPs
2*9*Cin*Cout per output position, divided by its average duration measured
with those HIP events on the launch stream over the timed steps.  The CPU baseline is
the float64 oracle timed on a bounded sample of the same workload (a strip of
the frame), scaled to the full clip.  A second object reports the 121-frame
CV8x8x8-720p-shaped chain (two factorized conv layers and the 1x1), where the
convolution's MFMA fraction is quoted; a third, FSQ quantize and dequantize at a
bandwidth-bound size (64 x 6 x 13 x 180 x 320 bf16) against the HBM peak; a fourth,
the factorized self-attention (spatial and causal temporal) on the 16 x 90 x 160 token
grid of the CV8x8x8-720p model, 256 channels in 4 heads; a fifth, sliding windows of 17
frames over a 50-frame 1080p clip (pad, Haar, inverse Haar, crop); a sixth, the encoder's
residual and downsampling blocks and the decoder's upsampling block on the CV8x8x8-720p grids; a
seventh, the batched DV4x8x8-360p decode (8 clips: dequantize + 1x1, conv 192->192, inverse Haar); an
eighth, the 121-frame clip encoded as a stream of chunks against one whole-clip pass.  The 49- and
121-frame clips and the decode also time the cross-stage fusions inside the conv's operand loads
(Haar of the pixels in the first spatial conv; dequantize + 1x1 in the decoder's conv) against
the unfused calls, interleaved in one process; a ninth object runs a 129-frame 1080p clip through
Haar and the conv chain, whose 2.19 GB activation exceeds 2 GiB.

The default 25 warmup steps matter: with 3 the GPU clocks have not settled and every
stage measures about 10% slower.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "720p frames/sec through Haar+causal conv+FSQ; HBM GB/s & MFMA % of peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_CAL_BYTES = 256 * 1024 * 1024

# HBM traffic of one launch of the dominant kernel (the spatial conv_rows_kernel,
# 1x3x3 192->256 on the 13 x 180 x 320 latent grid), from two rocprofv3 --pmc passes over
# this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  Each counter is scaled by
# what it reads for the 256 MiB device copy this script issues after timing: FETCH_SIZE
# reads 131106.7 KiB there (factor 2.0), WRITE_SIZE 262144 KiB (factor 1.0).  Only valid
# for the kernel version the counters were taken on: set to None when it changes.
SPATIAL_FETCH_KIB, SPATIAL_WRITE_KIB = 162925.8, 374400.0
COPY_FETCH_KIB, COPY_WRITE_KIB = 131106.7, 262144.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=25,
                    help="untimed steps first; below about 20 the GPU clocks have not settled (~10%% slower)")
    ap.add_argument("--workload", default="c4_dv8x16x16_720p_49f")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c3", action="store_true", help="skip the 121-frame chain measurement")
    ap.add_argument("--no-fsq-bw", action="store_true", help="skip the FSQ bandwidth-size measurement")
    ap.add_argument("--no-attention", action="store_true", help="skip the factorized-attention measurement")
    ap.add_argument("--no-window", action="store_true", help="skip the sliding-window measurement")
    ap.add_argument("--no-blocks", action="store_true", help="skip the encoder/decoder block measurement")
    ap.add_argument("--no-c5", action="store_true", help="skip the batched 360p decode measurement")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-encode measurement")
    ap.add_argument("--no-fusion", action="store_true", help="skip the fused-versus-unfused measurements")
    ap.add_argument("--no-1080p", action="store_true", help="skip the 129-frame 1080p chain (activations above 2 GiB)")
    ap.add_argument("--cpu-width", type=int, default=1280,
                    help="pixel width of the strip the CPU oracle is timed on")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def interleaved(torch, fns, reps, rounds=6, warm_s=0.5):
    """Median milliseconds per call of each function: after warm_s seconds of calling them all
    (the clocks settle only after some tens of milliseconds of work), `rounds` rounds each
    time every function `reps` times back to back with HIP events on the current stream,
    alternating the order from round to round (the first-measured one otherwise reads
    slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for fn in fns:
            fn()
        torch.cuda.synchronize()
    res = [[] for _ in fns]
    for r in range(rounds):
        order = list(range(len(fns))) if r % 2 == 0 else list(reversed(range(len(fns))))
        for i in order:
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                fns[i]()
            e.record()
            torch.cuda.synchronize()
            res[i].append(s.elapsed_time(e) / reps)
    return [float(np.median(v)) for v in res]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is not sharded "
              "across GPUs in this library", file=sys.stderr)
        sys.exit(2)
    import torch

    import causal_video_tokenizer_amd as cvt
    import synthetic_inputs as si

    wl = si.WORKLOADS[args.workload]
    if args.workload != "c4_dv8x16x16_720p_49f":
        raise SystemExit("only the DV8x16x16-720p-shaped workload is wired into the benchmark step")
    dev = torch.device("cuda:0")
    B, C, T, H, W = wl["x"]
    Tq, Hq, Wq = 1 + (T - 1) // 4, H // 4, W // 4
    P = B * Tq * Hq * Wq
    cid = 4

    log(f"generating inputs {wl['x']} ...")
    xbits = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    zbits = si.to_bf16_bits(si.normal(wl["latent"], wl["latent_seed"], wl["latent_std"]))

    def bf16_dev(bits, cl=False):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return t.to(memory_format=torch.channels_last_3d) if cl else t

    ws_b = si.to_bf16_bits(si.normal((256, 192, 1, 3, 3), si.weight_seed(cid, 0), 0.02))
    wt_b = si.to_bf16_bits(si.normal((256, 256, 3, 1, 1), si.weight_seed(cid, 1), 0.02))
    pj_b = si.to_bf16_bits(si.normal((6, 256, 1, 1, 1), si.weight_seed(cid, 2), 0.02))
    x = bf16_dev(xbits)
    z_sep = bf16_dev(zbits)
    w_s, w_t, w_p = bf16_dev(ws_b), bf16_dev(wt_b), bf16_dev(pj_b)

    cl = torch.channels_last_3d
    hz = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    s1 = torch.empty((B, 256, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    lat = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    idx = torch.empty((B, Tq, Hq, Wq), dtype=torch.int32, device=dev)
    idx2 = torch.empty_like(idx)
    codes = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    xr = torch.empty_like(x)
    ws_sp = torch.empty(cvt.conv_workspace_bytes(hz.shape, 256, 3, True, False), dtype=torch.uint8, device=dev)

    # (FSQ can also run inside the projection epilogue, causal_conv3d_fact_proj_fsq; on this
    # workload that is 4% slower than the FSQ kernel after the conv, so the step keeps two calls)
    stages = ["haar_fwd", "conv_spatial", "conv_temporal_proj", "fsq_quantize", "fsq_quantize_sep",
              "fsq_dequantize", "haar_inv"]
    # the weights are fixed across steps: packed once here, outside the timed region, in the
    # order the conv kernels read them (the per-call repack costs about 4.5 us per weight tensor)
    pw_s, pw_t, pw_p = cvt.conv_weights_pack(w_s), cvt.conv_weights_pack(w_t), cvt.conv_weights_pack(w_p)
    calls = {
        "haar_fwd": lambda: cvt.haar3d_fwd(x, out=hz),
        "conv_spatial": lambda: cvt.causal_conv3d_fact_packed(hz, pw_s, None, out=s1),
        "conv_temporal_proj": lambda: cvt.causal_conv3d_fact_proj_packed(s1, None, pw_t, pw_p, out=lat),
        "fsq_quantize": lambda: cvt.fsq_quantize(lat, indices=idx),
        "fsq_quantize_sep": lambda: cvt.fsq_quantize(z_sep, indices=idx2),
        "fsq_dequantize": lambda: cvt.fsq_dequantize(idx2, out=codes),
        "haar_inv": lambda: cvt.haar3d_inv(hz, out=xr),
    }
    stream = torch.cuda.current_stream(dev)

    def step(evs=None, dom_evs=None):
        # evs: an event before every stage and after the last (the per-stage breakdown);
        # dom_evs: a pair of events around the dominant kernel's call only (the roofline)
        for i, name in enumerate(stages):
            if evs is not None:
                evs[i].record(stream)
            if dom_evs is not None and name == "conv_spatial":
                dom_evs[0].record(stream)
            calls[name]()
            if dom_evs is not None and name == "conv_spatial":
                dom_evs[1].record(stream)
        if evs is not None:
            evs[len(stages)].record(stream)

    log("warmup ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: K steps with one pair of events around the dominant kernel (an event
    # between every stage costs about 4 us each, 3% of the step)
    dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(dom_evs=dev_ev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = float(np.mean([dev_ev[k][0].elapsed_time(dev_ev[k][1]) for k in range(args.steps)]))
    # then K more steps with an event between every stage, for the per-stage breakdown
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]))
                for i, name in enumerate(stages)}

    # algorithmic work per stage
    conv_flops = {
        "conv_spatial": 2.0 * 9 * 192 * 256 * P,
        "conv_temporal_proj": 2.0 * 3 * 256 * 256 * P + 2.0 * 256 * 6 * P,
    }
    hbm_bytes = {
        "haar_fwd": 2.0 * B * C * T * H * W + 2.0 * P * 192,
        "haar_inv": 2.0 * P * 192 + 2.0 * B * C * T * H * W,
        "fsq_quantize": P * (6 * 2 + 4.0),
        "fsq_quantize_sep": P * (6 * 2 + 4.0),
        "fsq_dequantize": P * (4 + 6 * 2.0),
    }
    per_stage = {}
    for name in stages:
        d = {"ms": round(stage_ms[name], 4)}
        if name in conv_flops:
            d["TFLOPs"] = round(conv_flops[name] / (stage_ms[name] * 1e-3) / 1e12, 2)
        if name in hbm_bytes:
            d["GBps"] = round(hbm_bytes[name] / (stage_ms[name] * 1e-3) / 1e9, 1)
        per_stage[name] = d

    dom = "conv_spatial"
    achieved = conv_flops[dom] / (dom_ms * 1e-3) / 1e12  # HIP events inside the timed region
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic_bytes(),
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": 2.0 * P * (192 + 256) + 2.0 * 256 * 192 * 9,
                "kernel": "conv_rows_kernel<RowsCfg<SPATIAL3,R=4,WCH=4,FA=2,BK=32,NW=4>,false,false> (1x3x3 conv 192->256, bf16 MFMA)",
                "flops_per_launch": conv_flops[dom], "avg_launch_ms": round(dom_ms, 4),
                "timing": "HIP events on the launch stream around each timed step's call (weights packed once, before timing)"}

    fusion = None
    if not args.no_fusion:
        # the Haar patcher inside the spatial conv's loads, against the two calls of the step
        hz_conv = torch.empty_like(s1)
        ws_fz = torch.empty(cvt.haar3d_conv3d_fact_workspace_bytes(x.shape, 256, False), dtype=torch.uint8, device=dev)
        # both routes repack their weights per call (there is no packed form of the fused call)
        unf, fus = interleaved(torch, [lambda: (calls["haar_fwd"](),
                                                cvt.causal_conv3d_fact(hz, w_s, None, workspace=ws_sp, out=s1)),
                                       lambda: cvt.haar3d_conv3d_fact(x, w_s, workspace=ws_fz, out=hz_conv)],
                               max(5, args.steps // 2))
        fusion = {"haar_then_spatial_conv_ms": round(unf, 4), "haar_inside_spatial_conv_ms": round(fus, 4),
                  "fused_over_unfused": round(fus / unf, 4),
                  "note": "the step keeps the two calls: its inverse-Haar stage reads the coefficients"}
        del hz_conv, ws_fz
    c3 = None if args.no_c3 else cv8x8x8_chain(cvt, si, torch, dev, args)
    fsq_bw = None if args.no_fsq_bw else fsq_bandwidth(cvt, si, torch, dev, args)
    attn = None if args.no_attention else attention_tokens(cvt, si, torch, dev, args)
    win = None if args.no_window else windowed_1080p(cvt, si, torch, dev, args)
    blk = None if args.no_blocks else blocks_cv8x8x8(cvt, si, torch, dev, args)
    c5 = None if args.no_c5 else decode_c5(cvt, si, torch, dev, args)
    stream = None if args.no_stream else stream_encode(cvt, si, torch, dev, args)
    long1080 = None if args.no_1080p else clip_1080p_chain(cvt, si, torch, dev, args)

    # Copy calibration for the HBM-traffic counters: one device copy of a known
    # number of bytes, outside the timed region (its FETCH_SIZE / WRITE_SIZE readings
    # scale the dominant kernel's).
    cal = torch.empty(COPY_CAL_BYTES // 2, dtype=torch.bfloat16, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(xbits, zbits, ws_b, wt_b, pj_b, (B, C, T, H, W), args.cpu_width)

    frames = B * T
    out = {
        "metric": METRIC,
        "value": round(frames / (ms_per_step * 1e-3), 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DV8x16x16-720p-shaped discrete path, 1x3x49x720x1280 bf16 "
                               "(Haar -> conv 192->256 k3 with the 1x1 ->6 fused -> FSQ; FSQ+dequant of a 6x13x180x320 "
                               "N(0,1.5) latent; inverse Haar)",
                   "frames_per_step": frames, "latent_grid": [Tq, Hq, Wq]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": per_stage,
        "stages_timing": "K further steps with an event between every stage (not part of value)",
        "fusion_haar_conv_49f": fusion,
        "cv8x8x8_720p_121f": c3,
        "fsq_bandwidth_size": fsq_bw,
        "attention_cv8x8x8_720p_tokens": attn,
        "window_1080p_50f": win,
        "blocks_cv8x8x8_720p": blk,
        "dv4x8x8_360p_decode_c5": c5,
        "stream_encode_121f_720p": stream,
        "clip_1080p_129f": long1080,
        "copy_calibration_bytes": COPY_CAL_BYTES,
    }
    print(json.dumps(out), flush=True)


def traffic_bytes():
    if SPATIAL_FETCH_KIB is None:
        return None
    cal = COPY_CAL_BYTES / 1024.0
    return round(1024.0 * (SPATIAL_FETCH_KIB * cal / COPY_FETCH_KIB + SPATIAL_WRITE_KIB * cal / COPY_WRITE_KIB))


def cv8x8x8_chain(cvt, si, torch, dev, args):
    """The 121-frame 720p chain (Haar -> conv 192->256 k3 -> conv 256->256 k3 with the 1x1 -> 16
    in its temporal epilogue),
    timed per stage with HIP events; reports frames/s of the chain and the MFMA
    fraction of each convolution (the conv target is quoted on this clip)."""
    wl = si.WORKLOADS["c3_cv8x8x8_720p_121f"]
    B, C, T, H, W = wl["x"]
    Tq, Hq, Wq = 1 + (T - 1) // 4, H // 4, W // 4
    P = B * Tq * Hq * Wq
    log(f"121-frame chain: generating {wl['x']} ...")
    xbits = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))

    def dev_bits(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = dev_bits(xbits)
    del xbits
    w = [dev_bits(si.to_bf16_bits(si.normal(shape, si.weight_seed(3, i), 0.02)))
         for i, shape in enumerate([(256, 192, 1, 3, 3), (256, 256, 3, 1, 1), (256, 256, 1, 3, 3),
                                    (256, 256, 3, 1, 1), (16, 256, 1, 1, 1)])]
    cl = torch.channels_last_3d
    hz = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    a = torch.empty((B, 256, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    b = torch.empty_like(a)
    lat = torch.empty((B, 16, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    ws = {"s1": torch.empty(cvt.conv_workspace_bytes(hz.shape, 256, 3, True, False), dtype=torch.uint8, device=dev)}
    pw = [cvt.conv_weights_pack(wi) for wi in w]  # fixed weights: packed once, outside the timed region
    stages = [
        ("haar_fwd", lambda: cvt.haar3d_fwd(x, out=hz), None),
        ("l1_spatial", lambda: cvt.causal_conv3d_fact_packed(hz, pw[0], None, out=a), 2.0 * 9 * 192 * 256 * P),
        ("l1_temporal", lambda: cvt.causal_conv3d_fact_packed(a, None, pw[1], out=b), 2.0 * 3 * 256 * 256 * P),
        ("l2_spatial", lambda: cvt.causal_conv3d_fact_packed(b, pw[2], None, out=a), 2.0 * 9 * 256 * 256 * P),
        ("l2_temporal_proj", lambda: cvt.causal_conv3d_fact_proj_packed(a, None, pw[3], pw[4], out=lat),
         2.0 * 3 * 256 * 256 * P + 2.0 * 256 * 16 * P),
    ]
    stream = torch.cuda.current_stream(dev)
    steps = max(2, args.steps // 2)
    for _ in range(max(1, min(args.warmup, 10))):  # the clocks drop while the host generates the clip
        for _, fn, _ in stages:
            fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    for k in range(steps):
        for i, (_, fn, _) in enumerate(stages):
            evs[k][i].record(stream)
            fn()
        evs[k][len(stages)].record(stream)
    torch.cuda.synchronize()
    out = {"steps": steps, "stages": {}}
    total = 0.0
    conv_flops = conv_ms = 0.0
    for i, (name, _, flops) in enumerate(stages):
        ms = float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
        total += ms
        d = {"ms": round(ms, 4)}
        if flops:
            d["TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
            d["mfma_frac"] = round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
            conv_flops += flops
            conv_ms += ms
        else:
            d["GBps"] = round((2.0 * B * C * T * H * W + 2.0 * P * 192) / (ms * 1e-3) / 1e9, 1)
        out["stages"][name] = d
    out["frames_per_s"] = round(B * T / (total * 1e-3), 1)
    out["conv_TFLOPs"] = round(conv_flops / (conv_ms * 1e-3) / 1e12, 1)
    out["conv_mfma_frac"] = round(conv_flops / (conv_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    if not args.no_fusion:  # the Haar patcher inside layer 1's spatial conv
        ws_fz = torch.empty(cvt.haar3d_conv3d_fact_workspace_bytes(x.shape, 256, False), dtype=torch.uint8, device=dev)
        a2 = torch.empty_like(a)
        # both routes repack their weights per call (there is no packed form of the fused call)
        unf, fus = interleaved(torch, [lambda: (stages[0][1](),
                                                cvt.causal_conv3d_fact(hz, w[0], None, workspace=ws["s1"], out=a)),
                                       lambda: cvt.haar3d_conv3d_fact(x, w[0], workspace=ws_fz, out=a2)],
                               max(3, args.steps // 4))
        rest = total - out["stages"]["haar_fwd"]["ms"] - out["stages"]["l1_spatial"]["ms"]
        out["fusion"] = {"haar_then_l1_spatial_ms": round(unf, 4), "haar_inside_l1_spatial_ms": round(fus, 4),
                         "fused_over_unfused": round(fus / unf, 4),
                         "frames_per_s_fused_route": round(B * T / ((rest + fus) * 1e-3), 1)}
        del ws_fz, a2
    del x, hz, a, b, lat, ws
    torch.cuda.empty_cache()
    return out


def fsq_bandwidth(cvt, si, torch, dev, args):
    """FSQ quantize and dequantize at a size where HBM bandwidth, not launch latency,
    bounds them: 64 latents of the 49-frame grid, 64 x 6 x 13 x 180 x 320 bf16 N(0, 1.5)
    (575 MB of latents, 192 MB of indices), planar (NCTHW) and channels-last (NTHWC).
    Each call moves 6 x 2 + 4 bytes per position; timed over back-to-back calls with HIP
    events and reported against the 8 TB/s HBM peak."""
    wl = si.WORKLOADS["fsq_bw"]
    shape = wl["latent"]
    B, D, T, H, W = shape
    P = B * T * H * W
    log(f"FSQ bandwidth size: generating {shape} ...")
    zb = si.to_bf16_bits(si.normal(shape, wl["latent_seed"], wl["latent_std"]))
    z = torch.from_numpy(np.ascontiguousarray(zb).view(np.int16)).view(torch.bfloat16).to(dev)
    del zb
    zc = z.to(memory_format=torch.channels_last_3d)
    idx = torch.empty((B, T, H, W), dtype=torch.int32, device=dev)
    codes = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    codes_c = torch.empty_like(zc)
    cases = [
        ("quantize_ncthw", lambda: cvt.fsq_quantize(z, indices=idx)),
        ("dequantize_ncthw", lambda: cvt.fsq_dequantize(idx, layout="NCTHW", out=codes)),
        ("quantize_nthwc", lambda: cvt.fsq_quantize(zc, indices=idx)),
        ("dequantize_nthwc", lambda: cvt.fsq_dequantize(idx, out=codes_c)),
    ]
    reps = max(10, args.steps // 2)
    nbytes = P * (D * 2 + 4.0)
    out = {"shape": list(shape), "bytes_per_call": nbytes, "reps": reps,
           "timing": "median of 6 rounds alternating the case order, after 1 s of warm-up calls"}
    # the GPU idled while the host generated the latents: interleaved() warms it up first
    times = interleaved(torch, [fn for _, fn in cases], reps, warm_s=1.0)
    for (name, fn), ms in zip(cases, times):
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    del z, zc, idx, codes, codes_c
    torch.cuda.empty_cache()
    return out


def attention_tokens(cvt, si, torch, dev, args):
    """Factorized self-attention on the CV8x8x8-720p token grid of a 121-frame clip
    (1 x 256 x 16 x 90 x 160, 4 heads of 64): spatial attention over each frame's 14,400
    positions (4 N^2 d FLOP per frame and head, MFMA) and causal temporal attention over
    each position's 16 frames (q, k, v read and the output written once: HBM).  Timed
    over back-to-back calls with HIP events."""
    wl = si.WORKLOADS["attn_cv8x8x8_720p_tokens"]
    shape, heads = wl["x"], wl["heads"]
    B, C, T, H, W = shape
    N, d = H * W, C // heads
    log(f"attention: generating q, k, v {shape} ...")

    def dev_bits(seed):
        bits = si.to_bf16_bits(si.normal(shape, seed, wl["std"]))
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return t.to(memory_format=torch.channels_last_3d)

    q, k, v = (dev_bits(wl["seed"] + i) for i in range(3))
    o = torch.empty_like(q)
    calls = {"spatial": lambda: cvt.attention3d(q, k, v, heads, "spatial", out=o),
             "temporal_causal": lambda: cvt.attention3d(q, k, v, heads, "temporal", out=o)}
    for _ in range(max(3, min(args.warmup, 10))):
        for fn in calls.values():
            fn()
    torch.cuda.synchronize()
    out = {"shape": list(shape), "heads": heads}
    for name, fn in calls.items():
        reps = max(5, args.steps // 2) if name == "spatial" else max(10, args.steps)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        if name == "spatial":
            flops = 4.0 * N * N * d * heads * B * T
            tf = flops / (ms * 1e-3) / 1e12
            out[name] = {"ms": round(ms, 4), "flops": flops, "TFLOPs": round(tf, 1),
                         "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        else:
            nbytes = 4.0 * q.numel() * 2
            gbps = nbytes / (ms * 1e-3) / 1e9
            out[name] = {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(gbps, 1),
                         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    del q, k, v, o
    torch.cuda.empty_cache()
    return out


def windowed_1080p(cvt, si, torch, dev, args):
    """Sliding windows over a clip the tokenizer does not accept as it is (1 x 3 x 50 x
    1080 x 1920 bf16): per window of 17 frames, pad (mirror in time to 1 + 4k frames, zeros
    to 1088 rows), 2-level Haar, inverse Haar, crop back into the output clip.  Reports the
    whole windowed round trip in frames/s, unfused (four calls per window) and fused (the
    padding inside the Haar's loads, the crop inside the inverse's stores: two calls), and
    the pad and crop kernels against the HBM peak (bytes read + written by each call,
    summed over the windows)."""
    wl = si.WORKLOADS["window_1080p_50f"]
    shape = wl["x"]
    B, C, T, H, W = shape
    log(f"sliding windows: generating {shape} ...")
    xb = si.to_bf16_bits(si.normal(shape, wl["seed"], wl["std"]))
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    del xb
    out = torch.empty_like(x)
    wins = cvt.video_windows(T, H, W, wl["window"], wl["t_align"], wl["s_align"])
    bufs = [torch.empty((B, C, Tp, Hp, Wp), dtype=torch.bfloat16, device=dev) for _, _, Tp, Hp, Wp in wins]
    coef = [torch.empty((B, 64 * C, 1 + (Tp - 1) // 4, Hp // 4, Wp // 4), dtype=torch.bfloat16, device=dev)
            .to(memory_format=torch.channels_last_3d) for _, _, Tp, Hp, Wp in wins]
    rec = [torch.empty_like(b) for b in bufs]

    def pads():
        for (t0, nt, Tp, Hp, Wp), b in zip(wins, bufs):
            cvt.video_pad(x, t0, nt, Tp, Hp, Wp, out=b)

    def crops():
        for (t0, nt, _, _, _), r in zip(wins, rec):
            cvt.video_unpad(r, out, t0, nt)

    def round_trip():
        for (t0, nt, Tp, Hp, Wp), b, c, r in zip(wins, bufs, coef, rec):
            cvt.video_pad(x, t0, nt, Tp, Hp, Wp, out=b)
            cvt.haar3d_fwd(b, 2, out=c)
            cvt.haar3d_inv(c, 2, out=r)
            cvt.video_unpad(r, out, t0, nt)

    out_f = torch.empty_like(x)

    def round_trip_fused():  # the padding inside the Haar's loads, the crop inside the inverse's stores
        for (t0, nt, Tp, Hp, Wp), c in zip(wins, coef):
            cvt.haar3d_fwd_window(x, t0, nt, Tp, Hp, Wp, 2, out=c)
            cvt.haar3d_inv_window(c, out_f, t0, nt, 2)

    for _ in range(max(3, min(args.warmup, 10))):
        round_trip_fused()
        round_trip()
    torch.cuda.synchronize()
    reps = max(5, args.steps // 2)
    res = {"shape": list(shape), "windows": [list(w) for w in wins]}
    res["fused_equals_unfused"] = bool(torch.equal(out_f.view(torch.int16), out.view(torch.int16)))
    pad_bytes = sum(2.0 * B * C * (nt * H * W + Tp * Hp * Wp) for _, nt, Tp, Hp, Wp in wins)
    crop_bytes = sum(2.0 * B * C * 2 * nt * H * W for _, nt, _, _, _ in wins)
    for name, fn, nbytes in (("pad", pads, pad_bytes), ("crop", crops, crop_bytes), ("round_trip", round_trip, None),
                             ("round_trip_fused", round_trip_fused, None)):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        if nbytes is None:
            res[name] = {"ms": round(ms, 4), "frames_per_s": round(B * T / (ms * 1e-3), 1)}
        else:
            gbps = nbytes / (ms * 1e-3) / 1e9
            res[name] = {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(gbps, 1),
                         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    # the round trip must give back the clip (Haar is orthonormal; bf16 storage of the
    # coefficients and pixels rounds)
    err = (out.float() - x.float()).abs().max().item()
    res["round_trip_max_abs_err"] = err
    del x, out, out_f, bufs, coef, rec
    torch.cuda.empty_cache()
    return res


def blocks_cv8x8x8(cvt, si, torch, dev, args):
    """Encoder and decoder blocks on the CV8x8x8-720p grids of a 121-frame clip, 256 channels:
    the residual block at the post-Haar grid 31 x 180 x 320 (LayerNorm + Swish, two
    factorized convs, LayerNorm + Swish and the residual add fused into the temporal convs),
    the stride-2 downsampling block to 16 x 90 x 160, and the decoder's upsampling block back
    (repetition inside the conv loads).  The blocks' weights are fixed, so they are packed once
    (the _packed entry points); the residual block that repacks them every call is timed beside
    it.  FLOP =
    2 * taps * Cin * Cout per output position of each conv; timed over back-to-back calls with
    HIP events."""
    wl = si.WORKLOADS["blocks_cv8x8x8_720p"]
    B, C, T, H, W = wl["x"]
    _, _, Tl, Hl, Wl = wl["low"]
    seed, std = wl["seed"], wl["w_std"]
    log(f"blocks: generating {wl['x']} ...")

    def bf(shape, sd, s_):
        bits = si.to_bf16_bits(si.normal(shape, sd, s_))
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf((B, C, T, H, W), seed, 1.0).to(memory_format=torch.channels_last_3d)
    xl = bf((B, C, Tl, Hl, Wl), seed + 1, 1.0).to(memory_format=torch.channels_last_3d)
    ones = torch.ones(C, dtype=torch.float32, device=dev)
    zeros = torch.zeros(C, dtype=torch.float32, device=dev)
    p = {"ln1_g": ones, "ln1_b": zeros, "ln2_g": ones, "ln2_b": zeros,
         "c1_s": bf((C, C, 1, 3, 3), seed + 2, std), "c1_t": bf((C, C, 3, 1, 1), seed + 3, std),
         "c2_s": bf((C, C, 1, 3, 3), seed + 4, std), "c2_t": bf((C, C, 3, 1, 1), seed + 5, std)}
    ds_s, ds_t = bf((C, C, 1, 3, 3), seed + 6, std), bf((C, C, 3, 1, 1), seed + 7, std)
    us_s, us_t = bf((C, C, 1, 3, 3), seed + 8, std), bf((C, C, 3, 1, 1), seed + 9, std)
    y = torch.empty_like(x)
    yd = torch.empty_like(xl)
    yu = torch.empty_like(x)
    ws_r = torch.empty(int(cvt.lib.cvt_resblock3d_workspace(B, C, T, H, W)), dtype=torch.uint8, device=dev)
    # the block's weights are fixed: packed once, as in the step (the per-call repack timed beside it)
    pp = dict(p)
    for k in ("c1_s", "c1_t", "c2_s", "c2_t"):
        pp[k] = cvt.conv_weights_pack(p[k])
    ws_rp = torch.empty(int(cvt.lib.cvt_resblock3d_packed_workspace(B, C, T, H, W)), dtype=torch.uint8, device=dev)
    pds_s, pds_t, pus_s, pus_t = (cvt.conv_weights_pack(w) for w in (ds_s, ds_t, us_s, us_t))
    ws_d = torch.empty(int(cvt.lib.cvt_downsample3d_packed_workspace(B, C, C, T, H, W, 3)), dtype=torch.uint8,
                       device=dev)
    ws_u = torch.empty(int(cvt.lib.cvt_upsample3d_packed_workspace(B, C, C, Tl, Hl, Wl, 1, 1)), dtype=torch.uint8,
                       device=dev)
    P = B * T * H * W
    conv = 2.0 * C * C * (9 + 3)
    calls = {
        "resblock_31x180x320": (lambda: cvt.resblock3d_packed(x, pp, workspace=ws_rp, out=y), 2 * conv * P),
        "resblock_31x180x320_repack_per_call": (lambda: cvt.resblock3d(x, p, workspace=ws_r, out=y), 2 * conv * P),
        "downsample_to_16x90x160": (lambda: cvt.downsample3d_packed(x, pds_s, pds_t, workspace=ws_d, out=yd),
                                    2.0 * C * C * 9 * B * T * Hl * Wl + 2.0 * C * C * 3 * B * Tl * Hl * Wl),
        "upsample_to_31x180x320": (lambda: cvt.upsample3d_packed(xl, pus_s, pus_t, workspace=ws_u, out=yu),
                                   2.0 * C * C * 9 * B * Tl * H * W + 2.0 * C * C * 3 * P),
    }
    for _ in range(max(3, min(args.warmup, 10))):
        for fn, _ in calls.values():
            fn()
    torch.cuda.synchronize()
    reps = max(5, args.steps // 2)
    out = {"grid": [T, H, W], "low_grid": [Tl, Hl, Wl], "channels": C}
    for name, (fn, flops) in calls.items():
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "flops": flops, "TFLOPs": round(tf, 1),
                     "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    del x, xl, y, yd, yu, ws_r, ws_rp, ws_d, ws_u, p, pp, pds_s, pds_t, pus_s, pus_t
    torch.cuda.empty_cache()
    return out


def decode_c5(cvt, si, torch, dev, args):
    """The batched DV4x8x8-360p decode: 8 clips of int32 indices 8 x 13 x 90 x 160 -> FSQ
    dequantize fused with the 1x1 6 -> 192 -> factorized causal conv 192 -> 192 (k = 3) ->
    inverse Haar to 8 x 3 x 49 x 360 x 640 bf16.  Reports 392 output frames / the chain's
    time, each stage's rate, and the unfused dequantize + 1x1 for comparison."""
    cid = 5
    wl = si.WORKLOADS["c5_dv4x8x8_360p_decode"]
    B, Tq, Hq, Wq = wl["indices"]
    P = B * Tq * Hq * Wq
    log(f"c5 decode: generating indices {wl['indices']} ...")
    idx = torch.from_numpy(si.uniform_indices(wl["indices"], wl["seed"])).to(dev)

    def bf(shape, seed):
        bits = si.to_bf16_bits(si.normal(shape, seed, 0.02))
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    lift, w_s, w_t = bf((192, 6, 1, 1, 1), si.weight_seed(cid, 0)), bf((192, 192, 1, 3, 3), si.weight_seed(cid, 1)), \
        bf((192, 192, 3, 1, 1), si.weight_seed(cid, 2))
    cl = torch.channels_last_3d
    z = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    yc = torch.empty_like(z)
    codes = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    xo = torch.empty(wl["out_x"], dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cvt.conv_workspace_bytes(z.shape, 192, 3, True, True), dtype=torch.uint8, device=dev)
    ws1 = torch.empty(cvt.conv_workspace_bytes(codes.shape, 192, 1, True, False), dtype=torch.uint8, device=dev)
    pw_s, pw_t = cvt.conv_weights_pack(w_s), cvt.conv_weights_pack(w_t)  # fixed weights: packed once
    ws_pk = torch.empty(cvt.conv_packed_workspace_bytes(z.shape, 192), dtype=torch.uint8, device=dev)
    stages = {
        "dequantize_proj": lambda: cvt.fsq_dequantize_proj(idx, lift, out=z),
        "conv_192_192": lambda: cvt.causal_conv3d_fact_packed(z, pw_s, pw_t, workspace=ws_pk, out=yc),
        "haar_inv": lambda: cvt.haar3d_inv(yc, out=xo),
    }
    unfused = lambda: (cvt.fsq_dequantize(idx, out=codes), cvt.causal_conv3d_fact(codes, lift, None, workspace=ws1,
                                                                                   out=z))
    for _ in range(max(3, min(args.warmup, 10))):
        for fn in stages.values():
            fn()
        unfused()
    torch.cuda.synchronize()
    reps = max(5, args.steps // 2)
    out = {"indices": list(wl["indices"]), "out_frames": B * wl["out_x"][2],
           "timing": "median of 6 rounds alternating the stage order, after 0.5 s of warm-up calls"}
    total = 0.0
    named = list(stages.items()) + [("dequantize_then_proj_unfused", unfused)]
    times = interleaved(torch, [fn for _, fn in named], reps)
    for (name, fn), ms in zip(named, times):
        d = {"ms": round(ms, 4)}
        if name == "conv_192_192":
            flops = (2.0 * 9 * 192 * 192 + 2.0 * 3 * 192 * 192) * P
            d.update(TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1), mfma_frac=round(flops / (ms * 1e-3) / 1e12 /
                                                                                   BF16_PEAK_TFLOPS, 4))
        elif name == "haar_inv":
            nbytes = 2.0 * P * 192 + 2.0 * int(np.prod(wl["out_x"]))
            d.update(GBps=round(nbytes / (ms * 1e-3) / 1e9, 1), hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4))
        else:
            nbytes = 4.0 * P + 2.0 * 192 * P
            d.update(GBps=round(nbytes / (ms * 1e-3) / 1e9, 1), hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4))
        if name in stages:
            total += ms
        out[name] = d
    out["chain_ms"] = round(total, 4)
    out["frames_per_s"] = round(out["out_frames"] / (total * 1e-3), 1)
    if not args.no_fusion:  # dequantize + 1x1 inside the conv's loads
        ws_fz = torch.empty(cvt.fsq_dequantize_conv3d_fact_workspace_bytes(idx.shape, 192, 192, True),
                            dtype=torch.uint8, device=dev)
        yf = torch.empty_like(yc)
        # both routes repack their weights per call (there is no packed form of the fused call)
        unf, fus = interleaved(torch, [lambda: (stages["dequantize_proj"](),
                                                cvt.causal_conv3d_fact(z, w_s, w_t, workspace=ws, out=yc)),
                                       lambda: cvt.fsq_dequantize_conv3d_fact(idx, lift, w_s, w_t, workspace=ws_fz,
                                                                              out=yf)],
                               max(3, args.steps // 4))
        out["fusion"] = {"dequantize_proj_then_conv_ms": round(unf, 4), "dequantize_proj_inside_conv_ms": round(fus, 4),
                         "fused_over_unfused": round(fus / unf, 4),
                         "frames_per_s_fused_route": round(out["out_frames"] /
                                                           ((fus + out["haar_inv"]["ms"]) * 1e-3), 1)}
        del ws_fz, yf
    del idx, z, yc, codes, xo, ws, ws1, ws_pk
    torch.cuda.empty_cache()
    return out


def stream_encode(cvt, si, torch, dev, args):
    """Streaming causal encode of a 121-frame 720p clip (the CV8x8x8-720p shape, G_trans
    pixels) to FSQ indices, chunk by chunk: a first chunk of 17 frames (Haar with the causal
    first frame), then chunks of 16 frames (Haar continuation), each through the spatial conv
    192 -> 256 and the causal temporal conv 256 -> 256 with the 1x1 -> 6 fused, reading the
    previous chunk's last two frames in place of the zero padding, then FSQ.  The result
    equals the whole-clip encode bit for bit; reported against the whole clip in one pass."""
    wl = si.WORKLOADS["c3_cv8x8x8_720p_121f"]
    B, C, T, H, W = wl["x"]
    log(f"stream encode: generating {wl['x']} ...")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    del xb

    def bf(shape, seed):
        bits = si.to_bf16_bits(si.normal(shape, seed, 0.02))
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    w_s, w_t, w_p = bf((256, 192, 1, 3, 3), 3101), bf((256, 256, 3, 1, 1), 3102), bf((6, 256, 1, 1, 1), 3103)
    cl = torch.channels_last_3d
    Hq, Wq = H // 4, W // 4
    cuts = [(0, 17, 2)] + [(t, t + 16, 3) for t in range(17, T, 16)]  # 17 + 7 x 16 = 129 > 121: clip the last
    cuts = [(a, min(b, T), tl) for a, b, tl in cuts if a < T]
    assert all((b - a) % 4 == 0 for a, b, tl in cuts if tl == 3), "continuation chunks of 4k frames"
    bufs = []
    for a, b, tl in cuts:
        tq = 1 + (b - a - 1) // 4 if tl == 2 else (b - a) // 4
        bufs.append(dict(
            x=x[:, :, a:b],
            hz=torch.empty((B, 192, tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl),
            s=torch.empty((B, 256, tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl),
            lat=torch.empty((B, 6, tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl),
            idx=torch.empty((B, tq, Hq, Wq), dtype=torch.int32, device=dev), tl=tl))
    xs = [bb["x"].contiguous() for bb in bufs]  # chunk inputs as the caller would hand them over
    ws_s = torch.empty(cvt.conv_workspace_bytes(bufs[1]["hz"].shape, 256, 3, True, False), dtype=torch.uint8,
                       device=dev)
    ws_t = torch.empty(cvt.temporal_stream_workspace_bytes(256, 6), dtype=torch.uint8, device=dev)
    Tq = 1 + (T - 1) // 4
    hz_w = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    s_w = torch.empty((B, 256, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    lat_w = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    idx_w = torch.empty((B, Tq, Hq, Wq), dtype=torch.int32, device=dev)
    ws_sw = torch.empty(cvt.conv_workspace_bytes(hz_w.shape, 256, 3, True, False), dtype=torch.uint8, device=dev)
    ws_tw = torch.empty(cvt.conv_proj_workspace_bytes(s_w.shape, 256, 6, 3, False, True), dtype=torch.uint8,
                        device=dev)

    def streamed():
        prev = None
        for xc, bb in zip(xs, bufs):
            cvt.haar3d_fwd(xc, bb["tl"], out=bb["hz"])
            cvt.causal_conv3d_fact(bb["hz"], w_s, None, workspace=ws_s, out=bb["s"])
            hist = None if prev is None else prev[:, :, -2:]
            cvt.causal_conv3d_temporal_stream(bb["s"], w_t, hist=hist, w_p=w_p, workspace=ws_t, out=bb["lat"])
            cvt.fsq_quantize(bb["lat"], indices=bb["idx"])
            prev = bb["s"]

    def whole():
        cvt.haar3d_fwd(x, 2, out=hz_w)
        cvt.causal_conv3d_fact(hz_w, w_s, None, workspace=ws_sw, out=s_w)
        cvt.causal_conv3d_fact_proj(s_w, None, w_t, w_p, workspace=ws_tw, out=lat_w)
        cvt.fsq_quantize(lat_w, indices=idx_w)

    for _ in range(max(3, min(args.warmup, 10))):
        streamed()
        whole()
    torch.cuda.synchronize()
    same = bool(torch.equal(torch.cat([bb["idx"] for bb in bufs], dim=1), idx_w))
    reps = max(3, args.steps // 4)
    out = {"clip": list(wl["x"]), "chunks_frames": [b - a for a, b, _ in cuts], "indices_equal_whole_clip": same}
    for name, fn in (("streamed", streamed), ("whole_clip", whole)):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        out[name] = {"ms": round(ms, 4), "frames_per_s": round(B * T / (ms * 1e-3), 1)}
    del x, xs, bufs, hz_w, s_w, lat_w, idx_w
    torch.cuda.empty_cache()
    return out


def clip_1080p_chain(cvt, si, torch, dev, args):
    """A 129-frame 1080p clip (1 x 3 x 129 x 1080 x 1920 bf16, G_trans pixels) through Haar ->
    spatial conv 192 -> 256 -> causal temporal conv 256 -> 256 with the 1x1 -> 16 fused: the
    spatial conv's 2.19 GB output is the temporal conv's input, so the row-tiled kernels run
    beyond 2 GiB.  Per-stage times with HIP events, MFMA fraction of each conv, frames/s."""
    wl = si.WORKLOADS["clip_1080p_129f"]
    B, C, T, H, W = wl["x"]
    Tq, Hq, Wq = 1 + (T - 1) // 4, H // 4, W // 4
    P = B * Tq * Hq * Wq
    log(f"1080p chain: generating {wl['x']} ...")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    del xb

    def bf(shape, seed):
        bits = si.to_bf16_bits(si.normal(shape, seed, 0.02))
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ws, wt, wp = bf((256, 192, 1, 3, 3), wl["seed"] + 1), bf((256, 256, 3, 1, 1), wl["seed"] + 2), \
        bf((16, 256, 1, 1, 1), wl["seed"] + 3)
    cl = torch.channels_last_3d
    hz = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    s1 = torch.empty((B, 256, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    lat = torch.empty((B, 16, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    w1 = torch.empty(cvt.conv_workspace_bytes(hz.shape, 256, 3, True, False), dtype=torch.uint8, device=dev)
    w2 = torch.empty(cvt.conv_proj_workspace_bytes(s1.shape, 256, 16, 3, False, True), dtype=torch.uint8, device=dev)
    stages = [("haar_fwd", lambda: cvt.haar3d_fwd(x, out=hz), None),
              ("spatial_192_256", lambda: cvt.causal_conv3d_fact(hz, ws, None, workspace=w1, out=s1),
               2.0 * 9 * 192 * 256 * P),
              ("temporal_256_256_proj16", lambda: cvt.causal_conv3d_fact_proj(s1, None, wt, wp, workspace=w2, out=lat),
               2.0 * 3 * 256 * 256 * P + 2.0 * 256 * 16 * P)]
    times = interleaved(torch, [fn for _, fn, _ in stages], max(2, args.steps // 4), rounds=4)
    out = {"clip": list(wl["x"]), "latent_grid": [Tq, Hq, Wq], "spatial_output_bytes": s1.numel() * 2, "stages": {}}
    for (name, _, flops), ms in zip(stages, times):
        d = {"ms": round(ms, 4)}
        if flops:
            d["TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
            d["mfma_frac"] = round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        else:
            d["GBps"] = round((2.0 * B * C * T * H * W + 2.0 * P * 192) / (ms * 1e-3) / 1e9, 1)
        out["stages"][name] = d
    out["frames_per_s"] = round(B * T / (sum(times) * 1e-3), 1)
    del x, hz, s1, lat, w1, w2
    torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where the file has none)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(xbits, zbits, ws_b, wt_b, pj_b, shape, width):
    """The float64 oracle on a strip of the clip (all frames, all rows, `width`
    pixel columns), scaled to the whole clip by the width ratio."""
    from threadpoolctl import threadpool_info

    from oracle import bf16 as obf16
    from oracle import conv as oconv
    from oracle import fsq as ofsq
    from oracle import haar as ohaar

    B, C, T, H, W = shape
    width = max(4, min(W, width - width % 4))
    wq = width // 4
    log(f"cpu baseline: oracle on a {T}x{H}x{width} strip ...")
    t0 = time.perf_counter()
    xs = obf16.decode(xbits[:, :, :, :, :width])
    hz = ohaar.haar3d_fwd(xs, 2)
    hzb = obf16.round_to_bf16(hz)
    y = oconv.causal_conv3d_fact(hzb, obf16.decode(ws_b), obf16.decode(wt_b))
    lat = oconv.pointwise(obf16.round_to_bf16(y), obf16.decode(pj_b))
    ofsq.quantize(obf16.round_to_bf16(lat))
    i2, _, _ = ofsq.quantize(obf16.decode(zbits[:, :, :, :, :wq]))
    ofsq.dequantize(i2)
    ohaar.haar3d_inv(hzb, 2)
    dt = time.perf_counter() - t0
    scale = W / width
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(B * T / (dt * scale), 4), "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"all {T} frames x {H} rows x {width} of {W} pixel columns (1/{scale:g} of the clip), "
                      f"{dt:.1f} s, scaled by {scale:g}; float64 NumPy, BLAS threads={threads}",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
