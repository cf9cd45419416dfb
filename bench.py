"""Benchmark: DDIM steps/s and clips/min of the batched two-stage denoiser on one
MI355X, 16 clips x 150 frames, classifier-free guidance (2 rows per clip), the
full 16 + 16 layer model with bf16 weights, seeded synthetic inputs.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload c2] [--no-cpu-baseline]
    python bench.py --workload timeline [--steps 3] [--warmup 1]
    python bench.py --workload fk [--steps 200] [--warmup 20]

A step is one DDIM iteration of the whole batch: root transformer, global ->
local root conversion, body transformer, CFG combine, DDIM update. The timed
region is one kimodo_sample call of exactly K steps (graph replays; per-call
set-up of the conditioning tokens included), bracketed by device syncs. After
it, kimodo_profile_step times every kernel of one step with HIP events that the
dispatch records on the launch stream; the dominant kernel's average gives the
roofline entry. Prints one JSON line on stdout.

The timeline workload times whole kimodo_sample_timeline calls instead (three
90-frame segments, 2 transition frames, 35 steps, 4 takes batched); --steps
counts timelines there, and its value is takes per minute. The fk workload
times kimodo_fk launches decoding 128 clips x 300 frames (--steps counts
launches) and reports frames per second.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "DDIM steps/sec and clips/min (batch 16x150 frames, 100 steps, CFG); % bf16 MFMA peak"

WORKLOADS = {
    "c2": dict(config=2, name="16 clips x 150 frames, 100-step DDIM, CFG (2 rows per clip), 16+16 layers, bf16 weights"),
    "c1": dict(config=1, name="1 clip x 150 frames, 100-step DDIM, CFG (2 rows per clip), 16+16 layers, bf16 weights"),
    "c3": dict(config=3, name="32 clips x <=180 frames (ragged 60..180), 50-step DDIM, CFG, 16+16 layers, bf16 weights"),
    "c4": dict(config=4, name="128 clips x 300 frames (25% padded 150..300), 100-step DDIM, CFG, 16+16 layers, bf16 weights"),
    "fk": dict(config=None, name="FK decode: 128 clips x 300 frames (38,400 frames), 30-joint skeleton, positions and "
                                 "rotation matrices, fp32"),
    "timeline": dict(config=None, name="timeline: 3 segments x 90 frames, 2 transition frames, 35-step DDIM, CFG, "
                                       "4 takes batched, 16+16 layers, bf16 weights"),
}
FK_METRIC = "FK decode frames/s (128 clips x 300 frames, 30 joints, positions + rotation matrices)"
FK_BYTES_PER_FRAME = (5 + 30 * 6) * 4 + 30 * (3 + 9) * 4  # features read + positions and rotations written
TIMELINE_METRIC = "timeline takes/min (3 x 3 s segments, 2 transition frames, 35-step DDIM, CFG, 4 takes batched)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name: str, lengths: np.ndarray) -> tuple:
    """Algorithmic work of one application to the whole batch (both guidance
    rows of every clip): (flops, bytes) on valid tokens only. The library runs
    each guidance group as its own launch, so a launch does half of this."""
    # split-K launches ("gemm_out:splitk") do the work of their GEMM; the
    # fused split-K reduction + add + LayerNorm counts as the LayerNorm
    name = {"add_layernorm_splitk": "add_layernorm"}.get(name.split(":")[0], name.split(":")[0])
    n = lengths.astype(np.int64) + 2  # tokens per sequence, both guidance rows
    Mv = int(2 * n.sum())
    D, F = 1024, 2048
    gemm = {"gemm_qkv": (3 * D, D), "gemm_out": (D, D), "gemm_ffn1_gelu": (F, D), "gemm_ffn2": (D, F)}
    if name in gemm:
        N, K = gemm[name]
        return 2 * Mv * N * K, 2 * (Mv * K + N * K + Mv * N)
    if name == "attention":
        return int(2 * (4 * n * n * D).sum()), 2 * Mv * 4 * D
    if name == "qkv_attention":  # fused QKV projection + attention (sequences of <= 160 tokens)
        return 2 * Mv * 3 * D * D + int(2 * (4 * n * n * D).sum()), 2 * (Mv * D + 3 * D * D + Mv * D)
    if name == "add_layernorm":
        return 0, 3 * Mv * D * 2
    return 0, 0


LAYER_KERNELS = ("gemm_qkv", "gemm_out", "gemm_ffn1_gelu", "gemm_ffn2", "attention", "qkv_attention",
                 "add_layernorm")


def cpu_baseline(ci: dict, clips: int = 3) -> dict:
    """The oracle as it stands, on a bounded sample: one DDIM step of `clips`
    clips (each a B = 1 run: both guidance rows, both sub-networks), scaled to
    the whole batch (clips are independent, each costs the same)."""
    from oracle import kimodo_oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") == "openblas"] or [1])
    except Exception:
        cores = os.cpu_count()
    nets = O.unpack_params(ci["weights"], ci["dims"])
    _, abar = O.linear_beta_schedule()
    t = int(O.ddim_timesteps(ci["steps"])[-1])
    times = []
    for b in range(clips):
        t0 = time.perf_counter()
        O.denoise_step(nets, ci["dims"], ci["noise"][b:b + 1], ci["text"][b:b + 1], ci["lengths"][b:b + 1], t,
                       abar[t], abar[t - 1], ci["cfg_scale"])
        times.append(time.perf_counter() - t0)
    per_clip_step = float(np.median(times))
    steps_per_s = 1.0 / (per_clip_step * ci["B"])
    return {"value": round(steps_per_s, 6), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"numpy fp64 oracle, one DDIM step (t={t}) of {clips} of the {ci['B']} clips run one at a "
                      f"time (median {per_clip_step:.2f} s per clip-step), scaled x{ci['B']} to the batch",
            "clips_per_min": round(60.0 * steps_per_s / ci["steps"] * ci["B"], 4)}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "text_motion_diffusion_amd", "csrc", rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


def profile_kernels(K, sess, B, T, noise, text, lengths, cfg_scale, L, profile_steps, stream):
    """Per-kernel times of profiled steps (HIP events recorded by each dispatch
    on the launch stream) and the dominant kernel's roofline entry."""
    _, abar_full = K.kimodo_make_schedule(100, 1e-4, 0.02, 100)
    per = {}
    x = noise.clone()
    for i in range(profile_steps):
        t = 99 - i
        recs = K.kimodo_profile_step(sess.ctx, B, T, x, text, lengths, t, float(abar_full[t]),
                                     float(abar_full[t - 1]), cfg_scale, x, stream=stream)
        for name, ms in recs:
            per.setdefault(name, []).append(ms)
    steps_prof = max(profile_steps, 1)
    # applications of each layer kernel to the whole batch per step: L + L
    # layers, two LayerNorms per layer
    applications = {"add_layernorm": 4 * L}
    kernels = {}
    for name, v in per.items():
        launches = len(v) // steps_prof
        base = {"add_layernorm_splitk": "add_layernorm"}.get(name.split(":")[0], name.split(":")[0])
        share = applications.get(base, 2 * L) / launches if base in LAYER_KERNELS else 1.0
        flops, nbytes = (w * share for w in kernel_work(name, lengths))
        avg = float(np.mean(v))
        k = {"avg_ms": round(avg, 5), "launches_per_step": launches, "ms_per_step": round(sum(v) / steps_prof, 4),
             "work_per_launch": int(flops or nbytes)}
        if flops:
            k["tflops"] = round(flops / avg / 1e9, 1)
            k["mfma_frac"] = round(flops / avg / 1e9 / PEAK_MFMA_TFLOPS, 4)
        elif nbytes:
            k["gbs"] = round(nbytes / avg / 1e6, 1)
            k["hbm_frac"] = round(nbytes / avg / 1e6 / PEAK_HBM_GBS, 4)
        kernels[name] = k
    dominant = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    flops, nbytes = kernel_work(dominant, lengths)
    flops, nbytes = (flops and kernels[dominant]["work_per_launch"]), (nbytes and kernels[dominant]["work_per_launch"])
    avg_s = kernels[dominant]["avg_ms"] / 1e3
    if flops:
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2),
                "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(flops / avg_s / 1e12 / PEAK_MFMA_TFLOPS, 4)}
    else:
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(nbytes / avg_s / 1e9 / PEAK_HBM_GBS, 4)}
    roof["traffic"] = None
    roof["work_per_launch"] = flops if flops else nbytes
    mm_flops = sum(kernels[n]["work_per_launch"] * kernels[n]["launches_per_step"] for n in kernels
                   if kernel_work(n, lengths)[0])
    mm_ms = sum(kernels[n]["ms_per_step"] for n in kernels if kernel_work(n, lengths)[0])
    prof_ms = sum(k["ms_per_step"] for k in kernels.values())
    log("bench: per-kernel (profiled step): " + json.dumps(kernels))
    return kernels, roof, mm_flops, mm_ms, prof_ms


def bench_timeline(args, wl):
    """Whole timelines: kimodo_sample_timeline of V takes, segments one after
    another, each segment's first frames carried over from the previous one."""
    import torch

    from synthetic.inputs import TIMELINE, Dims, bf16_bits_to_f32, make_weights, round_to_bf16_bits, timeline_inputs
    from text_motion_diffusion_amd import kimodo as K
    from text_motion_diffusion_amd.session import Session

    tl = TIMELINE
    V, frames, n_tr, S, w = tl["V"], list(tl["frames"]), tl["n_transition"], tl["steps"], tl["cfg_scale"]
    dims = Dims()
    L = dims.layers_root
    bits = [round_to_bf16_bits(a) for a in make_weights(dims)]
    inp = timeline_inputs(V, frames, dims)
    dev = torch.device("cuda:0")
    log(f"bench: workload timeline: {wl['name']}; timelines={args.steps} warmup={args.warmup}")
    sess = Session(bits, L, L, V, max(frames), max_steps=S, dtype=K.KIMODO_BF16)
    text = torch.from_numpy(inp["text"]).to(dev)
    noise = [torch.from_numpy(n).to(dev) for n in inp["noise"]]
    ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, S)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        sess.sample_timeline(frames, text, noise, n_tr, ts, ab, w)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        out = sess.sample_timeline(frames, text, noise, n_tr, ts, ab, w)
    ev1.record(stream)
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")
    ms_per_timeline = ev0.elapsed_time(ev1) / args.steps
    passes = len(frames) * S
    ms_per_step = ms_per_timeline / passes
    takes_per_min = 60e3 * V / ms_per_timeline
    log(f"bench: {ms_per_timeline:.1f} ms per timeline of {V} takes ({passes} denoiser passes, "
        f"{ms_per_step:.3f} ms each); {takes_per_min:.1f} takes/min")
    lengths = np.full(V, frames[0], np.int32)
    kernels, roof, mm_flops, _, _ = profile_kernels(K, sess, V, frames[0], noise[0], text[0], lengths, w, L,
                                                    args.profile_steps, stream)
    cpu = None
    if not args.no_cpu_baseline:
        sess.close()
        del sess
        torch.cuda.empty_cache()
        log("bench: timing the CPU oracle on a bounded sample ...")
        ci = dict(weights=[bf16_bits_to_f32(b) for b in bits], dims=dims, steps=S,
                  noise=inp["noise"][0], text=inp["text"][0], lengths=lengths, cfg_scale=w, B=V)
        one = cpu_baseline(ci)
        # the oracle's per-clip step rate, scaled to whole takes of len(frames) x S passes
        per_clip_step = 1.0 / (one["value"] * V)
        cpu = {"value": round(60.0 / (per_clip_step * passes), 6), "unit": "takes/min", "cores": one["cores"],
               "kind": "oracle",
               "sample": one["sample"].replace(f"scaled x{V} to the batch",
                                               f"scaled to a take of {passes} denoiser passes")}
    line = {
        "metric": TIMELINE_METRIC,
        "value": round(takes_per_min, 2),
        "unit": "takes/min",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_timeline": round(ms_per_timeline, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "takes": V, "segment_frames": frames, "transition_frames": n_tr,
                   "ddim_steps": S, "cfg_scale": w, "layers": f"{L}+{L}",
                   "weights": "bf16 (matrices converted once to fp16)",
                   "compute": "fp16 MFMA operands, fp32 accumulation", "parallelism": "single GPU"},
        "mfma_frac_step": round(mm_flops / (ms_per_step / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_fk(args, wl):
    """kimodo_fk launches over the largest workload's output shape; HIP events
    on the launch stream around every launch."""
    import torch

    from synthetic.inputs import make_skeleton
    from text_motion_diffusion_amd import kimodo as K

    n = 128 * 300
    _, parents, offsets = make_skeleton()
    motion_h = np.random.default_rng(5).standard_normal((n, 279)).astype(np.float32)
    dev = torch.device("cuda:0")
    motion = torch.from_numpy(motion_h).to(dev)
    pos = torch.empty((n, 30, 3), device=dev)
    rot = torch.empty((n, 30, 3, 3), device=dev)
    stream = torch.cuda.current_stream()
    log(f"bench: workload fk: {wl['name']}; launches={args.steps} warmup={args.warmup}")
    for _ in range(args.warmup):
        K.kimodo_fk(n, motion, parents, offsets, pos, rot, stream=stream)
    torch.cuda.synchronize()
    # back-to-back launches between one event pair on the launch stream (an
    # event pair around every launch adds microseconds to a ~25 us kernel)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        K.kimodo_fk(n, motion, parents, offsets, pos, rot, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    avg_ms = ev0.elapsed_time(ev1) / args.steps
    frames_per_s = n / (avg_ms / 1e3)
    nbytes = n * FK_BYTES_PER_FRAME
    log(f"bench: fk {avg_ms * 1e3:.1f} us per launch, {nbytes / (avg_ms / 1e3) / 1e9:.0f} GB/s algorithmic")
    if not torch.isfinite(pos).all():
        raise RuntimeError("non-finite output")
    roof = {"kernel": "fk", "bound": "hbm", "achieved": round(nbytes / (avg_ms / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(nbytes / (avg_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": traffic_for("fk", args.workload), "work_per_launch": nbytes}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import kimodo_fk as FK

        log("bench: timing the CPU oracle on a bounded sample ...")
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 2.0:
            FK.forward_kinematics(motion_h, parents, offsets)
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * n / dt, 1), "unit": "frames/s", "cores": 1, "kind": "oracle",
               "sample": f"numpy fp64 FK oracle over all {n} frames, {reps} times ({dt:.2f} s)"}
    line = {
        "metric": FK_METRIC,
        "value": round(frames_per_s, 0),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": wl["name"], "frames": n, "joints": 30, "skeleton": "seeded 30-joint stand-in"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="DDIM steps to time (default 100); timelines for "
                                                             "--workload timeline (default 3)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10); timelines (default 1)")
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB, so hardware-counter runs can "
                         "scale FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (data parallel over clips would "
              "need no collective per step; see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from synthetic.inputs import config_inputs
    from text_motion_diffusion_amd import kimodo as K
    from text_motion_diffusion_amd.session import Session

    timeline = args.workload == "timeline"
    if args.steps is None:
        args.steps = {"timeline": 3, "fk": 200}.get(args.workload, 100)
    if args.warmup is None:
        args.warmup = {"timeline": 1, "fk": 20}.get(args.workload, 10)
    if args.steps < 1:
        ap.error("--steps must be >= 1")

    if args.calibration_copy_mb > 0:
        n = args.calibration_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: calibration copy of {args.calibration_copy_mb} MiB done")
        del src, dst

    wl = WORKLOADS[args.workload]
    if timeline:
        bench_timeline(args, wl)
        return
    if args.workload == "fk":
        bench_fk(args, wl)
        return
    ci = config_inputs(wl["config"])
    B, T, L = ci["B"], ci["T"], ci["layers"]
    lengths = ci["lengths"]
    dev = torch.device("cuda:0")
    log(f"bench: workload {args.workload}: {wl['name']}; steps={args.steps} warmup={args.warmup}")
    sess = Session(ci["weight_bits"], L, L, B, T, max_steps=100, dtype=K.KIMODO_BF16)
    noise = torch.from_numpy(ci["noise"]).to(dev)
    text = torch.from_numpy(ci["text"]).to(dev)
    out = torch.empty_like(noise)
    stream = torch.cuda.current_stream()

    def run_steps(n):
        done = 0
        while done < n:
            s = min(100, n - done)
            ts, ab = K.kimodo_make_schedule(100, 1e-4, 0.02, s)
            sess.sample(noise, text, lengths, ts, ab, ci["cfg_scale"], out=out)
            done += s

    if args.warmup > 0:
        run_steps(args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    run_steps(args.steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    steps_per_s = 1000.0 / ms_per_step
    log(f"bench: {args.steps} steps in {gpu_ms:.2f} ms (events), {wall * 1e3:.2f} ms (host); "
        f"{ms_per_step:.3f} ms/step, {steps_per_s:.1f} steps/s")
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")

    kernels, roof, mm_flops, mm_ms, prof_ms = profile_kernels(K, sess, B, T, noise, text, lengths, ci["cfg_scale"],
                                                              L, args.profile_steps, stream)
    roof["traffic"] = traffic_for(roof["kernel"], args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        sess.close()
        del sess
        torch.cuda.empty_cache()
        log("bench: timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(ci)

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "global_batch": B, "frames": T, "tokens_per_row": T + 2,
                   "cfg_rows": 2 * B, "ddim_steps": ci["steps"], "cfg_scale": ci["cfg_scale"],
                   "layers": f"{L}+{L}", "weights": "bf16 (matrices converted once to fp16)",
                   "compute": "fp16 MFMA operands, fp32 accumulation", "parallelism": "single GPU"},
        "clips_per_min": round(60.0 * steps_per_s / ci["steps"] * B, 1),
        # GEMM + attention flops over their summed kernel time (kernels timed one at a time)
        "mfma_frac_gemm_attention": round(mm_flops / (mm_ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4) if mm_ms else None,
        # the whole step: all GEMM + attention flops over the measured step time
        "mfma_frac_step": round(mm_flops / (ms_per_step / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "profiled_ms_per_step": round(prof_ms, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
