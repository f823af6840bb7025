"""Throughput of the per-frame decode step (one talker step + 15 code-predictor
micro-steps) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload bf16_b1]

A step is one qt_decode_frame call of `frames_per_step` frames for every
stream of the workload, always from the same prefilled state (the slot state
is restored before each step, so every step decodes the same positions).
Prints one JSON line.  Inputs are seeded and synthetic (weights N(0, 0.02));
they are resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
CSRC = os.path.join(ROOT, "autoregressive_codebook_tts_frame_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "frame_kernel_bf16_b1_traffic.json")


def kernel_source_hash() -> str:
    """sha256 of the persistent kernel's sources (frame.hip, frame.h)."""
    h = hashlib.sha256()
    for name in ("frame.hip", "frame.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, frames: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on this kernel source and workload; else None."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_source_hash() or t.get("workload") != workload or t.get("frames_per_step") != frames:
        return None
    return float(t["bytes_per_launch"])


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def frame_bytes(m, batch: int, mean_len: float) -> float:
    """Algorithmic bytes of one frame-step for `batch` streams: talker weights
    once, predictor weights for each of its 15 passes, every head once, K/V
    reads over valid positions only (talker: mean_len per layer; predictor:
    2 + 3 + ... + 16 positions per layer), K/V row writes and the gathered
    table rows.  The padded window tail and norm gains are not counted."""
    wb = {0: 4.0, 1: 2.0, 2: 34.0 / 32.0, 3: 18.0 / 32.0}[m.lin]
    tb = 2.0 if m.tab_bf16 else 4.0
    kvb = 2.0 if m.kv_bf16 else 4.0
    layer = (m.nqkv * m.H + m.H * m.nq * m.hd + 3 * m.F * m.H) * wb
    heads = m.G * m.Vc * m.H * wb
    weights = m.Lt * layer + (m.G - 1) * m.Lp * layer + heads
    kv_row = 2 * m.nkv * m.hd * kvb
    pred_positions = sum(range(2, m.G + 1))
    kv_read = batch * (m.Lt * mean_len + m.Lp * pred_positions) * kv_row
    kv_write = batch * (m.Lt + m.Lp * m.G) * kv_row
    gathers = batch * (m.G + 1 + m.G - 1) * m.H * tb
    return weights + kv_read + kv_write + gathers


def cpu_baseline(m, w, wl, frames_budget_s: float = 15.0, temperature: float = 0.0, seed: int = 0, top_k: int = 0):
    """The oracle as it stands, on the host cores: prefill (untimed) then as
    many frames as fit in the budget (at least 1)."""
    from autoregressive_codebook_tts_frame_amd import synth
    from oracle import Oracle

    o = Oracle(m, w, 1, pcap=wl.prompt + 64 + 1)
    if temperature:
        o.set_sampler(temperature, seed, top_k)
    codes, text = synth.make_prompt(wl, 0)
    t = time.time()
    o.prefill(0, codes, text)
    log(f"cpu baseline: oracle prefill {time.time() - t:.1f}s")
    ov = synth.make_overlays(wl, 64)
    n, t0 = 0, time.time()
    while n < 64:
        o.decode(1, ov[n:n + 1])
        n += 1
        if time.time() - t0 > frames_budget_s:
            break
    dt = time.time() - t0
    threads = o.lib.orc_num_threads()
    o.close()
    return {"value": n / dt, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} frames of {wl.name} (batch 1) after an untimed {wl.prompt}-row oracle prefill, "
                      f"{dt:.1f}s on {threads} threads"}


def talker_weight_bytes(m) -> float:
    """Talker projection weights plus its head: what one prefill chunk streams."""
    wb = {0: 4.0, 1: 2.0, 2: 34.0 / 32.0, 3: 18.0 / 32.0}[m.lin]
    layer = (m.nqkv * m.H + m.H * m.nq * m.hd + 3 * m.F * m.H) * wb
    return m.Lt * layer + m.Vc * m.H * wb


PF_CHUNK, PF_MIN, PF_STREAMS = 512, 16, 4  # the library's prompt-chunk rows, smallest bucket, streams per call


def prompt_chunks(lens, P):
    """Chunks (streams, rows per stream) of one qt_prefill_rows call, as the
    library plans them: the same positions of every stream still going, a
    power-of-two token bucket, at most PF_CHUNK rows in all."""
    out, r0, act = [], 0, list(lens)
    while act:
        cap = PF_CHUNK
        while cap * len(act) > PF_CHUNK:
            cap //= 2
        t = PF_MIN
        while t < max(act) - r0 and t < cap:
            t *= 2
        t = min(t, P - r0)
        out.append((len(act), t))
        r0 += t
        act = [L for L in act if L > r0]
    return out


def ttfa(args, d, m, wl, B):
    """Time to first frame: the prompts' prefill (qt_prefill_rows, up to 4
    streams of similar length per call, in prompt chunks that replay a graph
    per shape) then one qt_decode_frame.  Host wall clock around each step
    (both calls are synchronous)."""
    import numpy as np
    from autoregressive_codebook_tts_frame_amd import synth

    ctx = synth.make_context_lengths(wl)  # the workload's (ragged) prompt lengths
    prompts = [synth.make_prompt(wl, b, T=int(ctx[b])) for b in range(B)]
    ov = synth.make_overlays(wl, 1, B)
    order = sorted(range(B), key=lambda b: len(prompts[b][1]))
    groups = [order[i:i + PF_STREAMS] for i in range(0, B, PF_STREAMS)]

    def prefill_all():
        for g in groups:
            d.prefill_rows(g, [prompts[b][0] for b in g], [prompts[b][1] for b in g])

    def step():  # one frame, whatever the frames per replay (adaptive K: a 1-frame graph)
        prefill_all()
        d.decode(1, ov)

    for _ in range(args.warmup):
        step()
    times = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    # the prefill alone, for its roofline: the talker weights once per prompt chunk
    pre = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        prefill_all()
        pre.append(time.perf_counter() - t0)
    T = int(np.mean([len(t) for _, t in prompts]))  # (mean prompt rows, for the record)
    chunks = sum(len(prompt_chunks([len(prompts[b][1]) for b in g], m.P)) for g in groups)
    wbytes = talker_weight_bytes(m)
    ms = 1e3 * float(np.median(times))
    pre_ms = 1e3 * float(np.median(pre))
    achieved = chunks * wbytes / (pre_ms * 1e-3) / 1e9
    return {
        "metric": f"time to first frame (prefill of {T} rows + 1 frame)", "value": ms, "unit": "ms",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": {0: "f32", 1: "bf16", 2: "q8_0+bf16", 3: "q4+bf16"}[m.lin],
        "data": "synthetic (seeded N(0,0.02) weights, uniform codes and text ids)",
        "config": {"workload": wl.name + "_ttfa", "batch": B, "prompt": T, "prefill_chunk": PF_CHUNK,
                   "prompt_chunks": chunks, "streams_per_prefill_call": min(B, PF_STREAMS),
                   "path": "per-op prefill + " + {1: "persistent frame kernel", 2: "per-op hipGraph",
                                                  3: "per-op eager"}[d.path]},
        "prefill_ms": pre_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "prefill (talker weights streamed once per prompt chunk)",
                     "bytes_per_launch": chunks * wbytes, "avg_launch_us": pre_ms * 1e3},
        "cpu_baseline": None,
    }


def setup(qt, synth, wl, dw, nf, flags, args, paged=False):
    """A decoder for wl with every stream prefilled from its seeded prompt;
    returns it, the context lengths, the slot states and the overlay ids.
    paged: a paged talker ring holding exactly the prompts plus nf frames of
    every stream (a step restores the states, so its rows are reused)."""
    B = wl.batch
    ctx = synth.make_context_lengths(wl)  # ragged per-stream contexts where the workload has them
    pool = int(sum(int(c) for c in ctx)) + B * nf if paged else 0
    d = qt.Decoder(wl.model, dw, B, frames_per_replay=wl.frames_per_replay, max_frames_per_call=nf, flags=flags,
                   pool_rows=pool)
    if args.temperature:
        d.set_sampler(args.temperature, args.seed, top_k=args.top_k)
    lens = []
    for b in range(B):
        codes, text = synth.make_prompt(wl, b, T=int(ctx[b]))
        d.prefill(b, codes, text)
        lens.append(len(text))
    states = [d.get_state(b) for b in range(B)]
    ov = synth.make_overlays(wl, nf, B)
    log("prefill done")
    return d, lens, states, ov


def time_steps(d, states, ov, nf, steps, warmup):
    """Warm up, then time `steps` steps between HIP events on the library's
    stream and the host clock; a step restores every slot's state and
    decodes nf frames.  Returns (wall seconds, event seconds)."""
    import torch

    def step():
        for b, (pos, c0, br) in enumerate(states):
            d.set_state(b, pos, c0, br)
        return d.decode(nf, ov)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {steps} steps")
    t0 = time.perf_counter()
    ev0.record(d.stream)
    for _ in range(steps):
        step()
    ev1.record(d.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / 1e3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="bf16_b1")
    ap.add_argument("--frames", type=int, default=None, help="frames per step (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ops", action="store_true", help="force the per-op hipGraph path")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="sample every code at this temperature (0: greedy, the default)")
    ap.add_argument("--seed", type=int, default=42, help="sampler seed")
    ap.add_argument("--top-k", type=int, default=0, help="with --temperature: only the k largest logits compete "
                                                          "(per-op path: use with --ops for one stream)")
    ap.add_argument("--frames-per-replay", type=int, default=None,
                    help="frames per graph replay on the per-op path (default: the workload's)")
    ap.add_argument("--ttfa", action="store_true",
                    help="time to first frame instead: a step is the prompt prefill of every stream plus "
                         "one decoded frame")
    ap.add_argument("--paged", action="store_true",
                    help="decode on a paged talker ring holding exactly the streams' contexts (per-op path)")
    ap.add_argument("--no-b32", action="store_true",
                    help="skip the 32-stream leg that the default run times after the batch-1 workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device-to-device three times (a plain copy kernel "
                         "of known size, to scale hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build decodes on a single MI355X and has no "
              "multi-GPU path (streams would shard by slot with no exchange; see DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from autoregressive_codebook_tts_frame_amd import qt, synth

    wl = synth.WORKLOADS[args.workload]
    m = wl.model
    B = wl.batch
    nf = args.frames or wl.frames
    log(f"workload {wl.name}: B={B}, prompt {wl.prompt}, {nf} frames/step; drawing weights")
    t = time.time()
    w = synth.make_weights(m)
    log(f"weights drawn in {time.time() - t:.1f}s; uploading")
    if args.frames_per_replay:
        import dataclasses
        wl = dataclasses.replace(wl, frames_per_replay=args.frames_per_replay)
    dw = qt.DeviceWeights(m, w, "cuda")
    d, lens, states, ov = setup(qt, synth, wl, dw, nf, qt.QT_F_OPS if args.ops else 0, args, paged=args.paged)
    if args.ttfa:
        print(json.dumps(ttfa(args, d, m, wl, B)), flush=True)
        d.close()
        return

    wall, gpu_s = time_steps(d, states, ov, nf, args.steps, args.warmup)
    frames = B * nf * args.steps
    ms_per_step = 1e3 * wall / args.steps
    mean_len = float(np.mean(lens)) + (nf + 1) / 2.0
    fb = frame_bytes(m, B, mean_len)
    ms_per_frame_step = 1e3 * wall / (nf * args.steps)

    path = d.path
    if path == qt.QT_PATH_FRAME:
        # dominant kernel: the persistent frame kernel, one launch per step;
        # its average duration from the HIP events on the library's stream
        # around the timed region (the step's id copies are on the same stream)
        kname = "frame_kernel (persistent: every phase of a step's frames)"
        us = gpu_s * 1e6 / args.steps
        kbytes = fb * nf
    else:
        # dominant kernel: the gate/up projection, timed live with HIP events
        # on the library's stream over every layer's weights
        batched = m.lin != 0 and m.act_bf16  # bf16 / q8 / q4 projections take the GEMM at any row count
        kname = ("gemm_kernel<gated> (MFMA: RMSNorm + gate/up + SiLU-mul, %d rows)" % B if batched
                 else "gemv_kernel<gated> (RMSNorm + gate/up + SiLU-mul)")
        us, kbytes = d.time_kernel(qt.QT_KERNEL_GEMV_GATE_UP, 3)
    achieved = kbytes / (us * 1e-6) / 1e9
    log(f"path {path}: {frames / wall:.1f} frames/s, {ms_per_frame_step:.3f} ms per frame-step; "
        f"{kname}: {us:.1f} us/launch = {achieved:.0f} GB/s")
    d.close()

    # the achievable HBM read bandwidth, measured in the same run: a plain
    # streaming-read kernel over 4 GiB (far above the 256 MB last-level cache)
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2 << 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sread_us = qt.qt_stream_read(src, sink, 5)
    achievable = src.numel() / (sread_us * 1e-6) / 1e9
    del src, sink
    log(f"streaming read: {achievable:.0f} GB/s ({achievable / HBM_PEAK_GBS:.3f} of the 8 TB/s peak)")

    # the 32-stream workload, timed in the same run (the metric is quoted at
    # batch 1 and at 32 streams)
    b32 = None
    if args.workload == "bf16_b1" and not args.no_b32 and not args.frames:
        wl32 = synth.WORKLOADS["bf16_b32"]
        nf32 = wl32.frames
        log(f"workload {wl32.name}: B={wl32.batch}, ragged contexts, {nf32} frames/step, "
            f"{wl32.frames_per_replay} frames per graph replay")
        d32, lens32, states32, ov32 = setup(qt, synth, wl32, dw, nf32, 0, args)
        wall32, gpu32 = time_steps(d32, states32, ov32, nf32, args.steps, args.warmup)
        fb32 = frame_bytes(m, wl32.batch, float(np.mean(lens32)) + (nf32 + 1) / 2.0)
        ms32 = 1e3 * wall32 / (nf32 * args.steps)
        b32 = {"workload": wl32.name, "value": wl32.batch * nf32 * args.steps / wall32, "unit": "frames/s",
               "ms_per_frame_step": ms32, "steps": args.steps, "warmup": args.warmup,
               "batch": wl32.batch, "frames_per_step": nf32, "frames_per_replay": wl32.frames_per_replay,
               "path": {1: "persistent frame kernel", 2: "per-op hipGraph", 3: "per-op eager"}[d32.path],
               "mean_context": float(np.mean(lens32)),
               "frame_roofline": {"bytes_per_frame_step": fb32, "achieved_gbs": fb32 / (ms32 * 1e-3) / 1e9,
                                  "frac": fb32 / (ms32 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "frac_of_achievable": fb32 / (ms32 * 1e-3) / 1e9 / achievable},
               "gpu_event_s": gpu32, "wall_s": wall32}
        log(f"{wl32.name}: {b32['value']:.1f} frames/s, {ms32:.3f} ms per frame-step, "
            f"{b32['frame_roofline']['frac']:.3f} of HBM peak")
        dense_ring = int(d32.ring.numel())
        d32.close()
        # the same 32 streams on a paged ring (page size 1) holding exactly
        # their contexts: its memory against the dense rings', and its rate
        d32, lens32, states32, ov32 = setup(qt, synth, wl32, dw, nf32, 0, args, paged=True)
        wallp, gpup = time_steps(d32, states32, ov32, nf32, args.steps, args.warmup)
        b32["paged"] = {"value": wl32.batch * nf32 * args.steps / wallp, "unit": "frames/s",
                        "ms_per_frame_step": 1e3 * wallp / (nf32 * args.steps), "pool_rows": d32.pool_rows,
                        "ring_bytes": int(d32.ring.numel()), "dense_ring_bytes": dense_ring,
                        "gpu_event_s": gpup, "wall_s": wallp}
        log(f"{wl32.name} paged: {b32['paged']['value']:.1f} frames/s, ring {d32.ring.numel() / 2**30:.2f} GiB "
            f"against {dense_ring / 2**30:.2f} GiB dense")
        d32.close()

    res = {
        "metric": "codec frames/s (talker step + 15 predictor steps)",
        "value": frames / wall,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "q8_0+bf16", 3: "q4+bf16"}[m.lin],
        "data": "synthetic (seeded N(0,0.02) weights, uniform codes and text ids)",
        "config": {"workload": wl.name, "batch": B, "prompt": wl.prompt, "frames_per_step": nf,
                   "path": {1: "persistent frame kernel", 2: "per-op hipGraph", 3: "per-op eager"}[path],
                   "frames_per_replay": wl.frames_per_replay, "talker_layers": m.Lt,
                   "predictor_layers": m.Lp, "hidden": m.H,
                   "sampler": (f"temperature {args.temperature}, seed {args.seed}"
                               + (f", top-k {args.top_k}" if args.top_k else "")) if args.temperature else "greedy"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name, nf) if path == qt.QT_PATH_FRAME else None,
                     "kernel": kname,
                     "bytes_per_launch": kbytes, "avg_launch_us": us,
                     "achievable_gbs": achievable, "frac_of_achievable": achieved / achievable},
        "frame_roofline": {"bytes_per_frame_step": fb, "ms_per_frame_step": ms_per_frame_step,
                           "achieved_gbs": fb / (ms_per_frame_step * 1e-3) / 1e9,
                           "frac": fb / (ms_per_frame_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "gpu_event_s": gpu_s, "wall_s": wall},
        "cpu_baseline": None,
        "b32": b32,
    }
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 device copies of {n} bytes")
        del src, dst
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(m, w, wl, temperature=args.temperature, seed=args.seed, top_k=args.top_k)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
