"""Batch-1 Dual-AR decode benchmark on one MI355X.

A step is one decoded frame (the Fast AR's nine greedy steps plus the Slow AR
step, i.e. every row of the hot path) of the full FishAudio S2 shape on
synthetic bf16 weights: 41-token prompt, then frames of greedy decode, one
stream ("s2pro-native", Where it stands, measures this workload).  The timed
region holds exactly K frames; weights, KV and state are resident in HBM.

Prints one JSON line.  --gpus N with N > 1 exits: the benchmark drives one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, weights, budget_s: float):
    """The oracle as it stands, on this host's cores: a one-token prompt, then
    whole frames (Fast loop + Slow step) until the budget is spent."""
    import numpy as np

    import oracle

    m = oracle.Model(cfg, weights)
    st = m.new_state()
    pre = st.prefill(np.array([7], np.int32))
    h, c0 = pre["h"], pre["c0"]
    frames = 0
    t0 = time.perf_counter()
    while True:
        fl = m.fast_loop(h)
        codes = np.concatenate([[c0], fl["codes"]]).astype(np.int32)
        s = st.slow_step(codes)
        h, c0 = s["h"], s["c0"]
        frames += 1
        if time.perf_counter() - t0 >= budget_s or frames + 2 >= cfg["max_context"]:
            break
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    from dual_ar_codec_amd import metrics
    wbytes = metrics.frame_bytes(cfg, 2)["total"]  # the frame's bf16-stored weights (+ a 2-position KV)
    return {"value": frames / dt, "unit": "frames/s", "cores": min(cores, os.cpu_count() or cores), "kind": "oracle",
            "sample": f"{frames} frames of the {cfg['name']} shape after a 1-token prompt ({dt:.1f} s, fp64 oracle)",
            "host": host_cpu(), "effective_host_gbps": round(wbytes * frames / dt / 1e9, 2),
            "ms_per_frame": round(dt / frames * 1e3, 2), "codebook_tok_s": round(10 * frames / dt, 2)}


def host_cpu():
    """Model name, sockets and logical CPUs of this host (from /proc/cpuinfo)."""
    model, sockets, cpus = None, set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "processor":
                    cpus += 1
                elif key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    sockets.add(val)
    except OSError:
        pass
    return {"model": model, "sockets": len(sockets) or None, "logical_cpus": cpus or os.cpu_count()}


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed FETCH_SIZE / WRITE_SIZE passes
    (profiles/gate_up_hbm_traffic.json), or None when the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gate_up_hbm_traffic.json")
    src = os.path.join(ROOT, "dual_ar_codec_amd", "csrc", "kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["kernels_hip_sha256"]:
                return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def multi_stream(args, w, log, kv_dtype="f32", weight_dtype="bf16"):
    """16 streams with ragged contexts (256..4096 random text positions, pages of 16 handed out in
    a scrambled order), then batched decode steps: one step = one frame for every stream."""
    import torch

    from dual_ar_codec_amd import metrics, s2ar, synth

    cfg = synth.config("multi_stream", kv_dtype=kv_dtype, weight_dtype=weight_dtype)
    lens = synth.prompt_lengths(cfg)
    n = cfg["n_streams"]
    ctx = s2ar.Context(cfg, w, max_streams=n)
    log(f"[bench] multi-stream prefill: {n} streams, {sum(lens)} positions")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(n):
        toks, _, _ = synth.make_prompt(cfg, s_)
        ctx.prefill(s_, toks)
    torch.cuda.synchronize()
    tp = time.perf_counter() - t0
    ids = list(range(n))
    ctx.decode_frames(ids, 2)  # warm-up (captures the batch graph)
    torch.cuda.synchronize()
    steps = args.multi_steps
    t0 = time.perf_counter()
    out = ctx.decode_frames(ids, steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert out.shape == (steps, n, 10)
    ctx.close()
    w_bytes = (metrics.int8_frame_bytes(cfg, 0) if weight_dtype in ("i8", "f8") else metrics.frame_bytes(cfg, 0))["weights"]
    kv = sum(metrics.kv_bytes_per_position(cfg) * (L + 2 + steps // 2 + 1) for L in lens)
    step_s = dt / steps
    return {"workload": f"{n} streams, contexts {min(lens)}..{max(lens)} (sum {sum(lens)}), {steps} batched steps",
            "frames_per_s": round(n / step_s, 1), "codebook_tok_s": round(10 * n / step_s, 1),
            "ms_per_step": round(step_s * 1e3, 3), "per_stream_rtf": round(metrics.rtf(1.0 / step_s), 5),
            "step_bytes": w_bytes + kv, "hbm_gbps": round((w_bytes + kv) / step_s / 1e9, 1),
            "hbm_frac": round((w_bytes + kv) / step_s / 1e9 / HBM_PEAK_GBPS, 4),
            "prefill_s": round(tp, 2), "kv_dtype": kv_dtype, "weight_dtype": weight_dtype,
            "note": "same synthetic weights as the batch-1 line (shapes identical); " + {
                "k_bf16": "bf16 keys and fp32 values: a quarter fewer KV bytes than fp32, inside the parity bar",
                "f32": "fp32 keys and values",
                "bf16": "bf16 keys and values halve the KV bytes but miss the 0.9999 hidden-cosine bar at full "
                        "shape (the fp64 oracle itself drifts 1 - 1.2e-4 with its cache rounded to bf16), so this "
                        "line is context only"}[kv_dtype]}


def prefix_sharing(ctx, vc, vt, vm, vcodes):
    """Time to first frame of the voice-clone prompt on a fresh stream, prefilled whole against
    sharing the 1000-position reference-audio prefix with a stream that already holds it and
    prefilling only the 200 text positions (streams 1 and 2, graphs captured beforehand)."""
    import torch

    n_pref = vc["prompt"]["n_vq"]
    for s_ in (1, 2):  # capture each stream's frame graph outside the timed region
        ctx.prefill(s_, vt[:64], vm[:64], vcodes[:64])
        ctx.decode_frames([s_], 1)
        ctx.release(s_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.prefill(1, vt, vm, vcodes)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ctx.decode_frames([1], 1)
    t2 = time.perf_counter()
    ctx.share_prefix(1, 2, n_pref)
    ctx.prefill(2, vt[n_pref:], vm[n_pref:], vcodes[n_pref:])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ctx.decode_frames([2], 1)
    t4 = time.perf_counter()
    ctx.release(1)
    ctx.release(2)
    return {"shared_positions": n_pref, "own_positions": len(vt) - n_pref,
            "full_prefill_ms": round((t1 - t0) * 1e3, 2), "full_first_frame_ms": round((t2 - t0) * 1e3, 2),
            "shared_prefill_ms": round((t3 - t2) * 1e3, 2), "shared_first_frame_ms": round((t4 - t2) * 1e3, 2)}


def slice_head(steps, cfg, w, toks, log):
    """Batch-1 frames/s with the semantic-slice Slow head (the 4096 semantic rows plus a stop row;
    the stop id stands in as the last text id) on the same weights and prompt."""
    import torch

    from dual_ar_codec_amd import metrics, s2ar

    cs = dict(cfg, head_slice=1, eos_id=cfg["vocab_text"] - 1)
    log("[bench] semantic-slice head")
    ctx = s2ar.Context(cs, w, max_streams=1)
    ctx.prefill(0, toks)
    ctx.decode_frames([0], 3)
    ctx.release(0)
    ctx.prefill(0, toks)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = ctx.decode_frames([0], steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ctx.close()
    fps = steps / dt
    H, K = cfg["slow"]["hidden"], cfg["codebook_size"]
    fb = metrics.frame_bytes(cfg, len(toks) + steps // 2)
    dropped = (cfg["vocab_slow"] - K - 1) * H * 2  # bf16 head rows not read
    total = fb["total"] - dropped
    gbps = total * fps / 1e9
    return {"workload": f"{cfg['name']}: {len(toks)}-token prompt, {steps} greedy frames, 1 stream",
            "frames_per_s": round(fps, 2), "ms_per_frame": round(dt / steps * 1e3, 4),
            "frame_bytes": total, "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "stopped_at_frame": int(next((t for t in range(steps) if out[t, 0, 0] < 0), -1)),
            "note": "Slow head reads 4097 rows instead of 155776; the picks are those of the full head"}


def mid_workload(log):
    """The mid Dual-AR (8 + 2 layers, hidden 1024, bf16): its 64-token prompt, then its 32 greedy
    frames timed as one call.  Its Fast working set (56.6 MB per step) fits in the 256 MB last-level
    cache, so its GB/s is effective, not HBM: a probe of the per-launch overhead of a frame graph."""
    import torch

    from dual_ar_codec_amd import metrics, s2ar, synth

    cfg = synth.config("mid")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = s2ar.Context(cfg, w, max_streams=1)
    ctx.prefill(0, toks)
    ctx.decode_frames([0], 3)
    ctx.release(0)
    ctx.prefill(0, toks)
    n = cfg["frames"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.decode_frames([0], n)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ctx.close()
    fb = metrics.frame_bytes(cfg, len(toks) + n // 2)
    log(f"[bench] mid: {n / dt:.1f} frames/s")
    return {"workload": f"mid: {len(toks)}-token prompt, {n} greedy frames, 1 stream",
            "frames_per_s": round(n / dt, 1), "ms_per_frame": round(dt / n * 1e3, 4),
            "frame_bytes": fb["total"], "effective_gbps": round(fb["total"] * n / dt / 1e9, 1),
            "note": "the Fast working set fits in the last-level cache: effective GB/s, not a roofline claim"}


def quant_weights(steps, fmt, cfg, w, toks, forced, ref, log):
    """Batch-1 frames/s with the layer matrices and heads as 8-bit codes (fmt "i8": int8, "f8": FP8
    E4M3) plus per-row scales (the same synthetic weights, quantised by the library at create), and
    the drift from bf16 on the same teacher-forced frames (the GPU against itself: hidden cosine,
    logit error, agreeing picks)."""
    import numpy as np
    import torch

    from dual_ar_codec_amd import metrics, s2ar

    name = "int8" if fmt == "i8" else "FP8 E4M3"
    c8 = dict(cfg, weight_dtype=fmt)
    log(f"[bench] {name} weights: quantise + upload")
    ctx = s2ar.Context(c8, w, max_streams=2)
    ctx.prefill(0, toks)
    ctx.decode_frames([0], 3)
    ctx.release(0)
    ctx.prefill(0, toks)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.decode_frames([0], steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    fps = steps / dt
    ctx.prefill(1, toks)
    got = [ctx.debug_frame(1, forced=f) for f in forced]
    ctx.close()

    def cos(a, b):
        a, b = a.astype(np.float64).ravel(), b.astype(np.float64).ravel()
        return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))

    h_cos = min(cos(g["slow_h"], r["slow_h"]) for g, r in zip(got, ref))
    fz_cos = min(cos(g["fast_z"], r["fast_z"]) for g, r in zip(got, ref))
    lrel = max(float(np.max(np.abs(g["slow_logits"] - r["slow_logits"])) / np.max(np.abs(r["slow_logits"])))
               for g, r in zip(got, ref))
    agree = float(np.mean([np.mean(g["own_codes"] == r["own_codes"]) for g, r in zip(got, ref)]))
    fb = metrics.int8_frame_bytes(c8, len(toks) + steps // 2)
    gbps = fb["total"] * fps / 1e9
    return {"workload": f"{cfg['name']}: {len(toks)}-token prompt, {steps} greedy frames, 1 stream",
            "frames_per_s": round(fps, 2), "ms_per_frame": round(dt / steps * 1e3, 4),
            "frame_bytes": fb["total"], "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "drift_vs_bf16": {"frames": len(forced), "min_cos_slow_h": round(h_cos, 6),
                              "min_cos_fast_z": round(fz_cos, 6), "max_slow_logit_rel": round(lrel, 5),
                              "own_pick_agreement": round(agree, 4)},
            "note": f"{name} layer matrices and heads, one fp32 scale per row; parity is checked against the "
                    "oracle fed the same quantisation, drift against the bf16 context on the same forced codes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="full")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--kernel-iters", type=int, default=144)
    ap.add_argument("--prefill", type=int, default=1, help="also time a 1200-position voice-clone prefill")
    ap.add_argument("--multi-steps", type=int, default=20, help="batched 16-stream decode steps (0 = skip)")
    ap.add_argument("--multi-lines", default="k_bf16,f32,bf16,int8",
                    help="which 16-stream lines to run: k_bf16 (the workload's), f32, bf16, int8")
    ap.add_argument("--copy-probe", type=int, default=0, help="run a 256 MiB copy (counter calibration)")
    ap.add_argument("--int8-steps", type=int, default=40, help="batch-1 frames with int8 weights (0 = skip)")
    ap.add_argument("--fp8-steps", type=int, default=40, help="batch-1 frames with FP8 E4M3 weights (0 = skip)")
    ap.add_argument("--slice-steps", type=int, default=60, help="batch-1 frames with the semantic-slice head (0 = skip)")
    ap.add_argument("--mid", type=int, default=1, help="also time the mid workload (32 frames)")
    ap.add_argument("--counter-pass", type=int, default=0,
                    help="for rocprofv3 --pmc passes (1): prefill, 2 frames enqueued without graphs, the voice-clone "
                         "prefill at both precisions (unless --prefill 0), the gate/up and "
                         "streaming-read launches (--kernel-iters each) and the 256 MiB copy probe, then exit; "
                         "(2): one eager batched step of the 16-stream workload and the copy probe")
    ap.add_argument("--prefix-share", type=int, default=1,
                    help="time to first frame of the voice-clone prompt with its 1000-position prefix shared")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py drives one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dual_ar_codec_amd import metrics, s2ar, synth

    torch.cuda.set_device(0)
    cfg = synth.config(args.config)
    n_prompt = synth.prompt_lengths(cfg)[0]
    vc = synth.config("voice_clone") if args.prefill else None
    vc_len = synth.prompt_lengths(vc)[0] if vc else 0
    vc_frames = vc["frames"] if vc else 0
    need = max(n_prompt + max(args.steps, args.warmup) + 1, vc_len + vc_frames + 2)
    if need > cfg["max_context"]:
        cfg = synth.config(args.config, max_context=(need + 63) // 64 * 64)
    log(f"[bench] generating {cfg['name']} weights ({synth.weight_bytes(cfg) / 1e9:.2f} GB)")
    t = time.perf_counter()
    w = synth.make_weights(cfg)
    log(f"[bench] weights in {time.perf_counter() - t:.1f} s; uploading")
    toks, mask, codes = synth.make_prompt(cfg)
    ctx = s2ar.Context(cfg, w, max_streams=3 if args.prefix_share else 2)
    if args.counter_pass == 2:
        # one batched step of the 16-stream workload (bf16 keys), enqueued eagerly (no graph), then
        # the copy probe
        mcfg = synth.config("multi_stream", kv_dtype="k_bf16")
        n = mcfg["n_streams"]
        ctx.close()
        mctx = s2ar.Context(mcfg, w, max_streams=n)
        for s_ in range(n):
            mt, _, _ = synth.make_prompt(mcfg, s_)
            mctx.prefill(s_, mt)
        mctx.debug_frame_batch(list(range(n)))
        mctx.close()
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": 2, "streams": n, "copy_bytes": 256 << 20}))
        return
    if args.counter_pass:
        ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
        out = ctx.decode_frames_noalloc(0, 2)
        if vc is not None:  # the voice-clone prefill (matrix-core GEMMs and attention, no graph), both precisions
            vt, vm, vcodes = synth.make_prompt(vc)
            ctx.prefill(1, vt, vm, vcodes)
            ctx.release(1)
            ctx.set_prefill_precision(1)
            ctx.prefill(1, vt, vm, vcodes)
            ctx.set_prefill_precision(0)
        ms, nbytes = ctx.time_kernel(0, args.kernel_iters)
        sms, sbytes = ctx.time_kernel(1, args.kernel_iters)
        ctx.close()
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": True, "frames": out.tolist(), "gate_up_us": round(ms * 1e3, 2),
                          "gate_up_bytes": nbytes, "stream_us": round(sms * 1e3, 2), "copy_bytes": 256 << 20}))
        return
    log("[bench] prefill + warmup")
    ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
    if args.warmup:
        ctx.decode_frames([0], args.warmup)
    ctx.release(0)
    ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} frames")
    t0 = time.perf_counter()
    out = ctx.decode_frames([0], args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert out.shape == (args.steps, 1, 10)
    fps = args.steps / dt
    ctx_mid = n_prompt + args.steps // 2
    fb = metrics.frame_bytes(cfg, ctx_mid)
    gbps = fb["total"] * fps / 1e9
    # the same frames again, each graph replay between its own pair of HIP events
    ctx.release(0)
    ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
    fms = np.sort(ctx.time_frames(0, args.steps).astype(np.float64))
    frame_events = {"frames": args.steps, "median_ms": round(float(np.median(fms)), 4),
                    "p10_ms": round(float(np.percentile(fms, 10)), 4), "p90_ms": round(float(np.percentile(fms, 90)), 4),
                    "min_ms": round(float(fms[0]), 4), "max_ms": round(float(fms[-1]), 4)}

    prefill = None
    if vc is not None:
        # voice-clone prompt (1000 VQ positions + 200 text positions) on a second stream: the
        # prefill's projections run as MFMA GEMMs
        vt, vm, vcodes = synth.make_prompt(vc)
        ctx.prefill(1, vt[:64], vm[:64], vcodes[:64])  # warm-up; the decode captures stream 1's frame graph
        ctx.decode_frames([1], 1)
        ctx.release(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.prefill(1, vt, vm, vcodes)
        torch.cuda.synchronize()
        pt = time.perf_counter() - t0
        s = cfg["slow"]
        lin = 2.0 * vc_len * s["n_layers"] * metrics.layer_matrix_params(s)
        att = 2.0 * 2 * s["n_layers"] * s["n_q_heads"] * s["head_dim"] * vc_len * (vc_len + 1) / 2
        prefill = {"positions": vc_len, "ms": round(pt * 1e3, 2), "tflop": round((lin + att) / 1e12, 3),
                   "tflop_s": round((lin + att) / pt / 1e12, 1), "peak_tflop_s": 2500.0,
                   "mfma_frac": round((lin + att) / pt / 1e12 / 2500.0, 4),
                   "note": "bf16 hi+lo split activations: 2 MFMA passes per algorithmic product"}
        # the voice-clone workload's decode: 200 frames at contexts 1201..1400
        t0 = time.perf_counter()
        ctx.decode_frames([1], vc_frames)
        torch.cuda.synchronize()
        dt_vc = time.perf_counter() - t0
        fb_vc = metrics.frame_bytes(cfg, vc_len + vc_frames // 2)
        prefill["decode"] = {"frames": vc_frames, "frames_per_s": round(vc_frames / dt_vc, 2),
                             "ms_per_frame": round(dt_vc / vc_frames * 1e3, 4), "frame_bytes": fb_vc["total"],
                             "hbm_frac": round(fb_vc["total"] * vc_frames / dt_vc / 1e9 / HBM_PEAK_GBPS, 4)}
        ctx.release(1)
        # the same prefill with one fp16 activation plane per product (prefill precision 1)
        ctx.set_prefill_precision(1)
        ctx.prefill(1, vt[:64], vm[:64], vcodes[:64])  # warm-up of the fp16 kernels
        ctx.release(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.prefill(1, vt, vm, vcodes)
        torch.cuda.synchronize()
        pt16 = time.perf_counter() - t0
        ctx.release(1)
        ctx.set_prefill_precision(0)
        prefill["fp16"] = {"ms": round(pt16 * 1e3, 2), "tflop_s": round((lin + att) / pt16 / 1e12, 1),
                           "mfma_frac": round((lin + att) / pt16 / 1e12 / 2500.0, 4),
                           "note": "prefill precision 1: activations, attention operands and softmax weights rounded "
                                   "once to fp16, weights taken as fp16, one fp16 MFMA pass per product"}
        if args.prefix_share:
            prefill["prefix_sharing"] = prefix_sharing(ctx, vc, vt, vm, vcodes)

    log("[bench] dominant kernel (fused RMSNorm + gate/up + SwiGLU GEMV)")
    ms, nbytes = ctx.time_kernel(0, args.kernel_iters)
    k_gbps = nbytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(k_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(),
                "kernel": "k_gemv2<bf16, NCH=5, GEMV_NORM_SWIGLU, R=2, WPB=8> (Slow gate/up, 19456x2560)",
                "bytes_per_launch": nbytes, "avg_launch_us": round(ms * 1e3, 2)}
    # context: a plain streaming read of the same weights, the rate no arithmetic slows down
    ctx.time_kernel(1, 4)  # first launches load the kernel's code object: not timed
    sms, sbytes = ctx.time_kernel(1, args.kernel_iters)
    s_gbps = sbytes / (sms * 1e-3) / 1e9
    roofline["stream_read_context"] = {"gbps": round(s_gbps, 1), "frac_of_peak": round(s_gbps / HBM_PEAK_GBPS, 4),
                                       "avg_launch_us": round(sms * 1e3, 2),
                                       "gemv_over_stream": round(k_gbps / s_gbps, 4)}
    # the whole frame against the same peak: the target is this figure, not the dominant kernel's
    roofline["frame"] = {"achieved": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "bytes_per_frame": fb["total"], "ms_per_frame": round(dt / args.steps * 1e3, 4),
                         "note": "algorithmic bytes of one whole frame (weights once, the Fast stack nine times, "
                                 "KV at the mid-run context) / measured ms per frame"}
    forced, ref = [], []
    if args.int8_steps > 0 or args.fp8_steps > 0:  # bf16 taps for the 8-bit drift, forced to this run's codes
        forced = [np.ascontiguousarray(out[t, 0]) for t in range(min(3, args.steps))]
        ctx.prefill(1, toks)
        ref = [ctx.debug_frame(1, forced=f) for f in forced]
        ctx.release(1)
    ctx.close()

    int8 = quant_weights(args.int8_steps, "i8", cfg, w, toks, forced, ref, log) if args.int8_steps > 0 else None
    fp8 = quant_weights(args.fp8_steps, "f8", cfg, w, toks, forced, ref, log) if args.fp8_steps > 0 else None
    sliced = slice_head(args.slice_steps, cfg, w, toks, log) if args.slice_steps > 0 else None
    mid = mid_workload(log) if args.mid else None

    multi = multi_f32 = multi_bf16 = multi_i8 = None
    lines = args.multi_lines.split(",") if args.multi_steps > 0 else []
    if "k_bf16" in lines:
        multi = multi_stream(args, w, log, "k_bf16")
    if "f32" in lines:
        multi_f32 = multi_stream(args, w, log, "f32")
    if "bf16" in lines:
        multi_bf16 = multi_stream(args, w, log, "bf16")
    if "int8" in lines:
        multi_i8 = multi_stream(args, w, log, "k_bf16", "i8")

    if args.copy_probe:
        # a plain 256 MiB device copy, the reference for scaling HBM byte counters
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] CPU oracle baseline ({args.cpu_budget:.0f} s budget)")
        cpu = cpu_baseline(cfg, w, args.cpu_budget)
        import oracle
        oracle.set_threads(1)  # the same oracle on one core, a shorter sample
        one = cpu_baseline(cfg, w, args.cpu_budget / 2)
        oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
        cpu["single_thread"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}

    line = {
        "metric": "frames/s at batch 1 (full S2 shape), with codebook tok/s, HBM GB/s and RTF",
        "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg["weight_dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: {n_prompt}-token prompt, {args.steps} greedy frames, 1 stream",
                   "slow_layers": cfg["slow"]["n_layers"], "fast_layers": cfg["fast"]["n_layers"],
                   "hidden": cfg["slow"]["hidden"], "prompt": n_prompt, "frames": args.steps, "streams": 1},
        "codebook_tok_s": round(metrics.codebook_tokens_per_s(fps), 1),
        "rtf": round(metrics.rtf(fps), 5),
        "frame_bytes": fb["total"],
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "frame_events": frame_events,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "multi_stream": multi,
        "multi_stream_f32_kv": multi_f32,
        "multi_stream_bf16_kv": multi_bf16,
        "multi_stream_int8": multi_i8,
        "int8": int8,
        "fp8": fp8,
        "semantic_slice_head": sliced,
        "mid": mid,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
