#!/usr/bin/env python3
"""Benchmark of the MoT world-action-model forward pass on one MI355X.

One "step" is one whole inference through the C ABI: the video expert once,
then S Euler steps of the action expert, in the wavefront (CEWP) schedule on
two HIP streams, inputs already in HBM.  It is timed as eager launches
(wam_infer_cewp) and as a replay of the same inference captured once into a
HIP graph (wam_graph_create / wam_graph_launch), each with the host running
ahead and in a closed loop (the host waits for each inference before the
next, as a control loop does); the fastest is the headline and the config
names which.

    python bench.py [--steps K] [--warmup W] [--workload fastwam_s1]

Prints ONE JSON line.  Besides the headline (mean ms per inference over the
K timed steps) it reports the sequential schedule, the video expert alone
(T_v), one action pass alone (T_a), per-kernel timings of the video
expert's GEMMs and attention and of the action expert's weight-streaming
GEMMs (each timed in isolation through the single-kernel entry points that
run the model's own kernel instantiations at the model's shapes: n launches
captured into a HIP graph, replayed between HIP events on the stream they
run on, so small kernels are timed on the GPU rather than by the host's
launch rate), the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per one-step action inference (CEWP) + % MFMA/HBM roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COLD_BYTES = 512 << 20      # weight copies cycled by a per-kernel timing: twice the 256 MB Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fastwam_s1")
    ap.add_argument("--S", type=int, default=None, help="action steps (default: the workload's first)")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="video blocks in the oracle timing sample (0 = all: one complete inference)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel timings")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the captured inference is timed too, and is the headline)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB five times: the known-size reference "
                         "that scales the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled run")
    return ap.parse_args()


# Kernel sources behind each timed entry: the HBM traffic recorded for an
# entry in profiles/ is used only while these files hash as they did when the
# counters were taken.
_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mot_diffusion_transformer_amd", "csrc")
_GEMM_SRC = ["common.h", "kernels.h", "gemm.hip"]
_MISC_SRC = ["common.h", "kernels.h", "misc.hip"]
_ATTN_SRC = ["common.h", "kernels.h", "attention.hip"]
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_fastwam_s1.md")


def source_sha(entry):
    import hashlib
    h = hashlib.sha256()
    for f in (_ATTN_SRC if "attention" in entry else _MISC_SRC if "norm" in entry else _GEMM_SRC):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(entry, workload):
    """HBM bytes per launch of `entry` from the committed counter summary, or
    None if there is none for this workload or the kernel changed since."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    for m in re.finditer(r"<!-- traffic: (.*?) -->", text):
        kv = dict(x.split("=", 1) for x in m.group(1).split())
        if kv.get("entry") == entry and kv.get("workload") == workload and kv.get("sources") == source_sha(entry):
            return float(kv["bytes"])
    return None


def percentile(xs, p):
    return float(np.percentile(np.asarray(xs), p))


def time_loop(torch, fn, n, stream):
    """Mean ms of fn() over n launches on `stream`, bracketed by HIP events on that stream."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def time_graph(torch, fn, n, stream):
    """Mean ms per fn() on `stream`, the GPU's time rather than the host's
    launch rate: n calls are captured once into a HIP graph and the graph is
    replayed three times between HIP events on that stream (fn must allocate
    nothing).  Eager launches as time_loop if the capture fails."""
    fn()
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                fn()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(3):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (3 * n)
        del g
        return ms, "graph"
    except Exception:  # noqa: BLE001 - capture refused: time eager launches instead
        torch.cuda.synchronize()
        return time_loop(torch, fn, n, stream), "eager"


def kernel_timings(torch, bd, wl, m, B, Tv, Ta, n, stream, Ba=None, action_passes=1, video_rows=None):
    """Isolated timings of the model's kernels at its shapes (bf16 only).

    B: video batch; Ba: action batch (default B); action_passes: action-expert
    passes per timed step.  Each entry is labelled by the roof it meets first
    (MFMA time vs HBM time of its algorithmic flops and bytes).  The action
    attention is timed only when Ba == B (its video keys are then per sample).
    video_rows: the video expert runs over that many rows of one sample
    (selective reuse), its queries over all Tv keys."""
    dev = "cuda"
    D, dv, da, r = m.d_attn, m.d_video, m.d_action, m.mlp_ratio
    Ba = B if Ba is None else Ba
    Mv, Ma = (B * Tv if video_rows is None else video_rows), Ba * Ta
    g = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape, dtype=torch.bfloat16, s=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * s).to(dtype)

    out = {}
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def gemm_entry(name, M, N, K, epi, launches, prefetched=False):
        # Weights cold, as in the model (3.3 GB of weights, read once per
        # inference): the captured launches cycle through distinct copies of W
        # totalling at least COLD_BYTES, beyond the 256 MB Infinity Cache, so
        # each launch streams its weights from HBM.  prefetched: in the model
        # the video attention before this GEMM pulls its weights into the
        # Infinity Cache, so the entry is timed on one copy (warm); the cold
        # time is kept beside it.
        A, bias = rnd(M, K), rnd(N, s=0.02)
        ncopy = max(1, -(-COLD_BYTES // (2 * N * K)))
        Ws = [rnd(N, K, s=0.02) for _ in range(ncopy)]
        gate = torch.zeros(N, device=dev)
        if epi == bd.EPI_GATE_RES:
            o = torch.zeros(M, N, device=dev)
        elif epi == bd.EPI_QKV:
            o = torch.empty(3 * M * N // 3, dtype=torch.bfloat16, device=dev)
        else:
            o = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        nws = bd.load().wam_op_gemm_ws_bytes(bd.WAM_BF16, M, N, K)
        assert nws <= ws.numel()
        it = [0]

        def fn():
            W = Ws[it[0] % ncopy]
            it[0] += 1
            bd.op_gemm(A, W, bias, epi=epi, out=o, gate=gate, head_dim=m.head_dim, ws=ws, stream=stream)

        ms, how = time_graph(torch, fn, max(n, ncopy), stream)
        ms_cold = ms
        if prefetched:
            ncopy = 1
            ms, how = time_graph(torch, fn, n, stream)
        del Ws
        flops = 2.0 * M * N * K
        wbytes = 2.0 * (N * K + M * K) + (4.0 if epi == bd.EPI_GATE_RES else 2.0) * M * N
        kind = "mfma" if flops / PEAK_BF16_TFLOPS > wbytes / PEAK_HBM_GBS * 1e3 else "hbm"
        out[name] = {"kind": kind, "shape": [M, N, K], "ms": ms, "launches_per_inference": launches,
                     "tflops": flops / ms / 1e9, "gbs": wbytes / ms / 1e6,
                     "flop_per_launch": flops, "bytes_per_launch": wbytes, "timing": how,
                     "weights": f"cold ({ncopy} copies cycled)"}
        if prefetched:
            out[name]["weights"] = "warm (one copy): the model's attention prefetches them into the Infinity Cache"
            out[name]["ms_cold"] = ms_cold

    N = m.n_blocks
    NA = N * action_passes
    NV = N  # every video block runs in full (the KV-only last block is an off-by-default flag)
    gemm_entry("video_qkv", Mv, 3 * D, dv, bd.EPI_QKV, N)
    gemm_entry("video_o", Mv, dv, D, bd.EPI_GATE_RES, NV)
    gemm_entry("video_fc1", Mv, r * dv, dv, bd.EPI_GELU, NV)
    gemm_entry("video_fc2", Mv, dv, r * dv, bd.EPI_GATE_RES, NV, prefetched=video_rows is None)
    gemm_entry("action_qkv", Ma, 3 * D, da, bd.EPI_QKV, NA)
    gemm_entry("action_o", Ma, da, D, bd.EPI_GATE_RES, NA)
    gemm_entry("action_fc1", Ma, r * da, da, bd.EPI_GELU, NA)
    gemm_entry("action_fc2", Ma, da, r * da, bd.EPI_GATE_RES, NA)
    # video self-attention and the action joint attention
    H, dh = m.n_heads, m.head_dim
    Tq = Tv if video_rows is None else video_rows
    q, k, v = rnd(B, H, Tq, dh, s=0.3), rnd(B, H, Tv, dh, s=0.3), rnd(B, H, dh, Tv)  # v transposed
    oq = torch.empty(B, Tq, H * dh, dtype=torch.bfloat16, device=dev)
    ms, how = time_graph(torch, lambda: bd.op_attention(q, k, v, stream=stream, out=oq, ws=ws), n, stream)
    fl = 4.0 * B * H * Tq * Tv * dh
    by = 2.0 * B * H * dh * (2 * Tq + 2 * Tv)
    out["video_attention"] = {"kind": "mfma", "shape": [B, H, Tq, Tv, dh], "ms": ms, "launches_per_inference": NV,
                              "tflops": fl / ms / 1e9, "flop_per_launch": fl, "bytes_per_launch": by,
                              "gbs": by / ms / 1e6, "timing": how}
    if Ba == B:
        qa, ka, va = rnd(B, H, Ta, dh, s=0.3), rnd(B, H, Ta, dh, s=0.3), rnd(B, H, dh, Ta)
        oa = torch.empty(B, Ta, H * dh, dtype=torch.bfloat16, device=dev)
        ms, how = time_graph(torch, lambda: bd.op_attention(qa, ka, va, k, v, stream=stream, out=oa, ws=ws), n, stream)
        by = 2.0 * B * H * dh * (2 * (Tv + Ta) + 2 * Ta)
        fl = 4.0 * B * H * Ta * (Tv + Ta) * dh
        out["action_attention"] = {"kind": "hbm", "shape": [B, H, Ta, Ta + Tv, dh], "ms": ms,
                                   "launches_per_inference": NA, "tflops": fl / ms / 1e9, "gbs": by / ms / 1e6,
                                   "flop_per_launch": fl, "bytes_per_launch": by, "timing": how,
                                   "weights": "video K/V warm (one block's cache, as when it was just written)"}
    if m.qk_norm or m.rope_hw:
        # the block variant's fused QK-RMSNorm + RoPE: the model runs q and k in one launch, which
        # is the same work as one launch over a tensor of 2B samples
        xq = rnd(2 * B, H, Tv, dh)
        gq = rnd(H * dh, s=0.02) + 1.0
        gq = gq.to(torch.bfloat16)
        ms, how = time_graph(torch, lambda: bd.op_qk_norm_rope(xq, gq if m.qk_norm else None, m.ln_eps, m.rope_hw,
                                                                stream=stream), n, stream)
        by = 2.0 * 2 * (2 * B * H * Tv * dh) + 2.0 * H * dh
        out["video_qk_norm_rope"] = {"kind": "hbm", "shape": [2 * B, H, Tv, dh], "ms": ms, "launches_per_inference": N,
                                     "tflops": 0.0, "gbs": by / ms / 1e6, "flop_per_launch": 0.0, "bytes_per_launch": by,
                                     "timing": how}
    for k_, v_ in out.items():
        v_["ms_per_inference"] = v_["ms"] * v_["launches_per_inference"]
    return out


def cpu_baseline(wl, m, weights, video, noise, S, blocks):
    """The oracle, as it stands, on a bounded sample of the workload: video
    blocks 1..`blocks` of sample 0 (all of them by default: no scaling) and
    one full action pass, scaled to one inference of S steps."""
    from threadpoolctl import threadpool_info

    from oracle import wam_oracle as O
    P = O.Params(weights, "a.")
    x = video[0].astype(np.float64)
    a = noise[0].astype(np.float64)
    t0 = time.perf_counter()
    kv, _ = O.video_forward(P, m, x, 0.0, blocks=blocks)
    t1 = time.perf_counter()
    full_kv = [kv[i % len(kv)] for i in range(m.n_blocks)]  # the real cache when blocks == N
    for name in list(weights):
        if name.startswith("a."):
            P(name)  # float64 copies made once, like a resident model
    t2 = time.perf_counter()
    O.action_velocity(P, m, full_kv, a, 1.0)
    t3 = time.perf_counter()
    video_ms = (t1 - t0) * 1e3 * m.n_blocks / blocks
    action_ms = (t3 - t2) * 1e3
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": video_ms + S * action_ms, "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": (f"one complete inference of sample 0 (video expert, {S} action pass(es))"
                       if blocks == m.n_blocks and S == 1 else
                       f"video expert blocks 1-{blocks} of {m.n_blocks} on sample 0 (time x{m.n_blocks / blocks:g}) "
                       f"+ one full action pass (x{S} steps)")
                      + f"; float64 numpy oracle, BLAS threads={threads}, host cpus={os.cpu_count()}",
            "measured_s": (t1 - t0) + (t3 - t2)}


def kernel_report(result, ks, workload):
    """Per-kernel table, the dominant kernel's roofline and per-expert fractions."""
    result["kernels"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                         for k, v in ks.items()}
    dom_name, dom = max(ks.items(), key=lambda kv_: kv_[1]["ms_per_inference"])
    if dom["kind"] == "mfma":
        ach = dom["flop_per_launch"] / dom["ms"] / 1e9
        result["roofline"] = {"bound": "mfma", "kernel": dom_name, "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                              "traffic": recorded_traffic(dom_name, workload)}
    else:
        ach = dom["bytes_per_launch"] / dom["ms"] / 1e6
        result["roofline"] = {"bound": "hbm", "kernel": dom_name, "achieved": ach, "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                              "traffic": recorded_traffic(dom_name, workload)}
    result["roofline"]["algorithmic_bytes"] = dom["bytes_per_launch"]
    result["roofline"]["kernel_sources_sha256"] = source_sha(dom_name)
    vflops = sum(v["flop_per_launch"] * v["launches_per_inference"] for k, v in ks.items()
                 if k.startswith("video_"))
    vms = sum(v["ms_per_inference"] for k, v in ks.items() if k.startswith("video_"))
    result["video_expert_mfma_frac"] = vflops / vms / 1e9 / PEAK_BF16_TFLOPS
    abytes = sum(v["bytes_per_launch"] * v["launches_per_inference"] for k, v in ks.items()
                 if k.startswith("action_"))
    ams = sum(v["ms_per_inference"] for k, v in ks.items() if k.startswith("action_"))
    result["action_expert_hbm_frac"] = abytes / ams / 1e6 / PEAK_HBM_GBS
    result["kernel_timing_note"] = ("each kernel alone at the model's shape, n launches in a HIP graph between HIP "
                                    "events on its stream; GEMM weights cold (copies cycled past the Infinity "
                                    "Cache); attention inputs warm")


TARGETS_METRIC = "ms per teacher-anchored target batch (one observation: video expert once, R rollouts of K teacher steps + the student endpoint), 1 GPU"


def cpu_baseline_targets(wl, m, weights, student_w, video, a0, eps, ts, K):
    """The oracle on a bounded sample of a target batch: the video expert once
    and rollout 0 (K teacher passes + one student pass), the rollout time
    scaled by the R rollouts of the batch."""
    from threadpoolctl import threadpool_info

    from oracle import wam_oracle as O
    Pt, Ps = O.Params(weights, "a."), O.Params(student_w, "a.")
    for name in weights:
        if name.startswith("a."):
            Pt(name)
            Ps(name)  # float64 copies made once, like resident models
    t0 = time.perf_counter()
    kv, _ = O.video_forward(Pt, m, video[0].astype(np.float64), 0.0)
    t1 = time.perf_counter()
    O.teacher_targets(Pt, Ps, m, kv, a0[0], eps[0], float(ts[0]), K)
    t2 = time.perf_counter()
    R = len(ts)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": (t1 - t0) * 1e3 + R * (t2 - t1) * 1e3, "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": f"video expert once + rollout 0 of {R} (K={K} teacher passes + 1 student pass), the rollout "
                      f"time x{R}; float64 numpy oracle, BLAS threads={threads}, host cpus={os.cpu_count()}",
            "measured_s": t2 - t0}


def bench_targets(args, torch, bd, wl, w):
    """Teacher-anchored target generation.  One step = one observation's
    video forward (batch 1) and its R rollouts: a_t from (a0, eps, t), the
    teacher's K Euler steps to 0, u and the student's endpoint f."""
    m, R, Tv, Ta, K = w.model, w.batch, w.t_video, w.t_action, w.steps[0]
    t_setup = time.perf_counter()
    weights = wl.make_weights(m)
    student_w = wl.make_student_weights(m, weights)
    video = wl.make_video(m, 1, Tv)
    a0_h, eps_h, ts = wl.make_clean_actions(m, R, Ta), wl.make_noise(m, R, Ta), wl.target_times(R)
    teacher = bd.Model(m, weights, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    student = bd.Model(m, student_w, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    vid = bd.to_device(video, m.dtype == wl.BF16)
    a0, eps = torch.from_numpy(a0_h).cuda(), torch.from_numpy(eps_h).cuda()
    kv, vws = teacher.alloc_kv(1, Tv), teacher.alloc_ws(1, Tv, Ta, 1)
    tws = torch.empty(teacher.targets_workspace_bytes(R, Tv, Ta), dtype=torch.uint8, device="cuda")
    u, f, a_t = (torch.empty_like(a0) for _ in range(3))
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    def video_pass():
        teacher.video_forward(vid, 1, Tv, 0.0, kv, vws, stream=st)

    def targets():
        teacher.teacher_targets(kv, Tv, ts, a0, eps, K, u, f, a_t=a_t, ws=tws, student=student, stream=st)

    def step():
        video_pass()
        targets()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: exactly K steps, per-step HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(st)
        step()
        e1.record(st)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = [e0.elapsed_time(e1) for e0, e1 in evs]
    print(f"targets {wall_ms:.3f} ms/batch", file=sys.stderr, flush=True)
    tv_ms = time_loop(torch, video_pass, args.steps, st)
    tt_ms = time_loop(torch, targets, args.steps, st)
    result = {
        "metric": TARGETS_METRIC, "value": wall_ms, "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall_ms, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if m.dtype == wl.BF16 else "f32",
        "data": "synthetic: seeded random-init teacher and student N(0, 0.02^2), video tokens, clean actions and "
                "noise N(0,1), t ~ U(0,1]",
        "config": {"workload": args.workload, "mode": "targets", "rollouts": R, "teacher_steps": K,
                   "blocks": m.n_blocks, "d_video": m.d_video, "d_action": m.d_action, "heads": m.n_heads,
                   "head_dim": m.head_dim, "video_tokens": Tv, "action_tokens": Ta, "action_dim": m.action_dim},
        "ms_p10": percentile(per, 10), "ms_p50": percentile(per, 50), "ms_p90": percentile(per, 90),
        "rollouts_per_s": R / wall_ms * 1e3, "t_video_ms": tv_ms, "t_targets_ms": tt_ms,
        "ms_per_action_pass": tt_ms / (K + 1),
    }
    if m.dtype == wl.BF16 and not args.no_kernels:
        ks = kernel_timings(torch, bd, wl, m, 1, Tv, Ta, max(10, args.steps), st, Ba=R, action_passes=K + 1)
        kernel_report(result, ks, args.workload)
    if not args.no_cpu_baseline:
        print("cpu baseline (oracle sample)...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_targets(wl, m, weights, student_w, video, a0_h, eps_h, ts, K)
    teacher.close()
    student.close()
    print(json.dumps(result))


REUSE_METRIC = ("ms per one-step inference (CEWP) on the next observation with selective video-cache reuse "
                "(token selection + video expert over the changed tokens, overlapped with the action step), 1 GPU")


def cpu_baseline_reuse(wl, m, weights, prev, new, noise, tau):
    """The oracle on one whole reuse step: selection, the video expert over
    the active tokens, one action pass (the previous cache is made first and
    not timed)."""
    from threadpoolctl import threadpool_info

    from oracle import wam_oracle as O
    P = O.Params(weights, "a.")
    kv_prev, h_prev = O.video_forward(P, m, prev.astype(np.float64), 0.0)
    t0 = time.perf_counter()
    kv, act, _ = O.video_forward_selective(P, m, new, prev, kv_prev, tau, hidden_prev=h_prev)
    O.action_velocity(P, m, kv, noise[0].astype(np.float64), 1.0)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": dt * 1e3, "unit": "ms", "cores": threads, "kind": "oracle",
            "sample": f"one complete reuse step ({act.size} active tokens, one action pass); float64 numpy oracle, "
                      f"BLAS threads={threads}, host cpus={os.cpu_count()}",
            "measured_s": dt}


def bench_reuse(args, torch, bd, wl, w):
    """One step = the one-step inference on the next observation of a
    stream (wam_infer_reuse, wavefront schedule): select the tokens that
    moved, rerun the video expert over them on the previous observation's
    cache while the action expert follows block by block.  Stable rows never
    change and the active rows are recomputed from the same inputs, so every
    step does the same work."""
    m, Tv, Ta = w.model, w.t_video, w.t_action
    tau = wl.REUSE_TAU
    t_setup = time.perf_counter()
    weights = wl.make_weights(m)
    prev = wl.make_video(m, 1, Tv)[0]
    new = wl.make_next_observation(m, prev, wl.window_tokens(Tv))
    noise = wl.make_noise(m, 1, Ta)
    model = bd.Model(m, weights, max_batch=1, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    bf = m.dtype == wl.BF16
    prev_d, new_d = bd.to_device(prev, bf), bd.to_device(new, bf)
    a0 = torch.from_numpy(noise).cuda()
    kv, ws = model.alloc_kv(1, Tv), model.alloc_ws(1, Tv, Ta, 1)
    rws = torch.empty(model.reuse_workspace_bytes(Tv), dtype=torch.uint8, device="cuda")
    iws = torch.empty(model.reuse_workspace_bytes(Tv, Ta, 1), dtype=torch.uint8, device="cuda")
    a_next, v, f = (torch.empty_like(a0) for _ in range(3))
    st, sv = torch.cuda.Stream(), torch.cuda.Stream()
    grid = wl.t_grid(1)
    model.video_forward(prev_d, 1, Tv, 0.0, kv, ws, stream=st)
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)
    n_active = [0]

    def reuse():
        n_active[0] = model.video_forward_reuse(new_d, prev_d, Tv, 0.0, tau, kv, rws, stream=st)

    def step(mode=bd.WAM_CEWP):
        n_active[0] = model.infer_reuse(new_d, prev_d, tau, a0, grid, Tv, Ta, kv, a_next, v_last=v, f_last=f,
                                        mode=mode, ws=iws, s_video=sv, s_action=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: exactly K steps, per-step HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(st)
        step()
        e1.record(st)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = [e0.elapsed_time(e1) for e0, e1 in evs]
    print(f"reuse step {wall_ms:.3f} ms ({n_active[0]} active tokens)", file=sys.stderr, flush=True)
    seq_ms = time_loop(torch, lambda: step(bd.WAM_SEQUENTIAL), args.steps, st)
    reuse_ms = time_loop(torch, reuse, args.steps, st)
    ta_ms = time_loop(torch, lambda: model.action_step(kv, 1, Tv, Ta, a0, 1.0, 0.0, a_next, ws=ws, stream=st),
                      args.steps, st)
    # the same observation without reuse: the full wavefront inference
    kv2 = model.alloc_kv(1, Tv)
    full_ms = time_loop(torch, lambda: model.infer(new_d, a0, grid, 1, Tv, Ta, kv2, a_next, ws=ws,
                                                   mode=bd.WAM_CEWP, s_video=sv, s_action=st), args.steps, st)
    result = {
        "metric": REUSE_METRIC, "value": wall_ms, "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall_ms, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if bf else "f32",
        "data": "synthetic: seeded random-init weights N(0, 0.02^2); second observation = first with a changed "
                "window (fresh N(0,1) tokens) and N(0, 0.01^2) noise elsewhere",
        "config": {"workload": args.workload, "mode": "reuse", "batch": 1, "blocks": m.n_blocks, "d_video": m.d_video,
                   "d_action": m.d_action, "heads": m.n_heads, "head_dim": m.head_dim, "video_tokens": Tv,
                   "action_tokens": Ta, "action_dim": m.action_dim, "tau": tau, "active_tokens": n_active[0]},
        "ms_p10": percentile(per, 10), "ms_p50": percentile(per, 50), "ms_p90": percentile(per, 90),
        "ms_reuse_sequential": seq_ms, "t_video_reuse_ms": reuse_ms, "t_action_ms": ta_ms,
        "ms_full_inference_cewp": full_ms, "overlap_delta_ms": wall_ms - max(reuse_ms, ta_ms),
    }
    if bf and not args.no_kernels:
        ks = kernel_timings(torch, bd, wl, m, 1, Tv, Ta, max(10, args.steps), st, video_rows=n_active[0])
        kernel_report(result, ks, args.workload)
    if not args.no_cpu_baseline:
        print("cpu baseline (oracle sample)...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_reuse(wl, m, weights, prev, new, noise, tau)
    model.close()
    print(json.dumps(result))


def main():
    args = parse()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_read_bytes": n, "copy_write_bytes": n, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (several GPUs would each "
              "run their own observations, with no collective between them)", file=sys.stderr)
        sys.exit(2)
    import torch

    from mot_diffusion_transformer_amd import binding as bd
    from mot_diffusion_transformer_amd import workload as wl

    w = wl.WORKLOADS[args.workload]
    if w.kind == "targets":
        return bench_targets(args, torch, bd, wl, w)
    if w.kind == "reuse":
        return bench_reuse(args, torch, bd, wl, w)
    m = w.model
    S = args.S or w.steps[0]
    B, Tv, Ta = w.batch, w.t_video, w.t_action
    t_setup = time.perf_counter()
    weights = wl.make_weights(m)
    video = wl.make_video(m, B, Tv)
    noise = wl.make_noise(m, B, Ta)
    model = bd.Model(m, weights, max_batch=B, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=S)
    vid = bd.to_device(video, m.dtype == wl.BF16)
    a0 = torch.from_numpy(noise).cuda()
    grid = wl.t_grid(S)
    kv, ws = model.alloc_kv(B, Tv), model.alloc_ws(B, Tv, Ta, S)
    a_out, v_last, f_last = torch.empty_like(a0), torch.empty_like(a0), torch.empty_like(a0)
    sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    def infer(mode):
        model.infer(vid, a0, grid, B, Tv, Ta, kv, a_out, v_last, f_last, mode=mode, ws=ws, s_video=sv, s_action=sa)

    for _ in range(args.warmup):
        infer(bd.WAM_CEWP)
    torch.cuda.synchronize()

    def timed(launch, closed_loop=False):
        """Exactly K inferences between two device synchronisations; per-inference HIP events on s_action.
        closed_loop: the host waits for each inference before it enqueues the next, as a control loop
        does (its next observation comes after the actions), so no inference is queued behind another."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in evs:
            e0.record(sa)
            launch()
            e1.record(sa)
            if closed_loop:
                e1.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, [e0.elapsed_time(e1) for e0, e1 in evs]

    # ---- timed region: exactly K inferences, wavefront schedule (eager launches)
    eager_ms, eager_per = timed(lambda: infer(bd.WAM_CEWP))
    print(f"cewp eager {eager_ms:.3f} ms/inference", file=sys.stderr, flush=True)
    wall_ms, per, mode_name = eager_ms, eager_per, "cewp"
    eager_closed_ms, eager_closed_per = timed(lambda: infer(bd.WAM_CEWP), closed_loop=True)
    print(f"cewp eager closed loop {eager_closed_ms:.3f} ms/inference", file=sys.stderr, flush=True)
    if eager_closed_ms < wall_ms:
        wall_ms, per, mode_name = eager_closed_ms, eager_closed_per, "cewp, closed loop"
    graph_ms = closed_ms = None
    if not args.no_graph:
        # the same inference captured once as a HIP graph (both streams, event edges), replayed K times
        graph = model.graph(vid, a0, grid, B, Tv, Ta, kv, a_out, v_last, f_last, mode=bd.WAM_CEWP, ws=ws,
                            s_video=sv, s_action=sa)
        for _ in range(args.warmup):
            graph.launch(sa)
        graph_ms, graph_per = timed(lambda: graph.launch(sa))
        print(f"cewp graph {graph_ms:.3f} ms/inference", file=sys.stderr, flush=True)
        if graph_ms < wall_ms:
            wall_ms, per, mode_name = graph_ms, graph_per, "cewp+graph"
        # With the host ahead, the next inference's fork (s_video waiting on s_action) sits pending at the
        # head of the video queue while this inference's later action steps run, and a pending wait on
        # one queue slows every dispatch on the other (~8% per kernel here).  The closed loop has none.
        closed_ms, closed_per = timed(lambda: graph.launch(sa), closed_loop=True)
        print(f"cewp graph closed loop {closed_ms:.3f} ms/inference", file=sys.stderr, flush=True)
        if closed_ms < wall_ms:
            wall_ms, per, mode_name = closed_ms, closed_per, "cewp+graph, closed loop"

    # ---- the off-by-default cut of the last video block after its K, V (outputs identical), for reference
    kv_only_ms = None
    if not args.no_graph:
        g2 = model.graph(vid, a0, grid, B, Tv, Ta, kv, a_out, v_last, f_last,
                         mode=bd.WAM_CEWP | bd.WAM_VIDEO_KV_ONLY_LAST, ws=ws, s_video=sv, s_action=sa)
        for _ in range(args.warmup):
            g2.launch(sa)
        kv_only_ms = timed(lambda: g2.launch(sa), closed_loop=mode_name.endswith("closed loop"))[0]
        g2.close()
        print(f"cewp graph, last video block K/V only {kv_only_ms:.3f} ms/inference", file=sys.stderr, flush=True)
    # ---- the same kernels in program order on one stream
    seq_ms = time_loop(torch, lambda: infer(bd.WAM_SEQUENTIAL), args.steps, sa)
    # ---- the two experts alone
    tv_ms = time_loop(torch, lambda: model.video_forward(vid, B, Tv, 0.0, kv, ws, stream=sa), args.steps, sa)
    a_next = torch.empty_like(a0)
    ta_ms = time_loop(torch, lambda: model.action_step(kv, B, Tv, Ta, a0, 1.0, 0.0, a_next, ws=ws, stream=sa),
                      args.steps, sa)

    result = {
        "metric": METRIC, "value": wall_ms, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall_ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if m.dtype == wl.BF16 else "f32",
        "data": "synthetic: seeded random-init weights N(0, 0.02^2), video tokens N(0,1), action noise N(0,1)",
        "config": {"workload": args.workload, "mode": mode_name, "batch": B, "blocks": m.n_blocks,
                   "d_video": m.d_video, "d_action": m.d_action, "heads": m.n_heads, "head_dim": m.head_dim,
                   "video_tokens": Tv, "action_tokens": Ta, "action_dim": m.action_dim, "action_steps": S,
                   "video_last_block": "full"},
        "ms_p10": percentile(per, 10), "ms_p50": percentile(per, 50), "ms_p90": percentile(per, 90),
        "ms_cewp_eager": eager_ms, "ms_cewp_eager_closed_loop": eager_closed_ms, "ms_cewp_graph": graph_ms,
        "ms_cewp_graph_closed_loop": closed_ms,
        "ms_sequential": seq_ms, "t_video_ms": tv_ms, "t_action_ms": ta_ms,
        "overlap_delta_ms": wall_ms - max(tv_ms, S * ta_ms),
        # the step-count law of the sequential schedule, T_seq(S) = T_v + S T_a (one video pass, S action passes)
        "t_seq_law": {"S": S, "t_v_plus_S_t_a_ms": tv_ms + S * ta_ms, "ms_sequential": seq_ms,
                      "ratio": seq_ms / (tv_ms + S * ta_ms)},
        "ms_cewp_video_last_block_kv_only": kv_only_ms,
    }

    if m.dtype == wl.BF16 and not args.no_kernels:
        ks = kernel_timings(torch, bd, wl, m, B, Tv, Ta, max(10, args.steps), sa)
        kernel_report(result, ks, args.workload)

    if not args.no_cpu_baseline:
        print("cpu baseline (oracle sample)...", file=sys.stderr, flush=True)
        nb = m.n_blocks if args.cpu_blocks <= 0 else min(args.cpu_blocks, m.n_blocks)
        result["cpu_baseline"] = cpu_baseline(wl, m, weights, video, noise, S, nb)
    if not args.no_graph:
        graph.close()
    model.close()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
