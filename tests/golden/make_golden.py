"""Write the stored expected values for the full-size workloads.

Calls only the CPU oracle (oracle/wam_oracle.py) on the seeded synthetic
inputs of mot_diffusion_transformer_amd.workload; nothing here touches the
HIP library.  The pages print no worked numeric example for the network,
so these files pin the GPU path to the oracle, not to the pages: the
oracle itself is pinned by tests/test_oracle_pins.py.

    python tests/golden/make_golden.py [workload ...]

For batch-8 workloads only samples 0 and 7 are computed (samples are
independent: nothing attends across the batch).  Each file holds, per
computed sample: the final chunk a_out, the last step's velocity v_last
and endpoint f_last, and a fixed sample of the KV cache and of the last
video hidden state (rows KV_TOKENS of blocks KV_BLOCKS, every head and
feature).

Reuse workloads (kind "reuse": a second observation reusing the first's
video cache) store the active token indices, K/V and hidden rows of the
updated cache at the sampled tokens plus a few active ones, and the one-step
inference (a_out, v, f) from that cache.

Target workloads (kind "targets": R rollouts of one observation) store,
for rollouts 0 and R-1 only (rollouts are independent given the shared
video cache), a_t, the teacher's endpoint aT0, u and f, and the times t.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from mot_diffusion_transformer_amd import workload as wl  # noqa: E402
from oracle import wam_oracle as O  # noqa: E402


def kv_tokens(T_v):
    return np.unique(np.linspace(0, T_v - 1, 9).round().astype(int))


def kv_blocks(N):
    return np.array(sorted({0, N // 2, N - 1}))


def samples_of(B):
    return [0] if B == 1 else [0, B - 1]


def golden_path(name, S):
    return os.path.join(HERE, f"{name}_S{S}.npz")


def make_targets(name):
    w = wl.WORKLOADS[name]
    m, R, K = w.model, w.batch, w.steps[0]
    t0 = time.time()
    weights = wl.make_weights(m)
    student = wl.make_student_weights(m, weights)
    Pt, Ps = O.Params(weights, "a."), O.Params(student, "a.")
    rolls = samples_of(R)
    video = wl.make_video(m, 1, w.t_video)[0]
    a0 = wl.make_clean_actions(m, R, w.t_action, samples=rolls)
    eps = wl.make_noise(m, R, w.t_action, samples=rolls)
    ts = wl.target_times(R)
    print(f"[{name}] inputs ready in {time.time() - t0:.1f}s", flush=True)
    kv, _ = O.video_forward(Pt, m, video.astype(np.float64), 0.0)
    out = {"rollouts": np.array(rolls), "t": ts, "K": np.array(K)}
    for si, r in enumerate(rolls):
        t1 = time.time()
        o = O.teacher_targets(Pt, Ps, m, kv, a0[si], eps[si], float(ts[r]), K)
        for k in ("a_t", "aT0", "u", "f"):
            out[f"{k}_{r}"] = o[k]
        print(f"[{name}] K={K} rollout {r} (t={ts[r]:.4f}): oracle {time.time() - t1:.1f}s", flush=True)
    np.savez_compressed(golden_path(name, K), **out)
    with open(os.path.join(HERE, "manifest.json"), "a") as f:
        f.write(json.dumps({"workload": name, "steps": [K], "samples": rolls,
                            "generator": "tests/golden/make_golden.py (oracle only)"}) + "\n")


def reuse_tokens(T_v, active):
    """Sampled cache rows of a reuse workload: the evenly spaced sample plus four active tokens."""
    a = np.asarray(active)
    return np.unique(np.concatenate([kv_tokens(T_v), a[np.linspace(0, a.size - 1, 4).round().astype(int)]]))


def make_reuse(name):
    w = wl.WORKLOADS[name]
    m, Tv, Ta = w.model, w.t_video, w.t_action
    t0 = time.time()
    weights = wl.make_weights(m)
    P = O.Params(weights, "a.")
    prev = wl.make_video(m, 1, Tv)[0]
    new = wl.make_next_observation(m, prev, wl.window_tokens(Tv))
    noise = wl.make_noise(m, 1, Ta)[0]
    print(f"[{name}] inputs ready in {time.time() - t0:.1f}s", flush=True)
    kv_prev, h_prev = O.video_forward(P, m, prev.astype(np.float64), 0.0)
    print(f"[{name}] first observation: {time.time() - t0:.1f}s", flush=True)
    kv, active, hidden = O.video_forward_selective(P, m, new, prev, kv_prev, wl.REUSE_TAU, hidden_prev=h_prev)
    print(f"[{name}] reuse over {active.size} active tokens: {time.time() - t0:.1f}s", flush=True)
    v = O.action_velocity(P, m, kv, noise.astype(np.float64), 1.0)
    toks, blks = reuse_tokens(Tv, active), kv_blocks(m.n_blocks)
    out = {"active": active, "kv_tokens": toks, "kv_blocks": blks, "tau": np.float32(wl.REUSE_TAU),
           "k": np.stack([kv[i][0][:, toks] for i in blks]), "v": np.stack([kv[i][1][:, toks] for i in blks]),
           "hidden": hidden[toks], "v_last": v, "a_out": noise - v, "f_last": noise - v}
    np.savez_compressed(golden_path(name, 1), **out)
    with open(os.path.join(HERE, "manifest.json"), "a") as f:
        f.write(json.dumps({"workload": name, "steps": [1], "samples": [0],
                            "generator": "tests/golden/make_golden.py (oracle only)"}) + "\n")


def make(name):
    w = wl.WORKLOADS[name]
    if w.kind == "targets":
        return make_targets(name)
    if w.kind == "reuse":
        return make_reuse(name)
    m = w.model
    t0 = time.time()
    weights = wl.make_weights(m)
    P = O.Params(weights, "a.")
    samples = samples_of(w.batch)
    video = wl.make_video(m, w.batch, w.t_video, samples=samples)
    noise = wl.make_noise(m, w.batch, w.t_action, samples=samples)
    toks, blks = kv_tokens(w.t_video), kv_blocks(m.n_blocks)
    print(f"[{name}] inputs ready in {time.time() - t0:.1f}s", flush=True)
    for S in w.steps:
        out = {"samples": np.array(samples), "kv_tokens": toks, "kv_blocks": blks, "t_grid": wl.t_grid(S)}
        for si, b in enumerate(samples):
            t1 = time.time()
            r = O.infer(P, m, video[si], noise[si], wl.t_grid(S))
            out[f"a_out_{b}"] = r["a_out"]
            out[f"v_last_{b}"] = r["v"][-1]
            out[f"f_last_{b}"] = r["f"][-1]
            out[f"k_{b}"] = np.stack([r["kv"][i][0][:, toks] for i in blks])
            out[f"v_{b}"] = np.stack([r["kv"][i][1][:, toks] for i in blks])
            out[f"x_video_{b}"] = r["x_video"][toks]
            print(f"[{name}] S={S} sample {b}: oracle {time.time() - t1:.1f}s", flush=True)
        np.savez_compressed(golden_path(name, S), **out)
    with open(os.path.join(HERE, "manifest.json"), "a") as f:
        f.write(json.dumps({"workload": name, "steps": list(w.steps), "samples": samples,
                            "generator": "tests/golden/make_golden.py (oracle only)"}) + "\n")


if __name__ == "__main__":
    names = sys.argv[1:] or ["fastwam_s1", "fastwam_s10", "fastwam_b8"]
    for n in names:
        make(n)
