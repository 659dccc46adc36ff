"""Seeded synthetic workloads: model shapes, weights, video tokens, noise.

This module holds no model arithmetic.  It decides *what the inputs are*:
the shapes of the five workloads, the ordered list of parameter tensors,
and the seeded draws that fill them.  Both the HIP path (through the
binding) and the CPU oracle consume exactly these arrays.

Recipe (all draws are numpy ``default_rng``):
  * parameter tensor number ``k`` (in ``weight_specs`` order) is
    ``default_rng([seed, k]).standard_normal(shape, float32) * std`` with
    ``seed = 0``, ``std = 0.02``; weights *and* biases, every tensor
    (adaLN projections included, so gates are non-zero and every block
    does work);
  * video tokens: ``default_rng([1, b]).standard_normal((T_v, d_v), float32)``
    for batch element ``b``;
  * action noise at t = 1: ``default_rng([2, b]).standard_normal((T_a, A), float32)``;
  * the gains of the QK-RMSNorm block variant (tensors named ``*.qn.g`` /
    ``*.kn.g``, present only when ``qk_norm`` is on, listed after every other
    tensor so the base tensors keep their seeds) are ``1 +`` that draw: a
    gain near zero would silence q and k and leave attention uniform;
  * for a bf16 model the weights and video tokens are rounded once to the
    nearest bf16 (ties to even); the returned float32 arrays hold those
    rounded values exactly, so both sides see the same numbers.

Per-batch-element and per-tensor seeds let generation run in parallel and
let a checker regenerate one sample without drawing the others.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_blocks: int
    d_video: int
    d_action: int
    n_heads: int
    head_dim: int
    action_dim: int
    dtype: str = BF16
    mlp_ratio: int = 4
    t_freq_dim: int = 256
    ln_eps: float = 1e-6
    # Block variant: RMSNorm of each token's q and k over all heads (learned
    # gain, eps ln_eps) right after the q|k|v projection, in both experts ...
    qk_norm: bool = False
    # ... and a 3-D rotary embedding of the video tokens' q and k on a grid of
    # frames x rope_hw[0] x rope_hw[1] patches (frames = T_v / (h w); () = none)
    rope_hw: tuple = ()

    @property
    def d_attn(self) -> int:
        return self.n_heads * self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    t_video: int
    t_action: int
    steps: tuple  # action step counts S run on this workload (teacher steps K for "targets")
    description: str = ""
    kind: str = "infer"  # "infer": one inference per sample; "targets": batch = rollouts of one observation;
    # "reuse": a second observation that reuses the first one's video cache


# The five workloads: a tiny fp32 model, a small bf16 model, and the
# Fast-WAM-scale model at one step, ten steps and in a batch of eight.
TINY = ModelShape(n_blocks=2, d_video=128, d_action=128, n_heads=4, head_dim=32,
                  action_dim=14, dtype=F32)
SMALL = ModelShape(n_blocks=12, d_video=768, d_action=768, n_heads=12, head_dim=64,
                   action_dim=30, dtype=BF16)
FAST_WAM = ModelShape(n_blocks=30, d_video=1536, d_action=768, n_heads=12, head_dim=128,
                      action_dim=14, dtype=BF16)
FAST_WAM_A30 = dataclasses.replace(FAST_WAM, action_dim=30)
# the Wan-style block variant: QK-RMSNorm + 3-D RoPE on 16 x 16 patch frames
FAST_WAM_QKNR = dataclasses.replace(FAST_WAM, qk_norm=True, rope_hw=(16, 16))

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", TINY, 1, 256, 32, (1,),
                          "2 blocks, hidden 128, 4x32 heads, 256 video / 32 action tokens, fp32"),
    "small_bf16": Workload("small_bf16", SMALL, 1, 1024, 64, (1,),
                           "12 blocks, hidden 768, 12x64 heads, 1024 video / 64 action tokens"),
    "fastwam_s1": Workload("fastwam_s1", FAST_WAM, 1, 2048, 32, (1,),
                           "30 blocks, video 1536 / action 768, 12x128 heads, 2048 video / 32 action tokens, S=1"),
    "fastwam_s10": Workload("fastwam_s10", FAST_WAM, 1, 2048, 32, (10,),
                            "as fastwam_s1 with S=10 Euler steps on the uniform grid"),
    "fastwam_b8": Workload("fastwam_b8", FAST_WAM_A30, 8, 4096, 64, (1, 2),
                           "fastwam architecture, batch 8, 4096 video / 64 action tokens, action dim 30"),
    "fastwam_qknr_s1": Workload("fastwam_qknr_s1", FAST_WAM_QKNR, 1, 2048, 32, (1,),
                                "fastwam_s1 with QK-RMSNorm and 3-D RoPE (8 frames of 16 x 16 patches)"),
    "fastwam_targets_k10": Workload("fastwam_targets_k10", FAST_WAM, 16, 2048, 32, (10,),
                                    "teacher-anchored targets: one observation of 2048 video tokens, 16 rollouts "
                                    "of 32 action tokens, K=10 teacher Euler steps and the student's endpoint",
                                    kind="targets"),
    "fastwam_reuse_s1": Workload("fastwam_reuse_s1", FAST_WAM, 1, 2048, 32, (1,),
                                 "fastwam_s1 on the next observation of a stream: 25% of the video tokens changed "
                                 "(a 8 x 8 window of every 16 x 16 frame), the video expert reruns them only",
                                 kind="reuse"),
}

# the changed region of the reuse workload and the default threshold
REUSE_FRAME_HW = (16, 16)
REUSE_WINDOW = (4, 12)   # rows and columns [4, 12) of every frame
REUSE_TAU = 0.05


def weight_specs(m: ModelShape):
    """Ordered (name, shape) list of every parameter tensor.

    Linear maps are stored [out, in] row-major (y = x W^T + b).  Per block
    the adaLN projection emits six vectors in the order
    shift1, scale1, gate1, shift2, scale2, gate2.
    """
    D = m.d_attn
    specs = []
    for ex, d in (("v", m.d_video), ("a", m.d_action)):
        if ex == "a":
            specs += [("a.in.w", (d, m.action_dim)), ("a.in.b", (d,))]
        specs += [(f"{ex}.t1.w", (d, m.t_freq_dim)), (f"{ex}.t1.b", (d,)),
                  (f"{ex}.t2.w", (d, d)), (f"{ex}.t2.b", (d,))]
        for i in range(m.n_blocks):
            p = f"{ex}.{i}."
            specs += [(p + "ada.w", (6 * d, d)), (p + "ada.b", (6 * d,)),
                      (p + "qkv.w", (3 * D, d)), (p + "qkv.b", (3 * D,)),
                      (p + "o.w", (d, D)), (p + "o.b", (d,)),
                      (p + "fc1.w", (m.mlp_ratio * d, d)), (p + "fc1.b", (m.mlp_ratio * d,)),
                      (p + "fc2.w", (d, m.mlp_ratio * d)), (p + "fc2.b", (d,))]
        if ex == "a":
            specs += [("a.fada.w", (2 * d, d)), ("a.fada.b", (2 * d,)),
                      ("a.out.w", (m.action_dim, d)), ("a.out.b", (m.action_dim,))]
    if m.qk_norm:
        for ex in ("v", "a"):
            for i in range(m.n_blocks):
                specs += [(f"{ex}.{i}.qn.g", (D,)), (f"{ex}.{i}.kn.g", (D,))]
    return specs


def is_gain(name: str) -> bool:
    return name.endswith(".qn.g") or name.endswith(".kn.g")


def n_params(m: ModelShape) -> int:
    return sum(int(np.prod(s)) for _, s in weight_specs(m))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    NaN/Inf do not occur in these synthetic inputs and are not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bf16; round it first")
    return (u >> np.uint32(16)).astype(np.uint16)


def _draw(seed_key, shape, std, dtype, offset=0.0):
    a = np.random.default_rng(seed_key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if offset:
        a += np.float32(offset)
    if dtype == BF16:
        a = bf16_round(a)
    return a


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def make_weights(m: ModelShape, seed: int = 0, std: float = 0.02, names=None) -> dict:
    """All parameters as float32 arrays (bf16-rounded for a bf16 model).

    ``names`` restricts generation to a subset (the draws of the others are
    not needed because every tensor has its own seed).
    """
    specs = list(enumerate(weight_specs(m)))
    if names is not None:
        keep = set(names)
        specs = [(k, s) for k, s in specs if s[0] in keep]

    def one(item):
        k, (name, shape) = item
        return name, _draw([seed, k], shape, std, m.dtype, 1.0 if is_gain(name) else 0.0)

    with ThreadPoolExecutor(_workers()) as ex:
        return dict(ex.map(one, specs))


def make_video(m: ModelShape, batch: int, t_video: int, seed: int = 1, samples=None) -> np.ndarray:
    """Video tokens [B, T_v, d_v] (already embedded; no patchify here)."""
    idx = range(batch) if samples is None else samples
    with ThreadPoolExecutor(_workers()) as ex:
        rows = list(ex.map(lambda b: _draw([seed, b], (t_video, m.d_video), 1.0, m.dtype), idx))
    return np.stack(rows)


def make_noise(m: ModelShape, batch: int, t_action: int, seed: int = 2, samples=None) -> np.ndarray:
    """Action chunk at t = 1: standard normal noise [B, T_a, A], float32 always."""
    idx = range(batch) if samples is None else samples
    return np.stack([_draw([seed, b], (t_action, m.action_dim), 1.0, F32) for b in idx])


def make_clean_actions(m: ModelShape, R: int, t_action: int, seed: int = 4, samples=None) -> np.ndarray:
    """Stand-in for the data's clean action chunks a_0: standard normal [R, T_a, A], float32."""
    idx = range(R) if samples is None else samples
    return np.stack([_draw([seed, r], (t_action, m.action_dim), 1.0, F32) for r in idx])


def target_times(R: int, seed: int = 5) -> np.ndarray:
    """Per-rollout times t ~ U(0, 1] in float32 (1 - U[0, 1), never 0)."""
    u = np.random.default_rng([seed, R]).random(R)
    return np.maximum(1.0 - u, 1e-3).astype(np.float32)


STUDENT_SEED = 7


def make_student_weights(m: ModelShape, teacher: dict, seed: int = STUDENT_SEED) -> dict:
    """A student with its own action expert (independent draws) and the
    teacher's video expert (the same arrays: it only reads the teacher's cache)."""
    own = make_weights(m, seed=seed, names=[n for n, _ in weight_specs(m) if n.startswith("a.")])
    return {n: own.get(n, teacher[n]) for n in teacher}


def window_tokens(t_video: int, frame_hw=REUSE_FRAME_HW, window=REUSE_WINDOW) -> np.ndarray:
    """Ascending indices of the tokens inside rows and columns [lo, hi) of
    every frame (tokens frame by frame, each frame row-major)."""
    h, w = frame_hw
    lo, hi = window
    n = np.arange(t_video)
    r, c = (n // w) % h, n % w
    return n[(r >= lo) & (r < hi) & (c >= lo) & (c < hi)]


def make_next_observation(m: ModelShape, video: np.ndarray, changed, seed: int = 6, noise: float = 0.01) -> np.ndarray:
    """The next observation of a stream, [T_v, d_v]: tokens in ``changed`` are
    fresh N(0, 1) draws (a region that moved); the others are the previous
    tokens plus N(0, noise^2) sensor noise.  Rounded to bf16 for bf16 models."""
    video = np.asarray(video, dtype=np.float32)
    rng = np.random.default_rng([seed, video.shape[0]])
    new = video + np.float32(noise) * rng.standard_normal(video.shape, dtype=np.float32)
    changed = np.asarray(changed, dtype=np.int64)
    new[changed] = rng.standard_normal((changed.size, video.shape[1]), dtype=np.float32)
    return bf16_round(new) if m.dtype == BF16 else new


def t_grid(S: int) -> np.ndarray:
    """Uniform time grid t_j = j / S for j = 0..S, in float32 (t_grid[S] = 1, t_grid[0] = 0)."""
    if S < 1:
        raise ValueError("S must be >= 1")
    return (np.arange(S + 1, dtype=np.float32) / np.float32(S)).astype(np.float32)
