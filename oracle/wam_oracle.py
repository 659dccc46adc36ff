"""CPU oracle for the Mixture-of-Transformers world-action-model forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
runs this file: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library (its only import from the package is the seeded input generator,
which holds no model arithmetic).

Plain, slow, obviously-correct float64 numpy.  A matrix product
(``np.matmul``) is the only library primitive used as a step; everything else
is written out in the order the method states it.  Batch elements are
independent (nothing attends across samples), so every function here works
on ONE sample and the drivers loop over the batch.

Sources (the pages are web digests of the RealtimeWAM paper, arXiv 2610.06617):
  [digest]   "RealtimeWAM: One-Step Asynchronous World Action Models",
             paper.rainbus.top digest; sections Background (World Action
             Model, Mixture-of-Transformers, Flow matching and velocity-field
             denoising, KV cache, CUDA streams and events), Core method,
             Method steps, Novelty.
  [article]  tokendh.com article on the same paper; sections "why world
             action models are so slow" and "let the two experts stop
             waiting: cross-expert wavefront pipelining".
  [reuse]    "RealtimeWAM: How Fast Can I Run My World Action Model?",
             shd-paper.top page of a training-free paper (arXiv 2610.10079):
             abstract and method details, key design (selective reuse of
             observation features in visually stable regions).
The pages fix the structure (two experts, per-block KV sharing, the Euler
update and the endpoint map) but not the block internals.  The readings
taken where they are silent: a pre-norm LayerNorm DiT block (eps 1e-6, no
affine) modulated by six adaLN vectors from SiLU(c) in the order shift1,
scale1, gate1, shift2, scale2, gate2; exact-erf GELU MLP of ratio 4; a
sinusoidal embedding of 1000*t (256 features, cosines first); no positional
encoding; the video expert conditioned on t_v = 0; unmasked attention with
the action keys ordered [own ; video].  The block variant behind the pages'
fused RMSNorm/RoPE operator: q and k RMS-normalised per token over all
heads (gain, eps 1e-6), then a 3-D rotary embedding of the video tokens
(head dim cut into frame/row/column bands of dh-4[dh/6], 2[dh/6], 2[dh/6]
features, base 10000, tokens frame by frame on the patch grid); action
tokens carry no grid position and are only normalised.

Parity status: every primitive and every composition rule is pinned by
tests/test_oracle_pins.py (brute force on tiny inputs, closed forms,
invariants).  The composed network on random weights has no printed worked
example on the pages: beyond those pins its values are "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

__all__ = [
    "timestep_embedding", "linear", "layer_norm", "modulate", "silu", "gelu", "rms_norm",
    "rope_bands", "rope_positions", "rope3d",
    "attention", "t_conditioning", "block_modulation", "project", "rest",
    "video_forward", "action_velocity", "final_layer", "euler_step", "endpoint",
    "infer", "infer_interleaved", "infer_batch", "teacher_targets", "teacher_targets_batch",
    "select_tokens", "video_forward_selective", "Counters", "Params",
]


# ----------------------------------------------------------------------------
# parameters
# ----------------------------------------------------------------------------
class Params:
    """Read-only view of a weight dict that hands out float64 copies.

    ``cache`` keeps the float64 copies of a name prefix (the action expert's,
    reused by every Euler step); other tensors are converted on each use.
    """

    def __init__(self, weights: dict, cache_prefix: str | None = None):
        self.w = weights
        self.cache_prefix = cache_prefix
        self._cache = {}

    def __call__(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        a = np.asarray(self.w[name], dtype=np.float64)
        if self.cache_prefix is not None and name.startswith(self.cache_prefix):
            self._cache[name] = a
        return a


class Counters:
    """Network-function-evaluation counts: one video pass, S action passes."""

    def __init__(self):
        self.video_passes = 0
        self.action_passes = 0


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------
def timestep_embedding(t: float, dim: int = 256, max_period: float = 10000.0) -> np.ndarray:
    """Sinusoidal embedding of a flow time t in [0, 1], float64 [dim].

    The velocity field is conditioned on t ([digest] Background, flow
    matching: v_theta(a_t, t)); the embedding form is the DiT one: frequencies
    f_k = max_period^(-k/half) for k = 0..half-1, argument 1000*t*f_k, cosines
    first then sines.
    """
    half = dim // 2
    k = np.arange(half, dtype=np.float64)
    freqs = np.exp(-math.log(max_period) * k / half)
    args = 1000.0 * float(t) * freqs
    return np.concatenate([np.cos(args), np.sin(args)])


def linear(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y = x W^T + b with W stored [out, in]."""
    return np.matmul(x, W.T) + b


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, population variance, no affine."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(h: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """adaLN modulation h * (1 + scale) + shift."""
    return h * (1.0 + scale) + shift


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU: z * Phi(z)."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Multi-head softmax attention, no mask, scale 1/sqrt(dh).

    q [H, Tq, dh], k and v [H, L, dh] -> o [Tq, H*dh] with heads concatenated
    in head order.  For the action expert the key set is the concatenation
    [own action keys ; video block-i keys] ([digest] Background, KV cache:
    the action expert concatenates its own K/V with the video K/V).
    """
    H, Tq, dh = q.shape
    out = np.empty((Tq, H * dh))
    for h in range(H):
        s = np.matmul(q[h], k[h].T) / math.sqrt(dh)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[:, h * dh:(h + 1) * dh] = np.matmul(p, v[h])
    return out


# ----------------------------------------------------------------------------
# block variant: QK-RMSNorm and a 3-D rotary position embedding.  The pages
# name a fused RMSNorm/RoPE operator next to the merged QKV projection
# ([digest] Method steps, inference: operator fusion; [article] "let the two
# experts stop waiting", the efficient-operator step) without its form; the
# reading taken is stated at each function.
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis with gain g:
    x / sqrt(mean(x^2) + eps) * g (applied to a token's whole q or k, all heads)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_bands(dh: int):
    """Sizes of the (frame, row, column) bands the head dimension is cut into.

    Reading taken (the pages name a 3-D RoPE but not its split): the row and
    column axes get 2*floor(dh/6) features each, the frame axis the remaining
    dh - 4*floor(dh/6); every band is even, so it holds whole rotation pairs
    (44/42/42 for dh = 128, 24/20/20 for dh = 64).
    """
    dh = int(dh)
    side = 2 * (dh // 6)
    return (dh - 2 * side, side, side)


def rope_positions(T: int, hw) -> np.ndarray:
    """(frame, row, column) of token n = 0..T-1, tokens ordered frame by frame,
    each frame a row-major grid of hw[0] x hw[1] patches."""
    Hp, Wp = int(hw[0]), int(hw[1])
    if T % (Hp * Wp):
        raise ValueError("token count is not a whole number of frames")
    n = np.arange(T)
    return np.stack([n // (Hp * Wp), (n // Wp) % Hp, n % Wp], axis=1)


def rope3d(x: np.ndarray, pos: np.ndarray, bands, theta: float = 10000.0) -> np.ndarray:
    """Rotary embedding of x [H, T, dh] at positions pos [T, 3].

    The head dimension is cut into three contiguous bands (frame, row,
    column; sizes ``bands``).  In the band of size s for axis a, feature pair
    (2i, 2i+1) is rotated by the angle pos[:, a] * theta^(-2i/s):
    (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    start = 0
    for a, size in enumerate(bands):
        for i in range(size // 2):
            ang = pos[:, a].astype(np.float64) * theta ** (-2.0 * i / size)  # [T]
            c, sn = np.cos(ang), np.sin(ang)
            e0, e1 = start + 2 * i, start + 2 * i + 1
            out[:, :, e0] = x[:, :, e0] * c - x[:, :, e1] * sn
            out[:, :, e1] = x[:, :, e0] * sn + x[:, :, e1] * c
        start += size
    return out


def _split_heads(y: np.ndarray, H: int, dh: int) -> np.ndarray:
    """[T, H*dh] -> [H, T, dh]: head h is columns h*dh .. h*dh+dh-1."""
    T = y.shape[0]
    return y.reshape(T, H, dh).transpose(1, 0, 2)


# ----------------------------------------------------------------------------
# DiT block, split the way the pages split it: P (projection), Attn, R (rest)
# ([digest] Core method: each DiT block = projection, attention, remaining
# computation; [article] "cross-expert wavefront pipelining")
# ----------------------------------------------------------------------------
def t_conditioning(P: Params, ex: str, t: float, m) -> np.ndarray:
    """c = W_t2 SiLU(W_t1 temb(t) + b_t1) + b_t2 for expert ``ex`` ('v' or 'a')."""
    e = timestep_embedding(t, m.t_freq_dim)
    h = silu(linear(e, P(f"{ex}.t1.w"), P(f"{ex}.t1.b")))
    return linear(h, P(f"{ex}.t2.w"), P(f"{ex}.t2.b"))


def block_modulation(P: Params, ex: str, i: int, c: np.ndarray):
    """Six adaLN vectors of block i: shift1, scale1, gate1, shift2, scale2, gate2."""
    mvec = linear(silu(c), P(f"{ex}.{i}.ada.w"), P(f"{ex}.{i}.ada.b"))
    return np.split(mvec, 6)


def project(P: Params, ex: str, i: int, mod, x: np.ndarray, m):
    """P_i: h = LN(x)(1+scale1)+shift1; [q|k|v] = h W_qkv^T + b -> three [H, T, dh].

    Block variant (``m.qk_norm``, ``m.rope_hw``): q and k of every token are
    RMS-normalised over all heads with their gains, then (video expert
    only: its tokens have grid positions) rotated by the 3-D RoPE.
    """
    shift1, scale1 = mod[0], mod[1]
    h = modulate(layer_norm(x, m.ln_eps), shift1, scale1)
    qkv = linear(h, P(f"{ex}.{i}.qkv.w"), P(f"{ex}.{i}.qkv.b"))
    D = m.d_attn
    q, k, v = (qkv[:, j * D:(j + 1) * D] for j in range(3))
    if getattr(m, "qk_norm", False):
        q = rms_norm(q, P(f"{ex}.{i}.qn.g"), m.ln_eps)
        k = rms_norm(k, P(f"{ex}.{i}.kn.g"), m.ln_eps)
    q, k, v = (_split_heads(y, m.n_heads, m.head_dim) for y in (q, k, v))
    if getattr(m, "rope_hw", ()) and ex == "v":
        pos = rope_positions(x.shape[0], m.rope_hw)
        bands = rope_bands(m.head_dim)
        q, k = rope3d(q, pos, bands), rope3d(k, pos, bands)
    return q, k, v


def rest(P: Params, ex: str, i: int, mod, x: np.ndarray, o: np.ndarray, m) -> np.ndarray:
    """R_i: gated output projection and gated GELU MLP, both residual."""
    gate1, shift2, scale2, gate2 = mod[2], mod[3], mod[4], mod[5]
    x1 = x + gate1 * linear(o, P(f"{ex}.{i}.o.w"), P(f"{ex}.{i}.o.b"))
    h2 = modulate(layer_norm(x1, m.ln_eps), shift2, scale2)
    f = linear(gelu(linear(h2, P(f"{ex}.{i}.fc1.w"), P(f"{ex}.{i}.fc1.b"))),
               P(f"{ex}.{i}.fc2.w"), P(f"{ex}.{i}.fc2.b"))
    return x1 + gate2 * f


# ----------------------------------------------------------------------------
# the two experts
# ----------------------------------------------------------------------------
def video_forward(P: Params, m, video: np.ndarray, t_v: float = 0.0, counters=None,
                  blocks=None):
    """Video expert, run once per observation ([digest] Background, WAM / KV cache).

    video [T_v, d_v] (already-embedded tokens).  Returns (kv, x) with kv[i] =
    (K^v_i, V^v_i), each [H, T_v, dh], the per-block cache the action expert
    reuses, and x the last hidden state.  ``blocks`` limits the pass to the
    first few blocks (used only for bounded CPU timing).
    """
    if counters is not None:
        counters.video_passes += 1
    x = np.asarray(video, dtype=np.float64)
    c = t_conditioning(P, "v", t_v, m)
    kv = []
    n = m.n_blocks if blocks is None else blocks
    for i in range(n):
        mod = block_modulation(P, "v", i, c)
        q, k, v = project(P, "v", i, mod, x, m)
        kv.append((k, v))
        x = rest(P, "v", i, mod, x, attention(q, k, v), m)
    return kv, x


def final_layer(P: Params, m, y: np.ndarray, c: np.ndarray) -> np.ndarray:
    """v_theta = (LN(y)(1+scale_f)+shift_f) W_out^T + b_out, with (shift_f, scale_f) from c."""
    shift_f, scale_f = np.split(linear(silu(c), P("a.fada.w"), P("a.fada.b")), 2)
    return linear(modulate(layer_norm(y, m.ln_eps), shift_f, scale_f), P("a.out.w"), P("a.out.b"))


def action_velocity(P: Params, m, kv, a: np.ndarray, t: float, counters=None, hidden=None):
    """One action-expert pass: v_theta(a_t, t) given the video KV cache.

    Block i attends over [own k ; K^v_i] and [own v ; V^v_i] ([digest]
    Background, Mixture-of-Transformers: block i talks to block i by
    concatenating KV).  ``hidden``, if a list, receives y^1..y^N.
    """
    if counters is not None:
        counters.action_passes += 1
    y = linear(np.asarray(a, dtype=np.float64), P("a.in.w"), P("a.in.b"))
    c = t_conditioning(P, "a", t, m)
    for i in range(m.n_blocks):
        mod = block_modulation(P, "a", i, c)
        q, k, v = project(P, "a", i, mod, y, m)
        Kv, Vv = kv[i]
        o = attention(q, np.concatenate([k, Kv], axis=1), np.concatenate([v, Vv], axis=1))
        y = rest(P, "a", i, mod, y, o, m)
        if hidden is not None:
            hidden.append(y)
    return final_layer(P, m, y, c)


def euler_step(a: np.ndarray, v: np.ndarray, t_cur: float, t_next: float) -> np.ndarray:
    """a_{t_{j-1}} = a_{t_j} - (t_j - t_{j-1}) v ([digest] Background, flow matching)."""
    return a - (float(t_cur) - float(t_next)) * v


def endpoint(a: np.ndarray, v: np.ndarray, t: float) -> np.ndarray:
    """Endpoint map f(a_t, t) = a_t - t v ([digest] Background, flow matching)."""
    return a - float(t) * v


# ----------------------------------------------------------------------------
# teacher-anchored targets, forward only: the quantities the distillation
# trains on ([digest] Core method: the frozen teacher's K-step rollout end
# a^T_0 and the interval-average velocity u = (a_t - a^T_0) / t; Method steps,
# training: a_t = (1 - t) a_0 + t eps, one video KV cache per observation,
# the student's endpoint f = a_t - t v)
# ----------------------------------------------------------------------------
def teacher_targets(P_teacher, P_student, m, kv, a0: np.ndarray, eps: np.ndarray, t: float, K: int = 10):
    """One rollout: a_t, the teacher's endpoint a^T_0 after K Euler steps from
    t to 0 on the uniform grid t_j = t j / K (j = K .. 0), u = (a_t - a^T_0) / t
    and the student's endpoint f = a_t - t v_student(a_t, t).  ``kv`` is the
    video KV cache both action experts read."""
    t = float(t)
    if not (0.0 < t <= 1.0):
        raise ValueError("t must lie in (0, 1]")
    if int(K) < 1:
        raise ValueError("K must be >= 1")
    K = int(K)
    a0 = np.asarray(a0, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    a_t = (1.0 - t) * a0 + t * eps
    grid = [t * j / K for j in range(K + 1)]
    a = a_t
    for j in range(K, 0, -1):
        a = euler_step(a, action_velocity(P_teacher, m, kv, a, grid[j]), grid[j], grid[j - 1])
    u = (a_t - a) / t
    f = endpoint(a_t, action_velocity(P_student, m, kv, a_t, t), t)
    return {"a_t": a_t, "aT0": a, "u": u, "f": f}


def teacher_targets_batch(w_teacher, w_student, m, video: np.ndarray, a0: np.ndarray, eps: np.ndarray, ts,
                          K: int = 10, t_v: float = 0.0):
    """R rollouts of ONE observation: the video expert runs once (the frozen
    teacher's: the student shares it) and every rollout reuses its KV cache.
    video [T_v, d_v]; a0, eps [R, T_a, A]; ts [R].  Returns stacked a_t, aT0, u, f."""
    Pt = Params(w_teacher, "a.")
    Ps = Pt if w_student is None or w_student is w_teacher else Params(w_student, "a.")
    kv, _ = video_forward(Pt, m, video, t_v)
    outs = [teacher_targets(Pt, Ps, m, kv, a0[r], eps[r], ts[r], K) for r in range(len(ts))]
    return {k: np.stack([o[k] for o in outs]) for k in ("a_t", "aT0", "u", "f")}


# ----------------------------------------------------------------------------
# selective reuse of the video expert across consecutive observations ([reuse]
# abstract; method details, key design: observation features of visually
# stable regions are cached and reused, the rest recomputed).  The page names
# the idea but not its criterion or granularity.  Reading taken: tokens are
# the unit; a token is active when its input moved by more than tau relative
# to the previous observation's, ||x_new - x_prev||^2 > tau^2 ||x_prev||^2;
# every block recomputes the active tokens only (their queries attend over
# all keys, where stable tokens keep the previous observation's K and V) and
# writes their K, V into the cache.  Stable tokens are never recomputed.
# ----------------------------------------------------------------------------
def select_tokens(video_new: np.ndarray, video_prev: np.ndarray, tau: float) -> np.ndarray:
    """Ascending indices of the active tokens.

    Reading taken (the reuse page names caching of stable regions but no
    criterion and no precision): a token is active when
    ||x_new - x_prev||^2 > tau^2 ||x_prev||^2.  The comparison decides an
    index set, so it is taken in one stated precision: the inputs as float32,
    float32 squares and float32 sums of them (numpy's pairwise order).  A
    token whose two sides differ by less than the rounding bound of two
    float32 sums of d_v terms may be decided either way by another summation
    order; every other token is decided as exact arithmetic on the float32
    inputs decides it.
    """
    tau = float(tau)
    if not (tau >= 0.0):
        raise ValueError("tau must be >= 0")
    xn = np.asarray(video_new, dtype=np.float32)
    xp = np.asarray(video_prev, dtype=np.float32)
    if xn.shape != xp.shape or xn.ndim != 2:
        raise ValueError("video_new and video_prev must both be [T_v, d_v]")
    d = xn - xp
    d2 = np.sum(d * d, axis=1, dtype=np.float32)
    p2 = np.sum(xp * xp, axis=1, dtype=np.float32)
    t2 = np.float32(tau) * np.float32(tau)
    return np.nonzero(d2 > t2 * p2)[0]


def video_forward_selective(P: Params, m, video_new: np.ndarray, video_prev: np.ndarray, kv_prev, tau: float,
                            t_v: float = 0.0, hidden_prev=None):
    """Video expert for a new observation, reusing the previous one's cache.

    kv_prev[i] = (K_i, V_i), [H, T_v, dh]: the cache after the previous
    observation.  Returns (kv, active, hidden): the updated cache (stable
    rows unchanged), the active token indices, and hidden_prev with the
    active rows replaced by their last hidden state (None if not given).
    Base block only (no QK-norm / RoPE variant).
    """
    if getattr(m, "qk_norm", False) or getattr(m, "rope_hw", ()):
        raise ValueError("selective reuse is defined for the base block")
    active = select_tokens(video_new, video_prev, tau)
    kv = [(np.array(K, dtype=np.float64), np.array(V, dtype=np.float64)) for K, V in kv_prev]
    hidden = None if hidden_prev is None else np.array(hidden_prev, dtype=np.float64)
    if active.size == 0:
        return kv, active, hidden
    x = np.asarray(video_new, dtype=np.float64)[active]
    c = t_conditioning(P, "v", t_v, m)
    for i in range(m.n_blocks):
        mod = block_modulation(P, "v", i, c)
        q, k, v = project(P, "v", i, mod, x, m)
        K, V = kv[i]
        K[:, active] = k
        V[:, active] = v
        x = rest(P, "v", i, mod, x, attention(q, K, V), m)
    if hidden is not None:
        hidden[active] = x
    return kv, active, hidden


# ----------------------------------------------------------------------------
# drivers
# ----------------------------------------------------------------------------
def _check_grid(grid):
    g = np.asarray(grid, dtype=np.float64)
    if g.ndim != 1 or g.size < 2:
        raise ValueError("time grid needs S+1 >= 2 points")
    if np.any(np.diff(g) <= 0) or g[0] < 0 or g[-1] > 1:
        raise ValueError("time grid must increase strictly inside [0, 1]")
    return g


def infer(weights_or_params, m, video: np.ndarray, a_init: np.ndarray, grid,
          t_v: float = 0.0, counters=None, keep_kv: bool = True):
    """Sequential inference of ONE sample: video expert once, then S Euler steps.

    grid[j] = t_j, grid[S] = 1 (the noise a_init) down to grid[0] = 0.
    Returns a dict with the final chunk ``a_out``, per-step velocities
    ``v[j]`` and endpoints ``f[j]`` (index 0 = first step, at t_S), the KV
    cache and the last video hidden state.  Latency model: one video pass
    plus S action passes, T_seq = T_v + S T_a ([digest] Core method).
    """
    P = weights_or_params if isinstance(weights_or_params, Params) else Params(weights_or_params, "a.")
    g = _check_grid(grid)
    S = g.size - 1
    kv, xv = video_forward(P, m, video, t_v, counters)
    a = np.asarray(a_init, dtype=np.float64)
    vs, fs = [], []
    for j in range(S, 0, -1):
        v = action_velocity(P, m, kv, a, g[j], counters)
        vs.append(v)
        fs.append(endpoint(a, v, g[j]))
        a = euler_step(a, v, g[j], g[j - 1])
    return {"a_out": a, "v": vs, "f": fs, "kv": kv if keep_kv else None, "x_video": xv}


def infer_interleaved(weights_or_params, m, video, a_init, grid, t_v: float = 0.0, counters=None):
    """The same inference in the cross-expert wavefront order.

    Video stream: P^v_i -> publish (K^v_i, V^v_i) -> Attn^v_i -> R^v_i.
    Action stream (first step): P^a_i -> (needs block i published) ->
    Attn^a_i -> R^a_i, interleaved block by block ([digest] Method steps,
    inference; [article] cross-expert wavefront pipelining).  The action
    side can only read blocks already published, so this checks that action
    block i needs nothing from video blocks > i.  Later steps (S > 1) need
    every block and run after the video expert.  The pages state the two
    orders give identical results ([digest] Novelty: the asynchronous run is
    another topological order of the same graph).
    """
    P = weights_or_params if isinstance(weights_or_params, Params) else Params(weights_or_params, "a.")
    g = _check_grid(grid)
    S = g.size - 1
    if counters is not None:
        counters.video_passes += 1
        counters.action_passes += 1
    published = {}
    x = np.asarray(video, dtype=np.float64)
    a = np.asarray(a_init, dtype=np.float64)
    c_v = t_conditioning(P, "v", t_v, m)
    y = linear(a, P("a.in.w"), P("a.in.b"))
    c_a = t_conditioning(P, "a", g[S], m)
    for i in range(m.n_blocks):
        mod_v = block_modulation(P, "v", i, c_v)
        qv, kv_, vv_ = project(P, "v", i, mod_v, x, m)
        published[i] = (kv_, vv_)
        mod_a = block_modulation(P, "a", i, c_a)
        qa, ka, va = project(P, "a", i, mod_a, y, m)
        ov = attention(qv, kv_, vv_)
        Kv, Vv = published[i]
        oa = attention(qa, np.concatenate([ka, Kv], axis=1), np.concatenate([va, Vv], axis=1))
        x = rest(P, "v", i, mod_v, x, ov, m)
        y = rest(P, "a", i, mod_a, y, oa, m)
    v = final_layer(P, m, y, c_a)
    vs, fs = [v], [endpoint(a, v, g[S])]
    a = euler_step(a, v, g[S], g[S - 1])
    kv = [published[i] for i in range(m.n_blocks)]
    for j in range(S - 1, 0, -1):
        v = action_velocity(P, m, kv, a, g[j], counters)
        vs.append(v)
        fs.append(endpoint(a, v, g[j]))
        a = euler_step(a, v, g[j], g[j - 1])
    return {"a_out": a, "v": vs, "f": fs, "kv": kv, "x_video": x}


def infer_batch(weights, m, video: np.ndarray, a_init: np.ndarray, grid, t_v: float = 0.0,
                keep_kv: bool = False):
    """Loop ``infer`` over a batch; returns stacked a_out [B,T_a,A], v and f [S][B,T_a,A]."""
    P = Params(weights, "a.")
    outs = [infer(P, m, video[b], a_init[b], grid, t_v, keep_kv=keep_kv) for b in range(video.shape[0])]
    S = len(outs[0]["v"])
    return {
        "a_out": np.stack([o["a_out"] for o in outs]),
        "v": [np.stack([o["v"][j] for o in outs]) for j in range(S)],
        "f": [np.stack([o["f"][j] for o in outs]) for j in range(S)],
        "kv": [o["kv"] for o in outs] if keep_kv else None,
        "x_video": np.stack([o["x_video"] for o in outs]),
    }
