"""CPU model of the bfloat16 HIP path's rounding points (test infrastructure).

Not the oracle and not the product: a float32 numpy rendering of the same
forward pass that rounds to bfloat16 (nearest, ties to even) exactly where
the bf16 path stores a value in bf16, and nowhere else:
  * the LayerNorm + modulation output h (the GEMM operand);
  * q, k, v (k and v are the cache);
  * the softmax probabilities before the P.V product (their sum is kept in
    float32), and the attention output o;
  * the GELU output of the first MLP GEMM.
Residual streams, modulation vectors, GEMM accumulation, the final layer and
the Euler update stay float32.  Comparing it with the float64 oracle says how
far rounding alone moves each output, so a GPU error of the same size is
rounding, and one far beyond it is a defect.
"""
import math

import numpy as np

from mot_diffusion_transformer_amd.workload import bf16_round

F = np.float32


def _lin(x, W, b):
    return (np.asarray(x, F) @ np.asarray(W, F).T + np.asarray(b, F)).astype(F)


def _silu(z):
    return (z / (F(1) + np.exp(-z))).astype(F)


def _gelu(z):
    from scipy.special import erf
    return (F(0.5) * z * (F(1) + erf(z / F(math.sqrt(2.0))).astype(F))).astype(F)


def _ln_mod(x, shift, scale, eps):
    mu = x.mean(-1, keepdims=True, dtype=F)
    var = ((x - mu) ** 2).mean(-1, keepdims=True, dtype=F)
    return bf16_round(((x - mu) / np.sqrt(var + F(eps))) * (F(1) + scale) + shift)


def _temb(t, dim):
    half = dim // 2
    fr = np.exp(-math.log(10000.0) * np.arange(half) / half)
    a = 1000.0 * t * fr
    return np.concatenate([np.cos(a), np.sin(a)]).astype(F)


def _cond(w, ex, t, dim):
    h = _silu(_lin(_temb(t, dim), w[f"{ex}.t1.w"], w[f"{ex}.t1.b"]))
    return _lin(h, w[f"{ex}.t2.w"], w[f"{ex}.t2.b"])


def _attn(q, k, v, dh):
    """q [H,Tq,dh], k, v [H,L,dh] (bf16 values) -> o [Tq, H dh] rounded to bf16."""
    H, Tq, _ = q.shape
    o = np.empty((Tq, H * dh), F)
    for h in range(H):
        s = (q[h] @ k[h].T).astype(F) * F(1.0 / math.sqrt(dh))
        p = np.exp(s - s.max(-1, keepdims=True)).astype(F)
        l = p.sum(-1, keepdims=True, dtype=F)
        o[:, h * dh:(h + 1) * dh] = (bf16_round(p) @ v[h]).astype(F) / l
    return bf16_round(o)


def _heads(y, H, dh):
    return y.reshape(y.shape[0], H, dh).transpose(1, 0, 2)


def _block(w, ex, i, mod, x, m, kv=None):
    """One block; returns (x', k, v) with k, v the bf16 projections [H, T, dh]."""
    d = x.shape[1]
    H, dh, D = m.n_heads, m.head_dim, m.n_heads * m.head_dim
    sh1, sc1, g1, sh2, sc2, g2 = (mod[j * d:(j + 1) * d] for j in range(6))
    qkv = bf16_round(_lin(_ln_mod(x, sh1, sc1, m.ln_eps), w[f"{ex}.{i}.qkv.w"], w[f"{ex}.{i}.qkv.b"]))
    q, k, v = (_heads(qkv[:, j * D:(j + 1) * D], H, dh) for j in range(3))
    if kv is None:
        o = _attn(q, k, v, dh)
    else:
        o = _attn(q, np.concatenate([k, kv[0]], 1), np.concatenate([v, kv[1]], 1), dh)
    x = (x + g1 * _lin(o, w[f"{ex}.{i}.o.w"], w[f"{ex}.{i}.o.b"])).astype(F)
    g = bf16_round(_gelu(_lin(_ln_mod(x, sh2, sc2, m.ln_eps), w[f"{ex}.{i}.fc1.w"], w[f"{ex}.{i}.fc1.b"])))
    x = (x + g2 * _lin(g, w[f"{ex}.{i}.fc2.w"], w[f"{ex}.{i}.fc2.b"])).astype(F)
    return x, k, v


def infer(w, m, video, noise, grid):
    """One sample: video [T_v, d_v], noise [T_a, A] -> dict like the oracle's
    (a_out, v, f per step, kv list, x_video), all float32."""
    w = {k: np.asarray(v, F) for k, v in w.items()}
    x = np.asarray(video, F)
    cv = _cond(w, "v", 0.0, m.t_freq_dim)
    kv = []
    for i in range(m.n_blocks):
        mod = _lin(_silu(cv), w[f"v.{i}.ada.w"], w[f"v.{i}.ada.b"])
        x, k, v = _block(w, "v", i, mod, x, m)
        kv.append((k, v))
    a = np.asarray(noise, F)
    g = np.asarray(grid, F)
    S = g.size - 1
    vs, fs = [], []
    for j in range(S, 0, -1):
        ca = _cond(w, "a", float(g[j]), m.t_freq_dim)
        y = _lin(a, w["a.in.w"], w["a.in.b"])
        for i in range(m.n_blocks):
            mod = _lin(_silu(ca), w[f"a.{i}.ada.w"], w[f"a.{i}.ada.b"])
            y, _, _ = _block(w, "a", i, mod, y, m, kv[i])
        mf = _lin(_silu(ca), w["a.fada.w"], w["a.fada.b"])
        da = m.d_action
        mu = y.mean(-1, keepdims=True, dtype=F)
        var = ((y - mu) ** 2).mean(-1, keepdims=True, dtype=F)
        hf = ((y - mu) / np.sqrt(var + F(m.ln_eps))) * (F(1) + mf[da:]) + mf[:da]
        vel = _lin(hf, w["a.out.w"], w["a.out.b"])
        vs.append(vel)
        fs.append((a - g[j] * vel).astype(F))
        a = (a - (g[j] - g[j - 1]) * vel).astype(F)
    return {"a_out": a, "v": vs, "f": fs, "kv": kv, "x_video": x}
