"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Nothing here re-types an oracle formula in the same form.  Primitives are
checked by scalar brute force (python loops, math.fsum, math.erf/exp), the
composition rules by special cases with closed forms, and the method-level
claims of the pages by invariants:
  * Euler update and endpoint map (RealtimeWAM digest, Background: flow
    matching) -> constant-velocity closed form, S=1 endpoint identity, one
    step from t to 0 equals the endpoint;
  * step count T_seq = T_v + S*T_a (digest, Core method) -> NFE counts;
  * action block i needs only video block i's KV (digest, Core method and
    Method steps) -> perturbation test on hidden states;
  * the wavefront order is another topological order of the same graph
    (digest, Novelty) -> interleaved run == sequential run, bitwise.
"""
import dataclasses
import math

import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O

PICO = wl.ModelShape(n_blocks=2, d_video=8, d_action=6, n_heads=2, head_dim=4,
                     action_dim=3, dtype=wl.F32, t_freq_dim=16)


def pico_weights(std=0.3, seed=0):
    return wl.make_weights(PICO, seed=seed, std=std)


def pico_inputs(tv=5, ta=3, b=1):
    rng = np.random.default_rng(123)
    video = rng.standard_normal((b, tv, PICO.d_video))
    a = rng.standard_normal((b, ta, PICO.action_dim))
    return video, a


# ----------------------------------------------------------------------------- primitives

# ----------------------------------------------------------------------------- block variant: QK-RMSNorm + 3-D RoPE
def test_rms_norm_worked_example_and_closed_form():
    # [3, 4] has mean square 12.5: with eps = 0 it becomes [3, 4] / sqrt(12.5)
    out = O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(out, [0.848528137423857, 1.131370849898476], rtol=1e-14)
    # unit gain: the output mean square is ms / (ms + eps), ms the input's
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 24)) * 3
    eps = 1e-3
    y = O.rms_norm(x, np.ones(24), eps)
    ms = np.array([math.fsum(v * v for v in row) / 24 for row in x])
    assert np.allclose((y ** 2).mean(-1), ms / (ms + eps), rtol=1e-12)
    # a positive factor on x cancels (eps = 0); the gain acts feature by feature
    g = rng.standard_normal(24)
    ref = O.rms_norm(5.0 * x, np.ones(24), 0.0)
    assert np.allclose(O.rms_norm(x, g, 0.0), np.stack([ref[:, j] * g[j] for j in range(24)], 1), rtol=1e-12)


def test_rope_positions_grid():
    pos = O.rope_positions(24, (3, 4))  # two frames of 3 x 4 patches
    assert pos[0].tolist() == [0, 0, 0] and pos[5].tolist() == [0, 1, 1]
    assert pos[12].tolist() == [1, 0, 0] and pos[23].tolist() == [1, 2, 3]
    with pytest.raises(ValueError):
        O.rope_positions(25, (3, 4))


def test_rope_worked_examples():
    # one pair per band: pair b turns by coordinate b radians (theta^0 = 1)
    x = np.array([[[1.0, 0.0, 1.0, 0.0, 1.0, 0.0]]])
    out = O.rope3d(x, np.array([[1, 2, 3]]), (2, 2, 2))[0, 0]
    assert np.allclose(out, [math.cos(1), math.sin(1), math.cos(2), math.sin(2), math.cos(3), math.sin(3)], atol=1e-15)
    # the second feature of a pair turns to (-sin, cos)
    out2 = O.rope3d(np.array([[[0.0, 1.0, 0, 0, 0, 0]]]), np.array([[0.5, 0, 0]]), (2, 2, 2))[0, 0]
    assert np.allclose(out2[:2], [-math.sin(0.5), math.cos(0.5)], atol=1e-15)


def test_rope_frequencies():
    # bands of 4 features: pair 1 of a band turns by 10000^(-2/4) = 1/100 rad per position
    x = np.zeros((1, 1, 12))
    for band in range(3):
        x[:] = 0.0
        x[0, 0, 4 * band + 2] = 1.0
        for p in (1, 7, 100):
            pos = np.zeros((1, 3), dtype=int)
            pos[0, band] = p
            out = O.rope3d(x, pos, (4, 4, 4))[0, 0]
            ang = math.atan2(out[4 * band + 3], out[4 * band + 2])
            assert math.isclose(ang, math.remainder(p / 100.0, 2 * math.pi), abs_tol=1e-12)


def test_rope_band_sizes():
    # worked values of the band split: 44/42/42 features for the 128-wide heads
    # of the Fast-WAM-scale model, 24/20/20 for 64, 12/10/10 for 32
    assert O.rope_bands(128) == (44, 42, 42)
    assert O.rope_bands(64) == (24, 20, 20)
    assert O.rope_bands(32) == (12, 10, 10)
    for dh in range(6, 258, 2):
        f, r, c = O.rope_bands(dh)
        assert f + r + c == dh and r == c and f >= r and f % 2 == 0 and r % 2 == 0
        assert r == c == max(x for x in range(0, dh + 1, 2) if 3 * x <= dh)  # the widest even band with 3x <= dh


def test_rope_invariants():
    rng = np.random.default_rng(9)
    H, T, dh = 2, 10, 12
    bands = O.rope_bands(dh)
    assert bands == (4, 4, 4)
    q, k = rng.standard_normal((H, T, dh)), rng.standard_normal((H, T, dh))
    pos = rng.integers(0, 20, size=(T, 3))
    # position 0 is the identity; every feature pair keeps its length
    assert np.array_equal(O.rope3d(q, np.zeros((T, 3), dtype=int), bands), q)
    r = O.rope3d(q, pos, bands)
    assert np.allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, q[..., 0::2] ** 2 + q[..., 1::2] ** 2, rtol=1e-12)
    # scores depend on relative positions only
    s0 = np.einsum("htd,hsd->hts", r, O.rope3d(k, pos, bands))
    sh = pos + np.array([3, 5, 7])
    s1 = np.einsum("htd,hsd->hts", O.rope3d(q, sh, bands), O.rope3d(k, sh, bands))
    assert np.allclose(s0, s1, rtol=1e-10, atol=1e-12)
    # moving one column changes only the column band (the last 2[dh/6] features)
    p2 = pos.copy()
    p2[:, 2] += 1
    d = O.rope3d(q, p2, bands) - r
    assert np.all(d[..., :bands[0] + bands[1]] == 0) and np.all(np.any(d[..., bands[0] + bands[1]:] != 0, -1))


def test_qk_norm_spans_all_heads_and_rope_only_video():
    m = dataclasses.replace(PICO, qk_norm=True)
    w = wl.make_weights(m, std=0.3)
    for name in w:
        if wl.is_gain(name):
            w[name] = np.ones_like(w[name])
    P = O.Params(w)
    x = np.random.default_rng(4).standard_normal((6, m.d_video))
    c = O.t_conditioning(P, "v", 0.0, m)
    q, k, _ = O.project(P, "v", 0, O.block_modulation(P, "v", 0, c), x, m)
    full = lambda t: t.transpose(1, 0, 2).reshape(6, -1)  # [T, H dh]
    ms_all = (full(q) ** 2).mean(-1)
    assert np.allclose(ms_all, 1.0, atol=1e-4)             # one RMS over every head of a token ...
    assert not np.allclose((q ** 2).mean(-1), 1.0, atol=1e-2)  # ... not one per head
    # the rotary embedding turns the video expert's q and k, never the action expert's
    mr = dataclasses.replace(m, rope_hw=(1, 2))
    qr, kr, _ = O.project(P, "v", 0, O.block_modulation(P, "v", 0, c), x, mr)
    assert not np.allclose(qr, q) and np.allclose((qr ** 2).sum(-1), (q ** 2).sum(-1))
    ca = O.t_conditioning(P, "a", 0.5, m)
    y = np.random.default_rng(6).standard_normal((3, m.d_action))
    qa = O.project(P, "a", 1, O.block_modulation(P, "a", 1, ca), y, m)[0]
    qa_r = O.project(P, "a", 1, O.block_modulation(P, "a", 1, ca), y, mr)[0]
    assert np.array_equal(qa, qa_r)

def test_linear_brute_force():
    rng = np.random.default_rng(0)
    x, W, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    y = O.linear(x, W, b)
    for i in range(3):
        for j in range(4):
            ref = math.fsum([x[i, k] * W[j, k] for k in range(5)] + [b[j]])
            assert abs(y[i, j] - ref) <= 1e-13 * (1 + abs(ref))


def test_layer_norm_closed_form():
    rng = np.random.default_rng(1)
    eps = 1e-6
    x = rng.standard_normal((4, 17)) * 3 + 5
    y = O.layer_norm(x, eps)
    for r in range(4):
        row = list(x[r])
        mu = math.fsum(row) / len(row)
        var = math.fsum([(v - mu) ** 2 for v in row]) / len(row)  # population variance
        assert abs(math.fsum(y[r])) < 1e-12
        assert abs(math.fsum([v * v for v in y[r]]) / len(row) - var / (var + eps)) < 1e-12
        for k in range(len(row)):
            assert abs(y[r, k] - (row[k] - mu) / math.sqrt(var + eps)) < 1e-12
    # eps matters for a near-constant row: var/(var+eps) well below 1
    z = O.layer_norm(np.array([[1.0, 1.0 + 1e-3]]), 1e-6)
    assert abs((z ** 2).mean() - (0.25e-6 / (0.25e-6 + 1e-6))) < 1e-12


def test_modulate_reduces_to_layer_norm():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((3, 6))
    assert np.array_equal(O.modulate(h, np.zeros(6), np.zeros(6)), h)
    s = rng.standard_normal(6)
    assert np.array_equal(O.modulate(h, s, -np.ones(6)), np.broadcast_to(s, h.shape))


def test_gelu_silu():
    zs = np.linspace(-6, 6, 97)
    g = O.gelu(zs)
    for z, gz in zip(zs, g):
        assert abs(gz - 0.5 * z * (1 + math.erf(z / math.sqrt(2)))) < 1e-15 * (1 + abs(z))
        assert abs(O.silu(np.array(z)) - z / (1 + math.exp(-z))) < 1e-15 * (1 + abs(z))
    assert np.allclose(O.gelu(zs) - O.gelu(-zs), zs, atol=1e-14)
    assert np.allclose(O.silu(zs) - O.silu(-zs), zs, atol=1e-14)
    # exact-erf form, not the tanh approximation: they differ by ~1e-4 near |z|=2
    assert abs(O.gelu(np.array(2.0)) - 1.9544997361036416) < 1e-15


def test_timestep_embedding_structure():
    e0 = O.timestep_embedding(0.0, 256)
    assert np.array_equal(e0, np.concatenate([np.ones(128), np.zeros(128)]))
    for t in (0.0, 0.1, 0.5, 1.0):
        e = O.timestep_embedding(t, 256)
        assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-14)
    # recover the arguments at a small t (all below pi): arg_0 = 1000 t and a
    # geometric ladder of ratio 10000^(-1/128)
    t = 1e-4
    e = O.timestep_embedding(t, 256)
    args = np.arctan2(e[128:], e[:128])
    assert abs(args[0] - 1000 * t) < 1e-15
    assert np.allclose(args[1:] / args[:-1], 10000 ** (-1 / 128), rtol=1e-12)


def _attn_brute(q, k, v):
    H, Tq, dh = q.shape
    L = k.shape[1]
    out = np.zeros((Tq, H * dh))
    for h in range(H):
        for i in range(Tq):
            s = [math.fsum(q[h, i, d] * k[h, j, d] for d in range(dh)) / math.sqrt(dh) for j in range(L)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = math.fsum(w)
            for d in range(dh):
                out[i, h * dh + d] = math.fsum(w[j] * v[h, j, d] for j in range(L)) / z
    return out


def test_attention_brute_force():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((2, 3, 4)), rng.standard_normal((2, 5, 4)), rng.standard_normal((2, 5, 4))
    assert np.allclose(O.attention(q, k, v), _attn_brute(q, k, v), rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    H, dh = 2, 4
    q = rng.standard_normal((H, 3, dh))
    # one key -> that key's value, whatever the query
    k1, v1 = rng.standard_normal((H, 1, dh)), rng.standard_normal((H, 1, dh))
    o = O.attention(q, k1, v1)
    for h in range(H):
        assert np.allclose(o[:, h * dh:(h + 1) * dh], v1[h, 0], atol=1e-15)
    # identical keys, or a zero query -> mean of the values
    v = rng.standard_normal((H, 6, dh))
    kk = np.repeat(rng.standard_normal((H, 1, dh)), 6, axis=1)
    for qq, keys in ((q, kk), (np.zeros_like(q), rng.standard_normal((H, 6, dh)))):
        o = O.attention(qq, keys, v)
        for h in range(H):
            assert np.allclose(o[:, h * dh:(h + 1) * dh], v[h].mean(axis=0), atol=1e-14)
    # duplicating every key/value pair changes nothing (the concatenated key set
    # [own ; video] with video == own reduces to self-attention)
    k, v = rng.standard_normal((H, 5, dh)), rng.standard_normal((H, 5, dh))
    assert np.allclose(O.attention(q, np.concatenate([k, k], 1), np.concatenate([v, v], 1)),
                       O.attention(q, k, v), atol=1e-14)
    # key order does not matter
    perm = rng.permutation(5)
    assert np.allclose(O.attention(q, k[:, perm], v[:, perm]), O.attention(q, k, v), atol=1e-14)


# ----------------------------------------------------------------------------- block composition
def _block_weights(d, D, rng):
    w = {}
    w["x.0.qkv.w"], w["x.0.qkv.b"] = rng.standard_normal((3 * D, d)), rng.standard_normal(3 * D)
    w["x.0.o.w"], w["x.0.o.b"] = rng.standard_normal((d, D)), rng.standard_normal(d)
    w["x.0.fc1.w"], w["x.0.fc1.b"] = rng.standard_normal((4 * d, d)), rng.standard_normal(4 * d)
    w["x.0.fc2.w"], w["x.0.fc2.b"] = rng.standard_normal((d, 4 * d)), rng.standard_normal(d)
    return w


def _mod(d, **kw):
    names = ["shift1", "scale1", "gate1", "shift2", "scale2", "gate2"]
    return [np.asarray(kw.get(n, np.zeros(d)), dtype=np.float64) * np.ones(d) for n in names]


def _mv(W, x):
    return np.array([math.fsum(W[r, c] * x[c] for c in range(len(x))) for r in range(W.shape[0])])


def test_block_zero_gates_is_identity():
    m = dataclasses.replace(PICO, d_video=6)
    rng = np.random.default_rng(5)
    w = _block_weights(6, m.d_attn, rng)
    P = O.Params(w)
    x = rng.standard_normal((5, 6))
    mod = _mod(6, shift1=rng.standard_normal(6), scale1=rng.standard_normal(6),
               shift2=rng.standard_normal(6), scale2=rng.standard_normal(6))
    q, k, v = O.project(P, "x", 0, mod, x, m)
    assert np.array_equal(O.rest(P, "x", 0, mod, x, O.attention(q, k, v), m), x)


def test_block_modulation_order_closed_forms():
    """Each of the six adaLN vectors acts where the block definition puts it."""
    d = 6
    m = dataclasses.replace(PICO, d_video=d)
    D, H, dh = m.d_attn, m.n_heads, m.head_dim
    rng = np.random.default_rng(6)
    P_w = _block_weights(d, D, rng)
    x = rng.standard_normal((5, d))
    beta = rng.standard_normal(d)

    # gate1 = 1, W_o = 0, b_o = beta, gate2 = 0  ->  x + beta
    w = dict(P_w, **{"x.0.o.w": np.zeros((d, D)), "x.0.o.b": beta})
    P = O.Params(w)
    mod = _mod(d, gate1=1.0, shift1=rng.standard_normal(d), scale1=rng.standard_normal(d))
    q, k, v = O.project(P, "x", 0, mod, x, m)
    assert np.allclose(O.rest(P, "x", 0, mod, x, O.attention(q, k, v), m), x + beta, atol=1e-14)

    # gate2 = 1, W_fc2 = 0, b_fc2 = beta, gate1 = 0  ->  x + beta
    w = dict(P_w, **{"x.0.fc2.w": np.zeros((d, 4 * d)), "x.0.fc2.b": beta})
    P = O.Params(w)
    mod = _mod(d, gate2=1.0, shift2=rng.standard_normal(d), scale2=rng.standard_normal(d))
    q, k, v = O.project(P, "x", 0, mod, x, m)
    assert np.allclose(O.rest(P, "x", 0, mod, x, O.attention(q, k, v), m), x + beta, atol=1e-14)

    # scale1 = -1, shift1 = s: every token's normalised input is s, so every
    # query/key/value row is the same and attention returns the common value
    s = rng.standard_normal(d)
    P = O.Params(P_w)
    mod = _mod(d, shift1=s, scale1=-1.0, gate1=1.0)
    q, k, v = O.project(P, "x", 0, mod, x, m)
    Wqkv, bqkv = P_w["x.0.qkv.w"], P_w["x.0.qkv.b"]
    qkv_ref = _mv(Wqkv, s) + bqkv
    for which, t in enumerate((q, k, v)):
        for h in range(H):
            for r in range(5):
                assert np.allclose(t[h, r], qkv_ref[which * D + h * dh: which * D + (h + 1) * dh], atol=1e-13)
    o = O.attention(q, k, v)
    expect = x + (_mv(P_w["x.0.o.w"], qkv_ref[2 * D:]) + P_w["x.0.o.b"])
    assert np.allclose(O.rest(P, "x", 0, mod, x, o, m), expect, atol=1e-12)

    # scale2 = -1, shift2 = s2, gate2 = 1, gate1 = 0: MLP of the constant s2
    s2 = rng.standard_normal(d)
    mod = _mod(d, shift2=s2, scale2=-1.0, gate2=1.0)
    hid = _mv(P_w["x.0.fc1.w"], s2) + P_w["x.0.fc1.b"]
    hid = np.array([0.5 * z * (1 + math.erf(z / math.sqrt(2))) for z in hid])
    mlp = _mv(P_w["x.0.fc2.w"], hid) + P_w["x.0.fc2.b"]
    q, k, v = O.project(P, "x", 0, mod, x, m)
    assert np.allclose(O.rest(P, "x", 0, mod, x, O.attention(q, k, v), m), x + mlp, atol=1e-12)


def test_adaln_chunks_come_from_silu_of_c():
    # zero W_ada: the six vectors are the bias chunks in order
    m = PICO
    d = m.d_video
    b = np.arange(6 * d, dtype=np.float64)
    P = O.Params({"v.0.ada.w": np.zeros((6 * d, d)), "v.0.ada.b": b})
    mod = O.block_modulation(P, "v", 0, np.ones(d))
    for j in range(6):
        assert np.array_equal(mod[j], b[j * d:(j + 1) * d])
    # identity-like W_ada: chunk j of the output is SiLU(c)
    W = np.concatenate([np.eye(d)] * 6)
    c = np.linspace(-2, 2, d)
    mod = O.block_modulation(O.Params({"v.0.ada.w": W, "v.0.ada.b": np.zeros(6 * d)}), "v", 0, c)
    for j in range(6):
        assert np.allclose(mod[j], [z / (1 + math.exp(-z)) for z in c], atol=1e-15)


# ----------------------------------------------------------------------------- t-conditioning and the final layer
def _sinusoid_brute(t, dim):
    half = dim // 2
    args = [1000.0 * t * 10000.0 ** (-k / half) for k in range(half)]
    return [math.cos(a) for a in args] + [math.sin(a) for a in args]


def _silu_brute(z):
    return [x / (1.0 + math.exp(-x)) for x in z]


def test_t_conditioning_brute_force():
    """c = W_t2 SiLU(W_t1 temb(t) + b_t1) + b_t2, by scalar loops, for both experts."""
    m = PICO
    rng = np.random.default_rng(12)
    for ex, d in (("v", m.d_video), ("a", m.d_action)):
        w = {f"{ex}.t1.w": rng.standard_normal((d, m.t_freq_dim)), f"{ex}.t1.b": rng.standard_normal(d),
             f"{ex}.t2.w": rng.standard_normal((d, d)), f"{ex}.t2.b": rng.standard_normal(d)}
        P = O.Params(w)
        for t in (0.0, 3e-4, 0.37, 1.0):
            e = np.array(_sinusoid_brute(t, m.t_freq_dim))
            h = np.array(_silu_brute(_mv(w[f"{ex}.t1.w"], e) + w[f"{ex}.t1.b"]))
            c_ref = _mv(w[f"{ex}.t2.w"], h) + w[f"{ex}.t2.b"]
            assert np.allclose(O.t_conditioning(P, ex, t, m), c_ref, rtol=0, atol=1e-12)
        # a zero output layer leaves exactly its bias
        w0 = dict(w, **{f"{ex}.t2.w": np.zeros((d, d))})
        assert np.array_equal(O.t_conditioning(O.Params(w0), ex, 0.4, m), w[f"{ex}.t2.b"])
        # a zero first layer: the hidden vector is SiLU(b_t1) whatever t is
        w1 = dict(w, **{f"{ex}.t1.w": np.zeros((d, m.t_freq_dim))})
        c1 = _mv(w[f"{ex}.t2.w"], np.array(_silu_brute(w[f"{ex}.t1.b"]))) + w[f"{ex}.t2.b"]
        for t in (0.0, 0.8):
            assert np.allclose(O.t_conditioning(O.Params(w1), ex, t, m), c1, rtol=0, atol=1e-13)


def _final_weights(d, A, rng):
    return {"a.fada.w": rng.standard_normal((2 * d, d)), "a.fada.b": rng.standard_normal(2 * d),
            "a.out.w": rng.standard_normal((A, d)), "a.out.b": rng.standard_normal(A)}


def _ln_brute(row, eps):
    n = len(row)
    mu = math.fsum(row) / n
    var = math.fsum((z - mu) ** 2 for z in row) / n
    return [(z - mu) / math.sqrt(var + eps) for z in row]


def test_final_layer_closed_forms():
    """v = (LN(y)(1+scale_f)+shift_f) W_out^T + b_out with (shift_f, scale_f), in
    that order, from W_fada SiLU(c) + b_fada."""
    m = PICO
    d, A = m.d_action, m.action_dim
    rng = np.random.default_rng(13)
    w = _final_weights(d, A, rng)
    y = rng.standard_normal((4, d)) * 3 + 1
    c = rng.standard_normal(d)
    # W_fada = 0 and the scale chunk of the bias -1: the normalised tokens drop
    # out and every token's velocity is (first bias chunk) W_out^T + b_out
    s = rng.standard_normal(d)
    w1 = dict(w, **{"a.fada.w": np.zeros((2 * d, d)), "a.fada.b": np.concatenate([s, -np.ones(d)])})
    v = O.final_layer(O.Params(w1), m, y, c)
    expect = _mv(w["a.out.w"], s) + w["a.out.b"]
    for r in range(y.shape[0]):
        assert np.allclose(v[r], expect, rtol=0, atol=1e-13)
    # zero modulation: v = LN(y) W_out^T + b_out (LayerNorm by scalar loops)
    w2 = dict(w, **{"a.fada.w": np.zeros((2 * d, d)), "a.fada.b": np.zeros(2 * d)})
    v = O.final_layer(O.Params(w2), m, y, c)
    for r in range(y.shape[0]):
        ref = _mv(w["a.out.w"], np.array(_ln_brute(y[r], m.ln_eps))) + w["a.out.b"]
        assert np.allclose(v[r], ref, rtol=0, atol=1e-12)
    # the shift comes from SiLU(c): W_fada = [I ; 0], b_fada = [0 ; -1]
    w3 = dict(w, **{"a.fada.w": np.concatenate([np.eye(d), np.zeros((d, d))]),
                    "a.fada.b": np.concatenate([np.zeros(d), -np.ones(d)])})
    v = O.final_layer(O.Params(w3), m, y, c)
    expect = _mv(w["a.out.w"], np.array(_silu_brute(c))) + w["a.out.b"]
    for r in range(y.shape[0]):
        assert np.allclose(v[r], expect, rtol=0, atol=1e-13)
    # general weights, by scalar loops end to end
    P = O.Params(w)
    mv = _mv(w["a.fada.w"], np.array(_silu_brute(c))) + w["a.fada.b"]
    shift, scale = mv[:d], mv[d:]
    v = O.final_layer(P, m, y, c)
    for r in range(y.shape[0]):
        ln = _ln_brute(y[r], m.ln_eps)
        hmod = np.array([ln[j] * (1.0 + scale[j]) + shift[j] for j in range(d)])
        assert np.allclose(v[r], _mv(w["a.out.w"], hmod) + w["a.out.b"], rtol=0, atol=1e-11)
    # the LayerNorm removes a constant offset of every token
    assert np.allclose(O.final_layer(P, m, y + 7.5, c), v, rtol=0, atol=1e-11)
    assert not np.allclose(O.final_layer(P, m, y * np.linspace(0.5, 2.0, d), c), v, atol=1e-3)


def test_velocity_uses_the_final_layer_of_the_last_hidden_state():
    # the action pass ends in final_layer(y^N, c_a(t)): W_out = 0 leaves b_out
    # (the constant-velocity case), and with a zero final modulation the
    # velocity is LN(y^N) W_out^T + b_out of the pass's own last hidden state
    w = pico_weights()
    w["a.fada.w"] = np.zeros_like(w["a.fada.w"])
    w["a.fada.b"] = np.zeros_like(w["a.fada.b"])
    video, a = pico_inputs()
    P = O.Params(w)
    kv, _ = O.video_forward(P, PICO, video[0])
    hid = []
    v = O.action_velocity(P, PICO, kv, a[0], 0.6, hidden=hid)
    for r in range(a.shape[1]):
        ref = _mv(w["a.out.w"].astype(np.float64), np.array(_ln_brute(hid[-1][r], PICO.ln_eps))) + w["a.out.b"]
        assert np.allclose(v[r], ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- Euler / endpoint
def test_constant_velocity_closed_form():
    w = pico_weights()
    w["a.out.w"] = np.zeros_like(w["a.out.w"])  # v = b_out everywhere
    video, a = pico_inputs()
    for S in (1, 2, 5, 10):
        r = O.infer(w, PICO, video[0], a[0], wl.t_grid(S))
        for v in r["v"]:
            assert np.array_equal(v, np.broadcast_to(w["a.out.b"].astype(np.float64), v.shape))
        assert np.allclose(r["a_out"], a[0] - w["a.out.b"], atol=1e-14)


def test_endpoint_identities():
    w = pico_weights()
    video, a = pico_inputs()
    r = O.infer(w, PICO, video[0], a[0], wl.t_grid(1))
    assert np.array_equal(r["a_out"], r["f"][0])  # S = 1: one step to t=0 is the endpoint
    t = 0.37
    r = O.infer(w, PICO, video[0], a[0], np.array([0.0, t]))
    assert np.array_equal(r["a_out"], r["f"][0])
    assert np.array_equal(r["f"][0], a[0] - t * r["v"][0])
    # the velocity actually depends on t
    r2 = O.infer(w, PICO, video[0], a[0], np.array([0.0, 0.9]))
    assert not np.allclose(r2["v"][0], r["v"][0])


def test_grid_validation():
    w = pico_weights()
    video, a = pico_inputs()
    for bad in ([0.0], [0.5, 0.5], [0.0, 1.2], [1.0, 0.0]):
        with pytest.raises(ValueError):
            O.infer(w, PICO, video[0], a[0], np.array(bad))


def test_nfe_count_matches_tseq():
    w = pico_weights()
    video, a = pico_inputs()
    for S in (1, 3, 10):
        c = O.Counters()
        O.infer(w, PICO, video[0], a[0], wl.t_grid(S), counters=c)
        assert (c.video_passes, c.action_passes) == (1, S)
        c = O.Counters()
        O.infer_interleaved(w, PICO, video[0], a[0], wl.t_grid(S), counters=c)
        assert (c.video_passes, c.action_passes) == (1, S)


# ----------------------------------------------------------------------------- structure claims
def test_action_block_i_depends_only_on_video_block_i():
    w = pico_weights()
    video, a = pico_inputs()
    P = O.Params(w)
    kv, _ = O.video_forward(P, PICO, video[0])
    base = []
    O.action_velocity(P, PICO, kv, a[0], 1.0, hidden=base)
    for j in range(PICO.n_blocks):
        kv2 = list(kv)
        kv2[j] = (kv[j][0] + 0.5, kv[j][1] - 0.5)
        hid = []
        O.action_velocity(P, PICO, kv2, a[0], 1.0, hidden=hid)
        for i in range(j):
            assert np.array_equal(hid[i], base[i])
        for i in range(j, PICO.n_blocks):
            assert not np.allclose(hid[i], base[i])


def test_video_kv_independent_of_action():
    w = pico_weights()
    video, a = pico_inputs()
    r1 = O.infer(w, PICO, video[0], a[0], wl.t_grid(2))
    r2 = O.infer(w, PICO, video[0], -3 * a[0], wl.t_grid(3))
    for (k1, v1), (k2, v2) in zip(r1["kv"], r2["kv"]):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


@pytest.mark.parametrize("S", [1, 3])
def test_wavefront_order_equals_sequential_bitwise(S):
    w = pico_weights()
    video, a = pico_inputs()
    r1 = O.infer(w, PICO, video[0], a[0], wl.t_grid(S))
    r2 = O.infer_interleaved(w, PICO, video[0], a[0], wl.t_grid(S))
    assert np.array_equal(r1["a_out"], r2["a_out"])
    for j in range(S):
        assert np.array_equal(r1["v"][j], r2["v"][j]) and np.array_equal(r1["f"][j], r2["f"][j])
    assert np.array_equal(r1["x_video"], r2["x_video"])


def test_video_token_permutation_invariance():
    w = pico_weights()
    video, a = pico_inputs(tv=7)
    perm = np.random.default_rng(9).permutation(7)
    r1 = O.infer(w, PICO, video[0], a[0], wl.t_grid(2))
    r2 = O.infer(w, PICO, video[0][perm], a[0], wl.t_grid(2))
    assert np.allclose(r1["a_out"], r2["a_out"], rtol=1e-12, atol=1e-12)
    assert np.allclose(r1["v"][1], r2["v"][1], rtol=1e-12, atol=1e-12)
    assert np.allclose(r1["kv"][1][0][:, perm], r2["kv"][1][0], rtol=1e-12, atol=1e-12)


def test_batch_independence():
    w = pico_weights()
    video, a = pico_inputs(b=3)
    rb = O.infer_batch(w, PICO, video, a, wl.t_grid(2))
    for b in range(3):
        r = O.infer(w, PICO, video[b], a[b], wl.t_grid(2))
        assert np.array_equal(rb["a_out"][b], r["a_out"])
        assert np.array_equal(rb["v"][0][b], r["v"][0])


def test_no_video_tokens_is_self_attention():
    # T_v = 0: the action expert attends over its own keys only; with video
    # K/V equal to its own (duplicated pairs) the answer is the same
    w = pico_weights()
    _, a = pico_inputs()
    P = O.Params(w)
    H, dh = PICO.n_heads, PICO.head_dim
    empty = [(np.zeros((H, 0, dh)), np.zeros((H, 0, dh)))] * PICO.n_blocks
    v0 = O.action_velocity(P, PICO, empty, a[0], 1.0)
    assert np.all(np.isfinite(v0))


def test_workload_generators_deterministic_and_bf16():
    m = wl.SMALL
    w1 = wl.make_weights(m, names=["v.0.o.b", "a.out.w"])
    w2 = wl.make_weights(m, names=["a.out.w"])
    assert np.array_equal(w1["a.out.w"], w2["a.out.w"])
    assert not np.any(w1["a.out.w"].view(np.uint32) & 0xFFFF)  # bf16-representable
    # round-to-nearest-even on exact ties and a plain case
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], dtype=np.float32)
    assert list(wl.bf16_round(x)) == [1.0, 1.0 + 2 ** -6, 1.0, -2.5]
    v = wl.make_video(m, 2, 8)
    v1 = wl.make_video(m, 2, 8, samples=[1])
    assert np.array_equal(v[1], v1[0])
    assert list(wl.t_grid(4)) == [0.0, 0.25, 0.5, 0.75, 1.0]


# ----------------------------------------------------------------------------- teacher-anchored targets
def _targets_setup(seed=0, zero_out=False):
    w = pico_weights(seed=seed)
    if zero_out:
        w["a.out.w"] = np.zeros_like(w["a.out.w"])
    video, _ = pico_inputs(tv=5, ta=3)
    P = O.Params(w)
    kv, _ = O.video_forward(P, PICO, video[0])
    rng = np.random.default_rng(31)
    a0, eps = rng.standard_normal((3, PICO.action_dim)), rng.standard_normal((3, PICO.action_dim))
    return w, P, kv, a0, eps, video


def test_targets_constant_velocity_closed_form():
    # W_out = 0: every velocity is b_out, so the teacher lands at a_t - t b_out
    # and the interval-average velocity is b_out itself, for any t and K
    w, P, kv, a0, eps, _ = _targets_setup(zero_out=True)
    b = w["a.out.b"].astype(np.float64)
    for t, K in ((0.37, 10), (1.0, 3), (0.05, 7)):
        r = O.teacher_targets(P, P, PICO, kv, a0, eps, t, K)
        assert np.allclose(r["a_t"], (1 - t) * a0 + t * eps, rtol=0, atol=1e-15)
        assert np.allclose(r["u"], np.broadcast_to(b, r["u"].shape), rtol=1e-9, atol=1e-12)
        assert np.allclose(r["f"], r["aT0"], rtol=0, atol=1e-12)


def test_targets_one_step_teacher_is_the_endpoint():
    # K = 1 and the student equal to the teacher: one Euler step from t to 0 is the endpoint map
    w, P, kv, a0, eps, _ = _targets_setup()
    r = O.teacher_targets(P, P, PICO, kv, a0, eps, 0.6, 1)
    assert np.array_equal(r["f"], r["aT0"])
    v = O.action_velocity(P, PICO, kv, r["a_t"], 0.6)
    assert np.allclose(r["u"], v, rtol=1e-12, atol=1e-14)


def test_targets_from_pure_noise_match_inference():
    # t = 1: a_t is the noise, and the teacher rollout is the K-step inference of the pinned driver
    w, P, kv, a0, eps, video = _targets_setup()
    r = O.teacher_targets(P, P, PICO, kv, a0, eps, 1.0, 4)
    assert np.array_equal(r["a_t"], eps)
    ref = O.infer(P, PICO, video[0], eps, wl.t_grid(4))
    assert np.allclose(r["aT0"], ref["a_out"], rtol=1e-6, atol=1e-9)  # float32 vs float64 grid values
    with pytest.raises(ValueError):
        O.teacher_targets(P, P, PICO, kv, a0, eps, 0.0, 4)
    with pytest.raises(ValueError):
        O.teacher_targets(P, P, PICO, kv, a0, eps, 1.5, 4)


def test_targets_rollouts_are_independent_and_share_one_cache():
    w, P, kv, a0, eps, video = _targets_setup()
    rng = np.random.default_rng(8)
    A0, E = rng.standard_normal((3, 3, PICO.action_dim)), rng.standard_normal((3, 3, PICO.action_dim))
    ts = [0.9, 0.25, 0.6]
    w_s = pico_weights(seed=5)  # a different student
    batch = O.teacher_targets_batch(w, w_s, PICO, video[0], A0, E, ts, K=3)
    Ps = O.Params(w_s)
    for r in range(3):
        one = O.teacher_targets(P, Ps, PICO, kv, A0[r], E[r], ts[r], 3)
        for k in ("a_t", "aT0", "u", "f"):
            assert np.array_equal(batch[k][r], one[k])


# ----------------------------------------------------------------------------- selective reuse across observations
def _moved(prev, factors, rng):
    """Each token j moved by factors[j] * ||prev_j|| in a random direction."""
    new = prev.copy()
    for j, f in enumerate(factors):
        d = rng.standard_normal(prev.shape[1])
        new[j] = prev[j] + d / np.linalg.norm(d) * f * np.linalg.norm(prev[j])
    return new


def _brute_active(new, prev, tau):
    n32, p32 = np.asarray(new, np.float32).astype(np.float64), np.asarray(prev, np.float32).astype(np.float64)
    return [j for j in range(len(p32))
            if math.fsum((n32[j] - p32[j]) ** 2) > tau * tau * math.fsum(p32[j] ** 2)]


def test_select_tokens_brute_force():
    rng = np.random.default_rng(5)
    prev = rng.standard_normal((10, 8))
    tau = 0.1
    factors = [0.0, 0.05, 0.2, 2.0, 0.02, 3.0, 0.0, 0.5, 0.0, 0.0]
    new = _moved(prev, factors, rng)
    prev[8] = 0.0
    new[8] = 0.0                       # zero token, unchanged: stable
    prev[9] = 0.0
    new[9] = 1e-3                      # zero token that moved at all: active
    got = list(O.select_tokens(new, prev, tau))
    assert got == _brute_active(new, prev, tau) == [2, 3, 5, 7, 9]
    # threshold relative to the previous token: a token scaled by 1.6 moved 0.6 of its old norm
    # (active at tau = 0.5) but only 0.375 of its new one; one scaled by 0.5 moved 0.5 of its old
    # norm (stable at tau = 0.6) but 1.0 of its new one
    p2 = rng.standard_normal((2, 8))
    n2 = np.stack([1.6 * p2[0], 0.5 * p2[1]])
    assert list(O.select_tokens(n2[:1], p2[:1], 0.5)) == [0]
    assert list(O.select_tokens(n2[1:], p2[1:], 0.6)) == []
    # tau = 0: every token that moved at all
    assert list(O.select_tokens(new, prev, 0.0)) == [j for j in range(10) if np.any(new[j] != prev[j])]
    with pytest.raises(ValueError):
        O.select_tokens(new, prev, -0.1)


def test_select_tokens_near_threshold():
    """Which decisions are fixed and which are ties.

    The decision compares two float32 sums of d_v squares.  A token whose
    exact margin |D2 - tau^2 P2| (exact arithmetic on the float32 inputs) is
    below the rounding bound of those sums, (d_v + 4) 2^-24 (D2 + tau^2 P2),
    may be decided either way by another summation order; every other token
    must be decided as the exact arithmetic decides it.
    """
    from fractions import Fraction
    rng = np.random.default_rng(17)
    T, d, tau = 48, 1536, 0.05
    prev = rng.standard_normal((T, d)).astype(np.float32)
    margins = np.concatenate([-np.logspace(-8, -1, T // 2), np.logspace(-8, -1, T // 2)])
    dirs = rng.standard_normal((T, d))
    dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
    pn = np.linalg.norm(prev.astype(np.float64), axis=1, keepdims=True)
    new = (prev + dirs * (tau * (1.0 + margins[:, None]) * pn)).astype(np.float32)
    got = set(int(j) for j in O.select_tokens(new, prev, tau))
    t2 = Fraction(np.float32(tau).item()) ** 2
    n_fixed = n_tie = 0
    for j in range(T):
        D2 = sum((Fraction(a.item()) - Fraction(b.item())) ** 2 for a, b in zip(new[j], prev[j]))
        P2 = sum(Fraction(b.item()) ** 2 for b in prev[j])
        margin = D2 - t2 * P2
        band = Fraction(d + 4, 2 ** 24) * (D2 + t2 * P2)
        if abs(margin) > band:
            n_fixed += 1
            assert (j in got) == (margin > 0), f"token {j} decided against exact arithmetic"
        else:
            n_tie += 1
    assert n_fixed >= T // 3 and n_tie >= T // 3   # both kinds occur in this input


def _reuse_setup(tv=7):
    w = pico_weights()
    P = O.Params(w)
    rng = np.random.default_rng(41)
    prev = rng.standard_normal((tv, PICO.d_video))
    kv_prev, h_prev = O.video_forward(P, PICO, prev)
    return P, rng, prev, kv_prev, h_prev


def test_selective_all_tokens_active_is_the_full_forward():
    P, rng, prev, _, _ = _reuse_setup()
    new = rng.standard_normal(prev.shape)
    garbage = [(rng.standard_normal(K.shape), rng.standard_normal(V.shape))
               for K, V in O.video_forward(P, PICO, prev)[0]]
    kv, active, hidden = O.video_forward_selective(P, PICO, new, prev, garbage, 0.1,
                                                   hidden_prev=rng.standard_normal(prev.shape))
    assert list(active) == list(range(prev.shape[0]))
    kv_full, h_full = O.video_forward(P, PICO, new)
    for (K, V), (Kf, Vf) in zip(kv, kv_full):
        assert np.allclose(K, Kf, rtol=0, atol=1e-12) and np.allclose(V, Vf, rtol=0, atol=1e-12)
    assert np.allclose(hidden, h_full, rtol=0, atol=1e-12)


def test_selective_unchanged_observation_keeps_the_cache():
    P, rng, prev, kv_prev, h_prev = _reuse_setup()
    kv, active, hidden = O.video_forward_selective(P, PICO, prev.copy(), prev, kv_prev, 0.05, hidden_prev=h_prev)
    assert active.size == 0
    for (K, V), (Kp, Vp) in zip(kv, kv_prev):
        assert np.array_equal(K, Kp) and np.array_equal(V, Vp)
    assert np.array_equal(hidden, h_prev)


def test_selective_equals_masked_full_forward():
    # the same update written without gathering: run every token through every
    # block, and after each projection put the stable tokens' cached K, V back;
    # stable rows never reach an active row except through those K, V
    P, rng, prev, kv_prev, h_prev = _reuse_setup()
    tau = 0.1
    factors = [0.01, 1.5, 0.02, 0.0, 2.0, 0.8, 0.03]
    new = _moved(prev, factors, rng)
    kv, active, hidden = O.video_forward_selective(P, PICO, new, prev, kv_prev, tau, hidden_prev=h_prev)
    assert list(active) == [1, 4, 5]
    stable = [j for j in range(prev.shape[0]) if j not in (1, 4, 5)]
    x = np.array(new, dtype=np.float64)
    c = O.t_conditioning(P, "v", 0.0, PICO)
    for i in range(PICO.n_blocks):
        mod = O.block_modulation(P, "v", i, c)
        q, k, v = O.project(P, "v", i, mod, x, PICO)
        k[:, stable] = kv_prev[i][0][:, stable]
        v[:, stable] = kv_prev[i][1][:, stable]
        assert np.allclose(kv[i][0], k, rtol=0, atol=1e-12) and np.allclose(kv[i][1], v, rtol=0, atol=1e-12)
        assert np.array_equal(kv[i][0][:, stable], kv_prev[i][0][:, stable])
        x = O.rest(P, "v", i, mod, x, O.attention(q, k, v), PICO)
    assert np.allclose(hidden[[1, 4, 5]], x[[1, 4, 5]], rtol=0, atol=1e-12)
    assert np.array_equal(hidden[stable], h_prev[stable])


def test_selective_rejects_the_block_variant():
    P, rng, prev, kv_prev, _ = _reuse_setup()
    variant = dataclasses.replace(PICO, qk_norm=True)
    with pytest.raises(ValueError):
        O.video_forward_selective(P, variant, prev, prev, kv_prev, 0.1)
