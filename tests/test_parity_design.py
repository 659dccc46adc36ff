"""The parity cases can see the mistakes they are meant to catch.

On the CPU, with the oracle only: zeroing one branch of one block (the
video attention output of block 0, the action attention output of block 1,
the action MLP of the last block, the video MLP of the last block) or
dropping the video keys from the action attention must move a compared
output (final chunk, velocity, endpoint, KV cache, last video hidden state) of the sensitive models by
several times the parity tolerance.  If it did not, a GPU path with that
branch missing could pass.
"""
import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O
from tests.parity_cases import SENS_BF16, SENS_BF16_SIZES, SENS_F32, SENS_F32_SIZES, SENS_STD, TOL, rel


def _run(m, w, sizes, S):
    video = wl.make_video(m, sizes["B"], sizes["Tv"]).astype(np.float64)
    noise = wl.make_noise(m, sizes["B"], sizes["Ta"]).astype(np.float64)
    return O.infer_batch(w, m, video, noise, wl.t_grid(S), keep_kv=True)


def _kv(r, i, j):
    return np.stack([r["kv"][b][i][j] for b in range(len(r["kv"]))])


@pytest.mark.parametrize("m,sizes", [(SENS_BF16, SENS_BF16_SIZES), (SENS_F32, SENS_F32_SIZES)])
def test_dropped_branches_move_outputs_beyond_tolerance(m, sizes):
    tol = TOL[m.dtype]
    w = wl.make_weights(m, std=SENS_STD)
    base = _run(m, w, sizes, 2)
    last = m.n_blocks - 1

    def delta(mut):
        w2 = dict(w)
        for name in mut:
            w2[name] = np.zeros_like(w[name])
        r = _run(m, w2, sizes, 2)
        d = {"v": rel(r["v"][-1], base["v"][-1]), "a_out": rel(r["a_out"], base["a_out"])}
        d["kv"] = max(rel(_kv(r, i, j), _kv(base, i, j)) for i in range(m.n_blocks) for j in (0, 1))
        d["x_video"] = rel(r["x_video"], base["x_video"])
        return max(d.values())

    assert delta(["v.0.o.w", "v.0.o.b"]) > 4 * tol           # video attention branch, block 0
    # the last video block's MLP reaches only the last hidden state (compared by the call-chain test)
    assert delta([f"v.{last}.fc2.w", f"v.{last}.fc2.b"]) > 4 * tol
    assert delta(["a.1.o.w", "a.1.o.b"]) > 4 * tol           # action attention branch, block 1
    assert delta([f"a.{last}.fc2.w", f"a.{last}.fc2.b"]) > 4 * tol  # action MLP, last block


def test_dropping_video_keys_is_visible():
    m, sizes = SENS_BF16, SENS_BF16_SIZES
    w = wl.make_weights(m, std=SENS_STD)
    P = O.Params(w, "a.")
    video = wl.make_video(m, 1, sizes["Tv"]).astype(np.float64)[0]
    a = wl.make_noise(m, 1, sizes["Ta"]).astype(np.float64)[0]
    kv, _ = O.video_forward(P, m, video)
    v = O.action_velocity(P, m, kv, a, 1.0)
    empty = [(k[:, :0], vv[:, :0]) for k, vv in kv]
    v_no_video = O.action_velocity(P, m, empty, a, 1.0)
    assert rel(v_no_video, v) > 4 * TOL[m.dtype]


def test_qk_norm_rope_variant_parts_are_visible():
    # the block variant on the sensitive bf16 shape (200 video tokens = 10 frames of 5 x 4)
    import dataclasses
    m = dataclasses.replace(SENS_BF16, qk_norm=True, rope_hw=(5, 4))
    tol, sizes = TOL[m.dtype], SENS_BF16_SIZES
    w = wl.make_weights(m, std=SENS_STD)
    base = _run(m, w, sizes, 2)

    def delta(r):
        d = [rel(r["v"][-1], base["v"][-1]), rel(r["a_out"], base["a_out"]), rel(r["x_video"], base["x_video"])]
        d.append(max(rel(_kv(r, i, j), _kv(base, i, j)) for i in range(m.n_blocks) for j in (0, 1)))
        return max(d)

    no_rope = delta(_run(dataclasses.replace(m, rope_hw=()), w, sizes, 2))
    no_norm = delta(_run(dataclasses.replace(m, qk_norm=False), {k: v for k, v in w.items() if not wl.is_gain(k)},
                         sizes, 2))
    w1 = {k: (np.ones_like(v) if wl.is_gain(k) else v) for k, v in w.items()}
    unit_gains = delta(_run(m, w1, sizes, 2))
    print("no_rope", no_rope, "no_norm", no_norm, "unit_gains", unit_gains)
    assert no_rope > 4 * tol and no_norm > 4 * tol and unit_gains > 4 * tol
