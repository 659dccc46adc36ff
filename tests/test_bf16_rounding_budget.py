"""How far bfloat16 rounding alone moves the outputs (CPU).

tests/bf16_emulation.py renders the forward pass in float32 with a bf16
rounding exactly where the bf16 HIP path stores bf16 values.  Against the
float64 oracle it gives the error budget of rounding alone, which fixes two
choices of the GPU parity tests:

  * the "sensitive" models use weights of std 0.06: there, rounding alone
    stays under half the 2e-2 tolerance on every compared output (the KV
    cache after the one storage rounding of each element is removed);
  * at std 0.1 the same models exceed the tolerance by rounding alone.  The
    bf16 HIP path, measured on MI355X at std 0.1 on the sensitive bf16 model
    (B = 2, 200 video / 20 action tokens, S = 3), showed max|err|/RMS of
    0.036-0.041 on the KV cache and 0.0436 on the last video hidden state;
    the emulation predicts the same sizes, so those errors were rounding,
    not a defect.
"""
import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O
from tests import bf16_emulation as E
from tests.parity_cases import SENS_BF16, SENS_BF16_SIZES, SENS_STD, TOL, rel, rel_stored_bf16

MEASURED_STD01 = {"kv": (0.036, 0.041), "x_video": 0.0436}


def _errors(std, S=3):
    m = SENS_BF16
    B, Tv, Ta = SENS_BF16_SIZES["B"], SENS_BF16_SIZES["Tv"], SENS_BF16_SIZES["Ta"]
    w = wl.make_weights(m, std=std)
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    out = {k: 0.0 for k in ("a_out", "v", "f", "x_video", "kv", "kv_stored")}
    for b in range(B):
        r = O.infer(w, m, video[b].astype(np.float64), noise[b].astype(np.float64), grid)
        e = E.infer(w, m, video[b], noise[b], grid)
        cur = {"a_out": rel(e["a_out"], r["a_out"]), "v": rel(e["v"][-1], r["v"][-1]),
               "f": rel(e["f"][-1], r["f"][-1]), "x_video": rel(e["x_video"], r["x_video"]),
               "kv": max(rel(e["kv"][i][j], r["kv"][i][j]) for i in range(m.n_blocks) for j in (0, 1)),
               "kv_stored": max(rel_stored_bf16(e["kv"][i][j], r["kv"][i][j])
                                for i in range(m.n_blocks) for j in (0, 1))}
        out = {k: max(out[k], cur[k]) for k in out}
    return out


def test_emulation_is_exact_for_float32_roundings():
    # sanity of the harness: with every weight zero but the output bias, the
    # velocity is b_out exactly and no rounding enters
    m = SENS_BF16
    w = {k: np.zeros_like(v) for k, v in wl.make_weights(m, std=SENS_STD).items()}
    w["a.out.b"] = wl.bf16_round(np.linspace(-1, 1, m.action_dim).astype(np.float32))
    noise = wl.make_noise(m, 1, 5)[0]
    e = E.infer(w, m, wl.make_video(m, 1, 16)[0], noise, wl.t_grid(1))
    assert np.array_equal(e["v"][0], np.broadcast_to(w["a.out.b"], e["v"][0].shape))


def test_sensitive_models_leave_headroom_under_the_tolerance():
    err = _errors(SENS_STD)
    tol = TOL[wl.BF16]
    for k in ("a_out", "v", "f", "x_video", "kv_stored"):
        assert err[k] <= 0.5 * tol, (k, err)


def test_std01_errors_of_the_gpu_path_are_rounding():
    err = _errors(0.1)
    tol = TOL[wl.BF16]
    # rounding alone exceeds the tolerance at std 0.1 ...
    assert err["x_video"] > tol and err["kv"] > tol
    # ... by the amounts the bf16 HIP path showed there (within a factor of 2)
    lo, hi = MEASURED_STD01["kv"]
    assert 0.5 * lo <= err["kv"] <= 2.0 * hi, err
    assert 0.5 * MEASURED_STD01["x_video"] <= err["x_video"] <= 2.0 * MEASURED_STD01["x_video"], err


@pytest.mark.parametrize("std", [0.02])
def test_plain_kv_comparison_would_sit_at_the_tolerance(std):
    # why the bf16-stored tensors subtract their one storage rounding: at the
    # workloads' std the plain comparison of the cache is already most of the
    # tolerance by that rounding alone
    err = _errors(std, S=1)
    assert err["kv"] > 0.5 * TOL[wl.BF16] and err["kv_stored"] < 0.5 * err["kv"]
