"""Teacher-anchored targets on the GPU (wam_teacher_targets) against the oracle.

For R rollouts of one observation (its batch-1 video KV cache from
wam_video_forward), the library computes a_t = (1 - t) a0 + t eps, the
teacher's K-step Euler rollout from t to 0, u = (a_t - a^T_0) / t and the
student's endpoint f = a_t - t v_student(a_t, t); the oracle's
teacher_targets_batch computes the same in float64 (pinned in
tests/test_oracle_pins.py).  Tolerance: max|err| <= tol * RMS(reference)
per output, tol = 2e-2 (bf16 models) or 1e-4 (fp32 models), as for the
inference (tests/parity_cases.py).
"""
import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O
from tests.parity_cases import SENS_BF16, SENS_F32, SENS_STD, TOL, rel

pytestmark = pytest.mark.gpu

# small t values included: u divides by t, so its error must shrink with the rollout
T_VALUES = [0.83, 0.21, 1.0, 0.47, 0.05]


def _run(m, Tv, Ta, ts, K, separate_student=True):
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    R = len(ts)
    print(f"targets {m} T_v={Tv} T_a={Ta} R={R} K={K} student={'own' if separate_student else 'teacher'}", flush=True)
    w_t = wl.make_weights(m, seed=0, std=SENS_STD)
    w_s = wl.make_weights(m, seed=3, std=SENS_STD) if separate_student else None
    video = wl.make_video(m, 1, Tv)
    rng = np.random.default_rng(77)
    a0 = rng.standard_normal((R, Ta, m.action_dim)).astype(np.float32)
    eps = rng.standard_normal((R, Ta, m.action_dim)).astype(np.float32)
    teacher = bd.Model(m, w_t, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    student = bd.Model(m, w_s, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1) if w_s else None
    kv = teacher.alloc_kv(1, Tv)
    kv.fill_(0xFF)  # NaN: a read of a block the video expert did not write poisons the outputs
    vws = teacher.alloc_ws(1, Tv, Ta, 1)
    teacher.video_forward(bd.to_device(video, m.dtype == wl.BF16), 1, Tv, 0.0, kv, vws)
    tws = torch.full((teacher.targets_workspace_bytes(R, Tv, Ta),), 0xFF, dtype=torch.uint8, device="cuda")
    d = lambda x: torch.from_numpy(x).cuda()
    a0d, epsd = d(a0), d(eps)
    u, f, a_t = (torch.empty_like(a0d) for _ in range(3))
    teacher.teacher_targets(kv, Tv, ts, a0d, epsd, K, u, f, a_t=a_t, ws=tws, student=student)
    torch.cuda.synchronize()
    got = {"u": u.cpu().numpy(), "f": f.cpu().numpy(), "a_t": a_t.cpu().numpy()}
    ref = O.teacher_targets_batch(w_t, w_s if w_s else w_t, m, video[0].astype(np.float64), a0.astype(np.float64),
                                  eps.astype(np.float64), ts, K)
    errs = {k: rel(got[k], ref[k]) for k in ("u", "f", "a_t")}
    for r, t in enumerate(ts):  # per rollout, small t included
        errs[f"u{r}(t={t})"] = rel(got["u"][r], ref["u"][r])
    print(errs)
    tol = TOL[m.dtype]
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, bad
    assert np.isfinite(got["u"]).all() and np.isfinite(got["f"]).all()
    teacher.close()
    if student:
        student.close()


@pytest.mark.parametrize("K", [1, 3])
def test_targets_bf16_against_oracle(K):
    _run(SENS_BF16, 200, 20, T_VALUES, K)


def test_targets_bf16_student_is_teacher():
    _run(SENS_BF16, 200, 20, T_VALUES[:3], 2, separate_student=False)


def test_targets_fp32_against_oracle():
    _run(SENS_F32, 77, 9, T_VALUES, 3)


def test_targets_argument_errors():
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    m = SENS_BF16
    w = wl.make_weights(m, std=SENS_STD)
    model = bd.Model(m, w, max_batch=4, max_video_tokens=64, max_action_tokens=16, max_steps=1)
    kv = model.alloc_kv(1, 64)
    ws = torch.empty(model.targets_workspace_bytes(4, 64, 16), dtype=torch.uint8, device="cuda")
    a = torch.zeros(4, 16, m.action_dim, device="cuda")
    u, f = torch.empty_like(a), torch.empty_like(a)
    for bad_t, code in (([0.5, 0.0, 0.3, 0.2], -4), ([0.5, 1.5, 0.3, 0.2], -4)):
        with pytest.raises(bd.WamError) as e:
            model.teacher_targets(kv, 64, bad_t, a, a, 3, u, f, ws=ws)
        assert e.value.code == code
    with pytest.raises(bd.WamError):  # K = 0
        model.teacher_targets(kv, 64, [0.5] * 4, a, a, 0, u, f, ws=ws)
    with pytest.raises(bd.WamError):  # R beyond max_batch
        model.targets_workspace_bytes(5, 64, 16)
    other = bd.Model(SENS_F32, wl.make_weights(SENS_F32, std=SENS_STD), max_batch=4, max_video_tokens=64,
                     max_action_tokens=16, max_steps=1)
    with pytest.raises(bd.WamError) as e:  # teacher and student shapes differ
        model.teacher_targets(kv, 64, [0.5] * 4, a, a, 3, u, f, ws=ws, student=other)
    assert e.value.code == -2
    other.close()
    model.close()


def test_fastwam_targets_against_stored_oracle():
    """The full-size target workload (Fast-WAM shape, one observation of 2048
    video tokens, 16 rollouts, K = 10) in the launch configuration the
    benchmark times; rollouts 0 and 15 against values the oracle stored
    (tests/golden/make_golden.py)."""
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    from tests.golden.make_golden import golden_path
    w = wl.WORKLOADS["fastwam_targets_k10"]
    m, R, Tv, Ta, K = w.model, w.batch, w.t_video, w.t_action, w.steps[0]
    gold = np.load(golden_path(w.name, K))
    print(f"{w.name}: generating weights and inputs", flush=True)
    weights = wl.make_weights(m)
    student_w = wl.make_student_weights(m, weights)
    ts = wl.target_times(R)
    assert np.array_equal(ts, gold["t"])
    teacher = bd.Model(m, weights, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    student = bd.Model(m, student_w, max_batch=R, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    del weights, student_w
    d = lambda x: torch.from_numpy(x).cuda()
    a0 = d(wl.make_clean_actions(m, R, Ta))
    eps = d(wl.make_noise(m, R, Ta))
    kv = teacher.alloc_kv(1, Tv)
    vws = teacher.alloc_ws(1, Tv, Ta, 1)
    tws = torch.empty(teacher.targets_workspace_bytes(R, Tv, Ta), dtype=torch.uint8, device="cuda")
    u, f, a_t = (torch.empty_like(a0) for _ in range(3))
    print(f"{w.name}: video forward (batch 1) + targets R={R} K={K}", flush=True)
    teacher.video_forward(bd.to_device(wl.make_video(m, 1, Tv), True), 1, Tv, 0.0, kv, vws)
    teacher.teacher_targets(kv, Tv, ts, a0, eps, K, u, f, a_t=a_t, ws=tws, student=student)
    torch.cuda.synchronize()
    got = {"u": u.cpu().numpy(), "f": f.cpu().numpy(), "a_t": a_t.cpu().numpy()}
    errs = {}
    for r in gold["rollouts"]:
        for k in ("u", "f", "a_t"):
            errs[f"{k}{r}"] = rel(got[k][r], gold[f"{k}_{r}"])
    print(errs)
    assert np.isfinite(got["u"]).all() and np.isfinite(got["f"]).all()
    bad = {k: v for k, v in errs.items() if not (v <= TOL[m.dtype])}
    assert not bad, bad
    teacher.close()
    student.close()


@pytest.mark.parametrize("R", [1, 64])
def test_targets_bf16_rollout_count_edges(R):
    # one rollout: the shared cache is that sample's own (no broadcast); 64: the
    # largest batch of time values one call takes (16 groups of the attention)
    ts = [0.37] if R == 1 else [float(x) for x in np.linspace(0.02, 1.0, R, dtype=np.float32)]
    _run(SENS_BF16, 200, 20, ts, 2)
