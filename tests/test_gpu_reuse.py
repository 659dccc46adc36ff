"""Selective reuse of the video cache across consecutive observations, on
the GPU (wam_select_tokens, wam_video_forward_reuse) against the oracle.

The first observation's cache comes from wam_video_forward; the reuse call
updates it for the second observation, recomputing only the tokens whose
input moved (select_tokens / video_forward_selective in the oracle, pinned
in tests/test_oracle_pins.py).  The active index list is integer output and
must match exactly: the inputs move every token either by >= 25x or by
<= 1/4 of the threshold, so no float32 rounding order can flip a decision.
Values: max|err| <= tol * RMS(reference), tol 2e-2 (bf16) / 1e-4 (fp32); K
and V, stored in bf16, after removing one bf16 rounding (tests/parity_cases.py).
"""
import dataclasses

import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O
from tests.parity_cases import SENS_BF16, SENS_F32, SENS_STD, TOL, rel, rel_stored_bf16

pytestmark = pytest.mark.gpu
TAU = wl.REUSE_TAU


def _dev(x, bf16):
    from mot_diffusion_transformer_amd import binding as bd
    return bd.to_device(x, bf16)


def _cache(model, kv, Tv):
    K, V = model.kv_split(kv, 1, Tv)
    return K[:, 0].float().cpu().numpy(), V[:, 0].float().cpu().numpy()  # [N][H][Tv][dh] each


def _run(m, Tv, Ta, changed, tau=TAU, same=False):
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    bf = m.dtype == wl.BF16
    print(f"reuse {m} T_v={Tv} changed={len(changed)} tau={tau} same={same}", flush=True)
    w = wl.make_weights(m, std=SENS_STD)
    prev = wl.make_video(m, 1, Tv)[0]
    new = prev.copy() if same else wl.make_next_observation(m, prev, changed)
    noise = wl.make_noise(m, 1, Ta)
    model = bd.Model(m, w, max_batch=1, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    kv, ws = model.alloc_kv(1, Tv), model.alloc_ws(1, Tv, Ta, 1)
    kv.fill_(0xFF)
    ws.fill_(0xFF)
    prev_d, new_d = _dev(prev, bf), _dev(new, bf)
    hidden = torch.empty(Tv, m.d_video, dtype=torch.float32, device="cuda")
    model.video_forward(prev_d, 1, Tv, 0.0, kv, ws, hidden=hidden)
    torch.cuda.synchronize()
    K0, V0 = _cache(model, kv, Tv)
    h0 = hidden.cpu().numpy()
    rws = torch.full((model.reuse_workspace_bytes(Tv),), 0xFF, dtype=torch.uint8, device="cuda")
    n = model.video_forward_reuse(new_d, prev_d, Tv, 0.0, tau, kv, rws, hidden=hidden)
    a0 = torch.from_numpy(noise).cuda()
    a_next, v, f = (torch.empty_like(a0) for _ in range(3))
    model.action_step(kv, 1, Tv, Ta, a0, 1.0, 0.0, a_next, v=v, f=f, ws=ws)
    torch.cuda.synchronize()
    K1, V1 = _cache(model, kv, Tv)
    h1 = hidden.cpu().numpy()
    got = dict(n=n, K0=K0, V0=V0, h0=h0, K=K1, V=V1, h=h1, v=v.cpu().numpy()[0])
    P = O.Params(w, "a.")
    kv_p, h_p = O.video_forward(P, m, prev.astype(np.float64), 0.0)
    kv_o, act, h_o = O.video_forward_selective(P, m, new, prev, kv_p, tau, hidden_prev=h_p)
    v_o = O.action_velocity(P, m, kv_o, noise[0].astype(np.float64), 1.0)
    ref = dict(act=act, K=np.stack([k for k, _ in kv_o]), V=np.stack([v_ for _, v_ in kv_o]), h=h_o, v=v_o)
    model.close()
    return got, ref


def _check(m, got, ref):
    tol = TOL[m.dtype]
    kv_rel = rel_stored_bf16 if m.dtype == wl.BF16 else rel
    errs = {"K": kv_rel(got["K"], ref["K"]), "V": kv_rel(got["V"], ref["V"]),
            "hidden": rel(got["h"], ref["h"]), "v": rel(got["v"], ref["v"])}
    print(got["n"], errs)
    assert got["n"] == ref["act"].size
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    assert not bad, bad


@pytest.mark.parametrize("changed", [
    list(range(3, 41)) + [77, 150, 199],   # a ragged block plus scattered tokens
    [123],                                 # one token
    list(range(0, 200, 3)),                # every third token
])
def test_reuse_bf16_against_oracle(changed):
    got, ref = _run(SENS_BF16, 200, 20, changed)
    assert list(ref["act"]) == sorted(changed)
    _check(SENS_BF16, got, ref)
    # stable tokens keep the first observation's K, V and hidden rows exactly
    stable = np.setdiff1d(np.arange(200), changed)
    assert np.array_equal(got["K"][:, :, stable], got["K0"][:, :, stable])
    assert np.array_equal(got["V"][:, :, stable], got["V0"][:, :, stable])
    assert np.array_equal(got["h"][stable], got["h0"][stable])


def test_reuse_fp32_against_oracle():
    got, ref = _run(SENS_F32, 77, 9, list(range(10, 30)) + [76])
    _check(SENS_F32, got, ref)


def test_reuse_unchanged_observation_keeps_the_cache():
    got, ref = _run(SENS_BF16, 200, 20, [], same=True)
    assert got["n"] == 0 and ref["act"].size == 0
    assert np.array_equal(got["K"], got["K0"]) and np.array_equal(got["V"], got["V0"])
    assert np.array_equal(got["h"], got["h0"])


def test_reuse_all_tokens_is_the_full_forward():
    # tau = 0: the sensor noise moves every token, so all are recomputed, and the
    # result is the ordinary forward of the new observation, bit for bit
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    m, Tv, Ta = SENS_BF16, 200, 20
    got, ref = _run(m, Tv, Ta, [5, 6], tau=0.0)
    assert got["n"] == Tv and ref["act"].size == Tv
    _check(m, got, ref)
    w = wl.make_weights(m, std=SENS_STD)
    prev = wl.make_video(m, 1, Tv)[0]
    new = wl.make_next_observation(m, prev, [5, 6])
    model = bd.Model(m, w, max_batch=1, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=1)
    kv, ws = model.alloc_kv(1, Tv), model.alloc_ws(1, Tv, Ta, 1)
    hidden = torch.empty(Tv, m.d_video, dtype=torch.float32, device="cuda")
    model.video_forward(_dev(new, True), 1, Tv, 0.0, kv, ws, hidden=hidden)
    torch.cuda.synchronize()
    K, V = _cache(model, kv, Tv)
    assert np.array_equal(K, got["K"]) and np.array_equal(V, got["V"])
    assert np.array_equal(hidden.cpu().numpy(), got["h"])
    model.close()


@pytest.mark.parametrize("Tv", [1100, 2048])
def test_select_tokens_exact(Tv):
    # several 1024-token chunks of the compaction, a ragged tail at 1100
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    m = wl.FAST_WAM if Tv == 2048 else SENS_BF16
    print(f"select {m.d_video} T_v={Tv}", flush=True)
    model = bd.Model(m, wl.make_weights(m, std=SENS_STD if m is SENS_BF16 else 0.02), max_batch=1,
                     max_video_tokens=Tv, max_action_tokens=16, max_steps=1)
    prev = wl.make_video(m, 1, Tv)[0]
    changed = wl.window_tokens(Tv) if Tv == 2048 else np.r_[0:7, 1000:1030, 1099]
    new = wl.make_next_observation(m, prev, changed)
    idx = torch.full((Tv,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    for tau, want in ((TAU, O.select_tokens(new, prev, TAU)), (0.0, np.arange(Tv)), (1e3, np.arange(0))):
        model.select_tokens(_dev(new, True), _dev(prev, True), Tv, tau, idx, cnt)
        torch.cuda.synchronize()
        c = int(cnt.cpu()[0])
        assert c == want.size
        assert np.array_equal(idx.cpu().numpy()[:c], want)
    assert np.array_equal(O.select_tokens(new, prev, TAU), np.sort(changed))
    model.close()


def test_reuse_argument_errors():
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    m, Tv = SENS_BF16, 64
    model = bd.Model(m, wl.make_weights(m, std=SENS_STD), max_batch=1, max_video_tokens=Tv, max_action_tokens=16,
                     max_steps=1)
    vid = _dev(wl.make_video(m, 1, Tv)[0], True)
    kv = model.alloc_kv(1, Tv)
    ws = torch.empty(model.reuse_workspace_bytes(Tv), dtype=torch.uint8, device="cuda")
    assert model.lib.wam_reuse_workspace_bytes(model.handle, Tv, 17, 1) == 0  # T_a beyond max_action_tokens
    for bad, code in ((dict(tau=-0.1), -4), (dict(tau=float("nan")), -4), (dict(T_v=Tv + 1), -2),
                      (dict(t_v=1.5), -4)):
        args = dict(tau=0.1, T_v=Tv, t_v=0.0)
        args.update(bad)
        with pytest.raises(bd.WamError) as e:
            model.video_forward_reuse(vid, vid, args["T_v"], args["t_v"], args["tau"], kv, ws)
        assert e.value.code == code
    vm = dataclasses.replace(SENS_BF16, qk_norm=True)
    variant = bd.Model(vm, wl.make_weights(vm, std=SENS_STD), max_batch=1, max_video_tokens=Tv,
                       max_action_tokens=16, max_steps=1)
    with pytest.raises(bd.WamError) as e:
        variant.video_forward_reuse(vid, vid, Tv, 0.0, 0.1, kv, ws)
    assert e.value.code == -2
    variant.close()
    model.close()


def _infer_reuse_case(m, Tv, Ta, changed, S, w=None, std=SENS_STD, tau=TAU):
    """First observation (wam_video_forward), then the reuse inference on the
    second in both schedules from copies of that cache."""
    import torch
    from mot_diffusion_transformer_amd import binding as bd
    bf = m.dtype == wl.BF16
    w = wl.make_weights(m, std=std) if w is None else w
    prev = wl.make_video(m, 1, Tv)[0]
    new = wl.make_next_observation(m, prev, changed)
    noise = wl.make_noise(m, 1, Ta)
    model = bd.Model(m, w, max_batch=1, max_video_tokens=Tv, max_action_tokens=Ta, max_steps=S)
    kv0, ws = model.alloc_kv(1, Tv), model.alloc_ws(1, Tv, Ta, 1)
    prev_d, new_d = _dev(prev, bf), _dev(new, bf)
    h0 = torch.empty(Tv, m.d_video, dtype=torch.float32, device="cuda")
    model.video_forward(prev_d, 1, Tv, 0.0, kv0, ws, hidden=h0)
    a0 = torch.from_numpy(noise).cuda()
    sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
    out = {}
    for mode in (bd.WAM_CEWP, bd.WAM_SEQUENTIAL):
        kv, hidden = kv0.clone(), h0.clone()
        rws = torch.full((model.reuse_workspace_bytes(Tv, Ta, S),), 0xFF, dtype=torch.uint8, device="cuda")
        a_out, v, f = (torch.full_like(a0, float("nan")) for _ in range(3))
        torch.cuda.synchronize()
        n = model.infer_reuse(new_d, prev_d, tau, a0, wl.t_grid(S), Tv, Ta, kv, a_out, hidden=hidden, v_last=v,
                              f_last=f, mode=mode, ws=rws, s_video=sv, s_action=sa)
        sa.synchronize()
        torch.cuda.synchronize()
        out[mode] = dict(n=n, kv=kv.cpu().numpy(), h=hidden.cpu().numpy(), a=a_out.cpu().numpy(),
                         v=v.cpu().numpy(), f=f.cpu().numpy())
    for k in ("kv", "h", "a", "v", "f"):
        assert np.array_equal(out[bd.WAM_CEWP][k], out[bd.WAM_SEQUENTIAL][k]), k
    assert out[bd.WAM_CEWP]["n"] == out[bd.WAM_SEQUENTIAL]["n"]
    # without a hidden output the last video block stops after its K, V
    # projection: the cache and the actions are the same to the bit
    kv = kv0.clone()
    rws = torch.full((model.reuse_workspace_bytes(Tv, Ta, S),), 0xFF, dtype=torch.uint8, device="cuda")
    a_out = torch.full_like(a0, float("nan"))
    torch.cuda.synchronize()
    n = model.infer_reuse(new_d, prev_d, tau, a0, wl.t_grid(S), Tv, Ta, kv, a_out, mode=bd.WAM_CEWP, ws=rws,
                          s_video=sv, s_action=sa)
    sa.synchronize()
    torch.cuda.synchronize()
    assert n == out[bd.WAM_CEWP]["n"]
    assert np.array_equal(kv.cpu().numpy(), out[bd.WAM_CEWP]["kv"])
    assert np.array_equal(a_out.cpu().numpy(), out[bd.WAM_CEWP]["a"])
    res = out[bd.WAM_CEWP]
    res.update(model=model, kv0=kv0, h0=h0, prev=prev, new=new, noise=noise, prev_d=prev_d, new_d=new_d, a0=a0, w=w)
    return res


@pytest.mark.parametrize("S", [1, 3])
def test_infer_reuse_schedules_agree_and_match_oracle(S):
    m, Tv, Ta = SENS_BF16, 200, 20
    changed = list(range(50, 90)) + [3, 199]
    print(f"infer_reuse S={S}", flush=True)
    r = _infer_reuse_case(m, Tv, Ta, changed, S)
    assert r["n"] == len(changed)
    P = O.Params(r["w"], "a.")
    kv_p, h_p = O.video_forward(P, m, r["prev"].astype(np.float64), 0.0)
    kv_o, act, h_o = O.video_forward_selective(P, m, r["new"], r["prev"], kv_p, TAU, hidden_prev=h_p)
    g = wl.t_grid(S).astype(np.float64)
    a = r["noise"][0].astype(np.float64)
    for j in range(S, 0, -1):
        vj = O.action_velocity(P, m, kv_o, a, g[j])
        f_o = O.endpoint(a, vj, g[j])
        a = O.euler_step(a, vj, g[j], g[j - 1])
    errs = {"a_out": rel(r["a"][0], a), "v_last": rel(r["v"][0], vj), "f_last": rel(r["f"][0], f_o),
            "hidden": rel(r["h"], h_o)}
    print(errs)
    bad = {k: e for k, e in errs.items() if not (e <= TOL[m.dtype])}
    assert not bad, bad
    if S == 1:
        # the two-call path (reuse, then one action step) is the same computation, bit for bit
        import torch
        model = r["model"]
        kv, hidden = r["kv0"].clone(), r["h0"].clone()
        rws = torch.empty(model.reuse_workspace_bytes(Tv), dtype=torch.uint8, device="cuda")
        ws = model.alloc_ws(1, Tv, Ta, 1)
        model.video_forward_reuse(r["new_d"], r["prev_d"], Tv, 0.0, TAU, kv, rws, hidden=hidden)
        a_next, v, f = (torch.empty_like(r["a0"]) for _ in range(3))
        model.action_step(kv, 1, Tv, Ta, r["a0"], 1.0, 0.0, a_next, v=v, f=f, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(kv.cpu().numpy(), r["kv"]) and np.array_equal(hidden.cpu().numpy(), r["h"])
        assert np.array_equal(a_next.cpu().numpy(), r["a"]) and np.array_equal(v.cpu().numpy(), r["v"])
        # no hidden output: the last block stops after its K, V; the same cache
        kv2 = r["kv0"].clone()
        model.video_forward_reuse(r["new_d"], r["prev_d"], Tv, 0.0, TAU, kv2, rws)
        torch.cuda.synchronize()
        assert np.array_equal(kv2.cpu().numpy(), r["kv"])
    r["model"].close()


def test_fastwam_reuse_against_stored_oracle():
    """The full-size reuse workload (2048 video tokens, 512 of them changed) as
    the benchmark runs it (wam_infer_reuse, wavefront schedule, S = 1; the
    sequential schedule must agree bit for bit), against values the oracle
    stored (tests/golden/make_golden.py)."""
    import torch
    from tests.golden.make_golden import golden_path
    w = wl.WORKLOADS["fastwam_reuse_s1"]
    m, Tv, Ta = w.model, w.t_video, w.t_action
    gold = np.load(golden_path(w.name, 1))
    assert float(gold["tau"]) == np.float32(TAU)
    print(f"{w.name}: weights, first observation, reuse inference in both schedules", flush=True)
    r = _infer_reuse_case(m, Tv, Ta, wl.window_tokens(Tv), 1, w=wl.make_weights(m), std=0.02)
    assert r["n"] == gold["active"].size
    toks, blks = gold["kv_tokens"], gold["kv_blocks"]
    kv = torch.from_numpy(r["kv"]).cuda()
    K, V = r["model"].kv_split(kv, 1, Tv)
    bi, ti = torch.as_tensor(blks, device="cuda"), torch.as_tensor(toks, device="cuda")
    Ks = K[:, 0].index_select(0, bi).index_select(2, ti).float().cpu().numpy()
    Vs = V[:, 0].index_select(0, bi).index_select(2, ti).float().cpu().numpy()
    errs = {"K": rel_stored_bf16(Ks, gold["k"]), "V": rel_stored_bf16(Vs, gold["v"]),
            "hidden": rel(r["h"][toks], gold["hidden"]), "v_last": rel(r["v"][0], gold["v_last"]),
            "a_out": rel(r["a"][0], gold["a_out"]), "f_last": rel(r["f"][0], gold["f_last"])}
    print(r["n"], errs)
    bad = {k: e for k, e in errs.items() if not (e <= TOL[m.dtype])}
    assert not bad, bad
    r["model"].close()


def test_reuse_odd_token_count():
    # 203 tokens: the transposed-value scatter and the attention's ragged last
    # key tile, with changed tokens at both ends
    changed = [0, 1, 202] + list(range(100, 140))
    got, ref = _run(SENS_BF16, 203, 20, changed)
    assert list(ref["act"]) == sorted(changed)
    _check(SENS_BF16, got, ref)
