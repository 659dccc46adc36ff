"""Captured inference (wam_graph_*): every replay equals the eager call byte
for byte.  Between replays the program does its own eager work -- it
poisons the KV cache and the workspace with NaN -- so a replay that reused
stale results, or a graph that dropped a node, would show."""
import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from tests.parity_cases import SENS_BF16, SENS_STD

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case,mode", [("sens", 1), ("sens", 0), ("small", 1), ("fast_s10", 1)])
def test_graph_replays_equal_eager(case, mode):
    import torch

    from mot_diffusion_transformer_amd import binding as bd
    if case == "sens":
        m, B, Tv, Ta, S, std = SENS_BF16, 2, 200, 20, 3, SENS_STD
    elif case == "small":
        w = wl.WORKLOADS["small_bf16"]
        m, B, Tv, Ta, S, std = w.model, w.batch, w.t_video, w.t_action, 1, 0.02
    else:
        w = wl.WORKLOADS["fastwam_s10"]
        m, B, Tv, Ta, S, std = w.model, w.batch, w.t_video, w.t_action, 10, 0.02
    print(f"graph case {case} mode {mode}", flush=True)
    model = bd.Model(m, wl.make_weights(m, std=std), max_batch=B, max_video_tokens=Tv, max_action_tokens=Ta,
                     max_steps=S)
    vid = bd.to_device(wl.make_video(m, B, Tv), m.dtype == wl.BF16)
    a0 = torch.from_numpy(wl.make_noise(m, B, Ta)).cuda()
    grid = wl.t_grid(S)
    kv, ws = model.alloc_kv(B, Tv), model.alloc_ws(B, Tv, Ta, S)
    outs = [torch.empty_like(a0) for _ in range(3)]
    sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
    n_kv = model.kv_cache_bytes(B, Tv)

    def poison():
        kv.fill_(0xFF)
        ws.fill_(0xFF)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()

    poison()
    model.infer(vid, a0, grid, B, Tv, Ta, kv, *outs, mode=mode, ws=ws, s_video=sv, s_action=sa)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ref_kv = kv[:n_kv].clone()
    assert all(bool(torch.isfinite(r).all()) for r in ref)

    g = model.graph(vid, a0, grid, B, Tv, Ta, kv, *outs, mode=mode, ws=ws, s_video=sv, s_action=sa)
    for rep in range(3):
        poison()
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.launch(sa)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), r.view(torch.int32)), rep
        assert torch.equal(kv[:n_kv], ref_kv), rep
        del scratch
    g.close()
    model.close()


def test_graph_needs_streams():
    import torch

    from mot_diffusion_transformer_amd import binding as bd
    m = SENS_BF16
    model = bd.Model(m, wl.make_weights(m, std=SENS_STD), max_batch=1, max_video_tokens=64, max_action_tokens=16)
    vid = bd.to_device(wl.make_video(m, 1, 64), True)
    a0 = torch.from_numpy(wl.make_noise(m, 1, 16)).cuda()
    kv, ws = model.alloc_kv(1, 64), model.alloc_ws(1, 64, 16, 1)
    out = torch.empty_like(a0)
    with pytest.raises(bd.WamError) as e:
        model.lib.wam_graph_create  # noqa: B018
        bd._check(model.lib.wam_graph_create(model.handle, bd._ptr(vid), bd._ptr(a0),
                                             wl.t_grid(1).ctypes.data_as(bd.ctypes.c_void_p), 1, 1, 64, 16,
                                             bd._ptr(kv), bd._ptr(out), None, None, 1, bd._ptr(ws), None, None,
                                             bd.ctypes.byref(bd.ctypes.c_void_p())))
    assert e.value.code == -1
    torch.cuda.synchronize()
    model.close()
