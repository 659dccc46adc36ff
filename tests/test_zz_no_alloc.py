"""wam_action_step_noalloc: the action step without a workspace argument, on
the library's fixed per-GPU scratch.  Its output must equal wam_action_step's
(same kernels, same launch shapes) to the bit, on two calls in a row, the
second with smaller sizes; sizes needing more scratch than the limit are
refused before anything runs."""
import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from tests.parity_cases import SENS_BF16, SENS_F32, SENS_STD

pytestmark = pytest.mark.gpu


def _step(model, kv, B, Tv, Ta, a, noalloc, ws=None):
    import torch
    a_next, v, f = (torch.full_like(a, float("nan")) for _ in range(3))
    if noalloc:
        model.action_step_noalloc(kv, B, Tv, Ta, a, 0.7, 0.2, a_next, v=v, f=f)
    else:
        model.action_step(kv, B, Tv, Ta, a, 0.7, 0.2, a_next, v=v, f=f, ws=ws)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (a_next, v, f)]


@pytest.mark.parametrize("shape,sizes", [
    (SENS_BF16, [(2, 200, 20), (1, 77, 9)]),
    (SENS_F32, [(2, 77, 9), (1, 30, 5)]),
    (wl.FAST_WAM, [(1, 2048, 32), (1, 1000, 16)]),
])
def test_noalloc_action_step_equals_action_step(shape, sizes):
    import torch

    from mot_diffusion_transformer_amd import binding as bd
    std = 0.02 if shape == wl.FAST_WAM else SENS_STD
    Bm, Tvm, Tam = (max(s[i] for s in sizes) for i in range(3))
    print(f"noalloc case {shape.d_video}/{shape.d_action} sizes {sizes}", flush=True)
    model = bd.Model(shape, wl.make_weights(shape, std=std), max_batch=Bm, max_video_tokens=Tvm,
                     max_action_tokens=Tam, max_steps=1)
    bf = shape.dtype == wl.BF16
    for B, Tv, Ta in sizes:
        vid = bd.to_device(wl.make_video(shape, B, Tv), bf)
        a = torch.from_numpy(wl.make_noise(shape, B, Ta)).cuda()
        kv, ws = model.alloc_kv(B, Tv), model.alloc_ws(B, Tv, Ta, 1)
        model.video_forward(vid, B, Tv, 0.0, kv, ws)
        torch.cuda.synchronize()
        ref = _step(model, kv, B, Tv, Ta, a, False, ws)
        got = _step(model, kv, B, Tv, Ta, a, True)
        for r, g in zip(ref, got):
            assert np.isfinite(r).all()
            assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), (B, Tv, Ta)
    model.close()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import torch

    from mot_diffusion_transformer_amd import binding as bd
    m = SENS_BF16
    # 256 x 64 action rows: the step's buffers alone exceed 32 MiB
    model = bd.Model(m, wl.make_weights(m, std=SENS_STD), max_batch=256, max_video_tokens=16, max_action_tokens=64,
                     max_steps=1)
    dummy = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(bd.WamError) as e:
        model.action_step_noalloc(dummy, 256, 16, 64, dummy, 0.7, 0.2, dummy)
    assert e.value.code == -2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    model.close()
