"""Host-only checks of the C ABI: the library loads, exports every symbol the
headers declare, and its validation and layout logic behave as documented.
No call here launches GPU work (every call returns before any enqueue)."""
import ctypes
import os
import re

import numpy as np
import pytest

from mot_diffusion_transformer_amd import binding as bd
from mot_diffusion_transformer_amd import workload as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from mot_diffusion_transformer_amd import build
        build.build(verbose=False)
    return bd.load()


def header_symbols():
    names = set()
    for h in ("wam.h", "wam_ops.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(wam_[a-z_0-9]+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported(lib):
    declared = header_symbols()
    assert len(declared) >= 17
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(bd.EXPORTS)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "wam.h"\n#include "wam_ops.h"\nint main(void){wam_config c; (void)c; return 0;}\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c",
                        str(src), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def cfg_for(m, **kw):
    c = bd.make_config(m, 1, 256, 32, 4)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("d_video", 100, -2), ("d_action", 0, -2), ("head_dim", 48, -2), ("n_heads", 0, -2),
    ("action_dim", 65, -2), ("max_steps", 65, -2), ("max_batch", 0, -2), ("dtype", 7, -3),
    ("t_freq_dim", 12, -2), ("n_blocks", 0, -2),
])
def test_config_validation(lib, field, value, code):
    c = cfg_for(wl.TINY, **{field: value})
    assert lib.wam_config_check(ctypes.byref(c)) == code
    assert lib.wam_last_error().decode()
    assert lib.wam_weights_bytes(ctypes.byref(c)) == 0


def test_bf16_rejects_head_dim_32(lib):
    m = wl.ModelShape(2, 128, 128, 4, 32, 14, dtype=wl.BF16)
    c = bd.make_config(m, 1, 64, 32)
    assert lib.wam_config_check(ctypes.byref(c)) == -2


@pytest.mark.parametrize("m", [wl.TINY, wl.SMALL, wl.FAST_WAM, wl.FAST_WAM_A30])
def test_layout_matches_workload_specs(lib, m):
    c = bd.make_config(m, 1, 16, 16)
    layout = bd.weight_layout(c)
    specs = dict(wl.weight_specs(m))
    assert {n for n, *_ in layout} == set(specs)
    es = 4 if m.dtype == wl.F32 else 2
    spans = []
    for name, rows, cols, off in layout:
        shp = specs[name]
        assert rows * cols == int(np.prod(shp)), name
        assert (rows, cols) == (shp if len(shp) == 2 else (1, shp[0])), name
        assert off % 256 == 0, name
        spans.append((off, off + rows * cols * es, name))
    spans.sort()
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb)
    total = lib.wam_weights_bytes(ctypes.byref(c))
    assert spans[-1][1] <= total and total % 256 == 0
    # adaLN matrices of all blocks are contiguous (one pass produces every block's modulation)
    off = {n: o for n, _, _, o in layout}
    for ex, d in (("v", m.d_video), ("a", m.d_action)):
        for i in range(1, m.n_blocks):
            assert off[f"{ex}.{i}.ada.w"] == off[f"{ex}.0.ada.w"] + i * 6 * d * d * es
            assert off[f"{ex}.{i}.ada.b"] == off[f"{ex}.0.ada.b"] + i * 6 * d * es
    assert off["a.fada.w"] == off["a.0.ada.w"] + m.n_blocks * 6 * m.d_action ** 2 * es
    assert off["a.fada.b"] == off["a.0.ada.b"] + m.n_blocks * 6 * m.d_action * es


def test_tensor_info_out_of_range(lib):
    c = bd.make_config(wl.TINY, 1, 16, 16)
    info = bd.WamTensorInfo()
    n = lib.wam_weights_tensor_count(ctypes.byref(c))
    assert lib.wam_weights_tensor_info(ctypes.byref(c), n, ctypes.byref(info)) == -2
    assert lib.wam_weights_tensor_info(ctypes.byref(c), -1, ctypes.byref(info)) == -2


def test_null_arguments_fail_before_any_gpu_work(lib):
    c = bd.make_config(wl.TINY, 1, 16, 16)
    out = ctypes.c_void_p()
    assert lib.wam_model_create(ctypes.byref(c), None, ctypes.byref(out)) == -1
    assert lib.wam_model_create(ctypes.byref(c), ctypes.c_void_p(0x1000), None) == -1
    assert lib.wam_model_create(ctypes.byref(c), ctypes.c_void_p(0x1010), ctypes.byref(out)) == -6
    assert lib.wam_model_destroy(None) == -1
    assert lib.wam_video_forward(None, None, 1, 1, 0.0, None, None, None, None) == -1
    assert lib.wam_action_step(None, None, 1, 1, 1, None, 1.0, 0.0, None, None, None, None, None) == -1
    assert lib.wam_action_step_noalloc(None, None, 1, 1, 1, None, 1.0, 0.0, None, None, None, None) == -1
    g = (ctypes.c_float * 2)(0.0, 1.0)
    assert lib.wam_infer_cewp(None, None, None, g, 1, 1, 1, 1, None, None, None, None, 1, None, None, None) == -1
    assert lib.wam_kv_cache_bytes(None, 1, 1) == 0
    assert lib.wam_workspace_bytes(None, 1, 1, 1, 1) == 0
    assert "NULL" in lib.wam_last_error().decode()


def test_op_validation(lib):
    assert lib.wam_op_gemm(5, 0, 1, 1, 64, None, None, None, None, 0, None, None, None) == -3
    assert lib.wam_op_gemm(1, 0, 1, 1, 60, None, None, None, None, 0, None, None, None) == -2
    assert lib.wam_op_gemm(1, 0, 4, 4, 64, None, None, None, None, 0, None, None, None) == -1
    assert lib.wam_op_gemm(1, 9, 4, 4, 64, None, None, None, None, 0, None, None, None) == -2
    assert lib.wam_op_gemm(1, 3, 4, 100, 64, None, None, None, None, 64, None, None, None) == -2
    assert lib.wam_op_attention(1, 1, 1, 32, 1, None, 1, None, None, 0, None, None, None, None, None) == -2
    assert lib.wam_op_attention(0, 1, 1, 32, 1, None, 0, None, None, 0, None, None, None, None, None) == -2
    assert lib.wam_op_ln_modulate(1, 4, 6, None, None, None, 1e-6, None, None) == -2
    assert lib.wam_op_gemm_ws_bytes(1, 32, 768, 3072) > 0       # weight-streaming split-K
    assert lib.wam_op_gemm_ws_bytes(1, 2048, 1024, 1536) == 0   # tiled MFMA path, K unsplit
    assert lib.wam_op_gemm_ws_bytes(1, 512, 768, 3072) >= 4 * 512 * 768 * 4  # tiled, K split in 4
    assert lib.wam_op_attention_ws_bytes(1, 1, 12, 128, 32, 32, 2048) > 0  # split keys


@pytest.mark.parametrize("B,H,dh,Tq,L0,L1", [(1, 1, 128, 8, 8, 8192), (1, 1, 64, 32, 0, 65536),
                                             (1, 2, 128, 1, 1, 20000), (1, 12, 128, 32, 32, 2048)])
def test_attention_split_plan_fits_the_merge(lib, B, H, dh, Tq, L0, L1):
    """The split workspace holds nsplit records of (dh + 4) floats per query;
    the merge reads one split's (m, l) per lane, so nsplit <= 64 for any key
    range (one head over thousands of key tiles included)."""
    n = lib.wam_op_attention_ws_bytes(1, B, H, dh, Tq, L0, L1)
    assert n > 0 and n % (B * H * Tq * (dh + 4) * 4) == 0
    assert 1 < n // (B * H * Tq * (dh + 4) * 4) <= 64


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(bd, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        bd.load(str(tmp_path / "libwam.so"))
