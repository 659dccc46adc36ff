"""Whole-path parity on the GPU, through the C ABI (wam_infer_cewp,
wam_video_forward, wam_action_step), against the CPU oracle.

Tolerance: max|err| <= tol * RMS(reference) per output tensor (the final
chunk, the last step's velocity and endpoint, every KV-cache block, the last
video hidden state), with tol = 1e-4 for float32 models and 2e-2 for
bfloat16 models; for the bf16 KV cache the elementwise bound of its one
storage rounding is removed first (tests/parity_cases.py).  The velocity
is checked on its own: the final chunk is dominated by the noise it starts
from and would hide errors in v.

Bit-identity: the wavefront (CEWP) schedule and the sequential schedule
run the same kernels, so their outputs must be equal byte for byte.  The
KV cache and the workspace are filled with NaN before every call, so a
read of a block before the video expert has written it (a missing or
misplaced event wait) poisons the outputs.
"""
import dataclasses
import os

import numpy as np
import pytest

from mot_diffusion_transformer_amd import workload as wl
from oracle import wam_oracle as O

pytestmark = pytest.mark.gpu

from tests.parity_cases import SENS_BF16, SENS_F32, SENS_STD, TOL, rel, rel_stored_bf16

# the QK-RMSNorm + 3-D RoPE block variant on the sensitive shapes: 200 video
# tokens = 10 frames of 5 x 4 patches, 77 = 7 frames of 1 x 11
SENS_BF16_QKNR = dataclasses.replace(SENS_BF16, qk_norm=True, rope_hw=(5, 4))
SENS_F32_QKNR = dataclasses.replace(SENS_F32, qk_norm=True, rope_hw=(1, 11))

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# The sensitive models span several tiles and leave ragged tails (200 video
# tokens vs 64/128-wide tiles, 20 action tokens vs 16-row MFMA tiles).


def torch_mod():
    import torch
    return torch


class GpuModel:
    def __init__(self, shape, weights, B, Tv, Ta, S):
        from mot_diffusion_transformer_amd import binding as bd
        self.bd = bd
        self.shape = shape
        self.model = bd.Model(shape, weights, max_batch=B, max_video_tokens=max(Tv, 1), max_action_tokens=Ta,
                              max_steps=max(S, 1))

    def inputs(self, video, noise):
        torch = torch_mod()
        bf = self.shape.dtype == wl.BF16
        vid = self.bd.to_device(video, bf) if video.size else torch.empty(16, dtype=torch.uint8, device="cuda")
        a0 = torch.from_numpy(np.ascontiguousarray(noise, np.float32)).cuda()
        return vid, a0

    def infer(self, video, noise, grid, mode):
        """Run wam_infer_cewp; outputs stay on the device (kv is the raw byte buffer).
        ``mode`` may carry the WAM_VIDEO_KV_ONLY_LAST flag."""
        torch = torch_mod()
        B, Tv, Ta = noise.shape[0], video.shape[1], noise.shape[1]
        S = len(grid) - 1
        vid, a0 = self.inputs(video, noise)
        kv = self.model.alloc_kv(B, Tv)
        ws = self.model.alloc_ws(B, Tv, Ta, S)
        kv.fill_(0xFF)  # NaN in float32 and bfloat16
        ws.fill_(0xFF)
        a_out = torch.empty_like(a0)
        v_last = torch.empty_like(a0)
        f_last = torch.empty_like(a0)
        sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        self.model.infer(vid, a0, grid, B, Tv, Ta, kv, a_out, v_last, f_last, mode=mode, ws=ws, s_video=sv,
                         s_action=sa)
        torch.cuda.synchronize()
        return {"a_out": a_out, "v_last": v_last, "f_last": f_last, "kv": kv, "B": B, "Tv": Tv}

    def host(self, out):
        """Outputs on the host; kv as [N][2][B][H][T_v][dh] (values transposed back)."""
        torch = torch_mod()
        h = {k: out[k].cpu().numpy() for k in ("a_out", "v_last", "f_last")}
        if out["Tv"] > 0:
            K, V = self.model.kv_split(out["kv"], out["B"], out["Tv"])
            h["kv"] = torch.stack([K, V], 1).float().cpu().numpy()
        return h

    def hidden_rows(self, video, B, Tv, b, tokens):
        """wam_video_forward with the hidden output: rows `tokens` of sample b's
        last hidden state [len(tokens)][d_video] (indexed on the host)."""
        torch = torch_mod()
        vid, _ = self.inputs(video, np.zeros((B, 1, self.shape.action_dim), np.float32))
        kv = self.model.alloc_kv(B, Tv)
        ws = self.model.alloc_ws(B, Tv, 1, 1)
        ws.fill_(0xFF)
        hidden = torch.full((B, Tv, self.shape.d_video), float("nan"), device="cuda")
        torch.cuda.synchronize()
        self.model.video_forward(vid, B, Tv, 0.0, kv, ws, hidden=hidden)
        torch.cuda.synchronize()
        return hidden[b].cpu().numpy()[np.asarray(tokens)]

    def kv_sample(self, out, blocks, b, tokens):
        """K and V of the given blocks, sample b, token rows `tokens`: [len(blocks)][H][len(tokens)][dh] each."""
        torch = torch_mod()
        blocks, tokens = np.asarray(blocks), np.asarray(tokens)
        # host-side bounds check before any indexing kernel runs
        assert 0 <= b < out["B"]
        assert blocks.min() >= 0 and blocks.max() < self.shape.n_blocks
        assert tokens.min() >= 0 and tokens.max() < out["Tv"]
        # whole contiguous slabs come to the host by plain copies; the rows are
        # picked there (no indexing kernel on the device)
        K, Vt = self.model.kv_slabs(out["kv"], out["B"], out["Tv"])
        Ks, Vs = [], []
        for i in blocks:
            Ks.append(K[int(i), b].cpu().float().numpy()[:, tokens])                      # [H][tokens][dh]
            Vs.append(Vt[int(i), b].cpu().float().numpy()[:, :, tokens].transpose(0, 2, 1))
        return np.stack(Ks), np.stack(Vs)


def oracle_run(shape, weights, video, noise, grid):
    return O.infer_batch(weights, shape, video.astype(np.float64), noise.astype(np.float64), grid, keep_kv=True)


def compare(g, r, tol, B, check_kv=True, samples=None, bf16=False):
    samples = list(range(B)) if samples is None else samples
    rel_kv = rel_stored_bf16 if bf16 else rel
    errs = {"a_out": rel(g["a_out"][samples], r["a_out"]), "v_last": rel(g["v_last"][samples], r["v"][-1]),
            "f_last": rel(g["f_last"][samples], r["f"][-1])}
    if check_kv:
        for i in range(len(r["kv"][0])):
            for which in (0, 1):
                ref = np.stack([r["kv"][si][i][which] for si in range(len(samples))])
                errs[f"kv{i}{'kv'[which]}"] = rel_kv(g["kv"][i, which][samples], ref)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"parity beyond {tol}: {bad}"
    return errs


def run_case(shape, B, Tv, Ta, S, std=0.02, mode=1, seed=0):
    print(f"case {shape} B={B} T_v={Tv} T_a={Ta} S={S} std={std}", flush=True)
    weights = wl.make_weights(shape, seed=seed, std=std)
    video = wl.make_video(shape, B, Tv) if Tv > 0 else np.zeros((B, 0, shape.d_video), np.float32)
    noise = wl.make_noise(shape, B, Ta)
    grid = wl.t_grid(S)
    gm = GpuModel(shape, weights, B, Tv, Ta, S)
    g = gm.host(gm.infer(video, noise, grid, mode))
    r = oracle_run(shape, weights, video, noise, grid)
    return compare(g, r, TOL[shape.dtype], B, check_kv=Tv > 0, bf16=shape.dtype == wl.BF16)


# ---------------------------------------------------------------- parity vs the oracle
def test_tiny_fp32_workload():
    w = wl.WORKLOADS["tiny_fp32"]
    print(run_case(w.model, w.batch, w.t_video, w.t_action, w.steps[0]))


@pytest.mark.parametrize("S", [1, 2])
def test_qk_norm_rope_variant_bf16(S):
    print(run_case(SENS_BF16_QKNR, 2, 200, 20, S, std=SENS_STD))


def test_qk_norm_rope_variant_fp32():
    print(run_case(SENS_F32_QKNR, 2, 77, 9, 2, std=SENS_STD))


@pytest.mark.parametrize("S", [1, 3])
def test_sensitive_bf16(S):
    print(run_case(SENS_BF16, 2, 200, 20, S, std=SENS_STD))


@pytest.mark.parametrize("S", [1, 2])
def test_sensitive_fp32(S):
    print(run_case(SENS_F32, 2, 77, 9, S, std=SENS_STD))


# Action experts wider than the workloads': the final layer holds 8 row
# elements and 32 weights per lane up to 2048 features and reads them from
# memory past that (where the LayerNorm also holds only the row).  At 768
# and 1536 features the fc2 GEMM splits K and its split reduction also
# writes the next block's first LayerNorm (768: 3 row chunks per lane, 1536:
# 6), with W_o unsplit and followed by its own LayerNorm kernel; two blocks
# so that a LayerNorm written by the previous block's reduction is read.
@pytest.mark.parametrize("shape,B,Tv,Ta", [(dataclasses.replace(SENS_BF16, n_blocks=1, d_action=1024), 1, 64, 20),
                                           (dataclasses.replace(SENS_F32, n_blocks=1, d_action=2304), 1, 40, 9),
                                           (dataclasses.replace(SENS_BF16, n_blocks=2, d_action=768), 2, 64, 20),
                                           (dataclasses.replace(SENS_BF16, n_blocks=2, d_action=1536), 1, 64, 32)])
def test_wide_action_expert(shape, B, Tv, Ta):
    print(run_case(shape, B, Tv, Ta, 2))


def test_small_bf16_workload():
    w = wl.WORKLOADS["small_bf16"]
    print(run_case(w.model, w.batch, w.t_video, w.t_action, w.steps[0]))


def test_no_video_tokens():
    # T_v = 0: the action expert attends over its own keys only
    m = SENS_BF16
    weights = wl.make_weights(m, std=SENS_STD)
    noise = wl.make_noise(m, 1, 20)
    grid = wl.t_grid(2)
    gm = GpuModel(m, weights, 1, 0, 20, 2)
    g = gm.host(gm.infer(np.zeros((1, 0, m.d_video), np.float32), noise, grid, 1))
    P = O.Params(weights, "a.")
    empty = [(np.zeros((m.n_heads, 0, m.head_dim)), np.zeros((m.n_heads, 0, m.head_dim)))] * m.n_blocks
    a = noise[0].astype(np.float64)
    for j in (2, 1):
        v = O.action_velocity(P, m, empty, a, grid[j])
        f = O.endpoint(a, v, grid[j])
        a = O.euler_step(a, v, grid[j], grid[j - 1])
    assert rel(g["v_last"][0], v) <= TOL[m.dtype]
    assert rel(g["f_last"][0], f) <= TOL[m.dtype]
    assert rel(g["a_out"][0], a) <= TOL[m.dtype]


def _golden(name, S):
    path = os.path.join(GOLDEN, f"{name}_S{S}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}; run tests/golden/make_golden.py {name}")
    return np.load(path)


_FAST_CACHE = {}


def fast_model(shape):
    """One resident model per Fast-WAM-scale shape, sized for every workload that uses it."""
    if shape not in _FAST_CACHE:
        _FAST_CACHE.clear()
        import gc
        gc.collect()
        uses = [w for w in wl.WORKLOADS.values() if w.model == shape and w.kind == "infer"]
        B = max(w.batch for w in uses)
        Tv = max(w.t_video for w in uses)
        Ta = max(w.t_action for w in uses)
        S = max(max(w.steps) for w in uses)
        print(f"generating weights for {shape}", flush=True)
        _FAST_CACHE[shape] = GpuModel(shape, wl.make_weights(shape), B, Tv, Ta, S)
    return _FAST_CACHE[shape]


@pytest.mark.parametrize("name,S", [("fastwam_s1", 1), ("fastwam_s10", 10), ("fastwam_b8", 1), ("fastwam_b8", 2),
                                    ("fastwam_qknr_s1", 1)])
def test_fastwam_against_stored_oracle(name, S):
    w = wl.WORKLOADS[name]
    m = w.model
    gold = _golden(name, S)
    gm = fast_model(m)
    print(f"{name} S={S}: generating inputs", flush=True)
    video = wl.make_video(m, w.batch, w.t_video)
    noise = wl.make_noise(m, w.batch, w.t_action)
    out = gm.infer(video, noise, wl.t_grid(S), 1)
    g = {k: out[k].cpu().numpy() for k in ("a_out", "v_last", "f_last")}
    tol = TOL[m.dtype]
    errs = {}
    toks, blks = gold["kv_tokens"], gold["kv_blocks"]
    for b in gold["samples"]:
        errs[f"a_out{b}"] = rel(g["a_out"][b], gold[f"a_out_{b}"])
        errs[f"v_last{b}"] = rel(g["v_last"][b], gold[f"v_last_{b}"])
        errs[f"f_last{b}"] = rel(g["f_last"][b], gold[f"f_last_{b}"])
        K, V = gm.kv_sample(out, blks, int(b), toks)
        errs[f"K{b}"] = rel_stored_bf16(K, gold[f"k_{b}"])
        errs[f"V{b}"] = rel_stored_bf16(V, gold[f"v_{b}"])
    del out
    if S == w.steps[0]:
        # the last video hidden state (float32 output of wam_video_forward) at the stored rows
        for b in gold["samples"]:
            print(f"{name}: video hidden state, sample {b}", flush=True)
            errs[f"x_video{b}"] = rel(gm.hidden_rows(video, w.batch, w.t_video, int(b), toks), gold[f"x_video_{b}"])
    print(errs)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, bad


def test_fastwam_graph_against_stored_oracle():
    """The captured wavefront inference (wam_graph_create / wam_graph_launch,
    the path the headline is timed on) against the stored oracle values, on
    three replays with the cache, workspace and outputs poisoned in between."""
    torch = torch_mod()
    name = "fastwam_s1"
    w = wl.WORKLOADS[name]
    m, B, Tv, Ta = w.model, w.batch, w.t_video, w.t_action
    gold = _golden(name, 1)
    gm = fast_model(m)
    print(f"{name}: graph replays against the stored oracle", flush=True)
    video, noise = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta)
    vid, a0 = gm.inputs(video, noise)
    kv, ws = gm.model.alloc_kv(B, Tv), gm.model.alloc_ws(B, Tv, Ta, 1)
    outs = [torch.empty_like(a0) for _ in range(3)]
    sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
    g = gm.model.graph(vid, a0, wl.t_grid(1), B, Tv, Ta, kv, *outs, mode=1, ws=ws, s_video=sv, s_action=sa)
    toks, blks = gold["kv_tokens"], gold["kv_blocks"]
    tol = TOL[m.dtype]
    first = None
    for rep in range(3):
        kv.fill_(0xFF)
        ws.fill_(0xFF)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch(sa)
        torch.cuda.synchronize()
        got = [o.cpu().numpy() for o in outs]
        errs = {"a_out": rel(got[0][0], gold["a_out_0"]), "v_last": rel(got[1][0], gold["v_last_0"]),
                "f_last": rel(got[2][0], gold["f_last_0"])}
        K, V = gm.kv_sample({"kv": kv, "B": B, "Tv": Tv}, blks, 0, toks)
        errs["K"] = rel_stored_bf16(K, gold["k_0"])
        errs["V"] = rel_stored_bf16(V, gold["v_0"])
        print(rep, errs, flush=True)
        assert all(e <= tol for e in errs.values()), (rep, errs)
        if first is None:
            first = [x.copy() for x in got]
        for x, y in zip(got, first):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), rep
    g.close()


@pytest.mark.parametrize("case,S", [("sens_bf16", 3), ("fastwam_s1", 1), ("fastwam_b8", 2)])
def test_writes_stay_inside_caller_buffers(case, S):
    """Every kernel of an inference writes only inside the buffers it was
    given: the KV cache, the workspace and the outputs sit inside larger
    allocations whose 1 MiB head and tail guards hold a pattern that must be
    intact afterwards (wavefront and sequential schedules)."""
    torch = torch_mod()
    if case == "sens_bf16":
        m, B, Tv, Ta = SENS_BF16, 2, 200, 20
        gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, S)
    else:
        w = wl.WORKLOADS[case]
        m, B, Tv, Ta = w.model, w.batch, w.t_video, w.t_action
        gm = fast_model(m)
    print(f"guard case {case} S={S}", flush=True)
    G = 1 << 20
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    vid, a0 = gm.inputs(video, noise)
    sizes = {"kv": gm.model.kv_cache_bytes(B, Tv), "ws": gm.model.workspace_bytes(B, Tv, Ta, S)}
    for k in ("a_out", "v_last", "f_last"):
        sizes[k] = a0.numel() * 4
    raw = {k: torch.empty(n + 2 * G, dtype=torch.uint8, device="cuda") for k, n in sizes.items()}
    inner = {k: raw[k][G:G + n] for k, n in sizes.items()}
    sv, sa = torch.cuda.Stream(), torch.cuda.Stream()
    for mode in (1, 0):
        for k, r in raw.items():
            r.fill_(0xA5)
            inner[k].fill_(0xFF)
        torch.cuda.synchronize()
        gm.model.infer(vid, a0, grid, B, Tv, Ta, inner["kv"], inner["a_out"].view(torch.float32),
                       inner["v_last"].view(torch.float32), inner["f_last"].view(torch.float32), mode=mode,
                       ws=inner["ws"], s_video=sv, s_action=sa)
        torch.cuda.synchronize()
        for k, r in raw.items():
            n = sizes[k]
            head, tail = r[:G].cpu().numpy(), r[G + n:].cpu().numpy()
            assert np.all(head == 0xA5) and np.all(tail == 0xA5), (case, mode, k)
        assert bool(torch.isfinite(inner["a_out"].view(torch.float32)).all())


# ---------------------------------------------------------------- schedule equivalence
@pytest.mark.parametrize("case,S", [("sens_bf16", 2), ("fastwam_s1", 1)])
def test_last_block_kv_only_flag_changes_nothing(case, S):
    """WAM_VIDEO_KV_ONLY_LAST (off by default) stops the last video block after
    its K, V: the outputs and the whole cache are identical to the bit."""
    from mot_diffusion_transformer_amd import binding as bd
    torch = torch_mod()
    if case == "sens_bf16":
        m, B, Tv, Ta = SENS_BF16, 2, 200, 20
        gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, S)
    else:
        w = wl.WORKLOADS[case]
        m, B, Tv, Ta = w.model, w.batch, w.t_video, w.t_action
        gm = fast_model(m)
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    full = gm.infer(video, noise, grid, bd.WAM_CEWP)
    n = gm.model.kv_cache_bytes(B, Tv)
    for mode in (bd.WAM_CEWP | bd.WAM_VIDEO_KV_ONLY_LAST, bd.WAM_SEQUENTIAL | bd.WAM_VIDEO_KV_ONLY_LAST):
        cut = gm.infer(video, noise, grid, mode)
        for k in ("a_out", "v_last", "f_last"):
            assert torch.equal(full[k].view(torch.int32), cut[k].view(torch.int32)), (mode, k)
        assert torch.equal(full["kv"][:n], cut["kv"][:n]), mode
    with pytest.raises(bd.WamError) as e:
        gm.infer(video, noise, grid, 2)
    assert e.value.code == -2


@pytest.mark.parametrize("case", ["tiny", "sens_bf16", "sens_qknr", "small", "fastwam_s10", "fastwam_b8_s1",
                                  "fastwam_b8_s2"])
def test_wavefront_equals_sequential_bitwise(case):
    if case == "sens_qknr":
        m, B, Tv, Ta, S = SENS_BF16_QKNR, 2, 200, 20, 2
        gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, S)
    elif case == "tiny":
        w = wl.WORKLOADS["tiny_fp32"]
        m, B, Tv, Ta, S, std = w.model, 1, w.t_video, w.t_action, 2, 0.02
        gm = GpuModel(m, wl.make_weights(m, std=std), B, Tv, Ta, S)
    elif case == "sens_bf16":
        m, B, Tv, Ta, S = SENS_BF16, 2, 200, 20, 3
        gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, S)
    elif case == "small":
        w = wl.WORKLOADS["small_bf16"]
        m, B, Tv, Ta, S = w.model, w.batch, w.t_video, w.t_action, 1
        gm = GpuModel(m, wl.make_weights(m), B, Tv, Ta, S)
    elif case.startswith("fastwam_b8"):
        # batch 8: the only shape whose action expert (512 rows) runs the tiled
        # split-K GEMMs, here concurrently with the video stream
        w = wl.WORKLOADS["fastwam_b8"]
        m, B, Tv, Ta, S = w.model, w.batch, w.t_video, w.t_action, int(case[-1])
        gm = fast_model(m)
    else:
        w = wl.WORKLOADS["fastwam_s10"]
        m, B, Tv, Ta, S = w.model, w.batch, w.t_video, w.t_action, 10
        gm = fast_model(m)
    print(f"bitwise case {case} S={S}", flush=True)
    torch = torch_mod()
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    seq = gm.infer(video, noise, grid, 0)
    for rep in range(2):
        cewp = gm.infer(video, noise, grid, 1)
        for k in ("a_out", "v_last", "f_last"):
            assert torch.equal(seq[k].view(torch.int32), cewp[k].view(torch.int32)), (case, rep, k)
        n = gm.model.kv_cache_bytes(B, Tv)
        assert torch.equal(seq["kv"][:n], cewp["kv"][:n]), (case, rep, "kv")
    assert bool(torch.isfinite(seq["a_out"]).all()) and bool(torch.isfinite(seq["v_last"]).all())


@pytest.mark.parametrize("hook", ["WAM_DEBUG_VIDEO_DELAY_US", "WAM_DEBUG_ACTION_DELAY_US"])
def test_injected_delays_change_nothing(hook):
    """A late producer (every video block first waits 300 us) or a late
    consumer (every action block waits 300 us after its event) leaves the
    outputs and the cache unchanged to the bit, in both schedules; the wait
    shows in the time of the call, so the hook did run."""
    import time
    torch = torch_mod()
    m, B, Tv, Ta, S = SENS_BF16, 2, 200, 20, 2
    weights = wl.make_weights(m, std=SENS_STD)
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    ref = GpuModel(m, weights, B, Tv, Ta, S).infer(video, noise, grid, 1)
    os.environ[hook] = "300"
    try:
        gm = GpuModel(m, weights, B, Tv, Ta, S)  # the hooks are read when the model is created
    finally:
        del os.environ[hook]
    print(f"{hook}=300: CEWP and sequential against the undelayed run", flush=True)
    n = gm.model.kv_cache_bytes(B, Tv)
    for mode in (1, 0):
        t0 = time.perf_counter()
        out = gm.infer(video, noise, grid, mode)
        elapsed = time.perf_counter() - t0
        for k in ("a_out", "v_last", "f_last"):
            assert torch.equal(ref[k].view(torch.int32), out[k].view(torch.int32)), (hook, mode, k)
        assert torch.equal(ref["kv"][:n], out["kv"][:n]), (hook, mode, "kv")
        # the video blocks run once, the action blocks once per step
        waits = m.n_blocks * (1 if hook == "WAM_DEBUG_VIDEO_DELAY_US" else S)
        assert elapsed >= 0.9 * waits * 300e-6, (hook, mode, elapsed)


def test_call_chain_equals_infer_bitwise():
    """video_forward + S x action_step reproduces wam_infer_cewp exactly."""
    torch = torch_mod()
    m, B, Tv, Ta, S = SENS_BF16, 2, 200, 20, 3
    gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, S)
    video, noise, grid = wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(S)
    ref = gm.infer(video, noise, grid, 1)
    vid, a = gm.inputs(video, noise)
    kv = gm.model.alloc_kv(B, Tv)
    ws = gm.model.alloc_ws(B, Tv, Ta, 1)
    hidden = torch.empty(B, Tv, m.d_video, device="cuda")
    gm.model.video_forward(vid, B, Tv, 0.0, kv, ws, hidden=hidden)
    v = torch.empty_like(a)
    f = torch.empty_like(a)
    for j in range(S, 0, -1):
        gm.model.action_step(kv, B, Tv, Ta, a, grid[j], grid[j - 1], a, v=v, f=f, ws=ws)
    torch.cuda.synchronize()
    n = gm.model.kv_cache_bytes(B, Tv)
    assert torch.equal(kv[:n], ref["kv"][:n])
    # without a hidden output the cache is the same to the bit
    kv2 = gm.model.alloc_kv(B, Tv)
    kv2.fill_(0xFF)
    gm.model.video_forward(vid, B, Tv, 0.0, kv2, ws)
    torch.cuda.synchronize()
    assert torch.equal(kv2[:n], kv[:n])
    for got, k in ((a, "a_out"), (v, "v_last"), (f, "f_last")):
        assert torch.equal(got.view(torch.int32), ref[k].view(torch.int32)), k
    # last video hidden state against the oracle
    r = O.infer_batch(wl.make_weights(m, std=SENS_STD), m, video.astype(np.float64), noise.astype(np.float64),
                      grid)
    assert rel(hidden.cpu().numpy(), r["x_video"]) <= TOL[m.dtype]


def test_one_step_endpoint_identity_on_gpu():
    """S = 1: the final chunk equals the endpoint f(a_1, 1), bit for bit (same fused multiply-add)."""
    m, B, Tv, Ta = SENS_BF16, 1, 64, 16
    gm = GpuModel(m, wl.make_weights(m, std=SENS_STD), B, Tv, Ta, 1)
    g = gm.host(gm.infer(wl.make_video(m, B, Tv), wl.make_noise(m, B, Ta), wl.t_grid(1), 1))
    assert np.array_equal(g["a_out"].view(np.uint32), g["f_last"].view(np.uint32))


def test_errors_with_a_live_model():
    from mot_diffusion_transformer_amd import binding as bd
    torch = torch_mod()
    m = SENS_F32
    gm = GpuModel(m, wl.make_weights(m), 1, 32, 8, 2)
    vid, a = gm.inputs(wl.make_video(m, 1, 32), wl.make_noise(m, 1, 8))
    kv, ws = gm.model.alloc_kv(1, 32), gm.model.alloc_ws(1, 32, 8, 2)
    out = torch.empty_like(a)
    cases = [
        (dict(t_grid=np.array([0.0, 0.5, 0.5], np.float32)), -4),
        (dict(t_grid=np.array([0.0, 1.5], np.float32)), -4),
        (dict(t_grid=np.array([0.0, 0.2, 0.4, 0.6], np.float32)), -2),  # S = 3 > max_steps
        (dict(B=2), -2),
        (dict(T_v=33), -2),
    ]
    for kw, code in cases:
        args = dict(t_grid=wl.t_grid(1), B=1, T_v=32)
        args.update(kw)
        with pytest.raises(bd.WamError) as e:
            gm.model.infer(vid, a, args["t_grid"], args["B"], args["T_v"], 8, kv, out, ws=ws)
        assert e.value.code == code, (kw, e.value)
    with pytest.raises(bd.WamError) as e:
        gm.model.action_step(kv, 1, 32, 8, a, 0.3, 0.5, out, ws=ws)
    assert e.value.code == -4
    torch.cuda.synchronize()
