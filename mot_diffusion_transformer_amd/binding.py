"""ctypes binding of libwam.so (include/wam.h, include/wam_ops.h).

Argument marshalling only: torch provides device memory and streams, every
step of the forward pass runs in the library's HIP kernels.  There is no
fallback: if the library is missing or the GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import workload as wl

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwam.so")

WAM_F32, WAM_BF16 = 0, 1
WAM_SEQUENTIAL, WAM_CEWP = 0, 1
WAM_VIDEO_KV_ONLY_LAST = 0x10  # mode flag: the last video block stops after its K, V (off by default)
STATUS = {0: "WAM_OK", -1: "WAM_ERR_NULL", -2: "WAM_ERR_SHAPE", -3: "WAM_ERR_DTYPE", -4: "WAM_ERR_GRID",
          -5: "WAM_ERR_HIP", -6: "WAM_ERR_ALIGN"}

EXPORTS = [
    "wam_config_check", "wam_weights_tensor_count", "wam_weights_bytes", "wam_weights_tensor_info",
    "wam_model_create", "wam_model_destroy", "wam_kv_cache_bytes", "wam_workspace_bytes",
    "wam_video_forward", "wam_action_step", "wam_action_step_noalloc", "wam_infer_cewp", "wam_last_error",
    "wam_graph_create", "wam_graph_launch", "wam_graph_destroy",
    "wam_targets_workspace_bytes", "wam_teacher_targets",
    "wam_reuse_workspace_bytes", "wam_select_tokens", "wam_video_forward_reuse", "wam_infer_reuse",
    "wam_op_gemm_ws_bytes", "wam_op_gemm", "wam_op_attention_ws_bytes", "wam_op_attention",
    "wam_op_ln_modulate", "wam_op_qk_norm_rope",
]


class WamConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_blocks", "d_video", "d_action", "n_heads", "head_dim", "mlp_ratio", "t_freq_dim",
        "action_dim", "max_batch", "max_video_tokens", "max_action_tokens", "max_steps", "dtype")] + [
        ("ln_eps", ctypes.c_float), ("qk_norm", ctypes.c_int), ("rope_height", ctypes.c_int),
        ("rope_width", ctypes.c_int)]


class WamTensorInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("rows", ctypes.c_int), ("cols", ctypes.c_int),
                ("offset_bytes", ctypes.c_size_t)]


class WamError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load libwam.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- HIP runtime first, from torch
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mot_diffusion_transformer_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(WamConfig)
    sig = {
        "wam_config_check": (I, [cfgp]),
        "wam_weights_tensor_count": (I, [cfgp]),
        "wam_weights_bytes": (Z, [cfgp]),
        "wam_weights_tensor_info": (I, [cfgp, I, ctypes.POINTER(WamTensorInfo)]),
        "wam_model_create": (I, [cfgp, P, ctypes.POINTER(P)]),
        "wam_model_destroy": (I, [P]),
        "wam_kv_cache_bytes": (Z, [P, I, I]),
        "wam_workspace_bytes": (Z, [P, I, I, I, I]),
        "wam_video_forward": (I, [P, P, I, I, F, P, P, P, P]),
        "wam_action_step": (I, [P, P, I, I, I, P, F, F, P, P, P, P, P]),
        "wam_action_step_noalloc": (I, [P, P, I, I, I, P, F, F, P, P, P, P]),
        "wam_infer_cewp": (I, [P, P, P, P, I, I, I, I, P, P, P, P, I, P, P, P]),
        "wam_last_error": (ctypes.c_char_p, []),
        "wam_graph_create": (I, [P, P, P, P, I, I, I, I, P, P, P, P, I, P, P, P, ctypes.POINTER(P)]),
        "wam_graph_launch": (I, [P, P]),
        "wam_graph_destroy": (I, [P]),
        "wam_targets_workspace_bytes": (Z, [P, I, I, I]),
        "wam_teacher_targets": (I, [P, P, P, I, I, I, P, P, P, I, P, P, P, P, P]),
        "wam_reuse_workspace_bytes": (Z, [P, I, I, I]),
        "wam_select_tokens": (I, [P, P, P, I, F, P, P, P]),
        "wam_video_forward_reuse": (I, [P, P, P, I, F, F, P, P, ctypes.POINTER(I), P, P]),
        "wam_infer_reuse": (I, [P, P, P, F, P, P, I, I, I, P, P, P, P, P, ctypes.POINTER(I), I, P, P, P]),
        "wam_op_gemm_ws_bytes": (Z, [I, I, I, I]),
        "wam_op_gemm": (I, [I, I, I, I, I, P, P, P, P, I, P, P, P]),
        "wam_op_attention_ws_bytes": (Z, [I, I, I, I, I, I, I]),
        "wam_op_attention": (I, [I, I, I, I, I, P, I, P, P, I, P, P, P, P, P]),
        "wam_op_ln_modulate": (I, [I, I, I, P, P, P, F, P, P]),
        "wam_op_qk_norm_rope": (I, [I, I, I, I, I, P, P, F, I, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise WamError(rc, _lib.wam_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_config(m: wl.ModelShape, max_batch: int, max_video_tokens: int, max_action_tokens: int,
                max_steps: int = 16) -> WamConfig:
    rh, rw = tuple(m.rope_hw) if m.rope_hw else (0, 0)
    return WamConfig(m.n_blocks, m.d_video, m.d_action, m.n_heads, m.head_dim, m.mlp_ratio, m.t_freq_dim,
                     m.action_dim, max_batch, max_video_tokens, max_action_tokens, max_steps,
                     WAM_BF16 if m.dtype == wl.BF16 else WAM_F32, m.ln_eps, int(m.qk_norm), rh, rw)


def weight_layout(cfg: WamConfig):
    """[(name, rows, cols, offset_bytes)] as the library packs them."""
    lib = load()
    n = lib.wam_weights_tensor_count(ctypes.byref(cfg))
    if n <= 0:
        _check(lib.wam_config_check(ctypes.byref(cfg)))
    out = []
    for i in range(n):
        info = WamTensorInfo()
        _check(lib.wam_weights_tensor_info(ctypes.byref(cfg), i, ctypes.byref(info)))
        out.append((info.name.decode(), info.rows, info.cols, info.offset_bytes))
    return out


def pack_weights(cfg: WamConfig, weights: dict, device="cuda"):
    """Copy the named float32 arrays into one packed device buffer (model dtype)."""
    import torch
    lib = load()
    total = lib.wam_weights_bytes(ctypes.byref(cfg))
    if total == 0:
        _check(lib.wam_config_check(ctypes.byref(cfg)))
    host = np.zeros(total, dtype=np.uint8)
    bf = cfg.dtype == WAM_BF16
    for name, rows, cols, off in weight_layout(cfg):
        a = np.asarray(weights[name], dtype=np.float32)
        if a.size != rows * cols:
            raise ValueError(f"{name}: expected {rows}x{cols}, got shape {a.shape}")
        raw = (wl.bf16_bits(a) if bf else a).reshape(-1).view(np.uint8)
        host[off:off + raw.size] = raw
    return torch.from_numpy(host).to(device)


def to_device(a: np.ndarray, bf16: bool, device="cuda"):
    """A float32 array as a device tensor in the model dtype (values must be bf16-exact for bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if bf16:
        bits = wl.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return t.to(device)


class Model:
    """A MoT world-action model resident on one GPU (weights packed once)."""

    def __init__(self, shape: wl.ModelShape, weights: dict, max_batch: int, max_video_tokens: int,
                 max_action_tokens: int, max_steps: int = 16, device="cuda"):
        import torch
        self.lib = load()
        self.shape = shape
        self.bf16 = shape.dtype == wl.BF16
        self.cfg = make_config(shape, max_batch, max_video_tokens, max_action_tokens, max_steps)
        self.device = torch.device(device)
        self.weights = pack_weights(self.cfg, weights, self.device)
        h = ctypes.c_void_p()
        _check(self.lib.wam_model_create(ctypes.byref(self.cfg), _ptr(self.weights), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _check(self.lib.wam_model_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # sizes --------------------------------------------------------------
    def kv_cache_bytes(self, B, T_v):
        return self.lib.wam_kv_cache_bytes(self.handle, B, T_v)

    def workspace_bytes(self, B, T_v, T_a, S=1):
        n = self.lib.wam_workspace_bytes(self.handle, B, T_v, T_a, S)
        if n == 0:
            raise WamError(-2, f"invalid sizes B={B} T_v={T_v} T_a={T_a} S={S}")
        return n

    def alloc_kv(self, B, T_v):
        import torch
        n = self.kv_cache_bytes(B, T_v)
        return torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)

    def alloc_ws(self, B, T_v, T_a, S=1):
        import torch
        return torch.empty(self.workspace_bytes(B, T_v, T_a, S), dtype=torch.uint8, device=self.device)

    def kv_split(self, kv, B, T_v):
        """Views (K, V) of the cache, both indexed [N][B][H][T_v][dh] (V is
        stored transposed, [N][B][H][dh][T_v]; the returned V is a transposed view)."""
        import torch
        m = self.shape
        dt = torch.bfloat16 if self.bf16 else torch.float32
        n = self.kv_cache_bytes(B, T_v)
        slabs = kv[:n].view(dt).view(m.n_blocks, 2, B * m.n_heads * T_v * m.head_dim)
        K = slabs[:, 0].view(m.n_blocks, B, m.n_heads, T_v, m.head_dim)
        V = slabs[:, 1].view(m.n_blocks, B, m.n_heads, m.head_dim, T_v).transpose(3, 4)
        return K, V

    def kv_slabs(self, kv, B, T_v):
        """Contiguous views (K, V^T) of the cache as stored: K [N][B][H][T_v][dh]
        and V^T [N][B][H][dh][T_v]."""
        import torch
        m = self.shape
        dt = torch.bfloat16 if self.bf16 else torch.float32
        n = self.kv_cache_bytes(B, T_v)
        slabs = kv[:n].view(dt).view(m.n_blocks, 2, B * m.n_heads * T_v * m.head_dim)
        return (slabs[:, 0].view(m.n_blocks, B, m.n_heads, T_v, m.head_dim),
                slabs[:, 1].view(m.n_blocks, B, m.n_heads, m.head_dim, T_v))

    # calls --------------------------------------------------------------
    def video_forward(self, video, B, T_v, t_v, kv, ws, hidden=None, stream=None):
        _check(self.lib.wam_video_forward(self.handle, _ptr(video), B, T_v, float(t_v), _ptr(kv), _ptr(hidden),
                                          _ptr(ws), _stream(stream)))

    def action_step(self, kv, B, T_v, T_a, a, t_cur, t_next, a_next, v=None, f=None, ws=None, stream=None):
        _check(self.lib.wam_action_step(self.handle, _ptr(kv), B, T_v, T_a, _ptr(a), float(t_cur), float(t_next),
                                        _ptr(a_next), _ptr(v), _ptr(f), _ptr(ws), _stream(stream)))

    def action_step_noalloc(self, kv, B, T_v, T_a, a, t_cur, t_next, a_next, v=None, f=None, stream=None):
        """wam_action_step without a workspace (the library's fixed per-GPU scratch)."""
        _check(self.lib.wam_action_step_noalloc(self.handle, _ptr(kv), B, T_v, T_a, _ptr(a), float(t_cur),
                                                float(t_next), _ptr(a_next), _ptr(v), _ptr(f), _stream(stream)))

    def targets_workspace_bytes(self, R, T_v, T_a):
        n = self.lib.wam_targets_workspace_bytes(self.handle, R, T_v, T_a)
        if n == 0:
            raise WamError(-2, f"invalid target sizes R={R} T_v={T_v} T_a={T_a}")
        return n

    def teacher_targets(self, kv, T_v, t, a0, eps, K, u, f, a_t=None, ws=None, student=None, stream=None):
        """Teacher-anchored targets for R = len(t) rollouts of one observation
        (kv: its batch-1 cache): u and f [R][T_a][A] (and a_t) on the device."""
        tt = np.ascontiguousarray(t, dtype=np.float32)
        R, T_a = int(tt.size), int(a0.shape[1])
        _check(self.lib.wam_teacher_targets(self.handle, None if student is None else student.handle, _ptr(kv), T_v,
                                            R, T_a, _ptr(a0), _ptr(eps), tt.ctypes.data_as(ctypes.c_void_p), int(K),
                                            _ptr(a_t), _ptr(u), _ptr(f), _ptr(ws), _stream(stream)))

    def reuse_workspace_bytes(self, T_v, T_a=1, S=1):
        n = self.lib.wam_reuse_workspace_bytes(self.handle, T_v, T_a, S)
        if n == 0:
            raise WamError(-2, f"invalid sizes T_v={T_v} T_a={T_a} S={S}")
        return n

    def select_tokens(self, video_new, video_prev, T_v, tau, idx, count, stream=None):
        """Active-token indices (ascending) into idx (T_v int32) and their number into count (1 int32)."""
        _check(self.lib.wam_select_tokens(self.handle, _ptr(video_new), _ptr(video_prev), T_v, float(tau), _ptr(idx),
                                          _ptr(count), _stream(stream)))

    def video_forward_reuse(self, video_new, video_prev, T_v, t_v, tau, kv, ws, hidden=None, stream=None):
        """Update the previous observation's cache kv (and hidden) for the new
        observation, recomputing the active tokens only; returns their count."""
        n = ctypes.c_int(-1)
        _check(self.lib.wam_video_forward_reuse(self.handle, _ptr(video_new), _ptr(video_prev), T_v, float(t_v),
                                                float(tau), _ptr(kv), _ptr(hidden), ctypes.byref(n), _ptr(ws),
                                                _stream(stream)))
        return n.value

    def infer_reuse(self, video_new, video_prev, tau, a_init, t_grid, T_v, T_a, kv, a_out, hidden=None, v_last=None,
                    f_last=None, mode=WAM_CEWP, ws=None, s_video=None, s_action=None):
        """The inference on the next observation of one stream with the reused
        cache kv (updated in place); returns the number of recomputed tokens."""
        g = np.ascontiguousarray(t_grid, dtype=np.float32)
        n = ctypes.c_int(-1)
        _check(self.lib.wam_infer_reuse(self.handle, _ptr(video_new), _ptr(video_prev), float(tau), _ptr(a_init),
                                        g.ctypes.data_as(ctypes.c_void_p), g.size - 1, T_v, T_a, _ptr(kv),
                                        _ptr(hidden), _ptr(a_out), _ptr(v_last), _ptr(f_last), ctypes.byref(n),
                                        int(mode), _ptr(ws), _stream(s_video), _stream(s_action)))
        return n.value

    def infer(self, video, a_init, t_grid, B, T_v, T_a, kv, a_out, v_last=None, f_last=None,
              mode=WAM_CEWP, ws=None, s_video=None, s_action=None):
        g = np.ascontiguousarray(t_grid, dtype=np.float32)
        S = g.size - 1
        _check(self.lib.wam_infer_cewp(self.handle, _ptr(video), _ptr(a_init),
                                       g.ctypes.data_as(ctypes.c_void_p), S, B, T_v, T_a, _ptr(kv), _ptr(a_out),
                                       _ptr(v_last), _ptr(f_last), int(mode), _ptr(ws), _stream(s_video),
                                       _stream(s_action)))


    def graph(self, video, a_init, t_grid, B, T_v, T_a, kv, a_out, v_last=None, f_last=None,
              mode=WAM_CEWP, ws=None, s_video=None, s_action=None):
        """Capture one inference on these buffers; returns a Graph to replay."""
        g = np.ascontiguousarray(t_grid, dtype=np.float32)
        h = ctypes.c_void_p()
        _check(self.lib.wam_graph_create(self.handle, _ptr(video), _ptr(a_init), g.ctypes.data_as(ctypes.c_void_p),
                                         g.size - 1, B, T_v, T_a, _ptr(kv), _ptr(a_out), _ptr(v_last), _ptr(f_last),
                                         int(mode), _ptr(ws), _stream(s_video), _stream(s_action), ctypes.byref(h)))
        return Graph(self.lib, h)


class Graph:
    """A captured inference; launch() replays it on a stream."""

    def __init__(self, lib, handle):
        self.lib, self.handle = lib, handle

    def launch(self, stream=None):
        _check(self.lib.wam_graph_launch(self.handle, _stream(stream)))

    def close(self):
        if self.handle:
            _check(self.lib.wam_graph_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------- single kernels
EPI_F32, EPI_GELU, EPI_GATE_RES, EPI_QKV = 0, 1, 2, 3


def op_gemm(A, W, bias, epi=EPI_F32, out=None, gate=None, head_dim=0, ws=None, stream=None):
    """acc = A W^T, then epilogue `epi` into `out` (allocated when None; for
    EPI_GATE_RES `out` is the float32 residual updated in place).
    A [M][K], W [N][K], bias [N] all float32 or all bfloat16."""
    import torch
    lib = load()
    bf = A.dtype == torch.bfloat16
    dt = WAM_BF16 if bf else WAM_F32
    M, K = A.shape
    N = W.shape[0]
    if out is None:
        if epi == EPI_F32:
            out = torch.empty(M, N, dtype=torch.float32, device=A.device)
        elif epi == EPI_GELU:
            out = torch.empty(M, N, dtype=A.dtype, device=A.device)
        elif epi == EPI_QKV:
            out = torch.empty(3, N // (3 * head_dim), M, head_dim, dtype=A.dtype, device=A.device)
        else:
            raise ValueError("EPI_GATE_RES needs `out` (the residual stream)")
    if ws is None:
        nws = lib.wam_op_gemm_ws_bytes(dt, M, N, K)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=A.device)
    _check(lib.wam_op_gemm(dt, epi, M, N, K, _ptr(A), _ptr(W), _ptr(bias), _ptr(gate), int(head_dim), _ptr(out),
                           _ptr(ws), _stream(stream)))
    return out


def op_attention(q, k0, v0, k1=None, v1=None, stream=None, out=None, ws=None):
    """o [B][Tq][H*dh] from q [B][H][Tq][dh] over keys [k0 ; k1] ([B][H][L][dh])
    with values v0, v1 stored transposed ([B][H][dh][L], contiguous).  out and
    ws (wam_op_attention_ws_bytes bytes) are allocated when None."""
    import torch
    lib = load()
    dt = WAM_BF16 if q.dtype == torch.bfloat16 else WAM_F32
    B, H, Tq, dh = q.shape
    L0 = k0.shape[2] if k0 is not None else 0
    L1 = k1.shape[2] if k1 is not None else 0
    o = torch.empty(B, Tq, H * dh, dtype=q.dtype, device=q.device) if out is None else out
    if ws is None:
        nws = lib.wam_op_attention_ws_bytes(dt, B, H, dh, Tq, L0, L1)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    _check(lib.wam_op_attention(dt, B, H, dh, Tq, _ptr(q), L0, _ptr(k0), _ptr(v0), L1, _ptr(k1), _ptr(v1),
                                _ptr(o), _ptr(ws), _stream(stream)))
    return o


def op_ln_modulate(x, shift, scale, eps, bf16: bool, stream=None):
    import torch
    lib = load()
    rows, d = x.shape
    h = torch.empty(rows, d, dtype=torch.bfloat16 if bf16 else torch.float32, device=x.device)
    _check(lib.wam_op_ln_modulate(WAM_BF16 if bf16 else WAM_F32, rows, d, _ptr(x), _ptr(shift), _ptr(scale),
                                  float(eps), _ptr(h), _stream(stream)))
    return h


def op_qk_norm_rope(x, gain=None, eps=1e-6, rope_hw=(), stream=None):
    """QK-RMSNorm (gain [H*dh] or None) + 3-D RoPE (rope_hw = (rows, columns) per frame,
    or () for none) of x [B][H][T][dh] in place; returns x."""
    lib = load()
    B, H, T, dh = x.shape
    bf16 = x.dtype != __import__("torch").float32
    rh, rw = tuple(rope_hw) if rope_hw else (0, 0)
    _check(lib.wam_op_qk_norm_rope(WAM_BF16 if bf16 else WAM_F32, B, H, T, dh, _ptr(x), _ptr(gain), float(eps),
                                   rh, rw, _stream(stream)))
    return x
