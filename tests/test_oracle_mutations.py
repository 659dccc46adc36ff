"""The oracle pins must catch plausible mistakes.

Each case copies the oracle into a temporary directory, plants one mistake
in the copy (a dropped term, a swapped operand, a wrong sign or index) and
runs tests/test_oracle_pins.py against the copy in a subprocess.  Every
mutant must fail at least one pin.  The real oracle file is never touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sample_variance": ("var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)",
                        "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
    "shift_scale_swapped": ("shift1, scale1 = mod[0], mod[1]", "scale1, shift1 = mod[0], mod[1]"),
    "gates_swapped": ("gate1, shift2, scale2, gate2 = mod[2], mod[3], mod[4], mod[5]",
                      "gate2, shift2, scale2, gate1 = mod[2], mod[3], mod[4], mod[5]"),
    "scale_1_over_dh": ("/ math.sqrt(dh)", "/ dh"),
    "tanh_gelu": ("0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))",
                  "0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))"),
    "sin_before_cos": ("np.concatenate([np.cos(args), np.sin(args)])",
                       "np.concatenate([np.sin(args), np.cos(args)])"),
    "no_time_scale": ("args = 1000.0 * float(t) * freqs", "args = float(t) * freqs"),
    "euler_sign": ("return a - (float(t_cur) - float(t_next)) * v",
                   "return a + (float(t_cur) - float(t_next)) * v"),
    "endpoint_without_t": ("return a - float(t) * v", "return a - v"),
    "wrong_video_block": ("Kv, Vv = kv[i]", "Kv, Vv = kv[-1]"),
    "video_kv_dropped": ("o = attention(q, np.concatenate([k, Kv], axis=1), np.concatenate([v, Vv], axis=1))",
                         "o = attention(q, k, v)"),
    "modulate_without_one": ("return h * (1.0 + scale) + shift", "return h * scale + shift"),
    "heads_interleaved": ("return y.reshape(T, H, dh).transpose(1, 0, 2)",
                          "return y.reshape(T, dh, H).transpose(2, 0, 1)"),
    "adaln_without_silu": ("mvec = linear(silu(c),", "mvec = linear(c,"),
    "mlp_bias_dropped": ('P(f"{ex}.{i}.fc2.w"), P(f"{ex}.{i}.fc2.b"))',
                         'P(f"{ex}.{i}.fc2.w"), 0 * P(f"{ex}.{i}.fc2.b"))'),
    "qkv_thirds_swapped": ("for j in range(3))", "for j in (1, 0, 2))"),
    "rms_sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "rope_sign": ("out[:, :, e1] = x[:, :, e0] * sn + x[:, :, e1] * c",
                  "out[:, :, e1] = -x[:, :, e0] * sn + x[:, :, e1] * c"),
    "rope_frequency_exponent": ("theta ** (-2.0 * i / size)", "theta ** (-1.0 * i / size)"),
    "rope_rows_columns_swapped": ("n // (Hp * Wp), (n // Wp) % Hp, n % Wp", "n // (Hp * Wp), n % Wp, (n // Wp) % Hp"),
    "qk_norm_per_head": ('q = rms_norm(q, P(f"{ex}.{i}.qn.g"), m.ln_eps)',
                         'q = rms_norm(q.reshape(-1, m.n_heads, m.head_dim), P(f"{ex}.{i}.qn.g").reshape(m.n_heads, m.head_dim), m.ln_eps).reshape(q.shape)'),
    "target_sign": ("u = (a_t - a) / t", "u = (a - a_t) / t"),
    "interpolation_swapped": ("a_t = (1.0 - t) * a0 + t * eps", "a_t = t * a0 + (1.0 - t) * eps"),
    "rollout_from_one": ("grid = [t * j / K for j in range(K + 1)]", "grid = [j / K for j in range(K + 1)]"),
    "student_at_time_zero": ("f = endpoint(a_t, action_velocity(P_student, m, kv, a_t, t), t)",
                             "f = endpoint(a_t, action_velocity(P_student, m, kv, a_t, 0.0), t)"),
    "rope_band_order": ("for a, size in enumerate(bands):", "for a, size in reversed(list(enumerate(bands))):"),
    "reuse_keys_not_written": ("        K[:, active] = k\n", "        K[:, active] = K[:, active]\n"),
    "reuse_active_keys_only": ('x = rest(P, "v", i, mod, x, attention(q, K, V), m)',
                               'x = rest(P, "v", i, mod, x, attention(q, K[:, active], V[:, active]), m)'),
    "reuse_threshold_vs_new_norm": ("p2 = np.sum(xp * xp, axis=1, dtype=np.float32)",
                                    "p2 = np.sum(xn * xn, axis=1, dtype=np.float32)"),
    "reuse_threshold_not_squared": ("t2 = np.float32(tau) * np.float32(tau)", "t2 = np.float32(tau)"),
    "reuse_previous_tokens_as_input": ("x = np.asarray(video_new, dtype=np.float64)[active]",
                                       "x = np.asarray(video_prev, dtype=np.float64)[active]"),
    "final_shift_scale_swapped": ('shift_f, scale_f = np.split(linear(silu(c), P("a.fada.w")',
                                  'scale_f, shift_f = np.split(linear(silu(c), P("a.fada.w")'),
    "final_no_layernorm": ("modulate(layer_norm(y, m.ln_eps), shift_f, scale_f)", "modulate(y, shift_f, scale_f)"),
    "final_without_silu": ('np.split(linear(silu(c), P("a.fada.w")', 'np.split(linear(c, P("a.fada.w")'),
    "final_out_bias_dropped": ('P("a.out.w"), P("a.out.b"))', 'P("a.out.w"), 0 * P("a.out.b"))'),
    "tmlp_no_silu": ('h = silu(linear(e, P(f"{ex}.t1.w"), P(f"{ex}.t1.b")))',
                     'h = linear(e, P(f"{ex}.t1.w"), P(f"{ex}.t1.b"))'),
    "tmlp_b2_dropped": ('return linear(h, P(f"{ex}.t2.w"), P(f"{ex}.t2.b"))',
                        'return linear(h, P(f"{ex}.t2.w"), 0 * P(f"{ex}.t2.b"))'),
    "tmlp_b1_dropped": ('h = silu(linear(e, P(f"{ex}.t1.w"), P(f"{ex}.t1.b")))',
                        'h = silu(linear(e, P(f"{ex}.t1.w"), 0 * P(f"{ex}.t1.b")))'),
    "rope_band_sizes": ("side = 2 * (dh // 6)", "side = 2 * (dh // 7)"),
}


def _run_pins_on_copy(tmp_path, old, new):
    src = open(os.path.join(ROOT, "oracle", "wam_oracle.py")).read()
    assert src.count(old) >= 1, f"mutation site {old!r} no longer exists"
    odir = tmp_path / "oracle"
    odir.mkdir()
    (odir / "__init__.py").write_text("")
    (odir / "wam_oracle.py").write_text(src.replace(old, new))
    shutil.copytree(os.path.join(ROOT, "mot_diffusion_transformer_amd"),
                    tmp_path / "mot_diffusion_transformer_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    test_src = open(os.path.join(ROOT, "tests", "test_oracle_pins.py")).read()
    (tmp_path / "test_pins_copy.py").write_text(test_src)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "--rootdir", str(tmp_path), str(tmp_path / "test_pins_copy.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    return r


def test_unmutated_copy_passes(tmp_path):
    # control: the harness itself works, so a failing mutant fails on a pin
    r = _run_pins_on_copy(tmp_path, "def linear(", "def linear(")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and "failed" not in r.stdout


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    r = _run_pins_on_copy(tmp_path, old, new)
    assert r.returncode == 1 and "failed" in r.stdout, f"mutant {name} not caught:\n{r.stdout[-2000:]}"
