"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake (a dropped term, a wrong sign, a swapped
operand, a wrong index or stride) in a private copy of oracle.c, or (the
whole-model compositions: a skipped norm, the memory of the wrong SSM layer,
the shared cache written by the wrong layer, a ring slot or a visible length
off by one) in a private copy of the oracle's Python module, rebuilds it in
a temporary directory and runs the pin file that should catch it; the case
passes only if that pin run fails.  Nothing here touches the product library
or a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, pin file, original text, planted text)
MUTANTS = [
    ("gmu_sigmoid_sign", "test_oracle_gmu.py",
     "double g = z / (1.0 + exp(-z));", "double g = z / (1.0 + exp(z));"),
    ("gmu_gate_without_memory", "test_oracle_gmu.py",
     "H[k] = widen(M, dt_m, r * d_inner + k) * g;", "H[k] = g;"),
    ("gmu_w2_transposed", "test_oracle_gmu.py",
     "acc += H[k] * widen(W2, dt_w, o * d_inner + k);", "acc += H[k] * widen(W2, dt_w, k * d_model + o);"),
    ("gmu_gate_on_wrong_channel", "test_oracle_gmu.py",
     "H[k] = widen(M, dt_m, r * d_inner + k) * g;", "H[k] = widen(M, dt_m, r * d_inner + (d_inner - 1 - k)) * g;"),
    ("xattn_scale_dropped", "test_oracle_xattn.py", "s[j] = dot * scale;", "s[j] = dot;"),
    ("xattn_no_normalisation", "test_oracle_xattn.py", "for (int64_t d = 0; d < D; ++d) out[d] /= den;",
     "for (int64_t d = 0; d < D; ++d) out[d] /= 1.0;"),
    ("xattn_wrong_group_map", "test_oracle_xattn.py",
     "int64_t b = bh / Hq, h = bh % Hq, g = h / G;\n            xattn_head(q, dt_q, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, out + bh * D, D, L, scale, s, tr, 0, 1, 2);",
     "int64_t b = bh / Hq, h = bh % Hq, g = h % Hkv;\n            xattn_head(q, dt_q, bh * D, K, V, dt_kv, (b * Hkv + g) * L * D, out + bh * D, D, L, scale, s, tr, 0, 1, 2);"),
    ("chunked_merge_without_rescale", "test_oracle_xattn.py",
     "for (int64_t c = 0; c < nc; ++c) l += lc[c] * exp(mc[c] - M);", "for (int64_t c = 0; c < nc; ++c) l += lc[c];"),
    ("round_bf16_truncates", "test_oracle_crossdecoder.py",
     "double r = nearbyint(ldexp(x, -q));", "double r = trunc(ldexp(x, -q));"),
    ("crossdecoder_no_residual", "test_oracle_crossdecoder.py",
     "        for (int64_t i = 0; i < B * d_model; ++i) {\n            trk_mark(tr, 0, i);\n            trk_mark(tr, 1, i);\n            double v = h[i] + y[i];",
     "        for (int64_t i = 0; i < B * d_model; ++i) {\n            trk_mark(tr, 0, i);\n            trk_mark(tr, 1, i);\n            double v = y[i];"),
    ("rmsnorm_sum_not_mean", "test_oracle_ex.py", "ss / (double)n + eps", "ss + eps"),
    ("rmsnorm_eps_outside_root", "test_oracle_ex.py", "1.0 / sqrt(ss / (double)n + eps)",
     "1.0 / (sqrt(ss / (double)n) + eps)"),
    ("swiglu_gate_up_swapped", "test_oracle_ex.py", "u[k] = a / (1.0 + exp(-a)) * b;",
     "u[k] = b / (1.0 + exp(-b)) * a;"),
    ("varlen_stride_uses_length", "test_oracle_ex.py",
     "(b * Hkv + g) * L * D, out + bh * D, D, lens[b], scale, s, NULL,",
     "(b * Hkv + g) * lens[b] * D, out + bh * D, D, lens[b], scale, s, NULL,"),
    ("ex_gmu_takes_unnormalised_h", "test_oracle_ex.py",
     "gmu_row(M, dt_act, x, OR_F64, wa[li], wb[li], dt_w, y + r * d_model, r, d_model, d_inner, H, NULL,",
     "gmu_row(M, dt_act, h, OR_F64, wa[li], wb[li], dt_w, y + r * d_model, r, d_model, d_inner, H, NULL,"),
    ("ex_mlp_uses_mixer_norm", "test_oracle_ex.py",
     "rmsnorm_row(h + r * d_model, norm2[li], dt_w, d_model, eps, x + r * d_model);",
     "rmsnorm_row(h + r * d_model, norm1[li], dt_w, d_model, eps, x + r * d_model);"),
    ("ex_attention_ignores_lengths", "test_oracle_ex.py", "int64_t Lb = lens ? lens[b] : L;", "int64_t Lb = L;"),
    ("diffattn_lambda_sign", "test_oracle_diffattn.py", "y[c] = o1[c] - lambda * o2[c];",
     "y[c] = o1[c] + lambda * o2[c];"),
    ("diffattn_second_map_on_first_half", "test_oracle_diffattn.py",
     "diff_map(q, dt_q, bh * D, K, V, dt_kv, kv, D, d, D, n, scale, s, o2);",
     "diff_map(q, dt_q, bh * D, K, V, dt_kv, kv, D, 0, d, n, scale, s, o2);"),
    ("diffattn_keys_half_swapped", "test_oracle_diffattn.py",
     "dot += widen(q, dt_q, q_off + c) * widen(K, dt_kv, kv_off + j * D + c);",
     "dot += widen(q, dt_q, q_off + c) * widen(K, dt_kv, kv_off + j * D + (c + D / 2) % D);"),
    ("diffattn_norm_sum_not_mean", "test_oracle_diffattn.py", "sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    ("diffattn_lambda_init_dropped", "test_oracle_diffattn.py", "const double r = (1.0 - lambda_init) /",
     "const double r = 1.0 /"),
    ("diffattn_reads_past_length", "test_oracle_diffattn.py", "int64_t n = lens ? lens[b] : L, kv",
     "int64_t n = L, kv"),
    ("selfattn_ring_slot_is_position", "test_oracle_selfattn.py",
     "const int64_t slot = window ? pos[b] % window : pos[b];",
     "const int64_t slot = window ? (pos[b] < window ? pos[b] : window - 1) : pos[b];"),
    ("selfattn_new_token_not_visible", "test_oracle_selfattn.py",
     "const int64_t n = p < 0 ? 0 : (window && p + 1 > window ? window : p + 1);",
     "const int64_t n = p < 0 ? 0 : (window && p > window ? window : p);"),
    ("selfattn_unfilled_ring_slots_visible", "test_oracle_selfattn.py",
     "const int64_t n = p < 0 ? 0 : (window && p + 1 > window ? window : p + 1);",
     "const int64_t n = p < 0 ? 0 : (window ? window : p + 1);"),
    ("mamba_conv_taps_reversed", "test_oracle_mamba.py",
     "for (int64_t k = 0; k < KS; ++k) acc += widen(conv_w, dt_p, c * K + k) * widen(conv_state, dt_s, so + k);\n        acc += widen(conv_w, dt_p, c * K + KS) * xi[c];",
     "for (int64_t k = 0; k < KS; ++k) acc += widen(conv_w, dt_p, c * K + KS - k) * widen(conv_state, dt_s, so + k);\n        acc += widen(conv_w, dt_p, c * K) * xi[c];"),
    ("mamba_step_without_softplus", "test_oracle_mamba.py", "const double dlt = softplus_def(a);",
     "const double dlt = a;"),
    ("mamba_decay_sign", "test_oracle_mamba.py", "const double A = -exp(widen(A_log, dt_p, c * N + n));",
     "const double A = exp(widen(A_log, dt_p, c * N + n));"),
    ("mamba_skip_dropped", "test_oracle_mamba.py", "m += widen(Dp, dt_p, c) * u[c];", "m += 0.0;"),
    ("mamba_gate_dropped", "test_oracle_mamba.py", "GM[b * d_inner + c] = m * (z[c] / (1.0 + exp(-z[c])));",
     "GM[b * d_inner + c] = m;"),
    ("mamba_B_C_swapped", "test_oracle_mamba.py", "const double *delta = xd, *Bv = xd + R, *Cv = xd + R + N;",
     "const double *delta = xd, *Cv = xd + R, *Bv = xd + R + N;"),
    ("mamba_window_not_shifted", "test_oracle_mamba.py",
     "for (int64_t k = 0; k + 1 < KS; ++k) conv_state_out[so + k] = widen(conv_state, dt_s, so + k + 1);",
     "for (int64_t k = 0; k + 1 < KS; ++k) conv_state_out[so + k] = widen(conv_state, dt_s, so + k);"),
    ("prefill_window_off_by_one", "test_oracle_prefill.py",
     "const int64_t j0 = window > 0 && i + 1 > window ? i + 1 - window : 0, j1 = i;",
     "const int64_t j0 = window > 0 && i > window ? i - window : 0, j1 = i;"),
    ("prefill_not_causal", "test_oracle_prefill.py", "? i + 1 - window : 0, j1 = i;", "? i + 1 - window : 0, j1 = T - 1;"),
    ("prefill_excludes_own_token", "test_oracle_prefill.py", "? i + 1 - window : 0, j1 = i;",
     "? i + 1 - window : 0, j1 = i > j0 ? i - 1 : i;"),
    ("prefill_wrong_group_map", "test_oracle_prefill.py",
     "const int64_t b = r / (T * Hq), i = (r / Hq) % T, h = r % Hq, g = h / G;",
     "const int64_t b = r / (T * Hq), i = (r / Hq) % T, h = r % Hq, g = h % Hkv;"),
    ("selfattn_value_row_not_stored", "test_oracle_selfattn.py",
     "V_out[((b * Hkv + g) * L + slot) * D + d] = widen(v_new, dt_new, (b * Hkv + g) * D + d);",
     "V_out[((b * Hkv + g) * L + slot) * D + d] = widen(V, dt_kv, ((b * Hkv + g) * L + slot) * D + d);"),
]


# Mistakes in the oracle's Python compositions (oracle/__init__.py).
PY_MUTANTS = [
    ("prefill_mlp_skips_norm2", "test_oracle_composition.py",
     'xm = rmsnorm(h.reshape(B * T, dm), ly["norm2"], eps) if ly.get("norm2") is not None \\',
     'xm = h.reshape(B * T, dm) if ly.get("norm2") is not None \\'),
    ("decode_mlp_skips_norm2", "test_oracle_composition.py",
     'xm = rmsnorm(h, ly["norm2"], eps) if ly.get("norm2") is not None else h', "xm = h"),
    ("prefill_mixer_skips_norm1", "test_oracle_composition.py",
     'xin = rmsnorm(h.reshape(B * T, dm), ly["norm1"], eps).reshape(B, T, dm) if ly.get("norm1") is not None else h',
     "xin = h"),
    ("prefill_memory_from_first_ssm", "test_oracle_composition.py",
     '            M_mem = M\n            per_layer.append({"conv_state": conv, "ssm_state": ssm})',
     '            M_mem = M if M_mem is None else M_mem\n            per_layer.append({"conv_state": conv, "ssm_state": ssm})'),
    ("decode_memory_from_first_ssm", "test_oracle_composition.py",
     '            M_mem = M\n            per_layer.append({"conv_state": cs, "ssm_state": ss})',
     '            M_mem = M if M_mem is None else M_mem\n            per_layer.append({"conv_state": cs, "ssm_state": ss})'),
    ("prefill_cache_from_window_layer", "test_oracle_composition.py",
     '            if kind == "attn":\n                K, V =', '            if kind == "swa":\n                K, V ='),
    ("decode_window_layer_writes_shared_cache", "test_oracle_composition.py",
     'o, kr, vr = selfattn(q, kn, vn, ly["kring"], ly["vring"], pa, window=window, scale=scale)',
     'o, Kc, Vc = selfattn(q, kn, vn, Kc, Vc, pa, window=0, scale=scale); kr, vr = ly["kring"], ly["vring"]'),
    ("decode_ring_slot_off_by_one", "test_oracle_composition.py",
     'selfattn(q, kn, vn, ly["kring"], ly["vring"], pa, window=window',
     'selfattn(q, kn, vn, ly["kring"], ly["vring"], pa + 1, window=window'),
    ("decode_cross_lengths_exclude_new_token", "test_oracle_composition.py",
     "lens = np.minimum(np.maximum(pa.astype(np.int64) + 1, 0), L)",
     "lens = np.minimum(np.maximum(pa.astype(np.int64), 0), L)"),
    ("prefill_window_ignored", "test_oracle_composition.py",
     'o = attn_prefill(q, k, v, window if kind == "swa" else 0, scale)', "o = attn_prefill(q, k, v, 0, scale)"),
    ("decode_ssm_residual_dropped", "test_oracle_composition.py",
     '            h = rnd(h + y)\n            M_mem = M\n            per_layer.append({"conv_state": cs',
     '            h = rnd(y)\n            M_mem = M\n            per_layer.append({"conv_state": cs'),
    ("prefill_cross_decoder_on_first_token", "test_oracle_composition.py",
     "h_last = np.ascontiguousarray(h[:, T - 1])", "h_last = np.ascontiguousarray(h[:, 0])"),
    ("mamba_prefill_state_not_carried", "test_oracle_mamba.py",
     "M, y, conv, ssm = mamba_step(np.ascontiguousarray(xa[:, t]), w, conv, ssm)",
     "M, y, _, _ = mamba_step(np.ascontiguousarray(xa[:, t]), w, conv, ssm)"),
]

CASES = [("oracle.c",) + m for m in MUTANTS] + [("__init__.py",) + m for m in PY_MUTANTS]


@pytest.fixture(scope="module")
def sources():
    return {f: open(os.path.join(ROOT, "oracle", f)).read() for f in ("oracle.c", "__init__.py")}


@pytest.mark.parametrize("target,name,pins,orig,planted", CASES, ids=[c[1] for c in CASES])
def test_pins_catch_planted_mistake(tmp_path, sources, target, name, pins, orig, planted):
    source = sources[target]
    assert source.count(orig) >= 1, "mutation site for %s not found in %s" % (name, target)
    for d in ("oracle", "workload", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    (tmp_path / "oracle" / target).write_text(source.replace(orig, planted, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join("tests", pins)], cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "planted mistake %r survived %s:\n%s" % (name, pins, r.stdout[-2000:])
