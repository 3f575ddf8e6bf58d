"""Each plausible mistake planted in a copy of the oracle source must fail at least one pin.

The copy is patched textually, compiled with gcc into a temporary directory and
loaded on its own; the real oracle is never modified.  This shows the pins in
pinlib.py can tell a correct oracle from a subtly wrong one.
"""
import os

import pytest

import oracle
import pinlib

SRC = os.path.join(pinlib.ROOT, "oracle", "dsa_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("no_relu", "double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    ("relu_keeps_negative", "double relu = dot > 0.0 ? dot : 0.0;",
     "double relu = dot > 0.0 ? dot : -dot;"),
    ("weight_before_relu",  # the earlier MLX variant: weights applied before the ReLU
     "double relu = dot > 0.0 ? dot : 0.0;\n        acc += (double)w[row * H + h] * relu;",
     "double wd = (double)w[row * H + h] * dot;\n        acc += wd > 0.0 ? wd : 0.0;"),
    ("no_head_sum", "acc += (double)w[row * H + h] * relu;",
     "acc = (double)w[row * H + h] * relu;"),
    ("weights_dropped", "acc += (double)w[row * H + h] * relu;", "acc += relu;"),
    ("wrong_head_of_q", "qv[h * D + d] = v;", "qv[h * D + d] = elem(q, dtype, (size_t)row * H * D + d) * qs;"),
    ("k_scale_dropped", "kvals[d] = (elem(k, dtype, krow * D + d) * ks);", "kvals[d] = elem(k, dtype, krow * D + d);"),
    ("q_scale_dropped", "double qs = dtype == ORACLE_FP8_E4M3 ? (double)q_scale[row * H + h] : 1.0;",
     "double qs = 1.0;"),
    ("scale_dropped", "out[(size_t)row * S_max + (size_t)s] = acc32 * scale;",
     "out[(size_t)row * S_max + (size_t)s] = acc32;"),
    ("bound_short_by_one", "int64_t bound = (int64_t)end_pos[b] - T + t;",
     "int64_t bound = (int64_t)end_pos[b] - T + t - 1;"),
    ("key_batch_offset_dropped", "size_t krow = (size_t)b * S_max + (size_t)s;",
     "size_t krow = (size_t)s;"),
    ("fp8_subnormal_wrong", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("fp8_bias_wrong", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("topk_ascending_scores", "if (a->score > b->score) return -1;\n  if (a->score < b->score) return 1;",
     "if (a->score < b->score) return -1;\n  if (a->score > b->score) return 1;"),
    ("topk_ties_to_larger", "return (a->pos > b->pos) - (a->pos < b->pos);",
     "return (a->pos < b->pos) - (a->pos > b->pos);"),
    ("topk_output_unsorted", "qsort(dst, (size_t)keep, sizeof(int32_t), ascending_int);", ""),
    ("topk_one_short", "int64_t keep = n < k ? n : k;", "int64_t keep = n < k ? n : k - 1;"),
    ("topk_no_padding", "for (int64_t j = keep; j < k; ++j) dst[j] = -1;", ""),
    ("mla_pe_dropped", "z[s] = (dot + dot_pe) * sc;", "z[s] = dot * sc;"),
    ("mla_scale_dropped", "z[s] = (dot + dot_pe) * sc;", "z[s] = (dot + dot_pe);"),
    ("mla_mask_ignored", "memset(keep, idx ? 0 : 1, (size_t)n);", "memset(keep, 1, (size_t)n);"),
    ("mla_not_normalised", "for (int c = 0; c < Dc; ++c) o[c] /= l;", ""),
    ("mla_lse_without_max", "lse[(size_t)row * H + h] = m + log(l);",
     "lse[(size_t)row * H + h] = log(l);"),
    ("mla_value_is_pe_row", "o[c] += z[s] * bf16_value(kvs[c]);",
     "o[c] += z[s] * bf16_value(kvs[(c + 1) % Dc]);"),
    ("mla_causal_off_by_one", "int64_t n = (int64_t)end_pos[b] - T + t + 1; /* valid positions 0..n-1 */",
     "int64_t n = (int64_t)end_pos[b] - T + t; /* valid positions 0..n-1 */"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle._load(oracle.build(str(path), str(tmp_path / f"lib{name}.so")))
    failures = []
    for check in pinlib.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError) as e:
            failures.append(check.__name__)
    assert failures, f"mutant {name} passed every pin"


# Planted mistakes in the Python part of the oracle (indexer input preparation,
# MHA-form prefill attention, query absorption and output up-projection):
# (name, text in oracle/__init__.py, replacement).  Each patched copy is loaded as
# a module of its own and run against the preparation, MHA and projection pins.
PY_SRC = os.path.join(pinlib.ROOT, "oracle", "__init__.py")
PY_MUTANTS = [
    ("rope_sign", "x1 * cos - x2 * sin", "x1 * cos + x2 * sin"),
    ("rope_interleaved", "x1, x2 = x[..., :ROPE_DIM // 2], x[..., ROPE_DIM // 2:ROPE_DIM]",
     "x1, x2 = x[..., 0:ROPE_DIM:2], x[..., 1:ROPE_DIM:2]"),
    ("rope_on_last_dims", "q[..., :ROPE_DIM] = rope_halves(q[..., :ROPE_DIM],",
     "q[..., -ROPE_DIM:] = rope_halves(q[..., -ROPE_DIM:],"),
    ("key_not_roped", "    k[..., :ROPE_DIM] = rope_halves(k[..., :ROPE_DIM], c, s)\n", ""),
    ("position_off_by_one", "- T + np.arange(T)[None, :]", "- T + 1 + np.arange(T)[None, :]"),
    ("hadamard_unscaled", "return y / np.sqrt(128.0) if scaled else y", "return y"),
    ("hadamard_sign", "np.stack([a + b, a - b], axis=-2)", "np.stack([a + b, b - a], axis=-2)"),
    ("e4m3_ties_to_odd", "(hi % 2 == 0)", "(hi % 2 == 1)"),
    ("e4m3_max_240", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("e4m3_subnormal_step", "m * 2.0 ** -9 if e == 0", "m * 2.0 ** -10 if e == 0"),
    ("amax_signed", "np.max(np.abs(u32), axis=-1)", "np.max(u32, axis=-1)"),
    ("post_scale_dropped", "(scale_u * np.float32(post_scale))", "(scale_u)"),
    ("mha_no_causal_mask", "        sel = sel[sel <= s]                                   # the causal mask\n", ""),
    ("mha_causal_strict", "sel = sel[sel <= s]", "sel = sel[sel < s]"),
    ("mha_duplicates_counted", "sel = np.unique(sel[(sel >= 0) & (sel < T)])",
     "sel = sel[(sel >= 0) & (sel < T)]"),
    ("mha_rope_key_dropped", "np.broadcast_to(kp[b, sel][:, None, :],",
     "np.broadcast_to(0 * kp[b, sel][:, None, :],"),
    ("mha_scale_dropped", "* float(softmax_scale)", ""),
    ("mha_lse_without_max", "lse[b, s] = (m + np.log(l))[:, 0]", "lse[b, s] = np.log(l)[:, 0]"),
    ("mha_value_of_wrong_key", 'np.einsum("hn,nhd->hd", p, vf[b, sel])',
     'np.einsum("hn,nhd->hd", p, vf[b, np.roll(sel, 1)])'),
    # query absorption and output up-projection
    ("absorb_uses_value_rows", "w = _as_f64(wkv_b)[:, :QK_NOPE, :]",
     "w = _as_f64(wkv_b)[:, -QK_NOPE:, :]"),
    ("absorb_wrong_head", 'return np.einsum("bthd,hdc->bthc", q, w)',
     'return np.einsum("bthd,hdc->bthc", q, np.roll(w, 1, axis=0))'),
    ("absorb_rows_reversed", 'return np.einsum("bthd,hdc->bthc", q, w)',
     'return np.einsum("bthd,hdc->bthc", q, w[:, ::-1, :])'),
    ("outproj_uses_key_rows", "w = _as_f64(wkv_b)[:, -V_HEAD:, :]",
     "w = _as_f64(wkv_b)[:, :V_HEAD, :]"),
    ("outproj_wrong_head", 'return np.einsum("bthc,hdc->bthd", xx, w)',
     'return np.einsum("bthc,hdc->bthd", xx, np.roll(w, 1, axis=0))'),
    ("outproj_latent_reversed", 'return np.einsum("bthc,hdc->bthd", xx, w)',
     'return np.einsum("bthc,hdc->bthd", xx[..., ::-1], w)'),
]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(name, old, new, tmp_path):
    import importlib.util
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"oracle_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failures = []
    lib = oracle._load()
    for check in pinlib.PREP_CHECKS + pinlib.MHA_CHECKS + pinlib.PROJ_CHECKS:
        try:
            check(lib, mod=mod)
        except (AssertionError, ValueError, IndexError) as e:
            failures.append(check.__name__)
    assert failures, f"mutant {name} passed every pin"
