"""The oracle pins catch plausible mistakes: each planted mistake must fail at least one pin.

Each mutant is the oracle's C source with one textual edit (a dropped term, a
wrong sign, index or stride, a swapped operand), compiled on the CPU into a
temporary library. The real oracle source is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "softmax drops the max shift": ("double e = exp(load_elem(x, row_off + j, dtype) - m);",
                                    "double e = exp(load_elem(x, row_off + j, dtype));"),
    "softmax takes the min": ("    if (v > m) m = v;\n  }\n  double d = 0.0;\n  for (int64_t j = 0; j < N; ++j) {\n    double e",
                              "    if (v < m) m = v;\n  }\n  double d = 0.0;\n  for (int64_t j = 0; j < N; ++j) {\n    double e"),
    "softmax skips the division": ("for (int64_t j = 0; j < N; ++j) y[j] = y[j] / d;",
                                   "for (int64_t j = 0; j < N; ++j) y[j] = y[j];"),
    "bf16 decoded with a wrong shift": ("uint32_t bits = (uint32_t)h << 16;",
                                        "uint32_t bits = (uint32_t)h << 15;"),
    "softmax ignores the row stride": ("softmax_row(x, i * ld_x, N, dtype, y + i * N);",
                                       "softmax_row(x, i * N, N, dtype, y + i * N);"),
    "softmax backward flips the sign of s": ("(load_elem(dy, i * ld_dy + j, dtype) - s);",
                                             "(load_elem(dy, i * ld_dy + j, dtype) + s);"),
    "softmax backward multiplies by dy": (
        "dx[i * N + j] = load_elem(y, i * ld_y + j, dtype) *",
        "dx[i * N + j] = load_elem(dy, i * ld_dy + j, dtype) *"),
    "softmax backward uses y's stride for dy": (
        "s += load_elem(y, i * ld_y + j, dtype) * load_elem(dy, i * ld_dy + j, dtype);",
        "s += load_elem(y, i * ld_y + j, dtype) * load_elem(dy, i * ld_y + j, dtype);"),
    "loss adds the target logit": ("loss[r] = (m - xt) + log(d);", "loss[r] = (m + xt) + log(d);"),
    "loss drops log d": ("loss[r] = (m - xt) + log(d);", "loss[r] = (m - xt);"),
    "loss formed as (m + log d) - x_t": ("loss[r] = (m - xt) + log(d);",
                                         "loss[r] = (m + log(d)) - xt;"),
    "target logit read from row 0": ("double xt = load_elem(logits, off + t, dtype);",
                                     "double xt = load_elem(logits, t, dtype);"),
    "gradient not divided by n": ("if (reduction == XRO_MEAN) w = w / (double)n;",
                                  "if (reduction == XRO_MEAN) w = w;"),
    "onehot at the wrong column": ("g[j] = w * ((j == t) ? p - 1.0 : p);",
                                   "g[j] = w * ((j == t + 1) ? p - 1.0 : p);"),
    "onehot added instead of subtracted": ("g[j] = w * ((j == t) ? p - 1.0 : p);",
                                           "g[j] = w * ((j == t) ? p + 1.0 : p);"),
    "upstream gradient ignored": ("double w = scale ? scale[i * scale_stride] : 1.0;",
                                  "double w = 1.0;"),
    "upstream gradient of row 0 for every row": ("double w = scale ? scale[i * scale_stride] : 1.0;",
                                                 "double w = scale ? scale[0] : 1.0;"),
    "upstream gradient indexed by list position": (
        "double w = scale ? scale[i * scale_stride] : 1.0;",
        "double w = scale ? scale[r * scale_stride] : 1.0;"),
    "sum reduction divides by n": ("if (reduction == XRO_MEAN) w = w / (double)n;",
                                   "if (reduction != XRO_NONE) w = w / (double)n;"),
    "none reduction divides by n": ("if (reduction == XRO_MEAN) w = w / (double)n;",
                                    "if (reduction != XRO_SUM) w = w / (double)n;"),
    "sum skips the first loss": ("for (int64_t i = 0; i < M; ++i) s += loss[i];\n  return s;",
                                 "for (int64_t i = 1; i < M; ++i) s += loss[i];\n  return s;"),
    "element_mul ignores the row stride": ("out[i * V + j] = load_elem(x, i * ld + j, dtype) * w;",
                                           "out[i * V + j] = load_elem(x, i * V + j, dtype) * w;"),
    "element_mul scales by row 0's value": ("double w = scale[i * scale_stride];",
                                            "double w = scale[0];"),
    "nll drops log d": ("out[i * N + j] = lse - (load_elem(x, i * ld_x + j, dtype) - m);",
                        "out[i * N + j] = 0.0 - (load_elem(x, i * ld_x + j, dtype) - m);"),
    "nll adds the logit": ("out[i * N + j] = lse - (load_elem(x, i * ld_x + j, dtype) - m);",
                           "out[i * N + j] = lse + (load_elem(x, i * ld_x + j, dtype) - m);"),
    "nll ignores the row stride": ("out[i * N + j] = lse - (load_elem(x, i * ld_x + j, dtype) - m);",
                                   "out[i * N + j] = lse - (load_elem(x, i * N + j, dtype) - m);"),
    "nll loss read at the next column": ("round_to_dtype(out[i * N + idx[i]], dtype)",
                                         "round_to_dtype(out[i * N + (idx[i] + 1) % N], dtype)"),
    "nll loss not rounded": ("round_to_dtype(out[i * N + idx[i]], dtype)", "out[i * N + idx[i]]"),
    "bf16 rounding keeps 9 bits": ("return ldexp(nearbyint(ldexp(f, 8)), e - 8);",
                                   "return ldexp(nearbyint(ldexp(f, 9)), e - 9);"),
    "bf16 rounding truncates": ("return ldexp(nearbyint(ldexp(f, 8)), e - 8);",
                                "return ldexp(trunc(ldexp(f, 8)), e - 8);"),
    "nll accepts an index equal to N": ("(idx[i] >= 0 && idx[i] < N)", "(idx[i] >= 0 && idx[i] <= N)"),
    "layer norm drops eps": ("double r = 1.0 / sqrt(v / (double)N + eps);\n    mean[i] = mu;",
                             "double r = 1.0 / sqrt(v / (double)N);\n    mean[i] = mu;"),
    "layer norm variance over N - 1": ("double r = 1.0 / sqrt(v / (double)N + eps);\n    mean[i] = mu;",
                                       "double r = 1.0 / sqrt(v / (double)(N - 1) + eps);\n    mean[i] = mu;"),
    "layer norm multiplies by std": ("double r = 1.0 / sqrt(v / (double)N + eps);\n    mean[i] = mu;",
                                     "double r = sqrt(v / (double)N + eps);\n    mean[i] = mu;"),
    "layer norm skips the weight": ("(load_elem(x, i * ld_x + j, dtype) - mu) * r * load_elem(w, j, dtype) +",
                                    "(load_elem(x, i * ld_x + j, dtype) - mu) * r +"),
    "layer norm bias at the wrong column": ("                     load_elem(b, j, dtype);",
                                            "                     load_elem(b, (j + 1) % N, dtype);"),
    "layer norm backward drops c1": ("dx[i * N + j] = r * (g - (xh * c1 + c2));",
                                     "dx[i * N + j] = r * (g - c2);"),
    "layer norm backward drops c2": ("dx[i * N + j] = r * (g - (xh * c1 + c2));",
                                     "dx[i * N + j] = r * (g - xh * c1);"),
    "layer norm backward drops rstd": ("dx[i * N + j] = r * (g - (xh * c1 + c2));",
                                       "dx[i * N + j] = (g - (xh * c1 + c2));"),
    "layer norm backward c2 unweighted": ("      c1 += xh * g;\n      c2 += g;",
                                          "      c1 += xh * g;\n      c2 += load_elem(dy, i * ld_dy + j, dtype);"),
    "layer norm dw uses x instead of xhat": (
        "sw += d * ((load_elem(x, r * ld_x + j, dtype) - mu[r]) * rs[r]);",
        "sw += d * load_elem(x, r * ld_x + j, dtype);"),
    "layer norm dw reads dy with x's stride": (
        "double d = load_elem(dy, r * ld_dy + j, dtype);",
        "double d = load_elem(dy, r * ld_x + j, dtype);"),
    "layer norm db skips the last row": ("for (int64_t r = 0; r < M; ++r) {\n      double d =",
                                         "for (int64_t r = 0; r + 1 < M; ++r) {\n      double d ="),
    "block-sparse backward drops the scale": (
        "out[base + c] = load_elem(y, base + c, dtype) * (load_elem(dy, base + c, dtype) - s) * scale;",
        "out[base + c] = load_elem(y, base + c, dtype) * (load_elem(dy, base + c, dtype) - s);"),
    "block-sparse backward adds s": (
        "out[base + c] = load_elem(y, base + c, dtype) * (load_elem(dy, base + c, dtype) - s) * scale;",
        "out[base + c] = load_elem(y, base + c, dtype) * (load_elem(dy, base + c, dtype) + s) * scale;"),
    "block-sparse table entries two words apart": (
        "        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;\n        for (int64_t c = 0; c < block; ++c)\n          s +=",
        "        int64_t base = z * stride_z + (int64_t)lut[offset + 2 * k] * block * block + i * block;\n        for (int64_t c = 0; c < block; ++c)\n          s +="),
    "block-sparse rows read as block columns": (
        "        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;\n        for (int64_t c = 0; c < block; ++c)\n          out",
        "        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i;\n        for (int64_t c = 0; c < block; ++c)\n          out"),
    "block-sparse sum skips the last block": (
        "      for (int32_t k = 0; k < size; ++k) {\n        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;\n        for (int64_t c = 0; c < block; ++c)\n          s +=",
        "      for (int32_t k = 0; k + 1 < size; ++k) {\n        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;\n        for (int64_t c = 0; c < block; ++c)\n          s +="),
    "block-sparse batches not offset": (
        "    int64_t z = zr / n_brows, r = zr % n_brows;",
        "    int64_t z = 0 * (zr / n_brows), r = zr % n_brows;"),
    "element_mul adds the scale": ("out[i * V + j] = load_elem(x, i * ld + j, dtype) * w;",
                                   "out[i * V + j] = load_elem(x, i * ld + j, dtype) + w;"),
    "ignored rows keep stale gradient": ("        for (int64_t j = 0; j < V; ++j) g[j] = 0.0;\n      continue;",
                                         "        for (int64_t j = 0; j < V; ++j) (void)g;\n      continue;"),
    "ignored rows counted in n": ("    if (target[i] == ignore_index) continue;\n    ++n;",
                                  "    ++n;"),
    "mean divides by the row count": ("return s / (double)n;", "return s / (double)M;"),
    "ignore_index checked only outside [0, V)": ("if (t == ignore_index || t < 0 || t >= V) {",
                                                 "if (t < 0 || t >= V) {"),
    "exp of the shifted logit uses the wrong sign": (
        "double p = exp(load_elem(logits, off + j, dtype) - m) / d;",
        "double p = exp(m - load_elem(logits, off + j, dtype)) / d;"),
    "sum of exponentials skips the last column": (
        "for (int64_t j = 0; j < V; ++j) d += exp(load_elem(logits, off + j, dtype) - m);",
        "for (int64_t j = 0; j + 1 < V; ++j) d += exp(load_elem(logits, off + j, dtype) - m);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, replace = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(find) == 1, f"mutation site for {name!r} must occur exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(find, replace))
    lib = oracle.compile_library(str(mutant_src), str(tmp_path / "libmutant.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
        if failed:
            break
    assert failed, f"no pin catches the planted mistake {name!r}"
