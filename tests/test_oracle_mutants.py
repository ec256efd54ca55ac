"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each mutant is a copy of oracle/fp8_oracle.c with one plausible mistake (a dropped
term, a wrong sign, index, constant or rounding rule), compiled with the same flags
into a temporary directory.  Nothing here touches the GPU or the real oracle build.
"""
import os
import time

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fp8_oracle.c")

MUTANTS = [
    ("ties_away_from_zero", "double n = nearbyint(ldexp(a, mbits - e));",
     "double n = round(ldexp(a, mbits - e));"),
    ("truncating_encode", "double n = nearbyint(ldexp(a, mbits - e));",
     "double n = trunc(ldexp(a, mbits - e));"),
    ("fnuz_e4m3_bias", "return fmt == ORC_E4M3 ? 7 : 15;", "return fmt == ORC_E4M3 ? 8 : 15;"),
    ("subnormals_flushed", "if (e < emin) e = emin;", "if (e < emin) return sign;"),
    ("decode_subnormal_exponent", "v = ldexp((double)m, 1 - bias - mbits);",
     "v = ldexp((double)m, -bias - mbits);"),
    ("e5m2_inf_as_nan", "v = (m == 0) ? INFINITY : NAN;", "v = NAN;"),
    ("no_saturation", "if (v > mx) v = mx;", ""),
    ("multiply_by_scale", "float v = x / scale;", "float v = x * scale;"),
    ("nan_sign_dropped", "return (uint8_t)(0x7F | (signbit(x) ? 0x80 : 0x00));",
     "return (uint8_t)0x7F;"),
    ("amax_keeps_sign", "uint32_t mag = f2u(x) & 0x7FFFFFFFu;", "uint32_t mag = f2u(x);"),
    ("amax_not_accumulated", "uint32_t acc = f2u(*amax);\n  for (int64_t i = 0; i < n; ++i) {\n    float x",
     "uint32_t acc = 0;\n  for (int64_t i = 0; i < n; ++i) {\n    float x"),
    ("no_history_roll", "hist_out[h * n + t] = hist_in[(h - 1) * n + t];",
     "hist_out[h * n + t] = hist_in[h * n + t];"),
    ("new_amax_not_in_window", "for (int64_t h = 0; h < H; ++h) {\n        uint32_t b",
     "for (int64_t h = 1; h < H; ++h) {\n        uint32_t b"),
    ("select_from_old_history", "uint32_t b = f2u(hist_out[h * n + t]);",
     "uint32_t b = f2u(hist_in[h * n + t]);"),
    ("most_recent_is_max", "if (algo == ORC_AMAX_MOST_RECENT) {", "if (algo == 12345) {"),
    ("margin_sign", "c = ldexpf(c, margin);", "c = ldexpf(c, -margin);"),
    ("scale_inverted", "float c = sel / mx;", "float c = mx / sel;"),
    ("scale_inv_from_amax", "scale_inv_out[t] = 1.0f / s;", "scale_inv_out[t] = mx / sel;"),
    # (dropping only the guard on sel is equivalent: the guard on c then catches 0,
    # inf and NaN; so the mistake planted is dropping the guard on the result)
    ("no_keep_previous_guard", "if (isfinite(c) && c > 0.0f) s = c;", "s = c;"),
    ("reset_ignored", "amax_out[t] = reset_amax ? 0.0f : amax[t];", "amax_out[t] = amax[t];"),
    ("formats_swapped", "float mx = oracle_fp8_max(formats[t] ? ORC_E5M2 : ORC_E4M3);",
     "float mx = oracle_fp8_max(formats[t] ? ORC_E4M3 : ORC_E5M2);"),
    ("dequant_divides", "float y = oracle_fp8_decode(fmt, src[i]) * scale;",
     "float y = oracle_fp8_decode(fmt, src[i]) / scale;"),
    ("bf16_truncates", "double r = ldexp(nearbyint(ldexp(a, 7 - e)), e - 7);   /*",
     "double r = ldexp(trunc(ldexp(a, 7 - e)), e - 7);   /*"),
    ("gelu_bf16_truncates", "double r = ldexp(nearbyint(ldexp(a, 7 - e)), e - 7);  /* nearest bf16",
     "double r = ldexp(trunc(ldexp(a, 7 - e)), e - 7);  /* nearest bf16"),
    ("gelu_cubic_coefficient", "const double u = c * (x + 0.044715 * x * x * x);",
     "const double u = c * (x + 0.04715 * x * x * x);"),
    ("gelu_half_argument", "return x / (1.0 + exp(-2.0 * u));", "return x / (1.0 + exp(-u));"),
    ("gelu_neg_inf_kept", "if (isinf(x)) return x > 0 ? x : -0.0;", "if (isinf(x)) return x;"),
    ("gelu_bf16_sign_dropped", "uint16_t sign = signbit(v) ? 0x8000 : 0;", "uint16_t sign = 0;"),
    ("ln_unbiased_variance", "const double V = (sv + cv) / (double)H;",
     "const double V = (sv + cv) / (double)(H - 1);"),
    ("ln_eps_outside_sqrt", "const double rr = 1.0 / sqrt(V + (double)eps);",
     "const double rr = 1.0 / (sqrt(V) + (double)eps);"),
    ("ln_beta_dropped", "const double v = g * d * rr + b;", "const double v = g * d * rr;"),
    ("ln_gamma_dropped", "const double v = g * d * rr + b;", "const double v = d * rr + b;"),
    ("ln_mean_off_by_one", "const double mu = (s + c) / (double)H;",
     "const double mu = (s + c) / (double)(H + 1);"),
    ("ln_nonfinite_row_kept", "for (int64_t i = 0; i < H; ++i) yr[i] = lr[i] = hr[i] = 0x7FC0;",
     "for (int64_t i = 0; i < H; ++i) yr[i] = lr[i] = hr[i] = xr[i];"),
    ("ln_nan_negative", "        yr[i] = lr[i] = hr[i] = 0x7FC0;\n        continue;",
     "        yr[i] = lr[i] = hr[i] = 0xFFC0;\n        continue;"),
    ("ln_window_dropped", "lr[i] = round_d_to_bf16(v - w, NULL, NULL);",
     "lr[i] = round_d_to_bf16(v, NULL, NULL);"),
    ("ln_window_one_sided", "hr[i] = round_d_to_bf16(v + w, NULL, NULL);",
     "hr[i] = round_d_to_bf16(v, NULL, NULL);"),
    ("gemm_b_transposed", "fp8_parts a = fp8_split(a_fmt, A[m * K + k]), b = fp8_split(b_fmt, B[n * K + k]);",
     "fp8_parts a = fp8_split(a_fmt, A[m * K + k]), b = fp8_split(b_fmt, B[k * N + n]);"),
    ("gemm_scale_dropped", "C_exact[m * N + n] = v * s;", "C_exact[m * N + n] = v;"),
    ("gemm_subnormal_exponent", "if (ex == 0) { p.m = man; p.e = 1 - bias - mbits; }",
     "if (ex == 0) { p.m = man; p.e = -bias - mbits; }"),
    ("gemm_sign_dropped", "  if (sign) p.m = -p.m;\n  return p;", "  return p;"),
    ("gemm_inf_times_zero", "if (sa_ == 0 || sb_ == 0) nan = 1;", "if (sa_ == 0 || sb_ == 0) continue;"),
    ("gemm_nan_ignored", "if (a.special == 2 || b.special == 2) { nan = 1; continue; }",
     "if (a.special == 2 || b.special == 2) { continue; }"),
    ("gemm_group_of_four", "if (k % 8 == 0) { gsum += gmax; gmax = 0.0; }",
     "if (k % 4 == 0) { gsum += gmax; gmax = 0.0; }"),
    ("amax_nan_canonical", "  *amax = u2f(acc);\n}\n\n/* The amax-history",
     "  *amax = isnan(u2f(acc)) ? NAN : u2f(acc);\n}\n\n/* The amax-history"),
    ("e4m3_max_480", "return fmt == ORC_E4M3 ? 448.0f : 57344.0f;",
     "return fmt == ORC_E4M3 ? 480.0f : 57344.0f;"),
    ("count_saturated_one_sided", "if (v > mx || v < -mx) ++c;", "if (v > mx) ++c;"),
    ("gelu_array_index_shift", "y[i] = oracle_gelu_bf16(x[i], &alt[i]);",
     "y[i] = oracle_gelu_bf16(x[i > 0 ? i - 1 : 0], &alt[i]);"),
    ("dequant_nan_unsigned", "uint32_t nan_bits = 0x7FC00000u | ((uint32_t)(src[i] & 0x80) << 24);",
     "uint32_t nan_bits = 0x7FC00000u;"),
]

# cheap pins first; a mutant stops at its first failing pin
_ORDER = sorted(oracle_pins.ALL_PINS,
                key=lambda p: p.__name__ in ("pin_quantize_exact_quotient",
                                             "pin_encode_bruteforce_all_bf16"))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found uniquely: %s" % name
    mpath = tmp_path / ("mut_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(lib_path=str(tmp_path / ("lib_%s.so" % name)), src=str(mpath))
    o = oracle.Oracle(lib)
    caught = []
    for pin in _ORDER:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
            break
        except Exception as e:          # a crash in the mutant also counts as caught
            caught.append("%s:%s" % (pin.__name__, type(e).__name__))
            break
    assert caught, "planted mistake %r passed every pin" % name


def _functions(src):
    """Top-level function definitions of the oracle source: name -> (is_static, body
    text from the signature to the closing brace at column 0)."""
    import re
    out = {}
    for m in re.finditer(r"^(static )?[a-z][\w ]*?\b(\w+)\(([^;{]*?)\)\s*\{", src, re.M):
        start = m.start()
        end = src.find("\n}", m.end())
        one_line = src.find("}\n", m.end())
        if one_line != -1 and "\n" not in src[m.end():one_line]:
            end = one_line            # a definition on one line
        out[m.group(2)] = (m.group(1) is not None, src[start:end + 2])
    return out


def test_every_exported_oracle_function_has_a_mutant():
    """Each exported oracle function contains (itself or through a static helper it
    calls) the site of at least one planted mistake above, so every function the tests
    rely on is pinned by a pin that the parametrized test shows catching that mistake."""
    src = open(SRC).read()
    fns = _functions(src)
    exported = sorted(k for k, (st, _) in fns.items() if not st and k.startswith("oracle_"))
    assert "oracle_quantize_amax" in exported and "oracle_fp8_encode" in exported

    def reach(name, seen=None):
        seen = seen or set()
        if name in seen:
            return ""
        seen.add(name)
        text = fns[name][1]
        for other, (st, _) in fns.items():
            if other != name and (st or other.startswith("oracle_")) and other + "(" in text:
                text += reach(other, seen)
        return text

    missing = [f for f in exported if not any(old in reach(f) for _, old, _ in MUTANTS)]
    assert not missing, "exported oracle functions without a planted mistake: %s" % missing
