"""The oracle's pins must catch plausible slips.

Each case below compiles a copy of the C oracle with one planted mistake (on
the CPU, in a temporary directory) and checks that at least one pin of
test_oracle.py fails against it. A mutant that every pin accepts would mean a
part of the oracle is not actually pinned.
"""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "bitnest_oracle.c")

MUTANTS = {
    "nibble order swapped": ("(k % 2 == 0) ? (b & 0x0F) : (b >> 4)", "(k % 2 == 0) ? (b >> 4) : (b & 0x0F)"),
    "byte index k instead of k/2": ("uint8_t b = plane_row[k / 2];", "uint8_t b = plane_row[k / 2 + (k & 1) * 0];\n    b = plane_row[(k / 2) ^ 1];"),
    "draft offset 7": ("int h = nibble_at(hi_row, k) - 8;", "int h = nibble_at(hi_row, k) - 7;"),
    "target /16 dropped": ("return (double)(16 * h + l) * sc / 16.0;", "return (double)(16 * h + l) * sc;"),
    "target factor 16 dropped": ("return (double)(16 * h + l) * sc / 16.0;", "return (double)(h + l) * sc / 16.0;"),
    "zero point 128": ("return (double)(16 * h + l) * sc / 16.0;", "return (double)(16 * h + l + 8) * sc / 16.0;"),
    "scale group index": ("double sc = oracle_half_to_double(scale_row[k / ORACLE_GROUP]);",
                          "double sc = oracle_half_to_double(scale_row[(k / ORACLE_GROUP) / 2]);"),
    "scale row stride": ("const uint16_t *sr = scale + (size_t)n * G;", "const uint16_t *sr = scale + (size_t)n;"),
    "round half away from zero": ("float rt = nearbyintf(t);", "float rt = roundf(t);"),
    "act scale /128": ("float sc = amax / 127.0f;", "float sc = amax / 128.0f;"),
    "act scale by reciprocal": ("float t = xr[k] / sc;", "float t = xr[k] * (1.0f / sc);"),
    "partials offset dropped": ("acc += (int64_t)q[(size_t)m * K + k] * (int64_t)(nibble_at(row, k) - 8);",
                                "acc += (int64_t)q[(size_t)m * K + k] * (int64_t)(nibble_at(row, k));"),
    "p8 factor 8": ("int64_t v = 16 * (int64_t)p_hi[i] + (int64_t)p_lo[i];",
                    "int64_t v = 8 * (int64_t)p_hi[i] + (int64_t)p_lo[i];"),
    "group act scale index": ("double sa = act_group ? (double)xs[(size_t)m * G + k / ORACLE_GROUP]",
                              "double sa = act_group ? (double)xs[(size_t)m * G]"),
    "half exponent bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "plane row stride": ("const uint8_t *hr = hi + (size_t)n * (K / 2);", "const uint8_t *hr = hi + (size_t)n * (K / 4);"),
    "hadamard difference reversed": ("z[i + h] = a - c;", "z[i + h] = c - a;"),
    "hadamard difference dropped": ("z[i + h] = a - c;", "z[i + h] = a + c;"),
    "hadamard normalisation dropped": ("z[i] = z[i] * rb;", "z[i] = z[i];"),
    "hadamard normalisation 1/sqrt(b/2)": ("(float)(1.0 / sqrt((double)block))", "(float)(1.0 / sqrt((double)block / 2))"),
    "hadamard first stage skipped": ("for (int h = 1; h < block; h *= 2)", "for (int h = 2; h < block; h *= 2)"),
    "hadamard last stage skipped": ("for (int h = 1; h < block; h *= 2)", "for (int h = 1; h < block / 2; h *= 2)"),
    "hadamard input block offset": ("const float *xr = x + (size_t)m * K + b0;", "const float *xr = x + (size_t)m * K;"),
    "pack scale amax/7": ("oracle_float_to_half(amax / 7.5f)", "oracle_float_to_half(amax / 7.0f)"),
    "pack rounding half away": ("    float r = nearbyintf(t);\n    if (r < (float)lo)", "    float r = roundf(t);\n    if (r < (float)lo)"),
    "pack residual step s/8": ("float s16th = s / 16.0f;", "float s16th = s / 8.0f;"),
    "pack nibble order": ("int shift = (k % 2 == 0) ? 0 : 4;", "int shift = (k % 2 == 0) ? 4 : 0;"),
    "pack hi zero point 7": ("hi[byte] |= (uint8_t)((ch + 8) << shift);", "hi[byte] |= (uint8_t)((ch + 7) << shift);"),
    "pack residual from W": ("float r = w[k] - (float)ch * s;", "float r = w[k];"),
    "pack hi clamp -7": ("ch = rne_clamp(w[k] / s, -8, 7);", "ch = rne_clamp(w[k] / s, -7, 7);"),
    "half conversion truncates": ("float q = nearbyintf(ldexpf(m, 11));", "float q = floorf(ldexpf(m, 11));"),
    "half subnormal truncates": ("float q = nearbyintf(a * 0x1p24f);", "float q = floorf(a * 0x1p24f);"),
    "accept argmax ties to the last": ("if (row[v] > row[best]) best = v;", "if (row[v] >= row[best]) best = v;"),
    "accept next token off by one": ("*next = targ[n];", "*next = targ[n < R - 1 ? n + 1 : n];"),
    "accept counts all matches": ("while (n < R - 1 && draft[n] == targ[n]) ++n;",
                                  "for (int r = 0; r < R - 1; ++r) n += draft[r] == targ[r];"),
    "accept compares with the next row": ("while (n < R - 1 && draft[n] == targ[n]) ++n;",
                                          "while (n < R - 1 && draft[n] == targ[n + 1]) ++n;"),
    "kv grouped heads interleaved": ("const int hk = h / G;", "const int hk = h % Hkv;"),
    "kv score scale dropped": ("double p = exp(sc * inv_sqrt_d - mx);", "double p = exp(sc - mx);"),
    "kv causal off by one": ("const int visible = T - M + i + 1;", "const int visible = T - M + i;"),
    "kv sees the whole cache": ("const int visible = T - M + i + 1;", "const int visible = T;"),
    "kv8 residual offset 7": ("int cl = nibble_at(lo + row * (ORACLE_HEAD_DIM / 2), j) - 8;",
                              "int cl = nibble_at(lo + row * (ORACLE_HEAD_DIM / 2), j) - 7;"),
    "kv scale head-major": ("const size_t row = (size_t)t * Hkv + h;\n    const uint8_t *hr = hi + row * (ORACLE_HEAD_DIM / 2);\n    double s = oracle_half_to_double(scale[row]);",
                            "const size_t row = (size_t)t * Hkv + h;\n    const uint8_t *hr = hi + row * (ORACLE_HEAD_DIM / 2);\n    double s = oracle_half_to_double(scale[(size_t)h * Hkv + t % Hkv]);"),
}


def _all_pins():
    out = []
    for name, fn in sorted(vars(pins).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = getattr(fn, "pytestmark", [])
        grid = [{}]
        for mark in params:
            if mark.name == "parametrize":
                argname, values = mark.args[0], mark.args[1]
                grid = [dict(g, **{argname: v}) for g in grid for v in values]
        out.append((name, fn, grid))
    return out


def _fails(golden_dir):
    failed = []
    for name, fn, grid in _all_pins():
        for kw in grid:
            args = dict(kw)
            if "golden_dir" in inspect.signature(fn).parameters:
                args["golden_dir"] = golden_dir
            try:
                fn(**args)
            except Exception:
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, tmp_path, monkeypatch, golden_dir):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: %s" % mutant
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c99", "-D_GNU_SOURCE",
                    "-fPIC", "-shared", str(msrc), "-o", str(lib), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB", str(lib))
    monkeypatch.setattr(oracle, "_SRC", str(msrc))
    try:
        failed = _fails(golden_dir)
    finally:
        monkeypatch.setattr(oracle, "_lib", None)
    assert failed, "no pin caught the mutant '%s'" % mutant


def test_unmutated_oracle_passes_every_pin(golden_dir):
    assert _fails(golden_dir) == []
