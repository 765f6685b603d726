"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of oracle/engram_oracle.c (a
dropped term, a wrong sign, index or rounding, a transposed operand), builds
it with gcc into a temporary library, and runs the pin file that covers that
function against the mutant in a fresh interpreter: the pins must fail.  The
unmutated copy, built the same way, must pass the same files, so a failure
is the planted mistake's doing.  Everything runs on the CPU.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "engram_oracle.c")

HASH, DEQ, WKV_GATE, OUT, MX, FMT = ("tests/test_oracle_hash.py", "tests/test_oracle_dequant.py",
                                     "tests/test_oracle_wkv_gate.py", "tests/test_oracle_gate_output.py",
                                     "tests/test_oracle_mx.py", "tests/test_oracle_scale_formats.py")

# name -> (text in the oracle, planted replacement, pin file that must fail)
MUTANTS = {
    "blocking_not_cumulative": ("if (p < s || source == dead) blocked = 1;",
                                "blocked = (p < s || source == dead);", HASH),
    "truncating_modulo": ("if (r != 0 && ((r < 0) != (p < 0))) r += p;", "(void)0;", HASH),
    "sequence_start_not_blocking": ("if (p < s || source == dead) blocked = 1;",
                                    "if (source == dead) blocked = 1;", HASH),
    "columns_head_outer": ("const int col = (i - 1) * H + h;", "const int col = h * (N - 1) + (i - 1);", HASH),
    "offsets_dropped": ("floor_mod(rolling, prime) + offsets[e * C + col]", "floor_mod(rolling, prime)", HASH),
    "first_product_dropped": ("int64_t rolling = products[0];", "int64_t rolling = 0;", HASH),
    "subnormal_exponent": ("ldexpf((float)mant, -9)", "ldexpf((float)mant, -10)", DEQ),
    "exponent_bias": ("ldexpf((float)(8 + mant), expo - 10)", "ldexpf((float)(8 + mant), expo - 11)", DEQ),
    "fnuz_nan": ("if (expo == 0xF && mant == 0x7) return NAN;", "if (byte == 0x80) return NAN;", DEQ),
    "scale_block_index": ("* sc[j / blk];", "* sc[(j / blk) ^ (S > 1)];", DEQ),
    "bf16_truncates": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;", "(void)rest;", DEQ),
    "bf16_ties_away": ("(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u)", DEQ),
    "invalid_rows_not_zeroed": ("out_bf16[o * D + j] = masked ? 0 : oracle_bf16_rne(prod);",
                                "out_bf16[o * D + j] = oracle_bf16_rne(prod);", DEQ),
    "w_transposed": ("w[(int64_t)o * K + k]", "w[(int64_t)k * Nout + o]", WKV_GATE),
    "dim_rsqrt_dropped": ("dot[t * hc + c] = hwk * rstd / sqrt((double)dim);", "dot[t * hc + c] = hwk * rstd;",
                          WKV_GATE),
    "weight_product_dropped": ("hwk += hv * wv * kv_;", "hwk += hv * kv_;", WKV_GATE),
    "key_rms_uses_stream": ("kk += kv_ * kv_;", "kk += hv * hv;", WKV_GATE),
    "eps_outside_sqrt": ("(1.0 / sqrt(hh / dim + eps))", "(1.0 / sqrt(hh / dim) + eps)", WKV_GATE),
    "signed_sqrt_dropped": ("const double mag = sqrt(fmax(fabs(d), 1e-6));", "const double mag = fmax(fabs(d), 1e-6);",
                            OUT),
    "clamp_dropped": ("sqrt(fmax(fabs(d), 1e-6))", "sqrt(fabs(d))", OUT),
    "mask_ignored": ("if (token_mask && !token_mask[t]) g = 0.0;", "(void)token_mask;", OUT),
    "value_of_copy_0": ("const uint16_t* value = kv + t * ld_kv + (int64_t)hc * dim;",
                        "const uint16_t* value = kv + t * ld_kv;", OUT),
    "e8m0_bias": ("return ldexp(1.0, (int)s - 127);", "return ldexp(1.0, (int)s - 128);", MX),
    "e4m3_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) return fl + 1.0;",
                       "if (frac >= 0.5) return fl + 1.0;", MX),
    "e4m3_no_saturation": ("if (m >= 448.0) return sign | 0x7E;", "if (m >= 464.0) return sign | 0x7F;", MX),
    "mx_exponent_ceil": ("shared = (e - 1) - 8;", "shared = e - 8;", MX),
    "mx_zero_block_exponent": ("int shared = -127;", "int shared = 0;", MX),
    "mx_sign_dropped": ("oracle_e4m3fn_encode_sat(ldexp(oracle_bf16_to_double(xb[k]), -shared))",
                        "oracle_e4m3fn_encode_sat(ldexp(fabs(oracle_bf16_to_double(xb[k])), -shared))", MX),
    "mx_subnormal_quantum": ("const int n = (int)round_half_even(m / ldexp(1.0, -9));",
                             "const int n = (int)round_half_even(m / ldexp(1.0, -8));", MX),
    "fmt_e4m3_scale_read_as_e8m0": ("sv = oracle_e4m3fn_decode(((const uint8_t*)scale)[si]);",
                                    "sv = (float)oracle_e8m0_decode(((const uint8_t*)scale)[si]);", FMT),
    "fmt_int32_ids_as_int16": ("(int64_t)((const int32_t*)hash_ids)[at]", "(int64_t)((const int16_t*)hash_ids)[at]",
                               FMT),
    "fmt_scale_in_double": ("const float prod = oracle_e4m3fn_decode(w[j]) * sv;",
                            "const float prod = (float)((double)oracle_e4m3fn_decode(w[j]) * (double)sv + 0x1p-40);",
                            FMT),
    "wkv_mx_first_block_scale": ("acc += oracle_e8m0_decode(a_s[t * nb + b])", "acc += oracle_e8m0_decode(a_s[t * nb])",
                                 MX),
}

_RUNNER = ("import sys; sys.path.insert(0, {root!r}); import oracle; oracle.LIB_PATH = sys.argv[1]; "
           "import pytest; sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu'] + sys.argv[2:]))")


def _build(src_text: str, out_dir: str, name: str) -> str:
    c_path = os.path.join(out_dir, name + ".c")
    with open(c_path, "w") as f:
        f.write(src_text)
    so = os.path.join(out_dir, name + ".so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), "-o", so, c_path, "-lm"], check=True)
    return so


def _pins(so: str, files) -> subprocess.CompletedProcess:
    env = dict(os.environ, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT), so, *files], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_planted_mistakes_fail_their_pins(tmp_path):
    src = open(SRC).read()
    for name, (old, new, _) in MUTANTS.items():
        assert src.count(old) == 1, f"{name}: the text to mutate must occur once in the oracle"
    builds = {"unmutated": _build(src, str(tmp_path), "unmutated")}
    for name, (old, new, _) in MUTANTS.items():
        builds[name] = _build(src.replace(old, new), str(tmp_path), name)
    files = sorted({f for _, _, f in MUTANTS.values()})
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        base = pool.submit(_pins, builds["unmutated"], files)
        runs = {name: pool.submit(_pins, builds[name], [f]) for name, (_, _, f) in MUTANTS.items()}
        r = base.result()
        assert r.returncode == 0, "the unmutated copy must pass its pins:\n" + r.stdout[-3000:]
        survivors = [name for name, fut in runs.items() if fut.result().returncode == 0]
    assert not survivors, f"planted mistakes the pins did not catch: {survivors}"


@pytest.mark.parametrize("name", ["truncating_modulo", "bf16_truncates"])
def test_a_mutant_fails_for_the_planted_reason(tmp_path, name):
    """Spot check that the pins fail on a numeric mismatch, not on a crash or a build problem."""
    src = open(SRC).read()
    old, new, f = MUTANTS[name]
    r = _pins(_build(src.replace(old, new), str(tmp_path), name), [f])
    assert r.returncode == 1, r.stdout[-2000:]  # pytest: tests failed (not an internal error or a crash)
    assert "AssertionError" in r.stdout or "assert" in r.stdout
