"""The oracle's pins must be able to fail: each case below plants one
plausible mistake in a copy of oracle/oracle.c (a dropped scale, gamma or
RMS factor, a scale read at the wrong index, a wrong sign, split or
summation order), builds it with the oracle's own flags, and runs the pin
suites against that build.  Every mutant must fail at least one pin.

Only copies are changed, in a temporary directory, on the CPU; the in-tree
oracle is untouched.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_norm_rope_pins.py", "tests/test_cache_pins.py"]

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("w8_drop_sx", "(float)(int32_t)acc1[n] * sx;", "(float)(int32_t)acc1[n];", 0),
    ("w8_drop_swa", "A[n] = a * swa[n];", "A[n] = a;", 0),
    ("w8_swa_col0", "A[n] = a * swa[n];", "A[n] = a * swa[0];", 0),
    ("w8_drop_gamma", "z[j] = c[j] * gamma[j];", "z[j] = c[j];", 0),
    ("w8_drop_sz", "(((float)(int32_t)acc2[m] * sz) * inv_t) * swb[m]",
     "((float)(int32_t)acc2[m] * inv_t) * swb[m]", 0),
    ("w8_drop_inv_in_B", "(((float)(int32_t)acc2[m] * sz) * inv_t) * swb[m]",
     "((float)(int32_t)acc2[m] * sz) * swb[m]", 0),
    ("w8_drop_swb", "(((float)(int32_t)acc2[m] * sz) * inv_t) * swb[m]",
     "(((float)(int32_t)acc2[m] * sz) * inv_t)", 0),
    ("w8_swb_col0", "(((float)(int32_t)acc2[m] * sz) * inv_t) * swb[m]",
     "(((float)(int32_t)acc2[m] * sz) * inv_t) * swb[0]", 0),
    ("w8_ckv_no_inv", "ckv[t * r + j] = z[j] * inv_t;", "ckv[t * r + j] = z[j];", 0),
    ("w8_rms_of_z", "const float inv_t = rms_inv(c, r, epsf);",
     "const float inv_t = rms_inv(z, r, epsf);", 0),
    ("w8_token0_scale", "quantize_row(X + t * H, H, qx)", "quantize_row(X, H, qx)", 0),
    ("w8_ties_away", "float rq = rintf(s);", "float rq = roundf(s);", 0),
    ("fp_drop_gamma", "y[j] = (c[j] * inv) * gamma[j];", "y[j] = c[j] * inv;", 0),
    ("fp_no_latent_rounding", "y[j] = (float)round_dtype((double)y[j], dtype);",
     "y[j] = y[j];", 0),
    ("fp_split_swapped", "const float* p = A + r;", "const float* p = A;", 0),
    ("w8_split_swapped", "const float* p = A + r;", "const float* p = A;", 1),
    ("kv_a_descending", "for (int64_t k = 0; k < H; ++k) {\n        const float xk",
     "for (int64_t k = H - 1; k >= 0; --k) {\n        const float xk", 0),
    ("rms_eps_outside_root", "1.0f / sqrtf(ss / (float)r + eps)",
     "1.0f / (sqrtf(ss / (float)r) + eps)", 0),
    ("rms_mean_r_plus_1", "1.0f / sqrtf(ss / (float)r + eps)",
     "1.0f / sqrtf(ss / (float)(r + 1) + eps)", 0),
    ("rope_sign", "out[i] = lo * cs - hi * sn;", "out[i] = lo * cs + hi * sn;", 0),
    ("rope_pairing", "hi = p[i + half];", "hi = p[half - 1 - i];", 0),
    ("rope_freq_ladder", "pow(theta, -2.0 * (double)i / (double)dr)",
     "pow(theta, -1.0 * (double)i / (double)dr)", 0),
    ("value_slice", "value[h * dv + e] = row[dn + e];", "value[h * dv + e] = row[e];", 0),
    ("cache_rope_slot", "cache[s * W + r + i] = kpe[t * dr + i];",
     "cache[s * W + i] = kpe[t * dr + i];", 0),
]


def _mutate(text, old, new, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


def _build_and_run(case, tmp):
    name, old, new, occ = case
    with open(SRC) as f:
        text = f.read()
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(_mutate(text, old, new, occ))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", src, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, MLA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-2000:]


def test_every_mutant_is_applied_once_where_expected():
    with open(SRC) as f:
        text = f.read()
    for name, old, _new, occ in MUTANTS:
        assert text.count(old) >= occ + 1, name


def test_unmutated_copy_passes(tmp_path):
    rc, out = _build_and_run(("identity", "", "", 0), str(tmp_path))
    assert rc == 0, out


def test_every_mutant_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        res = list(ex.map(lambda c: (c[0], _build_and_run(c, str(tmp_path))), MUTANTS))
    survivors = [name for name, (rc, _out) in res if rc == 0]
    assert not survivors, f"mutants that passed every pin: {survivors}"
