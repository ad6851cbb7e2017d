"""The pins must catch plausible mistakes: each case plants one mistake in a
copy of the oracle's source (on the CPU only), builds it, and checks that
the pin suite fails against that build."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "rotation_sign": ("y[i] = x[i] * c - x[i + h] * s;", "y[i] = x[i] * c + x[i + h] * s;"),
    "rotation_pairing": ("y[i + h] = x[i + h] * c + x[i] * s;",
                         "y[i + h] = x[i + h] * c + x[(i + 1) % h] * s;"),
    "freq_index": ("pow(theta, -2.0 * i / d)", "pow(theta, -2.0 * (i + 1) / d)"),
    "llama3_blend": ("(1.0 - smooth) * f / factor + smooth * f",
                     "smooth * f / factor + (1.0 - smooth) * f"),
    # a blend that is linear in the wavelength: same values at both band edges,
    # monotone, strictly inside (f/8, f), but not the published rule inside
    "llama3_blend_in_wavelength": ("const double smooth = (orig / wavelen - low) / (high - low);",
                                   "const double smooth = (orig / low - wavelen) / "
                                   "(orig / low - orig / high);"),
    "bf16_ties_away": ("nearbyint(x / quantum) * quantum", "floor(x / quantum + 0.5) * quantum"),
    "topk_tie_order": ("return (x->id > y->id) - (x->id < y->id);",
                       "return (x->id < y->id) - (x->id > y->id);"),
    "segment_offset": ("start[j] = pos;\n      pos += fact_len[fact_ids[j]];",
                       "pos += fact_len[fact_ids[j]];\n      start[j] = pos;"),
    "slot_in_block": ("const int64_t in_blk = p % block_size;",
                      "const int64_t in_blk = (p + 1) % block_size;"),
    "half_exponent": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "value_source": ("copy_elem(v_cache, dst + i, v_store, src + i, dtype);",
                     "copy_elem(v_cache, dst + i, k_store, src + i, dtype);"),
    "attend_scale": ("const double scale = 1.0 / sqrt((double)d);",
                     "const double scale = 1.0 / (double)d;"),
    "attend_kv_head": ("const int64_t kvh = hq / g;", "const int64_t kvh = hq % n_kv_heads;"),
    "attend_query_position": ("or_rotate(x, d, (double)qpos[r] + t, f, qr);",
                              "or_rotate(x, d, (double)qpos[r], f, qr);"),
    "attend_value_source": ("* load_elem(v_cache, vb + i, dtype);",
                            "* load_elem(k_cache, vb + i, dtype);"),
    "ingest_window": ("(w + len[i]) + w + t) * d;", "(w + len[i]) + t) * d;"),
    "ingest_row_stride": ("const int64_t s_row = ((int64_t)(l * n_heads + h) * (w + len[i])",
                          "const int64_t s_row = ((int64_t)(l * n_heads + h) * (len[i])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "oracle_mutant.c")
        so = os.path.join(tmp, "liboracle_mutant.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", c,
                        "-o", so, "-lm"], check=True, capture_output=True)
        env = dict(os.environ, ORACLE_SO=so, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           env=env, capture_output=True, text=True, cwd=ROOT)
        assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
