"""Boundaries of the product path, checked on the CPU:
  - the bench's GPU legs and the test harness load no part of the oracle
    (only the bench's CPU-baseline leg imports it, inside that function);
  - the binding fails loudly when the HIP library is missing, with no
    fallback;
  - the bench reports HBM traffic only from counters taken on the current
    inject kernel source."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _python(code: str, env=None) -> str:
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       env={**os.environ, **(env or {})}, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.strip()


def test_bench_and_harness_do_not_load_the_oracle():
    out = _python("import sys; sys.path.insert(0, '.'); import bench; "
                  "from tests import harness; "
                  "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    assert out == "False"


def test_missing_library_raises_instead_of_falling_back():
    out = _python("import sys; sys.path.insert(0, '.'); import kv_cache_injection_is_amd as K\n"
                  "try:\n    K.lib()\n    print('loaded')\n"
                  "except K.ISError as e:\n    print('raised', e.code)",
                  env={"INFERSCALE_SO": os.path.join(ROOT, "no_such_library.so")})
    assert out.startswith("raised")


def test_traffic_is_reported_only_for_the_counted_kernel(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    if not os.path.exists(bench.COUNTERS):
        pytest.skip("no counter summary")
    alg = 47249358848
    assert bench.traffic_from_counters(alg) is not None   # the committed kernel
    changed = tmp_path / "inject.hip"
    changed.write_bytes(open(bench.INJECT_SRC, "rb").read() + b"\n// changed\n")
    monkeypatch.setattr(bench, "INJECT_SRC", str(changed))
    assert bench.traffic_from_counters(alg) is None
