"""The seeded input generator: Philox known answers, the normal variate,
the fp16 rounding, and the structure of generated requests."""
import os

import numpy as np
import pytest

import synth
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(x, 16) for x in line.split()]
        assert synth.philox4x32_10(v[0:4], v[4:6]) == v[6:10]
        n += 1
    assert n == 3


def test_normal_variate_moments_and_support():
    nums = np.array([synth.normal_numerator(0, 1, 7, i) for i in range(20000)])
    x = nums / 65536.0
    assert np.all(np.abs(nums) <= 393210)
    assert abs(x.mean()) < 0.03
    assert abs(x.var() - 1.0) < 0.05
    # bulk host generation equals the per-element definition
    kv = synth.fact_kv(0, 1, 7, 20000, synth.F32)
    assert np.array_equal(kv, x.astype(np.float32))


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.normal(size=5000), rng.normal(size=5000) * 1e-5,
                         rng.uniform(-7e4, 7e4, size=2000),
                         [0.0, -0.0, 2.0**-25, 1.5 * 2.0**-24, 65504.0, 65519.99]])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([synth.double_to_f16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_kv_range_matches_per_fact():
    lens = np.array([3, 1, 5], dtype=np.int32)
    row = 2 * 2 * 8
    for dt in (synth.F32, synth.BF16):
        packed = synth.kv_range(0, 2, 4, lens, row, dt)
        off = 0
        for j, n in enumerate(lens):
            one = synth.fact_kv(0, 2, 4 + j, int(n) * row, dt)
            assert np.array_equal(packed[off:off + n * row], one)
            off += n * row


def test_block_tables_disjoint_and_sufficient():
    need = np.array([17, 1, 64, 200, 33], dtype=np.int64)
    bt = synth.block_tables(3, need, 16, 64)
    used = bt[bt >= 0]
    assert len(used) == len(set(used.tolist()))
    for r, n in enumerate(need):
        assert (bt[r] >= 0).sum() == -(-n // 16)
    with pytest.raises(ValueError):
        synth.block_tables(3, np.array([2000], dtype=np.int64), 16, 64)


def test_zipf_distinct_and_skewed():
    ids = synth.zipf_requests(0, 200, 50, 10000, 1.1)
    for row in ids:
        assert len(set(row.tolist())) == 50
    assert ids.min() >= 0 and ids.max() < 10000
    counts = np.bincount(ids.ravel(), minlength=10000)
    assert counts[0] == 200          # the most likely id is drawn in every request
    assert counts[:10].sum() > counts[5000:].sum()


def test_embeddings_unit_norm_and_queries():
    e = synth.embeddings(0, 0, 50, 64).view(np.float16).astype(np.float64)
    assert np.allclose(np.linalg.norm(e, axis=1), 1.0, atol=2e-3)
    q = synth.queries(0, 4, 64).view(np.float16).astype(np.float64)
    assert 0.5 < q.std() < 1.5


def test_workload_shapes():
    w = W.WORKLOADS["tiny"]
    lens = W.fact_lengths(w)
    assert lens.min() >= 8 and lens.max() <= 24 and len(lens) == 20
    w = W.WORKLOADS["mistral7b_batch"]
    lens = W.fact_lengths(w)
    assert lens.min() >= 8 and lens.max() <= 256
    assert 30 < np.median(lens) < 34


def test_sentinel_host_deterministic():
    a = synth.sentinel_host(5, 1 << 33, 100)
    b = synth.sentinel_host(5, (1 << 33) + 50, 50)
    assert np.array_equal(a[50:], b)
    assert len(set(a.tolist())) > 95
