"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each check uses something other than the oracle's own formula: closed
forms, invariants (rotation composition, the Theorem 6 relative-position
property, shift invariance), an independent form of the same map (complex
multiplication, the explicit block-rotation matrix), library routines
(numpy float16, torch's float32 -> bfloat16) and brute force on tiny inputs
(exact rational arithmetic, token-by-token walks of the block table).

Pages: "InferScale: GPU-Native KV Injection for Personalized LLM Serving"
(gist.science explainer), technical summary -- Online phase (pre-RoPE
storage, dynamic rotation, Theorem 6, scatter-copy injection) and
Contributions (retrieve-and-inject, Theorem 3; GPU-resident retrieval).
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

RNG = np.random.default_rng(12345)


# ------------------------------------------------------------------ numbers

def test_half_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _bf16_table():
    """All finite non-negative bf16 values, as exact fractions, sorted."""
    vals = []
    for b in range(0x7F80):
        f = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        vals.append((Fraction(float(f)), b))
    vals.sort()
    return vals


_TABLE = None


def _bf16_brute(x: float) -> int:
    """Nearest bf16 by table search; ties to the even significand."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _bf16_table()
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    fx = Fraction(abs(x))
    keys = [v for v, _ in _TABLE]
    i = bisect.bisect_left(keys, fx)
    cands = []
    for j in (i - 1, i):
        if 0 <= j < len(_TABLE):
            cands.append(_TABLE[j])
    best = min(cands, key=lambda vb: (abs(vb[0] - fx), vb[1] & 1))
    return sign | best[1]


def test_bf16_rounding_single_rounding_brute_force():
    xs = list(RNG.normal(size=300)) + list(RNG.normal(size=100) * 1e-3)
    # exact ties and just-above-tie values (a double->float->bf16 path fails these)
    for b in (0x3F80, 0x3F81, 0x4000, 0x3E55, 0xC0A3 & 0x7FFF):
        lo = float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
        hi = float(np.array([(b + 1) << 16], dtype=np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        xs += [mid, -mid, mid + (hi - lo) * 2.0**-30, mid - (hi - lo) * 2.0**-30]
    for x in xs:
        assert oracle.double_to_bf16(float(x)) == _bf16_brute(float(x)), x


def test_bf16_rounding_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    x = torch.randn(20000, dtype=torch.float32) * 3
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(v)) for v in x.numpy()], dtype=np.uint16)
    assert np.array_equal(got, ref)


# -------------------------------------------------------------- frequencies

def test_unscaled_frequencies_closed_form():
    for d, theta in ((64, 1e4), (128, 5e5), (128, 1e6)):
        f = oracle.rope_freqs(d, theta)
        assert f[0] == 1.0
        ref = 1.0 / theta ** (np.arange(0, d, 2, dtype=np.float64) / d)
        assert np.allclose(f, ref, rtol=1e-14, atol=0)
        ratios = f[1:] / f[:-1]
        assert np.allclose(ratios, theta ** (-2.0 / d), rtol=1e-13)


def test_llama3_scaling_bands():
    d, theta = 128, 500000.0
    f = oracle.rope_freqs(d, theta)
    g = oracle.rope_freqs(d, theta, "llama3", 8.0, 1.0, 4.0, 8192.0)
    lam = 2 * np.pi / f
    kept = lam < 8192 / 4
    divided = lam > 8192 / 1
    mid = ~kept & ~divided
    assert (kept.sum(), mid.sum(), divided.sum()) == (29, 6, 29)
    assert np.array_equal(g[kept], f[kept])
    assert np.array_equal(g[divided], f[divided] / 8.0)
    # the blended band lies strictly between f/8 and f, and the map is monotone
    assert np.all(g[mid] < f[mid]) and np.all(g[mid] > f[mid] / 8.0)
    assert np.all(np.diff(g) < 0)


def test_llama3_scaling_interior_closed_form():
    """Inside the blended band the published Llama-3.1 rule moves the
    multiplier f'/f from 1/factor to 1 in proportion to how far orig/lambda
    has moved from `low` to `high`.  At lambda = 4096, orig/lambda = 2, one
    third of the way from 1 to 4: f' = (2/3)(f/8) + (1/3)f = 5f/12.  At
    lambda = 3072, orig/lambda = 8/3, five ninths of the way:
    f' = (4/9)(f/8) + (5/9)f = 11f/18.  At lambda = 6553.6, orig/lambda =
    1.25, one twelfth: f' = (11/12)(f/8) + f/12 = 19f/96."""
    for lam, ratio in ((4096.0, 5 / 12), (3072.0, 11 / 18), (6553.6, 19 / 96)):
        f = 2 * math.pi / lam
        assert oracle.llama3_scale(f) == pytest.approx(ratio * f, rel=1e-13)
    # other parameters: factor 4, low 2, high 8, orig 16384; lambda = 4096 gives
    # orig/lambda = 4, one third of the way from 2 to 8: f' = (2/3)(f/4) + f/3 = f/2
    f = 2 * math.pi / 4096.0
    assert oracle.llama3_scale(f, 4.0, 2.0, 8.0, 16384.0) == pytest.approx(f / 2, rel=1e-13)


def test_llama3_scaling_multiplier_affine_in_frequency():
    """orig/lambda = orig f / 2pi is proportional to f, so across the band the
    multiplier f'/f is an affine function of f itself: 1/8 at the band's
    low-frequency edge (lambda = 8192) and 1 at its high-frequency edge
    (lambda = 2048).  Checked on the six blended frequencies of d = 128,
    theta = 5e5 and on a dense sweep of the band."""
    f_lo, f_hi = 2 * math.pi / 8192.0, 2 * math.pi / 2048.0
    f = oracle.rope_freqs(128, 500000.0)
    lam = 2 * np.pi / f
    band = f[(lam >= 2048) & (lam <= 8192)]
    sweep = np.linspace(f_lo, f_hi, 101)[1:-1]
    for ff in list(band) + list(sweep):
        m = oracle.llama3_scale(float(ff)) / ff
        assert m == pytest.approx(1 / 8 + (7 / 8) * (ff - f_lo) / (f_hi - f_lo), rel=1e-12)


def test_llama3_scaling_continuous_at_band_edges():
    for lam_edge, expect in ((2048.0, 1.0), (8192.0, 1 / 8.0)):
        f = 2 * np.pi / lam_edge
        for eps in (1e-9, -1e-9):
            ff = f * (1 + eps)
            assert oracle.llama3_scale(ff) == pytest.approx(expect * ff, rel=1e-8)


# ------------------------------------------------------------------ rotation

def _rot_matrix(d, p, f):
    """Explicit block rotation for rotate-half pairing (i, i + d/2)."""
    h = d // 2
    R = np.zeros((d, d))
    for i in range(h):
        c, s = math.cos(p * f[i]), math.sin(p * f[i])
        R[i, i], R[i, i + h] = c, -s
        R[i + h, i], R[i + h, i + h] = s, c
    return R


def test_rotation_position_zero_is_identity():
    f = oracle.rope_freqs(128, 5e5, "llama3")
    x = RNG.normal(size=128)
    assert np.array_equal(oracle.rotate(x, 0, f), x)


def test_rotation_first_pair_turns_by_p_radians():
    f = oracle.rope_freqs(64, 1e4)
    x = RNG.normal(size=64)
    for p in (1, 7, 1000, 13055):
        y = oracle.rotate(x, p, f)
        assert y[0] == pytest.approx(x[0] * math.cos(p) - x[32] * math.sin(p), abs=1e-12)
        assert y[32] == pytest.approx(x[32] * math.cos(p) + x[0] * math.sin(p), abs=1e-12)


def test_rotation_d2_is_plane_rotation():
    f = np.array([1.0])
    for p in (0.5, 3.0, -2.0, 100.0):
        x = RNG.normal(size=2)
        c, s = math.cos(p), math.sin(p)
        ref = np.array([[c, -s], [s, c]]) @ x
        assert np.allclose(oracle.rotate(x, p, f), ref, atol=1e-14)


def test_rotation_equals_complex_multiplication():
    d = 128
    f = oracle.rope_freqs(d, 1e6)
    x = RNG.normal(size=d)
    for p in (1, 35, 3455, 13055):
        z = (x[:64] + 1j * x[64:]) * np.exp(1j * p * f)
        y = oracle.rotate(x, p, f)
        assert np.allclose(y[:64], z.real, atol=1e-12)
        assert np.allclose(y[64:], z.imag, atol=1e-12)


def test_rotation_equals_block_matrix_and_preserves_pair_norms():
    d = 64
    f = oracle.rope_freqs(d, 1e4)
    x = RNG.normal(size=d)
    for p in (3, 135, 2000):
        y = oracle.rotate(x, p, f)
        assert np.allclose(y, _rot_matrix(d, p, f) @ x, atol=1e-12)
        assert np.allclose(y[:32] ** 2 + y[32:] ** 2, x[:32] ** 2 + x[32:] ** 2, atol=1e-12)


def test_rotations_compose():
    f = oracle.rope_freqs(128, 5e5, "llama3")
    x = RNG.normal(size=128)
    for a, b in ((3, 5), (100, 2000), (8191, 4864)):
        two = oracle.rotate(oracle.rotate(x, a, f), b, f)
        assert np.allclose(two, oracle.rotate(x, a + b, f), atol=1e-12)


def test_theorem6_rerotated_key_scores_like_prefilled_key():
    """<R(m) q, R(n) k> with k stored pre-RoPE and re-rotated equals the
    score of a key prefilled at n (explicit matrix), and the
    relative-position form <q, R(n - m) k>."""
    d = 128
    f = oracle.rope_freqs(d, 1e6)
    for _ in range(20):
        q, k = RNG.normal(size=d), RNG.normal(size=d)
        m, n = (int(v) for v in RNG.integers(0, 13056, size=2))
        injected = oracle.rotate(k, n, f)
        prefilled = _rot_matrix(d, n, f) @ k
        s_inj = oracle.rotate(q, m, f) @ injected
        s_pre = (_rot_matrix(d, m, f) @ q) @ prefilled
        s_rel = q @ (_rot_matrix(d, n - m, f) @ k)
        assert abs(s_inj - s_pre) < 1e-9
        assert abs(s_inj - s_rel) < 1e-9


def test_scores_invariant_under_shared_shift():
    d = 128
    f = oracle.rope_freqs(d, 5e5, "llama3")
    for s in (1, 1000, 99999, 100000):
        q, k = RNG.normal(size=d), RNG.normal(size=d)
        m, n = 40, 3000
        a = oracle.rotate(q, m, f) @ oracle.rotate(k, n, f)
        b = oracle.rotate(q, m + s, f) @ oracle.rotate(k, n + s, f)
        assert abs(a - b) < 1e-9


# --------------------------------------------------------------------- top-k

def _brute_topk(qb, eb, k):
    """Exact rational scores, full sort by (-score, id)."""
    qv = [Fraction(float(v)) for v in qb.view(np.float16).astype(np.float64)]
    out = []
    for f in range(eb.shape[0]):
        ev = [Fraction(float(v)) for v in eb[f].view(np.float16).astype(np.float64)]
        out.append((-sum(a * b for a, b in zip(qv, ev)), f))
    out.sort()
    return [f for _, f in out[:k]], [float(-s) for s, _ in out[:k]]


def test_topk_brute_force_tiny():
    e = synth.embeddings(0, 0, 20, 32)
    q = synth.queries(0, 3, 32)
    ids, scores = oracle.topk(q, e, 5)
    for r in range(3):
        bid, bsc = _brute_topk(q[r], e, 5)
        assert ids[r].tolist() == bid
        assert np.allclose(scores[r], bsc, rtol=0, atol=1e-15)


def test_topk_self_query_ranks_first_and_scaling_invariance():
    e = synth.embeddings(1, 0, 500, 64)
    for f in (0, 17, 499):
        ids, s = oracle.topk(e[f:f + 1], e, 3)
        assert ids[0, 0] == f
    q = synth.queries(2, 4, 64)
    q2 = (q.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    i1, s1 = oracle.topk(q, e, 10)
    i2, s2 = oracle.topk(q2, e, 10)
    assert np.array_equal(i1, i2)
    assert np.array_equal(s2, 2 * s1)


def test_topk_ties_go_to_lower_id():
    e = synth.embeddings(3, 0, 50, 32)
    e[40] = e[7]
    e[12] = e[7]
    ids, _ = oracle.topk(e[7:8], e, 3)
    assert ids[0].tolist() == [7, 12, 40]


# ----------------------------------------------------- composition and inject

def test_positions_brute_force():
    lens = np.array([5, 3, 9, 1, 4], dtype=np.int32)
    req_off = np.array([0, 3, 3, 5], dtype=np.int32)
    ids = np.array([2, 0, 4, 1, 1], dtype=np.int32)
    prefix = np.array([7, 2, 0], dtype=np.int32)
    start = oracle.positions(req_off, ids, lens, prefix)
    for r in range(3):
        seq = ["prefix"] * int(prefix[r])
        for j in range(req_off[r], req_off[r + 1]):
            seq += [j] * int(lens[ids[j]])
        for j in range(req_off[r], req_off[r + 1]):
            assert start[j] == seq.index(j)


def _small_problem(dtype, d=64, L=2, H=2, B=8, n_blocks=40, seed=4):
    lens = synth.len_uniform(seed, 12, 1, 13)
    tok_off = np.zeros(13, dtype=np.int64)
    tok_off[1:] = np.cumsum(lens)
    row = L * H * d
    K = synth.kv_range(seed, 1, 0, lens, row, dtype)
    V = synth.kv_range(seed, 2, 0, lens, row, dtype)
    req_off = np.array([0, 4, 5, 9], dtype=np.int32)
    ids = np.array([3, 0, 11, 3, 7, 1, 2, 5, 9], dtype=np.int32)  # a repeat in request 0
    prefix = np.array([5, 0, 13], dtype=np.int32)
    need = np.array([prefix[r] + lens[ids[req_off[r]:req_off[r + 1]]].sum() for r in range(3)])
    bt = synth.block_tables(seed, need, B, n_blocks)
    return dict(lens=lens, tok_off=tok_off, K=K, V=V, req_off=req_off, ids=ids,
                prefix=prefix, bt=bt, L=L, H=H, d=d, B=B, n_blocks=n_blocks)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_inject_brute_force_small(dtype):
    P = _small_problem(dtype)
    L, H, d, B, nb = P["L"], P["H"], P["d"], P["B"], P["n_blocks"]
    f = oracle.rope_freqs(d, 1e4)
    np_t = np.float32 if dtype == synth.F32 else np.uint16
    words = L * nb * B * H * d * (4 if dtype == synth.F32 else 2) // 4
    kc0 = synth.sentinel_host(1, 0, words).view(np_t)
    vc0 = synth.sentinel_host(2, 0, words).view(np_t)
    kc, vc = kc0.copy(), vc0.copy()
    strides = (nb * B * H * d, B * H * d, H * d, d)     # [layer][block][slot][head][d]
    oracle.inject(L, H, d, dtype, P["K"], P["V"], P["tok_off"], P["req_off"], P["ids"],
                  P["prefix"], P["bt"], B, nb, kc, vc, strides, f)
    kc5 = kc.reshape(L, nb, B, H, d)
    vc5 = vc.reshape(L, nb, B, H, d)
    touched = np.zeros((nb, B), dtype=bool)

    def as_f64(a):
        if dtype == synth.F32:
            return a.astype(np.float64)
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    for r in range(3):
        # walk the block table one token at a time
        blk_i, in_blk = 0, 0
        for _ in range(int(P["prefix"][r])):
            in_blk += 1
            if in_blk == B:
                blk_i, in_blk = blk_i + 1, 0
        pos = int(P["prefix"][r])
        for j in range(P["req_off"][r], P["req_off"][r + 1]):
            fid = int(P["ids"][j])
            n = int(P["lens"][fid])
            base = int(P["tok_off"][fid]) * L * H * d
            blk_of = P["bt"][r]
            for t in range(n):
                b = int(blk_of[blk_i])
                assert not touched[b, in_blk] or fid == 3   # the repeated fact rewrites nothing twice
                touched[b, in_blk] = True
                for l in range(L):
                    for h in range(H):
                        src = base + ((l * H + h) * n + t) * d
                        k_pre = as_f64(P["K"][src:src + d])
                        z = (k_pre[:d // 2] + 1j * k_pre[d // 2:]) * np.exp(1j * pos * f)
                        ref = np.concatenate([z.real, z.imag])
                        got = as_f64(kc5[l, b, in_blk, h])
                        if dtype == synth.F32:
                            assert np.allclose(got, ref, rtol=0, atol=2e-6)
                        else:
                            ulp = np.maximum(np.abs(ref), 2.0**-126) * 2.0**-7
                            assert np.all(np.abs(got - ref) <= ulp)
                        assert np.array_equal(vc5[l, b, in_blk, h], P["V"][src:src + d])
                pos += 1
                in_blk += 1
                if in_blk == B:
                    blk_i, in_blk = blk_i + 1, 0
    # every untouched slot keeps its sentinel, bit for bit
    k0 = kc0.reshape(L, nb, B, H, d)
    v0 = vc0.reshape(L, nb, B, H, d)
    mask = ~touched
    for l in range(L):
        assert np.array_equal(kc5[l][mask].view(np.uint8), k0[l][mask].view(np.uint8))
        assert np.array_equal(vc5[l][mask].view(np.uint8), v0[l][mask].view(np.uint8))


def test_inject_rejects_out_of_range_ids():
    P = _small_problem(synth.F32)
    f = oracle.rope_freqs(P["d"], 1e4)
    n = P["L"] * P["n_blocks"] * P["B"] * P["H"] * P["d"]
    kc = np.zeros(n, np.float32)
    vc = np.zeros(n, np.float32)
    ids = P["ids"].copy()
    ids[2] = 99
    with pytest.raises(ValueError):
        oracle.inject(P["L"], P["H"], P["d"], synth.F32, P["K"], P["V"], P["tok_off"],
                      P["req_off"], ids, P["prefix"], P["bt"], P["B"], P["n_blocks"],
                      kc, vc, (1, 1, 1, 1), f)


def test_theorem3_one_layer_attention_injection_equals_prefill():
    """One causal attention layer with RoPE and random weights (fp64): layer-0
    keys and values depend only on the token, so encoding each fact alone,
    storing its pre-RoPE key and raw value, and injecting them at their
    serving positions (oracle composition + rotation) gives the query tokens
    the same outputs as prefilling [prefix | facts | query]."""
    d_model, d, vocab = 48, 32, 97
    Wq, Wk, Wv = (RNG.normal(size=(d, d_model)) / 7 for _ in range(3))
    emb = RNG.normal(size=(vocab, d_model))
    f = oracle.rope_freqs(d, 1e4)
    facts = [RNG.integers(0, vocab, size=n) for n in (4, 7, 2, 5)]
    prefix = RNG.integers(0, vocab, size=6)
    query = RNG.integers(0, vocab, size=3)
    order = np.array([2, 0, 3], dtype=np.int32)

    def attend(qvec, qpos, keys, vals):
        qr = _rot_matrix(d, qpos, f) @ qvec
        s = keys @ qr / math.sqrt(d)
        w = np.exp(s - s.max())
        return (w / w.sum()) @ vals

    # full prefill: every token at its position
    seq = np.concatenate([prefix] + [facts[i] for i in order] + [query])
    K_full = np.stack([_rot_matrix(d, p, f) @ (Wk @ emb[t]) for p, t in enumerate(seq)])
    V_full = np.stack([Wv @ emb[t] for t in seq])
    n_ctx = len(seq) - len(query)
    ref = [attend(Wq @ emb[seq[p]], p, K_full[:p + 1], V_full[:p + 1])
           for p in range(n_ctx, len(seq))]

    # inject: facts encoded alone (pre-RoPE keys), placed by the oracle
    lens = np.array([len(x) for x in facts], dtype=np.int32)
    start = oracle.positions(np.array([0, 3], np.int32), order, lens,
                             np.array([len(prefix)], np.int32))
    Ks, Vs = [], []
    for p, t in enumerate(prefix):
        Ks.append(_rot_matrix(d, p, f) @ (Wk @ emb[t]))
        Vs.append(Wv @ emb[t])
    for j, fid in enumerate(order):
        for t, tok in enumerate(facts[fid]):
            Ks.append(oracle.rotate(Wk @ emb[tok], int(start[j]) + t, f))
            Vs.append(Wv @ emb[tok])
    out = []
    for i, t in enumerate(query):
        p = n_ctx + i
        Ks.append(_rot_matrix(d, p, f) @ (Wk @ emb[t]))
        Vs.append(Wv @ emb[t])
        out.append(attend(Wq @ emb[t], p, np.stack(Ks), np.stack(Vs)))
    assert np.max(np.abs(np.array(out) - np.array(ref))) < 1e-9


def test_token_slots_brute_force_walk():
    P = _small_problem(synth.F32)
    slots = oracle.token_slots(P["req_off"], P["ids"], P["lens"], P["prefix"], P["bt"], P["B"])
    B = P["B"]
    expect = []
    for r in range(3):
        blk_i, in_blk = 0, 0
        for _ in range(int(P["prefix"][r])):
            in_blk += 1
            if in_blk == B:
                blk_i, in_blk = blk_i + 1, 0
        for j in range(P["req_off"][r], P["req_off"][r + 1]):
            for _ in range(int(P["lens"][P["ids"][j]])):
                expect.append(int(P["bt"][r][blk_i]) * B + in_blk)
                in_blk += 1
                if in_blk == B:
                    blk_i, in_blk = blk_i + 1, 0
    assert slots.tolist() == expect
    assert len(set(expect)) == len(expect)


def test_dot_exact_against_fractions():
    a = synth.queries(5, 1, 64)[0]
    b = synth.embeddings(5, 0, 1, 64)[0]
    ref = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in
              zip(a.view(np.float16).astype(np.float64), b.view(np.float16).astype(np.float64)))
    assert oracle.dot(a, b) == pytest.approx(float(ref), abs=1e-15)


# -------------------------------------------------------------- attention
# Query-only attention over the paged cache (the step after injection).

def _nhd(L, nb, B, H, d):
    return (nb * B * H * d, B * H * d, H * d, d)


def test_attention_single_position_returns_its_value():
    L, H, Hq, d, B, nb = 2, 2, 4, 8, 4, 6
    rng = np.random.default_rng(11)
    kc = rng.normal(size=(L, nb, B, H, d)).astype(np.float32)
    vc = rng.normal(size=(L, nb, B, H, d)).astype(np.float32)
    q = rng.normal(size=(L, 1, 3, Hq, d)).astype(np.float32)
    bt = np.array([[3, 1, 5]], np.int32)
    f = oracle.rope_freqs(d, 1e4)
    out = oracle.attend(L, H, Hq, d, synth.F32, q, [9], [6], [7], bt, B, nb, kc, vc,
                        _nhd(L, nb, B, H, d), f)
    for l in range(L):
        for hq in range(Hq):
            # position 6: block bt[0][1] = 1, slot 2; kv head hq // 2
            assert np.array_equal(out[l, 0, :, hq], np.tile(vc[l, 1, 2, hq // 2], (3, 1)))


def test_attention_zero_query_averages_values_and_empty_context_is_zero():
    L, H, Hq, d, B, nb = 1, 1, 2, 16, 4, 8
    rng = np.random.default_rng(12)
    kc = rng.normal(size=(L, nb, B, H, d)).astype(np.float32)
    vc = rng.normal(size=(L, nb, B, H, d)).astype(np.float32)
    bt = np.array([[7, 2, 4, 0], [1, 3, 5, 6]], np.int32)
    q = np.zeros((L, 2, 2, Hq, d), np.float32)
    f = oracle.rope_freqs(d, 1e4)
    out = oracle.attend(L, H, Hq, d, synth.F32, q, [12, 12], [1, 5], [10, 5], bt, B, nb, kc, vc,
                        _nhd(L, nb, B, H, d), f)
    rows = [vc[0, bt[0, p // B], p % B, 0].astype(np.float64) for p in range(1, 10)]
    assert np.allclose(out[0, 0], np.mean(rows, axis=0), atol=1e-12, rtol=0)
    assert np.array_equal(out[0, 1], np.zeros((2, Hq, d)))


def test_attention_two_positions_logistic_weights():
    """At position 0 RoPE is the identity; two context keys give weights
    1 / (1 + exp(s2 - s1)) with s = <q, k> / sqrt(d)."""
    L, H, Hq, d, B, nb = 1, 1, 1, 32, 8, 2
    rng = np.random.default_rng(13)
    kc = np.zeros((L, nb, B, H, d), np.float32)
    vc = rng.normal(size=(L, nb, B, H, d)).astype(np.float32)
    q = rng.normal(size=(L, 1, 1, Hq, d)).astype(np.float32)
    k1 = rng.normal(size=d).astype(np.float32)
    k2 = rng.normal(size=d).astype(np.float32)
    bt = np.array([[1, 0]], np.int32)
    kc[0, 1, 3, 0], kc[0, 1, 4, 0] = k1, k2          # positions 3 and 4
    f = oracle.rope_freqs(d, 1e4)
    out = oracle.attend(L, H, Hq, d, synth.F32, q, [0], [3], [5], bt, B, nb, kc, vc,
                        _nhd(L, nb, B, H, d), f)
    qq = q[0, 0, 0, 0].astype(np.float64)
    s1 = float(qq @ k1.astype(np.float64)) / math.sqrt(d)
    s2 = float(qq @ k2.astype(np.float64)) / math.sqrt(d)
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    ref = w1 * vc[0, 1, 3, 0].astype(np.float64) + (1 - w1) * vc[0, 1, 4, 0].astype(np.float64)
    assert np.allclose(out[0, 0, 0, 0], ref, atol=1e-12, rtol=0)


def _injected_attention(shift, n_qtok=3, Hq=4):
    """Injects the small problem's facts (fp32 cache, prefixes + shift) and
    attends over each request's segment from queries right after it."""
    P = _small_problem(synth.F32, n_blocks=256)
    L, H, d, B, nb = P["L"], P["H"], P["d"], P["B"], P["n_blocks"]
    f = oracle.rope_freqs(d, 1e4)
    prefix = P["prefix"] + shift
    T = np.array([P["lens"][P["ids"][P["req_off"][r]:P["req_off"][r + 1]]].sum()
                  for r in range(3)])
    need = prefix + T
    bt = synth.block_tables(4, need, B, nb)
    kc = np.zeros(L * nb * B * H * d, np.float32)
    vc = np.zeros_like(kc)
    oracle.inject(L, H, d, synth.F32, P["K"], P["V"], P["tok_off"], P["req_off"], P["ids"],
                  prefix, bt, B, nb, kc, vc, _nhd(L, nb, B, H, d), f)
    q = np.random.default_rng(14).normal(size=(L, 3, n_qtok, Hq, d)).astype(np.float32)
    qpos = prefix + T + 2
    out = oracle.attend(L, H, Hq, d, synth.F32, q, qpos, prefix, prefix + T, bt, B, nb, kc, vc,
                        _nhd(L, nb, B, H, d), f)
    return P, q, qpos, prefix, out, f


def test_attention_over_injected_keys_equals_relative_position_form():
    """Theorem 6 through attention: with the facts' pre-RoPE keys injected at
    positions n and the query at m, every score equals <q, R(n - m) k> (RoPE
    in complex form), so the output is the softmax-weighted sum of the raw
    values with those scores; kv head of query head hq is hq // g."""
    P, q, qpos, prefix, out, f = _injected_attention(0)
    L, H, d = P["L"], P["H"], P["d"]
    Hq = q.shape[3]
    g = Hq // H
    h2 = d // 2
    for r in range(3):
        keys, vals, pos = [], [], []
        n = int(prefix[r])
        for j in range(P["req_off"][r], P["req_off"][r + 1]):
            fid = int(P["ids"][j])
            ln = int(P["lens"][fid])
            base = int(P["tok_off"][fid]) * L * H * d
            blk = P["K"][base:base + ln * L * H * d].reshape(L, H, ln, d).astype(np.float64)
            vbl = P["V"][base:base + ln * L * H * d].reshape(L, H, ln, d).astype(np.float64)
            for t in range(ln):
                keys.append(blk[:, :, t])
                vals.append(vbl[:, :, t])
                pos.append(n + t)
            n += ln
        keys, vals, pos = np.array(keys), np.array(vals), np.array(pos)
        for l in range(L):
            for t in range(q.shape[2]):
                m = int(qpos[r]) + t
                for hq in range(Hq):
                    kk = keys[:, l, hq // g]
                    z = (kk[:, :h2] + 1j * kk[:, h2:]) * np.exp(1j * np.outer(pos - m, f))
                    rk = np.concatenate([z.real, z.imag], axis=1)
                    s = rk @ q[l, r, t, hq].astype(np.float64) / math.sqrt(d)
                    w = np.exp(s - s.max())
                    ref = (w / w.sum()) @ vals[:, l, hq // g]
                    assert np.allclose(out[l, r, t, hq], ref, atol=2e-6, rtol=0)


def test_attention_invariant_under_shared_shift():
    _, _, _, _, out0, _ = _injected_attention(0)
    _, _, _, _, out1, _ = _injected_attention(517)
    assert np.allclose(out0, out1, atol=2e-6, rtol=0)


def test_attention_rejects_positions_outside_the_table():
    L, H, d, B, nb = 1, 1, 8, 4, 2
    kc = np.zeros((L, nb, B, H, d), np.float32)
    q = np.zeros((L, 1, 1, H, d), np.float32)
    with pytest.raises(ValueError):
        oracle.attend(L, H, H, d, synth.F32, q, [9], [0], [9], np.array([[0, 1]], np.int32), B,
                      nb, kc, kc, _nhd(L, nb, B, H, d), oracle.rope_freqs(d, 1e4))


# ----------------------------------------------------------------- ingest
# Context-window-encoded facts packed into the store layout.

@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_ingest_round_trip_drops_exactly_the_window(dtype):
    """Encodings built by placing each fact's stored rows behind w rows of
    another sequence, per (layer, kv head): packing returns the facts' rows
    and nothing else."""
    L, H, d, w = 3, 2, 16, 5
    lens = np.array([4, 1, 9], np.int32)
    encs, facts = [], []
    for i, n in enumerate(lens):
        fact = synth.fact_kv(21, synth.TAG_K, i, L * H * int(n) * d, dtype).reshape(L, H, n, d)
        window = synth.fact_kv(21, synth.TAG_V, 100 + i, L * H * w * d, dtype).reshape(L, H, w, d)
        encs.append(np.concatenate([window, fact], axis=2).reshape(-1))
        facts.append(fact.reshape(-1))
    got = oracle.ingest(L, H, d, lens, w, np.concatenate(encs))
    assert np.array_equal(got.view(np.uint8), np.concatenate(facts).view(np.uint8))


def test_ingest_without_window_is_the_identity():
    L, H, d = 2, 4, 8
    lens = np.array([3, 7], np.int32)
    enc = synth.fact_kv(22, synth.TAG_K, 0, int(lens.sum()) * L * H * d, synth.BF16)
    assert np.array_equal(oracle.ingest(L, H, d, lens, 0, enc), enc)


# ----------------------------------------------------------------- eviction

def test_survivors_renumbering_closed_form():
    """New id of a kept fact = old id minus the number of removed ids below
    it; nothing removed survives; every kept fact appears once."""
    rng = np.random.default_rng(5)
    for n in (1, 2, 17, 300):
        removed = rng.choice(n, size=rng.integers(0, n + 1), replace=False)
        keep = oracle.survivors(n, removed)
        assert len(keep) == n - len(removed)
        assert not set(keep.tolist()) & set(removed.tolist())
        for new, old in enumerate(keep):
            assert new == old - int((removed < old).sum())


def test_survivors_special_cases():
    assert oracle.survivors(5, []).tolist() == [0, 1, 2, 3, 4]
    assert oracle.survivors(5, [4, 0]).tolist() == [1, 2, 3]
    assert oracle.survivors(3, [2, 1, 0]).tolist() == []
    for bad in ([1, 1], [5], [-1]):
        with pytest.raises(ValueError):
            oracle.survivors(5, bad)
