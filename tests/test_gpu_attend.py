"""is_attend (query-only attention over the paged cache) through the C ABI
against the fp64 oracle: on identical cache contents (the kernel alone), and
after injection (Theorem 6 end to end: attention over re-rotated injected
keys against attention over the oracle's keys prefilled at the same
positions).

Tolerance, same cache: the kernel rotates the query in fp32, splits it and
the probabilities into bf16 hi + lo (relative residual <= 2^-17) and
accumulates in fp32, so each score carries an error near
sqrt(d) * 2^-17 * |q| |k| / sqrt(d) ~ 1e-5 for N(0,1) data and the output,
a convex combination of V rows, moves by about that times |V|: the bound
used is 5e-5.  After injection the two caches also differ by the inject
tolerance (at most one bf16 ulp on a few rotated K elements), which moves a
score by at most sum_i |q_i| ulp(k_i) / sqrt(d); the bound used there is
2e-3."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu

SAME_CACHE_TOL = 5e-5
INJECTED_TOL = 2e-3


@pytest.fixture(autouse=True)
def _gpu_cleanup(gpu):
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _store_only(w):
    """A store handle with the workload's geometry (K/V are not read)."""
    lens = np.ones(4, np.int32)
    desc, keep = Hn.K.make_desc(w.n_layers, w.n_kv_heads, w.head_dim, w.dtype, lens, 0)
    return Hn.K.is_store_create(desc)


def _gpu_attend(st_handle, w, cache, q_bits, q_pos, cb, ce, bt, n_q_heads):
    import torch
    q = torch.from_numpy(q_bits.view(np.int16)).cuda()
    out = torch.empty(q_bits.shape, dtype=torch.float32, device="cuda")
    Hn.K.is_attend(st_handle, cache.desc, Hn.rope_of(w), q, q_bits.shape[2], n_q_heads, q_pos,
                   cb, ce, bt, out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _strides(w, nb, layout):
    B, H, d = w.block_size, w.n_kv_heads, w.head_dim
    return (nb * B * H * d, B * H * d, H * d, d) if layout == "NHD" else \
        (nb * B * H * d, H * B * d, d, B * d)


@pytest.mark.parametrize("layout,n_qtok,n_q_heads,block", [
    ("NHD", 16, 32, 32),   # 64 query rows per kv head: one group of two row tiles
    ("NHD", 3, 32, 32),    # 12 rows: one tile
    ("HND", 20, 32, 32),   # 80 rows: two groups on one XCD
    ("NHD", 5, 8, 32),     # no grouping (g = 1)
    ("NHD", 16, 32, 8),    # 8-slot blocks: a 32-token chunk spans 4-5 table entries
])
def test_attend_matches_oracle_on_the_same_cache(gpu, layout, n_qtok, n_q_heads, block):
    import torch
    w = W.WORKLOADS["mistral7b_batch"].scaled(name="attend", n_layers=2, block_size=block,
                                              n_blocks=64 * 32 // block)
    nb, B, H, d, L = w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.n_layers
    n = L * nb * B * H * d
    kc = synth.fact_kv(w.seed, synth.TAG_K, 1_000_000, n, synth.BF16)
    vc = synth.fact_kv(w.seed, synth.TAG_V, 1_000_000, n, synth.BF16)
    cache = Hn.make_cache(w, layout=layout)
    cache.k.copy_(torch.from_numpy(kc.view(np.uint8)))
    cache.v.copy_(torch.from_numpy(vc.view(np.uint8)))
    n_req = 4
    # ragged contexts: crossing blocks, shorter than a chunk, empty, long
    cb = np.array([5, 0, 40, 3], np.int32)
    ce = np.array([150, 17, 40, 1700], np.int32)
    q_pos = ce + np.array([0, 9, 2, 100], np.int32)
    need = (ce + B - 1) // B
    bt = np.full((n_req, int(need.max())), -1, np.int32)
    perm = synth.permutation(w.seed, nb)
    bt[3, :need[3]] = perm[:need[3]]                       # the long context uses most blocks
    for r in range(3):
        bt[r, :need[r]] = perm[(r * 7) % 10:(r * 7) % 10 + need[r]]
    q = synth.fact_kv(w.seed, synth.TAG_K, 2_000_000, L * n_req * n_qtok * n_q_heads * d,
                      synth.BF16).reshape(L, n_req, n_qtok, n_q_heads, d)
    Hn.log(f"attend: {layout}, {n_qtok} tokens x {n_q_heads} heads, block {block}, "
           f"contexts {list(ce - cb)}")
    st = _store_only(w)
    try:
        got = _gpu_attend(st, w, cache, q, q_pos, cb, ce, bt, n_q_heads)
    finally:
        Hn.K.is_store_destroy(st)
    ref = oracle.attend(L, H, n_q_heads, d, synth.BF16, q, q_pos, cb, ce, bt, B, nb, kc, vc,
                        _strides(w, nb, layout), Hn.oracle_freqs(w))
    err = np.abs(got - ref)
    Hn.log(f"  max |gpu - oracle| = {err.max():.3g}")
    assert err.max() <= SAME_CACHE_TOL
    assert np.array_equal(got[:, 2], np.zeros_like(got[:, 2]))    # empty context


def test_attend_after_inject_theorem6(gpu):
    """Inject the facts on the GPU, then attend from query tokens placed
    right after each request's segment; the oracle prefills the same keys
    directly at their positions and attends in fp64."""
    w = W.WORKLOADS["llama8b_batch"].scaled(name="attend_inject", n_facts=300, n_req=4, k=6,
                                            n_blocks=240, emb_dim=0, n_layers=3)
    lens = W.fact_lengths(w)
    ids = synth.zipf_requests(w.seed, w.n_req, w.k, w.n_facts, w.zipf_s)
    req_off, flat = Hn.requests_from_ids(ids)
    prefix = synth.prefixes(w.seed, w.n_req, w.prefix[0], w.prefix[1])
    T = np.array([lens[flat[req_off[r]:req_off[r + 1]]].sum() for r in range(w.n_req)], np.int32)
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        n_qtok, n_q_heads = 8, 32
        q = synth.fact_kv(w.seed, synth.TAG_V, 3_000_000,
                          w.n_layers * w.n_req * n_qtok * n_q_heads * w.head_dim,
                          synth.BF16).reshape(w.n_layers, w.n_req, n_qtok, n_q_heads, w.head_dim)
        cb, ce = prefix.astype(np.int32), (prefix + T).astype(np.int32)
        got = _gpu_attend(st.handle, w, cache, q, ce, cb, ce, bt, n_q_heads)
    finally:
        st.destroy()
    kc_o, vc_o = Hn.oracle_blocks(w, lens, req_off, flat, prefix, bt, np.arange(w.n_blocks),
                                  "NHD", w.n_blocks)
    ref = oracle.attend(w.n_layers, w.n_kv_heads, n_q_heads, w.head_dim, synth.BF16, q, ce, cb,
                        ce, bt, w.block_size, w.n_blocks, kc_o.view(np.uint16),
                        vc_o.view(np.uint16), _strides(w, w.n_blocks, "NHD"), Hn.oracle_freqs(w))
    err = np.abs(got - ref)
    Hn.log(f"  max |gpu inject+attend - oracle prefill+attend| = {err.max():.3g}")
    assert err.max() <= INJECTED_TOL


def test_attend_rejects_bad_tables_without_gpu_work(gpu):
    import torch
    w = W.WORKLOADS["mistral7b_batch"].scaled(name="attend_bad", n_layers=1, n_blocks=8)
    cache = Hn.make_cache(w)
    st = _store_only(w)
    try:
        q = torch.zeros((1, 1, 1, 8, 128), dtype=torch.int16, device="cuda")
        out = torch.zeros((1, 1, 1, 8, 128), dtype=torch.float32, device="cuda")
        for cb, ce, bt, code in (([0], [40], [[0]], -3),        # table too short
                                 ([0], [10], [[8]], -3),        # entry >= n_blocks
                                 ([5], [4], [[0]], -1)):        # begin > end
            with pytest.raises(Hn.K.ISError) as e:
                Hn.K.is_attend(st, cache.desc, Hn.rope_of(w), q, 1, 8, [50], cb, ce,
                               np.array(bt, np.int32), out)
            assert e.value.code == code
    finally:
        Hn.K.is_store_destroy(st)


def _dev_q(q):
    import torch
    return torch.from_numpy(q if q.dtype == np.float32 else q.view(np.int16)).cuda()


@pytest.mark.parametrize("dtype,d,H,G", [
    (synth.F32, 64, 2, 2),     # the tiny configuration's cache type and head size
    (synth.BF16, 64, 4, 4),
    (synth.BF16, 256, 2, 1),
])
def test_attend_plain_kernel_matches_oracle(gpu, dtype, d, H, G):
    """Shapes off the matrix-core path (fp32 caches, head_dim other than 128)
    run the plain fp32 kernel; same caches on both sides."""
    import torch
    w = W.WORKLOADS["tiny"].scaled(name="attend_plain", n_layers=2, n_kv_heads=H, head_dim=d,
                                   dtype=dtype, block_size=16, n_blocks=64)
    nb, B, L = w.n_blocks, w.block_size, w.n_layers
    n = L * nb * B * H * d
    kc = synth.fact_kv(w.seed, synth.TAG_K, 3_000_000, n, dtype)
    vc = synth.fact_kv(w.seed, synth.TAG_V, 3_000_000, n, dtype)
    cache = Hn.make_cache(w)
    cache.k.copy_(torch.from_numpy(kc.view(np.uint8)))
    cache.v.copy_(torch.from_numpy(vc.view(np.uint8)))
    n_req, n_qtok, n_q_heads = 4, 3, H * G
    cb = np.array([3, 0, 10, 2], np.int32)
    ce = np.array([70, 17, 10, 300], np.int32)
    q_pos = ce + np.array([0, 4, 1, 9], np.int32)
    need = (ce + B - 1) // B
    bt = np.full((n_req, int(need.max())), -1, np.int32)
    perm = synth.permutation(w.seed, nb)
    for r in range(n_req):
        bt[r, :need[r]] = perm[r:r + need[r]]
    q = synth.fact_kv(w.seed, synth.TAG_K, 4_000_000, L * n_req * n_qtok * n_q_heads * d,
                      dtype).reshape(L, n_req, n_qtok, n_q_heads, d)
    Hn.log(f"attend (plain kernel): dtype {dtype}, head_dim {d}, {H} kv heads x {G}")
    st = _store_only(w)
    try:
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        Hn.K.is_attend(st, cache.desc, Hn.rope_of(w), _dev_q(q), n_qtok, n_q_heads, q_pos, cb,
                       ce, bt, out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
    finally:
        Hn.K.is_store_destroy(st)
    ref = oracle.attend(L, H, n_q_heads, d, dtype, q, q_pos, cb, ce, bt, B, nb, kc, vc,
                        _strides(w, nb, "NHD"), Hn.oracle_freqs(w))
    err = np.abs(got - ref)
    Hn.log(f"  max |gpu - oracle| = {err.max():.3g}")
    assert err.max() <= SAME_CACHE_TOL
    assert np.array_equal(got[:, 2], np.zeros_like(got[:, 2]))    # empty context


def test_attend_after_inject_tiny_theorem6(gpu):
    """The tiny fp32 configuration end to end: facts injected on the GPU,
    then attended from query tokens right after the segment, against the
    oracle's keys prefilled at the same positions (fp32 caches: the inject
    tolerance is 1e-5 per element)."""
    import torch
    w = W.WORKLOADS["tiny"].scaled(name="attend_tiny", n_blocks=64)
    lens = W.fact_lengths(w)
    ids = np.array([[3, 11, 7, 0, 19]], np.int32)
    req_off, flat = Hn.requests_from_ids(ids)
    prefix = np.array([16], np.int32)
    T = int(lens[flat].sum())
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        n_qtok, n_q_heads = 4, 2 * w.n_kv_heads
        q = synth.fact_kv(w.seed, synth.TAG_V, 5_000_000,
                          w.n_layers * 1 * n_qtok * n_q_heads * w.head_dim,
                          synth.F32).reshape(w.n_layers, 1, n_qtok, n_q_heads, w.head_dim)
        cb, ce = prefix.astype(np.int32), (prefix + T).astype(np.int32)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        Hn.K.is_attend(st.handle, cache.desc, Hn.rope_of(w), _dev_q(q), n_qtok, n_q_heads, ce,
                       cb, ce, bt, out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
    finally:
        st.destroy()
    kc_o, vc_o = Hn.oracle_blocks(w, lens, req_off, flat, prefix, bt, np.arange(w.n_blocks),
                                  "NHD", w.n_blocks)
    ref = oracle.attend(w.n_layers, w.n_kv_heads, n_q_heads, w.head_dim, synth.F32, q, ce, cb,
                        ce, bt, w.block_size, w.n_blocks, kc_o.view(np.float32),
                        vc_o.view(np.float32), _strides(w, w.n_blocks, "NHD"),
                        Hn.oracle_freqs(w))
    err = np.abs(got - ref)
    Hn.log(f"  max |gpu inject+attend - oracle prefill+attend| (tiny) = {err.max():.3g}")
    assert err.max() <= 5e-4
