"""GPU parity through the C ABI against the fp64 oracle, at sizes the
oracle finishes in seconds (several tiles, ragged tails).  Tolerances are
stated in tests/harness.py."""
import numpy as np
import pytest

import synth
from synth import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_cleanup(gpu):
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_smoke_tiny(gpu):
    Hn.smoke()


def _zipf_problem(w, n_req, k, seed_fact_count=None):
    lens = W.fact_lengths(w)
    ids = synth.zipf_requests(w.seed, n_req, k, w.n_facts, w.zipf_s)
    req_off, flat = Hn.requests_from_ids(ids)
    prefix = synth.prefixes(w.seed, n_req, w.prefix[0], w.prefix[1])
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    return lens, req_off, flat, prefix, bt


SMALL_LLAMA = W.WORKLOADS["llama8b_batch"].scaled(name="llama_small", n_facts=300, n_req=6,
                                                  k=5, n_blocks=160, emb_dim=0)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_inject_llama_shape_small(gpu, layout):
    w = SMALL_LLAMA
    Hn.log(f"inject llama-shaped small, layout {layout}")
    lens, req_off, flat, prefix, bt = _zipf_problem(w, w.n_req, w.k)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w, layout=layout)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        n, err = Hn.check_inject_blocks(cache, lens, req_off, flat, prefix, bt,
                                        Hn.blocks_of(bt, range(w.n_req)))
        Hn.log(f"  {n} K elements, max err {err:.3g}")
        # blocks no request uses stay untouched
        used = set(Hn.blocks_of(bt, range(w.n_req)).tolist())
        free = np.array([b for b in range(w.n_blocks) if b not in used][:8])
        Hn.check_inject_blocks(cache, lens, np.array([0, 0], np.int32), flat[:0],
                               prefix[:1], bt[:1], free)
    finally:
        st.destroy()


def test_inject_fp32_head128_and_repeat(gpu):
    w = W.WORKLOADS["tiny"].scaled(name="f32_128", head_dim=128, n_layers=3, n_kv_heads=2,
                                   n_facts=40, len_dist=("uniform", 1, 70), n_blocks=64,
                                   emb_dim=0, theta=1e6)
    lens = W.fact_lengths(w)
    req_off = np.array([0, 3, 7], np.int32)
    flat = np.array([5, 5, 39, 0, 1, 2, 3], np.int32)     # fact 5 twice in request 0
    prefix = np.array([0, 131], np.int32)
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    st = Hn.make_store(w, lens, fill="host")
    try:
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        Hn.check_inject_blocks(cache, lens, req_off, flat, prefix, bt, np.arange(w.n_blocks))
    finally:
        st.destroy()


@pytest.mark.parametrize("dtype,head_dim", [(synth.BF16, 64), (synth.BF16, 256), (synth.F32, 32)])
def test_inject_other_head_dims(gpu, dtype, head_dim):
    """Shapes served by the general kernel (rows other than 256 bytes)."""
    w = SMALL_LLAMA.scaled(name=f"hd{head_dim}", n_layers=3, n_kv_heads=4, head_dim=head_dim,
                           dtype=dtype, n_facts=50, n_blocks=400, theta=1e4, scaling="none",
                           prefix=(0, 40))
    lens, req_off, flat, prefix, bt = _zipf_problem(w, 5, 6)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w, layout="HND" if head_dim == 256 else "NHD")
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        Hn.check_inject_blocks(cache, lens, req_off, flat, prefix, bt, np.arange(w.n_blocks))
    finally:
        st.destroy()


def test_inject_host_tier(gpu):
    """Facts beyond the HBM budget live in pinned host memory and are read
    from there by the same kernel."""
    w = SMALL_LLAMA.scaled(name="llama_offload", n_facts=120)
    lens, req_off, flat, prefix, bt = _zipf_problem(w, 4, 8)
    budget = int(lens[:60].sum()) * w.token_bytes * 2
    st = Hn.make_store(w, lens, hbm_budget=budget)
    try:
        info = Hn.K.is_store_get_info(st.handle)
        assert info.n_hbm_facts == 60 and info.host_kv_bytes > 0
        assert (flat >= 60).any() and (flat < 60).any()
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        Hn.check_inject_blocks(cache, lens, req_off, flat, prefix, bt,
                               Hn.blocks_of(bt, range(4)))
    finally:
        st.destroy()


@pytest.mark.parametrize("host_tier", [False, True])
def test_inject_short_facts_layer_groups(gpu, host_tier):
    """Facts of 1-3 tokens: a workgroup takes several layers (40 layers, 4
    kv heads: 16 layers per workgroup, groups of 16, 16 and 8), and with a
    host tier the host-tier facts take one workgroup for all layers."""
    w = SMALL_LLAMA.scaled(name="short", n_layers=40, n_kv_heads=4, n_facts=400,
                           len_dist=("uniform", 1, 3), n_blocks=300, prefix=(0, 40))
    lens, req_off, flat, prefix, bt = _zipf_problem(w, 12, 20)
    budget = int(lens[:200].sum()) * w.token_bytes * 2 if host_tier else -1
    st = Hn.make_store(w, lens, hbm_budget=budget)
    try:
        if host_tier:
            assert (flat >= 200).any() and (flat < 200).any()
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        Hn.check_inject_blocks(cache, lens, req_off, flat, prefix, bt, np.arange(w.n_blocks))
    finally:
        st.destroy()


def test_inject_deterministic_and_position_zero_identity(gpu):
    import torch
    w = SMALL_LLAMA
    lens, req_off, flat, prefix, bt = _zipf_problem(w, 3, 4)
    prefix[:] = 0
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    st = Hn.make_store(w, lens)
    try:
        c1 = Hn.make_cache(w)
        c2 = Hn.make_cache(w)
        Hn.gpu_inject(st, c1, req_off, flat, prefix, bt)
        Hn.gpu_inject(st, c2, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)
        # the first token of request 0 sits at position 0: its K is the stored K
        f = int(flat[0])
        k_pre = synth.fact_kv(w.seed, synth.TAG_K, f, int(lens[f]) * w.row_elems, w.dtype)
        k_pre = k_pre.reshape(w.n_layers, w.n_kv_heads, int(lens[f]), w.head_dim)[:, :, 0]
        blk = int(bt[0, 0])
        got = c1.k.view(w.n_layers, w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim * 2)
        got = got[:, blk, 0].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, k_pre)
    finally:
        st.destroy()


@pytest.mark.parametrize("dtype,head_dim", [(synth.F32, 64), (synth.F32, 128), (synth.F32, 32),
                                            (synth.BF16, 128), (synth.BF16, 64)])
def test_position_zero_identity_bit_exact(gpu, dtype, head_dim):
    """A key injected at position 0 turns by angle 0: the cache row equals the
    stored pre-RoPE row bit for bit, for every layer and head, in both cache
    dtypes and in both inject kernels (256-byte rows: fp32 d64, bf16 d128;
    other rows: fp32 d128 and d32, bf16 d64)."""
    w = SMALL_LLAMA.scaled(name=f"p0_{dtype}_{head_dim}", n_layers=3, n_kv_heads=4,
                           head_dim=head_dim, dtype=dtype, n_facts=60, n_blocks=200,
                           theta=1e6, scaling="none")
    lens, req_off, flat, _, _ = _zipf_problem(w, 5, 4)
    prefix = np.zeros(5, np.int32)
    bt = Hn.block_tables_for(w, lens, req_off, flat, prefix)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        import torch
        torch.cuda.synchronize()
        es = w.elem_size
        view = cache.k.view(w.n_layers, w.n_blocks, w.block_size, w.n_kv_heads,
                            w.head_dim * es)
        for r in range(5):
            f = int(flat[req_off[r]])
            k_pre = synth.fact_kv(w.seed, synth.TAG_K, f, int(lens[f]) * w.row_elems, w.dtype)
            k_pre = k_pre.reshape(w.n_layers, w.n_kv_heads, int(lens[f]), w.head_dim)[:, :, 0]
            got = view[:, int(bt[r, 0]), 0].cpu().numpy()
            want = np.ascontiguousarray(k_pre).view(np.uint8)
            assert np.array_equal(got.reshape(want.shape), want), f"request {r}"
    finally:
        st.destroy()


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_generator_device_build_matches_host_build(gpu, dtype):
    """The full-size checks take the oracle's K/V inputs from the generator's
    device build: it must give the host build's values bit for bit (runs of
    consecutive facts and single facts, long and short)."""
    w = SMALL_LLAMA.scaled(name="gen", dtype=dtype, n_facts=2000,
                           len_dist=("uniform", 1, 200))
    lens = W.fact_lengths(w)
    facts = np.array([0, 1, 2, 7, 500, 501, 1999], np.int64)
    for tag in (synth.TAG_K, synth.TAG_V):
        dev = Hn.generator_blocks(w, lens, facts, tag)
        host = np.concatenate([synth.fact_kv(w.seed, tag, int(f), int(lens[f]) * w.row_elems,
                                             dtype) for f in facts])
        assert np.array_equal(dev.view(np.uint8), host.view(np.uint8))


def test_inject_invalid_call_writes_nothing(gpu):
    import torch
    w = SMALL_LLAMA
    lens, req_off, flat, prefix, bt = _zipf_problem(w, 3, 4)
    st = Hn.make_store(w, lens)
    try:
        cache = Hn.make_cache(w)
        before = cache.k.clone()
        bad = flat.copy()
        bad[-1] = w.n_facts
        with pytest.raises(Hn.K.ISError) as e:
            Hn.gpu_inject(st, cache, req_off, bad, prefix, bt)
        assert e.value.code == -2
        # request 1 = request 0 with the same block table: every slot collides
        k0 = req_off[1]
        twice = np.concatenate([flat[:k0], flat[:k0]])
        with pytest.raises(Hn.K.ISError) as e:
            Hn.gpu_inject(st, cache, np.array([0, k0, 2 * k0], np.int32), twice,
                          np.array([prefix[0], prefix[0]], np.int32), np.stack([bt[0], bt[0]]))
        assert e.value.code == -4
        torch.cuda.synchronize()
        assert torch.equal(before, cache.k)
    finally:
        st.destroy()


@pytest.mark.parametrize("n_facts,dim,n_q,k", [
    (20, 32, 1, 5),          # tiny shape
    (1000, 128, 7, 10),      # several tiles, ragged tail
    (5003, 1024, 100, 50),   # 20 workgroups, the 100-query batch
    (3000, 256, 130, 64),    # two query blocks, k at its maximum
    (2000, 192, 40, 20),     # two 32-query tiles, width not a multiple of 128
    (70000, 128, 3, 1),      # all 256 workgroups, several tiles each
    (140001, 1024, 100, 50), # queries held in registers (stores of 131,072 facts and
                             # more): 1,094 tiles of 128, four or five per workgroup,
                             # ragged last tile
    (131072, 1024, 65, 7),   # queries in registers, one valid row in the third wave
    (131500, 1024, 130, 64), # 128 queries in registers (every wave full), the last two
                             # by the staged scan; k at its maximum
    (131100, 992, 70, 9),    # width 992: queries padded to 1024 through the scratch
                             # copy, then held in registers
    (50000, 1024, 1, 5),     # one request on the Mistral-shaped index: the query tile
                             # shared by the four waves, 391 tiles of 128
    (9001, 1024, 32, 64),    # shared query tile, every row valid, k at its maximum
    (300, 1024, 5, 7),       # shared query tile, three tiles (the sample is the store)
    (100, 1024, 3, 64),      # bound found inside the stream scan; fewer sample groups
                             # than k, so the bound is -inf and every fact is a candidate
    (20000, 1024, 4, 64),    # bound inside the stream scan, one query per wave
    (600000, 1024, 1, 9),    # shared query tile over a sample of 1,176 groups: the
                             # separate threshold kernel
    (140001, 128, 3, 5),     # staged scan on a store past the one-pass limit (8,752
                             # groups): sample, bound and stream, one query tile
    (140001, 256, 40, 20),   # the same with two query tiles
    (140001, 64, 100, 50),   # ... and four
    (6000, 1024, 50, 30),    # 33-64 queries at width 1024: the staged scan, one pass
    (131072, 1024, 1, 50),   # one pass at its limit: 8,192 groups, every thread of the
                             # final holds 32 group maxima
    (131100, 1024, 2, 7),    # just past it (8,200 groups): sample, bound and stream
])
def test_topk_parity(gpu, n_facts, dim, n_q, k):
    w = W.WORKLOADS["tiny"].scaled(name="topk", n_facts=n_facts, emb_dim=dim, n_req=n_q,
                                   len_dist=("uniform", 1, 2), seed=n_facts)
    Hn.log(f"top-k parity: {n_facts} facts x {dim}, {n_q} queries, k={k}")
    st = Hn.make_store(w, fill="host")
    try:
        q = W.query_embeddings(w)
        ids, sc = Hn.gpu_topk(st, q, k)
        Hn.check_topk(q, st.emb, ids, sc, k)
        ids2, sc2 = Hn.gpu_topk(st, q, k)
        assert np.array_equal(ids, ids2) and np.array_equal(sc, sc2)
    finally:
        st.destroy()


def test_topk_ties_and_self_match(gpu):
    w = W.WORKLOADS["tiny"].scaled(name="ties", n_facts=600, emb_dim=64, n_req=4,
                                   len_dist=("uniform", 1, 1))
    lens = W.fact_lengths(w)
    emb = W.fact_embeddings(w)
    emb[300] = emb[17]
    emb[599] = emb[17]
    desc, keep = Hn.K.make_desc(1, 2, 64, synth.F32, lens, 64, -1, None, None, emb)
    h = Hn.K.is_store_create(desc)
    st = Hn.Store(w, lens, np.concatenate([[0], np.cumsum(lens)]), h, emb)
    try:
        q = emb[[17, 5, 599, 42]]
        ids, sc = Hn.gpu_topk(st, q, 3)
        assert ids[0].tolist() == [17, 300, 599]
        assert ids[2].tolist() == [17, 300, 599]
        assert ids[1, 0] == 5 and ids[3, 0] == 42
    finally:
        st.destroy()


@pytest.mark.parametrize("n_facts,n_q", [(140001, 100), (140001, 20), (140001, 3),
                                         (300000, 100), (30000, 100), (30000, 20), (30000, 3)])
def test_topk_many_candidates_full_batch(gpu, n_facts, n_q):
    """A store where almost every fact shares one embedding.  Equal scores go
    to the lower ids.  140,001 facts (sample, bound, stream): every fact of a
    workgroup's tiles reaches the sample bound, so candidates overflow the
    scan's staging area and the final selection gathers from the full list,
    and every sample fact is a candidate that the threshold kernel takes
    from the sample's codes (more keys than it stages); 100 queries: one
    query tile per wave; 20: one tile shared by the waves, positions from
    the workgroup's counter; 3: the same, with the bound found inside the
    stream scan.  300,000 facts: 592 sample groups reach the bound, more
    than the threshold kernel lists, so each of its threads takes its own.
    30,000 facts (one pass): every group's maximum is the shared score, so
    every group holds candidates, more than the final kernel stages, and the
    selection reads them from the codes."""
    w = W.WORKLOADS["tiny"].scaled(name="flat1024", n_facts=n_facts, emb_dim=1024, n_req=n_q,
                                   len_dist=("uniform", 1, 1))
    lens = W.fact_lengths(w)
    emb = W.fact_embeddings(w)
    distinct = [3, 1000, n_facts // 2, n_facts - 2]
    common = emb[5].copy()
    keep_rows = emb[distinct].copy()
    emb[:] = common
    emb[distinct] = keep_rows
    desc, keep = Hn.K.make_desc(1, 2, 64, synth.F32, lens, 1024, -1, None, None, emb)
    h = Hn.K.is_store_create(desc)
    st = Hn.Store(w, lens, np.concatenate([[0], np.cumsum(lens)]), h, emb)
    try:
        q = W.query_embeddings(w)
        ids, sc = Hn.gpu_topk(st, q, 10)
        Hn.check_topk(q, st.emb, ids, sc, 10, queries=range(0, n_q, 9))
        for r in range(q.shape[0]):
            shared = [int(f) for f in ids[r] if f not in distinct]
            # facts of the shared embedding come in id order, the lowest first
            lowest = [f for f in range(20) if f not in distinct][:len(shared)]
            assert shared == lowest, f"query {r}: {shared}"
    finally:
        st.destroy()


@pytest.mark.parametrize("n_facts", [140001, 20000])
def test_topk_ties_full_batch_width_1024(gpu, n_facts):
    """Equal embeddings under the register-resident scan (100 queries x 1024;
    140,001 facts: sample, bound and stream; 20,000: one pass): equal scores
    are ordered by the lower id, a self-query ranks its copies first."""
    w = W.WORKLOADS["tiny"].scaled(name="ties1024", n_facts=n_facts, emb_dim=1024, n_req=100,
                                   len_dist=("uniform", 1, 1))
    lens = W.fact_lengths(w)
    emb = W.fact_embeddings(w)
    dups = [300, n_facts // 4, n_facts - 1]
    for dup in dups:
        emb[dup] = emb[17]
    desc, keep = Hn.K.make_desc(1, 2, 64, synth.F32, lens, 1024, -1, None, None, emb)
    h = Hn.K.is_store_create(desc)
    st = Hn.Store(w, lens, np.concatenate([[0], np.cumsum(lens)]), h, emb)
    try:
        q = W.query_embeddings(w)
        q[0] = emb[17]
        q[99] = emb[n_facts - 1]
        q[50] = emb[n_facts - 2]
        ids, sc = Hn.gpu_topk(st, q, 5)
        assert ids[0, :4].tolist() == [17] + dups
        assert ids[99, :4].tolist() == [17] + dups
        assert ids[50, 0] == n_facts - 2
        Hn.check_topk(q, st.emb, ids, sc, 5, queries=[0, 1, 50, 98, 99])
    finally:
        st.destroy()


@pytest.mark.parametrize("n_q", [100, 1])
def test_topk_one_pass_many_copies(gpu, n_q):
    """One pass over 30,000 facts, 1,500 of them copies of fact 7: a query
    equal to fact 7 has 1,501 candidates at its best score (more than the
    final kernel ranks one by one, fewer than it stages), so the radix
    select orders them -- the lowest ids first."""
    w = W.WORKLOADS["tiny"].scaled(name="copies1024", n_facts=30000, emb_dim=1024, n_req=n_q,
                                   len_dist=("uniform", 1, 1))
    lens = W.fact_lengths(w)
    emb = W.fact_embeddings(w)
    rng = np.random.default_rng(11)
    copies = np.sort(rng.choice(np.arange(8, 30000), size=1500, replace=False))
    emb[copies] = emb[7]
    desc, keep = Hn.K.make_desc(1, 2, 64, synth.F32, lens, 1024, -1, None, None, emb)
    h = Hn.K.is_store_create(desc)
    st = Hn.Store(w, lens, np.concatenate([[0], np.cumsum(lens)]), h, emb)
    try:
        q = W.query_embeddings(w)
        q[0] = emb[7]
        ids, sc = Hn.gpu_topk(st, q, 64)
        assert ids[0].tolist() == [7] + copies[:63].tolist()
        Hn.check_topk(q, st.emb, ids, sc, 64, queries=range(0, n_q, 11))
    finally:
        st.destroy()
