"""Parity at the configurations' full sizes, in the launch configuration the
bench times: full stores in HBM (and pinned host memory for the offload
workload), full caches, all requests injected in one call.  The oracle
checks every request element by element, ten requests at a time (every row
they write, all layers: V bit for bit, K within the tolerance), the whole
cache is checked on the device for untouched rows, and top-k is checked
against the exact oracle on every query."""
import os

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from tests import harness as Hn

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def _cleanup(gpu):
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sampled_inject_check(cache, lens, req_off, flat, prefix, bt, rows, touched_only=False):
    sub_off = np.array([req_off[r] for r in rows] + [req_off[rows[-1] + 1]], np.int32)
    sub_flat = flat[sub_off[0]:sub_off[-1]]
    # requests must be consecutive for the CSR slice
    assert list(rows) == list(range(rows[0], rows[-1] + 1))
    n, err = Hn.check_inject_blocks(cache, lens, sub_off - sub_off[0], sub_flat, prefix[rows],
                                    bt[rows], Hn.blocks_of(bt, rows), touched_only=touched_only)
    Hn.log(f"  requests {rows[0]}..{rows[-1]}: {n} rotated K elements, max |err| {err:.3g}")
    return n


def _every_request_check(cache, lens, req_off, flat, prefix, bt, group=10):
    """Every request of the call against the oracle, `group` at a time (the
    oracle's compact cache of ten requests is about 2.5 GB)."""
    n_req = len(prefix)
    total = 0
    for r0 in range(0, n_req, group):
        total += _sampled_inject_check(cache, lens, req_off, flat, prefix, bt,
                                       list(range(r0, min(n_req, r0 + group))),
                                       touched_only=True)
    w = cache.w
    assert total == int(lens[flat].sum()) * w.n_layers * w.n_kv_heads * w.head_dim
    Hn.log(f"  all {n_req} requests: {total} rotated K elements checked")


def test_llama8b_single_and_batch(gpu):
    """Llama-3.1-8B-shaped store (10,000 facts, 50 GB) and the 98,304-block
    cache (206 GB): the single request with top-5 retrieval, then the
    100-request x 50-fact Zipf batch."""
    import torch
    w1 = W.WORKLOADS["llama8b_single"]
    w3 = W.WORKLOADS["llama8b_batch"]
    Hn.log("llama8b: building the 50 GB store")
    st = Hn.make_store(w1)
    try:
        cache = Hn.make_cache(w1)
        # single request: top-5 of one query, then inject with the oracle's ids
        q = W.query_embeddings(w1)
        ids, sc = Hn.gpu_topk(st, q, w1.k)
        o_ids = Hn.check_topk(q, st.emb, ids, sc, w1.k)
        req_off, flat = Hn.requests_from_ids(o_ids)
        prefix = W.request_prefixes(w1)
        bt = Hn.block_tables_for(w1, st.lens, req_off, flat, prefix)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        _sampled_inject_check(cache, st.lens, req_off, flat, prefix, bt, [0])
        slots1 = oracle.token_slots(req_off, flat, st.lens, prefix, bt, w1.block_size)
        Hn.check_untouched(cache, slots1)
        del cache
        torch.cuda.empty_cache()
        # the batch, into a fresh cache
        Hn.log("llama8b batch: 100 requests x 50 Zipf facts")
        cache = Hn.make_cache(w3)
        ids3 = W.zipf_fact_ids(w3)
        req_off, flat = Hn.requests_from_ids(ids3)
        prefix = W.request_prefixes(w3)
        bt = Hn.block_tables_for(w3, st.lens, req_off, flat, prefix)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        _every_request_check(cache, st.lens, req_off, flat, prefix, bt)
        slots = oracle.token_slots(req_off, flat, st.lens, prefix, bt, w3.block_size)
        assert len(np.unique(slots)) == len(slots)
        Hn.check_untouched(cache, slots)
    finally:
        st.destroy()


def test_mistral7b_batch(gpu):
    """Mistral-7B-shaped store (50,000 facts, 237 GB), exact top-50 for 100
    queries, then the 100 x 50 inject (the bench's workload)."""
    import torch
    w = W.WORKLOADS["mistral7b_batch"]
    Hn.log("mistral7b: building the 237 GB store")
    st = Hn.make_store(w)
    try:
        q = W.query_embeddings(w)
        ids, sc = Hn.gpu_topk(st, q, w.k)
        o_ids = Hn.check_topk(q, st.emb, ids, sc, w.k)
        Hn.log("  top-50 of all 100 queries match the oracle")
        cache = Hn.make_cache(w)
        req_off, flat = Hn.requests_from_ids(o_ids)
        prefix = W.request_prefixes(w)
        bt = Hn.block_tables_for(w, st.lens, req_off, flat, prefix)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        _every_request_check(cache, st.lens, req_off, flat, prefix, bt)
        slots = oracle.token_slots(req_off, flat, st.lens, prefix, bt, w.block_size)
        Hn.check_untouched(cache, slots)
    finally:
        st.destroy()


def _host_tier_fits(w) -> bool:
    lens = W.fact_lengths(w)
    host_bytes = int(lens[int(len(lens) * (1 - w.host_fraction)):].sum()) * w.token_bytes * 2
    avail = os.sysconf("SC_AVPHYS_PAGES") * os.sysconf("SC_PAGE_SIZE")
    return host_bytes + (20 << 30) < min(avail - (10 << 30), 255 << 30)


def test_qwen7b_offload(gpu):
    """Qwen2.5-7B-shaped store of 1M facts: facts past the HBM budget (the
    upper half) in pinned host memory.  Exact top-50 over 1M x 1024
    embeddings for 100 queries, every query checked against the oracle,
    then the 100 requests x top-50 injected from both tiers (the bench's
    step; the ids injected are the oracle's)."""
    import torch
    w = W.WORKLOADS["qwen7b_offload"]
    if not _host_tier_fits(w):
        pytest.skip("host memory too small for the pinned tier")
    lens = W.fact_lengths(w)
    n_hbm = int(len(lens) * (1 - w.host_fraction))
    budget = int(lens[:n_hbm].sum()) * w.token_bytes * 2
    Hn.log(f"qwen7b: building the store ({budget / 1e9:.0f} GB HBM + the rest pinned on the host)")
    st = Hn.make_store(w, lens, hbm_budget=budget)
    try:
        info = Hn.K.is_store_get_info(st.handle)
        assert info.n_hbm_facts == n_hbm
        q = W.query_embeddings(w)
        ids, sc = Hn.gpu_topk(st, q, w.k)
        o_ids = Hn.check_topk(q, st.emb, ids, sc, w.k)
        Hn.log("  top-50 of all 100 queries match the oracle")
        req_off, flat = Hn.requests_from_ids(o_ids)
        Hn.log(f"  {int((flat >= n_hbm).sum())} of {len(flat)} selected facts on the host tier")
        assert (flat >= n_hbm).mean() > 0.3
        prefix = W.request_prefixes(w)
        cache = Hn.make_cache(w)
        bt = Hn.block_tables_for(w, st.lens, req_off, flat, prefix)
        Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        _every_request_check(cache, st.lens, req_off, flat, prefix, bt)
        slots = oracle.token_slots(req_off, flat, st.lens, prefix, bt, w.block_size)
        Hn.check_untouched(cache, slots)
    finally:
        st.destroy()


def test_qwen3_14b_one_request_from_both_tiers(gpu):
    """Qwen3-14B-shaped store (half of the facts pinned on the host): one
    request, top-50, injected by the host path and by the device path; both
    caches equal and match the oracle on every block the request uses."""
    import torch
    w = W.WORKLOADS["qwen3_14b_offload"]
    if not _host_tier_fits(w):
        pytest.skip("host memory too small for the pinned tier")
    lens = W.fact_lengths(w)
    n_hbm = int(len(lens) * (1 - w.host_fraction))
    budget = int(lens[:n_hbm].sum()) * w.token_bytes * 2
    Hn.log(f"qwen3-14b: building the store ({budget / 1e9:.0f} GB HBM + the rest pinned)")
    st = Hn.make_store(w, lens, hbm_budget=budget)
    try:
        q = W.query_embeddings(w)
        ids, sc = Hn.gpu_topk(st, q, w.k)
        Hn.check_topk(q, st.emb, ids, sc, w.k)
        req_off, flat = Hn.requests_from_ids(ids)
        Hn.log(f"  {int((flat >= n_hbm).sum())} of 50 facts on the host tier")
        assert (flat >= n_hbm).any() and (flat < n_hbm).any()
        prefix = W.request_prefixes(w)
        bt = Hn.block_tables_for(w, st.lens, req_off, flat, prefix)
        c_host = Hn.make_cache(w)
        c_dev = Hn.make_cache(w)
        Hn.gpu_inject(st, c_host, req_off, flat, prefix, bt)
        status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        Hn.K.is_retrieve_inject(st.handle, torch.from_numpy(q.view(np.int16)).cuda(), 1, w.k,
                                torch.from_numpy(prefix.astype(np.int32)).cuda(),
                                torch.from_numpy(bt).cuda(), c_dev.desc, Hn.rope_of(w), status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(c_host.k, c_dev.k) and torch.equal(c_host.v, c_dev.v)
        n, err = Hn.check_inject_blocks(c_dev, st.lens, req_off, flat, prefix, bt,
                                        Hn.blocks_of(bt, [0]))
        Hn.log(f"  {n} K elements vs oracle, max err {err:.3g}")
    finally:
        st.destroy()
