"""is_retrieve_inject (top-k, composition, validation and injection all on
the device) through the C ABI: the same cache bytes as the host path on the
same ids, the oracle's result, and device-side validation that leaves the
cache untouched on every failure."""
import numpy as np
import pytest

import oracle
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


SMALL = W.WORKLOADS["llama8b_batch"].scaled(name="device_small", n_facts=400, n_req=6, k=5,
                                            n_blocks=200, emb_dim=128)


def _device_call(st, w, q_bits, k, prefix, bt, cache):
    """Runs is_retrieve_inject; returns (status, ids)."""
    import torch
    n = q_bits.shape[0]
    q = torch.from_numpy(q_bits.view(np.int16)).cuda()
    d_prefix = torch.from_numpy(np.ascontiguousarray(prefix, np.int32)).cuda()
    d_bt = torch.from_numpy(np.ascontiguousarray(bt, np.int32)).cuda()
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    ids = torch.empty((n, k), dtype=torch.int32, device="cuda")
    Hn.K.is_retrieve_inject(st.handle, q, n, k, d_prefix, d_bt, cache.desc, Hn.rope_of(w),
                            status, ids, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return int(status.item()), ids.cpu().numpy()


def _problem(st, w, n_req, k):
    """Queries, their top-k ids (host path), prefixes and block tables
    sized for the segments those ids make."""
    q = W.query_embeddings(w)[:n_req]
    ids, _ = Hn.gpu_topk(st, q, k)
    req_off, flat = Hn.requests_from_ids(ids)
    prefix = synth.prefixes(w.seed, n_req, w.prefix[0], w.prefix[1])
    bt = Hn.block_tables_for(w, st.lens, req_off, flat, prefix)
    return q, ids, req_off, flat, prefix, bt


@pytest.mark.parametrize("hbm_half", [False, True])
def test_device_path_matches_host_path_and_oracle(gpu, hbm_half):
    import torch
    w = SMALL
    lens = W.fact_lengths(w)
    budget = int(lens[:200].sum()) * w.token_bytes * 2 if hbm_half else -1
    st = Hn.make_store(w, lens, hbm_budget=budget)
    try:
        q, ids, req_off, flat, prefix, bt = _problem(st, w, w.n_req, w.k)
        Hn.log(f"device path: {w.n_req} requests x top-{w.k}, host tier {hbm_half}")
        c_dev = Hn.make_cache(w)
        c_host = Hn.make_cache(w)
        status, d_ids = _device_call(st, w, q, w.k, prefix, bt, c_dev)
        assert status == 0
        assert np.array_equal(d_ids, ids)
        Hn.gpu_inject(st, c_host, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        assert torch.equal(c_dev.k, c_host.k) and torch.equal(c_dev.v, c_host.v)
        n, err = Hn.check_inject_blocks(c_dev, lens, req_off, flat, prefix, bt,
                                        Hn.blocks_of(bt, range(w.n_req)))
        Hn.log(f"  {n} K elements vs oracle, max err {err:.3g}")
        Hn.check_untouched(c_dev, oracle.token_slots(req_off, flat, lens, prefix, bt,
                                                        w.block_size))
    finally:
        st.destroy()


def test_device_validation_writes_nothing(gpu):
    import torch
    w = SMALL
    st = Hn.make_store(w)
    try:
        q, ids, req_off, flat, prefix, bt = _problem(st, w, 3, 4)
        cache = Hn.make_cache(w)
        before_k, before_v = cache.k.clone(), cache.v.clone()
        # the same query twice with the same block table: every slot collides
        q2 = np.stack([q[0], q[0]])
        status, _ = _device_call(st, w, q2, 4, np.array([prefix[0]] * 2),
                                 np.stack([bt[0], bt[0]]), cache)
        assert status == -4
        # a block table one block short
        T = int(st.lens[ids[0]].sum())
        need = (int(prefix[0]) + T - 1) // w.block_size + 1
        status, _ = _device_call(st, w, q[:1], 4, prefix[:1], bt[:1, :need - 1], cache)
        assert status == -3
        # an entry outside [0, n_blocks)
        bad = bt[:1].copy()
        bad[0, need - 1] = w.n_blocks
        status, _ = _device_call(st, w, q[:1], 4, prefix[:1], bad, cache)
        assert status == -3
        # a negative prefix
        status, _ = _device_call(st, w, q[:1], 4, np.array([-1]), bt[:1], cache)
        assert status == -1
        # one request whose table names one block twice inside its segment:
        # its own slots collide (a single request is composed by the top-k
        # final kernel)
        b0 = int(prefix[0]) // w.block_size
        assert need - 1 > b0
        dup = bt[:1].copy()
        dup[0, b0 + 1] = dup[0, b0]
        status, _ = _device_call(st, w, q[:1], 4, prefix[:1], dup, cache)
        assert status == -4
        # one good request next to a failing one: still nothing is written
        mixed = bt[:2].copy()
        mixed[1, :] = mixed[0, :]
        status, _ = _device_call(st, w, np.stack([q[0], q[0]]), 4,
                                 np.array([prefix[0], prefix[0]]), mixed, cache)
        assert status == -4
        torch.cuda.synchronize()
        assert torch.equal(before_k, cache.k) and torch.equal(before_v, cache.v)
        # host-side checks return directly
        with pytest.raises(Hn.K.ISError) as e:
            _device_call(st, w, q[:1], 65, prefix[:1], bt[:1], cache)
        assert e.value.code == -9
        # a clean call on the same store still works after the failures
        status, d_ids = _device_call(st, w, q, 4, prefix, bt, cache)
        assert status == 0 and np.array_equal(d_ids, ids)
        Hn.check_inject_blocks(cache, st.lens, req_off, flat, prefix, bt,
                               Hn.blocks_of(bt, range(3)))
    finally:
        st.destroy()


def test_device_path_many_requests(gpu):
    """1030 requests x top-64: several top-k query groups, and 65,920 work
    items, more than one inject launch can index."""
    w = W.WORKLOADS["tiny"].scaled(name="device_many", n_layers=2, n_kv_heads=1,
                                   head_dim=128, dtype=synth.BF16, n_facts=2000,
                                   len_dist=("uniform", 1, 1), emb_dim=64, n_req=1030, k=64,
                                   block_size=16, n_blocks=4200, prefix=(0, 0), theta=1e4,
                                   scaling="none")
    st = Hn.make_store(w)
    try:
        q, ids, req_off, flat, prefix, bt = _problem(st, w, w.n_req, w.k)
        cache = Hn.make_cache(w)
        status, d_ids = _device_call(st, w, q, w.k, prefix, bt, cache)
        assert status == 0 and np.array_equal(d_ids, ids)
        # requests 0-1 and the last ones (their items lie past 65,535); each
        # request owns its blocks, so the oracle runs on those requests alone
        for a, b in ((0, 1), (1024, 1029)):
            ro = req_off[a:b + 2] - req_off[a]
            fl = flat[req_off[a]:req_off[b + 1]]
            Hn.check_inject_blocks(cache, st.lens, ro, fl, prefix[a:b + 1], bt[a:b + 1],
                                   Hn.blocks_of(bt, range(a, b + 1)))
    finally:
        st.destroy()


def test_device_path_large_index(gpu):
    """100 requests x top-50 over 140,001 one-token facts with 1024-dim
    embeddings: the device path runs the register-resident top-k scan (the
    host path's is_topk the same kernel); ids, status and every cache byte
    equal the host path's, the ids pass the oracle on sampled queries."""
    import torch
    w = W.WORKLOADS["tiny"].scaled(name="device_large", n_layers=2, n_kv_heads=1,
                                   head_dim=128, dtype=synth.BF16, n_facts=140001,
                                   len_dist=("uniform", 1, 1), emb_dim=1024, n_req=100, k=50,
                                   block_size=16, n_blocks=600, prefix=(0, 16), theta=1e6,
                                   scaling="none")
    st = Hn.make_store(w)
    try:
        q, ids, req_off, flat, prefix, bt = _problem(st, w, w.n_req, w.k)
        c_dev = Hn.make_cache(w)
        c_host = Hn.make_cache(w)
        status, d_ids = _device_call(st, w, q, w.k, prefix, bt, c_dev)
        assert status == 0
        assert np.array_equal(d_ids, ids)
        Hn.gpu_inject(st, c_host, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        assert torch.equal(c_dev.k, c_host.k) and torch.equal(c_dev.v, c_host.v)
        _, sc = Hn.gpu_topk(st, q, w.k)
        Hn.check_topk(q, st.emb, ids, sc, w.k, queries=[0, 33, 66, 99])
        Hn.check_inject_blocks(c_dev, st.lens, req_off[:3], flat[:req_off[2]], prefix[:2],
                               bt[:2], Hn.blocks_of(bt, range(2)))
    finally:
        st.destroy()
