"""is_retrieve_inject captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay, with new query contents in the captured buffer and
eager work (cache refills, eager calls, synchronizations) between replays,
must write exactly what an eager call with the same query writes -- ids,
status and every cache byte.  After a capture the store refuses removal
(the graph reads its index)."""
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


def _refill(cache, stream):
    n = cache.k.numel()
    synth.gpu_sentinel(Hn.SENTINEL_SEED_K, cache.k.data_ptr(), n, stream)
    synth.gpu_sentinel(Hn.SENTINEL_SEED_V, cache.v.data_ptr(), n, stream)


@pytest.mark.parametrize("k", [5, 50])
def test_graph_replays_match_eager_calls(gpu, k):
    import torch
    K = Hn.K
    w = W.WORKLOADS["mistral7b_batch"].scaled(name="graph", n_facts=3000, n_layers=2,
                                              n_blocks=512, n_req=1, k=k)
    lens = W.fact_lengths(w)
    st = Hn.make_store(w, lens)
    graph = None
    try:
        rope = Hn.rope_of(w)
        cache_g, cache_e = Hn.make_cache(w), Hn.make_cache(w)
        qs = synth.queries(w.seed + 5, 4, w.emb_dim)
        prefix = np.array([40], np.int32)
        need = np.array([int(prefix[0]) + k * int(lens.max())], np.int64)
        bt = synth.block_tables(w.seed, need, w.block_size, w.n_blocks)
        d_prefix = torch.from_numpy(prefix).cuda()
        d_bt = torch.from_numpy(bt).cuda()
        q_buf = torch.empty((1, w.emb_dim), dtype=torch.int16, device="cuda")
        ids_g = torch.empty((1, k), dtype=torch.int32, device="cuda")
        ids_e = torch.empty_like(ids_g)
        status_g = torch.ones(1, dtype=torch.int32, device="cuda")
        status_e = torch.ones_like(status_g)

        def call(q, cache, ids, status, stream):
            K.is_retrieve_inject(st.handle, q, 1, k, d_prefix, d_bt, cache.desc, rope, status,
                                 ids, stream)

        main = torch.cuda.current_stream()
        q_buf.copy_(torch.from_numpy(qs[0:1].view(np.int16)))
        call(q_buf, cache_g, ids_g, status_g, main)          # sizes the graph workspace
        torch.cuda.synchronize()
        Hn.log(f"graph: capture one request, k = {k}")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(main)
        with torch.cuda.graph(graph, stream=side):
            call(q_buf, cache_g, ids_g, status_g, side)
        torch.cuda.synchronize()
        seen = set()
        for i in range(4):
            q_buf.copy_(torch.from_numpy(qs[i:i + 1].view(np.int16)))
            status_g.fill_(1)
            _refill(cache_g, main.cuda_stream)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            q_e = torch.from_numpy(qs[i:i + 1].view(np.int16)).cuda()
            status_e.fill_(1)
            _refill(cache_e, main.cuda_stream)
            call(q_e, cache_e, ids_e, status_e, main)
            torch.cuda.synchronize()
            Hn.log(f"  replay {i}: status {int(status_g.item())}")
            assert int(status_g.item()) == 0 and int(status_e.item()) == 0
            assert torch.equal(ids_g, ids_e), f"replay {i}: ids differ"
            assert torch.equal(cache_g.k, cache_e.k), f"replay {i}: K cache differs"
            assert torch.equal(cache_g.v, cache_e.v), f"replay {i}: V cache differs"
            seen.add(tuple(ids_g.cpu().numpy().ravel().tolist()))
        assert len(seen) > 1, "the replays retrieved the same facts for different queries"
        with pytest.raises(K.ISError) as e:
            K.is_store_remove(st.handle, [0])
        assert e.value.code == -9
    finally:
        del graph
        torch.cuda.synchronize()
        st.destroy()


def test_graph_batch_over_a_large_index(gpu):
    """100 requests x top-50 over 140,001 one-token facts with 1024-dim
    embeddings, captured once and replayed with new queries: the replays run
    the register-resident top-k scan inside the graph and match eager calls
    byte for byte (ids, status, both caches)."""
    import torch
    K = Hn.K
    w = W.WORKLOADS["tiny"].scaled(name="graph_large", n_layers=2, n_kv_heads=1, head_dim=128,
                                   dtype=synth.BF16, n_facts=140001, len_dist=("uniform", 1, 1),
                                   emb_dim=1024, n_req=100, k=50, block_size=16, n_blocks=600,
                                   prefix=(0, 16), theta=1e6, scaling="none")
    n, k = w.n_req, w.k
    st = Hn.make_store(w)
    graph = None
    try:
        rope = Hn.rope_of(w)
        cache_g, cache_e = Hn.make_cache(w), Hn.make_cache(w)
        qs = synth.queries(w.seed + 7, 3 * n, w.emb_dim)
        prefix = synth.prefixes(w.seed, n, w.prefix[0], w.prefix[1])
        need = prefix.astype(np.int64) + k   # one-token facts
        bt = synth.block_tables(w.seed, need, w.block_size, w.n_blocks)
        d_prefix = torch.from_numpy(np.ascontiguousarray(prefix, np.int32)).cuda()
        d_bt = torch.from_numpy(np.ascontiguousarray(bt, np.int32)).cuda()
        q_buf = torch.empty((n, w.emb_dim), dtype=torch.int16, device="cuda")
        ids_g = torch.empty((n, k), dtype=torch.int32, device="cuda")
        ids_e = torch.empty_like(ids_g)
        status_g = torch.ones(1, dtype=torch.int32, device="cuda")
        status_e = torch.ones_like(status_g)

        def call(q, cache, ids, status, stream):
            K.is_retrieve_inject(st.handle, q, n, k, d_prefix, d_bt, cache.desc, rope, status,
                                 ids, stream)

        main = torch.cuda.current_stream()
        q_buf.copy_(torch.from_numpy(qs[0:n].view(np.int16)))
        call(q_buf, cache_g, ids_g, status_g, main)          # sizes the graph workspace
        torch.cuda.synchronize()
        Hn.log(f"graph: capture {n} requests x top-{k} over {w.n_facts} facts")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(main)
        with torch.cuda.graph(graph, stream=side):
            call(q_buf, cache_g, ids_g, status_g, side)
        torch.cuda.synchronize()
        for i in range(3):
            qi = qs[i * n:(i + 1) * n]
            q_buf.copy_(torch.from_numpy(qi.view(np.int16)))
            status_g.fill_(1)
            _refill(cache_g, main.cuda_stream)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            status_e.fill_(1)
            _refill(cache_e, main.cuda_stream)
            call(torch.from_numpy(qi.view(np.int16)).cuda(), cache_e, ids_e, status_e, main)
            torch.cuda.synchronize()
            Hn.log(f"  replay {i}: status {int(status_g.item())}")
            assert int(status_g.item()) == 0 and int(status_e.item()) == 0
            assert torch.equal(ids_g, ids_e), f"replay {i}: ids differ"
            assert torch.equal(cache_g.k, cache_e.k), f"replay {i}: K cache differs"
            assert torch.equal(cache_g.v, cache_e.v), f"replay {i}: V cache differs"
        # the last replay's ids against the oracle on a few queries
        ids = ids_g.cpu().numpy()
        for r in (0, 57, 99):
            exact = np.array([oracle.dot(qi[r], st.emb[f]) for f in ids[r]])
            o_ids, o_sc = oracle.topk(qi[r:r + 1], st.emb, k + 1)
            s_k = o_sc[0, k - 1]
            assert np.all(exact >= s_k - 1e-3), f"query {r}: an id far below the k-th score"
            must = {int(f) for f, s in zip(o_ids[0, :k], o_sc[0, :k]) if s > s_k + 1e-3}
            assert must <= set(ids[r].tolist()), f"query {r}: missing {must - set(ids[r].tolist())}"
    finally:
        del graph
        torch.cuda.synchronize()
        st.destroy()
