"""is_topk_noalloc (scratch in a fixed per-GPU device array, no allocation)
against is_topk on the same inputs: two calls in a row, the second smaller
(another store, a width that needs padded queries), then the refusal of a
store above its limit.  Both entry points run the same kernels, so their
ids and scores must agree bit for bit; the oracle checks the ids."""
import numpy as np
import pytest

import synth
from synth import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu

BASE = W.WORKLOADS["tiny"].scaled(name="noalloc", n_layers=1, n_kv_heads=1, head_dim=128,
                                  dtype=synth.BF16, len_dist=("uniform", 1, 2))


def _both(st, q_bits, k):
    """(ids, scores) of is_topk and of is_topk_noalloc, the latter first."""
    import torch
    n_q = q_bits.shape[0]
    q = torch.from_numpy(q_bits.view(np.int16)).cuda()
    out = []
    for fn in (Hn.K.is_topk_noalloc, Hn.K.is_topk):
        ids = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((n_q, k), -7.0, dtype=torch.float32, device="cuda")
        fn(st.handle, q, n_q, k, ids, sc, torch.cuda.current_stream())
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), sc.cpu().numpy()))
    return out


def test_topk_noalloc_matches_topk(gpu):
    # call 1: 65,536 facts (the largest store it takes) at width 1024, 130
    # queries (two groups of the scratch, one after the other), k = 50; the
    # first group's 8.4M scores take the sample, bound and stream, whose
    # sample codes also live in the fixed scratch
    w1 = BASE.scaled(n_facts=65_536, emb_dim=1024)
    Hn.log("no-alloc top-k: 65,536 facts x 1024, 130 queries, k=50")
    st = Hn.make_store(w1)
    try:
        q1 = synth.queries(11, 130, 1024)
        (ia, sa), (ib, sb) = _both(st, q1, 50)
        assert np.array_equal(ia, ib) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        Hn.check_topk(q1, st.emb, ia, sa, 50, queries=range(0, 130, 13))
    finally:
        st.destroy()
    # call 2, smaller: 1,000 facts at width 992 (queries padded to 1024 in
    # the scratch), 5 queries, k = 7
    w2 = BASE.scaled(n_facts=1_000, emb_dim=992)
    Hn.log("no-alloc top-k: 1,000 facts x 992, 5 queries, k=7")
    st = Hn.make_store(w2)
    try:
        q2 = synth.queries(12, 5, 992)
        (ia, sa), (ib, sb) = _both(st, q2, 7)
        assert np.array_equal(ia, ib) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        Hn.check_topk(q2, st.emb, ia, sa, 7)
    finally:
        st.destroy()


def test_topk_noalloc_refuses_large_store(gpu):
    import torch
    w = BASE.scaled(n_facts=65_537, emb_dim=32, len_dist=("uniform", 1, 1))
    st = Hn.make_store(w)
    try:
        q = torch.from_numpy(synth.queries(13, 2, 32).view(np.int16)).cuda()
        ids = torch.full((2, 3), -7, dtype=torch.int32, device="cuda")
        sc = torch.zeros((2, 3), dtype=torch.float32, device="cuda")
        with pytest.raises(Hn.K.ISError) as e:
            Hn.K.is_topk_noalloc(st.handle, q, 2, 3, ids, sc, torch.cuda.current_stream())
        assert e.value.code == -9 and "65,536" in str(e.value)
        torch.cuda.synchronize()
        assert bool((ids == -7).all())
    finally:
        st.destroy()
