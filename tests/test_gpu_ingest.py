"""Store ingest through the C ABI: facts packed from context-window
encodings (is_store_append, is_store_update), checked by injecting them and
comparing with the oracle run on the facts' own rows, and by top-k finding
the appended embeddings."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from tests import harness as Hn

pytestmark = pytest.mark.gpu

L, H, D, B = 4, 2, 128, 16
EMB = 64
SEED = 31
WINDOW = 7


@pytest.fixture(autouse=True)
def _gpu_cleanup(gpu):
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _workload(n_facts):
    return W.WORKLOADS["llama8b_batch"].scaled(name="ingest", n_layers=L, n_kv_heads=H,
                                               head_dim=D, n_facts=n_facts, emb_dim=EMB,
                                               block_size=B, n_blocks=64, seed=SEED)


def _encodings(entities, lens, window, tag):
    """Each fact's rows (from the generator, entity e) behind `window` rows
    of another sequence, per (layer, kv head); returns (encodings back to
    back, the facts' rows back to back)."""
    encs, rows = [], []
    for e, n in zip(entities, lens):
        fact = synth.fact_kv(SEED, tag, int(e), L * H * int(n) * D, synth.BF16).reshape(L, H, n, D)
        pre = synth.fact_kv(SEED, tag, 50_000 + int(e), L * H * window * D,
                            synth.BF16).reshape(L, H, window, D)
        encs.append(np.concatenate([pre, fact], axis=2).reshape(-1))
        rows.append(fact.reshape(-1))
    return np.concatenate(encs), np.concatenate(rows)


def _inject_and_check(st, w, cache, lens_all, ids, rows):
    """Injects facts `ids` (one request, prefix 5) and compares the touched
    blocks with the oracle run on `rows` (fact -> (K, V) store blocks) for
    the facts packed from encodings, the generator's for the rest."""
    import torch
    req_off = np.array([0, len(ids)], np.int32)
    flat = np.asarray(ids, np.int32)
    prefix = np.array([5], np.int32)
    bt = Hn.block_tables_for(w, lens_all, req_off, flat, prefix)
    Hn.gpu_inject(st, cache, req_off, flat, prefix, bt)
    torch.cuda.synchronize()
    n, err = Hn.check_inject_blocks(cache, lens_all, req_off, flat, prefix, bt,
                                    Hn.blocks_of(bt, [0]), rows)
    Hn.log(f"  {n} K elements compared, worst {err:.3g}")


def test_append_update_and_retrieve(gpu):
    import torch
    w = _workload(20)
    lens = W.fact_lengths(w)
    row = L * H * D
    desc, keep = Hn.K.make_desc(L, H, D, synth.BF16, lens, EMB, spare_facts=8, spare_tokens=400)
    h = Hn.K.is_store_create(desc)
    try:
        # the first 20 facts through the plain loader
        Hn.K.is_store_load(h, 0, 20, synth.kv_range(SEED, synth.TAG_K, 0, lens, row, synth.BF16),
                           synth.kv_range(SEED, synth.TAG_V, 0, lens, row, synth.BF16),
                           synth.embeddings(SEED, 0, 20, EMB))
        # six more from window encodings, ragged (1 to 40 tokens)
        new_lens = np.array([3, 17, 1, 40, 9, 25], np.int32)
        ent = np.arange(100, 106)
        k_enc, k_rows = _encodings(ent, new_lens, WINDOW, synth.TAG_K)
        v_enc, v_rows = _encodings(ent, new_lens, WINDOW, synth.TAG_V)
        k_ora = oracle.ingest(L, H, D, new_lens, WINDOW, k_enc)
        v_ora = oracle.ingest(L, H, D, new_lens, WINDOW, v_enc)
        assert np.array_equal(k_ora, k_rows) and np.array_equal(v_ora, v_rows)
        emb_new = synth.embeddings(SEED, 100, 6, EMB)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        Hn.log(f"ingest: append {list(new_lens)} behind a window of {WINDOW}")
        first = Hn.K.is_store_append(h, new_lens, WINDOW, dev(k_enc), dev(v_enc), dev(emb_new))
        torch.cuda.synchronize()
        assert first == 20
        assert Hn.K.is_store_get_info(h).n_facts == 26
        lens_all = np.concatenate([lens, new_lens]).astype(np.int32)
        st = Hn.Store(w, lens_all, None, h, None)
        cut = np.concatenate([[0], np.cumsum(new_lens)]) * row
        rows = {20 + i: (k_ora[cut[i]:cut[i + 1]], v_ora[cut[i]:cut[i + 1]]) for i in range(6)}
        # appended facts injected next to loaded ones
        ids = [22, 3, 25, 20, 23, 11]
        _inject_and_check(st, w, Hn.make_cache(w), lens_all, ids, rows)
        # top-k sees the appended embeddings: each ranks first for itself
        got, _ = Hn.gpu_topk(st, emb_new, 1)
        assert got[:, 0].tolist() == list(range(20, 26))
        # fact 3 replaced in place from a window-free encoding of new values
        Hn.log("ingest: update fact 3")
        k_new, _ = _encodings([200], lens[3:4], 0, synth.TAG_K)
        v_new, _ = _encodings([200], lens[3:4], 0, synth.TAG_V)
        emb3 = synth.embeddings(SEED, 200, 1, EMB)
        Hn.K.is_store_update(h, 3, 0, dev(k_new), dev(v_new), dev(emb3))
        torch.cuda.synchronize()
        rows[3] = (oracle.ingest(L, H, D, lens[3:4], 0, k_new),
                   oracle.ingest(L, H, D, lens[3:4], 0, v_new))
        _inject_and_check(st, w, Hn.make_cache(w), lens_all, ids, rows)
        got, _ = Hn.gpu_topk(st, emb3, 1)
        assert got[0, 0] == 3
        # beyond the spare tokens (400, 95 used): out of memory, nothing appended
        big = np.array([200, 200], np.int32)
        k_big, _ = _encodings([300, 301], big, 0, synth.TAG_K)
        with pytest.raises(Hn.K.ISError) as e:
            Hn.K.is_store_append(h, big, 0, dev(k_big), dev(k_big),
                                 dev(synth.embeddings(SEED, 300, 2, EMB)))
        assert e.value.code == -7
        assert Hn.K.is_store_get_info(h).n_facts == 26
    finally:
        Hn.K.is_store_destroy(h)


def test_append_fp32_head64(gpu):
    """The packing is dtype-blind (rows of head_dim x element size bytes): an
    fp32 store with head_dim 64 (256-byte rows) and 3 kv heads, facts
    appended behind a window of 5, injected and checked against the oracle
    (fp32 K within 1e-5)."""
    import torch
    Lf, Hf, Df, win = 3, 3, 64, 5
    w = W.WORKLOADS["llama8b_batch"].scaled(name="ingest32", n_layers=Lf, n_kv_heads=Hf,
                                            head_dim=Df, dtype=synth.F32, n_facts=6,
                                            emb_dim=0, block_size=16, n_blocks=64, seed=SEED,
                                            scaling="none", theta=10000.0)
    lens = W.fact_lengths(w)
    row = Lf * Hf * Df
    desc, keep = Hn.K.make_desc(Lf, Hf, Df, synth.F32, lens, 0, spare_facts=3, spare_tokens=200)
    h = Hn.K.is_store_create(desc)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    try:
        Hn.K.is_store_load(h, 0, 6, synth.kv_range(SEED, synth.TAG_K, 0, lens, row, synth.F32),
                           synth.kv_range(SEED, synth.TAG_V, 0, lens, row, synth.F32))
        new_lens = np.array([1, 30, 7], np.int32)
        encs = {}
        for tag in (synth.TAG_K, synth.TAG_V):
            parts = []
            for e, n in zip((700, 701, 702), new_lens):
                fact = synth.fact_kv(SEED, tag, e, Lf * Hf * int(n) * Df, synth.F32)
                pre = synth.fact_kv(SEED, tag, 60_000 + e, Lf * Hf * win * Df, synth.F32)
                parts.append(np.concatenate([pre.reshape(Lf, Hf, win, Df),
                                             fact.reshape(Lf, Hf, n, Df)], axis=2).reshape(-1))
            encs[tag] = np.concatenate(parts)
        first = Hn.K.is_store_append(h, new_lens, win, dev(encs[synth.TAG_K]),
                                     dev(encs[synth.TAG_V]))
        torch.cuda.synchronize()
        assert first == 6
        k_ora = oracle.ingest(Lf, Hf, Df, new_lens, win, encs[synth.TAG_K])
        v_ora = oracle.ingest(Lf, Hf, Df, new_lens, win, encs[synth.TAG_V])
        cut = np.concatenate([[0], np.cumsum(new_lens)]) * row
        rows = {6 + i: (k_ora[cut[i]:cut[i + 1]], v_ora[cut[i]:cut[i + 1]]) for i in range(3)}
        lens_all = np.concatenate([lens, new_lens]).astype(np.int32)
        st = Hn.Store(w, lens_all, None, h, None)
        _inject_and_check(st, w, Hn.make_cache(w), lens_all, [7, 2, 8, 6], rows)
    finally:
        Hn.K.is_store_destroy(h)


def test_append_rejected_with_a_host_tier(gpu):
    w = _workload(12)
    lens = W.fact_lengths(w)
    budget = int(lens[:6].sum()) * L * H * D * 2 * 2
    desc, keep = Hn.K.make_desc(L, H, D, synth.BF16, lens, 0, budget)
    h = Hn.K.is_store_create(desc)
    try:
        with pytest.raises(Hn.K.ISError) as e:
            Hn.K.is_store_append(h, np.array([2], np.int32), 0, 16, 16)
        assert e.value.code == -9
    finally:
        Hn.K.is_store_destroy(h)
    desc, keep = Hn.K.make_desc(L, H, D, synth.BF16, lens, 0, budget, spare_facts=1)
    with pytest.raises(Hn.K.ISError) as e:
        Hn.K.is_store_create(desc)
    assert e.value.code == -9
    desc, keep = Hn.K.make_desc(L, H, D, synth.BF16, lens, 0, budget)
    h = Hn.K.is_store_create(desc)
    try:
        with pytest.raises(Hn.K.ISError) as e:
            Hn.K.is_store_remove(h, [0])
        assert e.value.code == -9
    finally:
        Hn.K.is_store_destroy(h)


def _gen_rows(lens, old_ids, new_ids, tag_offset=0):
    """fact -> (K, V) generator rows: new id `n` holds old fact `o`'s rows."""
    row = L * H * D
    return {int(n): (synth.fact_kv(SEED, synth.TAG_K, int(o) + tag_offset, int(lens[o]) * row,
                                   synth.BF16),
                     synth.fact_kv(SEED, synth.TAG_V, int(o) + tag_offset, int(lens[o]) * row,
                                   synth.BF16))
            for n, o in zip(new_ids, old_ids)}


def test_remove_renumbers_and_appends_reuse_the_room(gpu):
    """Eviction: the survivors are renumbered in order (the oracle's
    survivors), top-k and inject see the compacted store, appends fill the
    freed spans first fit (no spare tokens were reserved), and loads into
    facts whose blocks are no longer contiguous land where inject reads."""
    import torch
    n0 = 30
    w = _workload(n0)
    lens = W.fact_lengths(w)
    row = L * H * D
    desc, keep_alive = Hn.K.make_desc(L, H, D, synth.BF16, lens, EMB, spare_facts=4)
    h = Hn.K.is_store_create(desc)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    try:
        emb = synth.embeddings(SEED, 0, n0, EMB)
        Hn.K.is_store_load(h, 0, n0, synth.kv_range(SEED, synth.TAG_K, 0, lens, row, synth.BF16),
                           synth.kv_range(SEED, synth.TAG_V, 0, lens, row, synth.BF16), emb)
        removed = [0, 7, 8, 29, 15]
        Hn.log(f"remove {removed} of {n0}")
        Hn.K.is_store_remove(h, removed)
        keep = oracle.survivors(n0, removed)
        info = Hn.K.is_store_get_info(h)
        assert info.n_facts == len(keep) == 25
        assert info.total_tokens == int(lens[keep].sum())
        lens_now = lens[keep].astype(np.int32)
        st = Hn.Store(w, lens_now, None, h, None)
        q = synth.queries(SEED + 1, 12, EMB)
        ids, sc = Hn.gpu_topk(st, q, 10)
        Hn.check_topk(q, emb[keep], ids, sc, 10)
        got, _ = Hn.gpu_topk(st, emb[keep[[0, 6, 24]]], 1)
        assert got[:, 0].tolist() == [0, 6, 24]
        rows = _gen_rows(lens, keep, range(len(keep)))
        _inject_and_check(st, w, Hn.make_cache(w), lens_now, [0, 6, 24, 5, 13, 20], rows)
        # the freed spans, in arena order: fact 0's, facts 7-8 merged, fact
        # 15's; fact 29's was the arena's end.  Exact fits, first fit.
        new_lens = np.array([lens[0], lens[7] + lens[8], lens[15], lens[29]], np.int32)
        ent = np.arange(400, 404)
        k_enc, _ = _encodings(ent, new_lens, 3, synth.TAG_K)
        v_enc, _ = _encodings(ent, new_lens, 3, synth.TAG_V)
        Hn.log(f"append {list(new_lens)} into the freed room")
        first = Hn.K.is_store_append(h, new_lens, 3, dev(k_enc), dev(v_enc),
                                     dev(synth.embeddings(SEED, 400, 4, EMB)))
        torch.cuda.synchronize()
        assert first == 25
        k_ora = oracle.ingest(L, H, D, new_lens, 3, k_enc)
        v_ora = oracle.ingest(L, H, D, new_lens, 3, v_enc)
        cut = np.concatenate([[0], np.cumsum(new_lens)]) * row
        for i in range(4):
            rows[25 + i] = (k_ora[cut[i]:cut[i + 1]], v_ora[cut[i]:cut[i + 1]])
        lens_now = np.concatenate([lens_now, new_lens]).astype(np.int32)
        st = Hn.Store(w, lens_now, None, h, None)
        _inject_and_check(st, w, Hn.make_cache(w), lens_now, [26, 5, 25, 28, 6, 27, 0], rows)
        got, _ = Hn.gpu_topk(st, synth.embeddings(SEED, 400, 4, EMB), 1)
        assert got[:, 0].tolist() == [25, 26, 27, 28]
        # the arena is full now
        with pytest.raises(Hn.K.ISError) as e:
            one = np.array([1], np.int32)
            Hn.K.is_store_append(h, one, 0, dev(np.zeros(row, np.uint16)),
                                 dev(np.zeros(row, np.uint16)), dev(np.zeros(EMB, np.uint16)))
        assert e.value.code == -7
        # new values for facts 4..9 (old 5, 6, 9, 10, 11, 12): their blocks
        # are no longer one span
        sub = np.arange(4, 10)
        k_h = np.concatenate([synth.fact_kv(SEED, synth.TAG_K, 900 + int(f), int(lens_now[f]) * row,
                                            synth.BF16) for f in sub])
        v_h = np.concatenate([synth.fact_kv(SEED, synth.TAG_V, 900 + int(f), int(lens_now[f]) * row,
                                            synth.BF16) for f in sub])
        Hn.K.is_store_load(h, 4, 6, k_h, v_h)
        cut = np.concatenate([[0], np.cumsum(lens_now[sub])]) * row
        for i, f in enumerate(sub):
            rows[int(f)] = (k_h[cut[i]:cut[i + 1]], v_h[cut[i]:cut[i + 1]])
        _inject_and_check(st, w, Hn.make_cache(w), lens_now, [9, 4, 26, 5, 7, 8, 6], rows)
        # refusals change nothing
        for bad, code in (([3, 3], -1), ([29], -2), ([-1], -2)):
            with pytest.raises(Hn.K.ISError) as e:
                Hn.K.is_store_remove(h, bad)
            assert e.value.code == code
        assert Hn.K.is_store_get_info(h).n_facts == 29
        # everything out, then one fact back in
        Hn.K.is_store_remove(h, np.arange(29))
        assert Hn.K.is_store_get_info(h).n_facts == 0
        with pytest.raises(Hn.K.ISError):
            Hn.gpu_topk(st, q[:1], 1)
        k_enc, _ = _encodings([500], [20], 0, synth.TAG_K)
        assert Hn.K.is_store_append(h, np.array([20], np.int32), 0, dev(k_enc), dev(k_enc),
                                    dev(synth.embeddings(SEED, 500, 1, EMB))) == 0
        torch.cuda.synchronize()
        st = Hn.Store(w, np.array([20], np.int32), None, h, None)
        got, _ = Hn.gpu_topk(st, synth.embeddings(SEED, 500, 1, EMB), 1)
        assert got[0, 0] == 0
    finally:
        Hn.K.is_store_destroy(h)
