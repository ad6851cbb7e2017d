"""Shared GPU-test, smoke and bench plumbing: builds stores and caches from
the seeded generator, calls the library through its C ABI, and compares with
the oracle.  The oracle is imported only by the checking helpers, so the
bench's GPU legs, which use the builders, never load it.

Tolerances (what the GPU path must meet against the oracle):
  V rows, slot placement, untouched cache bytes   bit-exact
  rotated K, bf16 cache    |gpu - ref| <= max(ulp_bf16(ref), 2^-15)
  rotated K, fp32 cache    |gpu - ref| <= 1e-5
  top-k ids                exact wherever the oracle's score gap > 1e-3
"""
from __future__ import annotations

import os
import sys
import time
from dataclasses import dataclass

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cache_injection_is_amd as K  # noqa: E402
import synth  # noqa: E402
from synth import workloads as W  # noqa: E402

GAP = 1e-3
SENTINEL_SEED_K, SENTINEL_SEED_V = 101, 202


def log(msg: str) -> None:
    print(msg, flush=True)


def torch_mod():
    import torch
    return torch


# ------------------------------------------------------------------ store

@dataclass
class Store:
    w: W.Workload
    lens: np.ndarray
    tok_off: np.ndarray
    handle: int
    emb: np.ndarray | None

    def destroy(self):
        if self.handle:
            K.is_store_destroy(self.handle)
            self.handle = 0


def rope_of(w: W.Workload) -> "K.is_rope":
    return K.make_rope(w.theta, w.scaling, w.rope_factor, w.rope_low, w.rope_high, w.rope_orig)


def oracle_freqs(w: W.Workload) -> np.ndarray:
    import oracle
    return oracle.rope_freqs(w.head_dim, w.theta, w.scaling, w.rope_factor, w.rope_low,
                             w.rope_high, w.rope_orig)


def make_store(w: W.Workload, lens: np.ndarray | None = None, fill: str = "gpu",
               hbm_budget: int = -1, chunk_bytes: int = 1 << 30) -> Store:
    """Creates the store and fills K/V (on the GPU in chunks, or from host
    arrays) and the embeddings."""
    torch = torch_mod()
    if lens is None:
        lens = W.fact_lengths(w)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    tok_off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=tok_off[1:])
    emb = W.fact_embeddings(w) if w.emb_dim else None
    desc, keep = K.make_desc(w.n_layers, w.n_kv_heads, w.head_dim, w.dtype, lens, w.emb_dim,
                             hbm_budget)
    h = K.is_store_create(desc)
    s = Store(w, lens, tok_off, h, emb)
    try:
        row = w.row_elems
        es = w.elem_size
        if fill == "host":
            Kh = synth.kv_range(w.seed, synth.TAG_K, 0, lens, row, w.dtype)
            Vh = synth.kv_range(w.seed, synth.TAG_V, 0, lens, row, w.dtype)
            K.is_store_load(h, 0, len(lens), Kh, Vh, None)
        else:
            max_elems = max(chunk_bytes // es, int(lens.max()) * row)
            buf_k = torch.empty(max_elems * es, dtype=torch.uint8, device="cuda")
            buf_v = torch.empty(max_elems * es, dtype=torch.uint8, device="cuda")
            stream = torch.cuda.current_stream()
            f0 = 0
            n = len(lens)
            while f0 < n:
                # facts [f0, f1) fit the chunk
                lim = tok_off[f0] + max_elems // row
                f1 = int(np.searchsorted(tok_off, lim, side="right")) - 1
                f1 = max(f1, f0 + 1)
                f1 = min(f1, n)
                off = (tok_off[f0:f1 + 1] - tok_off[f0]) * row
                d_off = torch.from_numpy(off.astype(np.int64)).cuda()
                total = int(off[-1])
                synth.gpu_fill_kv(w.seed, synth.TAG_K, f0, d_off, total, w.dtype,
                                  buf_k.data_ptr(), stream.cuda_stream)
                synth.gpu_fill_kv(w.seed, synth.TAG_V, f0, d_off, total, w.dtype,
                                  buf_v.data_ptr(), stream.cuda_stream)
                torch.cuda.synchronize()
                K.is_store_load(h, f0, f1 - f0, buf_k, buf_v, None, src_on_device=True)
                f0 = f1
            del buf_k, buf_v
        if emb is not None:
            K.is_store_load(h, 0, len(lens), None, None, emb)
    except Exception:
        s.destroy()
        raise
    return s


# ------------------------------------------------------------------ cache

@dataclass
class Cache:
    w: W.Workload
    n_blocks: int
    layout: str              # "NHD" or "HND"
    k: object                # torch uint8 tensors
    v: object
    strides: tuple

    @property
    def desc(self) -> "K.is_cache":
        return K.make_cache(self.k, self.v, self.strides, self.w.block_size, self.n_blocks,
                            self.w.dtype)

    def block_bytes(self) -> int:
        w = self.w
        return w.block_size * w.n_kv_heads * w.head_dim * w.elem_size

    def layer_bytes(self) -> int:
        return self.n_blocks * self.block_bytes()


def make_cache(w: W.Workload, n_blocks: int | None = None, layout: str = "NHD") -> Cache:
    torch = torch_mod()
    nb = n_blocks or w.n_blocks
    B, H, d = w.block_size, w.n_kv_heads, w.head_dim
    n = w.n_layers * nb * B * H * d * w.elem_size
    k = torch.empty(n, dtype=torch.uint8, device="cuda")
    v = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    synth.gpu_sentinel(SENTINEL_SEED_K, k.data_ptr(), n, st)
    synth.gpu_sentinel(SENTINEL_SEED_V, v.data_ptr(), n, st)
    if layout == "NHD":
        strides = (nb * B * H * d, B * H * d, H * d, d)
    else:
        strides = (nb * B * H * d, H * B * d, d, B * d)
    return Cache(w, nb, layout, k, v, strides)


# ------------------------------------------------------------------- calls

def gpu_topk(store: Store, q_bits: np.ndarray, k: int):
    torch = torch_mod()
    q = torch.from_numpy(q_bits.view(np.int16)).cuda()
    n_q = q_bits.shape[0]
    ids = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((n_q, k), dtype=torch.float32, device="cuda")
    K.is_topk(store.handle, q, n_q, k, ids, sc, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def requests_from_ids(ids: np.ndarray):
    """[n_req][k] id matrix -> CSR (req_off, flat ids)."""
    n_req, k = ids.shape
    req_off = np.arange(0, (n_req + 1) * k, k, dtype=np.int32)
    return req_off, np.ascontiguousarray(ids.reshape(-1), dtype=np.int32)


def block_tables_for(w: W.Workload, lens, req_off, flat_ids, prefix, n_blocks=None):
    need = np.array([int(prefix[r]) + int(lens[flat_ids[req_off[r]:req_off[r + 1]]].sum())
                     for r in range(len(prefix))], dtype=np.int64)
    return synth.block_tables(w.seed, need, w.block_size, n_blocks or w.n_blocks)


def gpu_inject(store: Store, cache: Cache, req_off, flat_ids, prefix, bt, stream=None):
    torch = torch_mod()
    K.is_inject(store.handle, req_off, flat_ids, prefix, bt, cache.desc, rope_of(store.w),
                stream or torch.cuda.current_stream())


# ------------------------------------------------------------ parity: top-k

def check_topk(q_bits, e_bits, gpu_ids, gpu_scores, k, queries=None):
    """Checks the GPU top-k against the exact fp64 oracle (see module doc)."""
    qsel = list(range(q_bits.shape[0])) if queries is None else list(queries)
    # the oracle's (k+1)-th score bounds what may enter at the boundary
    import oracle
    o_ids1, o_sc1 = oracle.topk(q_bits[qsel], e_bits, min(k + 1, e_bits.shape[0]))
    o_ids, o_sc = o_ids1[:, :k], o_sc1[:, :k]
    for n, qi in enumerate(qsel):
        g = gpu_ids[qi]
        assert len(set(g.tolist())) == k, f"query {qi}: duplicate ids"
        assert np.all(g >= 0) and np.all(g < e_bits.shape[0]), f"query {qi}: id out of range"
        s_k = o_sc[n, k - 1]
        exact = np.array([oracle.dot(q_bits[qi], e_bits[f]) for f in g])
        assert np.all(np.abs(exact - gpu_scores[qi]) <= GAP), f"query {qi}: score error"
        must = set(int(f) for f, s in zip(o_ids[n], o_sc[n]) if s > s_k + GAP)
        assert must <= set(g.tolist()), f"query {qi}: missing {must - set(g.tolist())}"
        assert np.all(exact >= s_k - GAP), f"query {qi}: id far below the k-th score"
        # GPU order: its own scores descending, ties to the lower id
        gs = gpu_scores[qi]
        for i in range(k - 1):
            assert gs[i] > gs[i + 1] or (gs[i] == gs[i + 1] and g[i] < g[i + 1]), \
                f"query {qi}: order at rank {i}"
        # ranks isolated by more than the gap on both sides match exactly
        ext = np.concatenate([[np.inf], o_sc1[n], [-np.inf]])[:k + 2]
        for i in range(k):
            if ext[i] - ext[i + 1] > GAP and ext[i + 1] - ext[i + 2] > GAP:
                assert g[i] == o_ids[n, i], f"query {qi}: rank {i} differs"
    return o_ids


# ----------------------------------------------------------- parity: inject

def _as_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    with np.errstate(invalid="ignore"):      # sentinel bytes may spell NaNs
        if dtype == synth.F32:
            return a.view(np.float32).astype(np.float64)
        return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def k_tolerance(ref: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == synth.F32:
        return np.full(ref.shape, 1e-5)
    m, ex = np.frexp(np.abs(ref))
    ulp = np.where(ref == 0, 0.0, np.ldexp(1.0, ex - 8))
    return np.maximum(ulp, 2.0 ** -15)


def generator_blocks(w: W.Workload, lens, facts, tag: int) -> np.ndarray:
    """K (tag 1) or V (tag 2) blocks of `facts`, back to back, made by the
    generator's device build (bit-equal to its host build; the host build is
    slower at full size) and copied to the host.  The generator is the input
    module both sides share; no part of the library is involved."""
    torch = torch_mod()
    facts = np.asarray(facts, dtype=np.int64)
    row = w.row_elems
    n = lens[facts].astype(np.int64) * row
    off = np.zeros(len(facts) + 1, dtype=np.int64)
    np.cumsum(n, out=off[1:])
    out = torch.empty(max(int(off[-1]), 1) * w.elem_size, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    i = 0
    while i < len(facts):
        j = i + 1                      # a run of consecutive fact ids: one fill
        while j < len(facts) and facts[j] == facts[j - 1] + 1:
            j += 1
        d_off = torch.from_numpy(off[i:j + 1] - off[i]).cuda()
        synth.gpu_fill_kv(w.seed, tag, int(facts[i]), d_off, int(off[j] - off[i]), w.dtype,
                          out.data_ptr() + int(off[i]) * w.elem_size, st)
        i = j
    torch.cuda.synchronize()
    return out[:int(off[-1]) * w.elem_size].cpu().numpy().view(synth.kv_dtype_np(w.dtype))


def oracle_blocks(w: W.Workload, lens, req_off, flat_ids, prefix, bt, blocks, layout,
                  cache_nb, rows=None, touched_only=False):
    """Runs the oracle on the given requests into a compact host cache that
    holds only `blocks` (physical ids, remapped to 0..m-1), initialised to
    the same sentinel the GPU cache was filled with (to zeros when only the
    touched rows will be compared; the K/V inputs then come from the
    generator's device build).  Returns (k, v) arrays [L][m][B*H*d] in the
    cache's layout, raw bytes.  `rows` maps a fact id to its (K, V) store
    blocks where they are not the generator's."""
    L, H, d, B, es = w.n_layers, w.n_kv_heads, w.head_dim, w.block_size, w.elem_size
    uniq = np.unique(flat_ids)
    remap = {int(f): i for i, f in enumerate(uniq)}
    sub_lens = lens[uniq]
    sub_off = np.zeros(len(uniq) + 1, dtype=np.int64)
    np.cumsum(sub_lens, out=sub_off[1:])
    row = w.row_elems
    empty = [np.zeros(1, dtype=synth.kv_dtype_np(w.dtype))]
    rows = rows or {}

    def block(f, tag, i):
        if int(f) in rows:
            return rows[int(f)][i]
        return synth.fact_kv(w.seed, tag, int(f), int(lens[f]) * row, w.dtype)
    if touched_only and not rows and len(uniq):
        Kh = generator_blocks(w, lens, uniq, synth.TAG_K)
        Vh = generator_blocks(w, lens, uniq, synth.TAG_V)
    else:
        Kh = np.concatenate([block(f, synth.TAG_K, 0) for f in uniq] or empty)
        Vh = np.concatenate([block(f, synth.TAG_V, 1) for f in uniq] or empty)
    blocks = np.asarray(blocks, dtype=np.int64)
    bmap = {int(b): i for i, b in enumerate(blocks)}
    bt_c = np.vectorize(lambda b: bmap.get(int(b), -1))(bt).astype(np.int32)
    m = len(blocks)
    blk_words = B * H * d * es // 4
    if touched_only:
        kc = np.zeros((L, m, blk_words), dtype=np.uint32)
        vc = np.zeros((L, m, blk_words), dtype=np.uint32)
    else:
        kc = np.empty((L, m, blk_words), dtype=np.uint32)
        vc = np.empty((L, m, blk_words), dtype=np.uint32)
        for l in range(L):
            for i, b in enumerate(blocks):
                first = (l * cache_nb + int(b)) * blk_words
                kc[l, i] = synth.sentinel_host(SENTINEL_SEED_K, first, blk_words)
                vc[l, i] = synth.sentinel_host(SENTINEL_SEED_V, first, blk_words)
    if layout == "NHD":
        strides = (m * B * H * d, B * H * d, H * d, d)
    else:
        strides = (m * B * H * d, H * B * d, d, B * d)
    ids_c = np.array([remap[int(f)] for f in flat_ids], dtype=np.int32)
    import oracle
    oracle.inject(L, H, d, w.dtype, Kh, Vh, sub_off, req_off, ids_c, prefix, bt_c, B, m,
                  kc, vc, strides, oracle_freqs(w))
    return kc, vc


def touched_mask(w: W.Workload, lens, req_off, flat_ids, prefix, bt, blocks, layout):
    """Byte mask [m][B*H*d*es] of the elements the oracle writes (per layer
    the same), from the oracle's slot map."""
    B, H, d, es = w.block_size, w.n_kv_heads, w.head_dim, w.elem_size
    import oracle
    slots = oracle.token_slots(req_off, flat_ids, lens, prefix, bt, B)
    bidx = {int(b): i for i, b in enumerate(blocks)}
    mask = np.zeros((len(blocks), B, H, d), dtype=bool) if layout == "NHD" else \
        np.zeros((len(blocks), H, B, d), dtype=bool)
    for s in slots:
        i = bidx.get(int(s) // B)
        if i is None:
            continue
        if layout == "NHD":
            mask[i, int(s) % B] = True
        else:
            mask[i, :, int(s) % B] = True
    return mask.reshape(len(blocks), -1), len(slots)


def gpu_blocks(cache: Cache, blocks):
    """Copies the given physical blocks of every layer to the host:
    ([L][m][block bytes] uint8 for K, same for V)."""
    torch = torch_mod()
    w = cache.w
    bb = cache.block_bytes()
    kk = cache.k.view(w.n_layers, cache.n_blocks, bb)
    vv = cache.v.view(w.n_layers, cache.n_blocks, bb)
    idx = torch.as_tensor(np.asarray(blocks, dtype=np.int64), device="cuda")
    return (kk.index_select(1, idx).cpu().numpy(), vv.index_select(1, idx).cpu().numpy())


def check_inject_blocks(cache: Cache, lens, req_off, flat_ids, prefix, bt, blocks, rows=None,
                        touched_only=False):
    """Element-by-element comparison of the GPU cache and the oracle on the
    given physical blocks (all layers).  Returns (#elements compared, max K
    error).  `rows`: as for oracle_blocks.  With touched_only the comparison
    covers the rows the requests write (V bit-exact, K within tolerance) and
    leaves the untouched rows to check_untouched, which covers the whole
    cache on the device."""
    w = cache.w
    es = w.elem_size
    kc_o, vc_o = oracle_blocks(w, lens, req_off, flat_ids, prefix, bt, blocks, cache.layout,
                               cache.n_blocks, rows, touched_only)
    kg, vg = gpu_blocks(cache, blocks)
    mask_e, _ = touched_mask(w, lens, req_off, flat_ids, prefix, bt, blocks, cache.layout)
    L, m = w.n_layers, len(blocks)
    ko = kc_o.view(np.uint8).reshape(L, m, -1)
    vo = vc_o.view(np.uint8).reshape(L, m, -1)
    mask_b = np.repeat(mask_e, es, axis=1)
    if touched_only:
        for l in range(L):
            assert np.array_equal(vg[l][mask_b], vo[l][mask_b]), f"V differs (layer {l})"
    else:
        # V and every untouched byte: bit-exact
        assert np.array_equal(vg, vo), "V cache differs from the oracle"
        for l in range(L):
            assert np.array_equal(kg[l][~mask_b], ko[l][~mask_b]), \
                f"untouched K bytes changed (layer {l})"
    ew = 4 if w.dtype == synth.F32 else 2
    ref = _as_f64(np.ascontiguousarray(ko).view(f"u{ew}").reshape(L, m, -1)[:, mask_e], w.dtype)
    got = _as_f64(np.ascontiguousarray(kg).view(f"u{ew}").reshape(L, m, -1)[:, mask_e], w.dtype)
    tol = k_tolerance(ref, w.dtype)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"rotated K off by more than the tolerance at {int(bad.sum())} of "
                           f"{bad.size} elements; worst {float(err.max()):.3g}")
    return bad.size, float(err.max()) if err.size else 0.0


def blocks_of(bt, req_rows) -> np.ndarray:
    rows = bt[np.asarray(req_rows)]
    return np.unique(rows[rows >= 0])


# -------------------------------------------------------------------- smoke

def smoke() -> None:
    """Tiny workload on cuda:0: top-k, then inject, each checked against the
    oracle."""
    torch = torch_mod()
    assert torch.cuda.is_available(), "smoke needs a GPU"
    w = W.WORKLOADS["tiny"]
    log("smoke: tiny workload, top-k + inject through the C ABI")
    st = make_store(w, fill="host")
    try:
        q = W.query_embeddings(w)
        ids, sc = gpu_topk(st, q, w.k)
        o_ids = check_topk(q, st.emb, ids, sc, w.k)
        req_off, flat = requests_from_ids(o_ids)
        prefix = W.request_prefixes(w)
        bt = synth.permutation(w.seed, w.n_blocks)[None, :].copy()
        cache = make_cache(w)
        gpu_inject(st, cache, req_off, flat, prefix, bt)
        torch.cuda.synchronize()
        n, err = check_inject_blocks(cache, st.lens, req_off, flat, prefix, bt,
                                     np.arange(w.n_blocks))
        log(f"smoke: ok (top-{w.k} ids {ids[0].tolist()}, {n} rotated K elements, "
            f"max |err| {err:.2e})")
    finally:
        st.destroy()


def check_untouched(cache: Cache, written_slots: np.ndarray) -> None:
    """Every cache row (layer, slot) that no injected token maps to must
    still hold its sentinel, bit for bit: checked on the whole cache by the
    generator's device check against a row mask built from the oracle's
    slot list.  NHD layout only (a slot's heads form one row)."""
    torch = torch_mod()
    assert cache.layout == "NHD"
    w = cache.w
    n_rows_layer = cache.n_blocks * w.block_size
    mask = torch.zeros((w.n_layers, n_rows_layer), dtype=torch.uint8, device="cuda")
    if len(written_slots):
        idx = torch.as_tensor(np.asarray(written_slots, dtype=np.int64), device="cuda")
        mask[:, idx] = 1
    row_bytes = w.n_kv_heads * w.head_dim * w.elem_size
    bad = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    n = cache.k.numel()
    synth.gpu_sentinel_check(SENTINEL_SEED_K, cache.k.data_ptr(), n, row_bytes, mask.data_ptr(),
                             bad.data_ptr(), st)
    synth.gpu_sentinel_check(SENTINEL_SEED_V, cache.v.data_ptr(), n, row_bytes, mask.data_ptr(),
                             bad.data_ptr() + 8, st)
    torch.cuda.synchronize()
    k_bad, v_bad = (int(x) for x in bad.cpu())
    assert k_bad == 0 and v_bad == 0, f"untouched rows changed: {k_bad} K words, {v_bad} V words"
