"""ORACLE -- test infrastructure only.

A plain fp64 CPU statement of the retrieve-and-inject path (oracle.c), with
ctypes wrappers.  Only the tests, the smoke check and the bench's CPU-baseline
leg use it; the GPU library neither imports nor links it, and it shares no
code with the library.

What each function follows ("InferScale: GPU-Native KV Injection for
Personalized LLM Serving", gist.science explainer, technical summary):
  rope_freqs, rotate   Online phase, dynamic rotation of stored pre-RoPE keys
                       (textbook RoPE, rotate-half; Llama-3.1 scaling rule)
  positions            Online phase, facts composed into one contiguous
                       segment (after the request's prefix)
  token_slots, inject  Online phase, scatter-copy into the paged KV cache
  topk                 Contributions, GPU-resident retrieval (exact
                       inner-product top-k stands in for the index)
  attend               Online phase, query-only prefill over the cache that
                       holds the injected facts (Theorem 6 end to end)
  ingest               Offline phase, context-window encoding: only the
                       fact's own tokens' K/V are kept
  survivors            store maintenance (the pages define the store by what
                       it holds; eviction is plain removal with the survivors
                       renumbered in order)
Every function is pinned by tests/test_oracle_pins.py against closed forms,
invariants, library routines and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_SO points the wrapper at another build (the mutant tests use it).
SO = os.environ.get("ORACLE_SO") or os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
SCALING = {"none": 0, "llama3": 1}


def build() -> None:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "oracle.c"), "-o", SO, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stderr}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            build()
        L = ctypes.CDLL(SO)
        c = ctypes
        L.or_half_to_double.argtypes = [c.c_uint16]
        L.or_half_to_double.restype = c.c_double
        L.or_double_to_bf16.argtypes = [c.c_double]
        L.or_double_to_bf16.restype = c.c_uint16
        L.or_llama3_scale.argtypes = [c.c_double] * 5
        L.or_llama3_scale.restype = c.c_double
        L.or_rope_freqs.argtypes = [c.c_int, c.c_double, c.c_int, c.c_double,
                                    c.c_double, c.c_double, c.c_double, c.c_void_p]
        L.or_rotate.argtypes = [c.c_void_p, c.c_int, c.c_double, c.c_void_p,
                                c.c_void_p]
        L.or_topk.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int64,
                              c.c_int, c.c_void_p, c.c_void_p]
        L.or_topk.restype = c.c_int
        L.or_positions.argtypes = [c.c_int] + [c.c_void_p] * 5
        L.or_inject.argtypes = ([c.c_int] * 4 + [c.c_void_p] * 3 + [c.c_int64, c.c_int]
                                + [c.c_void_p] * 4 + [c.c_int, c.c_int, c.c_int64]
                                + [c.c_void_p] * 2 + [c.c_int64] * 4 + [c.c_void_p])
        L.or_inject.restype = c.c_int
        L.or_token_slots.argtypes = [c.c_int] + [c.c_void_p] * 5 + [c.c_int, c.c_int, c.c_void_p]
        L.or_token_slots.restype = c.c_int64
        L.or_dot.argtypes = [c.c_void_p, c.c_void_p, c.c_int64]
        L.or_dot.restype = c.c_double
        L.or_attend.argtypes = ([c.c_int] * 5 + [c.c_void_p, c.c_int, c.c_int]
                                + [c.c_void_p] * 4 + [c.c_int, c.c_int, c.c_int64]
                                + [c.c_void_p] * 2 + [c.c_int64] * 4 + [c.c_void_p] * 2)
        L.or_attend.restype = c.c_int
        L.or_ingest.argtypes = [c.c_int] * 5 + [c.c_void_p, c.c_int, c.c_void_p, c.c_void_p]
        L.or_set_threads.argtypes = [c.c_int]
        L.or_max_threads.restype = c.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def half_to_double(bits: int) -> float:
    return lib().or_half_to_double(bits)


def double_to_bf16(x: float) -> int:
    return lib().or_double_to_bf16(x)


def llama3_scale(f: float, factor=8.0, low=1.0, high=4.0, orig=8192.0) -> float:
    return lib().or_llama3_scale(f, factor, low, high, orig)


def rope_freqs(d: int, theta: float, scaling: str = "none", factor=8.0, low=1.0,
               high=4.0, orig=8192.0) -> np.ndarray:
    out = np.empty(d // 2, dtype=np.float64)
    lib().or_rope_freqs(d, theta, SCALING[scaling], factor, low, high, orig, _p(out))
    return out


def rotate(x: np.ndarray, p: float, freqs: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = np.ascontiguousarray(freqs, dtype=np.float64)
    y = np.empty_like(x)
    lib().or_rotate(_p(x), len(x), float(p), _p(f), _p(y))
    return y


def topk(q_bits: np.ndarray, e_bits: np.ndarray, k: int):
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    e = np.ascontiguousarray(e_bits, dtype=np.uint16)
    n_q, dim = q.shape
    n_f = e.shape[0]
    assert e.shape[1] == dim
    ids = np.empty((n_q, k), dtype=np.int32)
    scores = np.empty((n_q, k), dtype=np.float64)
    if lib().or_topk(_p(q), _p(e), n_q, n_f, dim, k, _p(ids), _p(scores)) != 0:
        raise ValueError("bad top-k arguments")
    return ids, scores


def positions(req_off, fact_ids, fact_len, prefix) -> np.ndarray:
    req_off = np.ascontiguousarray(req_off, dtype=np.int32)
    fact_ids = np.ascontiguousarray(fact_ids, dtype=np.int32)
    fact_len = np.ascontiguousarray(fact_len, dtype=np.int32)
    prefix = np.ascontiguousarray(prefix, dtype=np.int32)
    start = np.empty(len(fact_ids), dtype=np.int64)
    lib().or_positions(len(prefix), _p(req_off), _p(fact_ids), _p(fact_len),
                       _p(prefix), _p(start))
    return start


def token_slots(req_off, fact_ids, fact_len, prefix, block_tables, block_size) -> np.ndarray:
    """Cache slot of every injected token, in segment order."""
    req_off = np.ascontiguousarray(req_off, dtype=np.int32)
    fact_ids = np.ascontiguousarray(fact_ids, dtype=np.int32)
    fact_len = np.ascontiguousarray(fact_len, dtype=np.int32)
    prefix = np.ascontiguousarray(prefix, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = int(fact_len[fact_ids].sum()) if len(fact_ids) else 0
    out = np.empty(max(n, 1), dtype=np.int64)
    got = lib().or_token_slots(len(prefix), _p(req_off), _p(fact_ids), _p(fact_len), _p(prefix),
                               _p(bt), bt.shape[1], block_size, _p(out))
    if got < 0:
        raise ValueError("block table too short")
    return out[:got]


def dot(a_bits: np.ndarray, b_bits: np.ndarray) -> float:
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    return lib().or_dot(_p(a), _p(b), len(a))


def inject(n_layers, n_heads, d, dtype, k_store, v_store, tok_off, req_off, fact_ids,
           prefix, block_tables, block_size, n_blocks, k_cache, v_cache, strides,
           freqs) -> None:
    """Writes into the host caches k_cache / v_cache (numpy, modified in
    place).  strides = (layer, block, slot, head) in elements."""
    tok_off = np.ascontiguousarray(tok_off, dtype=np.int64)
    req_off = np.ascontiguousarray(req_off, dtype=np.int32)
    fact_ids = np.ascontiguousarray(fact_ids, dtype=np.int32)
    prefix = np.ascontiguousarray(prefix, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    f = np.ascontiguousarray(freqs, dtype=np.float64)
    rc = lib().or_inject(n_layers, n_heads, d, dtype, _p(k_store), _p(v_store),
                         _p(tok_off), len(tok_off) - 1, len(prefix), _p(req_off),
                         _p(fact_ids), _p(prefix), _p(bt), bt.shape[1], block_size,
                         n_blocks, _p(k_cache), _p(v_cache), *strides, _p(f))
    if rc != 0:
        raise ValueError("oracle inject: index out of range")


def attend(n_layers, n_kv_heads, n_q_heads, d, dtype, q, qpos, ctx_begin, ctx_end,
           block_tables, block_size, n_blocks, k_cache, v_cache, strides, freqs) -> np.ndarray:
    """Query-only attention over a paged host cache (see or_attend).  q:
    [n_layers][n_req][n_qtok][n_q_heads][d] raw dtype elements (uint16 bf16
    bits or float32); returns fp64 of the same shape."""
    q = np.ascontiguousarray(q)
    n_req, n_qtok = q.shape[1], q.shape[2]
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    cb = np.ascontiguousarray(ctx_begin, dtype=np.int32)
    ce = np.ascontiguousarray(ctx_end, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    f = np.ascontiguousarray(freqs, dtype=np.float64)
    out = np.zeros(q.shape, dtype=np.float64)
    rc = lib().or_attend(n_layers, n_kv_heads, n_q_heads, d, dtype, _p(q), n_req, n_qtok,
                         _p(qpos), _p(cb), _p(ce), _p(bt), bt.shape[1], block_size, n_blocks,
                         _p(np.ascontiguousarray(k_cache)), _p(np.ascontiguousarray(v_cache)),
                         *strides, _p(f), _p(out))
    if rc != 0:
        raise ValueError("oracle attend: position outside the block table or cache")
    return out


def ingest(n_layers, n_heads, d, lens, window, enc) -> np.ndarray:
    """Store blocks of n facts from their window encodings (see or_ingest);
    enc: 1-D array of the encodings back to back (uint16 bf16 bits or
    float32); returns the same dtype."""
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    enc = np.ascontiguousarray(enc)
    out = np.empty(int(lens.sum()) * n_layers * n_heads * d, dtype=enc.dtype)
    lib().or_ingest(n_layers, n_heads, d, enc.itemsize, len(lens), _p(lens), window, _p(enc),
                    _p(out))
    return out


def survivors(n_facts: int, removed) -> np.ndarray:
    """Eviction of `removed` (distinct ids in [0, n_facts)) from a store of
    n_facts facts: the old ids of the facts that stay, in id order, so that
    entry i is the old id of new fact i."""
    gone = [int(f) for f in removed]
    if len(set(gone)) != len(gone) or any(f < 0 or f >= n_facts for f in gone):
        raise ValueError("removed ids must be distinct and in range")
    drop = set(gone)
    return np.array([f for f in range(n_facts) if f not in drop], dtype=np.int32)


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not
    depend on it)."""
    lib().or_set_threads(int(n))


def max_threads() -> int:
    return int(lib().or_max_threads())
