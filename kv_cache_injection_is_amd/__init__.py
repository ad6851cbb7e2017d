"""Python binding of libinferscale.so (include/inferscale.h).

Argument marshalling only: every function forwards to the C entry point of
the same name; host arrays are numpy arrays, device arrays are torch tensors
(or raw device addresses), streams are torch streams (or raw hipStream_t
handles).  There is no fallback: if the library is not built, importing the
functions raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# INFERSCALE_SO points the binding at another build of the library (tuning builds).
SO = os.environ.get("INFERSCALE_SO") or os.path.join(PKG, "libinferscale.so")

IS_OK = 0
STATUS = {0: "IS_OK", -1: "IS_ERR_INVALID_ARG", -2: "IS_ERR_FACT_ID", -3: "IS_ERR_BLOCK_TABLE",
          -4: "IS_ERR_SLOT_OVERLAP", -5: "IS_ERR_DTYPE", -6: "IS_ERR_ALIGN", -7: "IS_ERR_OOM",
          -8: "IS_ERR_HIP", -9: "IS_ERR_UNSUPPORTED"}
IS_DTYPE_F32, IS_DTYPE_BF16 = 0, 1
IS_ROPE_NONE, IS_ROPE_LLAMA3 = 0, 1

EXPORTS = ("is_store_create", "is_store_load", "is_store_get_info", "is_topk",
           "is_topk_noalloc", "is_inject",
           "is_retrieve_inject", "is_attend", "is_store_append", "is_store_update",
           "is_store_remove", "is_inject_check", "is_store_destroy", "is_last_error")


class ISError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class is_store_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("n_facts", ctypes.c_int64), ("fact_len", ctypes.c_void_p),
                ("emb_dim", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("hbm_budget_bytes", ctypes.c_int64), ("k_src", ctypes.c_void_p),
                ("v_src", ctypes.c_void_p), ("emb_src", ctypes.c_void_p),
                ("spare_facts", ctypes.c_int64), ("spare_tokens", ctypes.c_int64)]


class is_cache(ctypes.Structure):
    _fields_ = [("k_base", ctypes.c_void_p), ("v_base", ctypes.c_void_p),
                ("stride_layer", ctypes.c_int64), ("stride_block", ctypes.c_int64),
                ("stride_slot", ctypes.c_int64), ("stride_head", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_blocks", ctypes.c_int64)]


class is_rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("scaling", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("factor", ctypes.c_double),
                ("low_freq_factor", ctypes.c_double), ("high_freq_factor", ctypes.c_double),
                ("orig_max_pos", ctypes.c_double)]


class is_store_info(ctypes.Structure):
    _fields_ = [("n_facts", ctypes.c_int64), ("n_hbm_facts", ctypes.c_int64),
                ("hbm_kv_bytes", ctypes.c_int64), ("host_kv_bytes", ctypes.c_int64),
                ("total_tokens", ctypes.c_int64), ("emb_bytes", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise ISError(-8, f"{SO} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(SO)
        c, P = ctypes, ctypes.c_void_p
        L.is_store_create.argtypes = [c.POINTER(is_store_desc), c.POINTER(P)]
        L.is_store_load.argtypes = [P, c.c_int64, c.c_int64, P, P, P, c.c_int]
        L.is_store_get_info.argtypes = [P, c.POINTER(is_store_info)]
        L.is_topk.argtypes = [P, P, c.c_int32, c.c_int32, P, P, P]
        L.is_topk_noalloc.argtypes = [P, P, c.c_int32, c.c_int32, P, P, P]
        L.is_inject.argtypes = [P, c.c_int32, P, P, P, P, c.c_int32, c.POINTER(is_cache),
                                c.POINTER(is_rope), P]
        L.is_retrieve_inject.argtypes = [P, P, c.c_int32, c.c_int32, P, P, c.c_int32,
                                         c.POINTER(is_cache), c.POINTER(is_rope), P, P, P]
        L.is_attend.argtypes = [P, c.POINTER(is_cache), c.POINTER(is_rope), c.c_int32,
                                c.c_int32, c.c_int32, P, P, P, P, P, c.c_int32, P, P]
        L.is_store_append.argtypes = [P, c.c_int32, P, c.c_int32, P, P, P,
                                      c.POINTER(c.c_int64), P]
        L.is_store_update.argtypes = [P, c.c_int64, c.c_int32, P, P, P, P]
        L.is_store_remove.argtypes = [P, c.c_int64, P, P]
        L.is_inject_check.argtypes = [c.POINTER(is_store_desc), c.c_int32, P, P, P, P,
                                      c.c_int32, c.POINTER(is_cache), c.POINTER(is_rope),
                                      c.POINTER(c.c_int64)]
        L.is_store_destroy.argtypes = [P]
        L.is_last_error.restype = c.c_char_p
        for name in EXPORTS:
            if name != "is_last_error":
                getattr(L, name).restype = c.c_int
        _lib = L
    return _lib


def is_last_error() -> str:
    return lib().is_last_error().decode()


def _check(rc: int) -> None:
    if rc != IS_OK:
        raise ISError(rc, is_last_error())


def _host(a, dtype):
    """numpy array (kept alive by the caller) -> address, or None."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data


def _dev(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_desc(n_layers, n_kv_heads, head_dim, kv_dtype, fact_len, emb_dim=0,
              hbm_budget_bytes=-1, k_src=None, v_src=None, emb_src=None, spare_facts=0,
              spare_tokens=0):
    """Builds an is_store_desc; returns (desc, keepalive)."""
    lens, lens_p = _host(fact_len, np.int32)
    keep = [lens]
    srcs = []
    for a in (k_src, v_src, emb_src):
        if a is None:
            srcs.append(None)
        else:
            arr = np.ascontiguousarray(a)
            keep.append(arr)
            srcs.append(arr.ctypes.data)
    d = is_store_desc(n_layers, n_kv_heads, head_dim, kv_dtype, len(lens), lens_p, emb_dim, 0,
                      hbm_budget_bytes, *srcs, spare_facts, spare_tokens)
    return d, keep


def is_store_create(desc: is_store_desc) -> int:
    h = ctypes.c_void_p()
    _check(lib().is_store_create(ctypes.byref(desc), ctypes.byref(h)))
    return h.value


def is_store_load(store: int, first_fact: int, n_facts: int, k=None, v=None, emb=None,
                  src_on_device: bool = False) -> None:
    """k, v, emb: numpy arrays (host) or torch tensors / addresses (device)."""
    if src_on_device:
        ptrs = [_dev(x) for x in (k, v, emb)]
        keep = None
    else:
        keep = [None if x is None else np.ascontiguousarray(x) for x in (k, v, emb)]
        ptrs = [None if x is None else x.ctypes.data for x in keep]
    _check(lib().is_store_load(store, first_fact, n_facts, *ptrs, 1 if src_on_device else 0))
    del keep


def is_store_get_info(store: int) -> is_store_info:
    out = is_store_info()
    _check(lib().is_store_get_info(store, ctypes.byref(out)))
    return out


def is_topk(store: int, q_f16, n_q: int, k: int, ids, scores, stream=None) -> None:
    """q_f16, ids, scores: device tensors (int16/uint16-viewed fp16, int32, float32)."""
    _check(lib().is_topk(store, _dev(q_f16), n_q, k, _dev(ids), _dev(scores), _stream(stream)))


def is_topk_noalloc(store: int, q_f16, n_q: int, k: int, ids, scores, stream=None) -> None:
    """As is_topk, with the library's fixed per-GPU scratch (no allocation)."""
    _check(lib().is_topk_noalloc(store, _dev(q_f16), n_q, k, _dev(ids), _dev(scores),
                                 _stream(stream)))


def is_retrieve_inject(store: int, q_f16, n_req: int, k: int, prefix_len, block_tables,
                       cache: is_cache, rope: is_rope, status, ids=None, stream=None) -> None:
    """q_f16, prefix_len, block_tables ([n_req][max_blocks] int32), status
    (int32, one element) and the optional ids ([n_req][k] int32) are device
    tensors; the status is written on the stream."""
    max_blocks = int(block_tables.shape[1]) if n_req > 0 else 1
    _check(lib().is_retrieve_inject(store, _dev(q_f16), n_req, k, _dev(prefix_len),
                                    _dev(block_tables), max_blocks, ctypes.byref(cache),
                                    ctypes.byref(rope), _dev(ids) if ids is not None else None,
                                    _dev(status), _stream(stream)))


def is_attend(store: int, cache: is_cache, rope: is_rope, q, n_qtok: int, n_q_heads: int,
              q_pos, ctx_begin, ctx_end, block_tables, out, stream=None) -> None:
    """q, out: device tensors [n_layers][n_req][n_qtok][n_q_heads][head_dim]
    (q in the store's dtype: bf16 bits as int16/uint16, or float32; out
    float32); q_pos, ctx_begin, ctx_end ([n_req]) and block_tables
    ([n_req][max_blocks]) are host arrays."""
    qp, qp_p = _host(q_pos, np.int32)
    cb, cb_p = _host(ctx_begin, np.int32)
    ce, ce_p = _host(ctx_end, np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    _check(lib().is_attend(store, ctypes.byref(cache), ctypes.byref(rope), len(qp), n_qtok,
                           n_q_heads, _dev(q), qp_p, cb_p, ce_p, bt.ctypes.data, bt.shape[1],
                           _dev(out), _stream(stream)))


def is_store_append(store: int, fact_len, window: int, k_enc, v_enc, emb=None,
                    stream=None) -> int:
    """fact_len: host array; k_enc, v_enc (the window encodings back to back)
    and emb ([n][emb_dim] fp16 bits) device tensors.  Returns the first new
    fact id."""
    fl, fl_p = _host(fact_len, np.int32)
    first = ctypes.c_int64(-1)
    _check(lib().is_store_append(store, len(fl), fl_p, window, _dev(k_enc), _dev(v_enc),
                                 _dev(emb), ctypes.byref(first), _stream(stream)))
    return first.value


def is_store_update(store: int, fact_id: int, window: int, k_enc, v_enc, emb=None,
                    stream=None) -> None:
    _check(lib().is_store_update(store, fact_id, window, _dev(k_enc), _dev(v_enc), _dev(emb),
                                 _stream(stream)))


def is_store_remove(store: int, ids, stream=None) -> None:
    """ids: host array of the fact ids to evict; the rest are renumbered
    densely in their order.  Returns once the stream has completed."""
    a, a_p = _host(ids, np.int32)
    _check(lib().is_store_remove(store, len(a), a_p, _stream(stream)))


def make_cache(k_base, v_base, strides, block_size, n_blocks, dtype) -> is_cache:
    return is_cache(_dev(k_base), _dev(v_base), *strides, block_size, dtype, n_blocks)


def make_rope(theta, scaling="none", factor=8.0, low=1.0, high=4.0, orig=8192.0) -> is_rope:
    sc = {"none": IS_ROPE_NONE, "llama3": IS_ROPE_LLAMA3}[scaling]
    return is_rope(theta, sc, 0, factor, low, high, orig)


def _inject_args(req_off, fact_ids, prefix_len, block_tables):
    ro, ro_p = _host(req_off, np.int32)
    fi, fi_p = _host(fact_ids, np.int32)
    pl, pl_p = _host(prefix_len, np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    if bt.ndim != 2:
        raise ValueError("block_tables must be [n_req][max_blocks]")
    return (ro, fi, pl, bt), (ro_p, fi_p, pl_p, bt.ctypes.data, bt.shape[1]), len(pl)


def is_inject(store: int, req_off, fact_ids, prefix_len, block_tables, cache: is_cache,
              rope: is_rope, stream=None) -> None:
    keep, (ro, fi, pl, bt, mb), n_req = _inject_args(req_off, fact_ids, prefix_len, block_tables)
    _check(lib().is_inject(store, n_req, ro, fi, pl, bt, mb, ctypes.byref(cache),
                           ctypes.byref(rope), _stream(stream)))
    del keep


def is_inject_check(desc: is_store_desc, req_off, fact_ids, prefix_len, block_tables,
                    cache: is_cache, rope: is_rope) -> int:
    """Returns the number of tokens; raises ISError with the status code."""
    keep, (ro, fi, pl, bt, mb), n_req = _inject_args(req_off, fact_ids, prefix_len, block_tables)
    n = ctypes.c_int64(0)
    _check(lib().is_inject_check(ctypes.byref(desc), n_req, ro, fi, pl, bt, mb,
                                 ctypes.byref(cache), ctypes.byref(rope), ctypes.byref(n)))
    del keep
    return n.value


def is_store_destroy(store: int) -> None:
    _check(lib().is_store_destroy(store))
