"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module holds none of the method's arithmetic.  It generates the inputs
(stored pre-RoPE keys and raw values, fact embeddings, queries, fact lengths,
fact ids, prefixes, block tables, the cache sentinel) with a counter-based
generator (Philox4x32-10), so that any single fact can be regenerated on the
host bit for bit while the full store is filled on the GPU.  See synth.c for
the recipe.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libsynth.so")
GPU_SO = os.path.join(_HERE, "libsynth_gpu.so")

TAG_K, TAG_V = 1, 2
F32, BF16 = 0, 1

_HIP_FLAGS = ["-O3", "-fPIC", "-shared", "-std=c++17", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    """Compile the host generator (gcc) and the device generator (hipcc)."""
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
         os.path.join(_HERE, "synth.c"), "-o", HOST_SO, "-lm"],
        ["/opt/rocm/bin/hipcc", *_HIP_FLAGS, os.path.join(_HERE, "synth_gpu.hip"),
         "-o", GPU_SO],
    ]
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"synth build failed: {' '.join(cmd)}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))


_host = None
_gpu = None


def host_lib() -> ctypes.CDLL:
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            build()
        L = ctypes.CDLL(HOST_SO)
        c = ctypes
        L.synth_philox4x32_10.argtypes = [c.POINTER(c.c_uint32)] * 3
        L.synth_normal_numerator.argtypes = [c.c_uint32] * 4
        L.synth_normal_numerator.restype = c.c_int32
        L.synth_fact_kv.argtypes = [c.c_uint32, c.c_uint32, c.c_int64, c.c_int64,
                                    c.c_int64, c.c_int, c.c_void_p]
        L.synth_kv_range.argtypes = [c.c_uint32, c.c_uint32, c.c_int64, c.c_int64,
                                     c.c_void_p, c.c_int, c.c_void_p]
        L.synth_double_to_f16.argtypes = [c.c_double]
        L.synth_double_to_f16.restype = c.c_uint16
        L.synth_embeddings.argtypes = [c.c_uint32, c.c_int64, c.c_int64, c.c_int,
                                       c.c_void_p]
        L.synth_queries.argtypes = [c.c_uint32, c.c_int64, c.c_int, c.c_void_p]
        L.synth_len_uniform.argtypes = [c.c_uint32, c.c_int64, c.c_int, c.c_int,
                                        c.c_void_p]
        L.synth_len_lognormal.argtypes = [c.c_uint32, c.c_int64, c.c_double,
                                          c.c_double, c.c_int, c.c_int, c.c_void_p]
        L.synth_zipf_requests.argtypes = [c.c_uint32, c.c_int, c.c_int, c.c_int64,
                                          c.c_double, c.c_void_p]
        L.synth_zipf_requests.restype = c.c_int
        L.synth_prefix.argtypes = [c.c_uint32, c.c_int, c.c_int, c.c_int, c.c_void_p]
        L.synth_permutation.argtypes = [c.c_uint32, c.c_int64, c.c_void_p]
        L.synth_block_tables.argtypes = [c.c_uint32, c.c_int, c.c_void_p, c.c_int,
                                         c.c_int64, c.c_int, c.c_void_p]
        L.synth_block_tables.restype = c.c_int
        L.synth_sentinel_host.argtypes = [c.c_uint32, c.c_uint64, c.c_int64,
                                          c.c_void_p]
        _host = L
    return _host


def gpu_lib() -> ctypes.CDLL:
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_SO):
            raise RuntimeError(f"{GPU_SO} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(GPU_SO)
        c = ctypes
        L.synth_gpu_fill_kv.argtypes = [c.c_uint32, c.c_uint32, c.c_int64, c.c_int64,
                                        c.c_int64, c.c_void_p, c.c_int, c.c_void_p,
                                        c.c_void_p]
        L.synth_gpu_fill_kv.restype = c.c_int
        L.synth_gpu_sentinel.argtypes = [c.c_uint32, c.c_uint64, c.c_int64,
                                         c.c_void_p, c.c_void_p]
        L.synth_gpu_sentinel.restype = c.c_int
        L.synth_gpu_sentinel_check.argtypes = [c.c_uint32, c.c_uint64, c.c_int64,
                                               c.c_void_p, c.c_int64, c.c_void_p,
                                               c.c_void_p, c.c_void_p]
        L.synth_gpu_sentinel_check.restype = c.c_int
        _gpu = L
    return _gpu


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ----------------------------------------------------------------- host side

def philox4x32_10(ctr, key) -> list[int]:
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    host_lib().synth_philox4x32_10(c, k, o)
    return list(o)


def normal_numerator(seed: int, tag: int, entity: int, n: int) -> int:
    return host_lib().synth_normal_numerator(seed, tag, entity, n)


def kv_dtype_np(dtype: int):
    return np.float32 if dtype == F32 else np.uint16


def fact_kv(seed: int, tag: int, fact: int, n_elems: int, dtype: int,
            first: int = 0) -> np.ndarray:
    """Elements [first, first+n_elems) of one fact's K (tag 1) or V (tag 2)
    block, laid out [layer][kv_head][token][head_dim]; fp32, or bf16 bits."""
    out = np.empty(n_elems, dtype=kv_dtype_np(dtype))
    host_lib().synth_fact_kv(seed, tag, fact, first, n_elems, dtype, _ptr(out))
    return out


def kv_range(seed: int, tag: int, first_fact: int, lens: np.ndarray,
             row_elems: int, dtype: int) -> np.ndarray:
    """K or V of consecutive facts, packed back to back in the ragged store
    layout; row_elems = n_layers * n_kv_heads * head_dim."""
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens * row_elems, out=off[1:])
    out = np.empty(int(off[-1]), dtype=kv_dtype_np(dtype))
    host_lib().synth_kv_range(seed, tag, first_fact, len(lens), _ptr(off), dtype,
                              _ptr(out))
    return out


def embeddings(seed: int, first: int, n: int, dim: int) -> np.ndarray:
    out = np.empty((n, dim), dtype=np.uint16)
    host_lib().synth_embeddings(seed, first, n, dim, _ptr(out))
    return out


def queries(seed: int, n: int, dim: int) -> np.ndarray:
    out = np.empty((n, dim), dtype=np.uint16)
    host_lib().synth_queries(seed, n, dim, _ptr(out))
    return out


def double_to_f16_bits(x: float) -> int:
    return host_lib().synth_double_to_f16(x)


def len_uniform(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    host_lib().synth_len_uniform(seed, n, lo, hi, _ptr(out))
    return out


def len_lognormal(seed: int, n: int, median: float, sigma: float, lo: int,
                  hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    host_lib().synth_len_lognormal(seed, n, median, sigma, lo, hi, _ptr(out))
    return out


def zipf_requests(seed: int, n_req: int, k: int, n_ids: int, s: float) -> np.ndarray:
    out = np.empty((n_req, k), dtype=np.int32)
    if host_lib().synth_zipf_requests(seed, n_req, k, n_ids, s, _ptr(out)) != 0:
        raise ValueError("k exceeds the number of ids")
    return out


def prefixes(seed: int, n_req: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n_req, dtype=np.int32)
    host_lib().synth_prefix(seed, n_req, lo, hi, _ptr(out))
    return out


def permutation(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    host_lib().synth_permutation(seed, n, _ptr(out))
    return out


def block_tables(seed: int, need_tokens: np.ndarray, block_size: int,
                 n_blocks: int) -> np.ndarray:
    """Non-overlapping random block tables, [n_req][max_blocks], -1 padded;
    need_tokens[r] is the number of cache positions request r must cover."""
    need = np.ascontiguousarray(need_tokens, dtype=np.int64)
    nb = (need + block_size - 1) // block_size
    max_blocks = max(1, int(nb.max()) if len(nb) else 1)
    out = np.empty((len(need), max_blocks), dtype=np.int32)
    rc = host_lib().synth_block_tables(seed, len(need), _ptr(need), block_size,
                                       n_blocks, max_blocks, _ptr(out))
    if rc != 0:
        raise ValueError(f"block tables do not fit the cache (code {rc})")
    return out


def sentinel_host(seed: int, first_word: int, n_words: int) -> np.ndarray:
    out = np.empty(n_words, dtype=np.uint32)
    host_lib().synth_sentinel_host(seed, first_word, n_words, _ptr(out))
    return out


# --------------------------------------------------------------- device side

def gpu_fill_kv(seed: int, tag: int, first_fact: int, d_elem_off, total_elems: int,
                dtype: int, d_out_ptr: int, stream_ptr: int) -> None:
    """Fill a device buffer with the K or V of facts first_fact.. (device
    int64 offsets d_elem_off, n_facts + 1 entries, relative to d_out_ptr)."""
    n_facts = d_elem_off.numel() - 1
    rc = gpu_lib().synth_gpu_fill_kv(seed, tag, first_fact, n_facts, total_elems,
                                     d_elem_off.data_ptr(), dtype, d_out_ptr,
                                     stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_kv failed ({rc})")


def gpu_sentinel(seed: int, d_ptr: int, n_bytes: int, stream_ptr: int,
                 first_word: int = 0) -> None:
    assert n_bytes % 4 == 0
    rc = gpu_lib().synth_gpu_sentinel(seed, first_word, n_bytes // 4, d_ptr,
                                      stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_sentinel failed ({rc})")


def gpu_sentinel_check(seed: int, d_ptr: int, n_bytes: int, row_bytes: int,
                       d_written_ptr: int, d_count_ptr: int, stream_ptr: int,
                       first_word: int = 0) -> None:
    """Adds to the device uint64 at d_count_ptr the number of 32-bit words that
    differ from the sentinel, skipping rows marked in the device byte mask
    d_written_ptr (0 = check every row)."""
    assert n_bytes % 4 == 0 and row_bytes % 4 == 0
    rc = gpu_lib().synth_gpu_sentinel_check(seed, first_word, n_bytes // 4, d_ptr,
                                            row_bytes // 4, d_written_ptr or None,
                                            d_count_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_sentinel_check failed ({rc})")
