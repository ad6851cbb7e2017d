"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and the host half of is_inject (validation and
composition) reports each error before any device work."""
import os
import re

import numpy as np
import pytest

import kv_cache_injection_is_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "inferscale.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(is_\w+)\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = K.lib()
    names = declared_functions()
    assert set(names) == set(K.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_null_arguments_are_rejected_without_gpu():
    lib = K.lib()
    assert lib.is_store_create(None, None) == -1
    assert "null" in K.is_last_error()
    assert lib.is_store_destroy(None) == 0
    assert lib.is_topk(None, None, 1, 1, None, None, None) == -1
    assert lib.is_topk_noalloc(None, None, 1, 1, None, None, None) == -1
    assert lib.is_inject(None, 0, None, None, None, None, 1, None, None, None) == -1
    assert lib.is_retrieve_inject(None, None, 1, 1, None, None, 1, None, None, None, None,
                                  None) == -1
    assert lib.is_attend(None, None, None, 1, 1, 1, None, None, None, None, None, 1, None,
                         None) == -1
    assert lib.is_store_append(None, 1, None, 0, None, None, None, None, None) == -1
    assert lib.is_store_update(None, 0, 0, None, None, None, None) == -1
    assert lib.is_store_remove(None, 1, None, None) == -1


def _desc(dtype=K.IS_DTYPE_BF16, head_dim=128, lens=(5, 7, 3, 9), emb_dim=0):
    return K.make_desc(2, 2, head_dim, dtype, np.array(lens, np.int32), emb_dim)


def _cache(dtype=K.IS_DTYPE_BF16, nb=16, B=4, H=2, d=128, base=0x10000):
    return K.make_cache(base, base + (1 << 30), (nb * B * H * d, B * H * d, H * d, d), B, nb,
                        dtype)


ROPE = K.make_rope(1e4)


def _ok_args():
    req_off = np.array([0, 2, 3], np.int32)
    ids = np.array([1, 0, 3], np.int32)
    prefix = np.array([2, 0], np.int32)
    bt = np.array([[3, 4, 5, 6, -1], [7, 8, 9, -1, -1]], np.int32)
    return req_off, ids, prefix, bt


def _code(fn):
    with pytest.raises(K.ISError) as e:
        fn()
    return e.value.code


def test_check_counts_tokens():
    d, keep = _desc()
    n = K.is_inject_check(d, *_ok_args(), _cache(), ROPE)
    assert n == 7 + 5 + 9


def test_check_error_paths():
    d, keep = _desc()
    req_off, ids, prefix, bt = _ok_args()
    c = _cache()
    chk = lambda **kw: K.is_inject_check(kw.get("d", d), kw.get("req_off", req_off),
                                         kw.get("ids", ids), kw.get("prefix", prefix),
                                         kw.get("bt", bt), kw.get("c", c), kw.get("rope", ROPE))
    assert _code(lambda: chk(ids=np.array([1, 0, 4], np.int32))) == -2         # fact id
    assert _code(lambda: chk(ids=np.array([1, -1, 3], np.int32))) == -2
    short = bt.copy()
    short[0, 3] = -1
    assert _code(lambda: chk(bt=short)) == -3                                 # table too short
    bad = bt.copy()
    bad[1, 1] = 16
    assert _code(lambda: chk(bt=bad)) == -3                                   # entry >= n_blocks
    over = bt.copy()
    over[1, 0] = 6                                                            # shares block 6
    assert _code(lambda: chk(bt=over)) == -4
    assert _code(lambda: chk(c=_cache(dtype=K.IS_DTYPE_F32))) == -5          # dtype mismatch
    assert _code(lambda: chk(c=_cache(base=0x10008))) == -6                  # misaligned base
    odd = _cache()
    odd.stride_slot = 2 * 128 + 4                                             # 8-byte slot stride
    assert _code(lambda: chk(c=odd)) == -6
    assert _code(lambda: chk(req_off=np.array([0, 3, 2], np.int32))) == -1   # decreasing offsets
    assert _code(lambda: chk(prefix=np.array([-1, 0], np.int32))) == -1
    assert _code(lambda: chk(rope=K.make_rope(0.5))) == -1
    assert _code(lambda: chk(rope=K.make_rope(1e4, "llama3", 8.0, 4.0, 1.0))) == -1
    far = np.array([(1 << 24) - 5, 0], np.int32)
    big = np.full((2, (1 << 24) // 4 + 8), 3, np.int32)
    assert _code(lambda: chk(prefix=far, bt=big)) == -1                      # positions >= 2^24


def test_two_requests_may_share_a_block_on_distinct_slots():
    d, keep = _desc(lens=(2, 2))
    req_off = np.array([0, 1, 2], np.int32)
    ids = np.array([0, 1], np.int32)
    prefix = np.array([0, 2], np.int32)            # request 1 uses slots 2..3 of block 5
    bt = np.array([[5], [5]], np.int32)
    assert K.is_inject_check(d, req_off, ids, prefix, bt, _cache(), ROPE) == 4
    prefix2 = np.array([0, 1], np.int32)           # now slot 1 of block 5 is used twice
    assert _code(lambda: K.is_inject_check(d, req_off, ids, prefix2, bt, _cache(), ROPE)) == -4


def test_store_description_errors():
    for kw, code in (({"head_dim": 96}, -9), ({"head_dim": 24}, -6),
                     ({"lens": (3, 0)}, -1), ({"emb_dim": 48}, -9)):
        args = dict(dtype=K.IS_DTYPE_BF16, head_dim=128, lens=(5, 7), emb_dim=0)
        args.update(kw)
        d, keep = _desc(**args)
        assert _code(lambda: K.is_inject_check(d, *_ok_args(), _cache(), ROPE)) == code


def test_empty_call_is_ok():
    d, keep = _desc()
    z = np.zeros((0, 1), np.int32)
    assert K.is_inject_check(d, np.array([0], np.int32), np.zeros(0, np.int32),
                             np.zeros(0, np.int32), z, _cache(), ROPE) == 0


@pytest.mark.parametrize("nb,B,bt,ok,bad", [
    # small cache (slot bitmap): runs of 40-slot blocks straddle 64-bit words
    (16, 40, [[2, 3], [3, 0]], [0, 10], [0, 9]),
    # 2^31 slots: the check sorts the runs instead
    (1 << 21, 1024, [[3, 0], [3, 0]], [0, 50], [0, 49]),
])
def test_slot_overlap_check_each_path_and_state_is_cleared(nb, B, bt, ok, bad):
    d, keep = _desc(lens=(50, 30))
    req_off = np.array([0, 1, 2], np.int32)
    ids = np.array([0, 1], np.int32)
    bt = np.array(bt, np.int32)
    c = _cache(nb=nb, B=B)
    ok = np.array(ok, np.int32)
    assert K.is_inject_check(d, req_off, ids, ok, bt, c, ROPE) == 80
    assert _code(lambda: K.is_inject_check(d, req_off, ids, np.array(bad, np.int32), bt, c,
                                           ROPE)) == -4
    # the failed call leaves nothing behind: the clean call passes again
    assert K.is_inject_check(d, req_off, ids, ok, bt, c, ROPE) == 80
