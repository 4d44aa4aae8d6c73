"""The C ABI without a GPU: the library loads, exports every function that
include/nvfp4kv.h declares, and rejects bad arguments on the host with the
documented status codes before anything touches a device."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kv():
    from nvfp4_quantized_kv_amd import build as B
    if B.stale():
        B.build()
    import nvfp4_quantized_kv_amd as kv
    return kv


def _declared():
    src = open(os.path.join(ROOT, "include", "nvfp4kv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4kv_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("nvfp4kv_append", "nvfp4kv_decode_attn", "nvfp4kv_dequant", "nvfp4kv_pool_bytes",
                 "nvfp4kv_decode_workspace_bytes", "nvfp4kv_decode_attn_multi", "nvfp4kv_last_error"):
        assert must in names


def test_every_declared_symbol_is_exported(kv):
    lib = ctypes.CDLL(kv.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) <= set(kv.EXPORTED)
    assert "gfx950" in kv.nvfp4kv_version()


def _desc(kv, **over):
    d = dict(base=256, num_pages=10, num_layers=2, num_kv_heads=4, head_dim=128, page_size=64,
             rotary_dim=32, hadamard=1)
    d.update(over)
    return kv._PoolDesc(d["base"], d["num_pages"], d["num_layers"], d["num_kv_heads"], d["head_dim"],
                        d["page_size"], d["rotary_dim"], d["hadamard"])


def test_pool_bytes_is_144_per_token_per_kv_head(kv):
    d = _desc(kv)
    assert kv.lib().nvfp4kv_pool_bytes(ctypes.byref(d)) == 2 * 10 * 4 * 64 * 144
    assert kv.lib().nvfp4kv_pool_bytes(None) == 0
    assert kv.lib().nvfp4kv_pool_bytes(ctypes.byref(_desc(kv, head_dim=64))) == 0


def test_rope_table_matches_oracle_bitwise(kv):
    import oracle
    for scale in (1.0, 2.3):
        c, s = kv.nvfp4kv_rope_table(1e7, 32, scale, 5000)
        oc, os_ = oracle.rope_table(1e7, 32, scale, 5000)
        assert (c.numpy() == oc).all() and (s.numpy() == os_).all()


def _append(kv, d, layer=0, n_tok=4, k=4096, v=4096, dtype=1, slots=4096, pos=4096, c=4096, s=4096,
            max_pos=10):
    return kv.lib().nvfp4kv_append(ctypes.byref(d) if d is not None else None, layer, n_tok, k, v,
                                   dtype, slots, pos, c, s, max_pos, None)


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=64), -2), (dict(page_size=32), -2), (dict(rotary_dim=23), -1),
    (dict(rotary_dim=-16), -1), (dict(rotary_dim=130), -1), (dict(hadamard=3), -1), (dict(num_pages=0), -1),
    (dict(num_kv_heads=0), -1), (dict(base=0), -1), (dict(base=4100), -1)])
def test_append_rejects_bad_pool(kv, over, code):
    """Bad descriptors are refused before any launch (rotary widths: any even
    width from 0 to 128 is accepted, an odd or out-of-range one is not)."""
    assert _append(kv, _desc(kv, **over)) == code
    assert kv.nvfp4kv_last_error() != ""


def test_append_rejects_bad_arguments(kv):
    d = _desc(kv)
    assert _append(kv, None) == -1
    assert _append(kv, d, layer=2) == -1
    assert _append(kv, d, layer=-1) == -1
    assert _append(kv, d, n_tok=-1) == -1
    assert _append(kv, d, k=None) == -1
    assert _append(kv, d, slots=None) == -1
    assert _append(kv, d, k=4100) == -1               # misaligned
    assert _append(kv, d, dtype=7) == -1
    assert _append(kv, d, c=None) == -1               # rotary needs the table
    assert _append(kv, d, pos=None) == -1
    assert _append(kv, d, max_pos=0) == -1
    assert "max_pos" in kv.nvfp4kv_last_error()
    assert _append(kv, d, n_tok=0) == 0               # nothing to do is not an error


def _decode(kv, d, n_seq=2, hq=24, q=4096, pt=4096, stride=100, lens=4096, max_len=6000,
            scale=0.1, out=4096, ws=4096, ws_bytes=1 << 30, pps=0, qpos=4096, k_new=None, v_new=None):
    return kv.lib().nvfp4kv_decode_attn(ctypes.byref(d), 0, n_seq, hq, q, k_new, v_new, 1, qpos, 4096,
                                        4096, 10, pt, stride, lens, max_len, scale, out, ws, ws_bytes,
                                        pps, None)


def test_decode_rejects_bad_arguments(kv):
    d = _desc(kv)
    assert _decode(kv, d, hq=25) == -1                # not a multiple of the kv heads
    assert _decode(kv, d, hq=4 * 17) == -2            # more than 16 query heads per kv head
    assert _decode(kv, d, n_seq=0) == -1
    assert _decode(kv, d, max_len=0) == -1
    assert _decode(kv, d, stride=10) == -1            # table narrower than max_seq_len's pages
    assert _decode(kv, d, scale=-1.0) == -1
    assert _decode(kv, d, scale=float("nan")) == -1
    assert _decode(kv, d, q=None) == -1
    assert _decode(kv, d, qpos=None) == -1
    assert _decode(kv, d, pps=5000) == -1
    assert _decode(kv, d, ws_bytes=16) == -3
    assert _decode(kv, d, ws=None) == -3
    assert _decode(kv, d, ws=4100) == -3
    assert "workspace" in kv.nvfp4kv_last_error()
    assert _decode(kv, d, k_new=4096) == -1           # k_new without v_new
    assert _decode(kv, d, v_new=4096) == -1
    assert _decode(kv, d, k_new=4100, v_new=4096) == -1   # misaligned
    assert "k_new" in kv.nvfp4kv_last_error()


def test_workspace_size_query(kv):
    d = _desc(kv)
    L = kv.lib()
    a = L.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), 3, 24, 470001, 0)
    b = L.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), 3, 24, 470001, 64)
    assert a > 0 and b > 0
    splits = (470001 + 63) // 64 // 64 + 1
    assert b >= 3 * 4 * splits * 6 * 130 * 4 - 3 * 4 * 6 * 130 * 4
    assert L.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), 3, 25, 1000, 0) == 0


def test_dequant_rejects_bad_arguments(kv):
    d = _desc(kv)
    L = kv.lib()
    assert L.nvfp4kv_dequant(ctypes.byref(d), 0, 4, None, 4096, 4096, 0, 0, None) == -1
    assert L.nvfp4kv_dequant(ctypes.byref(d), 0, 4, 4096, None, None, 0, 0, None) == -1
    assert L.nvfp4kv_dequant(ctypes.byref(d), 0, 4, 4096, 4096, 4096, 0, 3, None) == -1
    assert L.nvfp4kv_dequant(ctypes.byref(d), 5, 4, 4096, 4096, 4096, 0, 0, None) == -1
    assert L.nvfp4kv_dequant(ctypes.byref(d), 0, 0, 4096, 4096, 4096, 0, 0, None) == 0


def test_pool_rotation_modes(kv):
    """hadamard 0, 1 and 2 (the randomized rotation) are valid pools; 3 and -1
    are not (an empty dequant validates the pool and launches nothing)."""
    L = kv.lib()
    for h in (0, 1, 2):
        assert L.nvfp4kv_dequant(ctypes.byref(_desc(kv, hadamard=h)), 0, 0, 4096, 4096, 4096, 0, 0, None) == 0
    for h in (3, -1):
        assert L.nvfp4kv_dequant(ctypes.byref(_desc(kv, hadamard=h)), 0, 0, 4096, 4096, 4096, 0, 0, None) == -1


def test_page_bytes_and_spill_argument_checks(kv):
    """A spilled page is every layer's and kv head's 9216-byte block; the
    spill/restore calls reject bad sizes and pointers before any launch (a
    pageable host buffer is neither device nor pinned memory)."""
    d = _desc(kv)
    L = kv.lib()
    assert L.nvfp4kv_page_bytes(ctypes.byref(d)) == 2 * 4 * 9216
    assert L.nvfp4kv_page_bytes(None) == 0
    page = 2 * 4 * 9216
    host = (ctypes.c_uint8 * (3 * page + 16))()
    ids = (ctypes.c_int32 * 3)(0, 1, 2)
    a16 = (ctypes.addressof(host) + 15) // 16 * 16
    for fn in (L.nvfp4kv_spill_pages, L.nvfp4kv_restore_pages):
        assert fn(ctypes.byref(d), 0, None, None, 0, None) == 0            # nothing to do
        assert fn(ctypes.byref(d), -1, ctypes.addressof(ids), a16, 3 * page, None) == -1
        assert fn(ctypes.byref(d), 3, None, a16, 3 * page, None) == -1
        assert fn(ctypes.byref(d), 3, ctypes.addressof(ids), None, 3 * page, None) == -1
        assert fn(ctypes.byref(d), 3, ctypes.addressof(ids), a16 + 1, 3 * page, None) == -1
        assert fn(ctypes.byref(d), 3, ctypes.addressof(ids), a16, 3 * page - 1, None) == -1
        assert fn(ctypes.byref(d), 3, ctypes.addressof(ids), a16, 3 * page, None) == -1
        assert b"pinned" in L.nvfp4kv_last_error()


def _multi(kv, d, n_seq=2, n_qtok=3, hq=24, q=4096, pt=4096, stride=16, lens=4096, max_len=1000,
           scale=0.1, out=4096, ws=4096, ws_bytes=1 << 30, pps=0, qpos=4096):
    return kv.lib().nvfp4kv_decode_attn_multi(ctypes.byref(d), 0, n_seq, n_qtok, hq, q, 1, qpos, 4096, 4096,
                                              10, pt, stride, lens, max_len, scale, out, ws, ws_bytes, pps,
                                              None)


def test_decode_multi_rejects_bad_arguments(kv):
    d = _desc(kv)
    assert _multi(kv, d, n_qtok=0) == -1
    assert _multi(kv, d, n_qtok=65) == -1
    assert "n_qtok" in kv.nvfp4kv_last_error()
    assert _multi(kv, d, hq=25) == -1
    assert _multi(kv, d, hq=4 * 17) == -2
    assert _multi(kv, d, q=None) == -1
    assert _multi(kv, d, qpos=None) == -1
    assert _multi(kv, d, out=None) == -1
    assert _multi(kv, d, out=4100) == -1
    assert _multi(kv, d, ws_bytes=16) == -3


def test_decode_multi_workspace_query(kv):
    """The partials of the largest launch: a launch takes up to 48 query
    columns per kv head, so with 6 query heads per kv head (24 over 4) 7
    tokens are one launch of 42 columns (7x the one-token need at the same
    split), and 10 tokens are launches of 8 and 2 tokens (8x)."""
    d = _desc(kv)
    L = kv.lib()
    one = L.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), 3, 24, 470001, 64)
    m1 = L.nvfp4kv_decode_multi_workspace_bytes(ctypes.byref(d), 3, 1, 24, 470001, 64)
    m7 = L.nvfp4kv_decode_multi_workspace_bytes(ctypes.byref(d), 3, 7, 24, 470001, 64)
    m10 = L.nvfp4kv_decode_multi_workspace_bytes(ctypes.byref(d), 3, 10, 24, 470001, 64)
    assert m1 == one
    assert 7 * one - 1024 <= m7 <= 7 * one + 1024
    assert 8 * one - 1024 <= m10 <= 8 * one + 1024
    assert L.nvfp4kv_decode_multi_workspace_bytes(ctypes.byref(d), 3, 0, 24, 1000, 0) == 0


def test_stream_read_rejects_bad_arguments(kv):
    """The read-bandwidth probe checks its arguments on the host before any
    launch."""
    d = _desc(kv)
    L = kv.lib()
    f = L.nvfp4kv_stream_read
    assert f(ctypes.byref(d), 0, 0, 4096, 16, 4096, 64, 4096, None) == -1      # n_seq 0
    assert f(ctypes.byref(d), 0, 2, 4096, 16, 4096, 0, 4096, None) == -1      # no wavefronts
    assert "n_waves" in kv.nvfp4kv_last_error()
    assert f(ctypes.byref(d), 0, 2, 4096, 16, 4096, (1 << 24) + 1, 4096, None) == -1
    assert f(ctypes.byref(d), 0, 2, None, 16, 4096, 64, 4096, None) == -1
    assert f(ctypes.byref(d), 0, 2, 4096, 16, None, 64, 4096, None) == -1
    assert f(ctypes.byref(d), 0, 2, 4096, 16, 4096, 64, None, None) == -1
    assert f(ctypes.byref(d), 0, 2, 4096, 0, 4096, 64, 4096, None) == -1      # stride
    assert f(ctypes.byref(d), 99, 2, 4096, 16, 4096, 64, 4096, None) == -1     # layer


def test_global_scale_out_of_range_is_refused():
    """The pool's per-tensor global scales: 0 (meaning 1) or 2^-64..2^64; the
    descriptor check of every call refuses others (the workspace query returns 0)."""
    import ctypes
    import math
    import nvfp4_quantized_kv_amd as kv
    for ks, vs, ok in ((0.0, 0.0, True), (3.7, 0.25, True), (-1.0, 1.0, False), (1.0, math.inf, False),
                       (math.nan, 1.0, False), (1.0, 2.0 ** -70, False)):
        d = kv._PoolDesc(None, 4, 1, 2, 128, 64, 32, 1, (ctypes.c_uint32 * 4)(0, 0, 0, 0), ks, vs)
        assert (kv._lib.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), 1, 4, 1000, 0) > 0) == ok, (ks, vs)
