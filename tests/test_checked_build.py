"""The range checks of device-side tables (page ids, slots, positions,
sequence lengths), on the host, without a GPU: nvfp4kv_check_decode_tables,
nvfp4kv_check_slots and nvfp4kv_check_page_ids refuse every out-of-range or
racing entry with NVFP4KV_ERR_INVALID_ARG and name its index, and accept good
tables.  The checked build (libnvfp4kv_debug.so) runs the same routines inside
every entry point before launching; it loads, exports every declared symbol
and reports itself as checked.

(The release post of the gzenz/ninfer fork lists, in its section "Also
included", a use-after-free caused by a missing stream synchronization: the
checked build is the tool for catching a bad table before a kernel reads with
it.)"""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kv():
    from nvfp4_quantized_kv_amd import build as B
    if B.stale() or B.stale(B.DEBUG_LIB):
        B.build()
    import nvfp4_quantized_kv_amd as kv
    return kv


def _pool(kv, num_pages=10, hkv=2, rotary=32):
    return kv.Pool(None, num_pages, 1, hkv, rotary, 1)


class _FakeData:
    def data_ptr(self):
        return 256


def _pool_desc_only(kv, **kw):
    p = _pool(kv, **kw)
    p.data = _FakeData()
    return p


def _raises(fn, *args, match, **kw):
    import nvfp4_quantized_kv_amd as kv
    with pytest.raises(kv.NVFP4KVError) as e:
        fn(*args, **kw)
    assert e.value.code == kv.ERR_INVALID_ARG
    assert match in str(e.value), str(e.value)


def test_decode_tables_accept_good_and_name_bad_entries(kv):
    p = _pool_desc_only(kv)
    table = np.array([[3, 4, 9], [0, 1, 2]], np.int32)
    lens = np.array([130, 64], np.int32)
    kv.nvfp4kv_check_decode_tables(p, table, lens, 192, q_positions=np.array([129, 63]), max_pos=200)
    bad = table.copy()
    bad[0, 2] = 10                                     # the third page of sequence 0 is used (130 tokens)
    _raises(kv.nvfp4kv_check_decode_tables, p, bad, lens, 192, match="page_table[0][2] = 10")
    bad = table.copy()
    bad[1, 2] = -7                                     # not used: sequence 1 holds one page
    kv.nvfp4kv_check_decode_tables(p, bad, lens, 192)
    bad[1, 0] = -7
    _raises(kv.nvfp4kv_check_decode_tables, p, bad, lens, 192, match="page_table[1][0] = -7")
    _raises(kv.nvfp4kv_check_decode_tables, p, table, np.array([0, 64]), 192, match="seq_lens[0] = 0")
    _raises(kv.nvfp4kv_check_decode_tables, p, table, np.array([130, 193]), 192, match="seq_lens[1] = 193")
    _raises(kv.nvfp4kv_check_decode_tables, p, table, lens, 192, q_positions=np.array([129, 200]), max_pos=200,
            match="q_positions[1] = 200")
    _raises(kv.nvfp4kv_check_decode_tables, p, table, np.array([130, 2]), 192, n_qtok=3, match="seq_lens[1] = 2")
    # positions are not looked at without RoPE
    p0 = _pool_desc_only(kv, rotary=0)
    kv.nvfp4kv_check_decode_tables(p0, table, lens, 192, q_positions=np.array([-5, 10 ** 6]), max_pos=1)


def test_slots_checks_range_distinctness_and_positions(kv):
    p = _pool_desc_only(kv, num_pages=2)
    kv.nvfp4kv_check_slots(p, np.array([0, 127, 64, 5]), np.array([0, 1, 2, 3]), max_pos=4)
    _raises(kv.nvfp4kv_check_slots, p, np.array([0, 128]), match="slots[1] = 128")
    _raises(kv.nvfp4kv_check_slots, p, np.array([-1]), match="slots[0] = -1")
    _raises(kv.nvfp4kv_check_slots, p, np.array([5, 9, 5]), match="slots[0] and slots[2] both name slot 5")
    _raises(kv.nvfp4kv_check_slots, p, np.array([5, 9]), np.array([3, 4]), max_pos=4, match="positions[1] = 4")


def test_page_ids_restores_must_be_distinct(kv):
    p = _pool_desc_only(kv, num_pages=8)
    kv.nvfp4kv_check_page_ids(p, np.array([3, 3, 99, -1]), distinct=False)   # a spill may repeat; outside ids skip
    kv.nvfp4kv_check_page_ids(p, np.array([3, 99, 99, 4]), distinct=True)    # ids outside the pool are skipped
    _raises(kv.nvfp4kv_check_page_ids, p, np.array([1, 7, 1]), distinct=True,
            match="page_ids[0] and page_ids[2] both name page 1")


def test_checked_build_loads_and_exports_the_boundary(kv):
    from nvfp4_quantized_kv_amd import build as B
    dbg = kv.load_build(B.DEBUG_LIB)
    assert kv.nvfp4kv_checked_build(dbg) and not kv.nvfp4kv_checked_build(kv.load_build(B.LIB))
    import re
    src = open(os.path.join(ROOT, "include", "nvfp4kv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    for name in sorted(set(re.findall(r"\b(nvfp4kv_\w+)\s*\(", src))):
        assert hasattr(dbg, name), name
    # the routines behave the same in the checked build
    p = _pool_desc_only(kv, num_pages=2)
    _raises(kv.nvfp4kv_check_slots, p, np.array([0, 128]), match="slots[1] = 128", lib=dbg)
