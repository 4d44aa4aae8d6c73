"""The checked build (libnvfp4kv_debug.so) on the GPU: with good tables its
results equal the regular build's bit for bit; a bad page id, a racing slot,
a too-short sequence or a repeated restore id is refused with
NVFP4KV_ERR_INVALID_ARG before anything is launched (outputs and pool left
as they were).  Nothing out of range ever reaches a kernel here."""
import numpy as np
import pytest
import torch

from test_gpu_decode import Case

pytestmark = pytest.mark.gpu

SM = 1 / np.sqrt(128)


@pytest.fixture
def checked(monkeypatch):
    import nvfp4_quantized_kv_amd as kv
    from nvfp4_quantized_kv_amd import build as B
    dbg = kv.load_build(B.DEBUG_LIB)
    assert kv.nvfp4kv_checked_build(dbg)
    return lambda: monkeypatch.setattr(kv, "_lib", dbg)


def _refused(fn, match):
    import nvfp4_quantized_kv_amd as kv
    with pytest.raises(kv.NVFP4KVError) as e:
        fn()
    assert e.value.code == kv.ERR_INVALID_ARG and match in str(e.value), str(e.value)


def test_checked_build_matches_and_refuses(checked):
    import nvfp4_quantized_kv_amd as kv
    c = Case(1700, [700, 130, 65], 2, 12)
    good = c.gpu()
    held = Case(1701, [300, 64], 2, 12, hold_last=True)
    good_fused = held.gpu(fused=True)
    held_pool = held.pool.data.clone()
    checked()
    assert np.array_equal(c.gpu(), good)
    held.pool.data.copy_(held_pool)
    # (the fused call writes its token again, the same bytes)
    assert np.array_equal(held.gpu(fused=True), good_fused)
    assert torch.equal(held.pool.data, held_pool)

    q, qp = c.q.cuda(), torch.from_numpy(c.q_pos).cuda()
    lens = torch.tensor(c.lens, dtype=torch.int32).cuda()
    bad = c.table.copy()
    bad[0, 5] = c.num_pages + 5
    out = torch.full((3, 12, 128), 7.0, device="cuda")
    _refused(lambda: kv.nvfp4kv_decode_attn(c.pool, 0, q, qp, torch.from_numpy(bad).cuda(), lens, max(c.lens), SM,
                                            out=out, rope_cos=c.rc, rope_sin=c.rs), "page_table[0][5]")
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

    before = c.pool.data.clone()
    k = torch.zeros((3, 2, 128), dtype=torch.bfloat16, device="cuda")
    slots = torch.tensor([5, 9, 5], dtype=torch.int64, device="cuda")
    pos = torch.tensor([1, 2, 3], dtype=torch.int32, device="cuda")
    _refused(lambda: kv.nvfp4kv_append(c.pool, 0, k, k, slots, pos, c.rc, c.rs), "both name slot 5")
    slots = torch.tensor([5, c.num_pages * 64], dtype=torch.int64, device="cuda")
    _refused(lambda: kv.nvfp4kv_append(c.pool, 0, k[:2], k[:2], slots, pos[:2], c.rc, c.rs), "slots[1]")
    torch.cuda.synchronize()
    assert torch.equal(c.pool.data, before)

    qm = torch.zeros((3, 4, 12, 128), dtype=torch.float32, device="cuda")
    qpos = torch.zeros((3, 4), dtype=torch.int32, device="cuda")
    short = torch.tensor([700, 3, 65], dtype=torch.int32, device="cuda")
    _refused(lambda: kv.nvfp4kv_decode_attn_multi(c.pool, 0, qm, qpos, torch.from_numpy(c.table).cuda(), short,
                                                  700, SM, rope_cos=c.rc, rope_sin=c.rs), "seq_lens[1] = 3")

    ids = torch.tensor([1, 2, 1], dtype=torch.int32, device="cuda")
    arena = kv.nvfp4kv_spill_pages(c.pool, torch.tensor([1, 2, 3], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _refused(lambda: kv.nvfp4kv_restore_pages(c.pool, ids, arena), "both name page 1")
    torch.cuda.synchronize()
    assert torch.equal(c.pool.data, before)
