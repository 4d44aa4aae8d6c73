"""GPU parity of the page spill and restore calls against the oracle's
spill_pages / restore_pages: bit-exact bytes, pinned host and device arenas.

Release post of the gzenz/ninfer fork, section "Multi-level prefix reuse
with host-KV safety net": pages go to a pinned host arena before eviction
and come back on reuse."""
import numpy as np
import pytest
import torch

import nvfp4_quantized_kv_amd as kv
import oracle
from test_gpu_decode import Case

pytestmark = pytest.mark.gpu


def _random_pool(pages, layers, hkv, seed):
    pool = kv.Pool.allocate(pages, layers, hkv, 32, True, "cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    pool.data.copy_(torch.randint(0, 256, pool.data.shape, generator=g, dtype=torch.uint8, device="cuda"))
    return pool


@pytest.mark.parametrize("where", ["pinned", "device"])
def test_spill_matches_oracle(where):
    pool = _random_pool(40, 3, 2, 1)
    ids = np.array([7, 0, 39, 7, 12, 25, 1], np.int32)
    arena = None
    if where == "device":
        arena = torch.empty((len(ids), 3, 2, 9216), dtype=torch.uint8, device="cuda")
    got = kv.nvfp4kv_spill_pages(pool, torch.from_numpy(ids).cuda(), arena)
    torch.cuda.synchronize()
    assert got.is_pinned() if where == "pinned" else got.is_cuda
    ref = oracle.spill_pages(pool.data.cpu().numpy(), 3, 40, 2, ids)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("where", ["pinned", "device"])
def test_restore_matches_oracle(where):
    pool = _random_pool(30, 2, 4, 2)
    before = pool.data.cpu().numpy()
    ids = np.array([29, 3, 17, 14, 0], np.int32)
    src = np.random.default_rng(3).integers(0, 256, (len(ids), 2, 4, 9216), dtype=np.uint8)
    arena = torch.from_numpy(src).pin_memory() if where == "pinned" else torch.from_numpy(src).cuda()
    kv.nvfp4kv_restore_pages(pool, torch.from_numpy(ids).cuda(), arena)
    torch.cuda.synchronize()
    ref = oracle.restore_pages(before.copy(), 2, 30, 4, ids, src)
    assert np.array_equal(pool.data.cpu().numpy(), ref)


def test_page_ids_in_pinned_host_memory():
    pool = _random_pool(16, 2, 1, 4)
    ids = torch.tensor([5, 9, 2], dtype=torch.int32).pin_memory()
    got = kv.nvfp4kv_spill_pages(pool, ids)
    torch.cuda.synchronize()
    ref = oracle.spill_pages(pool.data.cpu().numpy(), 2, 16, 1, ids.numpy())
    assert np.array_equal(got.numpy(), ref)


def test_ids_out_of_range_are_skipped():
    pool = _random_pool(10, 1, 2, 5)
    before = pool.data.cpu().numpy()
    ids = torch.tensor([-1, 4, 10, 2], dtype=torch.int32, device="cuda")
    arena = torch.full((4, 1, 2, 9216), 0xA5, dtype=torch.uint8).pin_memory()
    kv.nvfp4kv_spill_pages(pool, ids, arena)
    torch.cuda.synchronize()
    a = arena.numpy()
    assert (a[0] == 0xA5).all() and (a[2] == 0xA5).all()
    ref = oracle.spill_pages(before, 1, 10, 2, [4, 2])
    assert np.array_equal(a[1], ref[0]) and np.array_equal(a[3], ref[1])
    arena[:] = 0
    kv.nvfp4kv_restore_pages(pool, ids, arena)
    torch.cuda.synchronize()
    want = oracle.restore_pages(before.copy(), 1, 10, 2, [4, 2], np.zeros((2, 1, 2, 9216), np.uint8))
    assert np.array_equal(pool.data.cpu().numpy(), want)


def test_pageable_arena_is_refused():
    pool = _random_pool(8, 1, 1, 6)
    ids = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    arena = torch.zeros((2, 1, 1, 9216), dtype=torch.uint8)        # ordinary host memory
    with pytest.raises(RuntimeError, match="pinned"):
        kv.nvfp4kv_spill_pages(pool, ids, arena)
    with pytest.raises(RuntimeError, match="pinned"):
        kv.nvfp4kv_restore_pages(pool, ids, arena)


def test_pages_moved_through_the_host_give_the_same_attention():
    """Spill every page of a cache, restore them under other page ids into a
    fresh pool, rename the page table: decode output is bit for bit the same."""
    c = Case(70, [3000, 777, 64], 4, 24)
    out0 = c.gpu()
    used = np.unique(c.table[c.table >= 0]).astype(np.int32)
    arena = kv.nvfp4kv_spill_pages(c.pool, torch.from_numpy(used).cuda())
    perm = np.random.default_rng(7).permutation(c.num_pages).astype(np.int32)[:len(used)]
    fresh = kv.Pool.allocate(c.num_pages, 1, c.hkv, c.rotary, c.hadamard, "cuda")
    fresh.data.fill_(0x3C)
    kv.nvfp4kv_restore_pages(fresh, torch.from_numpy(perm).cuda(), arena)
    rename = np.full(c.num_pages, -1, np.int32)
    rename[used] = perm
    table = np.where(c.table >= 0, rename[np.maximum(c.table, 0)], c.table).astype(np.int32)
    c.pool, c.table = fresh, table
    out1 = c.gpu()
    assert np.array_equal(out0, out1)


def test_spill_restore_full_page_size():
    """16 layers x 4 kv heads (589,824 bytes a page), 300 pages each way."""
    pool = _random_pool(1200, 16, 4, 8)
    before = pool.data.cpu().numpy()
    ids = np.random.default_rng(9).choice(1200, 300, replace=False).astype(np.int32)
    arena = kv.nvfp4kv_spill_pages(pool, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    ref = oracle.spill_pages(before, 16, 1200, 4, ids)
    assert np.array_equal(arena.numpy(), ref)
    back = np.roll(ids, 1)
    kv.nvfp4kv_restore_pages(pool, torch.from_numpy(back).cuda(), arena)
    torch.cuda.synchronize()
    assert np.array_equal(pool.data.cpu().numpy(), oracle.restore_pages(before.copy(), 16, 1200, 4, back, ref))
