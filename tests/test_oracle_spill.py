"""Pins of the oracle's page spill and restore (release post of the
gzenz/ninfer fork, section "Multi-level prefix reuse with host-KV safety
net": pages are copied to a pinned host arena and back).

The oracle gathers with numpy indexing; these tests fix it against the
pool's byte addressing written out element by element, against a round
trip, and against attention: a cache whose pages were spilled and restored
under other page ids, with the page table renamed to match, gives the same
decode output as the original."""
import numpy as np

import oracle

B = oracle.BLOCK_BYTES


def _pool(layers, pages, hkv, seed):
    return np.random.default_rng(seed).integers(0, 256, layers * pages * hkv * B, dtype=np.uint8)


def test_spill_matches_byte_addressing():
    layers, pages, hkv = 3, 5, 2
    pool = _pool(layers, pages, hkv, 0)
    ids = [4, 0, 4, 2]
    arena = oracle.spill_pages(pool, layers, pages, hkv, ids)
    assert arena.shape == (4, layers, hkv, B)
    flat = arena.reshape(-1)
    rng = np.random.default_rng(1)
    for _ in range(2000):
        i, l, g, x = rng.integers(0, 4), rng.integers(0, layers), rng.integers(0, hkv), rng.integers(0, B)
        pool_off = ((l * pages + ids[i]) * hkv + g) * B + x
        arena_off = ((i * layers + l) * hkv + g) * B + x
        assert flat[arena_off] == pool[pool_off]


def test_restore_round_trip_and_untouched_pages():
    layers, pages, hkv = 2, 6, 3
    pool = _pool(layers, pages, hkv, 2)
    ids = [5, 1, 3]
    arena = oracle.spill_pages(pool, layers, pages, hkv, ids)
    other = _pool(layers, pages, hkv, 3)
    before = other.copy()
    oracle.restore_pages(other, layers, pages, hkv, ids, arena)
    v_new = other.reshape(layers, pages, hkv, B)
    v_src = pool.reshape(layers, pages, hkv, B)
    v_old = before.reshape(layers, pages, hkv, B)
    for pid in range(pages):
        want = v_src[:, pid] if pid in ids else v_old[:, pid]
        assert np.array_equal(v_new[:, pid], want), pid


def test_restore_refuses_repeated_ids():
    layers, pages, hkv = 1, 3, 1
    pool = _pool(layers, pages, hkv, 4)
    arena = oracle.spill_pages(pool, layers, pages, hkv, [0, 1, 2])
    try:
        oracle.restore_pages(np.zeros_like(pool), layers, pages, hkv, [2, 0, 2], arena)
    except ValueError:
        return
    raise AssertionError("repeated ids accepted")


def test_moved_pages_give_the_same_attention():
    """Spill a sequence's pages, restore them under new page ids, rename the
    page table: decode attention is unchanged, bit for bit."""
    hkv, pages, layers, T = 2, 6, 2, 150
    rng = np.random.default_rng(5)
    pool = np.zeros(oracle.pool_bytes(layers, pages, hkv), np.uint8)
    table = np.array([[3, 0, 5, -1, -1, -1]], np.int32)
    k = rng.standard_normal((T, hkv, 128)).astype(np.float32)
    v = rng.standard_normal((T, hkv, 128)).astype(np.float32)
    slots = table[0, np.arange(T) // 64].astype(np.int64) * 64 + np.arange(T) % 64
    for layer in range(layers):
        oracle.append(pool, pages, hkv, 0, True, layer, k, v, slots, np.arange(T))
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    ref = oracle.decode_attention(pool, pages, hkv, 1, 0, True, q, [T - 1], table, [T], 1 / np.sqrt(128))
    used = [3, 0, 5]
    arena = oracle.spill_pages(pool, layers, pages, hkv, used)
    moved = np.zeros_like(pool)
    new_ids = [1, 4, 2]
    oracle.restore_pages(moved, layers, pages, hkv, new_ids, arena)
    table2 = np.array([[1, 4, 2, -1, -1, -1]], np.int32)
    out = oracle.decode_attention(moved, pages, hkv, 1, 0, True, q, [T - 1], table2, [T], 1 / np.sqrt(128))
    assert np.array_equal(out, ref)
