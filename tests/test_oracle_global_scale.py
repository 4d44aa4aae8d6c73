"""Pins of the oracle's per-tensor global scale (NVFP4's second scaling
level: one FP32 factor per tensor over the E4M3 block scales, NVIDIA's NVFP4
format description; the release post of the gzenz/ninfer fork, section
"NVFP4 KV cache", keeps it at 1).

What the format fixes, independent of the oracle's own arithmetic:
- a power-of-two scale 2^j leaves every E2M1 code unchanged and lowers every
  (normal) E4M3 scale code by 8 j, since the exponent field sits above three
  mantissa bits;
- the dequantized values, and so attention, are then the same as without it;
- a block whose amax/6 exceeds E4M3's largest value 448 saturates without a
  global scale, and with one each element lands within the block bound
  |x - x_hat| <= 1.0625 amax / 6 (grid gap at most 2 between 4 and 6, times
  a scale at most 2^-4 below amax/6)."""
import numpy as np
import pytest

import oracle

HKV, PAGES = 2, 3


def _pool():
    return np.zeros(oracle.pool_bytes(1, PAGES, HKV), np.uint8)


def _rows(seed, n, mult=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, HKV, 128)) * mult
    x[:, :, 5] *= 16.0
    return x.astype(np.float32)


def _fill(k, v, k_scale, v_scale, hadamard=1, rotary=32):
    n = k.shape[0]
    c, s = oracle.rope_table(1e7, rotary, 1.0, n + 1) if rotary else (None, None)
    pool = _pool()
    slots = np.arange(n, dtype=np.int64)
    oracle.append(pool, PAGES, HKV, rotary, hadamard, 0, k, v, slots, np.arange(n, dtype=np.int32), c, s,
                  k_scale=k_scale, v_scale=v_scale)
    return pool, c, s


def _read(pool, n, which):
    codes, scales = zip(*[oracle.pool_read_row(pool, PAGES, HKV, 0, t, h, which)
                          for t in range(n) for h in range(HKV)])
    return np.stack(codes), np.stack(scales).astype(np.int64)


@pytest.mark.parametrize("jk,jv", [(2, -1), (-3, 4)])
def test_power_of_two_scale_shifts_only_the_scale_exponent(jk, jv):
    n = 70
    k, v = _rows(1, n), _rows(2, n)
    p1, _, _ = _fill(k, v, 1.0, 1.0)
    p2, _, _ = _fill(k, v, 2.0 ** jk, 2.0 ** jv)
    for which, j in ((0, jk), (1, jv)):
        c1, s1 = _read(p1, n, which)
        c2, s2 = _read(p2, n, which)
        normal = (s1 >= 8 + 8 * max(j, 0)) & (s1 + 8 * max(-j, 0) <= 0x7E)
        assert normal.mean() > 0.8
        rows = normal.all(axis=1)
        assert np.array_equal(c1[rows], c2[rows])
        assert np.array_equal(s2[normal], s1[normal] - 8 * j)


def test_power_of_two_scales_leave_attention_unchanged():
    n = 150
    k, v = _rows(3, n), _rows(4, n)
    q = np.concatenate([_rows(5, 1)] * 3, axis=1)          # 6 query heads over 2 kv heads
    table = np.arange(PAGES, dtype=np.int32)[None, :]
    args = (np.array([n - 1], np.int32), table, np.array([n], np.int32), 1 / np.sqrt(128))
    p1, c, s = _fill(k, v, 1.0, 1.0)
    p2, _, _ = _fill(k, v, 4.0, 0.5)
    o1 = oracle.decode_attention(p1, PAGES, HKV, 0, 32, 1, q, *args, c, s)
    o2 = oracle.decode_attention(p2, PAGES, HKV, 0, 32, 1, q, *args, c, s, k_scale=4.0, v_scale=0.5)
    assert np.abs(o2 - o1).max() <= 1e-12 * np.abs(o1).max()
    # leaving either factor out of the decode changes the result
    o3 = oracle.decode_attention(p2, PAGES, HKV, 0, 32, 1, q, *args, c, s, k_scale=1.0, v_scale=0.5)
    o4 = oracle.decode_attention(p2, PAGES, HKV, 0, 32, 1, q, *args, c, s, k_scale=4.0, v_scale=1.0)
    assert np.abs(o3 - o1).max() > 1e-3 and np.abs(o4 - o1).max() > 1e-3


def test_global_scale_relieves_e4m3_saturation():
    """V rows of amax ~ 1e4 (no RoPE or rotation on V): the block scale
    saturates at 448 without a global scale; with v_scale 64 every element
    is within the block bound."""
    n = 64
    k = _rows(6, n)
    v = _rows(7, n, mult=600.0)
    for g, ok in ((1.0, False), (64.0, True)):
        pool, _, _ = _fill(k, v, 1.0, g)
        worst = 0.0
        for t in range(n):
            for h in range(HKV):
                codes, scales = oracle.pool_read_row(pool, PAGES, HKV, 0, t, h, 1)
                xh = oracle.dequant_row(codes, scales) * g
                x = v[t, h].astype(np.float64)
                for b in range(8):
                    blk = slice(16 * b, 16 * b + 16)
                    bound = 1.0625 * np.abs(x[blk]).max() / 6
                    worst = max(worst, np.abs(x[blk] - xh[blk]).max() / bound)
        assert (worst <= 1.0) == ok, (g, worst)


def test_zero_scale_means_one():
    n = 20
    k, v = _rows(8, n), _rows(9, n)
    p1, _, _ = _fill(k, v, 1.0, 1.0)
    p0, _, _ = _fill(k, v, 0.0, 0.0)
    assert np.array_equal(p0, p1)
