"""Pins of the oracle's fp16-V variant: NVFP4 K with V kept in IEEE binary16,
the upstream storage the release post of the gzenz/ninfer fork names as its
comparison point (section "NVFP4 KV cache (from scratch)", bullet 2: "fp16 V
storage ... no outlier suppression"), 328 bytes per token per KV head.

- The binary16 rounding equals NumPy's float32 -> float16 conversion (IEEE
  round to nearest, ties to even) on ties, subnormals, the overflow edge and
  random bit patterns, and a brute-force nearest search on a sample.
- The block layout is a bijection onto its 20992 bytes; K bytes equal those
  of the NVFP4 pool.
- Attention over an fp16-V pool equals the oracle's attention with the
  fp16-rounded V rows passed in (v_rows, itself pinned), bit for bit."""
import numpy as np
import pytest

import oracle

D = 128


def _np_f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_f16_rounding_matches_numpy_on_ties_and_edges():
    # every binary16 value and the midpoints between neighbours (ties), as float32
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                      # exact in float32 (12 significant bits)
    xs = np.concatenate([v, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)]).astype(np.float32)
    xs = np.concatenate([xs, -xs, np.float32([65504, 65519.996, 65520, 65536, 1e30, np.inf, -np.inf, 0.0, -0.0,
                                              2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-30])])
    got = oracle.f16_bits(xs)
    want = _np_f16_bits(xs)
    assert np.array_equal(got, want)


def test_f16_rounding_matches_numpy_on_random_bit_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 400_000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    xs = xs[np.isfinite(xs)]
    assert np.array_equal(oracle.f16_bits(xs), _np_f16_bits(xs))
    # the values a V cache sees: normal and heavy-tailed activations
    ys = np.concatenate([rng.standard_normal(200_000) * s for s in (1.0, 32.0, 1e-3)]).astype(np.float32)
    assert np.array_equal(oracle.f16_bits(ys), _np_f16_bits(ys))


def test_f16_rounding_is_nearest_with_ties_to_even_by_search():
    """Brute force: the finite binary16 value nearest to x (in exact
    arithmetic; ties to the even bit pattern), for a sample of x."""
    fin = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = fin.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(0, 65504, 300), np.exp(rng.uniform(-20, 11, 300)),
                         (vals[:-1:97] + vals[1::97]) / 2]).astype(np.float32)
    for x in xs:
        d = np.abs(vals - float(x))
        best = np.flatnonzero(d == d.min())
        pick = best[0] if len(best) == 1 else best[(fin[best] & 1) == 0][0]
        assert oracle.f16_bits(np.float32([x]))[0] == fin[pick], x


def test_f16_value_decodes_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(b)) for b in h])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_fp16v_block_is_328_bytes_per_token_and_a_bijection():
    assert oracle.pool_bytes(1, 1, 1, v_format=1) == 64 * 328 == 20992
    assert oracle.pool_bytes(3, 5, 2, v_format=1) == 3 * 5 * 2 * 20992
    seen = np.zeros(20992, np.int32)
    for t in range(64):
        for j in range(64):
            seen[(t // 16) * 1024 + (j // 16) * 256 + (t % 16) * 16 + j % 16] += 1      # K codes
        for d in range(D):
            o = (4096 + (t // 32) * 8192 + (d % 8) * 1024 + (((t % 16) // 4) * 16 + d // 8) * 16
                 + ((t % 4) + 4 * ((t % 32) // 16)) * 2)
            seen[o] += 1
            seen[o + 1] += 1
        seen[20480 + 8 * t: 20488 + 8 * t] += 1                                           # K scales
    assert (seen == 1).all()


def _two_pools(seed, lens, hkv, rotary=32, hadamard=1, v_scale=1.0):
    rng = np.random.default_rng(seed)
    mult = np.ones(D, np.float32)
    mult[rng.choice(D, 3, replace=False)] = 32.0
    pages = [(T + 63) // 64 for T in lens]
    num_pages = sum(pages) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.zeros((len(lens), max(pages)), np.int32)
    at = 0
    for n, p in enumerate(pages):
        table[n, :p] = perm[at:at + p]
        at += p
    c, s = oracle.rope_table(1e7, rotary, 1.0, max(lens) + 1) if rotary else (None, None)
    p4 = np.zeros(oracle.pool_bytes(1, num_pages, hkv), np.uint8)
    p16 = np.zeros(oracle.pool_bytes(1, num_pages, hkv, v_format=1), np.uint8)
    ks, vs = [], []
    for n, T in enumerate(lens):
        k = (rng.standard_normal((T, hkv, D)) * mult).astype(np.float32)
        v = (rng.standard_normal((T, hkv, D)) * mult).astype(np.float32)
        pos = np.arange(T)
        sl = table[n, pos // 64].astype(np.int64) * 64 + pos % 64
        for pool, vf in ((p4, 0), (p16, 1)):
            oracle.append(pool, num_pages, hkv, rotary, hadamard, 0, k, v, sl, pos, c, s, v_scale=v_scale,
                          v_format=vf)
        ks.append(k)
        vs.append(v)
    return p4, p16, num_pages, table, ks, vs, c, s


def test_fp16v_pool_holds_the_rounded_v_rows_and_the_nvfp4_k_bytes():
    lens = [130, 64]
    hkv = 2
    p4, p16, num_pages, table, ks, vs, c, s = _two_pools(3, lens, hkv)
    for n, T in enumerate(lens):
        for t in (0, 1, 31, 32, 63, T - 1):
            slot = int(table[n, t // 64]) * 64 + t % 64
            for g in range(hkv):
                k4 = oracle.pool_read_row(p4, num_pages, hkv, 0, slot, g, 0)
                k16 = oracle.pool_read_row(p16, num_pages, hkv, 0, slot, g, 0, v_format=1)
                assert np.array_equal(k4[0], k16[0]) and np.array_equal(k4[1], k16[1])
                got = oracle.pool_read_v16(p16, num_pages, hkv, 0, slot, g)
                assert np.array_equal(got, _np_f16_bits(vs[n][t, g]))


@pytest.mark.parametrize("hadamard,v_scale", [(1, 1.0), (0, 1.0), (1, 0.25), (1, 3.0)])
def test_fp16v_attention_equals_attention_on_rounded_rows(hadamard, v_scale):
    lens = [300]
    hkv, hq = 2, 12
    p4, p16, num_pages, table, ks, vs, c, s = _two_pools(7, lens, hkv, hadamard=hadamard, v_scale=v_scale)
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    sm = 1 / np.sqrt(D)
    got = oracle.decode_attention(p16, num_pages, hkv, 0, 32, hadamard, q, [lens[0] - 1], table, lens, sm, c, s,
                                  v_scale=v_scale, v_format=1)
    # the stored values: V times the binary32 1/v_scale, rounded to fp16
    inv = np.float32(1.0) / np.float32(v_scale)
    rows = (vs[0] * inv).astype(np.float16).astype(np.float32)
    want = oracle.decode_attention(p4, num_pages, hkv, 0, 32, hadamard, q, [lens[0] - 1], table, lens, sm, c, s,
                                   v_rows=rows) * v_scale
    assert np.array_equal(got, want)


def test_fp16v_multi_query_is_one_token_decode_per_prefix():
    lens = [200, 90]
    hkv, hq, m = 2, 4, 3
    p4, p16, num_pages, table, ks, vs, c, s = _two_pools(11, lens, hkv)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, m, hq, D)).astype(np.float32)
    pos = np.array([[T - m + j for j in range(m)] for T in lens], np.int32)
    got = oracle.decode_attention_multi(p16, num_pages, hkv, 0, 32, 1, q, pos, table, lens, 1 / np.sqrt(D), c, s,
                                        v_format=1)
    for n in range(2):
        for j in range(m):
            one = oracle.decode_attention(p16, num_pages, hkv, 0, 32, 1, q[n, j][None], [pos[n, j]],
                                          table[n:n + 1], [lens[n] - m + j + 1], 1 / np.sqrt(D), c, s, v_format=1)
            assert np.array_equal(got[n, j], one[0])
