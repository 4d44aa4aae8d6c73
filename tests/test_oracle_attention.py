"""Pins of the oracle's pool layout, append and decode attention.

Method: release post of the gzenz/ninfer fork, section "NVFP4 KV cache (from
scratch)": Q and K rotated and quantized to NVFP4, V quantized without
rotation and dequantized for PV, the current token appended in place, KV
scales row-major, 144 bytes per token per KV head."""
import mpmath
import numpy as np

import oracle

D = 128


def _pool(num_pages, hkv, layers=1):
    return np.zeros(oracle.pool_bytes(layers, num_pages, hkv), np.uint8)


def test_layout_is_a_bijection_with_row_major_scales():
    """Writing distinct rows into all 64 slots of a page touches every byte of
    the 9216-byte block exactly once, and the scales of token t sit at
    t*8 .. t*8+7 of their region (row-major, release post bullet 4)."""
    hkv = 1
    pool = _pool(1, hkv)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((64, 1, D)).astype(np.float32)
    v = rng.standard_normal((64, 1, D)).astype(np.float32)
    oracle.append(pool, 1, hkv, 0, False, 0, k, v, np.arange(64), np.zeros(64))
    seen = np.zeros(9216, np.int32)
    for t in range(64):
        for which, x in ((0, k), (1, v)):
            codes, scales = oracle.quant_row(x[t, 0], 0, None, None, False)
            c2, s2 = oracle.pool_read_row(pool, 1, hkv, 0, t, 0, which)
            assert (c2 == codes).all() and (s2 == scales).all()
            base = 8192 if which == 0 else 8704
            assert (pool[base + 8 * t: base + 8 * t + 8] == scales).all()
    # bijection: mark each byte a row read touches
    for t in range(64):
        for j in range(64):
            seen[(t // 16) * 1024 + (j // 16) * 256 + (t % 16) * 16 + j % 16] += 1
            seen[4096 + (t // 4) * 256 + (j // 4) * 16 + (t % 4) * 4 + j % 4] += 1
        seen[8192 + 8 * t: 8200 + 8 * t] += 1
        seen[8704 + 8 * t: 8712 + 8 * t] += 1
    assert (seen == 1).all()


def test_append_rotates_k_but_not_v():
    hkv = 2
    pool = _pool(2, hkv)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((3, hkv, D)).astype(np.float32)
    v = rng.standard_normal((3, hkv, D)).astype(np.float32)
    c, s = oracle.rope_table(1e7, 32, 1.0, 50)
    slots = np.array([5, 64 + 9, 127])
    pos = np.array([3, 40, 49])
    oracle.append(pool, 2, hkv, 32, True, 0, k, v, slots, pos, c, s)
    for i in range(3):
        for g in range(hkv):
            kc, ks = oracle.pool_read_row(pool, 2, hkv, 0, slots[i], g, 0)
            kh = oracle.dequant_row(kc, ks)
            # un-rotating K-hat (H is its own inverse) recovers RoPE(k) to quantization accuracy
            kr = oracle.rope_apply(k[i, g], 32, c[pos[i]], s[pos[i]]).astype(np.float64)
            back = oracle.hadamard128(kh.astype(np.float32)).astype(np.float64)
            assert np.linalg.norm(back - kr) <= 0.15 * np.linalg.norm(kr)
            vc, vs = oracle.pool_read_row(pool, 2, hkv, 0, slots[i], g, 1)
            assert (vc == oracle.quant_row(v[i, g])[0]).all()
            assert (vs == oracle.quant_row(v[i, g])[1]).all()


def _mp_attention(qh, kh, vh, scale):
    """Brute force in 50-digit arithmetic, softmax without max subtraction."""
    mpmath.mp.dps = 50
    T = kh.shape[0]
    z = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                          for a, b in zip(qh, kh[t])) for t in range(T)]
    e = [mpmath.exp(x) for x in z]
    tot = mpmath.fsum(e)
    return np.array([float(mpmath.fsum(e[t] * mpmath.mpf(float(vh[t, d])) for t in range(T)) / tot)
                     for d in range(D)])


def _small_case(seed, T, hkv, hq, rotary, hadamard, scale=1 / np.sqrt(128)):
    rng = np.random.default_rng(seed)
    n_pages = (T + 63) // 64 + 2
    pool = _pool(n_pages, hkv)
    perm = rng.permutation(n_pages)
    table = perm[: (T + 63) // 64].astype(np.int32)[None, :]
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    pos = np.arange(T)
    slots = table[0, pos // 64].astype(np.int64) * 64 + pos % 64
    c = s = None
    if rotary:
        c, s = oracle.rope_table(1e7, rotary, 1.0, T + 1)
    oracle.append(pool, n_pages, hkv, rotary, hadamard, 0, k, v, slots, pos, c, s)
    out = oracle.decode_attention(pool, n_pages, hkv, 0, rotary, hadamard, q, [T - 1], table, [T],
                                  scale, c, s)
    return dict(pool=pool, n_pages=n_pages, table=table, q=q, k=k, v=v, c=c, s=s, out=out,
                slots=slots)


def test_attention_brute_force_tiny():
    for seed, T in ((10, 1), (11, 2), (12, 3), (13, 4)):
        hkv, hq = 1, 2
        cs = _small_case(seed, T, hkv, hq, 32, True)
        for h in range(hq):
            codes, scales = oracle.quant_row(cs["q"][0, h], 32, cs["c"][T - 1], cs["s"][T - 1], True)
            qh = oracle.dequant_row(codes, scales)
            kh = np.stack([oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][t], 0, 0)) for t in range(T)])
            vh = np.stack([oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][t], 0, 1)) for t in range(T)])
            ref = _mp_attention(qh, kh, vh, 1 / np.sqrt(128))
            assert np.abs(cs["out"][0, h] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_single_token_returns_v_hat():
    cs = _small_case(20, 1, 1, 2, 0, True)
    vh = oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][0], 0, 1))
    assert (cs["out"][0, 0] == vh).all() and (cs["out"][0, 1] == vh).all()


def test_zero_scale_gives_mean_and_weights_sum_to_one():
    cs = _small_case(21, 150, 1, 2, 0, True)
    out0 = oracle.decode_attention(cs["pool"], cs["n_pages"], 1, 0, 0, True, cs["q"], [149],
                                   cs["table"], [150], 0.0)
    vh = np.stack([oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][t], 0, 1)) for t in range(150)])
    assert np.abs(out0[0, 0] - vh.mean(0)).max() <= 1e-12 * np.abs(vh).max()
    # a cache whose V rows all dequantize to the same vector returns that vector
    # whatever the weights are: the weights sum to one
    pool = cs["pool"].copy()
    c0, s0 = oracle.pool_read_row(pool, cs["n_pages"], 1, 0, cs["slots"][0], 0, 1)
    blocks = pool.reshape(-1, 9216)
    for t in range(150):
        blk = blocks[cs["slots"][t] // 64]
        tt = cs["slots"][t] % 64
        for j in range(64):
            blk[4096 + (tt // 4) * 256 + (j // 4) * 16 + (tt % 4) * 4 + j % 4] = c0[j]
        blk[8704 + 8 * tt: 8712 + 8 * tt] = s0
    out = oracle.decode_attention(pool, cs["n_pages"], 1, 0, 0, True, cs["q"], [149], cs["table"], [150],
                                  1 / np.sqrt(128))
    v0 = oracle.dequant_row(c0, s0)
    assert np.abs(out[0] - v0[None]).max() <= 1e-12 * np.abs(v0).max()


def test_gqa_mapping_consecutive_heads_share_a_kv_head():
    """Query head h reads kv head h // (hq/hkv): give each kv head a constant V."""
    hkv, hq, T = 3, 6, 70
    n_pages = 2
    pool = _pool(n_pages, hkv)
    rng = np.random.default_rng(30)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = np.zeros((T, hkv, D), np.float32)
    for g in range(hkv):
        v[:, g, :] = (g + 1) * 0.75      # 6 * s with s = 0.125, 0.25, 0.375: a fixed point
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    oracle.append(pool, n_pages, hkv, 0, True, 0, k, v, np.arange(T), np.arange(T))
    out = oracle.decode_attention(pool, n_pages, hkv, 0, 0, True, q, [T - 1],
                                  np.array([[0, 1]], np.int32), [T], 1 / np.sqrt(128))
    for h in range(hq):
        assert np.allclose(out[0, h], (h // 2 + 1) * 0.75, rtol=0, atol=1e-12)


def test_page_permutation_invariance():
    T, hkv, hq = 300, 2, 4
    rng = np.random.default_rng(40)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    c, s = oracle.rope_table(1e7, 32, 1.0, T + 1)
    outs = []
    for perm_seed in (0, 1):
        n_pages = 8
        table = np.random.default_rng(perm_seed).permutation(n_pages)[:5].astype(np.int32)[None]
        pool = _pool(n_pages, hkv)
        pos = np.arange(T)
        slots = table[0, pos // 64].astype(np.int64) * 64 + pos % 64
        oracle.append(pool, n_pages, hkv, 32, True, 0, k, v, slots, pos, c, s)
        outs.append(oracle.decode_attention(pool, n_pages, hkv, 0, 32, True, q, [T - 1], table, [T],
                                            1 / np.sqrt(128), c, s))
    assert (outs[0] == outs[1]).all()


def test_representable_query_is_used_as_is():
    """With no RoPE and no rotation, a query whose blocks are already NVFP4
    values quantizes to itself, so the output equals attention computed with
    the raw query (closed-form softmax over the cached K-hat, V-hat)."""
    T, hkv, hq = 40, 1, 1
    rng = np.random.default_rng(50)
    nib = rng.integers(0, 16, 128)
    nib[::16] = 7
    scodes = rng.integers(40, 60, 8)
    qv = np.array([oracle.e2m1_value(nib[d]) * oracle.e4m3_value(scodes[d // 16]) for d in range(128)],
                  np.float32)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    pool = _pool(1, hkv)
    oracle.append(pool, 1, hkv, 0, False, 0, k, v, np.arange(T), np.arange(T))
    out = oracle.decode_attention(pool, 1, hkv, 0, 0, False, qv[None, None], [T - 1],
                                  np.array([[0]], np.int32), [T], 0.05)
    kh = np.stack([oracle.dequant_row(*oracle.pool_read_row(pool, 1, 1, 0, t, 0, 0)) for t in range(T)])
    vh = np.stack([oracle.dequant_row(*oracle.pool_read_row(pool, 1, 1, 0, t, 0, 1)) for t in range(T)])
    ref = _mp_attention(qv.astype(np.float64), kh, vh, 0.05)
    assert np.abs(out[0, 0] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_quantized_attention_close_to_unquantized_reference():
    """Not a parity gate: NVFP4 attention tracks fp64 attention on the raw rows."""
    T, hkv, hq = 256, 1, 2
    rng = np.random.default_rng(60)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    pool = _pool(4, hkv)
    oracle.append(pool, 4, hkv, 0, True, 0, k, v, np.arange(T), np.arange(T))
    out = oracle.decode_attention(pool, 4, hkv, 0, 0, True, q, [T - 1], np.array([[0, 1, 2, 3]], np.int32),
                                  [T], 1 / np.sqrt(128))
    ref = oracle.reference_attention(q[0], T - 1, k, v, np.arange(T), 0, 1 / np.sqrt(128))
    rel = np.linalg.norm(out[0] - ref) / np.linalg.norm(ref)
    assert rel < 0.25


def _multi_case(seed, T, m, hkv, hq, rotary=32, hadamard=True):
    """T cached tokens (the last m are the new ones) and m query tokens per sequence."""
    rng = np.random.default_rng(seed)
    n_pages = (T + 63) // 64 + 1
    pool = _pool(n_pages, hkv)
    table = rng.permutation(n_pages)[: (T + 63) // 64].astype(np.int32)[None, :]
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    pos = np.arange(T)
    slots = table[0, pos // 64].astype(np.int64) * 64 + pos % 64
    c = s = None
    if rotary:
        c, s = oracle.rope_table(1e7, rotary, 1.0, T + 1)
    oracle.append(pool, n_pages, hkv, rotary, hadamard, 0, k, v, slots, pos, c, s)
    q = rng.standard_normal((1, m, hq, D)).astype(np.float32)
    q_pos = (T - m + np.arange(m))[None, :]
    return dict(pool=pool, n_pages=n_pages, table=table, q=q, q_pos=q_pos, c=c, s=s, slots=slots,
                k=k, v=v, T=T, m=m, hkv=hkv, hq=hq, rotary=rotary, hadamard=hadamard)


def _multi(cs, pool=None, scale=1 / np.sqrt(128)):
    return oracle.decode_attention_multi(cs["pool"] if pool is None else pool, cs["n_pages"], cs["hkv"], 0,
                                         cs["rotary"], cs["hadamard"], cs["q"], cs["q_pos"], cs["table"],
                                         [cs["T"]], scale, cs["c"], cs["s"])


def test_multi_query_brute_force_causal():
    """Query token j of m new tokens attends to tokens 0 .. T-m+j: 50-digit
    softmax over exactly that prefix (ai-manual.ru "Ninfer 4080", section
    "Key features": several drafted tokens checked in one step)."""
    cs = _multi_case(40, 6, 3, 1, 2)
    out = _multi(cs)
    kh = np.stack([oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][t], 0, 0)) for t in range(6)])
    vh = np.stack([oracle.dequant_row(*oracle.pool_read_row(cs["pool"], cs["n_pages"], 1, 0, cs["slots"][t], 0, 1)) for t in range(6)])
    for j in range(3):
        p = cs["q_pos"][0, j]
        for h in range(2):
            codes, scales = oracle.quant_row(cs["q"][0, j, h], 32, cs["c"][p], cs["s"][p], True)
            ref = _mp_attention(oracle.dequant_row(codes, scales), kh[: 6 - 3 + j + 1], vh[: 6 - 3 + j + 1], 1 / np.sqrt(128))
            assert np.abs(out[0, j, h] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), (j, h)


def test_multi_query_one_token_is_decode():
    cs = _multi_case(41, 200, 1, 2, 4)
    single = oracle.decode_attention(cs["pool"], cs["n_pages"], 2, 0, 32, True, cs["q"][:, 0], [199],
                                     cs["table"], [200], 1 / np.sqrt(128), cs["c"], cs["s"])
    assert (_multi(cs)[:, 0] == single).all()


def test_multi_query_is_causal():
    """Rewriting the last token's K and V changes only the last query token's
    output; rewriting token T-m changes all of them."""
    cs = _multi_case(42, 130, 4, 1, 2)
    base = _multi(cs)
    for t, changed in ((129, [3]), (126, [0, 1, 2, 3])):
        pool = cs["pool"].copy()
        k2 = cs["k"][t:t + 1] * -2.0
        v2 = cs["v"][t:t + 1] + 3.0
        oracle.append(pool, cs["n_pages"], 1, 32, True, 0, k2, v2, cs["slots"][t:t + 1], [t], cs["c"], cs["s"])
        out = _multi(cs, pool)
        diff = [j for j in range(4) if not (out[0, j] == base[0, j]).all()]
        assert diff == changed, (t, diff)


def test_random_sign_attention_close_to_unquantized_reference():
    """Not a parity gate: with the randomized rotation on K (append) and Q
    (decode), NVFP4 attention still tracks fp64 attention on the raw rows."""
    T, hkv, hq = 256, 1, 2
    rng = np.random.default_rng(61)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    mask = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
    pool = _pool(4, hkv)
    oracle.append(pool, 4, hkv, 0, 2, 0, k, v, np.arange(T), np.arange(T), signs=mask)
    out = oracle.decode_attention(pool, 4, hkv, 0, 0, 2, q, [T - 1], np.array([[0, 1, 2, 3]], np.int32),
                                  [T], 1 / np.sqrt(128), signs=mask)
    ref = oracle.reference_attention(q[0], T - 1, k, v, np.arange(T), 0, 1 / np.sqrt(128))
    rel = np.linalg.norm(out[0] - ref) / np.linalg.norm(ref)
    assert rel < 0.25


def test_v_rows_option_reads_the_given_values():
    """Given the pool's own dequantized V rows, the V-rows option reproduces
    the plain decode bit for bit; given other rows it uses them (a row of
    zeros everywhere gives a zero output)."""
    T, hkv, hq = 150, 2, 4
    rng = np.random.default_rng(62)
    k = rng.standard_normal((T, hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, hkv, D)).astype(np.float32)
    q = rng.standard_normal((1, hq, D)).astype(np.float32)
    pool = _pool(3, hkv)
    table = np.array([[2, 0, 1]], np.int32)
    slots = table[0, np.arange(T) // 64].astype(np.int64) * 64 + np.arange(T) % 64
    oracle.append(pool, 3, hkv, 0, True, 0, k, v, slots, np.arange(T))
    plain = oracle.decode_attention(pool, 3, hkv, 0, 0, True, q, [T - 1], table, [T], 0.1)
    vh = np.stack([[oracle.dequant_row(*oracle.pool_read_row(pool, 3, hkv, 0, s, g, 1)) for g in range(hkv)]
                   for s in slots]).astype(np.float32)
    same = oracle.decode_attention(pool, 3, hkv, 0, 0, True, q, [T - 1], table, [T], 0.1, v_rows=vh)
    assert np.array_equal(plain, same)
    zero = oracle.decode_attention(pool, 3, hkv, 0, 0, True, q, [T - 1], table, [T], 0.1,
                                   v_rows=np.zeros_like(vh))
    assert not zero.any()
