"""GPU parity of nvfp4kv_append and nvfp4kv_dequant against the CPU oracle:
packed codes and scales must match bit for bit, dequantized values exactly.

Method: release post of the gzenz/ninfer fork, section "NVFP4 KV cache (from
scratch)", bullets 1-4."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _kv():
    import nvfp4_quantized_kv_amd as kv
    return kv


def _run_append(num_pages, hkv, rotary, hadamard, k, v, slots, pos, pos_scale=1.0, layers=1, layer=0):
    """Append on the GPU and with the oracle; return (gpu_pool_bytes, oracle_pool_bytes)."""
    kv = _kv()
    pool = kv.Pool.allocate(num_pages, layers, hkv, rotary, hadamard)
    pool.data.zero_()
    max_pos = int(np.max(pos)) + 1
    rc = rs = None
    oc = os_ = None
    if rotary:
        c, s = kv.nvfp4kv_rope_table(1e7, rotary, pos_scale, max_pos)
        rc, rs = c.cuda(), s.cuda()
        oc, os_ = oracle.rope_table(1e7, rotary, pos_scale, max_pos)
    kt = torch.from_numpy(np.ascontiguousarray(k)).cuda()
    vt = torch.from_numpy(np.ascontiguousarray(v)).cuda()
    if kt.dtype == torch.float32 and k.dtype != np.float32:
        raise AssertionError
    kv.nvfp4kv_append(pool, layer, kt, vt, torch.from_numpy(np.asarray(slots, np.int64)).cuda(),
                      torch.from_numpy(np.asarray(pos, np.int32)).cuda(), rc, rs)
    torch.cuda.synchronize()
    gpu = pool.data.cpu().numpy()
    ref = np.zeros(oracle.pool_bytes(layers, num_pages, hkv), np.uint8)
    oracle.append(ref, num_pages, hkv, rotary, hadamard, layer, k.astype(np.float32),
                  v.astype(np.float32), slots, pos, oc, os_)
    return gpu, ref


def _assert_same_bytes(gpu, ref):
    bad = np.nonzero(gpu != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}: gpu {gpu[bad[:8]].tolist()} oracle {ref[bad[:8]].tolist()}"


def test_append_tiny_workload_bitexact():
    """1 kv head, 256 cached + 1 appended fp32 tokens, 4 outlier channels x20,
    Hadamard on K, no RoPE."""
    from nvfp4_quantized_kv_amd import workloads as W
    wl = W.config("tiny")
    T = wl.cached[0] + 1
    k = W.rows(wl, "k", 0, 0, T, wl.hkv).numpy()
    v = W.rows(wl, "v", 0, 0, T, wl.hkv).numpy()
    table, num_pages = W.page_table(wl)
    pos = np.arange(T)
    gpu, ref = _run_append(num_pages, wl.hkv, 0, True, k, v, W.slots(table, 0, pos), pos)
    _assert_same_bytes(gpu, ref)


def test_append_layer8k_bitexact():
    """One 8K-token layer: 4 kv heads, bf16 with 3 outlier channels x16, RoPE
    on 32 dims (theta 1e7), randomly permuted pages."""
    from nvfp4_quantized_kv_amd import workloads as W
    wl = W.config("layer8k")
    T = wl.cached[0] + 1
    k = W.rows(wl, "k", 0, 0, T, wl.hkv)
    v = W.rows(wl, "v", 0, 0, T, wl.hkv)
    table, num_pages = W.page_table(wl)
    pos = np.arange(T)
    kv = _kv()
    pool = kv.Pool.allocate(num_pages, 1, wl.hkv, wl.rotary_dim, True)
    pool.data.zero_()
    c, s = kv.nvfp4kv_rope_table(wl.theta, wl.rotary_dim, 1.0, T)
    kv.nvfp4kv_append(pool, 0, k.cuda(), v.cuda(), torch.from_numpy(W.slots(table, 0, pos)).cuda(),
                      torch.from_numpy(pos.astype(np.int32)).cuda(), c.cuda(), s.cuda())
    torch.cuda.synchronize()
    ref = np.zeros(oracle.pool_bytes(1, num_pages, wl.hkv), np.uint8)
    oc, os_ = oracle.rope_table(wl.theta, wl.rotary_dim, 1.0, T)
    oracle.append(ref, num_pages, wl.hkv, wl.rotary_dim, True, 0, k.float().numpy(), v.float().numpy(),
                  W.slots(table, 0, pos), pos, oc, os_)
    _assert_same_bytes(pool.data.cpu().numpy(), ref)


@pytest.mark.parametrize("rotary,hadamard,dtype", [
    (0, False, np.float32), (16, True, np.float32), (32, True, "bf16"), (64, False, "bf16"),
    (128, True, np.float32), (48, True, np.float32), (112, True, "bf16"), (32, 2, "bf16"), (0, 2, np.float32),
    # even widths that are not multiples of 16 (pairs split across lanes at every in-lane offset)
    (2, True, np.float32), (8, True, "bf16"), (14, False, np.float32), (24, True, "bf16"), (40, True, np.float32),
    (50, 2, "bf16"), (86, True, np.float32), (126, True, "bf16"), (6, True, np.float32), (108, False, "bf16")])
def test_append_shapes_and_flags_bitexact(rotary, hadamard, dtype):
    """hadamard 2: the randomized rotation, with a drawn element mask."""
    rng = np.random.default_rng(rotary * 7 + int(hadamard))
    signs = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32) if hadamard == 2 else None
    hkv, n_tok, num_pages = 3, 150, 9
    k = rng.standard_normal((n_tok, hkv, 128)).astype(np.float32) * np.exp(rng.uniform(-4, 4, (n_tok, hkv, 1)))
    v = rng.standard_normal((n_tok, hkv, 128)).astype(np.float32) * np.exp(rng.uniform(-4, 4, (n_tok, hkv, 1)))
    k = k.astype(np.float32)
    v = v.astype(np.float32)
    if dtype == "bf16":
        k = torch.from_numpy(k).bfloat16().float().numpy()
        v = torch.from_numpy(v).bfloat16().float().numpy()
    slots = rng.choice(num_pages * 64, size=n_tok, replace=False)
    pos = rng.integers(0, 100000, size=n_tok)
    kv = _kv()
    pool = kv.Pool.allocate(num_pages, 2, hkv, rotary, hadamard,
                            signs=tuple(signs) if signs is not None else (0, 0, 0, 0))
    pool.data.zero_()
    rc = rs = oc = os_ = None
    if rotary:
        c, s = kv.nvfp4kv_rope_table(1e7, rotary, 1.0, 100000)
        rc, rs = c.cuda(), s.cuda()
        oc, os_ = oracle.rope_table(1e7, rotary, 1.0, 100000)
    kt = torch.from_numpy(k)
    vt = torch.from_numpy(v)
    if dtype == "bf16":
        kt, vt = kt.bfloat16(), vt.bfloat16()
    kv.nvfp4kv_append(pool, 1, kt.cuda(), vt.cuda(), torch.from_numpy(slots.astype(np.int64)).cuda(),
                      torch.from_numpy(pos.astype(np.int32)).cuda(), rc, rs)
    torch.cuda.synchronize()
    ref = np.zeros(oracle.pool_bytes(2, num_pages, hkv), np.uint8)
    oracle.append(ref, num_pages, hkv, rotary, hadamard, 1, k, v, slots, pos, oc, os_, signs=signs)
    _assert_same_bytes(pool.data.cpu().numpy(), ref)


def test_append_edge_values_bitexact():
    """Zero rows, rows too small for any non-zero scale, rows past the E4M3
    range, signed zeros, and rows built on exact rounding ties."""
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.zeros(128))
    rows.append(-np.zeros(128))
    rows.append(rng.standard_normal(128) * 1e-4)          # amax/6 below 2^-10: zero scale
    rows.append(rng.standard_normal(128) * 1e-3)          # E4M3 subnormal scales
    rows.append(rng.standard_normal(128) * 1e4)           # saturated scale 448
    rows.append(rng.standard_normal(128) * 1e35)          # large, transform still finite
    # exact ties: block scale s = 1 (amax 6), elements at the E2M1 decision points
    tie = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, 0])
    rows.append(np.tile(tie, 8))
    # amax/6 exactly on E4M3 midpoints
    mids = []
    for c in (3, 8, 40, 100, 120):
        mids.append(3 * (oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)))
    r = rng.uniform(-1, 1, 128)
    for b, m in enumerate(mids + mids[:3]):
        r[16 * b] = m
        r[16 * b + 1:16 * b + 16] *= m / 2
    rows.append(r)
    rows.append(rng.standard_normal(128))
    x = np.stack(rows).astype(np.float32)
    n = x.shape[0]
    k = x[:, None, :]
    v = x[::-1].copy()[:, None, :]
    for hadamard in (False, True):
        gpu, ref = _run_append(1, 1, 0, hadamard, k, v, np.arange(n), np.zeros(n))
        _assert_same_bytes(gpu, ref)


def test_append_overwrites_in_place():
    """A second append to the same slots replaces the first (the decode-time
    append writes the current token in place)."""
    rng = np.random.default_rng(5)
    kv = _kv()
    pool = kv.Pool.allocate(2, 1, 2, 32, True)
    pool.data.zero_()
    c, s = kv.nvfp4kv_rope_table(1e7, 32, 1.0, 200)
    slots = torch.tensor([3, 70, 127], dtype=torch.int64).cuda()
    pos = torch.tensor([3, 70, 127], dtype=torch.int32).cuda()
    for trial in range(2):
        k = rng.standard_normal((3, 2, 128)).astype(np.float32)
        v = rng.standard_normal((3, 2, 128)).astype(np.float32)
        kv.nvfp4kv_append(pool, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), slots, pos, c.cuda(), s.cuda())
    torch.cuda.synchronize()
    ref = np.zeros(oracle.pool_bytes(1, 2, 2), np.uint8)
    oc, os_ = oracle.rope_table(1e7, 32, 1.0, 200)
    oracle.append(ref, 2, 2, 32, True, 0, k, v, slots.cpu().numpy(), pos.cpu().numpy(), oc, os_)
    _assert_same_bytes(pool.data.cpu().numpy(), ref)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequant_exact(out_dtype):
    rng = np.random.default_rng(9)
    hkv, n_tok, num_pages = 2, 200, 5
    k = (rng.standard_normal((n_tok, hkv, 128)) * 3).astype(np.float32)
    v = (rng.standard_normal((n_tok, hkv, 128)) * 3).astype(np.float32)
    slots = rng.choice(num_pages * 64, size=n_tok, replace=False).astype(np.int64)
    kv = _kv()
    pool = kv.Pool.allocate(num_pages, 1, hkv, 0, True)
    pool.data.zero_()
    st = torch.from_numpy(slots).cuda()
    kv.nvfp4kv_append(pool, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), st,
                      torch.zeros(n_tok, dtype=torch.int32).cuda())
    kh, vh = kv.nvfp4kv_dequant(pool, 0, st, out_dtype)
    kh2, _ = kv.nvfp4kv_dequant(pool, 0, st, torch.float32, unrotate=True, want_v=False)
    torch.cuda.synchronize()
    pb = pool.data.cpu().numpy()
    kh, vh, kh2 = kh.float().cpu().numpy(), vh.float().cpu().numpy(), kh2.cpu().numpy()
    for i in range(n_tok):
        for g in range(hkv):
            kref = oracle.dequant_row(*oracle.pool_read_row(pb, num_pages, hkv, 0, slots[i], g, 0))
            vref = oracle.dequant_row(*oracle.pool_read_row(pb, num_pages, hkv, 0, slots[i], g, 1))
            assert (kh[i, g] == kref).all() and (vh[i, g] == vref).all()
            # un-rotated K-hat is the quantized K back in the input domain
            assert np.linalg.norm(kh2[i, g] - k[i, g]) <= 0.2 * np.linalg.norm(k[i, g])


def test_dequant_unrotates_the_randomized_rotation():
    """With the randomized rotation, un-rotating applies the transform again
    and then the element negations: K-hat back in the input domain, which
    must equal the oracle's dequantized row pushed through H then D in fp64
    (to float rounding) and stay near the input row."""
    rng = np.random.default_rng(19)
    hkv, n_tok, num_pages = 2, 64, 2
    signs = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
    k = (rng.standard_normal((n_tok, hkv, 128)) * 3).astype(np.float32)
    v = (rng.standard_normal((n_tok, hkv, 128)) * 3).astype(np.float32)
    slots = rng.choice(num_pages * 64, size=n_tok, replace=False).astype(np.int64)
    kv = _kv()
    pool = kv.Pool.allocate(num_pages, 1, hkv, 0, 2, signs=tuple(signs))
    pool.data.zero_()
    st = torch.from_numpy(slots).cuda()
    kv.nvfp4kv_append(pool, 0, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), st,
                      torch.zeros(n_tok, dtype=torch.int32).cuda())
    kh, _ = kv.nvfp4kv_dequant(pool, 0, st, torch.float32, unrotate=True, want_v=False)
    torch.cuda.synchronize()
    pb = pool.data.cpu().numpy()
    kh = kh.cpu().numpy()
    idx = np.arange(128)
    H = np.where(np.array([[bin(i & j).count("1") % 2 for j in idx] for i in idx]) == 1, -1.0, 1.0) / np.sqrt(128)
    d = np.array([-1.0 if (int(signs[j // 32]) >> (j % 32)) & 1 else 1.0 for j in idx])
    for i in range(n_tok):
        for g in range(hkv):
            rot = oracle.dequant_row(*oracle.pool_read_row(pb, num_pages, hkv, 0, slots[i], g, 0))
            want = d * (H @ rot)
            assert np.abs(kh[i, g] - want).max() <= 1e-5 * max(1.0, np.abs(want).max())
            assert np.linalg.norm(kh[i, g] - k[i, g]) <= 0.2 * np.linalg.norm(k[i, g])
