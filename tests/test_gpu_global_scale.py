"""GPU parity with per-tensor global scales on the pool (NVFP4's second
scaling level, one FP32 factor per tensor over the E4M3 block scales;
NVIDIA's NVFP4 format description): append and in-decode append bytes and
dequantized values bit-exact against the oracle, attention within the decode
bar."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_decode import Case, assert_attention_close

pytestmark = pytest.mark.gpu

SCALES = [(3.7, 0.3), (0.02, 41.0)]


def _oracle_pool(c, upto_last=True):
    """The pool bytes the oracle writes for the Case's appends."""
    pool = np.full(c.pool.data.numel(), 0x7F, np.uint8)
    for n, T in enumerate(c.lens):
        pos = np.arange(T if upto_last else T - 1)
        if len(pos) == 0:
            continue
        sl = c.table[n, pos // 64].astype(np.int64) * 64 + pos % 64
        oracle.append(pool, c.num_pages, c.hkv, c.rotary, c.hadamard, 0, c.k[n][:len(pos)].float().numpy(),
                      c.v[n][:len(pos)].float().numpy(), sl, pos.astype(np.int32), c.oc, c.os, signs=c.signs,
                      k_scale=c.k_scale, v_scale=c.v_scale)
    return pool


@pytest.mark.parametrize("ks,vs", SCALES)
@pytest.mark.parametrize("dtype,hadamard", [(torch.bfloat16, 1), (torch.float32, 2), (torch.bfloat16, 0)])
def test_append_bytes_and_dequant_with_global_scales(ks, vs, dtype, hadamard):
    c = Case(900, [200, 77], 2, 12, hadamard=hadamard, dtype=dtype, k_scale=ks, v_scale=vs)
    got = c.pool.data.cpu().numpy()
    assert np.array_equal(got, _oracle_pool(c))
    slots = torch.from_numpy(np.concatenate([c.table[n, np.arange(T) // 64].astype(np.int64) * 64 + np.arange(T) % 64
                                             for n, T in enumerate(c.lens)])).cuda()
    kh, vh = c.kv.nvfp4kv_dequant(c.pool, 0, slots, torch.float32)
    torch.cuda.synchronize()
    kh, vh = kh.cpu().numpy(), vh.cpu().numpy()
    for i, s in enumerate(slots.cpu().numpy()[:: 7]):
        for h in range(c.hkv):
            for which, g, out in ((0, ks, kh), (1, vs, vh)):
                codes, scales = oracle.pool_read_row(got, c.num_pages, c.hkv, 0, int(s), h, which)
                want = oracle.dequant_row(codes, scales).astype(np.float32) * np.float32(g)
                assert np.array_equal(out[7 * i, h], want), (i, h, which)


@pytest.mark.parametrize("ks,vs", SCALES)
def test_decode_with_global_scales(ks, vs):
    c = Case(910, [3000, 1234, 65], 4, 24, k_scale=ks, v_scale=vs)
    assert_attention_close(c.gpu(), c.oracle(), f"scales {ks} {vs}")


@pytest.mark.parametrize("ks,vs", SCALES)
def test_fused_new_token_with_global_scales(ks, vs):
    c = Case(920, [700, 64, 129], 4, 24, hold_last=True, k_scale=ks, v_scale=vs)
    out = c.gpu(fused=True)
    assert np.array_equal(c.pool.data.cpu().numpy(), _oracle_pool(c))
    assert_attention_close(out, c.oracle(), f"fused scales {ks} {vs}")


def test_multi_query_with_global_scales():
    c = Case(930, [3000, 1234], 4, 24, k_scale=5.5, v_scale=0.125)
    m = 4
    q = torch.from_numpy(np.random.default_rng(931).standard_normal((2, m, 24, 128)).astype(np.float32))
    pos = np.array([[T - m + j for j in range(m)] for T in c.lens], np.int32)
    out = c.kv.nvfp4kv_decode_attn_multi(
        c.pool, 0, q.cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), 1 / np.sqrt(128), rope_cos=c.rc,
        rope_sin=c.rs)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_multi(c.pool.data.cpu().numpy(), c.num_pages, c.hkv, 0, c.rotary, c.hadamard,
                                        q.numpy(), pos, c.table, c.lens, 1 / np.sqrt(128), c.oc, c.os,
                                        signs=c.signs, k_scale=5.5, v_scale=0.125)
    assert_attention_close(out.cpu().numpy(), ref, "multi with scales")
