"""GPU parity of the fp16-V pool format: NVFP4 K with V kept in IEEE fp16,
the upstream storage the release post of the gzenz/ninfer fork compares its
NVFP4 V against (section "NVFP4 KV cache (from scratch)", bullet 2), 328
bytes per token per KV head.

Append and in-decode append bytes against the oracle's fp16-V pool, bit for
bit; decode attention against the oracle's fp64 attention on the GPU's own
pool within the decode bar; dequantized fp16 V exact.  The Case pools start
filled with 0x7F bytes, which are NaN as fp16: every slot past a sequence's
end holds NaN V values, so the masking of those slots is exercised on every
case."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_decode import Case, assert_attention_close, oracle_pool

pytestmark = pytest.mark.gpu

SM = 1 / np.sqrt(128)


@pytest.mark.parametrize("dtype,hadamard,scales", [(torch.bfloat16, 1, (1.0, 1.0)), (torch.float32, 2, (1.0, 1.0)),
                                                   (torch.bfloat16, 0, (3.7, 0.3)), (torch.float32, 1, (0.02, 41.0))])
def test_fp16v_append_bytes_match_oracle(dtype, hadamard, scales):
    c = Case(1100, [200, 77, 64, 1], 2, 12, hadamard=hadamard, dtype=dtype, k_scale=scales[0],
             v_scale=scales[1], v_format=1)
    assert c.pool.data.numel() == c.num_pages * 2 * 20992
    assert np.array_equal(c.pool.data.cpu().numpy(), oracle_pool(c))


@pytest.mark.parametrize("lens,hkv,hq,pps", [
    ([257], 1, 2, 0), ([8193], 4, 24, 0), ([1], 2, 12, 0), ([63, 64, 65], 2, 12, 0),
    ([1000, 3, 2049, 777], 2, 4, 0), ([3000, 1234], 4, 24, 1), ([3000, 1234], 4, 32, 4096),
    ([700, 1500], 2, 2, 0), ([5000, 2300], 4, 24, 7)])
def test_fp16v_decode_matches_oracle(lens, hkv, hq, pps):
    c = Case(1200 + sum(lens), lens, hkv, hq, v_format=1, outlier_scale=32.0)
    assert_attention_close(c.gpu(pages_per_split=pps), c.oracle(), f"fp16 V {lens}")


@pytest.mark.parametrize("pps", [0, 1, 4096])
def test_fp16v_decode_quantizes_current_token_in_place(pps):
    """The decode launch writes the new token (K quantized, V in fp16) into
    the cache itself: the whole pool then equals the oracle's, and the
    attention equals append + decode and the oracle's."""
    lens = [1000, 64, 65, 3]
    full = Case(1300, lens, 2, 12, v_format=1, k_scale=2.5, v_scale=0.75)
    held = Case(1300, lens, 2, 12, v_format=1, k_scale=2.5, v_scale=0.75, hold_last=True)
    out_full = full.gpu(pages_per_split=pps)
    out_fused = held.gpu(pages_per_split=pps, fused=True)
    assert np.array_equal(held.pool.data.cpu().numpy(), oracle_pool(held))
    assert torch.equal(held.pool.data, full.pool.data)
    assert np.array_equal(out_fused, out_full)
    assert_attention_close(out_fused, held.oracle(), "fp16 V fused")


def test_fp16v_dequant_is_exact():
    c = Case(1400, [130, 64], 2, 4, v_format=1, v_scale=3.0)
    T = sum(c.lens)
    slots = np.concatenate([c.table[n, np.arange(L) // 64].astype(np.int64) * 64 + np.arange(L) % 64
                            for n, L in enumerate(c.lens)])
    kh, vh = c.kv.nvfp4kv_dequant(c.pool, 0, torch.from_numpy(slots).cuda(), torch.float32)
    kb, vb = c.kv.nvfp4kv_dequant(c.pool, 0, torch.from_numpy(slots).cuda(), torch.bfloat16)
    torch.cuda.synchronize()
    pool = c.pool.data.cpu().numpy()
    vh, kh, vb = vh.cpu().numpy(), kh.cpu().numpy(), vb.float().cpu().numpy()
    for i in range(0, T, 5):
        for g in range(c.hkv):
            bits = oracle.pool_read_v16(pool, c.num_pages, c.hkv, 0, int(slots[i]), g)
            want = bits.view(np.float16).astype(np.float32) * np.float32(3.0)
            assert np.array_equal(vh[i, g], want)
            want_bf16 = torch.from_numpy(want).to(torch.bfloat16).float().numpy()   # nearest, ties to even
            assert np.array_equal(vb[i, g], want_bf16)
            codes, scales = oracle.pool_read_row(pool, c.num_pages, c.hkv, 0, int(slots[i]), g, 0, v_format=1)
            assert np.array_equal(kh[i, g], oracle.dequant_row(codes, scales).astype(np.float32))


def test_fp16v_static_entry_point_and_spill_round_trip():
    c = Case(1500, [700, 130], 2, 12, v_format=1)
    kv = c.kv
    out = torch.empty((2, 12, 128), dtype=torch.float32, device="cuda")
    kv.nvfp4kv_decode_attn_static(c.pool, 0, c.q.cuda(), torch.from_numpy(c.q_pos).cuda(),
                                  torch.from_numpy(c.table).cuda(), torch.tensor(c.lens, dtype=torch.int32).cuda(),
                                  max(c.lens), SM, out, rope_cos=c.rc, rope_sin=c.rs)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), c.oracle(), "fp16 V static workspace")
    ids = torch.from_numpy(c.table[0, :5].copy()).cuda()
    assert kv.nvfp4kv_page_bytes(c.pool) == 2 * 20992
    arena = kv.nvfp4kv_spill_pages(c.pool, ids)
    torch.cuda.synchronize()
    want = oracle.spill_pages(c.pool.data.cpu().numpy(), 1, c.num_pages, c.hkv, c.table[0, :5], v_format=1)
    assert np.array_equal(arena.numpy(), want)


def test_fp16v_refuses_what_it_does_not_cover():
    import nvfp4_quantized_kv_amd as kv
    c = Case(1600, [300], 1, 16, v_format=1)
    with pytest.raises(kv.NVFP4KVError) as e:
        c.gpu()
    assert e.value.code == kv.ERR_UNSUPPORTED
    c2 = Case(1601, [300], 2, 4, v_format=1)
    q = torch.zeros((1, 2, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kv.NVFP4KVError) as e:
        kv.nvfp4kv_decode_attn_multi(c2.pool, 0, q, torch.tensor([[298, 299]], dtype=torch.int32).cuda(),
                                     torch.from_numpy(c2.table).cuda(), torch.tensor([300], dtype=torch.int32).cuda(),
                                     300, SM, rope_cos=c2.rc, rope_sin=c2.rs)
    assert e.value.code == kv.ERR_UNSUPPORTED
