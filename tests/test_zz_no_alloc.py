"""The allocation-free decode entry point (nvfp4kv_decode_attn_static, for
callers that cannot allocate device memory) against nvfp4kv_decode_attn with
a caller-allocated workspace: the same kernels and split plan, so the outputs
must be identical, and within the oracle's bar.  Two calls in a row on the
library's static workspace, the second with a smaller input (the array keeps
the first call's partials), then a call that reads the new token from
k_new/v_new."""
import numpy as np
import pytest
import torch

from test_gpu_decode import Case, assert_attention_close

pytestmark = pytest.mark.gpu

SM = 1 / np.sqrt(128)


def _both(c, fused=False, pps=0):
    kv = c.kv
    args = (c.pool, 0, c.q.cuda(), torch.from_numpy(c.q_pos).cuda(), torch.from_numpy(c.table).cuda(),
            torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), SM)
    k_new = v_new = None
    if fused:
        k_new, v_new = (x.cuda() for x in c.new_token_rows())
    out_static = torch.full((len(c.lens), c.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    pool_before = c.pool.data.clone()
    kv.nvfp4kv_decode_attn_static(*args, out_static, rope_cos=c.rc, rope_sin=c.rs, pages_per_split=pps,
                                  k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    pool_static = c.pool.data.clone()
    c.pool.data.copy_(pool_before)
    out_ws = kv.nvfp4kv_decode_attn(*args, rope_cos=c.rc, rope_sin=c.rs, pages_per_split=pps,
                                    k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert torch.equal(pool_static, c.pool.data), "pool bytes differ between the two entry points"
    return out_static.cpu().numpy(), out_ws.cpu().numpy()


def test_static_workspace_matches_caller_workspace_two_calls():
    big = Case(500, [3000, 1234, 65, 700], 4, 24)
    a, b = _both(big)
    assert np.array_equal(a, b)
    assert_attention_close(a, big.oracle(), "static workspace, first call")
    small = Case(501, [300], 2, 8)
    a, b = _both(small)
    assert np.array_equal(a, b)
    assert_attention_close(a, small.oracle(), "static workspace, second (smaller) call")


def test_static_workspace_in_decode_append_and_explicit_split():
    c = Case(502, [1000, 130, 64], 2, 12, hold_last=True)
    a, b = _both(c, fused=True, pps=3)
    assert np.array_equal(a, b)
    assert_attention_close(a, c.oracle(), "static workspace with the new token")


def test_static_workspace_refuses_oversized_plans():
    """A plan whose partials do not fit the static array is refused before
    anything runs, with the reason; nothing is written."""
    import nvfp4_quantized_kv_amd as kv
    c = Case(503, [70], 1, 16)
    n_seq = 4000
    lens = torch.full((n_seq,), 70, dtype=torch.int32, device="cuda")
    table = torch.from_numpy(np.tile(c.table, (n_seq, 1))).cuda()
    q = torch.zeros((n_seq, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((n_seq, 16, 128), 7.0, dtype=torch.float32, device="cuda")
    need = kv.nvfp4kv_decode_workspace_bytes(c.pool, n_seq, 16, 70, 1)
    assert need > kv.STATIC_WORKSPACE_BYTES
    with pytest.raises(kv.NVFP4KVError) as e:
        kv.nvfp4kv_decode_attn_static(c.pool, 0, q, torch.zeros(n_seq, dtype=torch.int32, device="cuda"), table,
                                      lens, 70, SM, out, rope_cos=c.rc, rope_sin=c.rs, pages_per_split=1)
    assert e.value.code == kv.ERR_WORKSPACE and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
