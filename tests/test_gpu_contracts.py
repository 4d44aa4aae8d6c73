"""GPU checks of the interface contracts around decode attention (release
post of the gzenz/ninfer fork, section "NVFP4 KV cache (from scratch)",
bullets 1-3, and its section "Also included": a workspace reused before the
stream that used it had finished was a use-after-free there):

- masking: slots past a sequence's end on its last page never change the
  output, whatever bytes they hold;
- the split partials mean what the header says: combined in NumPy with the
  pool's global scales they give nvfp4kv_decode_reduce's output;
- a decode queued on a side stream with the binding allocating its
  workspace stays correct while the default stream reuses memory."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_decode import Case, assert_attention_close

pytestmark = pytest.mark.gpu

SM = 1 / np.sqrt(128)


def _token_bytes(t):
    """Byte offsets, inside a 9216-byte block, of everything token t owns:
    its K and V code bytes and its K and V scale bytes (pool layout of the
    C header)."""
    j = np.arange(64)
    k = (t // 16) * 1024 + (j // 16) * 256 + (t % 16) * 16 + j % 16
    v = 4096 + (t // 4) * 256 + (j // 4) * 16 + (t % 4) * 4 + j % 4
    ks = 8192 + 8 * t + np.arange(8)
    vs = 8704 + 8 * t + np.arange(8)
    return np.concatenate([k, v, ks, vs])


def _fill_past_end(c, pattern, rng):
    """Overwrite every slot past the end of each sequence on its last page
    (all kv heads) with `pattern` ("zeros" or "random")."""
    pool = c.pool.data.cpu().numpy().reshape(c.num_pages, c.hkv, 9216)
    for n, T in enumerate(c.lens):
        if T % 64 == 0:
            continue
        page = int(c.table[n, T // 64])
        for t in range(T % 64, 64):
            off = _token_bytes(t)
            for g in range(c.hkv):
                pool[page, g, off] = 0 if pattern == "zeros" else rng.integers(0, 256, off.size, dtype=np.uint8)
    c.pool.data.copy_(torch.from_numpy(pool.reshape(-1)))


def _multi(c, q, pos):
    out = c.kv.nvfp4kv_decode_attn_multi(
        c.pool, 0, q.cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), SM, rope_cos=c.rc, rope_sin=c.rs)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("hq,pps", [(24, 0), (8, 0), (32, 0), (24, 2)])
def test_slots_past_the_end_are_masked_exactly(hq, pps):
    """Two pools equal except for the bytes of the slots past each sequence's
    end (zeros in one, random bytes in the other): decode and multi-query
    outputs are bit-identical."""
    lens = [700, 65, 3, 130, 64 + 63]
    rng = np.random.default_rng(5)
    a = Case(60, lens, 4, hq)
    b = Case(60, lens, 4, hq)
    _fill_past_end(a, "zeros", rng)
    _fill_past_end(b, "random", rng)
    assert not torch.equal(a.pool.data, b.pool.data)
    out_a, out_b = a.gpu(pages_per_split=pps), b.gpu(pages_per_split=pps)
    assert np.array_equal(out_a, out_b)
    assert_attention_close(out_a, a.oracle(), "masked decode")
    m = 3
    q = torch.from_numpy(rng.standard_normal((len(lens), m, hq, 128)).astype(np.float32))
    pos = np.array([[T - m + j for j in range(m)] for T in lens], np.int32)
    assert np.array_equal(_multi(a, q, pos), _multi(b, q, pos))


def _plan_slots(lens, hkv, W):
    """Partial slots of every (sequence, kv head) segment under the split of
    the C header: segment pages plus 5 empty units each, W equal ranges of
    the flat unit list, slot = segment + wavefront for every overlapping
    (segment, wavefront) pair."""
    pages = [(T + 63) // 64 for T in lens]
    TU = sum(hkv * (p + 5) for p in pages)
    slots = {}
    U = 0
    for n, p in enumerate(pages):
        for kvh in range(hkv):
            g = n * hkv + kvh
            S, E = U, U + p
            U += p + 5
            slots[g] = [g + w for w in range(W) if max(w * TU // W, S) < min((w + 1) * TU // W, E)]
    return slots


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (3.7, 0.3)])
def test_split_partials_combine_as_documented(ks, vs):
    """Partials from nvfp4kv_decode_attn_splits (explicit plan: 3 pages per
    wavefront), read from the workspace with the documented layout and
    combined in NumPy as out = v_scale * sum 2^(m - M) acc / sum 2^(m - M) l,
    equal nvfp4kv_decode_reduce's output (to float rounding of the combine)
    and the oracle's attention."""
    lens = [700, 65, 1, 300]
    hkv, hq, pps = 2, 12, 3
    c = Case(70, lens, hkv, hq, k_scale=ks, v_scale=vs)
    kv = c.kv
    group = hq // hkv
    max_pages = (max(lens) + 63) // 64
    W = min(-(-len(lens) * hkv * max_pages // pps), len(lens) * hkv * max_pages)
    n_slots = len(lens) * hkv + W
    need = kv.nvfp4kv_decode_workspace_bytes(c.pool, len(lens), hq, max(lens), pps)
    acc_bytes = n_slots * group * 128 * 4
    ml_off = (acc_bytes + 255) // 256 * 256
    assert need == ml_off + n_slots * group * 8, "workspace size does not follow the documented layout"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    args = (c.pool, 0, c.q.cuda(), torch.from_numpy(c.q_pos).cuda(), torch.from_numpy(c.table).cuda(),
            torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), SM)
    kv.nvfp4kv_decode_attn_splits(*args, ws, rope_cos=c.rc, rope_sin=c.rs, pages_per_split=pps)
    out = torch.empty((len(lens), hq, 128), dtype=torch.float32, device="cuda")
    kv.nvfp4kv_decode_reduce(c.pool, len(lens), hq, args[5], max(lens), out, ws, pages_per_split=pps)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    acc = raw[:acc_bytes].view(np.float32).reshape(n_slots, group, 128).astype(np.float64)
    ml = raw[ml_off:ml_off + n_slots * group * 8].view(np.float32).reshape(n_slots, group, 2).astype(np.float64)
    mine = np.zeros((len(lens), hq, 128))
    for g, sl in _plan_slots(lens, hkv, W).items():
        n, kvh = divmod(g, hkv)
        assert sl, f"segment {g} has no partial"
        m, l, a = ml[sl, :, 0], ml[sl, :, 1], acc[sl]
        assert np.isfinite(m).all() and np.isfinite(l).all() and np.isfinite(a).all()
        M = m.max(0)
        wts = np.exp2(m - M)
        mine[n, kvh * group:(kvh + 1) * group] = vs * (wts[:, :, None] * a).sum(0) / (wts * l).sum(0)[:, None]
    got = out.cpu().numpy()
    assert np.abs(mine - got).max() <= 1e-5 * max(1.0, np.abs(got).max())
    assert_attention_close(mine, c.oracle(), "numpy combine of the partials")


def test_side_stream_decode_with_binding_workspace():
    """Decode queued on a side stream with out and workspace left to the
    binding: meanwhile the default stream allocates and fills memory, which
    must not land on the workspace while the side stream still uses it."""
    c = Case(80, [3000, 1234, 65], 4, 24)
    q, qp = c.q.cuda(), torch.from_numpy(c.q_pos).cuda()
    table, lens = torch.from_numpy(c.table).cuda(), torch.tensor(c.lens, dtype=torch.int32).cuda()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(c.kv.nvfp4kv_decode_attn(c.pool, 0, q, qp, table, lens, max(c.lens), SM,
                                             rope_cos=c.rc, rope_sin=c.rs, stream=side))
        # the binding's workspace of this call is free on the Python side now
        junk = [torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device="cuda") for _ in range(8)]
        del junk
    torch.cuda.synchronize()
    ref = c.oracle()
    for o in outs:
        assert_attention_close(o.cpu().numpy(), ref, "side stream")
