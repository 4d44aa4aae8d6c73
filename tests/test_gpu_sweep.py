"""Seeded random sweep over shapes and flags, each case against the oracle:
append bytes bit for bit, decode and multi-query attention within 2e-3
absolute or 1e-2 relative.  The cases mix kv heads (1-8), query heads per kv
head (1-16), RoPE widths (0-128), the three rotation modes, input dtypes,
split plans, many short sequences and single long ones.

Method: release post of the gzenz/ninfer fork, section "NVFP4 KV cache (from
scratch)"; several query tokens: ai-manual.ru article on "Ninfer 4080",
section "Key features"."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_decode import Case, assert_attention_close

pytestmark = pytest.mark.gpu

ROTARY = [0, 16, 32, 48, 64, 128]


def _draw(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    n_seq = int(rng.choice([1, 2, 5, 17, 64]))
    short = n_seq >= 17
    lens = [int(x) for x in rng.integers(1, 200 if short else 5000, n_seq)]
    return dict(rng=rng, hkv=hkv, hq=hkv * group, lens=lens, rotary=int(rng.choice(ROTARY)),
                hadamard=int(rng.choice([0, 1, 2])), pps=int(rng.choice([0, 0, 1, 2, 7, 64])),
                dtype=torch.bfloat16 if rng.random() < 0.7 else torch.float32,
                pos_scale=float(rng.choice([1.0, 2.3])))


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_case(seed):
    d = _draw(1000 + seed)
    c = Case(2000 + seed, d["lens"], d["hkv"], d["hq"], rotary=d["rotary"], hadamard=d["hadamard"],
             pos_scale=d["pos_scale"], dtype=d["dtype"], hold_last=bool(seed % 2))
    out = c.gpu(pages_per_split=d["pps"], fused=bool(seed % 2))
    what = f"seed {seed}: hkv {d['hkv']} hq {d['hq']} n_seq {len(d['lens'])} rotary {d['rotary']} " \
           f"hadamard {d['hadamard']} pps {d['pps']}"
    assert_attention_close(out, c.oracle(), what)


@pytest.mark.parametrize("seed", range(12))
def test_multi_query_random_case(seed):
    d = _draw(3000 + seed)
    rng = d["rng"]
    hq = d["hkv"] * int(rng.choice([1, 2, 6, 16]))
    lens = [max(int(x), 70) for x in d["lens"][:8]]
    m = int(rng.integers(1, min(min(lens), 20) + 1))
    c = Case(4000 + seed, lens, d["hkv"], hq, rotary=d["rotary"], hadamard=d["hadamard"], dtype=d["dtype"])
    q = torch.from_numpy(rng.standard_normal((len(lens), m, hq, 128)).astype(np.float32)).to(d["dtype"])
    pos = np.array([[T - m + j for j in range(m)] for T in lens], np.int32)
    out = c.kv.nvfp4kv_decode_attn_multi(
        c.pool, 0, q.contiguous().cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), 1 / np.sqrt(128), rope_cos=c.rc,
        rope_sin=c.rs, pages_per_split=d["pps"])
    torch.cuda.synchronize()
    ref = oracle.decode_attention_multi(c.pool.data.cpu().numpy(), c.num_pages, c.hkv, 0, c.rotary, c.hadamard,
                                        q.float().numpy(), pos, c.table, lens, 1 / np.sqrt(128), c.oc, c.os,
                                        signs=c.signs)
    assert_attention_close(out.cpu().numpy(), ref, f"seed {seed}: hkv {d['hkv']} hq {hq} m {m} lens {lens}")


@pytest.mark.parametrize("seed", range(12))
def test_append_random_case(seed):
    import nvfp4_quantized_kv_amd as kv
    d = _draw(5000 + seed)
    rng = d["rng"]
    hkv, rotary, had = d["hkv"], d["rotary"], d["hadamard"]
    num_pages = int(rng.integers(1, 40))
    n_tok = int(rng.integers(1, num_pages * 64 + 1))
    signs = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32) if had == 2 else None
    scale = np.exp(rng.uniform(-6, 6, (n_tok, hkv, 1)))
    k = (rng.standard_normal((n_tok, hkv, 128)) * scale).astype(np.float32)
    v = (rng.standard_normal((n_tok, hkv, 128)) * scale).astype(np.float32)
    kt, vt = torch.from_numpy(k).to(d["dtype"]), torch.from_numpy(v).to(d["dtype"])
    slots = rng.choice(num_pages * 64, n_tok, replace=False).astype(np.int64)
    pos = rng.integers(0, 50000, n_tok).astype(np.int32)
    pool = kv.Pool.allocate(num_pages, 2, hkv, rotary, had,
                            signs=tuple(signs) if signs is not None else (0, 0, 0, 0))
    pool.data.zero_()
    rc = rs = oc = os_ = None
    if rotary:
        c_, s_ = kv.nvfp4kv_rope_table(1e7, rotary, d["pos_scale"], 50000)
        rc, rs = c_.cuda(), s_.cuda()
        oc, os_ = oracle.rope_table(1e7, rotary, d["pos_scale"], 50000)
    kv.nvfp4kv_append(pool, 1, kt.cuda(), vt.cuda(), torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda(),
                      rc, rs)
    torch.cuda.synchronize()
    ref = np.zeros(oracle.pool_bytes(2, num_pages, hkv), np.uint8)
    oracle.append(ref, num_pages, hkv, rotary, had, 1, kt.float().numpy(), vt.float().numpy(), slots, pos,
                  oc, os_, signs=signs)
    got = pool.data.cpu().numpy()
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"seed {seed}: {bad.size} bytes differ (first at {bad[:5]}), hkv {hkv} rotary {rotary} " \
                          f"hadamard {had} n_tok {n_tok}"
