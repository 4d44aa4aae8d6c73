"""GPU parity of nvfp4kv_decode_attn_multi (several new query tokens per
sequence, causal among them) against the CPU oracle's
decode_attention_multi on the GPU's own pool bytes.  Bar: every element within
2e-3 absolute or 1e-2 relative, relative L2 error at most 1e-2.

The decode step of speculative verification: ai-manual.ru article on
"Ninfer 4080", section "Key features" (a draft model proposes K tokens, the
main model checks them in one step)."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_decode import Case, assert_attention_close

pytestmark = pytest.mark.gpu


def _queries(c, m, seed, dtype):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((len(c.lens), m, c.hq, 128)).astype(np.float32)).to(dtype)
    pos = np.array([[T - m + j for j in range(m)] for T in c.lens], np.int32)
    return q, pos


def _run(c, q, pos, pages_per_split=0):
    out = c.kv.nvfp4kv_decode_attn_multi(
        c.pool, 0, q.contiguous().cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), 1 / np.sqrt(128),
        rope_cos=c.rc, rope_sin=c.rs, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(c, q, pos):
    return oracle.decode_attention_multi(c.pool.data.cpu().numpy(), c.num_pages, c.hkv, 0, c.rotary, c.hadamard,
                                         q.float().numpy(), pos, c.table, c.lens, 1 / np.sqrt(128), c.oc, c.os,
                                         signs=c.signs)


MULTI_CASES = [
    # (lens, hkv, hq, m, rotary).  A launch takes floor(48 / heads) tokens,
    # every query head of a kv head per token: columns in tiles of 16 (one
    # to three per wavefront), packed weights at 8 columns or fewer.
    ([3000, 1234], 4, 24, 2, 32),      # 6 heads: 12 columns, one tile
    ([3000, 1234], 4, 24, 7, 32),      # 42 columns, three tiles, the last partial
    ([700, 65, 8], 4, 24, 8, 32),      # 48 columns; a sequence of exactly 8 tokens: token 0 sees one
    ([129, 4100], 2, 2, 16, 16),       # 1 head: 16 tokens, one tile
    ([513, 70], 2, 2, 5, 0),           # no RoPE; 5 columns, packed
    ([2000, 64 + 3], 2, 4, 4, 32),     # 2 heads: 8 columns, packed; a page edge inside the tail
    ([1500], 1, 8, 2, 128),            # 8 heads: 16 columns; full-width RoPE
    ([900, 300], 1, 16, 3, 32),        # 16 heads: 48 columns in one launch
    ([3000, 1234], 4, 24, 10, 32),     # launches of 8 tokens (three tiles) and 2 tokens (one tile)
    ([2500, 90], 2, 2, 40, 32),        # 1 head: 40 tokens, three tiles; causal cut over a page
    ([777, 1300], 2, 8, 5, 32),        # 4 heads: 20 columns, two tiles
    ([5000, 64], 1, 1, 64, 32),        # 64 tokens: launches of 48 and 16; a 64-token sequence
    ([1300, 90], 4, 24, 8, 24),        # RoPE width not a multiple of 16 (per-token query positions)
]

@pytest.mark.parametrize("idx", range(len(MULTI_CASES)))
def test_multi_query_matches_oracle(idx):
    lens, hkv, hq, m, rotary = MULTI_CASES[idx]
    c = Case(600 + idx, lens, hkv, hq, rotary=rotary)
    q, pos = _queries(c, m, 700 + idx, torch.bfloat16)
    assert_attention_close(_run(c, q, pos), _oracle(c, q, pos), f"multi {MULTI_CASES[idx]}")


@pytest.mark.parametrize("pages_per_split", [1, 3, 4096])
def test_multi_query_split_plans(pages_per_split):
    """Ranges that end inside the last tokens (1 page per wavefront), odd
    ranges, and one wavefront for everything."""
    c = Case(620, [1000, 3, 2049, 777], 2, 12, rotary=32)
    q, pos = _queries(c, 3, 720, torch.float32)
    assert_attention_close(_run(c, q, pos, pages_per_split), _oracle(c, q, pos), f"pps {pages_per_split}")


@pytest.mark.parametrize("m", [3, 8])
def test_multi_query_ignores_unwritten_workspace(m):
    """Short sequences, far more wavefronts than pages, and a workspace full of
    NaN bytes: slots of wavefronts with empty ranges are never written and
    must not reach the output (one and three column tiles)."""
    c = Case(650 + m, [700, 65, 8], 4, 24, rotary=32)
    q, pos = _queries(c, m, 750 + m, torch.bfloat16)
    need = c.kv.nvfp4kv_decode_multi_workspace_bytes(c.pool, len(c.lens), m, c.hq, max(c.lens), 0)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = c.kv.nvfp4kv_decode_attn_multi(
        c.pool, 0, q.contiguous().cuda(), torch.from_numpy(pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), 1 / np.sqrt(128), workspace=ws,
        rope_cos=c.rc, rope_sin=c.rs)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), _oracle(c, q, pos), f"NaN-filled workspace, m {m}")


def test_multi_query_one_token_is_decode():
    """n_qtok = 1 runs the plain decode kernel: same output as
    nvfp4kv_decode_attn without k_new/v_new, bit for bit."""
    c = Case(630, [5000, 2300], 4, 24)
    q, pos = _queries(c, 1, 730, torch.bfloat16)
    multi = _run(c, q, pos)[:, 0]
    single = c.kv.nvfp4kv_decode_attn(
        c.pool, 0, q[:, 0].contiguous().cuda(), torch.from_numpy(pos[:, 0].copy()).cuda(),
        torch.from_numpy(c.table).cuda(), torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens),
        1 / np.sqrt(128), rope_cos=c.rc, rope_sin=c.rs).cpu().numpy()
    assert np.array_equal(multi, single)


def test_multi_query_last_token_equals_decode_of_full_sequence():
    """The last query token sees the whole sequence: its output equals a
    one-token decode of that token's query (up to summation order)."""
    c = Case(640, [4097, 333], 4, 24)
    q, pos = _queries(c, 4, 740, torch.bfloat16)
    multi = _run(c, q, pos)[:, 3]
    single = c.kv.nvfp4kv_decode_attn(
        c.pool, 0, q[:, 3].contiguous().cuda(), torch.from_numpy(pos[:, 3].copy()).cuda(),
        torch.from_numpy(c.table).cuda(), torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens),
        1 / np.sqrt(128), rope_cos=c.rc, rope_sin=c.rs).cpu().numpy()
    assert np.abs(multi - single).max() <= 1e-5 * max(1.0, np.abs(single).max())
