"""GPU parity of nvfp4kv_decode_attn against the CPU oracle.

The oracle computes fp64 attention on the GPU's own pool bytes (the same
dequantized cache) with its own query quantization.  Bar: every element
within 2e-3 absolute or 1e-2 relative, and relative L2 error at most 1e-2.

Method: release post of the gzenz/ninfer fork, section "NVFP4 KV cache (from
scratch)", bullets 1-3."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ABS_TOL, REL_TOL = 2e-3, 1e-2


def assert_attention_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(gpu).all(), what
    err = np.abs(gpu - ref)
    ok = (err <= ABS_TOL) | (err <= REL_TOL * np.abs(ref))
    if not ok.all():
        i = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} elements out of tolerance, worst at {i}: "
                             f"gpu {gpu[i]} oracle {ref[i]} (max abs err {err.max():.3g})")
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_TOL, f"{what}: relative L2 error {rel}"


class Case:
    """A small paged cache filled on the GPU, plus queries."""

    def __init__(self, seed, lens, hkv, hq, rotary=32, hadamard=True, pos_scale=1.0,
                 dtype=torch.bfloat16, outliers=3, outlier_scale=16.0, extra_pages=3,
                 student_t=False, hold_last=False, k_scale=1.0, v_scale=1.0, v_format=0):
        import nvfp4_quantized_kv_amd as kv
        self.kv = kv
        rng = np.random.default_rng(seed)
        self.lens = list(lens)
        self.hkv, self.hq, self.rotary, self.hadamard = hkv, hq, rotary, int(hadamard)
        self.k_scale, self.v_scale = k_scale, v_scale
        self.v_format = v_format
        # hadamard 2: the randomized rotation's element mask, drawn here
        self.signs = (rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
                      if self.hadamard == 2 else None)
        pages = [(t + 63) // 64 for t in lens]
        self.num_pages = sum(pages) + extra_pages
        perm = rng.permutation(self.num_pages).astype(np.int32)
        width = max(pages)
        self.table = np.zeros((len(lens), width), np.int32)
        at = 0
        for n, p in enumerate(pages):
            self.table[n, :p] = perm[at:at + p]
            at += p
        mult = np.ones(128, np.float32)
        if outliers:
            mult[rng.choice(128, outliers, replace=False)] = outlier_scale

        def draw(*shape):
            x = rng.standard_normal(shape)
            if student_t:
                x = x / np.sqrt((rng.standard_normal((3,) + shape) ** 2).sum(0) / 3)
            x = (x * mult).astype(np.float32)
            return torch.from_numpy(x).to(dtype)

        self.max_pos = max(lens) + 1
        self.pool = kv.Pool.allocate(self.num_pages, 1, hkv, rotary, hadamard,
                                     signs=tuple(self.signs) if self.signs is not None else (0, 0, 0, 0),
                                     k_scale=k_scale, v_scale=v_scale, v_format=v_format)
        # stale bytes: 0x7F in every byte never written.  The decode kernels
        # clear scale sign bits, so these read as finite values (scale 1.875,
        # codes +-6): a masking mistake shows as an error, not as NaN
        # (test_gpu_contracts.py pins the masking exactly)
        self.pool.data.fill_(0x7F)
        self.rc = self.rs = self.oc = self.os = None
        if rotary:
            c, s = kv.nvfp4kv_rope_table(1e7, rotary, pos_scale, self.max_pos)
            self.rc, self.rs = c.cuda(), s.cuda()
            self.oc, self.os = oracle.rope_table(1e7, rotary, pos_scale, self.max_pos)
        self.k, self.v = [], []
        for n, T in enumerate(lens):
            k, v = draw(T, hkv, 128), draw(T, hkv, 128)
            self.k.append(k)
            self.v.append(v)
            # hold_last: the current token (the last) is left for the decode
            # call to quantize into the cache itself
            pos = np.arange(T - 1 if hold_last else T)
            if len(pos) == 0:
                continue
            sl = self.table[n, pos // 64].astype(np.int64) * 64 + pos % 64
            kv.nvfp4kv_append(self.pool, 0, k[:len(pos)].contiguous().cuda(), v[:len(pos)].contiguous().cuda(),
                              torch.from_numpy(sl).cuda(), torch.from_numpy(pos.astype(np.int32)).cuda(),
                              self.rc, self.rs)
        self.q = draw(len(lens), hq, 128)
        self.q_pos = np.array([T - 1 for T in lens], np.int32)

    def new_token_rows(self):
        """The current token's K and V, [n_seq][hkv][128]."""
        k = torch.stack([x[-1] for x in self.k]).contiguous()
        v = torch.stack([x[-1] for x in self.v]).contiguous()
        return k, v

    def gpu(self, pages_per_split=0, sm_scale=1 / np.sqrt(128), fused=False):
        k_new = v_new = None
        if fused:
            k_new, v_new = (x.cuda() for x in self.new_token_rows())
        out = self.kv.nvfp4kv_decode_attn(
            self.pool, 0, self.q.cuda(), torch.from_numpy(self.q_pos).cuda(),
            torch.from_numpy(self.table).cuda(), torch.tensor(self.lens, dtype=torch.int32).cuda(),
            max(self.lens), sm_scale, rope_cos=self.rc, rope_sin=self.rs,
            pages_per_split=pages_per_split, k_new=k_new, v_new=v_new)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, sm_scale=1 / np.sqrt(128)):
        pool = self.pool.data.cpu().numpy()
        return oracle.decode_attention(pool, self.num_pages, self.hkv, 0, self.rotary, self.hadamard,
                                       self.q.float().numpy(), self.q_pos, self.table, self.lens,
                                       sm_scale, self.oc, self.os, signs=self.signs, k_scale=self.k_scale,
                                       v_scale=self.v_scale, v_format=self.v_format)


def test_decode_tiny_workload():
    """1 sequence, 1 kv head, 2 query heads, 256 cached + 1 appended token,
    fp32 N(0,1) with 4 outlier channels x20, no RoPE, Hadamard on."""
    c = Case(1, [257], 1, 2, rotary=0, dtype=torch.float32, outliers=4, outlier_scale=20.0)
    assert_attention_close(c.gpu(), c.oracle(), "tiny")


def test_decode_layer8k_workload():
    """1 sequence of 8192 + 1 tokens, 24 query / 4 kv heads, bf16 with 3
    outlier channels x16, RoPE on 32 dims."""
    c = Case(2, [8193], 4, 24)
    assert_attention_close(c.gpu(), c.oracle(), "layer8k")


@pytest.mark.parametrize("lens", [[1], [2], [63], [64], [65], [127, 128, 129], [1000, 3, 2049, 777]])
def test_decode_ragged_lengths(lens):
    c = Case(sum(lens), lens, 2, 12)
    assert_attention_close(c.gpu(), c.oracle(), str(lens))


@pytest.mark.parametrize("group", [1, 2, 3, 6, 8, 16])
def test_decode_group_sizes(group):
    c = Case(100 + group, [700, 1500], 2, 2 * group, rotary=16)
    assert_attention_close(c.gpu(), c.oracle(), f"group {group}")


@pytest.mark.parametrize("hadamard,rotary,pos_scale", [(False, 32, 2.3), (True, 32, 2.3), (True, 0, 1.0),
                                                        (True, 128, 1.0), (False, 0, 1.0), (2, 32, 2.3),
                                                        (2, 0, 1.0), (True, 24, 2.3), (True, 50, 1.0),
                                                        (2, 10, 1.0)])
def test_decode_flags(hadamard, rotary, pos_scale):
    c = Case(7, [3000, 1234], 4, 24, rotary=rotary, hadamard=hadamard, pos_scale=pos_scale,
             outlier_scale=32.0)
    assert_attention_close(c.gpu(), c.oracle(), f"hadamard={hadamard} rotary={rotary}")


def test_decode_heavy_tailed_f32_inputs():
    c = Case(8, [4096, 5000, 300], 4, 24, dtype=torch.float32, student_t=True, outliers=0)
    assert_attention_close(c.gpu(), c.oracle(), "student-t")


def test_decode_split_count_invariance():
    c = Case(9, [5000, 2300], 4, 24)
    ref = c.oracle()
    outs = [c.gpu(pages_per_split=p) for p in (1, 2, 3, 7, 64, 4096)]
    for o in outs:
        assert_attention_close(o, ref, "split")
        assert np.abs(o - outs[0]).max() <= 1e-4 * max(1.0, np.abs(outs[0]).max())


def test_decode_reduce_piece_counts():
    """One 64K-token segment split over 1 to 1024 wavefronts, so its partials
    take every combine path of the reduce (up to 8, 32, 64, 256 and 512
    pieces, and the staged one past 512): all match the oracle and each
    other."""
    c = Case(21, [65536], 1, 6)
    ref = c.oracle()
    outs = []
    for p in (4096, 128, 40, 20, 8, 3, 2, 1):
        o = c.gpu(pages_per_split=p)
        assert_attention_close(o, ref, f"pages_per_split {p}")
        outs.append(o)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-4 * max(1.0, np.abs(outs[0]).max())


def test_decode_ignores_unwritten_workspace():
    """More wavefronts than pages leaves wavefronts with empty ranges inside a
    segment's span; their partial slots are never written.  With the
    workspace filled with NaN bytes beforehand the output must still match
    the oracle (the reduce gives those slots no weight and never multiplies
    them)."""
    c = Case(12, [70, 3, 200], 2, 12)
    need = c.kv.nvfp4kv_decode_workspace_bytes(c.pool, len(c.lens), c.hq, max(c.lens), 0)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = c.kv.nvfp4kv_decode_attn(
        c.pool, 0, c.q.cuda(), torch.from_numpy(c.q_pos).cuda(), torch.from_numpy(c.table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max(c.lens), 1 / np.sqrt(128), workspace=ws,
        rope_cos=c.rc, rope_sin=c.rs)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), c.oracle(), "NaN-filled workspace")


@pytest.mark.parametrize("reps", [1, 8])
@pytest.mark.parametrize("pages_per_split", [1, 2, 4, 8, 32, 64, 512])
def test_decode_unwritten_slots_every_combine_path(pages_per_split, reps):
    """max_seq_len far past the actual lengths gives far more wavefronts than
    work units, so most partial slots inside every segment's span are never
    written.  With the workspace filled with NaN bytes, every combine path of
    the reduce (chosen by the pieces per segment: from 2 to about 1060 here,
    the staged path included) must give those slots no weight: with 3
    sequences in its one-dim-per-thread form, with 24 in its four-dim form
    (a launch of 1152 column blocks of 32 dims)."""
    c = Case(22, [700, 3, 200] * reps, 2, 12)
    max_len = 70000
    table = np.zeros((len(c.lens), (max_len + 63) // 64), np.int32)
    table[:, :c.table.shape[1]] = c.table
    need = c.kv.nvfp4kv_decode_workspace_bytes(c.pool, len(c.lens), c.hq, max_len, pages_per_split)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = c.kv.nvfp4kv_decode_attn(
        c.pool, 0, c.q.cuda(), torch.from_numpy(c.q_pos).cuda(), torch.from_numpy(table).cuda(),
        torch.tensor(c.lens, dtype=torch.int32).cuda(), max_len, 1 / np.sqrt(128), workspace=ws,
        rope_cos=c.rc, rope_sin=c.rs, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    assert_attention_close(out.cpu().numpy(), c.oracle(), f"NaN-filled workspace, pages_per_split {pages_per_split}")


def test_decode_sm_scale_zero_and_large():
    c = Case(10, [900], 2, 4)
    assert_attention_close(c.gpu(sm_scale=0.0), c.oracle(sm_scale=0.0), "sm_scale 0")
    assert_attention_close(c.gpu(sm_scale=0.5), c.oracle(sm_scale=0.5), "sm_scale 0.5")


def test_decode_page_permutation_invariance():
    a = Case(11, [3000], 2, 8, extra_pages=5)
    b_out = None
    # same inputs, different page placement: rebuild with a shifted table
    import nvfp4_quantized_kv_amd as kv
    pool2 = kv.Pool.allocate(a.num_pages, 1, a.hkv, a.rotary, a.hadamard)
    table2 = np.roll(a.table, 7, axis=1) % a.num_pages
    table2[0] = np.random.default_rng(3).permutation(a.num_pages)[:a.table.shape[1]]
    pos = np.arange(3000)
    sl = table2[0, pos // 64].astype(np.int64) * 64 + pos % 64
    kv.nvfp4kv_append(pool2, 0, a.k[0].cuda(), a.v[0].cuda(), torch.from_numpy(sl).cuda(),
                      torch.from_numpy(pos.astype(np.int32)).cuda(), a.rc, a.rs)
    b_out = kv.nvfp4kv_decode_attn(pool2, 0, a.q.cuda(), torch.from_numpy(a.q_pos).cuda(),
                                   torch.from_numpy(table2.astype(np.int32)).cuda(),
                                   torch.tensor(a.lens, dtype=torch.int32).cuda(), 3000, 1 / np.sqrt(128),
                                   rope_cos=a.rc, rope_sin=a.rs).cpu().numpy()
    assert np.abs(a.gpu() - b_out).max() <= 1e-5 * max(1.0, np.abs(b_out).max())


FUSED_CASES = [
    dict(lens=[1]),                                   # empty cache before the step
    dict(lens=[64]),                                  # new token in the last slot of a page
    dict(lens=[65], rotary=0, hadamard=False),        # new token opens a page
    dict(lens=[1000, 3, 2049, 777], dtype=torch.float32),
    dict(lens=[700, 1500], hq=32, rotary=16),         # 16 query heads per kv head
    dict(lens=[3000, 1234], rotary=128, pos_scale=2.3),
    dict(lens=[1000, 130], hadamard=2),               # randomized rotation of the new K and of Q
    dict(lens=[700, 65], rotary=24, pos_scale=2.3),  # a rotary width that is not a multiple of 16
    dict(lens=[300, 64], rotary=126, hadamard=2),
]


def oracle_pool(c):
    """The pool bytes the oracle writes for every token of a Case (each
    sequence's tokens 0 .. T-1), on the Case's 0x7F background."""
    pool = np.full(c.pool.data.numel(), 0x7F, np.uint8)
    for n, T in enumerate(c.lens):
        pos = np.arange(T)
        sl = c.table[n, pos // 64].astype(np.int64) * 64 + pos % 64
        oracle.append(pool, c.num_pages, c.hkv, c.rotary, c.hadamard, 0, c.k[n].float().numpy(),
                      c.v[n].float().numpy(), sl, pos.astype(np.int32), c.oc, c.os, signs=c.signs,
                      k_scale=c.k_scale, v_scale=c.v_scale, v_format=c.v_format)
    return pool


@pytest.mark.parametrize("idx", range(len(FUSED_CASES)))
@pytest.mark.parametrize("pages_per_split", [0, 1, 4096])
def test_decode_quantizes_current_token_in_place(idx, pages_per_split):
    """Decode with k_new/v_new on a cache missing the current token: the
    whole pool afterwards equals the oracle's append of every token (so the
    new token's bytes are the oracle's and no other slot is touched), and
    equals append + decode on the GPU; the attention output equals that of
    append + decode exactly and is within the oracle's tolerance.
    pages_per_split 1 puts a token's page first in a wavefront's range, 4096
    gives one wavefront many segments (appends and query switches past the
    preloaded slots)."""
    kw = dict(FUSED_CASES[idx])
    lens = kw.pop("lens")
    hq = kw.pop("hq", 8)
    full = Case(300 + idx, lens, 2, hq, **kw)
    held = Case(300 + idx, lens, 2, hq, hold_last=True, **kw)
    out_full = full.gpu(pages_per_split=pages_per_split)
    out_fused = held.gpu(pages_per_split=pages_per_split, fused=True)
    assert np.array_equal(held.pool.data.cpu().numpy(), oracle_pool(held)), "pool bytes differ from the oracle"
    assert torch.equal(held.pool.data, full.pool.data), "pool bytes differ from append + decode"
    assert np.array_equal(out_fused, out_full), "output differs from append + decode"
    assert_attention_close(out_fused, held.oracle(), f"fused {lens}")


def test_decode_quantizes_current_token_many_segments_one_wave():
    """16 (sequence, kv head) segments of 1 to 3 pages in one wavefront's
    range: every segment end appends its token, every segment switch makes
    its own query operands."""
    lens = [5, 70, 130, 1]
    full = Case(400, lens, 4, 8)
    held = Case(400, lens, 4, 8, hold_last=True)
    out_full = full.gpu(pages_per_split=4096)
    out_fused = held.gpu(pages_per_split=4096, fused=True)
    assert np.array_equal(held.pool.data.cpu().numpy(), oracle_pool(held))
    assert torch.equal(held.pool.data, full.pool.data)
    assert np.array_equal(out_fused, out_full)
    assert_attention_close(out_fused, held.oracle(), "many segments")


def _many_lens(n_seq):
    return [int(t) for t in np.random.default_rng(n_seq).integers(1, 300, n_seq)]


@pytest.mark.parametrize("n_seq", [64, 65, 200, 256, 257, 300])
@pytest.mark.parametrize("pages_per_split", [0, 16])
def test_decode_many_sequences(n_seq, pages_per_split):
    """More sequences than a wavefront has lanes.  The kernels scan the
    sequences' page offsets across the wavefront in chunks of 64 sequences,
    up to 256 (past that they walk the lengths): 64 and 65 sit on the first
    chunk boundary, 200 spans four chunks, 256 fills them, 257 and 300 take
    the walk.  Ragged lengths of 1-299 tokens; at 16 units per wavefront a
    range spans several segments."""
    c = Case(600 + n_seq, _many_lens(n_seq), 2, 8)
    assert_attention_close(c.gpu(pages_per_split=pages_per_split), c.oracle(),
                           f"{n_seq} sequences, pages_per_split {pages_per_split}")


@pytest.mark.parametrize("n_seq", [65, 300])
def test_decode_many_sequences_fused(n_seq):
    """The same with each sequence's current token quantized by the decode
    launch: the pool bytes equal the oracle's append of every token, the
    output equals append + decode."""
    lens = _many_lens(n_seq)
    full = Case(700 + n_seq, lens, 2, 8)
    held = Case(700 + n_seq, lens, 2, 8, hold_last=True)
    out_full = full.gpu()
    out_fused = held.gpu(fused=True)
    assert np.array_equal(held.pool.data.cpu().numpy(), oracle_pool(held)), "pool bytes differ from the oracle"
    assert np.array_equal(out_fused, out_full), "output differs from append + decode"
    assert_attention_close(out_fused, held.oracle(), f"fused, {n_seq} sequences")
