"""Parity at the full workload sizes, in the launch configuration the benchmark
times (automatic split plan), on sampled outputs the CPU oracle can compute:

- three concurrent sequences of 330K/400K/470K cached tokens, 16 layers,
  24 query / 4 KV heads, randomly permuted pages;
- one 600K-token sequence with linear RoPE scaling x2.3 and outlier
  channels x32, with and without the Hadamard rotation;
- 64 sequences of 4K-64K tokens (Student-t inputs) plus an 8192-token
  prefill-style append per sequence.

Sampled rows must be bit-exact against the oracle's quantization of the same
input rows; sampled sequences' attention outputs must be within 2e-3 absolute
or 1e-2 relative of the oracle's fp64 result on the GPU's own pool bytes.
Method: release post of the gzenz/ninfer fork, section "NVFP4 KV cache (from
scratch)"."""
import numpy as np
import pytest
import torch

import oracle

from test_gpu_decode import assert_attention_close

pytestmark = pytest.mark.gpu


def _step(name, **over):
    from nvfp4_quantized_kv_amd import workloads as W
    from nvfp4_quantized_kv_amd.runner import DecodeStep
    wl = W.config(name)
    for k, v in over.items():
        setattr(wl, k, v)
    st = DecodeStep(wl)
    st.fill()
    torch.cuda.synchronize()
    return wl, st


def _oracle_tables(wl, st):
    if not wl.rotary_dim:
        return None, None
    return oracle.rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, st.max_pos)


def _check_rows(wl, st, layer, seq, positions, oc, os_):
    """Pool bytes of the given token positions == oracle quantization of the
    same input rows (regenerated on the device, copied to the host)."""
    from nvfp4_quantized_kv_amd import workloads as W
    pool = st.pool.data.view(wl.layers, st.pool.num_pages, wl.hkv * 9216)
    for t in positions:
        t = int(t)
        k = W.rows(wl, "k", layer, st.base[seq] + t, 1, wl.hkv, "cuda").float().cpu().numpy()[0]
        v = W.rows(wl, "v", layer, st.base[seq] + t, 1, wl.hkv, "cuda").float().cpu().numpy()[0]
        page = int(st.table_np[seq, t // 64])
        blk = pool[layer, page].cpu().numpy()
        for g in range(wl.hkv):
            c = oc[t] if oc is not None else None
            s = os_[t] if os_ is not None else None
            kc, ks = oracle.quant_row(k[g], wl.rotary_dim, c, s, wl.hadamard)
            vc, vs = oracle.quant_row(v[g])
            gk = oracle.pool_read_row(blk, 1, wl.hkv, 0, t % 64, g, 0)
            gv = oracle.pool_read_row(blk, 1, wl.hkv, 0, t % 64, g, 1)
            assert (gk[0] == kc).all() and (gk[1] == ks).all(), (layer, seq, t, g, "K")
            assert (gv[0] == vc).all() and (gv[1] == vs).all(), (layer, seq, t, g, "V")


def _check_attention(wl, st, layer, seq, out, oc, os_):
    """The oracle on a compact host copy of the sequence's pages (all kv heads)."""
    from nvfp4_quantized_kv_amd import workloads as W
    T = wl.seq_lens[seq]
    npg = (T + 63) // 64
    pages = torch.from_numpy(st.table_np[seq, :npg].astype(np.int64)).cuda()
    pool = st.pool.data.view(wl.layers, st.pool.num_pages, wl.hkv * 9216)[layer]
    compact = pool.index_select(0, pages).contiguous().view(-1).cpu().numpy()
    table = np.arange(npg, dtype=np.int32)[None]
    q = st.q[layer][seq:seq + 1].float().cpu().numpy()
    ref = oracle.decode_attention(compact, npg, wl.hkv, 0, wl.rotary_dim, wl.hadamard, q,
                                  [wl.cached[seq]], table, [T], W.sm_scale(), oc, os_)
    assert_attention_close(out[seq:seq + 1], ref, f"{wl.name} layer {layer} seq {seq}")


def test_three_long_sequences_full_size():
    """The path the benchmark times: the cache holds tokens 0 .. T-2 of every
    sequence, and the decode launch (automatic split plan, the benchmark's
    workspace) quantizes token T-1 into the cache itself; its bytes and
    sampled cached rows must equal the oracle's quantization, the attention
    the oracle's on the resulting pool."""
    wl, st = _step("three_long")
    oc, os_ = _oracle_tables(wl, st)
    rng = np.random.default_rng(0)
    for layer in (0, wl.layers - 1):
        st.decode_splits(layer, fused=True)
        out = st.decode_reduce(layer).cpu().numpy()
        for seq in range(wl.n_seq):
            pos = np.concatenate([rng.integers(0, wl.cached[seq], 6), [wl.cached[seq]]])
            _check_rows(wl, st, layer, seq, pos, oc, os_)
        _check_attention(wl, st, layer, 2, out, oc, os_)      # the 470K sequence
    _check_attention(wl, st, wl.layers - 1, 0, out, oc, os_)  # and the 330K one
    del st
    torch.cuda.empty_cache()


def test_three_long_multi_query_full_size():
    """Speculative verification at the full three-session size: the last 8
    tokens of every sequence as queries (48 columns per kv head, one launch),
    sampled sequences against the oracle."""
    from nvfp4_quantized_kv_amd import workloads as W
    wl, st = _step("three_long", layers=2)
    oc, os_ = _oracle_tables(wl, st)
    layer = 1
    st.append(layer)
    st.prepare_multi(8)
    out = st.decode_multi(layer).cpu().numpy()
    for seq in (2, 0):
        T = wl.seq_lens[seq]
        npg = (T + 63) // 64
        pages = torch.from_numpy(st.table_np[seq, :npg].astype(np.int64)).cuda()
        pool = st.pool.data.view(wl.layers, st.pool.num_pages, wl.hkv * 9216)[layer]
        compact = pool.index_select(0, pages).contiguous().view(-1).cpu().numpy()
        ref = oracle.decode_attention_multi(compact, npg, wl.hkv, 0, wl.rotary_dim, wl.hadamard,
                                            st.mq[layer][seq:seq + 1].float().cpu().numpy(),
                                            st.mq_pos[seq:seq + 1].cpu().numpy(),
                                            np.arange(npg, dtype=np.int32)[None], [T], W.sm_scale(), oc, os_)
        assert_attention_close(out[seq:seq + 1], ref, f"three_long multi-query seq {seq}")
    del st
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["single600k", "single600k_nohad"])
def test_single_600k_sequence_full_size(name):
    wl, st = _step(name, layers=2)
    oc, os_ = _oracle_tables(wl, st)
    rng = np.random.default_rng(1)
    layer = 1
    out = st.decode(layer, fused=True).cpu().numpy()     # the new token quantized by the decode launch
    _check_rows(wl, st, layer, 0, np.concatenate([rng.integers(0, wl.cached[0], 6), [wl.cached[0]]]), oc, os_)
    _check_attention(wl, st, layer, 0, out, oc, os_)
    del st
    torch.cuda.empty_cache()


def test_batch64_prefill_append_and_decode_full_size():
    from nvfp4_quantized_kv_amd import workloads as W
    wl, st = _step("batch64")
    oc, os_ = _oracle_tables(wl, st)
    rng = np.random.default_rng(2)
    # prefill-style append of an 8192-token chunk per sequence, after the new token
    for seq in range(wl.n_seq):
        st.append_range(0, seq, wl.cached[seq] + 1, wl.prefill_chunk)
    st.append(0)
    out = st.decode(0).cpu().numpy()
    torch.cuda.synchronize()
    for seq in rng.choice(wl.n_seq, 3, replace=False):
        first = wl.cached[seq] + 1
        pos = np.concatenate([[first, first + wl.prefill_chunk - 1], rng.integers(first, first + wl.prefill_chunk, 3)])
        _check_rows(wl, st, 0, int(seq), pos, oc, os_)
    for seq in rng.choice(wl.n_seq, 2, replace=False):
        _check_attention(wl, st, 0, int(seq), out, oc, os_)
    del st
    torch.cuda.empty_cache()
