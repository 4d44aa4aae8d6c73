"""Drive the library on a named workload: fill the pool, run decode steps.

A decode step is, for every layer, decode attention for every sequence with
the new token's K and V handed to the decode kernel, which quantizes them into
the cache itself (nvfp4kv_decode_attn with k_new/v_new).  The unfused form,
nvfp4kv_append followed by nvfp4kv_decode_attn, is kept for comparison.
Inputs come from `workloads`; every computation runs in the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Pool, nvfp4kv_append, nvfp4kv_decode_attn, nvfp4kv_decode_attn_multi,
               nvfp4kv_decode_attn_splits, nvfp4kv_decode_multi_workspace_bytes,
               nvfp4kv_decode_reduce, nvfp4kv_decode_workspace_bytes, nvfp4kv_rope_table)
from . import workloads as W


class DecodeStep:
    def __init__(self, wl: W.Workload, device="cuda", pages_per_split: int = 0,
                 fill_chunk: int = 1 << 16, signs=(0, 0, 0, 0), v_format: int = 0):
        self.wl = wl
        self.device = device
        self.pages_per_split = pages_per_split
        table, num_pages = W.page_table(wl)
        self.table_np = table
        self.pool = Pool.allocate(num_pages, wl.layers, wl.hkv, wl.rotary_dim, int(wl.hadamard), device,
                                  signs=signs, v_format=v_format)
        self.pool.data.zero_()
        self.table = torch.from_numpy(table).to(device)
        self.seq_lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=device)
        self.max_pos = max(wl.cached) + 1 + wl.prefill_chunk + 1
        if wl.rotary_dim:
            c, s = nvfp4kv_rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, self.max_pos)
            self.rope_cos, self.rope_sin = c.to(device), s.to(device)
        else:
            self.rope_cos = self.rope_sin = None
        self.base = W.token_base(wl)
        self.fill_chunk = fill_chunk
        # the step's own inputs: new token K/V and the query, per layer
        n = wl.n_seq
        self.new_pos = torch.tensor(wl.cached, dtype=torch.int32, device=device)
        self.new_slots = torch.from_numpy(
            np.concatenate([W.slots(table, i, [wl.cached[i]]) for i in range(n)])
        ).to(device)
        self.k_new, self.v_new, self.q = [], [], []
        for layer in range(wl.layers):
            ks = torch.cat([W.rows(wl, "k", layer, self.base[i] + wl.cached[i], 1, wl.hkv, device) for i in range(n)])
            vs = torch.cat([W.rows(wl, "v", layer, self.base[i] + wl.cached[i], 1, wl.hkv, device) for i in range(n)])
            qs = torch.cat([W.rows(wl, "q", layer, i, 1, wl.hq, device) for i in range(n)])
            self.k_new.append(ks.contiguous())
            self.v_new.append(vs.contiguous())
            self.q.append(qs.contiguous())
        self.out = torch.empty((n, wl.hq, 128), dtype=torch.float32, device=device)
        ws = nvfp4kv_decode_workspace_bytes(self.pool, n, wl.hq, wl.max_seq_len, pages_per_split)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)

    # -- cache fill (prefill-style appends of the cached tokens) --------------
    def fill(self, layers=None) -> None:
        wl = self.wl
        layers = range(wl.layers) if layers is None else layers
        for layer in layers:
            for i, T in enumerate(wl.cached):
                for start in range(0, T, self.fill_chunk):
                    cnt = min(self.fill_chunk, T - start)
                    self.append_range(layer, i, start, cnt)

    def append_range(self, layer: int, seq: int, start: int, count: int) -> None:
        """Append tokens start .. start+count-1 of sequence `seq` (positions = indices)."""
        wl = self.wl
        k = W.rows(wl, "k", layer, self.base[seq] + start, count, wl.hkv, self.device)
        v = W.rows(wl, "v", layer, self.base[seq] + start, count, wl.hkv, self.device)
        pos = torch.arange(start, start + count, dtype=torch.int32, device=self.device)
        sl = self.table[seq].to(torch.int64)[pos.to(torch.int64) // 64] * 64 + pos.to(torch.int64) % 64
        nvfp4kv_append(self.pool, layer, k, v, sl.contiguous(), pos, self.rope_cos, self.rope_sin)

    # -- the step -------------------------------------------------------------
    def append(self, layer: int) -> None:
        nvfp4kv_append(self.pool, layer, self.k_new[layer], self.v_new[layer], self.new_slots,
                       self.new_pos, self.rope_cos, self.rope_sin)

    def decode(self, layer: int, out=None, fused: bool = False) -> torch.Tensor:
        """Decode attention of `layer`; fused=True also quantizes the new token
        into the cache (no append needed before it)."""
        return nvfp4kv_decode_attn(self.pool, layer, self.q[layer], self.new_pos, self.table,
                                   self.seq_lens, self.wl.max_seq_len, W.sm_scale(),
                                   out=self.out if out is None else out, workspace=self.workspace,
                                   rope_cos=self.rope_cos, rope_sin=self.rope_sin,
                                   pages_per_split=self.pages_per_split,
                                   k_new=self.k_new[layer] if fused else None,
                                   v_new=self.v_new[layer] if fused else None)

    def decode_splits(self, layer: int, fused: bool = False) -> None:
        nvfp4kv_decode_attn_splits(self.pool, layer, self.q[layer], self.new_pos, self.table,
                                   self.seq_lens, self.wl.max_seq_len, W.sm_scale(), self.workspace,
                                   rope_cos=self.rope_cos, rope_sin=self.rope_sin,
                                   pages_per_split=self.pages_per_split,
                                   k_new=self.k_new[layer] if fused else None,
                                   v_new=self.v_new[layer] if fused else None)

    def decode_reduce(self, layer: int, out=None) -> torch.Tensor:
        return nvfp4kv_decode_reduce(self.pool, self.wl.n_seq, self.wl.hq, self.seq_lens,
                                     self.wl.max_seq_len, self.out if out is None else out,
                                     self.workspace, pages_per_split=self.pages_per_split)

    # -- several new query tokens per sequence (speculative verification) ----
    def prepare_multi(self, m: int) -> None:
        """Queries of the last m tokens of every sequence, per layer, and a
        workspace for them; the m tokens must be in the cache (fill + append)."""
        wl, n = self.wl, self.wl.n_seq
        self.m = m
        self.mq = [torch.stack([W.rows(wl, "q", layer, 1000 + i, m, wl.hq, self.device) for i in range(n)])
                   .contiguous() for layer in range(wl.layers)]
        self.mq_pos = torch.tensor([[T - m + j for j in range(m)] for T in wl.seq_lens], dtype=torch.int32,
                                   device=self.device)
        self.mq_out = torch.empty((n, m, wl.hq, 128), dtype=torch.float32, device=self.device)
        need = nvfp4kv_decode_multi_workspace_bytes(self.pool, n, m, wl.hq, wl.max_seq_len, self.pages_per_split)
        self.mq_ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)

    def decode_multi(self, layer: int) -> torch.Tensor:
        return nvfp4kv_decode_attn_multi(self.pool, layer, self.mq[layer], self.mq_pos, self.table,
                                         self.seq_lens, self.wl.max_seq_len, W.sm_scale(), out=self.mq_out,
                                         workspace=self.mq_ws, rope_cos=self.rope_cos, rope_sin=self.rope_sin,
                                         pages_per_split=self.pages_per_split)

    def run(self, fused: bool = True) -> None:
        for layer in range(self.wl.layers):
            if not fused:
                self.append(layer)
            self.decode(layer, fused=fused)
