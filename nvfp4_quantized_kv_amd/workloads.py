"""Seeded synthetic inputs for the benchmark and the tests.

Inputs only: shapes, value distributions, outlier channels, page tables and
slots.  None of the method's arithmetic lives here; both the HIP path and the
CPU oracle receive what these functions produce.

The shapes follow the workloads this library targets (one tiny case, one
8K-token layer, three long sessions of 330K/400K/470K tokens, a batch of 64
sequences of 4K-64K tokens with an 8K-token prefill chunk, one 600K-token
session with linear RoPE scaling).  Values are N(0, 1) or Student-t(3), with
a seeded set of outlier channels multiplied into Q, K and V alike.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
PAGE = 64


@dataclass
class Workload:
    name: str
    cached: list                 # cached tokens per sequence (before the appended one)
    layers: int
    hq: int
    hkv: int
    rotary_dim: int
    theta: float
    pos_scale: float
    dtype: str                   # "f32" or "bf16"
    dist: str                    # "normal" or "student_t"
    outliers: int                # number of outlier channels
    outlier_scale: float
    hadamard: bool = True
    seed: int = 0
    prefill_chunk: int = 0       # tokens appended per sequence by the prefill-style append
    extra_pages: int = 0         # pool pages beyond what the sequences use
    nu: int = 3                  # Student-t degrees of freedom

    @property
    def n_seq(self) -> int:
        return len(self.cached)

    @property
    def seq_lens(self) -> list:
        """Tokens attended in the decode step: cached + the appended one."""
        return [t + 1 for t in self.cached]

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens)

    def pages_of(self, n_tokens: int) -> int:
        return (n_tokens + PAGE - 1) // PAGE

    @property
    def seq_pages(self) -> list:
        return [self.pages_of(t + 1 + self.prefill_chunk) for t in self.cached]

    @property
    def num_pages(self) -> int:
        return sum(self.seq_pages) + self.extra_pages

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def decode_bytes_per_layer(self, v_format: int = 0) -> int:
        """Algorithmic bytes one decode pass reads per layer: 144 per token per
        kv head, or 328 when the pool keeps V in fp16 (72 B of NVFP4 K and
        256 B of V)."""
        return (144 if v_format == 0 else 328) * self.hkv * sum(self.seq_lens)


def _c4_lengths(seed: int) -> list:
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(4096, 65536 + 1, size=64)]


def config(name: str) -> Workload:
    """Named workloads.  `tiny` and `layer8k` are small enough for full oracle checks."""
    if name == "tiny":
        return Workload("tiny", [256], 1, 2, 1, 0, 1e7, 1.0, "f32", "normal", 4, 20.0, seed=1000)
    if name == "layer8k":
        return Workload("layer8k", [8192], 1, 24, 4, 32, 1e7, 1.0, "bf16", "normal", 3, 16.0, seed=2000)
    if name == "three_long":
        return Workload("three_long", [330000, 400000, 470000], 16, 24, 4, 32, 1e7, 1.0, "bf16",
                        "normal", 3, 16.0, seed=3000)
    if name == "batch64":
        return Workload("batch64", _c4_lengths(4000), 1, 24, 4, 32, 1e7, 1.0, "bf16", "student_t",
                        3, 1.0, seed=4000, prefill_chunk=8192)
    if name == "single600k":
        return Workload("single600k", [600000], 16, 24, 4, 32, 1e7, 2.3, "bf16", "normal", 3, 32.0,
                        seed=5000)
    if name == "single600k_nohad":
        w = config("single600k")
        w.name, w.hadamard = "single600k_nohad", False
        return w
    raise KeyError(name)


ALL = ["tiny", "layer8k", "three_long", "batch64", "single600k", "single600k_nohad"]


def outlier_channels(wl: Workload) -> np.ndarray:
    rng = np.random.default_rng(wl.seed + 17)
    return np.sort(rng.choice(HEAD_DIM, size=wl.outliers, replace=False)) if wl.outliers else np.zeros(0, np.int64)


def _multiplier(wl: Workload, device) -> torch.Tensor:
    m = torch.ones(HEAD_DIM, dtype=torch.float32)
    ch = outlier_channels(wl)
    if len(ch):
        m[torch.from_numpy(ch)] = float(wl.outlier_scale)
    return m.to(device)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def rows(wl: Workload, kind: str, layer: int, start: int, count: int, heads: int,
         device="cpu") -> torch.Tensor:
    """Rows [count][heads][128] of input `kind` ("k", "v", "q", "kp", "vp") for
    a layer.  Rows are drawn in fixed chunks of 4096 tokens, each chunk from
    its own seed, so any token range can be regenerated on its own.  For "k"
    and "v", `start` is the sequence-wide token index over all sequences laid
    end to end (see token_base)."""
    kind_id = {"k": 1, "v": 2, "q": 3, "kp": 4, "vp": 5}[kind]
    out = torch.empty((count, heads, HEAD_DIM), dtype=torch.float32, device=device)
    mult = _multiplier(wl, device)
    CH = 4096
    done = 0
    while done < count:
        tok = start + done
        ch = tok // CH
        off = tok - ch * CH
        n = min(CH - off, count - done)
        seed = (wl.seed * 1_000_003 + layer * 7919 + kind_id * 104729 + ch) % (2 ** 62)
        g = _generator(device, seed)
        full = torch.randn((CH, heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
        if wl.dist == "student_t":
            chi = torch.zeros_like(full)
            for _ in range(wl.nu):
                z = torch.randn((CH, heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
                chi += z * z
            full = full / torch.sqrt(chi / wl.nu)
        out[done:done + n] = full[off:off + n]
        done += n
    out *= mult
    return out.to(wl.torch_dtype)


def token_base(wl: Workload) -> list:
    """Start of each sequence in the sequence-wide token index used by rows()."""
    base, acc = [], 0
    for t in wl.cached:
        base.append(acc)
        acc += t + 1 + wl.prefill_chunk
    return base


def page_table(wl: Workload) -> tuple[np.ndarray, int]:
    """Randomly permuted page ids: sequence n owns table[n][:seq_pages[n]].
    Returns (table [n_seq][max_pages] int32, num_pages)."""
    rng = np.random.default_rng(wl.seed + 99)
    perm = rng.permutation(wl.num_pages).astype(np.int32)
    width = max(wl.seq_pages)
    table = np.zeros((wl.n_seq, width), np.int32)
    at = 0
    for n, npg in enumerate(wl.seq_pages):
        table[n, :npg] = perm[at:at + npg]
        at += npg
    return table, wl.num_pages


def slots(table: np.ndarray, seq: int, positions: np.ndarray) -> np.ndarray:
    positions = np.asarray(positions, np.int64)
    return table[seq, positions // PAGE].astype(np.int64) * PAGE + positions % PAGE


def sm_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)
