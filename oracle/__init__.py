"""CPU oracle for attention over an NVFP4 KV cache.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
path never imports it.  It wraps ``nvfp4_oracle.c`` (plain C, built with gcc)
through ctypes and shares no code with the HIP library.

Every function follows the release post of the gzenz/ninfer fork
(prismix.dev), section "NVFP4 KV cache (from scratch)" and section "YaRN
context extension"; the C source states, per function, what it computes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

HEAD_DIM = 128
PAGE = 64
BLOCK_BYTES = 9216          # NVFP4 K and V: 144 bytes per token per kv head
BLOCK_BYTES_F16V = 20992    # NVFP4 K, fp16 V: 328 bytes per token per kv head


def block_bytes(v_format: int = 0) -> int:
    return BLOCK_BYTES_F16V if v_format else BLOCK_BYTES


def build() -> str:
    """Compile the oracle with gcc (binary32 steps without contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, f64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_float
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_e4m3_value.argtypes = [ctypes.c_int]
        L.orc_e4m3_value.restype = f64
        L.orc_e4m3_scale_code.argtypes = [f32]
        L.orc_e4m3_scale_code.restype = ctypes.c_int
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e2m1_value.restype = f64
        L.orc_e2m1_code.argtypes = [f32, f64]
        L.orc_e2m1_code.restype = ctypes.c_int
        L.orc_rope_table.argtypes = [f64, ctypes.c_int, f64, ctypes.c_int, P, P]
        L.orc_rope_apply.argtypes = [P, ctypes.c_int, P, P]
        L.orc_hadamard128.argtypes = [P]
        L.orc_quant_row.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P, P]
        L.orc_dequant_row.argtypes = [P, P, P]
        L.orc_f32_to_f16.argtypes = [f32]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = f64
        L.orc_f32_to_f16_array.argtypes = [P, i64, P]
        L.orc_pool_bytes.argtypes = [ctypes.c_int, i64, ctypes.c_int, ctypes.c_int]
        L.orc_pool_bytes.restype = ctypes.c_size_t
        L.orc_pool_read_row.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, i64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, P, P]
        L.orc_pool_read_v16.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, i64, ctypes.c_int, P]
        L.orc_append.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
                                 ctypes.c_int, P, P, P, P, P, P, ctypes.c_int]
        L.orc_decode_attention.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, P, ctypes.c_int, ctypes.c_int, P, P, P, P,
                                           P, ctypes.c_int, P, f64, P, ctypes.c_int, P]
        L.orc_reference_attention.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, P, i32, P, P, P, P, P, f64, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> int:
    """Threads of the oracle's OpenMP loops; returns the count now in use."""
    lib().orc_set_threads(int(n))
    return lib().orc_max_threads()


# -- scalar codecs -----------------------------------------------------------
def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_scale_code(amax: float) -> int:
    return lib().orc_e4m3_scale_code(float(np.float32(amax)))


def e2m1_value(nibble: int) -> float:
    return lib().orc_e2m1_value(int(nibble))


def e2m1_code(y: float, s: float) -> int:
    return lib().orc_e2m1_code(float(np.float32(y)), float(s))


# -- row operations ----------------------------------------------------------
def rope_table(theta: float, rotary_dim: int, pos_scale: float, max_pos: int):
    half = rotary_dim // 2
    c = np.zeros((max_pos, max(half, 1)), np.float32)
    s = np.zeros((max_pos, max(half, 1)), np.float32)
    if half:
        lib().orc_rope_table(theta, rotary_dim, pos_scale, max_pos, _p(c), _p(s))
    return c[:, :half].copy(), s[:, :half].copy()


def rope_apply(x: np.ndarray, rotary_dim: int, c_row: np.ndarray, s_row: np.ndarray):
    x = _c(x, np.float32).copy()
    lib().orc_rope_apply(_p(x), rotary_dim, _p(_c(c_row, np.float32)), _p(_c(s_row, np.float32)))
    return x


def hadamard128(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32).copy()
    assert x.shape == (HEAD_DIM,)
    lib().orc_hadamard128(_p(x))
    return x


def _rotation(hadamard, signs):
    """(mode, sign mask) for the C side: mode 0 none, 1 the Hadamard rotation,
    2 the rotation after negating the elements whose bit is set in `signs`
    (4 x uint32, bit j of element j)."""
    mode = int(hadamard)
    if mode not in (0, 1, 2):
        raise ValueError("hadamard must be 0, 1 or 2")
    if mode == 2:
        m = _c(signs, np.uint32)
        if m.shape != (4,):
            raise ValueError("signs must be 4 uint32 words")
        return mode, m
    return mode, None


def quant_row(x, rotary_dim=0, c_row=None, s_row=None, hadamard=False, signs=None):
    mode, m = _rotation(hadamard, signs)
    x = _c(x, np.float32)
    codes = np.zeros(64, np.uint8)
    scales = np.zeros(8, np.uint8)
    cr = _c(c_row, np.float32) if rotary_dim else np.zeros(1, np.float32)
    sr = _c(s_row, np.float32) if rotary_dim else np.zeros(1, np.float32)
    lib().orc_quant_row(_p(x), rotary_dim, _p(cr), _p(sr), mode, _p(m) if m is not None else None, _p(codes),
                        _p(scales))
    return codes, scales


def dequant_row(codes, scales) -> np.ndarray:
    out = np.zeros(HEAD_DIM, np.float64)
    lib().orc_dequant_row(_p(_c(codes, np.uint8)), _p(_c(scales, np.uint8)), _p(out))
    return out


# -- fp16 (the V storage of the upstream variant) ---------------------------
def f16_bits(x) -> np.ndarray:
    """binary16 bits of float32 values, nearest with ties to even."""
    x = _c(x, np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().orc_f32_to_f16_array(_p(x), x.size, _p(out))
    return out


def f16_value(bits: int) -> float:
    return lib().orc_f16_value(int(bits))


# -- pool --------------------------------------------------------------------
def pool_bytes(num_layers: int, num_pages: int, num_kv_heads: int, v_format: int = 0) -> int:
    return lib().orc_pool_bytes(num_layers, num_pages, num_kv_heads, int(v_format))


def pool_read_row(pool, num_pages, hkv, layer, slot, kvh, which, v_format=0):
    """Codes and scales of one cached NVFP4 row (which 0 = K, 1 = V; V only
    in a v_format 0 pool)."""
    if which and v_format:
        raise ValueError("an fp16-V pool holds no V codes (pool_read_v16)")
    codes = np.zeros(64, np.uint8)
    scales = np.zeros(8, np.uint8)
    lib().orc_pool_read_row(_p(pool), num_pages, hkv, layer, int(slot), kvh, which, int(v_format),
                            _p(codes), _p(scales))
    return codes, scales


def pool_read_v16(pool, num_pages, hkv, layer, slot, kvh) -> np.ndarray:
    """The 128 fp16 V values (bits, uint16) of one cached row of an fp16-V pool."""
    out = np.zeros(HEAD_DIM, np.uint16)
    lib().orc_pool_read_v16(_p(pool), num_pages, hkv, layer, int(slot), kvh, _p(out))
    return out


def _inverse_scale(g) -> np.float32:
    """binary32 1/g of a per-tensor global scale (0 meaning 1)."""
    g = np.float32(1.0 if g == 0 else g)
    return np.float32(1.0) / g


def append(pool, num_pages, hkv, rotary_dim, hadamard, layer, k, v, slots, positions,
           cos_tab=None, sin_tab=None, signs=None, k_scale=1.0, v_scale=1.0, v_format=0):
    """Quantize and write n_tok tokens into `pool` (a writable uint8 array).

    k_scale, v_scale: NVFP4's second scaling level, one FP32 factor per tensor
    over the E4M3 block scales (NVIDIA's NVFP4 format description; the release
    post keeps it at 1).  Reading taken: each input element is first
    multiplied, in binary32, by the binary32 reciprocal of the scale; RoPE,
    rotation and block quantization then run on those values unchanged.

    v_format 1 keeps V in fp16 (the upstream storage the release post names,
    NVFP4 section, bullet 2): each V element, after the multiplication by
    1/v_scale, is rounded to binary16 (nearest, ties to even)."""
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    mode, m = _rotation(hadamard, signs)
    k = _c(k, np.float32) * _inverse_scale(k_scale)
    v = _c(v, np.float32) * _inverse_scale(v_scale)
    n_tok = k.shape[0]
    slots = _c(slots, np.int64)
    positions = _c(positions, np.int32)
    ct = _c(cos_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    st = _c(sin_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    lib().orc_append(_p(pool), num_pages, hkv, rotary_dim, mode, _p(m) if m is not None else None, layer, n_tok,
                     _p(k), _p(v), _p(slots), _p(positions), _p(ct), _p(st), int(v_format))


def decode_attention(pool, num_pages, hkv, layer, rotary_dim, hadamard, q, q_pos,
                     page_table, seq_lens, sm_scale, cos_tab=None, sin_tab=None, signs=None, v_rows=None,
                     k_scale=1.0, v_scale=1.0, v_format=0):
    """fp64 attention for every sequence and query head over the pool's bytes.
    v_rows [T][hkv][128] (one sequence only): V values taken from it instead
    of the pool, for the variant that keeps V unquantized.

    k_scale, v_scale: the pool's global scales; a cached K value is its block
    value times k_scale, a V value its block value times v_scale.  The factors
    are applied as sm_scale * k_scale on every score and v_scale on the
    output, the same products regrouped (exact in real arithmetic).

    v_format 1: the pool keeps V in fp16; a cached V value is its fp16
    value times v_scale."""
    gk = 1.0 if k_scale == 0 else float(k_scale)
    gv = 1.0 if (v_scale == 0 or v_rows is not None) else float(v_scale)
    sm_scale = float(sm_scale) * gk
    mode, m = _rotation(hadamard, signs)
    vr = None
    if v_rows is not None:
        vr = _c(v_rows, np.float32)
        if len(seq_lens) != 1 or vr.shape != (int(seq_lens[0]), hkv, HEAD_DIM):
            raise ValueError("v_rows needs one sequence and [T][hkv][128] rows")
    q = _c(q, np.float32)
    n_seq, hq, _ = q.shape
    page_table = _c(page_table, np.int32)
    out = np.zeros((n_seq, hq, HEAD_DIM), np.float64)
    ct = _c(cos_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    st = _c(sin_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    lib().orc_decode_attention(_p(_c(pool, np.uint8)), num_pages, hkv, layer, rotary_dim,
                               mode, _p(m) if m is not None else None, n_seq, hq, _p(q), _p(_c(q_pos, np.int32)),
                               _p(ct), _p(st), _p(page_table), page_table.shape[1],
                               _p(_c(seq_lens, np.int32)), float(sm_scale), _p(vr) if vr is not None else None,
                               int(v_format), _p(out))
    return out * gv


def decode_attention_multi(pool, num_pages, hkv, layer, rotary_dim, hadamard, q, q_pos,
                           page_table, seq_lens, sm_scale, cos_tab=None, sin_tab=None, signs=None,
                           k_scale=1.0, v_scale=1.0, v_format=0):
    """fp64 attention of M new query tokens per sequence over the pool's bytes,
    causal among the new tokens: the decode step of speculative verification
    (ai-manual.ru article on "Ninfer 4080", section "Key features": the draft
    model proposes K tokens, the main model checks them in one step).

    q [n_seq][M][hq][128], q_pos [n_seq][M]; seq_lens[n] counts all M tokens,
    which are the last M of the sequence.  Query token j of sequence n sees
    tokens 0 .. seq_lens[n] - M + j, so its output is a one-token decode over
    that prefix: this function is that definition, one decode_attention call
    over the n_seq * M (sequence, token) pairs."""
    q = _c(q, np.float32)
    n_seq, m = q.shape[0], q.shape[1]
    lens = np.asarray(seq_lens, np.int64)
    if (lens < m).any():
        raise ValueError("every sequence must hold its M new tokens")
    rows = np.repeat(_c(page_table, np.int32), m, axis=0)
    pref = (lens[:, None] - m + 1 + np.arange(m)[None, :]).reshape(-1).astype(np.int32)
    out = decode_attention(pool, num_pages, hkv, layer, rotary_dim, hadamard,
                           q.reshape(n_seq * m, q.shape[2], HEAD_DIM),
                           np.asarray(q_pos, np.int32).reshape(-1), rows, pref, sm_scale,
                           cos_tab, sin_tab, signs, k_scale=k_scale, v_scale=v_scale, v_format=v_format)
    return out.reshape(n_seq, m, q.shape[2], HEAD_DIM)


def spill_pages(pool, num_layers, num_pages, hkv, page_ids, v_format=0):
    """Host copy of whole cache pages, for the pinned host arena of the
    release post's section "Multi-level prefix reuse with host-KV safety
    net" (pages are spilled device to host before eviction and restored
    later).  A page is every layer's and every kv head's 9216-byte block of
    that page id; the arena holds page i of the list at
    arena[i][layer][kvh][block].  Pool layout [layer][page][kvh][block]; a
    block is 9216 bytes (20992 in an fp16-V pool)."""
    bb = block_bytes(v_format)
    pool = np.asarray(pool, np.uint8).reshape(num_layers, num_pages, hkv, bb)
    ids = np.asarray(page_ids, np.int64)
    arena = np.empty((len(ids), num_layers, hkv, bb), np.uint8)
    for i, pid in enumerate(ids):
        arena[i] = pool[:, pid]
    return arena


def restore_pages(pool, num_layers, num_pages, hkv, page_ids, arena, v_format=0):
    """The reverse of spill_pages: page i of the arena back into page id
    page_ids[i] of the pool (every layer and kv head), in place.  The ids
    must be distinct (two arena pages cannot both become one page)."""
    ids = np.asarray(page_ids, np.int64)
    if len(np.unique(ids)) != len(ids):
        raise ValueError("restore_pages: page ids must be distinct")
    bb = block_bytes(v_format)
    view = np.asarray(pool).reshape(num_layers, num_pages, hkv, bb)
    arena = np.asarray(arena, np.uint8).reshape(-1, num_layers, hkv, bb)
    for i, pid in enumerate(ids):
        view[:, pid] = arena[i]
    return pool


def reference_attention(q, q_pos, k, v, k_pos, rotary_dim, sm_scale, cos_tab=None, sin_tab=None):
    """fp64 attention on unquantized rows for one sequence: q [hq][128], k/v [T][hkv][128]."""
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    hq = q.shape[0]
    T, hkv, _ = k.shape
    out = np.zeros((hq, HEAD_DIM), np.float64)
    ct = _c(cos_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    st = _c(sin_tab, np.float32) if rotary_dim else np.zeros(1, np.float32)
    lib().orc_reference_attention(hkv, hq, T, rotary_dim, _p(q), int(q_pos), _p(k), _p(v),
                                  _p(_c(k_pos, np.int32)), _p(ct), _p(st), float(sm_scale), _p(out))
    return out
