"""Python binding of libnvfp4kv (attention over an NVFP4 KV cache on MI355X).

Argument marshalling only: every step of append, decode attention and
dequantization runs in the HIP kernels of ``libnvfp4kv.so``.  PyTorch supplies
device memory and the stream.  The functions carry the names of the C entry
points declared in ``include/nvfp4kv.h`` and take torch tensors in place of
pointers.  There is no CPU fallback: if the library cannot be loaded, import
fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# NVFP4KV_DEBUG=1 loads the checked build (device-side tables range-checked
# on the host before every launch); NVFP4KV_LIB names another build outright
LIB_PATH = os.environ.get("NVFP4KV_LIB") or os.path.join(
    _PKG, "libnvfp4kv_debug.so" if os.environ.get("NVFP4KV_DEBUG", "0") not in ("", "0") else "libnvfp4kv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
HEAD_DIM, PAGE_SIZE, BLOCK_BYTES = 128, 64, 9216
BLOCK_BYTES_F16V = 20992       # v_format 1: NVFP4 K, fp16 V
V_NVFP4, V_FP16 = 0, 1


class NVFP4KVError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class _PoolDesc(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("hadamard", ctypes.c_int32),
        ("hadamard_signs", ctypes.c_uint32 * 4),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("v_format", ctypes.c_int32),
    ]


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """ctypes signatures of the C entry points on a loaded build."""
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PD = ctypes.POINTER(_PoolDesc)
    L.nvfp4kv_pool_bytes.argtypes = [PD]
    L.nvfp4kv_pool_bytes.restype = sz
    L.nvfp4kv_rope_table.argtypes = [ctypes.c_double, i32, ctypes.c_double, i32, P, P]
    L.nvfp4kv_rope_table.restype = ctypes.c_int
    L.nvfp4kv_append.argtypes = [PD, i32, i32, P, P, ctypes.c_int, P, P, P, P, i32, P]
    L.nvfp4kv_append.restype = ctypes.c_int
    L.nvfp4kv_decode_workspace_bytes.argtypes = [PD, i32, i32, i64, i32]
    L.nvfp4kv_decode_workspace_bytes.restype = sz
    L.nvfp4kv_decode_attn.argtypes = [PD, i32, i32, i32, P, P, P, ctypes.c_int, P, P, P, i32, P, i32,
                                      P, i64, ctypes.c_float, P, P, sz, i32, P]
    L.nvfp4kv_decode_attn.restype = ctypes.c_int
    L.nvfp4kv_decode_attn_static.argtypes = [PD, i32, i32, i32, P, P, P, ctypes.c_int, P, P, P, i32, P, i32,
                                             P, i64, ctypes.c_float, P, i32, P]
    L.nvfp4kv_decode_attn_static.restype = ctypes.c_int
    L.nvfp4kv_decode_attn_splits.argtypes = [PD, i32, i32, i32, P, P, P, ctypes.c_int, P, P, P, i32,
                                             P, i32, P, i64, ctypes.c_float, P, sz, i32, P]
    L.nvfp4kv_decode_attn_splits.restype = ctypes.c_int
    L.nvfp4kv_decode_multi_workspace_bytes.argtypes = [PD, i32, i32, i32, i64, i32]
    L.nvfp4kv_decode_multi_workspace_bytes.restype = sz
    L.nvfp4kv_decode_attn_multi.argtypes = [PD, i32, i32, i32, i32, P, ctypes.c_int, P, P, P, i32, P, i32,
                                            P, i64, ctypes.c_float, P, P, sz, i32, P]
    L.nvfp4kv_decode_attn_multi.restype = ctypes.c_int
    L.nvfp4kv_decode_reduce.argtypes = [PD, i32, i32, P, i64, P, P, sz, i32, P]
    L.nvfp4kv_decode_reduce.restype = ctypes.c_int
    L.nvfp4kv_dequant.argtypes = [PD, i32, i32, P, P, P, ctypes.c_int, i32, P]
    L.nvfp4kv_dequant.restype = ctypes.c_int
    L.nvfp4kv_page_bytes.argtypes = [PD]
    L.nvfp4kv_page_bytes.restype = sz
    L.nvfp4kv_spill_pages.argtypes = [PD, i32, P, P, sz, P]
    L.nvfp4kv_spill_pages.restype = ctypes.c_int
    L.nvfp4kv_restore_pages.argtypes = [PD, i32, P, P, sz, P]
    L.nvfp4kv_restore_pages.restype = ctypes.c_int
    L.nvfp4kv_stream_read.argtypes = [PD, i32, i32, P, i32, P, i32, P, P]
    L.nvfp4kv_stream_read.restype = ctypes.c_int
    L.nvfp4kv_last_error.argtypes = []
    L.nvfp4kv_last_error.restype = ctypes.c_char_p
    L.nvfp4kv_version.argtypes = []
    L.nvfp4kv_version.restype = ctypes.c_char_p
    L.nvfp4kv_check_decode_tables.argtypes = [PD, i32, i32, P, i32, P, i64, P, i32]
    L.nvfp4kv_check_decode_tables.restype = ctypes.c_int
    L.nvfp4kv_check_slots.argtypes = [PD, i32, P, P, i32]
    L.nvfp4kv_check_slots.restype = ctypes.c_int
    L.nvfp4kv_check_page_ids.argtypes = [PD, i32, P, i32]
    L.nvfp4kv_check_page_ids.restype = ctypes.c_int
    L.nvfp4kv_checked_build.argtypes = []
    L.nvfp4kv_checked_build.restype = ctypes.c_int
    return L


def load_build(path: str) -> ctypes.CDLL:
    """Load a build of the library (e.g. the checked one) with its signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m nvfp4_quantized_kv_amd.build`")
    return _declare(ctypes.CDLL(path))


_lib = load_build(LIB_PATH)

EXPORTED = ["nvfp4kv_pool_bytes", "nvfp4kv_rope_table", "nvfp4kv_append",
            "nvfp4kv_decode_workspace_bytes", "nvfp4kv_decode_attn", "nvfp4kv_decode_attn_static",
            "nvfp4kv_decode_attn_splits",
            "nvfp4kv_decode_reduce", "nvfp4kv_decode_multi_workspace_bytes", "nvfp4kv_decode_attn_multi",
            "nvfp4kv_dequant", "nvfp4kv_page_bytes", "nvfp4kv_spill_pages", "nvfp4kv_restore_pages",
            "nvfp4kv_stream_read", "nvfp4kv_last_error", "nvfp4kv_version", "nvfp4kv_check_decode_tables",
            "nvfp4kv_check_slots", "nvfp4kv_check_page_ids", "nvfp4kv_checked_build"]


def lib() -> ctypes.CDLL:
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != OK:
        raise NVFP4KVError(fn, rc, _lib.nvfp4kv_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _scratch(t: torch.Tensor, stream) -> torch.Tensor:
    """A tensor this binding allocated (on torch's current stream) that the
    library's kernels use on `stream`: if that is another stream, the
    caching allocator is told, so the block is not handed to a later
    allocation before the work queued on `stream` has finished with it."""
    if stream is not None and stream.cuda_stream != torch.cuda.current_stream(t.device).cuda_stream:
        t.record_stream(stream)
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


@dataclass
class Pool:
    """A paged NVFP4 KV pool: one uint8 device tensor plus its descriptor."""
    data: torch.Tensor          # uint8, nvfp4kv_pool_bytes(...) bytes
    num_pages: int
    num_layers: int
    num_kv_heads: int
    rotary_dim: int = 0
    hadamard: int = 1           # 0 none, 1 Hadamard rotation, 2 randomized rotation
    signs: tuple = (0, 0, 0, 0)  # hadamard 2: 128-bit element mask, 4 uint32 words
    k_scale: float = 1.0        # per-tensor global scales of K and V (stored values are x / scale)
    v_scale: float = 1.0
    v_format: int = V_NVFP4     # V_FP16: V kept in fp16 (328 bytes per token per kv head)

    @classmethod
    def allocate(cls, num_pages: int, num_layers: int, num_kv_heads: int, rotary_dim: int = 0,
                 hadamard: int = 1, device="cuda", signs=(0, 0, 0, 0), k_scale: float = 1.0,
                 v_scale: float = 1.0, v_format: int = V_NVFP4) -> "Pool":
        signs = tuple(int(x) & 0xFFFFFFFF for x in signs)
        desc = _PoolDesc(None, num_pages, num_layers, num_kv_heads, HEAD_DIM, PAGE_SIZE,
                         rotary_dim, int(hadamard), (ctypes.c_uint32 * 4)(*signs), k_scale, v_scale,
                         int(v_format))
        nbytes = _lib.nvfp4kv_pool_bytes(ctypes.byref(desc))
        if nbytes == 0:
            raise ValueError("invalid pool shape")
        data = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return cls(data, num_pages, num_layers, num_kv_heads, rotary_dim, int(hadamard), signs, float(k_scale),
                   float(v_scale), int(v_format))

    @property
    def block_bytes(self) -> int:
        return BLOCK_BYTES_F16V if self.v_format else BLOCK_BYTES

    def desc(self) -> _PoolDesc:
        return _PoolDesc(self.data.data_ptr(), self.num_pages, self.num_layers, self.num_kv_heads,
                         HEAD_DIM, PAGE_SIZE, self.rotary_dim, int(self.hadamard),
                         (ctypes.c_uint32 * 4)(*self.signs), self.k_scale, self.v_scale, int(self.v_format))


def nvfp4kv_version() -> str:
    return _lib.nvfp4kv_version().decode()


def nvfp4kv_last_error() -> str:
    return _lib.nvfp4kv_last_error().decode()


def nvfp4kv_pool_bytes(num_pages: int, num_layers: int, num_kv_heads: int, v_format: int = V_NVFP4) -> int:
    desc = _PoolDesc(None, num_pages, num_layers, num_kv_heads, HEAD_DIM, PAGE_SIZE, 0, 1,
                     (ctypes.c_uint32 * 4)(0, 0, 0, 0), 0.0, 0.0, int(v_format))
    return _lib.nvfp4kv_pool_bytes(ctypes.byref(desc))


def nvfp4kv_rope_table(theta: float, rotary_dim: int, pos_scale: float, max_pos: int):
    """Host RoPE table (cos, sin), each a float32 CPU tensor [max_pos][rotary_dim/2]."""
    half = rotary_dim // 2
    c = torch.empty((max_pos, half), dtype=torch.float32)
    s = torch.empty((max_pos, half), dtype=torch.float32)
    _check("nvfp4kv_rope_table",
           _lib.nvfp4kv_rope_table(float(theta), int(rotary_dim), float(pos_scale), int(max_pos),
                                   c.data_ptr(), s.data_ptr()))
    return c, s


def nvfp4kv_append(pool: Pool, layer: int, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor,
                   positions: torch.Tensor | None = None, rope_cos: torch.Tensor | None = None,
                   rope_sin: torch.Tensor | None = None, stream=None) -> None:
    """Quantize k, v [n_tok][Hkv][128] into `slots` (int64) of `layer`."""
    assert k.is_contiguous() and v.is_contiguous() and k.dtype == v.dtype and k.shape == v.shape
    assert slots.dtype == torch.int64 and slots.is_contiguous()
    assert positions is None or (positions.dtype == torch.int32 and positions.is_contiguous())
    n_tok = k.shape[0]
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    d = pool.desc()
    _check("nvfp4kv_append",
           _lib.nvfp4kv_append(ctypes.byref(d), layer, n_tok, _ptr(k), _ptr(v), _dtype_code(k),
                               _ptr(slots), _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), max_pos,
                               _stream(stream)))


def _check_new(q, k_new, v_new) -> None:
    if k_new is None and v_new is None:
        return
    assert k_new is not None and v_new is not None, "k_new and v_new go together"
    assert k_new.is_contiguous() and v_new.is_contiguous()
    assert k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new/v_new take the dtype of q"
    assert k_new.shape == v_new.shape and k_new.shape[0] == q.shape[0] and k_new.shape[2] == HEAD_DIM


def nvfp4kv_decode_workspace_bytes(pool: Pool, n_seq: int, n_q_heads: int, max_seq_len: int,
                                   pages_per_split: int = 0) -> int:
    d = pool.desc()
    return _lib.nvfp4kv_decode_workspace_bytes(ctypes.byref(d), n_seq, n_q_heads, max_seq_len,
                                               pages_per_split)


def nvfp4kv_decode_attn(pool: Pool, layer: int, q: torch.Tensor, q_positions: torch.Tensor | None,
                        page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                        sm_scale: float, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, rope_cos: torch.Tensor | None = None,
                        rope_sin: torch.Tensor | None = None, pages_per_split: int = 0,
                        k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Decode attention; q [n_seq][Hq][128] -> out [n_seq][Hq][128] float32.

    With k_new/v_new [n_seq][Hkv][128] (same dtype as q) the current token is
    quantized into the cache by the decode kernel itself (no separate append)."""
    assert q.is_contiguous() and page_table.is_contiguous() and seq_lens.is_contiguous()
    _check_new(q, k_new, v_new)
    assert page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    n_seq, n_q_heads, _ = q.shape
    if out is None:
        out = _scratch(torch.empty((n_seq, n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device), stream)
    need = nvfp4kv_decode_workspace_bytes(pool, n_seq, n_q_heads, max_seq_len, pages_per_split)
    if workspace is None:
        workspace = _scratch(torch.empty(max(need, 256), dtype=torch.uint8, device=q.device), stream)
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    d = pool.desc()
    _check("nvfp4kv_decode_attn",
           _lib.nvfp4kv_decode_attn(ctypes.byref(d), layer, n_seq, n_q_heads, _ptr(q), _ptr(k_new),
                                    _ptr(v_new), _dtype_code(q),
                                    _ptr(q_positions), _ptr(rope_cos), _ptr(rope_sin), max_pos,
                                    _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                                    int(max_seq_len), float(sm_scale), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), pages_per_split,
                                    _stream(stream)))
    return out


STATIC_WORKSPACE_BYTES = 32 << 20


def nvfp4kv_decode_attn_static(pool: Pool, layer: int, q: torch.Tensor, q_positions: torch.Tensor | None,
                               page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                               sm_scale: float, out: torch.Tensor, rope_cos: torch.Tensor | None = None,
                               rope_sin: torch.Tensor | None = None, pages_per_split: int = 0,
                               k_new: torch.Tensor | None = None, v_new: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    """nvfp4kv_decode_attn on the library's own static workspace: nothing is
    allocated, so `out` [n_seq][Hq][128] float32 must be given."""
    assert q.is_contiguous() and page_table.is_contiguous() and seq_lens.is_contiguous()
    _check_new(q, k_new, v_new)
    assert page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert out is not None and out.dtype == torch.float32 and out.is_contiguous()
    n_seq, n_q_heads, _ = q.shape
    assert tuple(out.shape) == (n_seq, n_q_heads, HEAD_DIM)
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    d = pool.desc()
    _check("nvfp4kv_decode_attn_static",
           _lib.nvfp4kv_decode_attn_static(ctypes.byref(d), layer, n_seq, n_q_heads, _ptr(q), _ptr(k_new),
                                           _ptr(v_new), _dtype_code(q), _ptr(q_positions), _ptr(rope_cos),
                                           _ptr(rope_sin), max_pos, _ptr(page_table), page_table.shape[1],
                                           _ptr(seq_lens), int(max_seq_len), float(sm_scale), _ptr(out),
                                           pages_per_split, _stream(stream)))
    return out


def nvfp4kv_decode_attn_splits(pool: Pool, layer: int, q: torch.Tensor,
                               q_positions: torch.Tensor | None, page_table: torch.Tensor,
                               seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                               workspace: torch.Tensor, rope_cos: torch.Tensor | None = None,
                               rope_sin: torch.Tensor | None = None, pages_per_split: int = 0,
                               k_new: torch.Tensor | None = None,
                               v_new: torch.Tensor | None = None, stream=None) -> None:
    """First stage of decode attention: split partials into `workspace` (and, with
    k_new/v_new, the current token into the cache)."""
    assert q.is_contiguous() and page_table.is_contiguous() and seq_lens.is_contiguous()
    _check_new(q, k_new, v_new)
    n_seq, n_q_heads, _ = q.shape
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    d = pool.desc()
    _check("nvfp4kv_decode_attn_splits",
           _lib.nvfp4kv_decode_attn_splits(ctypes.byref(d), layer, n_seq, n_q_heads, _ptr(q),
                                           _ptr(k_new), _ptr(v_new), _dtype_code(q), _ptr(q_positions), _ptr(rope_cos),
                                           _ptr(rope_sin), max_pos, _ptr(page_table),
                                           page_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                                           float(sm_scale), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           pages_per_split, _stream(stream)))


def nvfp4kv_decode_reduce(pool: Pool, n_seq: int, n_q_heads: int, seq_lens: torch.Tensor,
                          max_seq_len: int, out: torch.Tensor, workspace: torch.Tensor,
                          pages_per_split: int = 0, stream=None) -> torch.Tensor:
    """Second stage: combine the split partials into out [n_seq][n_q_heads][128]."""
    d = pool.desc()
    _check("nvfp4kv_decode_reduce",
           _lib.nvfp4kv_decode_reduce(ctypes.byref(d), n_seq, n_q_heads, _ptr(seq_lens),
                                      int(max_seq_len), _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), pages_per_split,
                                      _stream(stream)))
    return out


def nvfp4kv_decode_multi_workspace_bytes(pool: Pool, n_seq: int, n_qtok: int, n_q_heads: int,
                                         max_seq_len: int, pages_per_split: int = 0) -> int:
    d = pool.desc()
    return _lib.nvfp4kv_decode_multi_workspace_bytes(ctypes.byref(d), n_seq, n_qtok, n_q_heads,
                                                     max_seq_len, pages_per_split)


def nvfp4kv_decode_attn_multi(pool: Pool, layer: int, q: torch.Tensor, q_positions: torch.Tensor | None,
                              page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                              sm_scale: float, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None,
                              rope_cos: torch.Tensor | None = None, rope_sin: torch.Tensor | None = None,
                              pages_per_split: int = 0, stream=None) -> torch.Tensor:
    """Decode attention for several new query tokens per sequence, causal among
    them: q [n_seq][n_qtok][Hq][128] -> out [n_seq][n_qtok][Hq][128] float32.
    The n_qtok tokens must already be in the cache."""
    assert q.dim() == 4 and q.is_contiguous() and page_table.is_contiguous() and seq_lens.is_contiguous()
    assert page_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    n_seq, n_qtok, n_q_heads, _ = q.shape
    if out is None:
        out = _scratch(torch.empty((n_seq, n_qtok, n_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device),
                       stream)
    if workspace is None:
        need = nvfp4kv_decode_multi_workspace_bytes(pool, n_seq, n_qtok, n_q_heads, max_seq_len,
                                                    pages_per_split)
        workspace = _scratch(torch.empty(max(need, 256), dtype=torch.uint8, device=q.device), stream)
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    d = pool.desc()
    _check("nvfp4kv_decode_attn_multi",
           _lib.nvfp4kv_decode_attn_multi(ctypes.byref(d), layer, n_seq, n_qtok, n_q_heads, _ptr(q),
                                          _dtype_code(q), _ptr(q_positions), _ptr(rope_cos),
                                          _ptr(rope_sin), max_pos, _ptr(page_table), page_table.shape[1],
                                          _ptr(seq_lens), int(max_seq_len), float(sm_scale), _ptr(out),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          pages_per_split, _stream(stream)))
    return out


def nvfp4kv_dequant(pool: Pool, layer: int, slots: torch.Tensor, out_dtype=torch.float32,
                    unrotate: bool = False, want_k: bool = True, want_v: bool = True, stream=None):
    """Dequantized K-hat, V-hat [n_tok][Hkv][128] of the given slots."""
    assert slots.dtype == torch.int64 and slots.is_contiguous()
    n_tok = slots.shape[0]
    shape = (n_tok, pool.num_kv_heads, HEAD_DIM)
    k_out = _scratch(torch.empty(shape, dtype=out_dtype, device=slots.device), stream) if want_k else None
    v_out = _scratch(torch.empty(shape, dtype=out_dtype, device=slots.device), stream) if want_v else None
    code = F32 if out_dtype == torch.float32 else BF16
    d = pool.desc()
    _check("nvfp4kv_dequant",
           _lib.nvfp4kv_dequant(ctypes.byref(d), layer, n_tok, _ptr(slots), _ptr(k_out), _ptr(v_out),
                                code, int(unrotate), _stream(stream)))
    return k_out, v_out


def nvfp4kv_page_bytes(pool: Pool) -> int:
    d = pool.desc()
    return _lib.nvfp4kv_page_bytes(ctypes.byref(d))


def nvfp4kv_spill_pages(pool: Pool, page_ids: torch.Tensor, arena: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Copy whole pages (every layer and kv head) to arena [n][num_layers]
    [num_kv_heads][block bytes] uint8: pinned host memory by default, or the
    given pinned-host or device tensor.  page_ids: int32 on the device or
    pinned."""
    assert page_ids.dtype == torch.int32 and page_ids.is_contiguous()
    n = page_ids.numel()
    shape = (n, pool.num_layers, pool.num_kv_heads, pool.block_bytes)
    if arena is None:
        arena = torch.empty(shape, dtype=torch.uint8, pin_memory=True)
    assert arena.dtype == torch.uint8 and arena.is_contiguous()
    d = pool.desc()
    _check("nvfp4kv_spill_pages",
           _lib.nvfp4kv_spill_pages(ctypes.byref(d), n, _ptr(page_ids), _ptr(arena),
                                    arena.numel(), _stream(stream)))
    return arena


def nvfp4kv_stream_read(pool: Pool, layer: int, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        n_waves: int, words: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Read-bandwidth probe: read every block of `layer` that decode over these
    sequences reads, n_waves wavefronts; returns the [n_waves] int32 (uint32
    bits) XOR words."""
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.is_contiguous()
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous()
    if words is None:
        words = _scratch(torch.empty(n_waves, dtype=torch.int32, device=page_table.device), stream)
    d = pool.desc()
    _check("nvfp4kv_stream_read",
           _lib.nvfp4kv_stream_read(ctypes.byref(d), int(layer), seq_lens.numel(), _ptr(page_table),
                                    page_table.shape[1], _ptr(seq_lens), int(n_waves), _ptr(words),
                                    _stream(stream)))
    return words


def nvfp4kv_restore_pages(pool: Pool, page_ids: torch.Tensor, arena: torch.Tensor, stream=None) -> None:
    """Copy arena entry i back into page page_ids[i] of every layer and kv
    head; the ids must be distinct."""
    assert page_ids.dtype == torch.int32 and page_ids.is_contiguous()
    assert arena.dtype == torch.uint8 and arena.is_contiguous()
    d = pool.desc()
    _check("nvfp4kv_restore_pages",
           _lib.nvfp4kv_restore_pages(ctypes.byref(d), page_ids.numel(), _ptr(page_ids), _ptr(arena),
                                      arena.numel(), _stream(stream)))


def _host_i32(t) -> torch.Tensor:
    t = torch.as_tensor(t)
    assert t.device.type == "cpu", "the range checks take host (CPU) tables"
    return t.to(torch.int32).contiguous()


def nvfp4kv_check_decode_tables(pool: Pool, page_table, seq_lens, max_seq_len: int, q_positions=None,
                                max_pos: int = 0, n_qtok: int = 1, lib: ctypes.CDLL | None = None) -> None:
    """Range check of a decode call's page table, lengths and query positions
    on host copies (CPU tensors or arrays); raises NVFP4KVError naming the
    first offending index."""
    L = lib or _lib
    pt = _host_i32(page_table)
    sl = _host_i32(seq_lens)
    qp = _host_i32(q_positions) if q_positions is not None else None
    d = pool.desc()
    rc = L.nvfp4kv_check_decode_tables(ctypes.byref(d), sl.numel(), int(n_qtok), pt.data_ptr(), pt.shape[-1],
                                       sl.data_ptr(), int(max_seq_len), qp.data_ptr() if qp is not None else None,
                                       int(max_pos))
    if rc != OK:
        raise NVFP4KVError("nvfp4kv_check_decode_tables", rc, L.nvfp4kv_last_error().decode())


def nvfp4kv_check_slots(pool: Pool, slots, positions=None, max_pos: int = 0, lib: ctypes.CDLL | None = None) -> None:
    """Range and distinctness check of an append's slots (and positions) on host copies."""
    L = lib or _lib
    sl = torch.as_tensor(slots).to(torch.int64).contiguous()
    ps = _host_i32(positions) if positions is not None else None
    d = pool.desc()
    rc = L.nvfp4kv_check_slots(ctypes.byref(d), sl.numel(), sl.data_ptr(), ps.data_ptr() if ps is not None else None,
                               int(max_pos))
    if rc != OK:
        raise NVFP4KVError("nvfp4kv_check_slots", rc, L.nvfp4kv_last_error().decode())


def nvfp4kv_check_page_ids(pool: Pool, page_ids, distinct: bool, lib: ctypes.CDLL | None = None) -> None:
    L = lib or _lib
    ids = _host_i32(page_ids)
    d = pool.desc()
    rc = L.nvfp4kv_check_page_ids(ctypes.byref(d), ids.numel(), ids.data_ptr(), int(bool(distinct)))
    if rc != OK:
        raise NVFP4KVError("nvfp4kv_check_page_ids", rc, L.nvfp4kv_last_error().decode())


def nvfp4kv_checked_build(lib: ctypes.CDLL | None = None) -> bool:
    return bool((lib or _lib).nvfp4kv_checked_build())


def default_sm_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)
