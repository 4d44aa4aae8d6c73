"""Pins of the oracle's unquantized reference attention (reference_attention,
orc_reference_attention): the attention that the NVFP4 cache's error is
reported against.

RoPE follows the release post of the gzenz/ninfer fork, section "YaRN
context extension" (rotary part of the head, theta 1e7, linear position
scaling); attention is plain softmax attention with grouped query heads.

The reference is re-derived here in NumPy from its definition: RoPE on q at
the query's position and on every key at that key's own position, applied in
binary32 with one rounding per product and sum (NumPy float32 arithmetic does
exactly that), then fp64 scores, softmax and the weighted sum of V, query head
h reading kv head h // (hq / hkv).  Two mutated copies of the oracle source
(keys rotated at the query's position; query head h reading kv head h % hkv)
are built and must fail the same comparison, so the comparison is shown to
see both mistakes."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

D = 128


def _rope_f32(x, pos, rotary_dim, cos_tab, sin_tab):
    """Rotate-half RoPE on the first rotary_dim dims of float32 rows x[..., 128],
    row i at position pos[i]: x'[j] = x[j] c - x[j+R/2] s, x'[j+R/2] =
    x[j+R/2] c + x[j] s, every product and sum rounded to binary32."""
    x = np.array(x, np.float32, copy=True)
    half = rotary_dim // 2
    if half == 0:
        return x
    c = cos_tab[pos][..., None, :] if x.ndim == 3 else cos_tab[pos]
    s = sin_tab[pos][..., None, :] if x.ndim == 3 else sin_tab[pos]
    a = x[..., :half].copy()
    b = x[..., half:2 * half].copy()
    x[..., :half] = (a * c) - (b * s)
    x[..., half:2 * half] = (b * c) + (a * s)
    return x


def _numpy_reference(q, q_pos, k, v, k_pos, rotary_dim, sm_scale, cos_tab, sin_tab):
    hq = q.shape[0]
    T, hkv, _ = k.shape
    grp = hq // hkv
    qr = _rope_f32(q, np.full(hq, q_pos), rotary_dim, cos_tab, sin_tab).astype(np.float64)
    kr = _rope_f32(k, np.asarray(k_pos), rotary_dim, cos_tab, sin_tab).astype(np.float64)
    out = np.zeros((hq, D))
    for h in range(hq):
        g = h // grp
        z = sm_scale * (kr[:, g, :] @ qr[h])
        p = np.exp(z - z.max())
        out[h] = (p[:, None] * v[:, g, :].astype(np.float64)).sum(0) / p.sum()
    return out


def _inputs(seed=0, T=300, hq=24, hkv=4, rotary_dim=32, pos_scale=2.3, q_pos=None):
    rng = np.random.default_rng(seed)
    mult = np.ones(D, np.float32)
    mult[rng.integers(0, rotary_dim if rotary_dim else D)] = 16.0   # one outlier channel, in the rotary part
    q = (rng.standard_normal((hq, D)) * mult).astype(np.float32)
    k = (rng.standard_normal((T, hkv, D)) * mult).astype(np.float32)
    v = (rng.standard_normal((T, hkv, D)) * mult).astype(np.float32)
    q_pos = T + 5 if q_pos is None else q_pos
    k_pos = np.arange(T, dtype=np.int32)
    c, s = oracle.rope_table(1e7, rotary_dim, pos_scale, q_pos + 2000)
    return q, q_pos, k, v, k_pos, c, s


def _max_rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def test_reference_matches_numpy_rederivation():
    """RoPE 32 with linear scaling 2.3, keys at their own positions, 24 query
    / 4 kv heads, one outlier channel: the oracle equals the re-derivation to
    fp64 rounding (the binary32 RoPE steps are identical on both sides)."""
    q, q_pos, k, v, k_pos, c, s = _inputs()
    sm = 1.0 / np.sqrt(D)
    got = oracle.reference_attention(q, q_pos, k, v, k_pos, 32, sm, c, s)
    want = _numpy_reference(q, q_pos, k, v, k_pos, 32, sm, c, s)
    assert _max_rel(got, want) <= 1e-9


@pytest.mark.parametrize("rotary_dim", [0, 16, 128])
def test_reference_matches_numpy_other_rotary_widths(rotary_dim):
    q, q_pos, k, v, k_pos, c, s = _inputs(seed=rotary_dim + 1, T=130, hq=6, hkv=2, rotary_dim=rotary_dim)
    sm = 1.0 / np.sqrt(D)
    got = oracle.reference_attention(q, q_pos, k, v, k_pos, rotary_dim, sm, c, s)
    want = _numpy_reference(q, q_pos, k, v, k_pos, rotary_dim, sm, c, s)
    assert _max_rel(got, want) <= 1e-9


def test_reference_depends_only_on_relative_positions():
    """Moving the query and every key by the same offset leaves attention
    unchanged up to the binary32 rounding of the table and of the rotation
    (the scores move by ~1e-6 relative); a query moved alone changes it."""
    q, q_pos, k, v, k_pos, c, s = _inputs(seed=3)
    sm = 1.0 / np.sqrt(D)
    base = oracle.reference_attention(q, q_pos, k, v, k_pos, 32, sm, c, s)
    shifted = oracle.reference_attention(q, q_pos + 1500, k, v, k_pos + 1500, 32, sm, c, s)
    assert _max_rel(shifted, base) <= 2e-5
    moved = oracle.reference_attention(q, q_pos + 1500, k, v, k_pos, 32, sm, c, s)
    assert _max_rel(moved, base) > 1e-2


# -- the comparison above must catch plausible mistakes: mutated copies -------
_MUTATIONS = {
    # keys rotated at the query's position instead of their own
    "keys_at_query_position": [
        ("cos_tab + (size_t)k_pos[t] * half", "cos_tab + (size_t)q_pos * half"),
        ("sin_tab + (size_t)k_pos[t] * half", "sin_tab + (size_t)q_pos * half"),
    ],
    # query head h reading kv head h % hkv instead of h / (hq / hkv)
    "head_mapping_modulo": [
        ("int g = h / grp;", "int g = h % hkv;"),
    ],
}


def _build_mutant(tmp, name):
    src = open(oracle.SRC).read()
    start = src.index("void orc_reference_attention(")
    head, body = src[:start], src[start:]
    for old, new in _MUTATIONS[name]:
        assert body.count(old) == 1, f"mutation pattern not found once: {old!r}"
        body = body.replace(old, new)
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(head + body)
    so = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", so, path, "-lm"], check=True)
    L = ctypes.CDLL(so)
    P = ctypes.c_void_p
    L.orc_reference_attention.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                                          ctypes.c_int32, P, P, P, P, P, ctypes.c_double, P]
    return L


def _call(L, q, q_pos, k, v, k_pos, rotary_dim, sm, c, s):
    def p(a):
        return a.ctypes.data_as(ctypes.c_void_p)
    q, k, v = (np.ascontiguousarray(a, np.float32) for a in (q, k, v))
    c, s = np.ascontiguousarray(c, np.float32), np.ascontiguousarray(s, np.float32)
    kp = np.ascontiguousarray(k_pos, np.int32)
    out = np.zeros((q.shape[0], D))
    L.orc_reference_attention(k.shape[1], q.shape[0], k.shape[0], rotary_dim, p(q), int(q_pos), p(k), p(v),
                              p(kp), p(c), p(s), float(sm), p(out))
    return out


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_rederivation_catches_mutated_oracle(name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    q, q_pos, k, v, k_pos, c, s = _inputs()
    sm = 1.0 / np.sqrt(D)
    want = _numpy_reference(q, q_pos, k, v, k_pos, 32, sm, c, s)
    with tempfile.TemporaryDirectory() as tmp:
        L = _build_mutant(tmp, name)
        got = _call(L, q, q_pos, k, v, k_pos, 32, sm, c, s)
    assert _max_rel(got, want) > 1e-3, f"mutation {name} was not detected"
