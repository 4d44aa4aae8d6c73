"""Pins of the oracle's Hadamard rotation and RoPE.

Hadamard: release post of the gzenz/ninfer fork, section "NVFP4 KV cache
(from scratch)", bullet 2 (K and Q rotated before quantization, V not).
RoPE: same post, section "YaRN context extension" (theta 1e7, a quarter of
the dims rotary, linear position scaling)."""
import numpy as np
import scipy.linalg

import oracle

H = scipy.linalg.hadamard(128).astype(np.float64)


def test_hadamard_equals_sylvester_matrix_product():
    rng = np.random.default_rng(1)
    for _ in range(50):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        y = oracle.hadamard128(x).astype(np.float64)
        ref = H @ x.astype(np.float64) / np.sqrt(128.0)
        # 7 binary32 add stages and one multiply: error below 8 ulps of the l2 norm
        assert np.abs(y - ref).max() <= 8 * 2.0 ** -24 * np.abs(x).sum()


def test_hadamard_matrix_orthonormal_symmetric_and_sign_pattern():
    cols = np.stack([oracle.hadamard128(np.eye(128, dtype=np.float32)[j]) for j in range(128)], 1)
    cols = cols.astype(np.float64)
    # the sign pattern is exactly Sylvester's
    assert (np.sign(cols) == H).all()
    # symmetric, and every entry is the float nearest 1/sqrt(128)
    assert (cols == cols.T).all()
    assert (np.abs(cols) == np.float64(np.float32(2 ** -3.5))).all()
    # H H^T = I up to the rounding of 1/sqrt(128) to float
    err = np.abs(cols @ cols.T - np.eye(128)).max()
    assert err <= 128 * 2 ** -24


def test_hadamard_involution_and_outlier_spreading():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128).astype(np.float32)
    xx = oracle.hadamard128(oracle.hadamard128(x))
    assert np.abs(xx - x).max() <= 1e-5 * np.abs(x).max() + 1e-6
    e = np.zeros(128, np.float32)
    e[37] = 20.0
    y = oracle.hadamard128(e)
    assert np.allclose(np.abs(y), 20 / np.sqrt(128), rtol=1e-6)


def test_rotation_preserves_dot_products():
    rng = np.random.default_rng(3)
    for _ in range(50):
        q = rng.standard_normal(128).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        k[[3, 50, 90]] *= 16
        a = float(np.dot(oracle.hadamard128(q).astype(np.float64), oracle.hadamard128(k).astype(np.float64)))
        b = float(np.dot(q.astype(np.float64), k.astype(np.float64)))
        assert abs(a - b) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)


def test_rope_table_angles_follow_closed_form():
    theta, R = 1e7, 32
    for scale in (1.0, 2.3):
        c, s = oracle.rope_table(theta, R, scale, 4096)
        assert c.shape == (4096, 16)
        # position 0 is the identity rotation exactly
        assert (c[0] == 1.0).all() and (s[0] == 0.0).all()
        # the angle of pair i grows linearly in pos at rate theta^(-2i/R)/scale
        pos = np.array([1, 2, 3, 7, 100])
        for i in range(16):
            rate = theta ** (-2.0 * i / R) / scale
            ang = np.arctan2(s[pos, i].astype(np.float64), c[pos, i].astype(np.float64))
            want = np.angle(np.exp(1j * pos * rate))     # wrapped to (-pi, pi]
            assert np.abs(ang - want).max() < 1e-6
        assert np.abs(c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2 - 1).max() < 1e-6


def test_rope_linear_scaling_is_position_interpolation():
    # with scale f = 2, position 2p uses exactly the angles of position p at f = 1
    c1, s1 = oracle.rope_table(1e7, 32, 1.0, 600)
    c2, s2 = oracle.rope_table(1e7, 32, 2.0, 1200)
    assert (c2[0::2] == c1).all() and (s2[0::2] == s1).all()


def test_rope_relative_position_property():
    """RoPE(q, m) . RoPE(k, n) depends only on m - n (up to float rounding)."""
    rng = np.random.default_rng(4)
    R = 32
    c, s = oracle.rope_table(1e7, R, 1.0, 5000)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)

    def dot(m, n):
        a = oracle.rope_apply(q, R, c[m], s[m]).astype(np.float64)
        b = oracle.rope_apply(k, R, c[n], s[n]).astype(np.float64)
        return float(a @ b)

    for delta in (0, 1, 5, 63, 700):
        vals = [dot(m + delta, m) for m in (0, 17, 1000, 4000)]
        assert max(vals) - min(vals) <= 1e-4 * np.linalg.norm(q) * np.linalg.norm(k)


def test_rope_rotates_half_pairs_and_leaves_the_rest():
    R = 32
    c, s = oracle.rope_table(1e7, R, 1.0, 100)
    rng = np.random.default_rng(8)
    x = rng.standard_normal(128).astype(np.float32)
    y = oracle.rope_apply(x, R, c[77], s[77])
    assert (y[R:] == x[R:]).all()
    # each pair (i, i + R/2) keeps its length: it is a plane rotation
    for i in range(R // 2):
        n0 = np.hypot(float(x[i]), float(x[i + R // 2]))
        n1 = np.hypot(float(y[i]), float(y[i + R // 2]))
        assert abs(n0 - n1) <= 1e-6 * max(n0, 1e-30) + 1e-7
    # a unit vector on dim i comes out as (cos, sin) of pair i at (i, i + R/2)
    e = np.zeros(128, np.float32)
    e[5] = 1.0
    y = oracle.rope_apply(e, R, c[77], s[77])
    assert y[5] == c[77, 5] and y[5 + 16] == s[77, 5]
    assert np.count_nonzero(y) == 2


# -- randomized rotation (a variant, not the release post's): negate the
#    elements whose bit is set in a 128-bit mask, then the Hadamard rotation.
def _mask_signs(mask):
    """+-1 per element from the documented convention: element j's bit is
    bit j % 32 of word j // 32."""
    return np.array([-1.0 if (int(mask[j // 32]) >> (j % 32)) & 1 else 1.0 for j in range(128)], np.float32)


def test_random_sign_rotation_is_rotation_of_negated_row():
    rng = np.random.default_rng(70)
    for _ in range(20):
        x = (rng.standard_normal(128) * rng.choice([1, 30], 128)).astype(np.float32)
        mask = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
        got = oracle.quant_row(x, hadamard=2, signs=mask)
        want = oracle.quant_row(x * _mask_signs(mask), hadamard=1)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_random_sign_special_masks():
    """An empty mask is the plain rotation; a full mask negates the rotated
    row, which flips the sign bit of every code (0x88 per byte) and keeps
    every scale."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal(128).astype(np.float32)
    plain = oracle.quant_row(x, hadamard=1)
    zero = oracle.quant_row(x, hadamard=2, signs=np.zeros(4, np.uint32))
    full = oracle.quant_row(x, hadamard=2, signs=np.full(4, 0xFFFFFFFF, np.uint32))
    assert np.array_equal(zero[0], plain[0]) and np.array_equal(zero[1], plain[1])
    assert np.array_equal(full[0], plain[0] ^ 0x88) and np.array_equal(full[1], plain[1])


def test_random_sign_rotation_preserves_dot_products():
    """(H D q) . (H D k) = q . k for D = diag(+-1): checked in fp64 with the
    explicit Sylvester matrix."""
    rng = np.random.default_rng(72)
    idx = np.arange(128)
    H = np.where(np.array([[bin(i & j).count("1") % 2 for j in idx] for i in idx]) == 1, -1.0, 1.0) / np.sqrt(128)
    for _ in range(10):
        d = _mask_signs(rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)).astype(np.float64)
        q, k = rng.standard_normal(128), rng.standard_normal(128)
        assert abs((H @ (d * q)) @ (H @ (d * k)) - q @ k) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
