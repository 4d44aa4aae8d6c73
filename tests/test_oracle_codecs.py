"""Pins of the oracle's NVFP4 codecs (E4M3 scales, E2M1 elements) to things
other than the oracle itself: PyTorch's float8_e4m3fn conversion, exact
fractions, the format's closed-form values and brute force.

Format source: release post of the gzenz/ninfer fork, section "NVFP4 KV cache
(from scratch)", bullet 1 (E2M1 values with E4M3 block scales)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]


def test_e4m3_landmarks():
    # closed-form values of the OCP E4M3FN encoding
    assert oracle.e4m3_value(0x00) == 0.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6          # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0              # largest finite
    assert np.isnan(oracle.e4m3_value(0x7F))
    assert np.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0xB8) == -1.0


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert (mine[~nan] == ref[~nan]).all()


def test_e4m3_finite_values_increasing():
    vals = [oracle.e4m3_value(c) for c in range(127)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert len(set(vals)) == 127


def _torch_scale_code(amax: np.ndarray) -> np.ndarray:
    """RNE of fl32(amax/6) to float8_e4m3fn via PyTorch, saturated at 448."""
    x = torch.from_numpy((amax.astype(np.float32) / np.float32(6.0)).astype(np.float32))
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    codes[x.numpy() > 448.0] = 0x7E     # PyTorch gives NaN past the top; the method saturates
    return codes


def test_e4m3_scale_code_matches_torch_dense_sweep():
    rng = np.random.default_rng(11)
    amax = np.concatenate([
        np.exp(rng.uniform(np.log(1e-6), np.log(4000.0), 20000)),
        rng.uniform(0, 12, 5000),
        np.array([0.0, 6 * 448.0, 6 * 448.0 * 1.5, 6 * 2.0 ** -10, 6 * 2.0 ** -9]),
    ]).astype(np.float32)
    ref = _torch_scale_code(amax)
    mine = np.array([oracle.e4m3_scale_code(a) for a in amax])
    bad = np.nonzero(ref != mine)[0]
    assert bad.size == 0, [(float(amax[i]), int(ref[i]), int(mine[i])) for i in bad[:5]]


def test_e4m3_scale_ties_go_to_even_code():
    # amax = 6 * midpoint of two neighbouring codes is exactly representable,
    # and amax/6 sits exactly on the tie.
    for c in range(0, 126):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        amax = np.float32(6 * mid)
        assert float(amax) == 6 * mid
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_scale_code(amax) == want, c
        # one float step either side leaves the tie
        below = np.nextafter(amax, np.float32(0))
        above = np.nextafter(amax, np.float32(np.inf))
        assert oracle.e4m3_scale_code(below) == c
        assert oracle.e4m3_scale_code(above) == c + 1


def test_e4m3_scale_saturates():
    assert oracle.e4m3_scale_code(6 * 448.0) == 0x7E
    assert oracle.e4m3_scale_code(6 * 470.0) == 0x7E
    assert oracle.e4m3_scale_code(3.0e38) == 0x7E
    assert oracle.e4m3_scale_code(0.0) == 0


def test_e2m1_values():
    want = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for c in range(8):
        assert oracle.e2m1_value(c) == want[c]
        assert oracle.e2m1_value(c | 8) == -want[c]


def _nearest_even(r: Fraction) -> int:
    """Brute force on exact fractions: nearest E2M1 magnitude, ties to even code."""
    dists = [abs(r - m) for m in E2M1_MAG]
    best = min(dists)
    cands = [c for c, d in enumerate(dists) if d == best]
    if len(cands) == 1:
        return cands[0]
    return [c for c in cands if c % 2 == 0][0]


def test_e2m1_code_exact_fraction_grid():
    # every multiple of 1/64 in [0, 8] with unit scale, and with a few scales
    for s in (1.0, 0.5, 0.375, 2.0 ** -9, 3 * 2.0 ** -9, 448.0, 1.75 * 2 ** 5):
        sf = Fraction(s)
        for k in range(0, 8 * 64 + 1):
            r = Fraction(k, 64)
            y = r * sf
            yf = float(y)
            if Fraction(np.float32(yf).item()) != y:
                continue                      # skip grid points a float cannot hold
            want = _nearest_even(r)
            assert oracle.e2m1_code(yf, s) == want, (s, k)
            assert oracle.e2m1_code(-yf, s) == want | 8, (s, k)


def test_e2m1_tie_table():
    # the seven decision points of round-to-nearest-even on the E2M1 grid
    assert [oracle.e2m1_code(r, 1.0) for r in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == \
        [0, 2, 2, 4, 4, 6, 6]
    assert oracle.e2m1_code(100.0, 1.0) == 7            # saturates at 6
    # far beyond the grid every distance to v*s rounds to the same double;
    # the nearest value is still 6*s
    assert oracle.e2m1_code(1e35, 448.0) == 7
    assert oracle.e2m1_code(-3e38, 2.0 ** -9) == 15
    assert oracle.e2m1_code(6.0 * 448.0, 448.0) == 7
    assert oracle.e2m1_code(1.0, 0.0) == 0              # zero scale gives magnitude 0
    assert oracle.e2m1_code(-1.0, 0.0) == 8
    assert oracle.e2m1_code(-0.0, 1.0) == 8             # sign bit kept on zero


def test_quant_row_round_trip_of_representable_blocks():
    """A row built from E2M1 x E4M3 values, each block holding a +-6*s entry,
    quantizes back to the same codes and scales."""
    rng = np.random.default_rng(5)
    for trial in range(200):
        scodes = rng.integers(8, 0x7E, size=8)          # normal-range scales
        nib = rng.integers(0, 16, size=128)
        for b in range(8):
            nib[16 * b + rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
        x = np.array([oracle.e2m1_value(nib[d]) * oracle.e4m3_value(scodes[d // 16])
                      for d in range(128)], np.float32)
        codes, scales = oracle.quant_row(x)
        assert (scales == scodes).all(), trial
        back = np.array([(codes[d // 2] >> (4 * (d % 2))) & 15 for d in range(128)])
        # a value of +-0 may come back as the other signed zero only if it was -0 -> sign kept
        assert (back == nib).all(), trial


def test_quant_row_error_bound():
    """Each element lands within half a grid step of s (6 -> 4 step is 2),
    unless the block saturated; the scale is the nearest E4M3 to amax/6."""
    rng = np.random.default_rng(6)
    for _ in range(200):
        x = (rng.standard_normal(128) * np.exp(rng.uniform(-6, 6))).astype(np.float32)
        codes, scales = oracle.quant_row(x)
        xh = oracle.dequant_row(codes, scales)
        for b in range(8):
            s = oracle.e4m3_value(scales[b])
            blk = x[16 * b:16 * b + 16].astype(np.float64)
            err = np.abs(blk - xh[16 * b:16 * b + 16])
            amax = np.abs(blk).max()
            # elements at most 6*s: error at most half the widest gap (1*s)
            inside = np.abs(blk) <= 6 * s
            assert (err[inside] <= 1.0 * s + 1e-30).all()
            # saturated elements only exceed 6 s by the scale's own rounding
            assert (np.abs(blk[~inside]) <= amax).all()
            assert abs(amax / 6 - s) <= s / 16 + 2.0 ** -10


def test_byte_count_matches_pages():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_byte_counts.json")) as f:
        g = json.load(f)
    per_tok = oracle.pool_bytes(3, 5, 4) / (3 * 5 * 4 * 64)
    assert per_tok == g["bytes_per_token_per_kv_head"]["nvfp4"]
    d = g["head_dim"]
    assert 2 * (d // 2 + d // 16) == 144                 # codes + one scale per 16
    assert 2 * (d + 4) == g["bytes_per_token_per_kv_head"]["int8"]
    assert 2 * d * 2 == g["bytes_per_token_per_kv_head"]["bf16"]
    red = 100 * (1 - per_tok / g["bytes_per_token_per_kv_head"]["int8"])
    assert round(red) == g["vram_reduction_percent"]
