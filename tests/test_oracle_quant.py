"""Pins of the oracle's int8 exchange payload (OneFlow OneEmbedding page,
section "quantized compression": embeddings are quantized from float to int8
before the ranks exchange them and dequantized after; the page gives no
scheme, the reading is one symmetric fp32 scale per row, codes in
[-127, 127], round to nearest with ties to even).  Pinned by hand-worked rows
whose fp32 arithmetic is exact (ties included), and by properties that a wrong
rounding, scale or clamp breaks: the largest element maps to +-127, the
dequantized row is within half a step of the input, codes are odd in x, and a
power-of-two factor moves only the scale."""
import numpy as np
import pytest

from oracle import oracle as orc


def test_hand_worked_rows():
    x = np.array([[1.0, -0.5, 0.25, 0.0, -1.0],        # amax 1: inv = 127
                  [2.0, -1.0, 0.5, -0.25, 0.75],        # amax 2: inv = 63.5
                  [0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    codes, scales = orc.quantize_rows_int8(x)
    # -0.5 * 127 = -63.5 -> -64 (tie to even); 0.25 * 127 = 31.75 -> 32;
    # 63.5 * [2, -1, .5, -.25, .75] = [127, -63.5, 31.75, -15.875, 47.625]
    np.testing.assert_array_equal(codes, [[127, -64, 32, 0, -127],
                                          [127, -64, 32, -16, 48],
                                          [0, 0, 0, 0, 0]])
    np.testing.assert_array_equal(scales, np.array([1.0 / 127, 2.0 / 127, 0.0], np.float32))
    y = orc.dequantize_rows_int8(codes, scales)
    np.testing.assert_array_equal(y[0], np.float32(1.0 / 127) * codes[0].astype(np.float32))
    np.testing.assert_array_equal(y[2], 0.0)


def test_ties_go_to_even():
    # amax 127: inv = 1, so the codes are the inputs rounded: halves to even
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]], np.float32)
    codes, scales = orc.quantize_rows_int8(x)
    np.testing.assert_array_equal(codes[0], [127, 0, 2, 2, 0, -2, -2, 4])
    assert scales[0] == np.float32(1.0)


def _rows(seed, n=400, D=64):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, D)) * np.exp(rng.uniform(-8, 8, (n, 1)))).astype(np.float32)
    x[::17] = 0.0  # zero rows
    x[5, :] = -3.0  # constant row
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_properties(seed):
    x = _rows(seed)
    codes, scales = orc.quantize_rows_int8(x)
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    # the largest element of a nonzero row maps to +-127; a zero row to 0
    np.testing.assert_array_equal(np.abs(codes[nz].astype(np.int32)).max(axis=1), 127)
    assert np.all(codes[~nz] == 0) and np.all(scales[~nz] == 0)
    np.testing.assert_allclose(scales[nz], amax[nz] / 127, rtol=2 ** -23)
    # within half a step (plus fp32 rounding of the product and of the dequantized value)
    y = orc.dequantize_rows_int8(codes, scales)
    err = np.abs(y.astype(np.float64) - x.astype(np.float64))
    bound = scales[:, None].astype(np.float64) * (0.5 + 1e-5) + np.abs(x) * 2.0 ** -22
    assert np.all(err <= bound)
    # odd in x
    cn, sn = orc.quantize_rows_int8(-x)
    np.testing.assert_array_equal(cn, -codes)
    np.testing.assert_array_equal(sn, scales)
    # a power-of-two factor is exact in fp32: same codes, scaled scale
    for k in (-3, 5):
        ck, sk = orc.quantize_rows_int8(x * np.float32(2.0 ** k))
        np.testing.assert_array_equal(ck, codes)
        np.testing.assert_array_equal(sk, scales * np.float32(2.0 ** k))


def test_empty_and_single_column():
    codes, scales = orc.quantize_rows_int8(np.zeros((0, 8), np.float32))
    assert codes.shape == (0, 8) and scales.shape == (0,)
    codes, scales = orc.quantize_rows_int8(np.array([[-0.3], [0.0], [7.0]], np.float32))
    np.testing.assert_array_equal(codes[:, 0], [-127, 0, 127])
