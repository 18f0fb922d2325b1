"""Host checks of two integer decodings the interaction kernels take in fp32
arithmetic, over every value the kernels can meet (no GPU needed):

  * table = item // (D / 4) for a flat item index below 2048 and D / 4 up to
    64, as (int)(((float)item + 0.5f) * (1.0f / (D / 4))): the quotient of
    item + 1/2 lies at least 1/128 from an integer, so fp32 rounding of the
    reciprocal and of the product cannot move it across one;
  * the pair (i, j), i > j, at position p = i (i - 1) / 2 + j of the strict
    lower triangle, as i = (int)((1 + sqrt(8 p + 1)) / 2) corrected by at most
    one step each way: checked with the square root correctly rounded and one
    ulp off either way, and against numpy's tril_indices order."""
import numpy as np


def test_item_table_quotient_in_fp32():
    items = np.arange(2048, dtype=np.int64)
    for d4 in range(1, 65):
        rd4 = np.float32(1.0) / np.float32(d4)
        q = ((items.astype(np.float32) + np.float32(0.5)) * rd4).astype(np.float32)
        t = np.trunc(q).astype(np.int64)
        np.testing.assert_array_equal(t, items // d4, err_msg=f"D/4 = {d4}")
        np.testing.assert_array_equal(items - t * d4, items % d4)


def _pair_of(p, sqrt_ulps):
    x = np.float32(8 * p + 1)
    r = np.sqrt(x, dtype=np.float32)
    for _ in range(abs(sqrt_ulps)):
        r = np.nextafter(r, np.float32(np.inf if sqrt_ulps > 0 else -np.inf), dtype=np.float32)
    i = int(np.float32((np.float32(1.0) + r) * np.float32(0.5)))
    if i * (i - 1) // 2 > p:
        i -= 1
    elif (i + 1) * i // 2 <= p:
        i += 1
    return i, p - i * (i - 1) // 2


def test_pair_index_inversion():
    for n in (2, 9, 17, 27, 32):  # T + 1 rows
        li, lj = np.tril_indices(n, -1)
        for p in range(len(li)):
            for ulps in (-1, 0, 1):
                assert _pair_of(p, ulps) == (li[p], lj[p]), (n, p, ulps)
