"""The stream kernels behind the bench's HBM ceilings (emb_stream_copy, _fill,
_read): they move exactly the bytes they are given, including a ragged last
block, and touch nothing past them."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from recommender_embedding_tables_amd import embtab as eb  # noqa: E402

DEV = torch.device("cuda")
GUARD = 4096  # floats of guard band after the region


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 48, 1 << 20, (3 << 20) + 16 * 77])
def test_copy_and_fill_exact(nbytes):
    n = nbytes // 4
    src = torch.randn(n + GUARD, device=DEV)
    dst = torch.full((n + GUARD,), -7.0, device=DEV)
    eb.check(eb.emb_stream_copy(dst, src, nbytes), "copy")
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n])
    assert torch.all(dst[n:] == -7.0)
    eb.check(eb.emb_stream_fill(dst, 2.5, nbytes), "fill")
    torch.cuda.synchronize()
    assert torch.all(dst[:n] == 2.5)
    assert torch.all(dst[n:] == -7.0)


@pytest.mark.parametrize("nbytes", [16, 16384, 16384 + 16 * 5, (5 << 20) + 16 * 3])
def test_read_sums_every_word_once(nbytes):
    n = nbytes // 4
    # small integers: every partial sum is exact in fp32, whatever the order
    src = torch.from_numpy(np.random.default_rng(nbytes).integers(-8, 9, n + GUARD)
                           .astype(np.float32)).to(DEV)
    k = eb.emb_stream_read_sink_floats(nbytes)
    sink = torch.full((k + GUARD,), 1e9, device=DEV)
    eb.check(eb.emb_stream_read(src, nbytes, sink, k), "read")
    torch.cuda.synchronize()
    assert float(sink[:k].double().sum()) == float(src[:n].double().sum())
    assert torch.all(sink[k:] == 1e9)


def test_stream_argument_checks():
    x = torch.empty(1024, device=DEV)
    assert eb.emb_stream_copy(x, x[1:], 64) == eb.EMB_ERR_INVALID_ARG  # misaligned
    assert eb.emb_stream_fill(x, 0.0, 20) == eb.EMB_ERR_INVALID_ARG    # not a multiple of 16
    k = eb.emb_stream_read_sink_floats(4096)
    assert eb.emb_stream_read(x, 4096, x, k - 1) == eb.EMB_ERR_INVALID_ARG  # short sink
    assert eb.emb_stream_copy(x, x, 0) == eb.EMB_OK  # nothing to do
