"""The yardsticks of include/swan_measure.h on the GPU: the streaming read
reads every 16-byte unit of the buffer exactly once, whatever the grid, and
the fp64 matrix-core rate kernel runs every product it is asked for."""
import numpy as np
import pytest
import torch

from decode_attention_compressed_02_amd import swan as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("words,waves", [(4 * 250007, 1), (4 * 250007, 7), (4 * 250007, 1024), (4, 3), (4096, 4096)])
def test_stream_read_folds_every_word(words, waves):
    g = torch.Generator().manual_seed(words + waves)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    sink = torch.full((waves * 64,), 7, dtype=torch.int32, device="cuda")
    S.swan_measure_stream_read(buf, waves, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("waves,iters", [(1, 4), (3, 8), (256, 64)])
def test_mfma_f64_runs_every_product(waves, iters):
    # with A = B = x every 16x16x4 product adds 4 x^2 to each accumulator
    # element; a lane holds 4 elements of each of 8 accumulators
    sink = torch.full((waves * 64 + 64,), -1.0, dtype=torch.float64, device="cuda")
    S.swan_measure_mfma_f64(1.0, waves, iters, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert (got[:waves * 64] == 128.0 * iters).all()
    assert (got[waves * 64:] == -1.0).all()  # nothing written past the waves' slots
    S.swan_measure_mfma_f64(0.5, waves, iters, sink)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy()[:waves * 64] == 32.0 * iters).all()
