"""The streaming-read yardstick (include/swan_measure.h) on the GPU: it reads
every 16-byte unit of the buffer exactly once, whatever the grid."""
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
