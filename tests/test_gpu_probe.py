"""GPU check of the streaming-read probe (kvc_stream_read) the benchmark uses
for the HBM read ceiling: every 32-bit word of the buffer is read exactly once
(the workgroups' wrapping sums add up to the sum of all words), for sizes that
do and do not fill the grid evenly, and an empty buffer reads nothing."""
import numpy as np
import pytest
import torch

from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


@pytest.mark.parametrize("n_words", [4, 4 * 7, 4 * 4096 * 256, 4 * (4096 * 256 * 5 + 13),
                                     4 * 3_000_017])
def test_stream_read_reads_every_word_once(kvc, n_words):
    say(f"stream read probe over {n_words * 4} bytes")
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 32, n_words, dtype=np.uint64).astype(np.uint32)
    data = torch.from_numpy(host.view(np.int32)).cuda()
    out = kvc.stream_read(data)
    torch.cuda.synchronize()
    got = int(out.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % 2 ** 32)
    want = int(host.astype(np.uint64).sum() % 2 ** 32)
    assert got == want


def test_stream_read_empty_and_rejects(kvc):
    out = kvc.stream_read(torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0
    with pytest.raises(kvc.KvcError):
        kvc.stream_read(torch.empty(5, dtype=torch.int8, device="cuda"))   # not a multiple of 16
