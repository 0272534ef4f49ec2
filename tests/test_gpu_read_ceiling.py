"""Read-ceiling kernels (measurement aids): every word they are asked to read
is read exactly once, checked through the XOR of the sink against the XOR of
the words computed on the host; ids outside the buffer are skipped.  (Bad
arguments are rejected before any launch: tests/test_abi_host.py.)"""

import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _xor(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.view(np.uint32).ravel()))


@pytest.mark.parametrize("n_bytes,grid", [(16, 4), (1 << 20, 64), (3 * (1 << 20) + 48, 1024), (1 << 16, 7)])
def test_read_stream_reads_every_word_once(n_bytes, grid):
    import torch

    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(n_bytes)
    host = rng.integers(0, 2**32, size=n_bytes // 4, dtype=np.uint64).astype(np.uint32)
    gu.say("read_stream", n_bytes, "bytes, grid", grid)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = pkd.read_stream(buf, grid=grid)
    torch.cuda.synchronize()
    assert sink.numel() == grid * 512
    assert _xor(sink.cpu().numpy()) == _xor(host)


@pytest.mark.parametrize("page_bytes,grid", [(16, 3), (4096, 16), (65536, 16), (65536, 1024)])
def test_read_pages_reads_listed_pages_once(page_bytes, grid):
    import torch

    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(page_bytes)
    num_pages = 37
    host = rng.integers(0, 2**32, size=num_pages * page_bytes // 4,
                        dtype=np.uint64).astype(np.uint32)
    ids = rng.permutation(num_pages)[:29].astype(np.int32)
    # ids outside the buffer are skipped
    ids_dev = np.concatenate([ids[:10], [-1, num_pages, 1 << 30], ids[10:]]).astype(np.int32)
    gu.say("read_pages", page_bytes, "bytes per page,", ids_dev.size, "ids")
    base = torch.from_numpy(host.view(np.int32)).cuda()
    sink = pkd.read_pages(base, num_pages, page_bytes, torch.from_numpy(ids_dev).cuda(), grid=grid)
    torch.cuda.synchronize()
    pages = host.reshape(num_pages, page_bytes // 4)
    assert _xor(sink.cpu().numpy()) == _xor(pages[np.sort(ids)])
