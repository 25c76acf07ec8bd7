"""GPU check of the page-read measurement kernel: it reads exactly the listed
pages, each once per wave chunk (the XOR each wave stores equals the XOR of
the 32-bit words of its pages, computed on the host)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import paged_kv_cache_183_amd as P  # noqa: E402


@pytest.mark.parametrize("page_bytes,pages,listed,waves", [(4096, 300, 1000, 64), (2048, 50, 37, 8),
                                                          (1024, 9, 9, 64), (4096, 4, 4096, 4)])
def test_read_pages_xor(page_bytes, pages, listed, waves):
    g = torch.Generator().manual_seed(page_bytes + listed)
    buf = torch.randint(0, 256, (pages * page_bytes,), dtype=torch.uint8, generator=g)
    ids = torch.randint(0, pages, (listed,), dtype=torch.int32, generator=g)
    ids[::17] = pages + 5                     # outside the buffer: page 0
    sink = torch.full((waves,), -1, dtype=torch.int32, device="cuda")
    P.vllm_paged_read_pages(buf.cuda(), ids.cuda(), page_bytes, sink)
    words = buf.numpy().view(np.uint32).reshape(pages, page_bytes // 4)
    page_xor = np.bitwise_xor.reduce(words, axis=1)
    eff = np.where(ids.numpy() < pages, ids.numpy(), 0)
    per = -(-listed // waves)
    want = np.zeros(waves, np.uint32)
    for w in range(waves):
        sel = eff[w * per:(w + 1) * per]
        if sel.size:
            want[w] = np.bitwise_xor.reduce(page_xor[sel])
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
