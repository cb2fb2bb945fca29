"""The streaming-read measurement hook reads every 16-byte piece of its buffer exactly once: the XOR
of all words it reports equals the XOR of the buffer's words, for sizes with ragged tails and grids
from one workgroup up."""
import numpy as np
import pytest
import torch

import block_sparse_kv_plan_amd as bsk
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096 + 16, 7), (1 << 20, 2048), ((64 << 20) + 48, 2048),
                                         ((64 << 20) + 48, 3)])
def test_stream_read_reads_every_word_once(nbytes, grid):
    dev = require_gpu()
    rng = np.random.default_rng(nbytes % 1000 + grid)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.full((grid * 256,), -1, dtype=torch.int32, device=dev)
    say(f"stream read: {nbytes} bytes, grid {grid}")
    bsk.debug_stream_read(src, sink, grid, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
