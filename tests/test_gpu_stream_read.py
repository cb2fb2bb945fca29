"""The read measurement hooks read exactly what they say.  The streaming read covers every 16-byte
piece of its buffer once: the XOR of all words it reports equals the XOR of the buffer's words, for
sizes with ragged tails and grids from one workgroup up.  The block read covers the 4 KB blocks its
order lists (indices outside the buffer clamped to it), each once per listing: the XOR it reports
equals the XOR, over the listed blocks, of each block's words."""
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


@pytest.mark.parametrize("n_buf,order_kind,grid", [(256, "perm", 1), (256, "perm", 3), (4096, "perm", 512),
                                                    (4096, "short", 768), (64, "clamped", 5)])
def test_block_read_reads_the_listed_blocks(n_buf, order_kind, grid):
    dev = require_gpu()
    rng = np.random.default_rng(n_buf + grid)
    host = rng.integers(0, 1 << 32, size=n_buf * 1024, dtype=np.uint64).astype(np.uint32)
    if order_kind == "perm":
        order = rng.permutation(n_buf)
    elif order_kind == "short":  # an odd count, some blocks twice
        order = rng.integers(0, n_buf, size=1001)
    else:  # indices below 0 and past the end are clamped into the buffer
        order = np.concatenate([rng.integers(-50, n_buf + 50, size=77), [-1, n_buf, 1 << 30]])
    order = order.astype(np.int32)
    src = torch.from_numpy(host.view(np.int32)).to(dev)
    od = torch.from_numpy(order).to(dev)
    sink = torch.full((grid * 256,), -1, dtype=torch.int32, device=dev)
    say(f"block read: {n_buf} blocks, order {order_kind} ({order.size}), grid {grid}")
    bsk.debug_block_read(src, od, sink, grid, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    per_block = np.bitwise_xor.reduce(host.reshape(n_buf, 1024), axis=1)
    want = np.bitwise_xor.reduce(per_block[np.clip(order.astype(np.int64), 0, n_buf - 1)])
    assert got == want
