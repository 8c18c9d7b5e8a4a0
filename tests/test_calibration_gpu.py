"""GPU checks of the streaming-read calibration helper (da_read_calibration):
each lane XOR-folds the 16-byte chunks it reads and writes the one-word sink
only if its fold equals a fixed constant.  A buffer of zeros with one chunk
whose four words fold to the constant therefore reaches the sink exactly when
that chunk is read."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAGIC = np.uint32(0x9E3779B9)


@pytest.fixture(scope="module")
def da():
    import decode_attention_folded_amd as pkg
    pkg.load_library()
    return pkg


def _run(da, words):
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    da.read_calibration(buf, sink)
    torch.cuda.synchronize()
    return np.uint32(sink.item() & 0xFFFFFFFF)


# 16-byte chunks: one; a few; exactly one full block step of the grid
# (2048 workgroups x 256 lanes x 8 loads); a full step plus a ragged tail.
@pytest.mark.parametrize("n_chunks", [1, 7, 2048 * 256 * 8, 2048 * 256 * 8 + 3])
def test_every_chunk_is_read(da, n_chunks):
    rng = np.random.default_rng(n_chunks)
    places = sorted({0, n_chunks // 2, n_chunks - 1, int(rng.integers(0, n_chunks))})
    for c in places:
        w = np.zeros(4 * n_chunks, dtype=np.uint32)
        w[4 * c:4 * c + 3] = rng.integers(0, 2**32, size=3, dtype=np.uint64).astype(np.uint32)
        w[4 * c + 3] = np.bitwise_xor.reduce(w[4 * c:4 * c + 3]) ^ MAGIC
        assert _run(da, w) == MAGIC, (n_chunks, c)
        w[4 * c] ^= np.uint32(1)  # no lane's fold is the constant now
        assert _run(da, w) == np.uint32(0xFFFFFFFF), (n_chunks, c)
