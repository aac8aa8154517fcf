"""The HBM read-ceiling probe (moe_read_probe) reads every byte it is given: the xor of the words
it writes, one per block, equals the xor of every 32-bit word of the buffer, computed on the host.
Sizes cover a ragged tail (not a multiple of one grid step) and a buffer smaller than one grid step."""
import numpy as np
import pytest
import torch

from parity_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_expert_ffn_amd as m
    return m


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 * 8 * 3 + 16 * 37, 1 << 20, 64 << 20])
def test_read_probe_folds_every_word(M, nbytes):
    log(f"read probe: {nbytes} bytes")
    rng = np.random.default_rng(nbytes % 1000003)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((M.MOE_READ_PROBE_BLOCKS,), -1, dtype=torch.int32, device=DEV)
    M.moe_read_probe(buf, out)
    torch.cuda.synchronize()
    folded = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(folded) == int(np.bitwise_xor.reduce(host))
