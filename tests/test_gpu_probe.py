"""The measurement helpers through the C ABI: bd_hbm_copy moves every byte, bd_hbm_read
returns the XOR of every 32-bit word (checked against numpy on the host), including sizes
that leave a ragged tail and the empty read."""

import numpy as np
import pytest

from gpu_common import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def bd():
    import torch  # noqa: F401
    from block_diffusion_lm_router_amd import _binding
    _binding.load()
    return _binding


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 77, 64 << 20])
def test_copy_and_read(bd, nbytes):
    import torch
    say("hbm copy/read", nbytes)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.zeros_like(src)
    bd.hbm_copy(src, dst)
    chk = torch.full((bd.HBM_READ_WORDS + 64,), 7, dtype=torch.int32, device="cuda")
    bd.hbm_read(src, chk[:bd.HBM_READ_WORDS])
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), host.view(np.int32))
    want = np.bitwise_xor.reduce(host)
    assert np.uint32(chk[0].item() & 0xFFFFFFFF) == want
    assert np.all(chk[bd.HBM_READ_WORDS:].cpu().numpy() == 7)   # nothing written past it


def test_read_empty(bd):
    import torch
    say("hbm read empty")
    src = torch.zeros(4, dtype=torch.int32, device="cuda")
    chk = torch.full((bd.HBM_READ_WORDS + 4,), 5, dtype=torch.int32, device="cuda")
    bd.hbm_read(src[:0], chk[:bd.HBM_READ_WORDS])
    torch.cuda.synchronize()
    got = chk.cpu().tolist()
    assert got[0] == 0 and got[bd.HBM_READ_WORDS:] == [5, 5, 5, 5]
