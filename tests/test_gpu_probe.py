"""The HBM probe moves what it says it moves: a copy reproduces the source
and a write leaves its index pattern, for streaming and plain accesses and
for grids smaller and larger than the buffer (include/ep_probe.h)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
from tests.gpu_backend import say  # noqa: E402


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("wgs", [1, 37, 4096])
def test_probe_copy_and_write(nt, wgs):
    nbytes = (1 << 20) + 16 * 129  # not a multiple of the grid's stride
    say(f"probe nt={nt} workgroups={wgs} bytes={nbytes}")
    rng = np.random.default_rng(wgs + nt)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    ep.ep_hbm_probe(ep.EP_PROBE_COPY, nt, wgs, src, dst, nbytes)
    ep.ep_hbm_probe(ep.EP_PROBE_READ, nt, wgs, src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0  # nothing past the end
    ep.ep_hbm_probe(ep.EP_PROBE_WRITE, nt, wgs, None, dst, nbytes)
    torch.cuda.synchronize()
    words = dst[:nbytes].view(torch.int32).view(-1, 4).cpu().numpy()
    i = np.arange(nbytes // 16, dtype=np.int64)
    assert np.array_equal(words[:, 0], i.astype(np.int32))
    assert np.array_equal(words[:, 1], (i >> 32).astype(np.int32))
    assert not words[:, 2:].any()
    assert int(dst[nbytes:].count_nonzero()) == 0
