"""GPU check of the bandwidth probes that bench.py reports as the measured HBM
ceiling: the copy moves every byte (sizes with and without a partial last
step), and the read's XOR of all 32-bit words matches the host's."""
import sys

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import layer as L

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("nbytes", [16, 4096 * 16, 4096 * 16 + 48, (8 << 20) + 16 * 37])
def test_probe_copy_and_read(nbytes):
    g = torch.Generator().manual_seed(nbytes % 1000)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.to("cuda:0")
    dst = torch.zeros_like(src)
    L.probe_copy(src, dst)
    acc = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    L.probe_read(src, acc)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(acc.cpu().numpy().view(np.uint32)[0]) == int(want)
