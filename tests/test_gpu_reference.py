"""GPU test of the bench's streaming-read reference (a measurement aid, not
part of the sampling path): it must read every value once, so the maximum
bit pattern it folds equals the host's."""

import numpy as np
import pytest
import torch

from decode_step_sampling_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 4096, 64 * 151936, 1000004])
def test_stream_read_reference_sees_every_value(n):
    rng = np.random.default_rng(n)
    x = rng.random(n, dtype=np.float32)
    x[rng.integers(n)] = 3.5          # one maximum somewhere
    d = torch.from_numpy(x).to("cuda:0")
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    lib = _lib.load()
    st = lib.dss_stream_read_reference(d.data_ptr(), n, out.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == _lib.DSS_OK
    torch.cuda.synchronize()
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(x.view(np.uint32).max())
