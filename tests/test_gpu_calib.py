"""The benchmark's streaming-read calibration hook on the device: it reads
the whole buffer (any multiple of 16 bytes, grid-stride tail included) and
writes nothing for data whose fold is not its fixed key."""
import pytest
import torch

import bit_rank_post_amd as tq
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    need_gpu()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_calibrate_read_runs_and_writes_nothing(nbytes):
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    scratch = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    tq.calibrate_read(buf, scratch)
    torch.cuda.synchronize()
    assert int(scratch.item()) == -7
