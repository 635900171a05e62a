"""The read-floor probe the bench reports beside the HBM-bound rows: a
read-only launch over 32 MiB buffers rotated past the last-level cache must
take longer than an empty launch and read below the 8 TB/s datasheet rate;
bad arguments are refused before anything runs."""
import pytest

import gemm_autotuning_amd as gt

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_read_floor_is_plausible():
    torch = gu.torch()
    n = 32 << 20
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(12)]
    torch.cuda.synchronize()
    read_us, empty_us = gt.gt_test_read_floor(bufs, n, 48, torch.cuda.current_stream().cuda_stream)
    assert 0 < empty_us < read_us
    assert n / (read_us * 1e-6) < 8.0e12  # no faster than the HBM datasheet rate


def test_read_floor_rejects_bad_arguments():
    torch = gu.torch()
    buf = torch.ones(4096, dtype=torch.uint8, device="cuda")
    for bufs, n, reps in (([buf], 4008, 4), ([buf], 0, 4), ([buf], 4096, 0)):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_test_read_floor(bufs, n, reps)
    with pytest.raises(gt.GemmTuneError):  # misaligned buffer
        gt.gt_test_read_floor([buf.data_ptr() + 4], 1024, 4)
