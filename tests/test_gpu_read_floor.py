"""The read- and write-floor probes the bench reports beside the HBM-bound
rows: a read-only launch over 32 MiB buffers rotated past the last-level
cache must take longer than an empty launch and read below the 8 TB/s
datasheet rate; a write-only launch must write every byte it is given, and
no faster than that rate; bad arguments are refused before anything runs."""
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


def test_write_floor_is_plausible_and_writes_its_buffers():
    torch = gu.torch()
    n = 64 << 20
    bufs = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
    guard = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    write_us = gt.gt_test_write_floor(bufs, n - 4096, 8, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert n / (write_us * 1e-6) < 8.0e12
    for b in bufs:
        words = b.view(torch.int32).view(-1, 4)
        k = (n - 4096) // 16
        # chunk i of a buffer holds (v, v^1, v^2, i) for the last launch's v
        assert torch.equal(words[:k, 3].cpu(), torch.arange(k, dtype=torch.int32))
        assert torch.equal(words[:k, 1].cpu(), words[:k, 0].cpu() ^ 1)
        assert int(b[n - 4096:].abs().sum().item()) == 0  # nothing past `bytes`
    assert int(guard.abs().sum().item()) == 0


def test_write_floor_rejects_bad_arguments():
    torch = gu.torch()
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    for bufs, n, reps in (([buf], 4008, 4), ([buf], 0, 4), ([buf], 4096, 0)):
        with pytest.raises(gt.GemmTuneError):
            gt.gt_test_write_floor(bufs, n, reps)
    with pytest.raises(gt.GemmTuneError):  # misaligned buffer
        gt.gt_test_write_floor([buf.data_ptr() + 4], 1024, 4)
    assert int(buf.abs().sum().item()) == 0
