"""The measurement kernels the benchmark reads the block's timings against:
they launch through the C ABI, keep their work alive and report the work
they did (the ceilings themselves are printed by bench.py)."""

import pytest

from quantized_memory_bound_amd import ocq

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ocq.lib()


def test_window_read_writes_one_word_per_block():
    buf = torch.full((1 << 20,), 3, dtype=torch.uint8, device="cuda")
    out = torch.full((64,), -1, dtype=torch.int32, device="cuda")
    ocq.diag_window_read(buf, 1 << 20, 2, out, 64)
    torch.cuda.synchronize()
    # the xor of an even number of equal 16-byte pieces per lane is zero, and
    # so is the workgroup's or of those words
    assert (out == 0).all()


def test_window_read_rejects_bad_window():
    buf = torch.ones(1 << 16, dtype=torch.uint8, device="cuda")
    out = torch.empty(8, dtype=torch.int32, device="cuda")
    with pytest.raises(ocq.OcqError):
        ocq.diag_window_read(buf, 1000, 1, out, 8)


def test_mfma_rate_counts_its_flops():
    out = torch.zeros(512 * 4, dtype=torch.float32, device="cuda")
    fl = ocq.diag_mfma_rate(10, out, 4)
    torch.cuda.synchronize()
    assert fl == 2 * 16 * 16 * 32 * 16 * 10 * 8 * 4
    o = out.cpu()
    assert torch.isfinite(o).all() and (o != 0).all()
