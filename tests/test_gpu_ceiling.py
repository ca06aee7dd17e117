"""The matrix-core calibration kernel behind the roofline's measured
ceiling (bench.py reports its rate beside the published peak)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


def test_mfma_ceiling_kernel(ci8):
    """The matrix-core calibration kernel: zeros in, zeros out; random
    operands give the same checksums on every launch."""
    dev = torch.device("cuda:0")
    out = torch.full((8 * 256,), 5, dtype=torch.int32, device=dev)
    ci8.conv_i8_mfma_ceiling(8, 3, 0, out)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0
    ci8.conv_i8_mfma_ceiling(8, 3, 12345, out)
    first = out.clone()
    ci8.conv_i8_mfma_ceiling(8, 3, 12345, out)
    torch.cuda.synchronize()
    assert torch.equal(out, first) and int(first.abs().sum()) > 0
