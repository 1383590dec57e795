"""The streaming-read measurement export runs on the device, reads without
writing the result word for ordinary data, and reports launch-time errors
through the status code."""
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import block_quant_gemv_amd as qg  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 1024 + 16, 9_437_184, 57_671_696])
def test_stream_read_runs_and_leaves_out_alone(nbytes):
    say(f"stream read of {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    out = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    for _ in range(3):
        qg.debug_stream_read(buf, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 12345


def test_stream_read_rejects_unaligned_sizes():
    buf = torch.zeros(1000, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(qg.QgemvError):
        qg.debug_stream_read(buf, out)
