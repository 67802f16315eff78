"""GPU check of the streaming-read probe used to measure the HBM read rate:
every 64 KiB block's XOR of 32-bit words equals numpy's on the same bytes."""
import numpy as np
import pytest

from quantized_expert_ffn_topk_amd import abi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("n_blocks", [1, 64, 129])
def test_stream_read_reads_every_byte(n_blocks):
    rng = np.random.default_rng(n_blocks)
    host = rng.integers(0, 256, size=n_blocks * 65536, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    sink = torch.zeros(n_blocks, dtype=torch.int32, device="cuda")
    abi.moe_debug_stream_read(src, host.nbytes, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32).reshape(n_blocks, -1), axis=1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
