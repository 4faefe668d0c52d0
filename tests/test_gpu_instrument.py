"""The measurement references `bench.py` reads its achievable rates from (declared in
include/moet_instrument.h): the streaming read touches every byte once, and the tight loops run."""
import numpy as np
import pytest
import torch

from bit_moe_expert_nvfp4_amd import moet

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_probe_read_reads_every_word():
    """The xor of the per-wave sink words equals the xor of every 32-bit word of the buffer, for a
    buffer that is not a multiple of the grid's stride (ragged tail)."""
    print("[case] probe_read 1 MiB + 48 B", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    n = (1 << 20) // 4 + 12
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), generator=g, device=DEV, dtype=torch.int32)
    sink = torch.zeros((moet.PROBE_SINK_WORDS,), dtype=torch.int32, device=DEV)
    moet.probe_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("kind", [moet.PROBE_MFMA_BF16, moet.PROBE_DOT2_BF16])
def test_probe_peak_runs(kind):
    print(f"[case] probe_peak kind={kind}", flush=True)
    sink = torch.zeros((moet.PROBE_SINK_WORDS,), dtype=torch.int32, device=DEV)
    moet.probe_peak(kind, 16, sink)
    torch.cuda.synchronize()
    vals = sink[: moet.PROBE_PEAK_WAVES].cpu().numpy().view(np.float32)
    assert np.isfinite(vals).all() and (vals != 0).any()
