"""The measurement probes of libmoe_peaks give exactly the results their
header defines: the XOR of every word read, a bitwise copy, and MFMA sums
that are small integers (so exact in fp32)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    from grouped_gemm_gemv_amd import peaks
    peaks.lib()
    return peaks


CHUNKS = [(1, 1), (5, 1), (4099, 3), (4099, 512), (65536, 1024), (65539, 7)]


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("nch,blocks", CHUNKS)
def test_read_xor(P, nch, blocks, flags):
    rng = np.random.default_rng(nch + blocks)
    host = rng.integers(0, 2**32, size=nch * 256, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    P.moe_peak_read(buf, sink, blocks, flags)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("nch,blocks", CHUNKS)
def test_copy_bitwise(P, nch, blocks, flags):
    g = torch.Generator(device="cpu").manual_seed(nch * 7 + blocks)
    src = torch.randint(-2**31, 2**31 - 1, (nch * 256,), dtype=torch.int32, generator=g).cuda()
    dst = torch.zeros_like(src)
    P.moe_peak_copy(src, dst, blocks, flags)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("a,b,iters,blocks", [(1.0, 1.0, 1, 1), (1.0, 1.0, 100, 256), (2.0, 3.0, 10, 7),
                                              (1.0, 1.0, 65536, 2)])
def test_mfma_sums(P, a, b, iters, blocks):
    sink = torch.full((4 * blocks,), -1.0, dtype=torch.float32, device="cuda")
    flops = P.moe_peak_mfma(a, b, iters, sink, blocks)
    assert flops == blocks * 4 * 8 * iters * 16384
    assert bool((sink == 256.0 * iters * a * b).all()), sink[:8]


def test_invalid_size_raises(P):
    buf = torch.zeros(300, dtype=torch.int32, device="cuda")  # 1200 bytes: not whole 1 KB chunks
    with pytest.raises(RuntimeError):
        P.moe_peak_read(buf, torch.zeros(1, dtype=torch.int32, device="cuda"), 1)
    with pytest.raises(RuntimeError):
        P.moe_peak_read(torch.zeros(256, dtype=torch.int32, device="cuda"),
                        torch.zeros(1, dtype=torch.int32, device="cuda"), 1, flags=4)
