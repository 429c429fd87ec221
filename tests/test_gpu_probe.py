"""The bandwidth probe (kvq_probe_bandwidth) through the C ABI: the copy mode
reproduces its source byte for byte, including a tail that is not a multiple
of the loop's four-vector step; the read mode leaves the source unchanged
and writes nothing to its sink for data that cannot hit the sink value."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 7])
def test_probe_copy_and_read(nbytes):
    from bit_mixed_precision_page_amd import kvq
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    kvq.kvq_probe_bandwidth(1, src, dst, nbytes)
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    zeros = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    kvq.kvq_probe_bandwidth(0, zeros, sink, nbytes)  # all-zero data folds to 0, never the sink value
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert int(sink.sum()) == 0
    for bad in ((2, src, dst, nbytes), (1, src, dst, nbytes - 1 if nbytes > 16 else 0)):
        with pytest.raises(kvq.KvqError):
            kvq.kvq_probe_bandwidth(*bad)
