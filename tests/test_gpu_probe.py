"""The bandwidth probe on the GPU: the copy reproduces its source exactly (whole and
ragged sizes), the read leaves the destination untouched, and bad arguments raise."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def vj():
    import vocab_sharded_softmax_amd as v
    return v


@pytest.mark.parametrize("words", [1, 63, 64, 65, 1023, 1024 * 1024 + 5])
def test_probe_copy_is_exact(words):
    g = torch.Generator(device="cuda").manual_seed(words)
    src = torch.randint(-2**31, 2**31 - 1, (words * 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    dst = torch.full_like(src, 7)
    vj().vjsd_membw_probe(src, dst, 1)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_read_leaves_destination():
    src = torch.arange(4 * 4099, dtype=torch.int32, device="cuda")
    dst = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    vj().vjsd_membw_probe(src, dst, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), torch.full((4,), 7, dtype=torch.int32))


def test_probe_rejects_bad_arguments():
    v = vj()
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(v.VjsdArgumentError):
        v.vjsd_membw_probe(src, src, 1)  # overlapping copy
    with pytest.raises(v.VjsdArgumentError):
        v.vjsd_membw_probe(src, torch.zeros(64, dtype=torch.int32, device="cuda"), 3)
    with pytest.raises(v.VjsdArgumentError):
        v.vjsd_membw_probe(src[1:61], torch.zeros(64, dtype=torch.int32, device="cuda"), 1)
