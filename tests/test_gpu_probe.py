"""scape_copy_probe on a GPU: the plain stream-copy kernel bench.py times as
the HBM ceiling.  It must copy exactly the bytes asked for, for sizes that
are not whole workgroups, and leave the bytes after them alone.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_communication_adam_amd as sc
    sc.lib()
    yield


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 16, (64 << 20) + 48])
def test_copy_probe_copies_exactly(nbytes):
    import torch
    import sparse_communication_adam_amd as sc
    g = torch.Generator().manual_seed(nbytes)
    src_h = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g)
    src = src_h.to("cuda")
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sc.scape_copy_probe(src, dst, nbytes)
    torch.cuda.synchronize()
    out = dst.cpu()
    assert torch.equal(out[:nbytes], src_h[:nbytes])
    assert bool((out[nbytes:] == 0xA5).all())  # nothing past the end


def test_copy_probe_rejects_bad_sizes_before_launch():
    import torch
    import sparse_communication_adam_amd as sc
    a = torch.zeros(64, dtype=torch.uint8, device="cuda")
    b = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(sc.ScapeError) as e:
        sc.scape_copy_probe(a, b, 24)
    assert e.value.code == -2
    with pytest.raises(sc.ScapeError) as e:
        sc.scape_copy_probe(a[1:], b, 16)
    assert e.value.code == -3
