"""scape_copy_probe on a GPU: the plain stream-copy kernel bench.py times as
the HBM ceiling.  It must copy exactly the bytes asked for, for sizes that
are not whole workgroups, and leave the bytes after them alone.  And
scape_stream_probe, the pass of the dense pass's traffic shape bench.py
compares the dense pass with: it must write what its definition says.
"""
import numpy as np
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


def _xor_parts(a: np.ndarray, width: int) -> np.ndarray:
    """Per element of width bytes: the XOR of its 32-bit parts (a 2-byte
    element zero-extended)."""
    if width == 2:
        return a.view(np.uint16).astype(np.uint32)
    return np.bitwise_xor.reduce(a.view(np.uint32).reshape(-1, width // 4), axis=1)


@pytest.mark.parametrize("widths", [((16, 8, 4), (16, 2)), ((2,), (4, 8)), ((16, 16, 16, 16), (2, 4, 8, 16)),
                                    ((4,), ())])
def test_stream_probe_writes_the_xor_of_its_sources(widths):
    """Every destination element holds the XOR of the 32-bit parts its
    sources held, repeated to its width; a destination may be a source."""
    import torch
    import sparse_communication_adam_amd as sc
    sw, dw = widths
    n_words = 1000  # several workgroups and a partial last one
    n = n_words * 64
    rng = np.random.default_rng(5)
    srcs_np = [rng.integers(0, 2**32, n * w // 4, dtype=np.uint32) for w in sw]
    srcs = [torch.from_numpy(a.view(np.int32)).cuda() for a in srcs_np]
    dsts = [torch.zeros(n * w // 4 if w >= 4 else n // 2, dtype=torch.int32, device="cuda") for w in dw]
    if sw and dw and sw[0] == dw[0]:
        dsts[0] = srcs[0]  # in place, as the dense pass writes its residuals
    sc.scape_stream_probe(srcs, sw, dsts, dw, n_words)
    torch.cuda.synchronize()
    exp = np.zeros(n, np.uint32)
    for a, w in zip(srcs_np, sw):
        exp ^= _xor_parts(a.view(np.uint8), w)
    for t, w in zip(dsts, dw):
        got = t.cpu().numpy().view(np.uint8)[: n * w]
        if w == 2:
            assert np.array_equal(got.view(np.uint16), (exp & 0xFFFF).astype(np.uint16))
        else:
            assert np.array_equal(got.view(np.uint32).reshape(n, w // 4), np.repeat(exp[:, None], w // 4, axis=1))
