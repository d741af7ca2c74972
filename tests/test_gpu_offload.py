"""Parity of the step with the residuals in pinned host memory
(scape_step_offload: CPU offloading with double buffering, Memory
Optimization in the gist.science Technical Summary, s.2) with the oracle, on
a GPU, on both of its paths: the dense pass reading and writing the pinned
residuals over PCIe itself (the default for pinned memory), and the staged
path, which runs the same kernels as scape_step over chunks of 512 MB of
residuals (2^27 / W elements) copied through the GPU.  Every output is
expected bit-exact.
"""
import gc

import pytest

import synth
from synth.configs import Tensor
from harness import run_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_communication_adam_amd as sc
    sc.lib()  # fail loudly if the library is missing
    synth.gpu_lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _assert_bitexact(stats):
    assert stats["float_values"] > 0
    assert stats["float_not_bitexact"] == 0, stats


PATHS = pytest.mark.parametrize("path", ["direct", "staged"])


def _path(name):
    import sparse_communication_adam_amd as sc
    return sc.OFFLOAD_PATH_AUTO if name == "direct" else sc.OFFLOAD_PATH_STAGED


@PATHS
def test_offload_step_ragged_single_chunk(path):
    _assert_bitexact(run_parity(synth.ragged(), 5, offload=True, offload_path=_path(path)))


def _pad64(n):
    return (n + 63) // 64 * 64


@PATHS
def test_offload_step_three_chunks_with_boundaries_inside_layers(path):
    """About 87M elements at W = 4 (33,554,432 elements per chunk, the
    library's 512 MB staging slot): three residual chunks, staging slot 0
    reused, and the two chunk boundaries falling inside small layers, which
    the oracle checks (the large filler layers run on the GPU only)."""
    W = 4
    chunk = (512 << 20) // (W * 4)
    ts = [Tensor("fill0", (33_550_000,)), Tensor("across1", (10_000,)), Tensor("fill1", (33_540_000,)),
          Tensor("across2", (20_000,)), Tensor("fill2", (20_000_000,)), Tensor("tail", (4097,))]
    off = [0]
    for t in ts[:-1]:
        off.append(off[-1] + _pad64(t.numel))
    n_pad = off[-1] + _pad64(ts[-1].numel)
    assert off[1] < chunk < off[1] + ts[1].numel and off[3] < 2 * chunk < off[3] + ts[3].numel
    assert 2 * chunk < n_pad <= 3 * chunk
    wl = synth.ragged().with_tensors(ts, name="offload-chunks")
    _assert_bitexact(run_parity(wl, 4, sample=[1, 3, 5], W=W, offload=True, offload_path=_path(path)))


@PATHS
def test_offload_step_reduced_llama(path):
    _assert_bitexact(run_parity(synth.reduced(synth.LLAMA175), 3, offload=True, offload_path=_path(path)))


@pytest.mark.timeout(900)
def test_offload_step_full_size_direct():
    """The 1.75B shape at full size with its 28 GB of residuals in pinned
    host memory, read and written by the dense pass over PCIe: every output
    of sampled layers (norms, an attention output, the last layers) against
    the oracle for three steps."""
    wl = synth.WORKLOADS["llama-1.75b"]
    _assert_bitexact(run_parity(wl, 3, sample=[1, 3, 4, 190, 193], offload=True, offload_path=_path("direct")))
