"""Parity of the step with the residuals in pinned host memory
(scape_step_offload: CPU offloading with double buffering, Memory
Optimization in the gist.science Technical Summary, s.2) with the oracle, on
a GPU.  The offloaded step runs the same kernels as scape_step over chunks of
4,194,304 elements, so every output is expected bit-exact.
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


def test_offload_step_ragged_single_chunk():
    _assert_bitexact(run_parity(synth.ragged(), 5, offload=True))


def test_offload_step_three_chunks_with_boundaries_inside_layers():
    """10.5M elements: three residual chunks, both staging slots reused, and
    chunk boundaries falling inside layers."""
    ts = [Tensor("a", (3_000_001,)), Tensor("b", (37,)), Tensor("c", (2000, 2500)), Tensor("d", (64,)),
          Tensor("e", (2_500_000,))]
    wl = synth.ragged().with_tensors(ts, name="offload-chunks")
    _assert_bitexact(run_parity(wl, 4, offload=True))


def test_offload_step_reduced_llama():
    _assert_bitexact(run_parity(synth.reduced(synth.LLAMA175), 3, offload=True))
