"""Parity of the dense AdamS step (the baseline the pages compare SCAPE with)
through the C ABI against the oracle, on a GPU.

Same bar as the SCAPE step: fp32 state within rel 1e-5 / abs 1e-7 of the
oracle, and bit-exact in fact (same operation order, no contraction, IEEE
division and square root), which the tests assert.
"""
import gc

import pytest

import synth
from harness import run_dense_parity

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


@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "llama-0.55b", "llama-1.75b", "adversarial-ties"])
def test_dense_step_oracle_sized(name):
    wl = synth.WORKLOADS[name]
    small = wl if name == "single-1024x1024" else synth.reduced(wl)
    _assert_bitexact(run_dense_parity(small, 3))


@pytest.mark.parametrize("W", [1, 2, 3, 5, 32])
def test_dense_step_worker_counts(W):
    """W = 1, a count without its own kernel instance (5), and the maximum."""
    _assert_bitexact(run_dense_parity(synth.ragged(), 3, W=W))


def test_dense_step_weight_decay_ragged_layout():
    _assert_bitexact(run_dense_parity(synth.ragged(), 4, weight_decay=0.01))


FULL_SAMPLES = {
    "gpt-345m": [0, 2, 4, 291],
    "llama-1.75b": [1, 3, 190, 194],
    "adversarial-ties": [1, 2, 10, 1088],
}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_dense_step_full_size_sampled_layers(name):
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_dense_parity(wl, 2, sample=FULL_SAMPLES[name]))


def test_dense_step_maximum_size():
    """The largest layout the ABI takes (n_pad = 2^31 - 64, one worker); the
    last layer, whose positions end 64 elements short of 2^31, against the
    oracle."""
    from test_gpu_parity import max_size_workload
    _assert_bitexact(run_dense_parity(max_size_workload(), 2, sample=[31]))


@pytest.mark.parametrize("W", [1, 3, 4, 8, 32])
def test_dense_step_interleaved_gradients(W):
    """scape_dense_step_interleaved: the W gradients in one worker-interleaved
    array (word stride 64 W)."""
    _assert_bitexact(run_dense_parity(synth.ragged(), 3, W=W, interleaved=True))


def test_dense_step_interleaved_full_size_sampled_layers():
    wl = synth.WORKLOADS["llama-1.75b"]
    _assert_bitexact(run_dense_parity(wl, 2, sample=FULL_SAMPLES["llama-1.75b"], interleaved=True))
