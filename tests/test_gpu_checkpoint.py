"""Checkpoint and resume of the GPU step state (ScapeState.state_dict).

T steps straight through must equal t steps, a round trip of the state
through a file (torch.save, read back with weights_only=True) into a fresh
ScapeState, and T - t more steps: bit for bit, masks included.  The pending
mask is part of the state because masks are applied one step after they are
built (Delayed Mask Usage, gist.science Technical Summary s.2).
"""
import gc

import numpy as np
import pytest

import synth
from harness import scape_config, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_communication_adam_amd as sc
    sc.lib()
    synth.gpu_lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _new_state(wl, interleaved=False):
    from sparse_communication_adam_amd.state import ScapeState
    st = ScapeState(scape_config(wl), interleaved=interleaved)
    synth.params_flat_gpu(wl, st.layout.layer_offset, st.x)
    return st


def _steps(st, wl, grads, t0, t1):
    import torch
    import sparse_communication_adam_amd as sc
    for t in range(t0, t1 + 1):
        for i, g in enumerate(grads):
            synth.grads_flat_gpu(wl, st.layout.layer_offset, g, t, i)
        if st.interleaved:
            g_il = torch.zeros(st.layout.n_pad * wl.W, dtype=torch.int16, device="cuda")
            view = sc.interleaved_view(g_il, wl.W)
            for i, g in enumerate(grads):
                view[:, i, :].copy_(g.view(-1, 64))
            st.step(g_il, key_out=False)
        else:
            st.step(grads, key_out=False)


def _snapshot(st):
    import torch
    torch.cuda.synchronize()
    arrs = [st.x, st.m, st.v] + [st.residual(i) for i in range(st.cfg.workers)]
    arrs += [st.cur_mask.bits, st.cur_mask.idx, st.cur_mask.block_prefix]
    return [to_np(a).copy() for a in arrs]


@pytest.mark.parametrize("name,il_write,il_read", [("ragged", False, False), ("llama-1.75b-small", False, False),
                                                  ("ragged", True, True), ("ragged", True, False),
                                                  ("llama-1.75b-small", False, True)])
def test_gpu_resume_from_file_is_bitwise_identical(tmp_path, name, il_write, il_read):
    """The checkpoint stores each worker's residual flat, so a state saved in
    one residual layout resumes in the other."""
    import torch
    wl = synth.ragged() if name == "ragged" else synth.reduced(synth.LLAMA175)
    n = None
    T, t_cut = 5, 2
    a = _new_state(wl)
    n = a.layout.n_pad
    grads = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(wl.W)]
    _steps(a, wl, grads, 1, T)
    want = _snapshot(a)
    a.destroy()

    b = _new_state(wl, interleaved=il_write)
    _steps(b, wl, grads, 1, t_cut)
    path = tmp_path / "scape_state.pt"
    torch.save(b.state_dict(), path)
    b.destroy()
    del b
    gc.collect()

    c = _new_state(wl, interleaved=il_read)
    c.x.zero_()
    c.load_state_dict(torch.load(path, weights_only=True))
    assert c.t == t_cut
    _steps(c, wl, grads, t_cut + 1, T)
    got = _snapshot(c)
    c.destroy()
    for i, (g, w) in enumerate(zip(got, want)):
        assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), f"array {i} differs after resume"


def test_gpu_load_rejects_a_different_layout():
    import torch
    a = _new_state(synth.ragged())
    sd = a.state_dict()
    a.destroy()
    wl = synth.reduced(synth.LLAMA175)
    b = _new_state(wl)
    with pytest.raises(ValueError):
        b.load_state_dict(sd)
    b.destroy()
    torch.cuda.synchronize()
