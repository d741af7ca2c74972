"""The step captured as HIP graphs (ScapeState.capture / step_graph) against
the same step run eagerly: every state array and both mask slots bit-exact
after every step.  Between replays the test runs eager work of its own and
synchronizes, and every replay is checked, not only the last."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_communication_adam_amd as sc
    sc.lib()
    yield


def _state(wl, interleaved=False, update_in_dense=False):
    import sparse_communication_adam_amd as sc
    from sparse_communication_adam_amd.state import ScapeState
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    st = ScapeState(cfg, interleaved=interleaved)
    sc.scape_set_update_in_dense_pass(st.ctx, update_in_dense)
    synth.params_flat_gpu(wl, st.layout.layer_offset, st.x)
    return st


def _arrays(st):
    if st.interleaved:
        out = {"xv": st.xv, "m": st.m, "r_il": st.r_il}
    else:
        out = {"x": st.x, "m": st.m, "v": st.v}
        for i, r in enumerate(st.r):
            out[f"r{i}"] = r
    for s, mk in enumerate(st.masks):
        out[f"bits{s}"] = mk.bits
        out[f"idx{s}"] = mk.idx
        out[f"prefix{s}"] = mk.block_prefix
    return {k: v.view(-1).cpu().numpy().view(np.uint8) for k, v in out.items()}


@pytest.mark.parametrize("name,interleaved,update_in_dense", [
    ("ragged", False, False), ("single-1024x1024", False, False), ("ragged", True, False),
    ("single-1024x1024", True, False), ("ragged", False, True), ("ragged", True, True)])
def test_graph_replays_match_eager_steps(name, interleaved, update_in_dense):
    import torch
    import sparse_communication_adam_amd as sc
    wl = synth.ragged() if name == "ragged" else synth.WORKLOADS[name]
    eager, graphed = _state(wl, interleaved, update_in_dense), _state(wl, interleaved, update_in_dense)
    lay = eager.layout
    bufs = [torch.zeros(lay.n_pad, dtype=torch.int16, device="cuda") for _ in range(wl.W)]
    g_il = torch.zeros(lay.n_pad * wl.W, dtype=torch.int16, device="cuda")
    graphed.capture(g_il if interleaved else bufs)
    torch.cuda.synchronize()
    assert all(np.array_equal(a, b) for a, b in zip(_arrays(eager).values(), _arrays(graphed).values()))
    side = torch.randn(1 << 20, device="cuda")
    for t in range(1, 7):
        gs = [torch.zeros(lay.n_pad, dtype=torch.int16, device="cuda") for _ in range(wl.W)]
        for i, g in enumerate(gs):
            synth.grads_flat_gpu(wl, lay.layer_offset, g, t, i)
        if interleaved:
            view = sc.interleaved_view(g_il, wl.W)
            for i, g in enumerate(gs):
                view[:, i, :].copy_(g.view(-1, 64))
            eager.step(g_il.clone(), key_out=False)
        else:
            eager.step(gs, key_out=False)
            for b, g in zip(bufs, gs):
                b.copy_(g)
        graphed.step_graph()
        side.mul_(1.0001).sum()  # eager work of the program's own between replays
        torch.cuda.synchronize()
        a, b = _arrays(eager), _arrays(graphed)
        bad = [k for k in a if not np.array_equal(a[k], b[k])]
        assert not bad, f"step {t}: {bad} differ between the graph replay and the eager step"
    eager.destroy()
    graphed.destroy()
