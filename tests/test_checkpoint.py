"""Checkpoint and resume of the SCAPE step state, on the oracle (CPU).

Because the mask built at step t is applied only at step t+1 (Delayed Mask
Usage, gist.science Technical Summary s.2), the pending mask is part of the
optimizer state together with x, m, v and every worker's residual.  Running
T steps straight through must equal running t steps, writing that state to a
file, reading it back into fresh arrays and running the remaining T - t
steps, bit for bit; resuming without the pending mask must not.
"""
import numpy as np

import oracle
import synth


def _grads(wl, lay, t, W):
    return [synth.grads_flat(wl, lay.off, lay.n_pad, t, i) for i in range(W)]


def _save(path, st, cur, t):
    np.savez(path, x=st.x, m=st.m, v=st.v, pending=cur, t=np.int64(t), **{f"r{i}": a for i, a in enumerate(st.r)})


def _load(path, W):
    with np.load(path, allow_pickle=False) as d:
        st = oracle.State(d["x"].copy(), d["m"].copy(), d["v"].copy(), [d[f"r{i}"].copy() for i in range(W)])
        return st, d["pending"].copy(), int(d["t"])


def _run(wl, lay, hp, st, cur, t0, t1):
    outs = []
    for t in range(t0, t1 + 1):
        out = oracle.step(lay, hp, st, _grads(wl, lay, t, len(st.r)), cur)
        outs.append(out)
        cur = out.next_words
    return cur, outs


def test_resume_from_file_is_bitwise_identical(tmp_path):
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hp = oracle.Hyper(wl.beta1, wl.beta2, wl.lr, wl.eps, 0.01)
    x0 = synth.params_flat(wl, lay.off, lay.n_pad)
    T = 6
    straight = oracle.State.zeros(lay.n_pad, wl.W, x0)
    cur_s, outs_s = _run(wl, lay, hp, straight, np.zeros(lay.n_words, np.uint64), 1, T)
    for t_cut in (1, 3):
        st = oracle.State.zeros(lay.n_pad, wl.W, x0)
        cur, _ = _run(wl, lay, hp, st, np.zeros(lay.n_words, np.uint64), 1, t_cut)
        path = tmp_path / f"ckpt{t_cut}.npz"
        _save(path, st, cur, t_cut)
        del st, cur
        st, cur, t_done = _load(path, wl.W)
        assert t_done == t_cut
        cur, outs = _run(wl, lay, hp, st, cur, t_done + 1, T)
        for a, b in [(st.x, straight.x), (st.m, straight.m), (st.v, straight.v)] + list(zip(st.r, straight.r)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(cur, cur_s)
        for o, s in zip(outs, outs_s[t_cut:]):
            assert o.count == s.count
            for i in range(wl.W):
                assert np.array_equal(o.sent[i].view(np.uint32), s.sent[i].view(np.uint32))


def test_resume_without_the_pending_mask_differs():
    """The pending mask is state: dropping it (resuming with an empty mask)
    changes what the next step sends and updates."""
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hp = oracle.Hyper(wl.beta1, wl.beta2, wl.lr, wl.eps, 0.0)
    x0 = synth.params_flat(wl, lay.off, lay.n_pad)
    a = oracle.State.zeros(lay.n_pad, wl.W, x0)
    cur, _ = _run(wl, lay, hp, a, np.zeros(lay.n_words, np.uint64), 1, 2)
    b = a.copy()
    _run(wl, lay, hp, a, cur, 3, 3)
    _run(wl, lay, hp, b, np.zeros(lay.n_words, np.uint64), 3, 3)
    assert not np.array_equal(a.x, b.x) and not np.array_equal(a.r[0], b.r[0])
