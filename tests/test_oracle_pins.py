"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself: a
hand-worked dyadic example, brute-force ranking, numpy's packbits/cumsum/
lexsort, exact rational arithmetic, an fp64 dense average, an fp64 dense AdamS,
or a metamorphic relation.  The dense AdamS step (the comparison baseline) is
pinned by a hand-worked dyadic example, by its agreement with the SCAPE step
under a full mask, and by exact scaling and sign symmetries.  The passages behind each rule are cited in
oracle/scape_oracle.c.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # unit roundoff of fp32


def bf16_bits(x):
    """bfloat16 bits of values that are exactly representable (asserted)."""
    f = np.asarray(x, np.float32)
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exact in bfloat16"
    return (b >> 16).astype(np.uint16)


def bf16_to_f64(g):
    return (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def popcount_words(words):
    return np.unpackbits(words.view(np.uint8)).reshape(-1, 64).sum(1)


def random_grads(rng, lay, W, scale=1e-3):
    gs = []
    for _ in range(W):
        f = (rng.standard_normal(lay.n_pad) * scale).astype(np.float32)
        b = f.view(np.uint32)
        b = b + 0x7FFF + ((b >> 16) & 1)
        g = (b >> 16).astype(np.uint16)
        for l in range(lay.L):  # padding gradients are zero
            g[lay.off[l] + lay.sizes[l]:(lay.off[l + 1] if l + 1 < lay.L else lay.n_pad)] = 0
        gs.append(g)
    return gs


def layer_mask(lay):
    inl = np.zeros(lay.n_pad, bool)
    for l in range(lay.L):
        inl[lay.off[l]:lay.off[l] + lay.sizes[l]] = True
    return inl


# --------------------------------------------------------------------------
# layout, kept counts, ownership


@pytest.mark.parametrize("n,num,den", [(0, 1, 10), (1, 1, 10), (1024, 1, 10), (37, 3, 100),
                                       (1048576, 1, 10), (2 ** 40 + 3, 7, 1000), (999, 0, 5),
                                       (999, 5, 5), (131072000, 1, 1000)])
def test_keep_count_is_exact_ceiling(n, num, den):
    expect = -((-Fraction(n) * num) // den)  # exact ceiling
    assert oracle.keep_count(n, num, den) == expect
    if n:
        # density is in [keep, keep + 1/n)
        assert Fraction(num, den) <= Fraction(int(expect), n) < Fraction(num, den) + Fraction(1, n)


def test_owner_is_shard_of_layer_midpoint():
    rng = np.random.default_rng(7)
    for _ in range(50):
        sizes = rng.integers(1, 5000, size=rng.integers(1, 40))
        P = int(rng.integers(1, 33))
        lay = oracle.layout(sizes, 1, 10, P)
        N = lay.n_pad
        prev = 0
        for l in range(lay.L):
            mid = Fraction(int(lay.off[l])) + Fraction(int(lay.sizes[l]), 2)
            # the shard s with s*N/P <= mid < (s+1)*N/P, brute force
            s = next(s for s in range(P) if Fraction(s * N, P) <= mid < Fraction((s + 1) * N, P))
            assert lay.owner[l] == s
            assert lay.owner[l] >= prev  # layer-aligned shards are contiguous
            prev = lay.owner[l]


def test_owner_of_single_layer_workload():
    wl = synth.SINGLE
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    assert lay.owner.tolist() == [2]  # midpoint N/2 of four even shards lies in shard 2


def test_layout_alignment_and_sizes():
    for wl in list(synth.WORKLOADS.values()) + [synth.ragged()]:
        lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
        assert np.all(lay.off % 64 == 0)
        ends = lay.off + lay.sizes
        assert np.all(ends[:-1] <= lay.off[1:])
        assert lay.n_pad == (int(ends[-1]) + 63) // 64 * 64
    lay = oracle.layout(synth.LLAMA175.layer_sizes, 1, 100, 4)
    assert lay.n_pad == 1_750_206_464 and lay.k_total == 17_502_165
    assert sorted(set(lay.k.tolist())) == [21, 41944, 112722, 125830, 225444, 655360]


# --------------------------------------------------------------------------
# packing and indexing


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000, 4096, 12345])
def test_pack_matches_numpy_packbits_little(n):
    rng = np.random.default_rng(n)
    pred = (rng.random(n) < 0.3).astype(np.uint8)
    words = oracle.pack(pred)
    ref = np.packbits(pred, bitorder="little")
    ref = np.concatenate([ref, np.zeros(words.size * 8 - ref.size, np.uint8)]).view("<u8")
    assert np.array_equal(words, ref)
    assert np.array_equal(oracle.unpack(words, n), pred)


def test_mask_index_matches_numpy():
    rng = np.random.default_rng(3)
    for dens in (0.0, 0.01, 0.5, 1.0):
        pred = (rng.random(64 * 97) < dens).astype(np.uint8)
        words = oracle.pack(pred)
        idx, prefix, cnt = oracle.mask_index(words)
        assert np.array_equal(idx, np.flatnonzero(pred))
        assert cnt == pred.sum()
        ref = np.concatenate([[0], np.cumsum(popcount_words(words))])
        assert np.array_equal(prefix, ref)


# --------------------------------------------------------------------------
# top-k


def brute_topk(keys, k):
    """sel[j] iff fewer than k elements precede j in (key desc, position asc)."""
    keys = np.asarray(keys, np.int64)
    n = keys.size
    pos = np.arange(n)
    before = (keys[None, :] > keys[:, None]) | ((keys[None, :] == keys[:, None]) & (pos[None, :] < pos[:, None]))
    return (before.sum(1) < k).astype(np.uint8)


def test_topk_golden_ties():
    for line in open(os.path.join(GOLDEN, "topk_ties.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        keys, k, exp = [p.strip() for p in line.split(";")]
        keys = np.array([int(v) for v in keys.split(",")], np.uint32)
        exp = [int(v) for v in exp.split(",")] if exp else []
        sel = oracle.topk(keys, int(k))
        assert np.flatnonzero(sel).tolist() == exp, line


def test_topk_brute_force_small():
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(1, 160))
        kind = trial % 4
        if kind == 0:
            keys = rng.integers(0, 2 ** 31, n)
        elif kind == 1:
            keys = np.full(n, 12345)
        elif kind == 2:  # 16 quantised levels, |+-q| collide
            q = rng.integers(-8, 8, n).astype(np.float32) * np.float32(2 ** -12)
            keys = np.abs(q).view(np.uint32)
        else:  # +-pairs of one value
            v = rng.standard_normal(n).astype(np.float32)
            v[1::2] = -v[0::2][: v[1::2].size]
            keys = np.abs(v).view(np.uint32)
        keys = np.asarray(keys, np.uint32)
        k = int(rng.integers(0, n + 1))
        assert np.array_equal(oracle.topk(keys, k), brute_topk(keys, k))


def test_topk_matches_lexsort_large_with_ties():
    rng = np.random.default_rng(5)
    n = 200_000
    keys = (rng.integers(0, 50, n) * 1000003).astype(np.uint32)
    for k in (1, 2000, 99_999, n):
        order = np.lexsort((np.arange(n), -keys.astype(np.int64)))
        ref = np.zeros(n, np.uint8)
        ref[order[:k]] = 1
        assert np.array_equal(oracle.topk(keys, k), ref)


def test_keys_are_magnitude_bits():
    v = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -2.0 ** -140], np.float32)
    k = oracle.keys_of(v)
    assert k.tolist() == [0, 0, 0x3FC00000, 0x3FC00000, 0x7F800000, np.abs(v[5]).view(np.uint32)]


# --------------------------------------------------------------------------
# reduction


def test_reduce_error_bound_vs_fp64_mean():
    rng = np.random.default_rng(2)
    for W in (1, 2, 3, 4, 8, 32):
        bufs = [(rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 2)).astype(np.float32) for _ in range(W)]
        out = oracle.reduce(bufs).astype(np.float64)
        exact = np.mean([b.astype(np.float64) for b in bufs], axis=0)
        bound = (W - 1) * U * np.sum([np.abs(b.astype(np.float64)) for b in bufs], axis=0) / W + U * np.abs(exact) * 2
        assert np.all(np.abs(out - exact) <= bound + 1e-45)
        if W == 1:
            assert np.array_equal(out.astype(np.float32), bufs[0])


def test_reduce_sums_in_worker_order():
    # 1 + 2^24 rounds back to 2^24 in fp32, so only the order 0,1,2 gives 0.
    bufs = [np.array([1.0], np.float32), np.array([2.0 ** 24], np.float32), np.array([-(2.0 ** 24)], np.float32)]
    assert oracle.reduce(bufs)[0] == 0.0


# --------------------------------------------------------------------------
# the step


def _parse_golden(name="worked_step.txt"):
    d = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if "=" in line:
            k, v = [p.strip() for p in line.split("=", 1)]
            d[k] = v
    return d


def _vals(s, dtype=np.float32):
    return np.array([float(Fraction(x)) for x in s.split(",")] if s else [], dtype)


@pytest.mark.parametrize("name", ["worked_step.txt", "worked_step_wd.txt"])
def test_golden_worked_step(name):
    """Hand-worked dyadic steps: the three-step example without weight decay,
    and the one with decoupled weight decay (wd = 0.5) that starts from a full
    mask, so that the decay term is exercised at masked positions and shown
    absent off the mask."""
    d = _parse_golden(name)
    n, W, P = int(d["layer_n"]), int(d["W"]), int(d["P"])
    num, den = [int(v) for v in d["keep"].split("/")]
    lay = oracle.layout([n], num, den, P)
    assert lay.owner.tolist() == [0] and lay.k.tolist() == [2]
    hp = oracle.Hyper(float(d["beta1"]), float(d["beta2"]), float(d["lr"]), float(d["eps"]),
                      float(d.get("wd", "0")))
    x = np.zeros(lay.n_pad, np.float32)
    x[:n] = _vals(d["x0"])
    st = oracle.State.zeros(lay.n_pad, W, x)
    pred = np.zeros(lay.n_pad, np.uint8)
    if d.get("M1"):
        pred[[int(v) for v in d["M1"].split(",")]] = 1
    cur = oracle.pack(pred)
    for t in (1, 2, 3):
        gs = []
        for i in range(W):
            g = np.zeros(lay.n_pad, np.uint16)
            g[:n] = bf16_bits(_vals(d[f"step{t}.g{i}"]))
            gs.append(g)
        out = oracle.step(lay, hp, st, gs, cur)
        for i in range(W):
            assert np.array_equal(out.sent[i], _vals(d[f"step{t}.sent{i}"])), (t, i)
            assert np.array_equal(st.r[i][:n], _vals(d[f"step{t}.r{i}"])), (t, i)
        if f"step{t}.bbar" in d:
            assert np.array_equal(out.bbar, _vals(d[f"step{t}.bbar"]))
        if f"step{t}.x" in d:
            assert np.array_equal(st.x[:n], _vals(d[f"step{t}.x"])), t
        assert np.array_equal(st.m[:n], _vals(d[f"step{t}.m"])), t
        assert np.array_equal(st.v[:n], _vals(d[f"step{t}.v"])), t
        assert out.next_idx.tolist() == [int(v) for v in d[f"step{t}.next"].split(",")], t
        cur = out.next_words


def round_to_f32(q: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32 (normal range), by
    integer arithmetic on the significand."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while q * Fraction(2) ** (23 - e) >= 2 ** 24:
        e += 1
    while q * Fraction(2) ** (23 - e) < 2 ** 23:
        e -= 1
    t = q * Fraction(2) ** (23 - e)
    n = t.numerator // t.denominator
    rest = t - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))


@pytest.mark.parametrize("W", [3, 5, 6, 7])
def test_reduce_mean_is_one_correctly_rounded_division(W):
    """The mean is the fp32 sum in worker order followed by one correctly
    rounded division by W (the reading of "averaged" in the Single-Buffer
    Second-Moment Reconstruction paragraph).  At worker counts that are not
    powers of two, multiplying by the rounded reciprocal 1/W gives a different
    fp32 value for about a third of the sums; the expected values here are
    the exact quotients rounded by integer arithmetic."""
    rng = np.random.default_rng(W)
    k = 600
    bufs = [(rng.standard_normal(k) * 10.0 ** rng.integers(-3, 3, k)).astype(np.float32) for _ in range(W)]
    got = oracle.reduce(bufs)
    recip_differs = 0
    for q in range(k):
        s = Fraction(float(bufs[0][q]))
        for i in range(1, W):  # each fp32 addition rounds once
            s = Fraction(float(round_to_f32(s + Fraction(float(bufs[i][q])))))
        exp = round_to_f32(s / W)
        assert got[q].view(np.uint32) == exp.view(np.uint32), (q, got[q], exp)
        recip_differs += round_to_f32(s * Fraction(float(np.float32(1.0) / np.float32(W)))) != exp
    assert recip_differs > k // 10  # the cases do tell the two forms apart


def _run(lay, W, T, hp, grads_fn, cur=None, x=None, owner_map=None):
    st = oracle.State.zeros(lay.n_pad, W, x)
    cur = np.zeros(lay.n_words, np.uint64) if cur is None else cur
    hist = []
    for t in range(1, T + 1):
        prev = st.copy()
        gs = grads_fn(t)
        out = oracle.step(lay, hp, st, gs, cur, owner_map)
        hist.append((prev, gs, cur, out, st.copy()))
        cur = out.next_words
    return hist


def test_first_step_with_empty_mask_only_accumulates():
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    rng = np.random.default_rng(1)
    x0 = rng.standard_normal(lay.n_pad).astype(np.float32)
    gs = random_grads(rng, lay, wl.W)
    st = oracle.State.zeros(lay.n_pad, wl.W, x0)
    out = oracle.step(lay, oracle.Hyper(), st, gs, np.zeros(lay.n_words, np.uint64))
    assert out.count == 0
    for i in range(wl.W):
        assert np.array_equal(st.r[i], (gs[i].astype(np.uint32) << 16).view(np.float32))
    assert np.array_equal(st.x, x0) and not st.m.any() and not st.v.any()
    assert np.array_equal(popcount_words(out.next_words).sum(), lay.k_total)


def test_every_built_mask_has_exactly_k_per_layer():
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hist = _run(lay, wl.W, 4, oracle.Hyper(),
                lambda t: synth_grads(wl, lay, t))
    for (_, _, _, out, _) in hist:
        pred = oracle.unpack(out.next_words, lay.n_pad)
        for l in range(lay.L):
            seg = pred[lay.off[l]:lay.off[l] + lay.sizes[l]]
            assert seg.sum() == min(lay.k[l], lay.sizes[l])
        assert pred[~layer_mask(lay)].sum() == 0  # padding never selected
        # the mask is the top-k of the statistic, layer by layer (brute force on small layers)
        for l in range(lay.L):
            if lay.sizes[l] <= 5000:
                seg = slice(lay.off[l], lay.off[l] + lay.sizes[l])
                assert np.array_equal(pred[seg], brute_topk(out.key[seg], int(lay.k[l])))


def synth_grads(wl, lay, t, tensors=None):
    return [synth.grads_flat(wl, lay.off, lay.n_pad, t, i, tensors) for i in range(wl.W)]


def test_residual_conservation_exact_dyadic():
    """sum_t g = sum over sent steps of a + r_T, in exact arithmetic."""
    W, T = 4, 3
    lay = oracle.layout([512, 192, 64], 1, 4, W)
    hp = oracle.Hyper(0.5, 0.75, 0.25, 1.0, 0.0)
    rng = np.random.default_rng(9)
    gq = {t: [rng.integers(-8, 8, lay.n_pad) for _ in range(W)] for t in range(1, T + 1)}

    def gf(t):
        return [bf16_bits(q.astype(np.float32) * np.float32(1 / 16)) for q in gq[t]]

    cur = oracle.pack((rng.random(lay.n_pad) < 0.3).astype(np.uint8))  # arbitrary first mask
    hist = _run(lay, W, T, hp, gf, cur=cur)
    total_g = [np.zeros(lay.n_pad, object) for _ in range(W)]
    sent_a = [np.zeros(lay.n_pad, object) for _ in range(W)]
    for t, (prev, gs, curw, out, _) in enumerate(hist, 1):
        pos = np.flatnonzero(oracle.unpack(curw, lay.n_pad))
        for i in range(W):
            total_g[i] += np.array([Fraction(float(v)) for v in bf16_to_f64(gs[i])], object)
            for q, j in enumerate(pos):
                # the gradient mass carried by the sent candidate: a = (m~ - beta1*m)/(1-beta1)
                a = (Fraction(float(out.sent[i][q])) - Fraction(1, 2) * Fraction(float(prev.m[j]))) / Fraction(1, 2)
                sent_a[i][j] += a
                # and it equals the accumulated gradient r_prev + g exactly
                assert a == Fraction(float(prev.r[i][j])) + Fraction(float(bf16_to_f64(gs[i])[j]))
    final = hist[-1][4]
    for i in range(W):
        r = np.array([Fraction(float(v)) for v in final.r[i]], object)
        assert np.all(total_g[i] == sent_a[i] + r)


def test_reconstructed_gradient_is_the_dense_average():
    """On masked positions, (m_new - beta1*m_old)/(1-beta1) = mean_i (r_i + g_i)."""
    wl = synth.reduced(synth.GPT345M)
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hp = oracle.Hyper()
    hist = _run(lay, wl.W, 3, hp, lambda t: synth_grads(wl, lay, t))
    b1, c1 = np.float64(np.float32(0.9)), np.float64(np.float32(1) - np.float32(0.9))
    checked = 0
    for (prev, gs, curw, out, post) in hist:
        pos = np.flatnonzero(oracle.unpack(curw, lay.n_pad))
        if pos.size == 0:
            continue
        a = np.array([prev.r[i][pos].astype(np.float64) + bf16_to_f64(gs[i])[pos] for i in range(wl.W)])
        dense = a.mean(0)
        mo = prev.m[pos].astype(np.float64)
        ghat = (post.m[pos].astype(np.float64) - b1 * mo) / c1
        mt = np.abs(b1 * mo[None, :] + c1 * a).max(0)
        bound = (wl.W + 6) * U * (b1 * np.abs(mo) + mt) / c1
        assert np.all(np.abs(ghat - dense) <= bound)
        checked += pos.size
    assert checked > 0


def test_keep_one_reduces_to_dense_adams_fp64():
    """keep=1 from an all-ones mask: no residual, and m, v, x follow a dense
    fp64 AdamS on the mean gradient (the normaliser reading of the oracle),
    within a first-order fp32 rounding-error bound propagated over the steps."""
    W, T = 4, 5
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, 1, 1, W)
    hp = oracle.Hyper()
    rng = np.random.default_rng(4)
    x0 = (rng.standard_normal(lay.n_pad) * 0.02).astype(np.float32)
    inl = layer_mask(lay)
    cur = oracle.pack(inl.astype(np.uint8))
    grads = {t: random_grads(rng, lay, W) for t in range(1, T + 1)}
    hist = _run(lay, W, T, hp, lambda t: grads[t], cur=cur, x=x0)
    b1, b2 = np.float64(np.float32(0.9)), np.float64(np.float32(0.95))
    c1, c2 = 1 - b1, 1 - b2  # exact: these equal the fp32 constants
    lr, eps = np.float64(np.float32(1e-3)), np.float64(np.float32(1e-8))
    x, m, v = x0.astype(np.float64), np.zeros(lay.n_pad), np.zeros(lay.n_pad)
    Em = np.zeros(lay.n_pad)  # bound on |m_fp32 - m_fp64|
    Ex = np.zeros(lay.n_pad)  # bound on |x_fp32 - x_fp64|
    for t, (prev, gs, _, out, post) in enumerate(hist, 1):
        for i in range(W):
            assert not post.r[i].any()
        g = np.array([bf16_to_f64(gi) for gi in gs])
        gbar = g.mean(0)
        mo = m
        v = b2 * mo * mo + c2 * gbar * gbar
        m = b1 * mo + c1 * gbar
        x_new = x - lr * m / (np.sqrt(v) + eps)
        # candidates: 2 roundings each, W-1 in the sum; the previous error scaled by beta1
        mt_abs = b1 * np.abs(mo) + c1 * np.abs(g).max(0)
        Em_new = b1 * Em + (W + 3) * U * mt_abs
        # g_hat = (bbar - beta1*mo)/c1 and v = beta2*mo^2 + c2*g_hat^2
        Eg = (Em_new + b1 * Em + 3 * U * (np.abs(m) + b1 * np.abs(mo))) / c1 + U * np.abs(gbar)
        Ev = 2 * b2 * np.abs(mo) * Em + 2 * c2 * np.abs(gbar) * Eg + c2 * Eg * Eg + 4 * U * v
        den = np.sqrt(v) + eps
        Eq = Em_new / den + np.abs(m) * (Ev / (2 * np.sqrt(v) + 1e-300)) / den ** 2 + 4 * U * np.abs(m) / den
        Ex = Ex + lr * Eq + 2 * U * (np.abs(x_new) + lr * np.abs(m) / den)
        x, Em = x_new, Em_new
        sl = inl
        assert np.all(np.abs(post.m[sl] - m[sl]) <= 2 * Em[sl]), t
        assert np.all(np.abs(post.v[sl] - v[sl]) <= 2 * Ev[sl]), t
        assert np.all(np.abs(post.x[sl] - x[sl]) <= 2 * Ex[sl]), t
        assert np.array_equal(oracle.unpack(out.next_words, lay.n_pad), inl.astype(np.uint8))
    # the bound is tight enough to matter: a typical element agrees to ~1e-6 relative
    assert np.median(Ex[inl] / np.abs(x[inl])) < 1e-5


def test_single_worker_sends_its_candidate_unchanged():
    lay = oracle.layout([4096, 640], 1, 1, 1)
    rng = np.random.default_rng(8)
    inl = layer_mask(lay)
    hist = _run(lay, 1, 2, oracle.Hyper(), lambda t: random_grads(rng, lay, 1),
                cur=oracle.pack(inl.astype(np.uint8)))
    for (prev, gs, _, out, post) in hist:
        assert np.array_equal(out.bbar, out.sent[0])
        pos = np.flatnonzero(inl)
        assert np.array_equal(post.m[pos], out.sent[0])


def test_power_of_two_scaling_is_exact():
    """Gradients times 2^p (zero start, eps=0): m, r, sent scale by 2^p, v by
    4^p, masks and x are identical."""
    wl = synth.reduced(synth.LLAMA055)
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hp = oracle.Hyper(eps=0.0)
    x0 = synth.params_flat(wl, lay.off, lay.n_pad)
    base = {t: synth_grads(wl, lay, t) for t in (1, 2, 3)}
    ref = _run(lay, wl.W, 3, hp, lambda t: base[t], x=x0)
    for p in (-3, 4):
        def scaled(t):
            return [bf16_bits((g.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** p)) for g in base[t]]
        got = _run(lay, wl.W, 3, hp, scaled, x=x0)
        for (_, _, _, o1, s1), (_, _, _, o2, s2) in zip(ref, got):
            assert np.array_equal(o1.next_words, o2.next_words)
            # eps=0 makes 0/0 = NaN where the accumulated gradient is exactly 0, on both sides
            assert np.array_equal(s1.x, s2.x, equal_nan=True)
            assert np.array_equal(s1.m * np.float32(2.0 ** p), s2.m)
            assert np.array_equal(s1.v * np.float32(4.0 ** p), s2.v)
            for i in range(wl.W):
                assert np.array_equal(s1.r[i] * np.float32(2.0 ** p), s2.r[i])
                assert np.array_equal(o1.sent[i] * np.float32(2.0 ** p), o2.sent[i])


def test_statistic_at_t_does_not_touch_step_t_updates():
    """The mask built at t is only used at t+1: a different owner (a different
    statistic) changes M_{t+1} but nothing that step t writes."""
    wl = synth.reduced(synth.LLAMA175)
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    gs = synth_grads(wl, lay, 1)
    rng = np.random.default_rng(2)
    cur = oracle.pack((rng.random(lay.n_pad) < 0.05).astype(np.uint8) & layer_mask(lay))
    x0 = synth.params_flat(wl, lay.off, lay.n_pad)
    s1 = oracle.State.zeros(lay.n_pad, wl.W, x0)
    s2 = s1.copy()
    o1 = oracle.step(lay, oracle.Hyper(), s1, gs, cur)
    o2 = oracle.step(lay, oracle.Hyper(), s2, gs, cur, owner_map=(lay.owner + 1) % wl.W)
    assert not np.array_equal(o1.next_words, o2.next_words)
    for a, b in zip([s1.x, s1.m, s1.v] + s1.r, [s2.x, s2.m, s2.v] + s2.r):
        assert np.array_equal(a, b)
    for i in range(wl.W):
        assert np.array_equal(o1.sent[i], o2.sent[i])


def test_off_mask_state_is_unchanged():
    wl = synth.reduced(synth.ADVERSARIAL)
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    x0 = synth.params_flat(wl, lay.off, lay.n_pad)
    hist = _run(lay, wl.W, 3, oracle.Hyper(), lambda t: synth_grads(wl, lay, t), x=x0)
    for (prev, _, curw, out, post) in hist:
        on = oracle.unpack(curw, lay.n_pad).astype(bool)
        for a, b in ((prev.x, post.x), (prev.m, post.m), (prev.v, post.v)):
            assert np.array_equal(a[~on], b[~on])
        if on.any():
            assert np.array_equal(post.m[on], out.bbar)


def test_next_index_and_prefix_are_consistent():
    wl = synth.reduced(synth.GPT345M)
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    hist = _run(lay, wl.W, 2, oracle.Hyper(), lambda t: synth_grads(wl, lay, t))
    for (_, _, _, out, _) in hist:
        pred = oracle.unpack(out.next_words, lay.n_pad)
        assert np.array_equal(out.next_idx, np.flatnonzero(pred))
        assert np.all(np.diff(out.next_idx.astype(np.int64)) > 0)
        assert np.array_equal(out.next_prefix, np.concatenate([[0], np.cumsum(popcount_words(out.next_words))]))


def test_sub_layout_reproduces_full_run_on_its_layers():
    """Layers are independent: the oracle on a subset of layers (keeping their
    k and owner) equals the full run on those layers.  Full-size GPU parity
    relies on this to check sampled layers."""
    wl = synth.reduced(synth.LLAMA175)
    full = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    pick = [1, 5, 9, 14]
    sub = oracle.sub_layout(full, pick)
    hf = _run(full, wl.W, 3, oracle.Hyper(), lambda t: synth_grads(wl, full, t))
    hs = _run(sub, wl.W, 3, oracle.Hyper(), lambda t: synth_grads(wl, sub, t, pick))
    for (_, _, _, of, sf), (_, _, _, os_, ss) in zip(hf, hs):
        for a, l in enumerate(pick):
            fs = slice(full.off[l], full.off[l] + full.sizes[l])
            ssl = slice(sub.off[a], sub.off[a] + sub.sizes[a])
            for x, y in zip([sf.x, sf.m, sf.v] + sf.r, [ss.x, ss.m, ss.v] + ss.r):
                assert np.array_equal(x[fs], y[ssl])
            assert np.array_equal(oracle.unpack(of.next_words, full.n_pad)[fs],
                                  oracle.unpack(os_.next_words, sub.n_pad)[ssl])


# --------------------------------------------------------------------------
# the dense AdamS step (comparison baseline)


def _bf16_layer(lay, vals_by_layer):
    g = np.zeros(lay.n_pad, np.uint16)
    for l, vals in enumerate(vals_by_layer):
        g[lay.off[l]:lay.off[l] + len(vals)] = bf16_bits(vals)
    return g


@pytest.mark.parametrize("run,steps", [("A", 2), ("B", 1)])
def test_dense_golden_worked_steps(run, steps):
    d = _parse_golden("dense_adams.txt")
    n, W = int(d[f"{run}.n"]), int(d[f"{run}.W"])
    lay = oracle.layout([n], 1, 1, W)
    hp = oracle.Hyper(float(d[f"{run}.beta1"]), float(d[f"{run}.beta2"]), float(d[f"{run}.lr"]),
                      float(d[f"{run}.eps"]), float(d[f"{run}.wd"]))
    x = np.zeros(lay.n_pad, np.float32)
    x[:n] = _vals(d[f"{run}.x0"])
    m, v = np.zeros_like(x), np.zeros_like(x)
    for t in range(1, steps + 1):
        gs = [_bf16_layer(lay, [_vals(d[f"{run}.step{t}.g{i}"])]) for i in range(W)]
        oracle.dense_step(lay, hp, x, m, v, gs)
        assert np.array_equal(m[:n], _vals(d[f"{run}.step{t}.m"])), t
        assert np.array_equal(v[:n], _vals(d[f"{run}.step{t}.v"])), t
        assert np.array_equal(x[:n], _vals(d[f"{run}.step{t}.x"])), t
        assert not x[n:].any() and not m[n:].any() and not v[n:].any()  # padding untouched


def test_dense_agrees_with_scape_under_a_full_mask():
    """With every position masked at every step and zero residuals, the SCAPE
    step reaches m, v, x through the synchronized first-moment buffer and the
    reconstructed gradient; the dense step computes them from the averaged
    gradient directly.  Both are fp32 evaluations of the same exact values, so
    they differ by at most the sum of their rounding-error bounds (the bound of
    the keep=1 pin, propagated over the steps, taken for each side)."""
    W, T = 4, 5
    wl = synth.ragged()
    lay = oracle.layout(wl.layer_sizes, 1, 1, W)
    hp = oracle.Hyper()
    rng = np.random.default_rng(21)
    x0 = (rng.standard_normal(lay.n_pad) * 0.02).astype(np.float32)
    inl = layer_mask(lay)
    x0[~inl] = 0
    cur = oracle.pack(inl.astype(np.uint8))
    grads = {t: random_grads(rng, lay, W) for t in range(1, T + 1)}
    hist = _run(lay, W, T, hp, lambda t: grads[t], cur=cur, x=x0)
    x, m, v = x0.copy(), np.zeros_like(x0), np.zeros_like(x0)
    b1, b2 = np.float64(np.float32(0.9)), np.float64(np.float32(0.95))
    c1, c2 = 1 - b1, 1 - b2
    lr, eps = np.float64(np.float32(1e-3)), np.float64(np.float32(1e-8))
    Em, Ex = np.zeros(lay.n_pad), np.zeros(lay.n_pad)
    m64 = np.zeros(lay.n_pad)
    for t, (prev, gs, _, out, post) in enumerate(hist, 1):
        oracle.dense_step(lay, hp, x, m, v, gs)
        # magnitudes for the bound, from the exact values in fp64
        g = np.array([bf16_to_f64(gi) for gi in gs])
        gbar = g.mean(0)
        mo = m64
        v64 = b2 * mo * mo + c2 * gbar * gbar
        m64 = b1 * mo + c1 * gbar
        mt_abs = b1 * np.abs(mo) + c1 * np.abs(g).max(0)
        Em_new = b1 * Em + (W + 3) * U * mt_abs
        Eg = (Em_new + b1 * Em + 3 * U * (np.abs(m64) + b1 * np.abs(mo))) / c1 + U * np.abs(gbar)
        Ev = 2 * b2 * np.abs(mo) * Em + 2 * c2 * np.abs(gbar) * Eg + c2 * Eg * Eg + 4 * U * v64
        den = np.sqrt(v64) + eps
        Eq = Em_new / den + np.abs(m64) * (Ev / (2 * np.sqrt(v64) + 1e-300)) / den ** 2 + 4 * U * np.abs(m64) / den
        Ex = Ex + lr * Eq + 2 * U * (np.abs(post.x) + lr * np.abs(m64) / den)
        Em = Em_new
        sl = inl
        assert np.all(np.abs(m[sl] - post.m[sl]) <= 4 * Em[sl]), t
        assert np.all(np.abs(v[sl] - post.v[sl]) <= 4 * Ev[sl]), t
        assert np.all(np.abs(x[sl] - post.x[sl]) <= 4 * Ex[sl]), t
        assert not x[~inl].any() and not m[~inl].any() and not v[~inl].any()
    # the two are different computations, not the same one twice
    assert not np.array_equal(m[inl], hist[-1][4].m[inl])
    # and the bound is tight enough to matter
    assert np.median(Ex[inl] / np.abs(x[inl])) < 1e-5


def test_dense_power_of_two_scaling_is_exact():
    """Gradients times 2^p from a zero start with eps=0: m scales by 2^p, v by
    4^p, and the update m/sqrt(v) - hence x - is unchanged, bit for bit."""
    W = 3
    lay = oracle.layout([1000, 37, 4096], 1, 1, W)
    rng = np.random.default_rng(22)
    hp = oracle.Hyper(eps=0.0)
    x0 = (rng.standard_normal(lay.n_pad) * 0.02).astype(np.float32)
    gseq = [random_grads(rng, lay, W) for _ in range(3)]
    ref = (x0.copy(), np.zeros_like(x0), np.zeros_like(x0))
    for gs in gseq:
        oracle.dense_step(lay, hp, *ref, gs)
    for p in (-5, 3):
        got = (x0.copy(), np.zeros_like(x0), np.zeros_like(x0))
        for gs in gseq:
            sg = [bf16_bits((gi.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** p)) for gi in gs]
            oracle.dense_step(lay, hp, *got, sg)
        assert np.array_equal(ref[0], got[0], equal_nan=True)
        assert np.array_equal(ref[1] * np.float32(2.0 ** p), got[1])
        assert np.array_equal(ref[2] * np.float32(4.0 ** p), got[2])


def test_dense_sign_symmetry_is_exact():
    """Negated gradients from x = m = v = 0 give negated m and x and the same
    v (round to nearest even is symmetric), and a single worker's step sees its
    own gradient unchanged by the mean."""
    W = 2
    lay = oracle.layout([3000, 65], 1, 1, W)
    rng = np.random.default_rng(23)
    hp = oracle.Hyper()
    gseq = [random_grads(rng, lay, W) for _ in range(3)]
    a = [np.zeros(lay.n_pad, np.float32) for _ in range(3)]
    b = [np.zeros(lay.n_pad, np.float32) for _ in range(3)]
    for gs in gseq:
        oracle.dense_step(lay, hp, *a, gs)
        oracle.dense_step(lay, hp, *b, [gi ^ np.uint16(0x8000) for gi in gs])
    assert np.array_equal(a[0], -b[0]) and np.array_equal(a[1], -b[1]) and np.array_equal(a[2], b[2])
    # W = 2 with identical workers equals W = 1: the mean of equal values is exact
    one = [np.zeros(lay.n_pad, np.float32) for _ in range(3)]
    two = [np.zeros(lay.n_pad, np.float32) for _ in range(3)]
    for gs in gseq:
        oracle.dense_step(lay, hp, *one, [gs[0]])
        oracle.dense_step(lay, hp, *two, [gs[0], gs[0]])
    for u, w in zip(one, two):
        assert np.array_equal(u, w)


# --------------------------------------------------------------------------
# the fill-in union (each worker ranks every layer; the masks are OR-ed)


def _union_brute(lay, keys):
    sel = np.zeros(lay.n_pad, bool)
    for kk in keys:
        for l in range(lay.L):
            o, n, k = int(lay.off[l]), int(lay.sizes[l]), int(lay.k[l])
            order = sorted(range(n), key=lambda j: (-int(kk[o + j]), j))
            for j in order[:k]:
                sel[o + j] = True
    return sel


def test_union_hand_example_with_ties():
    """Two workers, one layer of 6, k = 2 (keep 1/3).  Worker 0's keys
    [5,5,5,1,1,1] tie three ways at the top: positions 0 and 1 win.  Worker 1's
    [0,0,9,9,9,0]: positions 2 and 3.  The union is {0,1,2,3}: four bits, the
    fill-in of two masks of two."""
    lay = oracle.layout([6], 1, 3, 2)
    k0 = np.zeros(lay.n_pad, np.uint32)
    k1 = np.zeros(lay.n_pad, np.uint32)
    k0[:6] = [5, 5, 5, 1, 1, 1]
    k1[:6] = [0, 0, 9, 9, 9, 0]
    got = oracle.unpack(oracle.union_mask(lay, [k0, k1]), lay.n_pad)
    assert np.flatnonzero(got).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("W", [1, 2, 5])
@pytest.mark.parametrize("levels", [3, 50, 1 << 31])
def test_union_matches_brute_force(W, levels):
    rng = np.random.default_rng(W * 1000 + levels % 997)
    lay = oracle.layout([1, 7, 64, 130, 333], 1, 4, W)
    keys = [rng.integers(0, levels, lay.n_pad).astype(np.uint32) for _ in range(W)]
    got = oracle.unpack(oracle.union_mask(lay, keys), lay.n_pad).astype(bool)
    assert np.array_equal(got, _union_brute(lay, keys))


def test_union_bounds_and_monotone_in_workers():
    """Per layer the union has between k and min(n, W*k) bits, and adding a
    worker never removes one."""
    rng = np.random.default_rng(31)
    lay = oracle.layout([5000, 777, 64, 1], 1, 20, 8)
    keys = [rng.integers(0, 1 << 20, lay.n_pad).astype(np.uint32) for _ in range(8)]
    prev = None
    for w in range(1, 9):
        bits = oracle.unpack(oracle.union_mask(lay, keys[:w]), lay.n_pad).astype(bool)
        for l in range(lay.L):
            c = int(bits[lay.off[l]:lay.off[l] + lay.sizes[l]].sum())
            assert lay.k[l] <= c <= min(lay.sizes[l], w * lay.k[l]), (w, l, c)
            assert not bits[lay.off[l] + lay.sizes[l]:lay.off[l] + (lay.sizes[l] + 63) // 64 * 64].any()
        if prev is not None:
            assert np.all(bits[prev])
        prev = bits


def test_union_of_disjoint_and_of_identical_workers():
    """Worker i's largest keys on its own block of k positions: the union is
    exactly the first W*k positions.  W identical workers: the union is one
    worker's mask."""
    W, k = 4, 25
    n = 3 * W * k
    lay = oracle.layout([n], k, n, W)
    assert lay.k.tolist() == [k]
    rng = np.random.default_rng(32)
    keys = []
    for i in range(W):
        kk = np.zeros(lay.n_pad, np.uint32)
        kk[:n] = rng.integers(0, 1000, n)
        kk[i * k:(i + 1) * k] = rng.integers(10_000, 20_000, k)
        keys.append(kk)
    got = oracle.unpack(oracle.union_mask(lay, keys), lay.n_pad)
    assert np.flatnonzero(got).tolist() == list(range(W * k))
    one = oracle.union_mask(lay, keys[:1])
    assert np.array_equal(oracle.union_mask(lay, [keys[0]] * W), one)
    assert np.array_equal(one, oracle.mask_from_keys(lay, keys[0]))


_THREAD_PROBE = r"""
import hashlib, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle, synth
wl = synth.reduced(synth.GPT345M)
lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
st = oracle.State.zeros(lay.n_pad, wl.W, synth.params_flat(wl, lay.off, lay.n_pad))
cur = np.zeros(lay.n_words, np.uint64)
h = hashlib.sha256()
for t in (1, 2, 3):
    out = oracle.step(lay, oracle.Hyper(wl.beta1, wl.beta2, wl.lr, wl.eps, 0.01), st,
                      [synth.grads_flat(wl, lay.off, lay.n_pad, t, i) for i in range(wl.W)], cur)
    cur = out.next_words
    for a in [st.x, st.m, st.v, cur, out.bbar] + st.r + out.sent:
        h.update(a.tobytes())
print(oracle.threads(), h.hexdigest())
"""


def test_oracle_results_do_not_depend_on_thread_count():
    """The oracle's loops run in parallel over layers and positions, never
    splitting a floating-point sum: one thread and several give the same bits."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for n in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        r = subprocess.run([sys.executable, "-c", _THREAD_PROBE, root], env=env, capture_output=True, text=True,
                           check=True)
        outs.append(r.stdout.split())
    assert outs[0][0] == "1" and outs[1][0] == "4"
    assert outs[0][1] == outs[1][1]
