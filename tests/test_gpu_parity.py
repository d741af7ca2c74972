"""Parity of the HIP path (through the C ABI) with the oracle, on a GPU.

The bar: masks, index lists, prefixes, statistic keys and packed bits
bit-exact; fp32 state within rel 1e-5 / abs 1e-7 of the oracle (the harness
also counts positions that are not bit-exact; the fp32 operation order is the
same on both sides, so the expected count is zero and the tests assert it).
"""
import dataclasses
import gc

import numpy as np
import pytest

import oracle
import synth
from harness import GpuSession, log, release, run_parity, scape_config, to_np, u32, u64

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


def _ctx(sizes, W=2, keep=(1, 10), path=None):
    import sparse_communication_adam_amd as sc
    ctx = sc.scape_init(sc.ScapeConfig(layer_numel=list(sizes), workers=W, keep_num=keep[0], keep_den=keep[1]))
    if path is not None:
        sc.scape_set_select_path(ctx, path)
    return ctx


# The two ways of selecting a mask (the sampled multi-pass path and the
# two-launch compact path, which the library takes by default where every
# layer of a range has at most 2^22 elements): both must give the oracle's
# mask, so the tests that build masks run each of them.
SAMPLED, COMPACT = 1, 2
PATHS = pytest.mark.parametrize("path", [SAMPLED, COMPACT], ids=["sampled", "compact"])


# ----------------------------------------------------------------------------
# inputs: the GPU generator twin equals the host generator


@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "adversarial-ties"])
def test_gpu_generator_matches_host(name):
    import torch
    wl = synth.WORKLOADS[name]
    lay = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    tensors = sorted({t for t in (0, 1, 2, 10, len(wl.tensors) - 1) if t < len(wl.tensors)})
    sub = oracle.sub_layout(lay, tensors)
    for step, worker in [(1, 0), (3, wl.W - 1)]:
        g = torch.zeros(sub.n_pad, dtype=torch.int16, device="cuda")
        synth.grads_flat_gpu(wl, sub.off, g, step, worker, tensors)
        host = synth.grads_flat(wl, sub.off, sub.n_pad, step, worker, tensors)
        assert np.array_equal(to_np(g).view(np.uint16), host)
    x = torch.zeros(sub.n_pad, dtype=torch.float32, device="cuda")
    synth.params_flat_gpu(wl, sub.off, x, tensors)
    assert np.array_equal(to_np(x).view(np.uint32), synth.params_flat(wl, sub.off, sub.n_pad, tensors).view(np.uint32))


# ----------------------------------------------------------------------------
# kernels one by one


# sizes around the 16-element lane and 1024-element wave chunks, and one with
# more chunks than the grid covers in a trip; offset 0 takes the 16-byte
# path, offsets 1 and 8 (pred not 16-byte aligned) the byte path
@pytest.mark.parametrize("n", [1, 15, 16, 17, 63, 64, 65, 1000, 1023, 1024, 1025, 100003, (1 << 20) + 17,
                               (1 << 26) + 1043])
@pytest.mark.parametrize("offset", [0, 1, 8])
def test_pack_unpack(n, offset):
    import torch
    import sparse_communication_adam_amd as sc
    if offset and n > (1 << 21):
        pytest.skip("the byte path is covered at the smaller sizes")
    rng = np.random.default_rng(n + offset)
    pred = (rng.random(n) < 0.3).astype(np.uint8)
    pred[rng.integers(0, n, 3)] = 7  # any nonzero byte counts as set
    pred[rng.integers(0, n, 3)] = 0x80
    buf = torch.zeros(n + offset, dtype=torch.uint8, device="cuda")
    d_pred = buf[offset:]
    d_pred.copy_(torch.from_numpy(pred))
    bits = torch.full(((n + 63) // 64,), -1, dtype=torch.int64, device="cuda")
    sc.scape_pack(d_pred, bits)
    assert np.array_equal(u64(bits), oracle.pack(pred != 0))
    out = torch.full((n + offset + 16,), 0xA5, dtype=torch.uint8, device="cuda")
    back = out[offset:offset + n]
    sc.scape_unpack(bits, back)
    assert np.array_equal(to_np(back), (pred != 0).astype(np.uint8))
    rest = to_np(out)
    assert (rest[:offset] == 0xA5).all() and (rest[offset + n:] == 0xA5).all()  # nothing outside the range


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8, 32])
@pytest.mark.parametrize("k", [0, 1, 4097, (1 << 20) + 3])
def test_reduce_sparse(W, k):
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(W * 7 + k)
    bufs = [(rng.standard_normal(max(k, 1)) * 10.0 ** rng.integers(-8, 3, max(k, 1))).astype(np.float32)
            for _ in range(W)]
    d = [torch.from_numpy(b).cuda() for b in bufs]
    out = torch.full((max(k, 1),), 7.0, device="cuda")
    sc.scape_reduce_sparse(d, out, k)
    if k:
        assert np.array_equal(to_np(out)[:k].view(np.uint32), oracle.reduce([b[:k] for b in bufs]).view(np.uint32))
    else:
        assert to_np(out)[0] == 7.0


def _mtilde_cases():
    rng = np.random.default_rng(42)
    return {
        "normal": lambda n: rng.standard_normal(n).astype(np.float32) * 1e-3,
        "levels16": lambda n: (rng.integers(-8, 8, n) * 2.0 ** -12).astype(np.float32),
        "all_equal": lambda n: np.full(n, -0.25, np.float32),
        "zeros": lambda n: np.zeros(n, np.float32),
        "pm_pairs": lambda n: np.repeat(rng.standard_normal((n + 1) // 2).astype(np.float32), 2)[:n]
        * np.tile(np.float32([1, -1]), (n + 1) // 2)[:n],
        "specials": lambda n: np.where(rng.random(n) < 0.01, np.float32(np.inf),
                                       np.where(rng.random(n) < 0.005, np.float32(np.nan),
                                                rng.standard_normal(n).astype(np.float32))),
        "narrow": lambda n: (1.0 + rng.integers(0, 3000, n) * 2.0 ** -23).astype(np.float32),
        # 2% of the keys in one cluster of 50 values inside one run of 64 keys
        # (each tied some hundred times), the rest far below: at keep 1/100 the
        # threshold lies in the cluster, so the position digits decide among
        # records whose keys share all but their lowest 6 bits
        "cluster": lambda n: np.where(rng.random(n) < 0.02,
                                      (1.0 + rng.integers(0, 50, n) * 2.0 ** -23).astype(np.float32),
                                      (rng.standard_normal(n) * 1e-3).astype(np.float32)).astype(np.float32),
    }


@PATHS
@pytest.mark.parametrize("case", list(_mtilde_cases()))
@pytest.mark.parametrize("keep", [(0, 1), (1, 1000), (1, 100), (1, 10), (1, 2), (1, 1)])
def test_mask_build_matches_oracle(case, keep, path):
    import torch
    import sparse_communication_adam_amd as sc
    sizes = [1, 37, 1000, 64, 4097, 70000, 1 << 20, 300001]
    ctx = _ctx(sizes, W=3, keep=keep, path=path)
    lay = oracle.layout(sizes, keep[0], keep[1], 3)
    mt = np.zeros(lay.n_pad, np.float32)
    gen = _mtilde_cases()[case]
    for off, n in zip(lay.off, lay.sizes):
        mt[off:off + n] = gen(int(n))
    out = sc.alloc_mask(ctx.layout)
    out.bits.fill_(-1)
    sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
    exp_bits = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    exp_idx, exp_pre, cnt = oracle.mask_index(exp_bits)
    assert cnt == lay.k_total
    got = u64(out.bits)
    if not np.array_equal(got, exp_bits):
        g = oracle.unpack(got, lay.n_pad)
        e = oracle.unpack(exp_bits, lay.n_pad)
        j = int(np.flatnonzero(g != e)[0])
        raise AssertionError(f"{case} keep={keep}: first difference at {j}: gpu {g[j]} oracle {e[j]} "
                             f"key {oracle.keys_of(mt[j:j + 1])[0]:#x}")
    assert np.array_equal(u32(out.idx)[:cnt], exp_idx)
    assert np.array_equal(u32(out.block_prefix), exp_pre)
    ctx.destroy()


@PATHS
def test_mask_build_heavy_ties_across_many_candidate_blocks(path):
    """One 6M-element layer of 16 levels: the threshold key is tied across
    hundreds of thousands of positions spread over many candidate blocks, so
    every position-digit pass runs (on the compact path, one workgroup
    resolves those records, or at keep 1/3 the layer's keys)."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(5)
    sizes = [6_000_000, 4096]
    for keep in [(1, 1000), (37, 1000), (1, 3)]:
        ctx = _ctx(sizes, W=2, keep=keep, path=path)
        lay = oracle.layout(sizes, keep[0], keep[1], 2)
        mt = (rng.integers(-8, 8, lay.n_pad) * 2.0 ** -12).astype(np.float32)
        out = sc.alloc_mask(ctx.layout)
        sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
        exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
        assert np.array_equal(u64(out.bits), exp), keep
        ctx.destroy()


@PATHS
@pytest.mark.parametrize("case,keep,want_flags", [
    ("normal", (1, 100), 0),          # records fit: no fallback
    ("levels16", (1, 2), 3),          # window and exact bucket both beyond the record space
    ("all_equal", (1, 10), 3),        # one bucket holds every key
    ("zeros", (37, 1000), 3),
])
def test_mask_build_record_space_overflow(case, keep, want_flags, path):
    """A record segment holds 1/16 of its elements plus 1024 records.  When a
    layer's window holds more, the layer is redone from an exact histogram;
    when even its exact threshold bucket does not fit, the remaining digits
    are decided by passes over its keys.  The mask is the oracle's either
    way, and scape_selection_flags reports which path ran (the compact path
    has no window: only its exact bucket can overflow)."""
    import torch
    import sparse_communication_adam_amd as sc
    if path == COMPACT:
        want_flags &= sc.SELECT_KEY_PASSES
    sizes = [2_000_000, 300_001, 5000]
    ctx = _ctx(sizes, W=2, keep=keep, path=path)
    lay = oracle.layout(sizes, keep[0], keep[1], 2)
    gen = _mtilde_cases()[case]
    mt = np.zeros(lay.n_pad, np.float32)
    for off, n in zip(lay.off, lay.sizes):
        mt[off:off + n] = gen(int(n))
    out = sc.alloc_mask(ctx.layout)
    sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
    flags = sc.scape_selection_flags(ctx)
    exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    assert np.array_equal(u64(out.bits), exp), (case, keep, flags)
    idx, pre, cnt = oracle.mask_index(exp)
    assert np.array_equal(u32(out.idx)[:cnt], idx) and np.array_equal(u32(out.block_prefix), pre)
    assert flags == want_flags, (case, keep, flags)
    ctx.destroy()


@PATHS
def test_mask_build_alternating_inputs(path):
    """Two inputs built in turn, twenty times each, on one context: every
    build must be its own input's mask, not one made from records or counts
    the other build left behind (the compact path hands records and counts
    between workgroups of one launch)."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(13)
    sizes = [1 << 20, 300_001, 4097]
    ctx = _ctx(sizes, W=2, keep=(1, 10), path=path)
    lay = oracle.layout(sizes, 1, 10, 2)
    ins, exps = [], []
    for scale in (1e-3, 3e-3):
        mt = (rng.standard_normal(lay.n_pad) * scale).astype(np.float32)
        ins.append(torch.from_numpy(mt).cuda())
        exps.append(oracle.mask_from_keys(lay, oracle.keys_of(mt)))
    out = sc.alloc_mask(ctx.layout)
    for it in range(40):
        sc.scape_mask_build(ctx, ins[it % 2], out)
        assert np.array_equal(u64(out.bits), exps[it % 2]), f"build {it}"
    ctx.destroy()


@PATHS
def test_mask_build_more_segments_than_lds_map(path):
    """Over 4096 record segments (one per tiny layer)."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(11)
    sizes = [int(x) for x in rng.integers(1, 300, 5000)] + [600_000]
    for keep in [(1, 10), (1, 2)]:
        ctx = _ctx(sizes, W=2, keep=keep, path=path)
        lay = oracle.layout(sizes, keep[0], keep[1], 2)
        mt = (rng.standard_normal(lay.n_pad) * 1e-3).astype(np.float32)
        out = sc.alloc_mask(ctx.layout)
        sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
        exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
        assert np.array_equal(u64(out.bits), exp), keep
        idx, pre, cnt = oracle.mask_index(exp)
        assert np.array_equal(u32(out.idx)[:cnt], idx) and np.array_equal(u32(out.block_prefix), pre)
        ctx.destroy()


@PATHS
def test_mask_build_empty_layers(path):
    """Zero-size layers own no words, tiles or record segments; a shard that
    owns only empty layers writes nothing."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(12)
    sizes = [0, 100, 0, 0, 5000, 0]
    ctx = _ctx(sizes, W=2, keep=(1, 10), path=path)
    lay = oracle.layout(sizes, 1, 10, 2)
    mt = (rng.standard_normal(lay.n_pad) * 1e-3).astype(np.float32)
    d_mt = torch.from_numpy(mt).cuda()
    out = sc.alloc_mask(ctx.layout)
    sc.scape_mask_build(ctx, d_mt, out)
    exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    assert np.array_equal(u64(out.bits), exp)
    owners = sc.scape_owner_map(ctx.cfg, 6)
    for s in range(6):
        out.bits.fill_(7)
        sc.scape_mask_build(ctx, d_mt, out, num_shards=6, shard=s)
        got = u64(out.bits)
        for l in range(lay.L):
            w0, w1 = lay.off[l] // 64, (lay.off[l] + lay.sizes[l] + 63) // 64
            want = exp[w0:w1] if owners[l] == s else np.full(w1 - w0, 7, np.uint64)
            assert np.array_equal(got[w0:w1], want), (s, l)
    ctx.destroy()


def _sampled_words(lw0, lwords):
    """Words the key-sampling pass reads in a layer of more than 4096 words:
    one per aligned group of 16, at a hashed offset (the kernel's rule,
    restated here to build inputs that defeat the sample)."""
    out = []
    for g in range((lwords + 15) // 16):
        w = lw0 + (g << 4)
        h = (w * 0x9E3779B1) & 0xFFFFFFFF
        h ^= h >> 15
        h = (h * 0x85EBCA77) & 0xFFFFFFFF
        h ^= h >> 13
        if (g << 4) + (h & 15) < lwords:
            out.append(w + (h & 15))
    return np.array(out, np.int64)


@PATHS
@pytest.mark.parametrize("sampled_small", [True, False])
def test_mask_build_exact_after_a_sampling_miss(sampled_small, path):
    """The sampled words hold values unlike the rest of the layer, so the
    sample's window misses the k-th key: the exact fallback (full first-digit
    histogram and reclassification) must still give the oracle's mask.  (The
    compact path samples nothing; the same input checks it too.)"""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(41 + sampled_small)
    sizes = [400_000, 5000]
    keep = (1, 10)
    ctx = _ctx(sizes, W=2, keep=keep, path=path)
    lay = oracle.layout(sizes, keep[0], keep[1], 2)
    n0 = sizes[0]
    small = (rng.random(lay.n_pad) * 0.5 + 0.5).astype(np.float32) * np.float32(2.0 ** -10)
    large = (rng.random(lay.n_pad) * 0.5 + 0.5).astype(np.float32) * np.float32(2.0 ** 10)
    sampled = np.zeros(lay.n_pad, bool)
    for w in _sampled_words(0, (n0 + 63) // 64):
        sampled[w * 64:(w + 1) * 64] = True
    sampled[n0:] = False
    mt = np.where(sampled == sampled_small, small, large).astype(np.float32)
    mt[lay.off[1]:lay.off[1] + sizes[1]] = rng.standard_normal(sizes[1]).astype(np.float32)
    out = sc.alloc_mask(ctx.layout)
    sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
    exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    assert np.array_equal(u64(out.bits), exp)
    idx, pre, cnt = oracle.mask_index(exp)
    assert np.array_equal(u32(out.idx)[:cnt], idx) and np.array_equal(u32(out.block_prefix), pre)
    if path == SAMPLED:
        assert sc.scape_selection_flags(ctx) & sc.SELECT_EXACT_HISTOGRAM
    ctx.destroy()


def test_mask_build_window_wider_than_the_record_histogram():
    """Half of a sampled layer near 2^60, half near 2^-60, keep 1/2: the k-th
    key sits at the edge of an empty gap of about 120 octaves, so the
    sampled window spans thousands of first-digit buckets and the record
    pass counts straight into the global histogram row."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(43)
    sizes = [600_000]
    keep = (1, 2)
    ctx = _ctx(sizes, W=2, keep=keep, path=SAMPLED)
    lay = oracle.layout(sizes, keep[0], keep[1], 2)
    n = sizes[0]
    mag = np.where(rng.random(n) < 0.5, 2.0 ** 60, 2.0 ** -60) * (1.0 + rng.random(n))
    mt = np.zeros(lay.n_pad, np.float32)
    mt[:n] = (mag * np.where(rng.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    out = sc.alloc_mask(ctx.layout)
    sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
    exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    assert np.array_equal(u64(out.bits), exp)
    ctx.destroy()


@PATHS
@pytest.mark.parametrize("P", [3, 32])
def test_mask_build_one_shard_at_a_time(P, path):
    import torch
    import sparse_communication_adam_amd as sc
    wl = synth.reduced(synth.GPT345M)
    ctx = _ctx(wl.layer_sizes, W=wl.W, keep=(1, 10), path=path)
    lay = oracle.layout(wl.layer_sizes, 1, 10, wl.W)
    rng = np.random.default_rng(P)
    mt = (rng.standard_normal(lay.n_pad) * 1e-3).astype(np.float32)
    d_mt = torch.from_numpy(mt).cuda()
    owners = sc.scape_owner_map(ctx.cfg, P)
    keys = oracle.keys_of(mt)
    sentinel = np.int64(0x5A5A5A5A5A5A5A5A)
    out = sc.alloc_mask(ctx.layout)
    gathered = np.zeros(lay.n_words, np.uint64)
    for s in range(P):
        out.bits.fill_(int(sentinel))
        sc.scape_mask_build(ctx, d_mt, out, num_shards=P, shard=s)
        got = u64(out.bits)
        exp = oracle.mask_from_keys(lay, keys, shard=s, owner_map=np.array(owners, np.int32),
                                    words=np.full(lay.n_words, np.uint64(sentinel), np.uint64))
        assert np.array_equal(got, exp), f"shard {s}"
        for l in range(lay.L):
            if owners[l] == s:
                w0, w1 = lay.off[l] // 64, (lay.off[l] + lay.sizes[l] + 63) // 64
                gathered[w0:w1] = got[w0:w1]
    # the gathered shards form the full mask; the index pass then builds idx/prefix
    out.bits.copy_(torch.from_numpy(gathered.view(np.int64)).cuda())
    sc.scape_mask_index(ctx, out)
    full = oracle.mask_from_keys(lay, keys)
    assert np.array_equal(gathered, full)
    idx, pre, cnt = oracle.mask_index(full)
    assert np.array_equal(u32(out.idx)[:cnt], idx) and np.array_equal(u32(out.block_prefix), pre)
    ctx.destroy()


def test_mask_index_of_arbitrary_bits():
    import torch
    import sparse_communication_adam_amd as sc
    sizes = [300_000, 5, 1 << 18]
    ctx = _ctx(sizes, keep=(1, 1))  # k_total = all elements: idx can hold any mask
    lay = oracle.layout(sizes, 1, 1, 2)
    rng = np.random.default_rng(1)
    for dens in (0.0, 0.001, 0.3, 1.0):
        pred = np.zeros(lay.n_pad, np.uint8)
        for off, n in zip(lay.off, lay.sizes):
            pred[off:off + n] = rng.random(int(n)) < dens
        words = oracle.pack(pred)
        m = sc.alloc_mask(ctx.layout)
        m.bits.copy_(torch.from_numpy(words.view(np.int64)).cuda())
        sc.scape_mask_index(ctx, m)
        idx, pre, cnt = oracle.mask_index(words)
        assert np.array_equal(u32(m.idx)[:cnt], idx) and np.array_equal(u32(m.block_prefix), pre)
    ctx.destroy()


# ----------------------------------------------------------------------------
# the whole step


def _assert_bitexact(stats):
    assert stats["float_values"] > 0
    assert stats["float_not_bitexact"] == 0, stats


@PATHS
@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "llama-0.55b", "llama-1.75b", "adversarial-ties"])
def test_step_parity_oracle_sized(name, path):
    """Every output of every step, all layers: the single-layer workload at its
    full size, the others with the same tensor kinds at reduced sizes."""
    wl = synth.WORKLOADS[name]
    small = wl if name == "single-1024x1024" else synth.reduced(wl)
    _assert_bitexact(run_parity(small, wl.steps, select_path=path))


@PATHS
def test_step_parity_ragged_layout(path):
    _assert_bitexact(run_parity(synth.ragged(), 5, select_path=path))


@pytest.mark.parametrize("W", [1, 2, 4, 5, 16])
def test_step_parity_ragged_layout_worker_counts(W):
    """The dense pass takes 8 consecutive words per wave at W = 1 and 4 at
    W = 2..4: the ragged layout's word count leaves the last workgroup
    partly past the end, and its layers end inside words.  W = 5 runs the
    kernels' instance for a worker count without its own, W = 16 its own."""
    _assert_bitexact(run_parity(synth.ragged(), 4, W=W))


@pytest.mark.parametrize("W", [3, 5])
@pytest.mark.parametrize("key_out", [True, False])
def test_step_parity_weight_decay(W, key_out):
    """Decoupled weight decay (wd = 0.1) on the ragged layout, at worker counts
    that are not powers of two (so the mean's division by W rounds): from an
    empty first mask and from a full one, so the decay term is applied at
    masked positions from the first step; off the mask x must not change."""
    wl = dataclasses.replace(synth.ragged(), weight_decay=0.1)
    _assert_bitexact(run_parity(wl, 4, W=W, key_out=key_out))
    _assert_bitexact(run_parity(wl, 3, W=W, key_out=key_out, keep=(1, 1), init_mask_all=True))


def test_step_keep_all_is_dense_from_full_mask():
    wl = synth.ragged()
    _assert_bitexact(run_parity(wl, 4, keep=(1, 1), init_mask_all=True))


def test_step_keep_nothing_only_accumulates():
    _assert_bitexact(run_parity(synth.ragged(), 3, keep=(0, 1), check_buffers=False))


def test_step_single_worker():
    _assert_bitexact(run_parity(synth.reduced(synth.LLAMA055), 3, W=1))


@PATHS
def test_step_zero_gradients_tie_everywhere(path):
    wl = synth.ragged()
    zero = lambda step, worker, t: np.zeros(wl.tensors[t].numel, np.uint16)  # noqa: E731
    _assert_bitexact(run_parity(wl, 3, grad_override=zero, x_zero=True, select_path=path))


# bfloat16 bit patterns of special gradient values: +-Inf, +-0, subnormals
# (smallest and largest), the largest finite value, and quiet NaNs.  Keys are
# the bits of |m-tilde| with the sign cleared, so the NaN an invalid
# operation makes is 0x7FC00000 on both sides whatever its sign.
SPECIAL_BF16 = np.array([0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x7FC0, 0xFFC0], np.uint16)


def _special_grads(wl):
    def grad(step, worker, t):
        n = wl.tensors[t].numel
        rng = np.random.default_rng([step, worker, t, 77])
        g = (rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)).view(np.uint32)
        g = ((g + 0x7FFF + ((g >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even bf16
        hit = rng.random(n) < 0.01
        g[hit] = SPECIAL_BF16[rng.integers(0, SPECIAL_BF16.size, int(hit.sum()))]
        return g
    return grad


@PATHS
@pytest.mark.parametrize("key_out", [True, False])
def test_step_special_gradient_values(key_out, path):
    """1% of every worker's gradients are +-Inf, +-0, subnormal, the largest
    finite bfloat16 or NaN: the masks, indices and keys stay bit-exact and
    the state matches (NaN where the oracle has NaN)."""
    wl = synth.ragged()
    _assert_bitexact(run_parity(wl, 4, grad_override=_special_grads(wl), key_out=key_out, select_path=path))


def test_step_is_deterministic():
    import torch
    wl = synth.reduced(synth.ADVERSARIAL)
    outs = []
    for _ in range(2):
        run = GpuSession(wl)
        for t in range(1, 4):
            run.step(t)
        torch.cuda.synchronize()
        st = run.state
        outs.append([to_np(a).copy() for a in [st.x, st.m, st.v, st.key, st.cur_mask.bits, st.cur_mask.idx]
                     + st.r + st.sparse])
        release(run)
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


FULL_SAMPLES = {
    # tensor indices checked against the oracle; every layer is checked for
    # exact per-layer counts and index consistency
    "gpt-345m": [2, 4, 7, 10, 291],          # ln1.w, qkv.w, ln2.w, fc1.w, final_ln.b
    "llama-0.55b": [1, 3, 4, 6, 97],         # attn_norm, o, mlp_norm, down, final_norm
    "llama-1.75b": [1, 3, 4, 190, 193],      # attn_norm, o, mlp_norm, last o, final_norm
    "adversarial-ties": [1, 2, 10, 18, 20, 1088],  # mat, norm, quantised norm, mat, quantised norm, last norm
}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_step_parity_full_size_sampled_layers(name):
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_parity(wl, wl.steps, sample=FULL_SAMPLES[name]))


# The largest tensor of each workload (and the 1.75B shape's fused gate_up),
# compared against the oracle at full size: their selections keep 131,072 to
# 655,360 positions, and their tie positions reach past 2^25 inside the layer.
FULL_LARGEST = {
    "gpt-345m": [0],              # word_emb, 51.5M elements, keep 1/10
    "llama-0.55b": [0, 98],       # emb and lm_head, 49.2M each
    "llama-1.75b": [0, 5, 194],   # emb, l0.gate_up, lm_head (65.5M, 22.5M, 65.5M)
    "adversarial-ties": [0],      # emb, 131M elements, quantised to 16 levels, W = 32
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(FULL_LARGEST))
def test_step_parity_full_size_largest_layers(name):
    """Three full-size steps in the configuration bench.py times
    (worker-interleaved residuals and gradients, candidates' keys
    recomputed), every output of the largest layers against the oracle."""
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_parity(wl, 3, sample=FULL_LARGEST[name], key_out=False, interleaved=True))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("keep", [(1, 2), (1, 100)])
def test_mask_build_largest_layer_sixteen_levels(keep):
    """One layer of 67,108,927 elements (2^26 + 63, a ragged last word) holding
    16 levels: at keep 1/2 the threshold level is tied over millions of
    positions spread to about 2^25, so every position digit is decided at
    large in-layer positions; at 1/100 the cut lies inside the top level."""
    import torch
    import sparse_communication_adam_amd as sc
    rng = np.random.default_rng(keep[1])
    sizes = [(1 << 26) + 63, 1000]
    ctx = _ctx(sizes, W=2, keep=keep)
    lay = oracle.layout(sizes, keep[0], keep[1], 2)
    mt = (rng.integers(-8, 8, lay.n_pad) * 2.0 ** -12).astype(np.float32)
    log(f"mask build: layer of {sizes[0]} elements, 16 levels, keep {keep}")
    out = sc.alloc_mask(ctx.layout)
    sc.scape_mask_build(ctx, torch.from_numpy(mt).cuda(), out)
    exp = oracle.mask_from_keys(lay, oracle.keys_of(mt))
    got = u64(out.bits)
    if not np.array_equal(got, exp):
        d = np.flatnonzero(got != exp)
        raise AssertionError(f"{d.size} mask words differ, first word {d[0]}")
    idx, pre, cnt = oracle.mask_index(exp)
    assert cnt == lay.k_total
    assert np.array_equal(u32(out.idx)[:cnt], idx) and np.array_equal(u32(out.block_prefix), pre)
    ctx.destroy()


# The worker-interleaved layout (scape_step_interleaved): one residual array
# and one gradient array, each 64-element word holding the W workers' values
# in turn.  bench.py times the step in this layout.


@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "llama-0.55b", "llama-1.75b", "adversarial-ties"])
def test_step_interleaved_oracle_sized(name):
    wl = synth.WORKLOADS[name]
    small = wl if name == "single-1024x1024" else synth.reduced(wl)
    _assert_bitexact(run_parity(small, wl.steps, key_out=False, interleaved=True))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 16, 32])
def test_step_interleaved_ragged_worker_counts(W):
    """Every worker count with its own kernel instance, and 3 and 5 without:
    the word stride of the interleaved arrays is 64 W."""
    _assert_bitexact(run_parity(synth.ragged(), 4, W=W, key_out=False, interleaved=True))


def test_step_interleaved_edge_cases():
    wl = synth.ragged()
    _assert_bitexact(run_parity(wl, 3, key_out=True, interleaved=True))
    _assert_bitexact(run_parity(wl, 3, keep=(1, 1), init_mask_all=True, key_out=False, interleaved=True))
    _assert_bitexact(run_parity(dataclasses.replace(wl, weight_decay=0.1), 3, W=5, key_out=False, interleaved=True))
    _assert_bitexact(run_parity(wl, 4, grad_override=_special_grads(wl), key_out=False, interleaved=True))


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_step_interleaved_full_size_sampled_layers(name):
    """Full size, in the configuration bench.py times: worker-interleaved
    residuals and gradients, candidates' keys recomputed."""
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_parity(wl, wl.steps, sample=FULL_SAMPLES[name], key_out=False, interleaved=True))


def max_size_workload() -> "synth.Workload":
    """The largest layout the ABI takes: n_pad = 2^31 - 64 (30 layers of 2^26
    elements, one of 133,217,600, and a ragged last layer of 1,000,003 whose
    positions end 64 elements short of 2^31), one worker."""
    ts = [synth.configs.Tensor(f"big{i}", (1 << 26,)) for i in range(30)]
    ts += [synth.configs.Tensor("big30", (133217600,)), synth.configs.Tensor("last", (1000003,))]
    return synth.Workload(name="max-size", tensors=tuple(ts), W=1, keep_num=1, keep_den=100, steps=2,
                          seed=1098, grad_kind="loguniform")


def test_step_parity_maximum_size():
    """Every layer's counts and the index at the largest positions the ABI
    allows; the last layer against the oracle; candidates' keys recomputed
    (the configuration bench.py times)."""
    wl = max_size_workload()
    assert sum((t.numel + 63) // 64 * 64 for t in wl.tensors) == (1 << 31) - 64
    _assert_bitexact(run_parity(wl, wl.steps, sample=[31], key_out=False))


# Without key_out the step keeps only 16-bit keys and recomputes each
# candidate's full key from m, the owner's residual and its sparse buffer:
# the configuration bench.py times.


@PATHS
@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "llama-0.55b", "llama-1.75b", "adversarial-ties"])
def test_step_recomputed_keys_oracle_sized(name, path):
    wl = synth.WORKLOADS[name]
    small = wl if name == "single-1024x1024" else synth.reduced(wl)
    _assert_bitexact(run_parity(small, wl.steps, key_out=False, select_path=path))


@PATHS
def test_step_recomputed_keys_edge_cases(path):
    wl = synth.ragged()
    _assert_bitexact(run_parity(wl, 5, key_out=False, select_path=path))
    _assert_bitexact(run_parity(wl, 3, W=1, key_out=False, select_path=path))
    _assert_bitexact(run_parity(wl, 3, keep=(1, 1), init_mask_all=True, key_out=False, select_path=path))
    zero = lambda step, worker, tensor: np.zeros(wl.tensors[tensor].numel, np.uint16)  # noqa: E731
    _assert_bitexact(run_parity(wl, 3, grad_override=zero, key_out=False, select_path=path))


@pytest.mark.parametrize("name", ["llama-1.75b", "adversarial-ties"])
def test_step_recomputed_keys_full_size_sampled_layers(name):
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_parity(wl, wl.steps, sample=FULL_SAMPLES[name], key_out=False))


# The update inside the dense pass (scape_set_update_in_dense_pass): the
# dense pass itself reduces the W candidates and updates x, v and m at the
# mask's positions, in both residual layouts.  Where the mask keeps at most
# 1/32 of the elements it touches x, v and m at those positions only (the
# cases at keep 1/100 and 1/1000); on denser masks it streams them whole and
# stores the old values back elsewhere (keep 1/10 and 1/1).
LAYOUTS = pytest.mark.parametrize("interleaved", [False, True], ids=["per-worker", "interleaved"])


@LAYOUTS
@pytest.mark.parametrize("name", ["single-1024x1024", "gpt-345m", "llama-0.55b", "llama-1.75b", "adversarial-ties"])
def test_step_update_in_dense_pass_oracle_sized(name, interleaved):
    wl = synth.WORKLOADS[name]
    small = wl if name == "single-1024x1024" else synth.reduced(wl)
    _assert_bitexact(run_parity(small, wl.steps, key_out=False, interleaved=interleaved, update_in_dense=True))


@LAYOUTS
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 16, 32])
def test_step_update_in_dense_pass_ragged_worker_counts(W, interleaved):
    """Every worker count with its own kernel instance, and 3 and 5 without;
    the ragged layout's last workgroup lies partly past the end."""
    _assert_bitexact(run_parity(synth.ragged(), 4, W=W, key_out=False, interleaved=interleaved,
                                update_in_dense=True))


@LAYOUTS
def test_step_update_in_dense_pass_edge_cases(interleaved):
    """Weight decay at worker counts whose mean rounds, from an empty and a
    full first mask; special gradient values; zero gradients tied
    everywhere; keys kept in full; a kept fraction of 1/100."""
    wl = synth.ragged()
    kw = dict(interleaved=interleaved, update_in_dense=True)
    wd = dataclasses.replace(wl, weight_decay=0.1)
    for W in (3, 5):
        _assert_bitexact(run_parity(wd, 4, W=W, key_out=False, **kw))
        _assert_bitexact(run_parity(wd, 3, W=W, key_out=False, keep=(1, 1), init_mask_all=True, **kw))
    _assert_bitexact(run_parity(wl, 4, grad_override=_special_grads(wl), key_out=False, **kw))
    zero = lambda step, worker, t: np.zeros(wl.tensors[t].numel, np.uint16)  # noqa: E731
    _assert_bitexact(run_parity(wl, 3, grad_override=zero, x_zero=True, key_out=False, **kw))
    _assert_bitexact(run_parity(wl, 4, key_out=True, **kw))
    _assert_bitexact(run_parity(wl, 4, keep=(1, 100), key_out=False, **kw))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama-1.75b", "gpt-345m"])
def test_step_update_in_dense_pass_full_size(name):
    """At full size, worker-interleaved, as bench.py times them: the 1.75B
    shape (keep 1/100: x, v and m touched at the masked elements only) and
    the GPT-345M shape (keep 1/10: streamed whole); every output of the
    largest layers and of sampled small ones against the oracle."""
    wl = synth.WORKLOADS[name]
    _assert_bitexact(run_parity(wl, 3, sample=FULL_LARGEST[wl.name], key_out=False, interleaved=True,
                                update_in_dense=True))
    _assert_bitexact(run_parity(wl, wl.steps, sample=FULL_SAMPLES[wl.name], key_out=False, interleaved=True,
                                update_in_dense=True))


def test_step_update_in_dense_pass_matches_separate_update():
    """Both settings give the same bytes for every output, step after step."""
    import torch
    wl = synth.reduced(synth.LLAMA175)
    outs = []
    for on in (False, True):
        run = GpuSession(wl, interleaved=True, key_out=False, update_in_dense=on)
        for t in range(1, 5):
            run.step(t)
        torch.cuda.synchronize()
        st = run.state
        outs.append([to_np(a).copy() for a in [st.xv, st.m, st.r_il, st.cur_mask.bits, st.cur_mask.idx]
                     + st.sparse])
        release(run)
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
