"""Parity of the fill-in union (scape_mask_union_add) with the oracle's, on a
GPU: bits and the union's per-word prefix bit-exact.

The union is what Partitioned Mask Synchronization (gist.science Technical
Summary, s.2) avoids: every worker ranking every layer on its own statistic.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from harness import log, u32, u64

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


def _ctx(sizes, W, keep):
    import sparse_communication_adam_amd as sc
    return sc.scape_init(sc.ScapeConfig(layer_numel=list(sizes), workers=W, keep_num=keep[0], keep_den=keep[1]))


def _union_gpu(ctx, mts):
    import torch
    import sparse_communication_adam_amd as sc
    acc = torch.zeros(ctx.layout.n_words, dtype=torch.int64, device="cuda")
    for mt in mts:
        sc.scape_mask_union_add(ctx, mt, acc)
    mask = sc.alloc_mask(ctx.layout)
    mask.bits.copy_(acc)
    sc.scape_mask_index(ctx, mask)
    torch.cuda.synchronize()
    return u64(acc), u32(mask.idx), u32(mask.block_prefix)


def _statistics(kind, rng, n):
    if kind == "normal":
        return (rng.standard_normal(n) * 1e-3).astype(np.float32)
    if kind == "levels16":
        return (rng.integers(-8, 8, n) * 2.0 ** -12).astype(np.float32)
    return np.repeat(rng.standard_normal((n + 1) // 2).astype(np.float32), 2)[:n] * \
        np.tile(np.float32([1, -1]), (n + 1) // 2)[:n]


@pytest.mark.parametrize("kind", ["normal", "levels16", "pm_pairs"])
@pytest.mark.parametrize("W,keep", [(1, (1, 100)), (3, (1, 100)), (8, (1, 10)), (32, (1, 1000))])
def test_union_matches_oracle(kind, W, keep):
    import torch
    rng = np.random.default_rng(W * 7 + keep[1])
    sizes = [1, 37, 1000, 64, 4097, 70000, 300001, 0, 129]
    ctx = _ctx(sizes, W, keep)
    lay = oracle.layout(sizes, keep[0], keep[1], W)
    mts = [_statistics(kind, rng, lay.n_pad) for _ in range(W)]
    bits, idx, pre = _union_gpu(ctx, [torch.from_numpy(m).cuda() for m in mts])
    exp = oracle.union_mask(lay, [oracle.keys_of(m) for m in mts])
    assert np.array_equal(bits, exp)
    e_idx, e_pre, cnt = oracle.mask_index(exp, idx_cap=lay.k_total)
    assert np.array_equal(pre, e_pre) and int(pre[-1]) == cnt
    assert np.array_equal(idx[:min(cnt, lay.k_total)], e_idx)
    ctx.destroy()


def test_union_full_size_sampled_layers():
    """The 1.75B-shaped workload, W = 4: the workers' step-1 gradients as
    statistics (at step 1 each candidate is (1-beta1) times the gradient, so
    the ranking is the gradient's); the union bits of sampled layers against
    the oracle on those layers alone, and the per-layer bounds on every layer."""
    import torch
    import sparse_communication_adam_amd as sc
    wl = synth.WORKLOADS["llama-1.75b"]
    W = wl.W
    sample = [1, 3, 4, 190, 193]
    full = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, W)
    lay = oracle.sub_layout(full, sample)
    ctx = _ctx(wl.layer_sizes, W, (wl.keep_num, wl.keep_den))
    offs = ctx.layout.layer_offset
    g = torch.zeros(full.n_pad, dtype=torch.int16, device="cuda")
    acc = torch.zeros(full.n_words, dtype=torch.int64, device="cuda")
    keys = []
    for i in range(W):
        synth.grads_flat_gpu(wl, offs, g, 1, i)
        mt = g.view(torch.bfloat16).float()
        sc.scape_mask_union_add(ctx, mt, acc)
        del mt
        host = synth.grads_flat(wl, lay.off, lay.n_pad, 1, i, sample)
        keys.append(oracle.keys_of((host.astype(np.uint32) << 16).view(np.float32)))
    mask = sc.alloc_mask(ctx.layout)
    mask.bits.copy_(acc)
    sc.scape_mask_index(ctx, mask)
    torch.cuda.synchronize()
    bits, pre = u64(acc), u32(mask.block_prefix)
    exp = oracle.union_mask(lay, keys)
    for a, l in enumerate(sample):
        gw0, gw1 = full.off[l] // 64, (full.off[l] + full.sizes[l] + 63) // 64
        ow0, ow1 = lay.off[a] // 64, (lay.off[a] + lay.sizes[a] + 63) // 64
        assert np.array_equal(bits[gw0:gw1], exp[ow0:ow1]), f"layer {l}"
    for l in range(full.L):
        w0, w1 = full.off[l] // 64, (full.off[l] + full.sizes[l] + 63) // 64
        c = int(pre[w1]) - int(pre[w0])
        assert full.k[l] <= c <= min(full.sizes[l], W * full.k[l]), (l, c)
    log(f"union of {W} workers: {int(pre[-1])} bits = {int(pre[-1]) / wl.numel:.4%} of N "
        f"(one mask: {full.k_total / wl.numel:.4%})")
    ctx.destroy()
    del g, acc, mask
    gc.collect()
    torch.cuda.empty_cache()
