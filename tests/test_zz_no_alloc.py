"""scape_mask_index_static: the mask index without a context or any
allocation (its partial sums in the library's static device array), against
scape_mask_index, the entry point it is a variant of, through the C ABI: two
calls in a row, the second on a smaller mask, so the second call runs on the
scratch the first one left behind."""
import ctypes
import gc

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_communication_adam_amd as sc
    sc.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _case(sizes, density, seed):
    """A context over `sizes` (keep 1/1, so idx can hold every position), a
    random mask of that layout, and the existing entry point's index of it."""
    import torch
    import sparse_communication_adam_amd as sc
    ctx = sc.scape_init(sc.ScapeConfig(layer_numel=list(sizes), workers=1, keep_num=1, keep_den=1))
    lay = ctx.layout
    rng = np.random.default_rng(seed)
    pred = np.zeros(lay.n_pad, np.uint8)
    for off, n in zip(lay.layer_offset, sizes):
        pred[off:off + n] = rng.random(n) < density
    words = oracle.pack(pred)
    want = sc.alloc_mask(lay)
    want.bits.copy_(torch.from_numpy(words.view(np.int64)).cuda())
    sc.scape_mask_index(ctx, want)
    return ctx, words, want


def _static(words, k_cap):
    """The no-allocation entry point, called through the C ABI."""
    import torch
    import sparse_communication_adam_amd as sc
    bits = torch.from_numpy(words.view(np.int64)).cuda()
    idx = torch.full((max(k_cap, 1),), -7, dtype=torch.int32, device="cuda")
    pre = torch.full((words.size + 1,), -7, dtype=torch.int32, device="cuda")
    rc = sc.lib().scape_mask_index_static(ctypes.c_void_p(bits.data_ptr()), words.size, ctypes.c_void_p(idx.data_ptr()),
                                          k_cap, ctypes.c_void_p(pre.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sc.scape_last_error()
    torch.cuda.synchronize()
    return idx.cpu().numpy().view(np.uint32), pre.cpu().numpy().view(np.uint32)


def test_static_index_matches_the_context_index_on_two_calls():
    import torch
    big = [300_001, 5, 1 << 20, 77_777]      # 20 index workgroups
    small = [4_097, 1, 64]                     # 1 index workgroup
    for sizes, dens, seed in [(big, 0.3, 1), (small, 0.01, 2)]:
        ctx, words, want = _case(sizes, dens, seed)
        k_cap = ctx.layout.k_total
        idx, pre = _static(words, k_cap)
        torch.cuda.synchronize()
        w_idx = want.idx.cpu().numpy().view(np.uint32)
        w_pre = want.block_prefix.cpu().numpy().view(np.uint32)
        cnt = int(w_pre[-1])
        assert np.array_equal(pre, w_pre), sizes
        assert np.array_equal(idx[:cnt], w_idx[:cnt]), sizes
        o_idx, o_pre, o_cnt = oracle.mask_index(words)
        assert o_cnt == cnt and np.array_equal(pre, o_pre) and np.array_equal(idx[:cnt], o_idx)
        ctx.destroy()


def test_static_index_stores_at_most_k_cap_positions():
    import torch
    ctx, words, want = _case([100_000], 0.5, 3)
    cnt = int(want.block_prefix.cpu().numpy()[-1])
    idx, pre = _static(words, 1000)
    assert int(pre[-1]) == cnt
    assert np.array_equal(idx[:1000], want.idx.cpu().numpy().view(np.uint32)[:1000])
    ctx.destroy()
    torch.cuda.synchronize()


def test_static_index_rejects_sizes_beyond_its_scratch():
    import sparse_communication_adam_amd as sc
    lib = sc.lib()
    # validated on the host: nothing is launched and no pointer is touched
    rc = lib.scape_mask_index_static(ctypes.c_void_p(8), (1 << 25) + 1, ctypes.c_void_p(8), 0, ctypes.c_void_p(8), None)
    from sparse_communication_adam_amd._scape import SCAPE_ERR_INVALID_ARG, SCAPE_ERR_SHAPE
    assert rc == SCAPE_ERR_SHAPE and "maximum" in sc.scape_last_error()
    rc = lib.scape_mask_index_static(None, 10, None, 0, ctypes.c_void_p(8), None)
    assert rc == SCAPE_ERR_INVALID_ARG
