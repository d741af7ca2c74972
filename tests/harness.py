"""Parity harness: the HIP path (through the C ABI) against the oracle.

Both sides get the same seeded inputs: the oracle from the host generator,
the GPU from its bit-identical GPU twin (checked in test_gpu_parity.py).  No
oracle input and no expected value comes from the GPU.

Full-size workloads are compared on a sample of layers: layers are
independent within a step, so the oracle runs the sampled layers alone
(``oracle.sub_layout``, keeping each layer's kept count and owner) and its
results must equal the GPU's on those layers, for every step.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle
import synth

RTOL, ATOL = 1e-5, 1e-7  # float-state tolerance of the parity bar (fp32)


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def scape_config(wl: synth.Workload, keep=None, W=None):
    import sparse_communication_adam_amd as sc
    num, den = keep if keep is not None else (wl.keep_num, wl.keep_den)
    return sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=W or wl.W, keep_num=num, keep_den=den,
                          owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                          weight_decay=wl.weight_decay)


def oracle_layout(wl: synth.Workload, keep=None, W=None) -> oracle.Layout:
    num, den = keep if keep is not None else (wl.keep_num, wl.keep_den)
    return oracle.layout(wl.layer_sizes, num, den, wl.P or (W or wl.W))


def hyper(wl: synth.Workload) -> oracle.Hyper:
    return oracle.Hyper(wl.beta1, wl.beta2, wl.lr, wl.eps, wl.weight_decay)


def to_np(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def u64(t) -> np.ndarray:
    return to_np(t).view(np.uint64)


def u32(t) -> np.ndarray:
    return to_np(t).view(np.uint32)


def check_float(name: str, got: np.ndarray, exp: np.ndarray, stats: Dict[str, int]) -> None:
    """Parity bar for fp32 state: |got-exp| <= ATOL + RTOL*|exp| everywhere,
    equal values (infinities included) match, and NaN only where the oracle
    has NaN; bit-exact positions are counted."""
    assert got.shape == exp.shape, (name, got.shape, exp.shape)
    g64, e64 = got.astype(np.float64), exp.astype(np.float64)
    both_nan = np.isnan(g64) & np.isnan(e64)
    with np.errstate(invalid="ignore"):  # inf - inf, only where the values are equal or infinite
        ok = both_nan | (g64 == e64) | (np.abs(g64 - e64) <= ATOL + RTOL * np.abs(e64))
    if not ok.all():
        bad = np.flatnonzero(~ok)
        i = bad[0]
        raise AssertionError(f"{name}: {bad.size} of {got.size} outside rel {RTOL}/abs {ATOL}; first at {i}: "
                             f"gpu {got[i]!r} oracle {exp[i]!r}")
    stats["float_values"] = stats.get("float_values", 0) + got.size
    stats["float_not_bitexact"] = stats.get("float_not_bitexact", 0) + int(
        np.count_nonzero((got.view(np.uint32) != exp.view(np.uint32)) & ~both_nan))


def first_mask_diff(lay: oracle.Layout, got_bits: np.ndarray, exp_bits: np.ndarray, key: np.ndarray) -> str:
    g = oracle.unpack(got_bits, lay.n_pad)
    e = oracle.unpack(exp_bits, lay.n_pad)
    d = np.flatnonzero(g != e)
    j = int(d[0])
    l = int(np.searchsorted(lay.off, j, side="right") - 1)
    return f"{d.size} mask bits differ; first: layer {l} position {j - lay.off[l]} key {key[j]:#x} gpu {g[j]} oracle {e[j]}"


@dataclass
class GpuSession:
    """A ScapeState driven with GPU-generated inputs for one workload."""
    wl: synth.Workload
    keep: Optional[tuple] = None
    W: Optional[int] = None
    init_mask_all: bool = False
    x_zero: bool = False
    grad_override: Optional[object] = None  # callable(step, worker, tensor) -> np.uint16 array
    offload: bool = False  # residuals in pinned host memory (scape_step_offload)
    key_out: bool = True  # ask the step for the full statistic keys (else candidates' keys are recomputed)
    interleaved: bool = False  # residuals and gradients in the worker-interleaved layout
    select_path: Optional[int] = None  # scape_set_select_path (None: the library's default)
    update_in_dense: bool = False  # scape_set_update_in_dense_pass
    offload_path: Optional[int] = None  # scape_set_offload_path (None: the library's default)
    state: object = None
    grads: List[object] = field(default_factory=list)

    def __post_init__(self):
        import torch
        from sparse_communication_adam_amd.state import ScapeState
        cfg = scape_config(self.wl, self.keep, self.W)
        self.state = ScapeState(cfg, offload=self.offload, interleaved=self.interleaved)
        import sparse_communication_adam_amd as sc
        if self.select_path is not None:
            sc.scape_set_select_path(self.state.ctx, self.select_path)
        sc.scape_set_update_in_dense_pass(self.state.ctx, self.update_in_dense)
        if self.offload_path is not None:
            sc.scape_set_offload_path(self.state.ctx, self.offload_path)
        self.layout = self.state.layout
        n = self.layout.n_pad
        if not self.x_zero:
            synth.params_flat_gpu(self.wl, self.layout.layer_offset, self.state.x)
        self.grads = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(cfg.workers)]
        self.g_il = torch.zeros(n * cfg.workers, dtype=torch.int16, device="cuda") if self.interleaved else None
        if self.init_mask_all:
            import sparse_communication_adam_amd as sc
            pred = torch.zeros(n, dtype=torch.uint8, device="cuda")
            for off, t in zip(self.layout.layer_offset, self.wl.tensors):
                pred[off:off + t.numel] = 1
            m = self.state.cur_mask
            sc.scape_pack(pred, m.bits)
            sc.scape_mask_index(self.state.ctx, m)

    def gen(self, step: int) -> None:
        import torch
        for i, g in enumerate(self.grads):
            if self.grad_override is not None:
                host = np.zeros(self.layout.n_pad, np.uint16)
                for off, t in zip(self.layout.layer_offset, range(len(self.wl.tensors))):
                    a = self.grad_override(step, i, t)
                    host[off:off + a.size] = a
                g.copy_(torch.from_numpy(host.view(np.int16)))
            else:
                synth.grads_flat_gpu(self.wl, self.layout.layer_offset, g, step, i)
        if self.interleaved:
            import sparse_communication_adam_amd as sc
            view = sc.interleaved_view(self.g_il, len(self.grads))
            for i, g in enumerate(self.grads):
                view[:, i, :].copy_(g.view(-1, 64))

    def step(self, t: int) -> None:
        self.gen(t)
        self.state.step(self.g_il if self.interleaved else self.grads, key_out=self.key_out)


def worker_slice(st, i: int, fs: slice):
    """Elements fs (a slice starting on a 64-element word) of worker i's
    residual, in either residual layout."""
    if not st.interleaved:
        return st.r[i][fs]
    import sparse_communication_adam_amd as sc
    a, b = fs.start, fs.stop
    assert a % 64 == 0
    v = sc.interleaved_view(st.r_il, st.cfg.workers)[a // 64:(b + 63) // 64, i, :]
    return v.reshape(-1)[:b - a]


def oracle_inputs(wl: synth.Workload, lay: oracle.Layout, tensors: Sequence[int], step: int, W: int,
                  grad_override=None) -> List[np.ndarray]:
    out = []
    for i in range(W):
        if grad_override is not None:
            g = np.zeros(lay.n_pad, np.uint16)
            for off, t in zip(lay.off, tensors):
                a = grad_override(step, i, t)
                g[off:off + a.size] = a
            out.append(g)
        else:
            out.append(synth.grads_flat(wl, lay.off, lay.n_pad, step, i, tensors))
    return out


def run_parity(wl: synth.Workload, steps: int, sample: Optional[Sequence[int]] = None, keep=None, W=None,
               init_mask_all=False, x_zero=False, grad_override=None, check_buffers=True,
               offload=False, key_out=True, interleaved=False, select_path=None,
               update_in_dense=False, offload_path=None) -> Dict[str, int]:
    """Run `steps` steps on the GPU (all layers) and the oracle (all layers, or
    the sampled ones) and compare every output of every step."""
    import torch
    W = W or wl.W
    full = oracle_layout(wl, keep, W)
    tensors = list(range(len(wl.tensors))) if sample is None else list(sample)
    lay = full if sample is None else oracle.sub_layout(full, tensors)
    log(f"{wl.name}: W={W} L={full.L} n_pad={full.n_pad} k_total={full.k_total} steps={steps} "
        f"oracle layers={len(tensors)} ({lay.n_pad} elements){' residuals on the host' if offload else ''}"
        f"{'' if key_out else ', candidate keys recomputed'}{', worker-interleaved layout' if interleaved else ''}"
        f"{'' if select_path is None else f', selection path {select_path}'}"
        f"{', update in the dense pass' if update_in_dense else ''}"
        f"{'' if offload_path is None else f', offload path {offload_path}'}")
    run = GpuSession(wl, keep, W, init_mask_all, x_zero, grad_override, offload, key_out, interleaved, select_path,
                 update_in_dense, offload_path)
    glay = run.layout
    assert glay.n_pad == full.n_pad and glay.k_total == full.k_total
    assert list(glay.layer_offset) == full.off.tolist() and list(glay.layer_k) == full.k.tolist()
    assert list(glay.layer_owner) == full.owner.tolist()

    x0 = np.zeros(lay.n_pad, np.float32) if x_zero else synth.params_flat(wl, lay.off, lay.n_pad, tensors)
    ost = oracle.State.zeros(lay.n_pad, W, x0)
    cur = np.zeros(lay.n_words, np.uint64)
    if init_mask_all:
        cur = oracle.pack(np.concatenate([np.r_[np.ones(n, np.uint8), np.zeros((-n) % 64, np.uint8)]
                                          for n in lay.sizes]) if lay.L else np.zeros(0, np.uint8))
    stats: Dict[str, int] = {}
    hp = hyper(wl)
    for t in range(1, steps + 1):
        gs = oracle_inputs(wl, lay, tensors, t, W, grad_override)
        out = oracle.step(lay, hp, ost, gs, cur)
        cur_gpu_prefix = u32(run.state.cur_mask.block_prefix).copy()
        run.step(t)
        torch.cuda.synchronize()
        st = run.state
        nm = st.cur_mask  # the mask just built (M_{t+1})
        g_bits, g_idx, g_pre = u64(nm.bits), u32(nm.idx), u32(nm.block_prefix)
        # whole-model invariants of the GPU's new mask (any size)
        assert g_pre[0] == 0 and int(g_pre[-1]) == full.k_total, (g_pre[-1], full.k_total)
        pc = np.unpackbits(g_bits.view(np.uint8)).reshape(-1, 64).sum(1)
        assert np.array_equal(np.diff(g_pre.astype(np.int64)), pc), "block_prefix inconsistent with bits"
        idx = g_idx[:full.k_total].astype(np.int64)
        assert np.all(np.diff(idx) > 0), "idx not strictly ascending"
        assert np.array_equal((g_bits[idx >> 6] >> (idx & 63).astype(np.uint64)) & 1, np.ones(idx.size, np.uint64))
        for l in range(full.L):
            w0, w1 = full.off[l] // 64, (full.off[l] + full.sizes[l] + 63) // 64
            assert g_pre[w1] - g_pre[w0] == full.k[l], f"layer {l}: {g_pre[w1] - g_pre[w0]} bits, k={full.k[l]}"
        # per-layer comparison against the oracle (only the sampled slices leave the GPU)
        cur_bits_np = oracle.unpack(cur, lay.n_pad) if out.count else None
        o_pos = np.flatnonzero(cur_bits_np) if out.count else None
        for a, l in enumerate(tensors):
            fs = slice(int(full.off[l]), int(full.off[l] + full.sizes[l]))
            os_ = slice(int(lay.off[a]), int(lay.off[a] + lay.sizes[a]))
            tag = f"step {t} layer {l} ({wl.tensors[l].name})"
            if key_out:
                assert np.array_equal(u32(st.key[fs]), out.key[os_]), f"{tag}: statistic keys differ"
            gw0, gw1 = full.off[l] // 64, (full.off[l] + full.sizes[l] + 63) // 64
            ow0, ow1 = lay.off[a] // 64, (lay.off[a] + lay.sizes[a] + 63) // 64
            if not np.array_equal(g_bits[gw0:gw1], out.next_words[ow0:ow1]):
                sub = oracle.Layout(lay.sizes[a:a + 1], np.zeros(1, np.int64), lay.k[a:a + 1], lay.owner[a:a + 1],
                                    int(ow1 - ow0) * 64)
                raise AssertionError(f"{tag}: " + first_mask_diff(sub, g_bits[gw0:gw1], out.next_words[ow0:ow1],
                                                                   out.key[os_.start:os_.start + sub.n_pad]))
            g_loc = idx[g_pre[gw0]:g_pre[gw1]] - full.off[l]
            o_loc = out.next_idx[out.next_prefix[ow0]:out.next_prefix[ow1]].astype(np.int64) - lay.off[a]
            assert np.array_equal(g_loc, o_loc), f"{tag}: idx differs"
            check_float(f"{tag} x", to_np(st.x[fs]), ost.x[os_], stats)
            check_float(f"{tag} m", to_np(st.m[fs]), ost.m[os_], stats)
            check_float(f"{tag} v", to_np(st.v[fs]), ost.v[os_], stats)
            for i in range(W):
                check_float(f"{tag} r[{i}]", to_np(worker_slice(st, i, fs)), ost.r[i][os_], stats)
            if check_buffers and out.count:
                # this layer's segment of every worker's sparse buffer
                oa = np.searchsorted(o_pos, lay.off[a])
                ob = np.searchsorted(o_pos, lay.off[a] + lay.sizes[a])
                ga, gb = int(cur_gpu_prefix[gw0]), int(cur_gpu_prefix[gw1])
                assert gb - ga == ob - oa, f"{tag}: sent count {gb - ga} vs {ob - oa}"
                for i in range(W):
                    check_float(f"{tag} sparse[{i}]", to_np(st.sparse[i][ga:gb]), out.sent[i][oa:ob], stats)
        stats["mask_bits_checked"] = stats.get("mask_bits_checked", 0) + lay.n_pad
        log(f"step {t}: |M_t|={out.count} sampled ok (float values so far {stats['float_values']}, "
            f"not bit-exact {stats['float_not_bitexact']})")
        cur = out.next_words
    release(run)
    return stats


def release(run) -> None:
    import gc
    import torch
    run.state.destroy()
    run.state = None
    run.grads = []
    run.g_il = None
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_dense_parity(wl: synth.Workload, steps: int, sample: Optional[Sequence[int]] = None, W=None,
                     weight_decay=None, interleaved=False) -> Dict[str, int]:
    """The dense AdamS step through the C ABI against the oracle's, on every
    layer or on the sampled ones, for every step: x, m and v within the parity
    bar (bit-exact expected), padding untouched."""
    import dataclasses
    import torch
    import sparse_communication_adam_amd as sc
    W = W or wl.W
    if weight_decay is not None:
        wl = dataclasses.replace(wl, weight_decay=weight_decay)
    full = oracle_layout(wl, None, W)
    tensors = list(range(len(wl.tensors))) if sample is None else list(sample)
    lay = full if sample is None else oracle.sub_layout(full, tensors)
    log(f"dense {wl.name}: W={W} L={full.L} n_pad={full.n_pad} steps={steps} wd={wl.weight_decay} "
        f"oracle layers={len(tensors)} ({lay.n_pad} elements)")
    ctx = sc.scape_init(scape_config(wl, None, W))
    offs = ctx.layout.layer_offset
    assert list(offs) == full.off.tolist()
    n = full.n_pad
    x = torch.zeros(n, dtype=torch.float32, device="cuda")
    synth.params_flat_gpu(wl, offs, x)
    m = torch.zeros_like(x)
    v = torch.zeros_like(x)
    x_pad0 = x.clone()
    grads = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(W)]
    g_il = torch.zeros(n * W, dtype=torch.int16, device="cuda") if interleaved else None
    ox = synth.params_flat(wl, lay.off, lay.n_pad, tensors)
    om, ov = np.zeros(lay.n_pad, np.float32), np.zeros(lay.n_pad, np.float32)
    hp = hyper(wl)
    stats: Dict[str, int] = {}
    for t in range(1, steps + 1):
        for i, g in enumerate(grads):
            synth.grads_flat_gpu(wl, offs, g, t, i)
        if interleaved:
            view = sc.interleaved_view(g_il, W)
            for i, g in enumerate(grads):
                view[:, i, :].copy_(g.view(-1, 64))
            sc.scape_dense_step_interleaved(ctx, x, m, v, g_il)
        else:
            sc.scape_dense_step(ctx, x, m, v, grads)
        oracle.dense_step(lay, hp, ox, om, ov, oracle_inputs(wl, lay, tensors, t, W))
        torch.cuda.synchronize()
        for a, l in enumerate(tensors):
            fs = slice(int(full.off[l]), int(full.off[l] + full.sizes[l]))
            os_ = slice(int(lay.off[a]), int(lay.off[a] + lay.sizes[a]))
            tag = f"dense step {t} layer {l} ({wl.tensors[l].name})"
            check_float(f"{tag} x", to_np(x[fs]), ox[os_], stats)
            check_float(f"{tag} m", to_np(m[fs]), om[os_], stats)
            check_float(f"{tag} v", to_np(v[fs]), ov[os_], stats)
            pad = slice(fs.stop, int((fs.stop + 63) // 64 * 64))
            assert not to_np(m[pad]).any() and not to_np(v[pad]).any(), f"{tag}: padding written"
            assert np.array_equal(to_np(x[pad]), to_np(x_pad0[pad])), f"{tag}: padding written"
        log(f"dense step {t}: sampled ok (float values so far {stats['float_values']}, "
            f"not bit-exact {stats['float_not_bitexact']})")
    ctx.destroy()
    del x, m, v, grads, x_pad0, g_il
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return stats
