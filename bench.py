#!/usr/bin/env python3
"""Throughput of the fused SCAPE optimizer step on one MI355X.

One step = one scape_step call: the whole hot path (error feedback into W
residuals, first-moment candidates, compaction of the current mask's
positions into W sparse buffers, the W-way reduction, single-buffer
reconstruction and the v/m/x update, per-layer top-k of the next mask, its
packed bits and index) over one batch of synthetic gradients that is already
resident in HBM when the timed region starts.

Prints one JSON line.  `value` is parameters per second (N / step time).
`roofline` is the dominant kernel (the dense pass, SCAPE_PHASE_EF_COMPACT)
timed with HIP events on the step's stream: algorithmic bytes per launch
divided by its mean duration, against the 8 TB/s HBM peak.  `cpu_baseline`
is the oracle (plain single-threaded C) timed on this host on a bounded
sample of the same workload.  `dense_adams` times the dense AdamS step (the
baseline the pages measure SCAPE against) on the same workload, state and
gradient batches, with HIP events on its stream.  `fill_in` measures the
alternative the pages' partitioned masks avoid: the union of per-worker masks
over every layer, its density as workers are added, and the time to add one
worker's mask.  `offload` times the step with the W residuals in pinned host
memory (scape_step_offload), whose rate is bound by PCIe: with the dense pass
reading and writing them in host memory, and (`staged`) with copies through
the GPU.
`workloads` times the same step on every other workload shape (a few steps
each, after everything above), with the same byte accounting.
`shard_mask_build` times the mask build one worker runs on its own
layer-aligned 1/32 shard (scape_mask_build with num_shards = 32), shard by
shard, beside the build over every layer.  `one_worker_step` times the step
of the main workload with W = 1: one GPU's share when every worker has a GPU
of its own (its residual and gradient, the whole model's x, m and v).
`pack_unpack` times the standalone 1-bit pack and unpack over N elements.
`graph_step` times the single-layer workload's step replayed from HIP graphs
beside the same step launched eagerly.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused SCAPE step: params/sec and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "llama-1.75b"
# oracle sample per workload: a contiguous run of tensors (a few transformer
# blocks or their equivalent, about 10-15 s of single-threaded oracle work per
# step), timed on the host for one step with a built mask
CPU_SAMPLE = {
    "single-1024x1024": [0],
    "gpt-345m": list(range(2, 2 + 12 * 6)),        # six blocks, 75.6M params, W = 8
    "llama-0.55b": list(range(1, 1 + 6 * 3)),      # three blocks, 84.9M params, W = 8
    "llama-1.75b": list(range(1, 1 + 6 * 8)),      # eight blocks, 404.8M params, W = 4
    "adversarial-ties": list(range(1, 1 + 17 * 4)),  # four blocks, 16.8M params, W = 32
}


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def fused_update(N_pad: int, ksum: int, on: bool = True) -> bool:
    """Whether the dense pass finishes the update itself: with that switched
    on (scape_set_update_in_dense_pass) the library does so at every mask
    density (residuals on the device)."""
    return on


def streams_whole(N_pad: int, ksum: int) -> bool:
    """Whether the update inside the dense pass streams x, v and m whole
    (masks keeping more than 1/32 of the elements) rather than touching the
    masked elements only."""
    return ksum * 32 > N_pad


def alg_bytes(N: int, W: int, ksum: int, L: int, fused: bool):
    """Algorithmic bytes of one step and of its dense pass.  Per element the
    dense pass reads W bf16 gradients, W fp32 residuals, m and the mask bit,
    and writes the W residuals and a 16-bit statistic key (10W + 6.125); it
    zeroes the selection's histogram rows (8192 words per layer); at each
    masked element it writes the W sparse-buffer entries and either the m
    stash (4W + 4; the update pass then reads the buffers, the stash, idx and
    x and writes x, m, v: 4W + 20) or, when it finishes the update itself,
    reads x and writes x, m, v (4W + 16; on dense masks the kernel moves x, v
    and m whole, by choice, but only the masked elements' bytes count).  The step adds the key's read by the
    selection and the new mask's bits (2.125 per element) and the next mask's
    idx (4 per masked element)."""
    rows = 4 * 8192 * L
    per_masked_dense = 4 * W + 16 if fused else 4 * W + 4
    per_masked_step = 4 * W + 20 if fused else 8 * W + 28
    dense = N * (10 * W + 6.125) + per_masked_dense * ksum + rows
    step = N * (10 * W + 8.25) + per_masked_step * ksum + rows
    return dense, step


def dense_kernel_name(W: int, interleaved: bool, fused: bool, whole: bool = False) -> str:
    """The dense-pass kernel the library launches for this configuration
    (residuals on the device, keys not asked for)."""
    if fused:
        upd = (4 if interleaved else 3) if whole else (2 if interleaved else 1)
        return f"k_ef_compact<{W if W in (1, 2, 3, 4, 8, 16, 32) else 0}, false, {upd}> (with the update)"
    if interleaved and W == 4:
        return "k_ef_wl<4>"
    return f"k_ef_compact<{W if W in (1, 2, 3, 4, 8, 16, 32) else 0}, false, 0>"


def kernel_source_hash() -> str:
    """Hash of what the dense pass is compiled from: its kernels and launcher,
    the device helpers, and the constants and argument structs it uses, with
    comments left out."""
    csrc = os.path.join(ROOT, "sparse_communication_adam_amd", "csrc")
    el = open(os.path.join(csrc, "k_elementwise.hip")).read()
    a = el.index("// Dense pass, one-shot layout")   # the dense pass's section: helpers, knobs, kernel
    b = el.index("#undef SCAPE_EF_CASE", a)         # ... through its launcher
    parts = [el[a:b], open(os.path.join(csrc, "scape_device.h")).read()]
    hdr = open(os.path.join(csrc, "scape_internal.h")).read()
    for pat in (r"constexpr int kBlock = .*?;", r"constexpr int kWaves = .*?;", r"struct WorkerPtrs \{.*?\};",
                r"struct StepScalars \{.*?\};"):
        parts.append(re.search(pat, hdr, re.S).group(0))
    # comments and blank lines do not change the compiled kernel
    code = []
    for part in parts:
        for line in part.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def counter_traffic(workload: str, fused: bool):
    """HBM bytes per dense-pass launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source and on the same
    kind of pass (with or without the update in it)."""
    path = os.path.join(ROOT, "profiles", f"ef_compact_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel source hash:\s*`?([0-9a-f]+)", text)
    val = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", text)
    kind = re.search(r"update in the dense pass:\s*(yes|no)", text)
    if not src or not val or not kind or src.group(1) != kernel_source_hash():
        return None
    if (kind.group(1) == "yes") != fused:
        return None
    return float(val.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, steps_needed: int = 2):
    """The oracle (plain C, OpenMP over layers and positions, no parallel
    floating-point sum) on a contiguous run of the workload's tensors, timing
    the step after the first (which has a built mask)."""
    import numpy as np
    import oracle
    import synth
    tensors = CPU_SAMPLE[wl.name]
    full = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.P or wl.W)
    lay = oracle.sub_layout(full, tensors)
    hp = oracle.Hyper(wl.beta1, wl.beta2, wl.lr, wl.eps, wl.weight_decay)
    st = oracle.State.zeros(lay.n_pad, wl.W, synth.params_flat(wl, lay.off, lay.n_pad, tensors))
    cur = np.zeros(lay.n_words, np.uint64)
    times = []
    for t in range(1, steps_needed + 1):
        gs = [synth.grads_flat(wl, lay.off, lay.n_pad, t, i, tensors) for i in range(wl.W)]
        t0 = time.perf_counter()
        out = oracle.step(lay, hp, st, gs, cur)
        times.append(time.perf_counter() - t0)
        cur = out.next_words
        log(f"cpu baseline step {t}: {times[-1]:.2f} s on {int(lay.sizes.sum())} params")
    n = int(lay.sizes.sum())
    names = [wl.tensors[t].name for t in tensors]
    threads = oracle.threads()
    return {"value": n / times[-1], "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(tensors)} tensors ({names[0]}..{names[-1]}, {n} params, W={wl.W}) of {wl.name}; "
                      f"step {steps_needed} timed (mask built by step {steps_needed - 1}); C oracle, OpenMP over "
                      f"layers and positions with {threads} threads",
            "seconds": times[-1], "threads": threads, "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def grad_set(wl, layer_offset, n_pad: int, step: int, interleaved: bool):
    """One batch of the W workers' bf16 gradients (as int16), generated on
    the GPU: a list of W flat tensors, or one worker-interleaved tensor of
    n_pad*W elements (each 64-element word holding the W workers' values)."""
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    W = wl.W
    if not interleaved:
        gs = [torch.zeros(n_pad, dtype=torch.int16, device="cuda") for _ in range(W)]
        for i, g in enumerate(gs):
            synth.grads_flat_gpu(wl, layer_offset, g, step, i)
        return gs
    g_il = torch.zeros(n_pad * W, dtype=torch.int16, device="cuda")
    view = sc.interleaved_view(g_il, W)
    tmp = torch.zeros(n_pad, dtype=torch.int16, device="cuda")
    for i in range(W):
        synth.grads_flat_gpu(wl, layer_offset, tmp, step, i)
        view[:, i, :].copy_(tmp.view(-1, 64))
    del tmp
    return g_il


def dense_alg_bytes(N: int, W: int) -> float:
    """Algorithmic bytes of one dense AdamS step: read the W bf16 gradients,
    read m and x, write m, v and x."""
    return N * (2 * W + 20)


def dense_adams(wl, layer_offset, n_pad: int, sets, steps: int, warmup: int, interleaved: bool) -> dict:
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    ctx = sc.scape_init(cfg)
    x = torch.zeros(n_pad, dtype=torch.float32, device="cuda")
    synth.params_flat_gpu(wl, layer_offset, x)
    m, v = torch.zeros_like(x), torch.zeros_like(x)
    step = sc.scape_dense_step_interleaved if interleaved else sc.scape_dense_step
    for s in range(warmup):
        step(ctx, x, m, v, sets[s % len(sets)])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(steps):
        step(ctx, x, m, v, sets[(warmup + s) % len(sets)])
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    ctx.destroy()
    del x, m, v
    torch.cuda.empty_cache()
    N = wl.numel
    gbps = dense_alg_bytes(N, wl.W) / (ms * 1e-3) / 1e9
    return {"kernel": "scape_k_dense_adams", "gradient_layout": "worker-interleaved" if interleaved else "per worker",
            "ms_per_step": ms, "params_per_s": N / (ms * 1e-3),
            "alg_bytes_per_step": dense_alg_bytes(N, wl.W), "alg_GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}


def offload_step(cfg, wl, steps: int, warmup: int, staged: bool = False) -> dict:
    """The step with the residuals in pinned host memory: W*N*4 bytes read
    and written over PCIe per step (one gradient batch, per-worker arrays),
    by the dense pass itself, or through the staging slots (staged)."""
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    from sparse_communication_adam_amd.state import ScapeState
    state = ScapeState(cfg, offload=True)
    sc.scape_set_offload_path(state.ctx, sc.OFFLOAD_PATH_STAGED if staged else sc.OFFLOAD_PATH_AUTO)
    lay = state.layout
    synth.params_flat_gpu(wl, lay.layer_offset, state.x)
    sets = [grad_set(wl, lay.layer_offset, lay.n_pad, 1, False)]
    torch.cuda.synchronize()
    for s in range(warmup):
        state.step(sets[s % len(sets)], key_out=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        state.step(sets[(warmup + s) % len(sets)], key_out=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    state.destroy()
    del state, sets
    torch.cuda.empty_cache()
    pcie = 2 * wl.W * lay.n_pad * 4
    return {"ms_per_step": ms, "params_per_s": wl.numel / (ms * 1e-3), "residuals_on_host_GB": pcie / 2 / 1e9,
            "pcie_bytes_per_step": pcie, "pcie_GBps": pcie / (ms * 1e-3) / 1e9, "steps": steps, "warmup": warmup}


FILL_IN_WORKERS = (1, 2, 4, 8, 16, 32)


def fill_in(wl, cfg, layer_offset, n_pad: int) -> dict:
    """Union density of per-worker per-layer top-k masks over every layer as
    workers are added.  Worker i's statistic is its step-1 gradient widened
    to fp32: at step 1 the candidate is (1 - beta1) times the gradient, so its
    per-layer ranking is the gradient's."""
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    ctx = sc.scape_init(cfg)
    g = torch.zeros(n_pad, dtype=torch.int16, device="cuda")
    acc = torch.zeros(n_pad // 64, dtype=torch.int64, device="cuda")
    mask = sc.alloc_mask(ctx.layout)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    add_ms, density = [], {}
    for i in range(max(FILL_IN_WORKERS)):
        synth.grads_flat_gpu(wl, layer_offset, g, 1, i)
        mt = g.view(torch.bfloat16).float()
        ev0.record()
        sc.scape_mask_union_add(ctx, mt, acc)
        ev1.record()
        torch.cuda.synchronize()
        add_ms.append(ev0.elapsed_time(ev1))
        del mt
        if i + 1 in FILL_IN_WORKERS:
            mask.bits.copy_(acc)
            sc.scape_mask_index(ctx, mask)
            torch.cuda.synchronize()
            density[str(i + 1)] = int(mask.block_prefix[-1].item()) / wl.numel
    k_total = ctx.layout.k_total
    ctx.destroy()
    del g, acc, mask
    torch.cuda.empty_cache()
    return {"statistic": "workers' step-1 gradients (independent draws)", "one_mask_density": k_total / wl.numel,
            "union_density": density, "ms_per_worker_added": sum(add_ms[1:]) / max(len(add_ms) - 1, 1)}


def other_workload(name: str, steps: int, warmup: int, workers: int = 0, interleaved: bool = True,
                   update_in_dense: bool = True) -> dict:
    """The fused step on another workload shape (with `workers` workers instead
    of the workload's own W when given): state and two gradient batches
    resident, `warmup` untimed steps, then `steps` timed ones."""
    import dataclasses
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    from sparse_communication_adam_amd.state import ScapeState
    wl = synth.WORKLOADS[name]
    if workers:
        wl = dataclasses.replace(wl, W=workers, P=0)
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    state = ScapeState(cfg, interleaved=interleaved)
    sc.scape_set_update_in_dense_pass(state.ctx, update_in_dense)
    lay = state.layout
    synth.params_flat_gpu(wl, lay.layer_offset, state.x)
    sets = [grad_set(wl, lay.layer_offset, lay.n_pad, s + 1, interleaved) for s in range(2)]
    for s in range(warmup):
        state.step(sets[s % 2], key_out=False)
    torch.cuda.synchronize()
    sc.scape_profile_enable(state.ctx, True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(steps):
        state.step(sets[(warmup + s) % 2], key_out=False)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    phase_ms, nrec = sc.scape_profile_read(state.ctx)
    N, ksum = wl.numel, lay.k_total
    state.destroy()
    del state, sets
    torch.cuda.empty_cache()
    fused = fused_update(lay.n_pad, ksum, update_in_dense)
    dense_b, step_b = alg_bytes(N, wl.W, ksum, len(wl.tensors), fused)
    ef_ms = phase_ms["ef_compact"] / nrec
    return {"params": N, "workers": wl.W, "keep": f"{wl.keep_num}/{wl.keep_den}",
            "layout": "worker-interleaved" if interleaved else "per worker", "update_in_dense_pass": fused,
            "dense_pass_kernel": dense_kernel_name(wl.W, interleaved, fused, streams_whole(lay.n_pad, ksum)),
            "steps": steps, "warmup": warmup, "ms_per_step": ms, "params_per_s": N / (ms * 1e-3), "worker_elements_per_s": wl.W * N / (ms * 1e-3),
            "step_alg_GBps": step_b / (ms * 1e-3) / 1e9, "step_hbm_frac": step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "dense_pass_ms": ef_ms, "dense_pass_GBps": dense_b / (ef_ms * 1e-3) / 1e9,
            "dense_pass_hbm_frac": dense_b / (ef_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "phase_ms": {k: v / nrec for k, v in phase_ms.items()}}


def shard_mask_build(name: str) -> dict:
    """The per-layer top-k one worker builds on its own layer-aligned shard:
    scape_mask_build(num_shards = shard_P, shard = s) for every s, from worker
    0's step-1 gradient widened to fp32 as the statistic (at step 1 the
    candidate is (1 - beta1) times the gradient, so the ranking is the
    gradient's), each build timed with HIP events, beside one build over
    every layer.  Algorithmic bytes of a build: read the statistic (4 B per
    element), write and read its 16-bit key, write the mask bits."""
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    wl = synth.WORKLOADS[name]
    P = wl.shard_P
    # the build's shard count is a per-call argument; the config keeps the
    # step's owners (at most W shards)
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    ctx = sc.scape_init(cfg)
    lay = ctx.layout
    g = torch.zeros(lay.n_pad, dtype=torch.int16, device="cuda")
    synth.grads_flat_gpu(wl, lay.layer_offset, g, 1, 0)
    mt = g.view(torch.bfloat16).float()
    del g
    mask = sc.alloc_mask(lay)
    owner = sc.scape_owner_map(cfg, P)
    sizes = wl.layer_sizes
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(shards: int, shard: int, reps: int = 3) -> float:
        sc.scape_mask_build(ctx, mt, mask, shards, shard)
        ev0.record()
        for _ in range(reps):
            sc.scape_mask_build(ctx, mt, mask, shards, shard)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    per, elems = [], []
    for s in range(P):
        n_s = sum(n for n, o in zip(sizes, owner) if o == s)
        if n_s == 0:
            continue
        per.append(timed(P, s))
        elems.append(n_s)
    full_ms = timed(0, -1)
    ctx.destroy()
    del mt, mask
    torch.cuda.empty_cache()
    bpe = 4 + 2 + 2 + 0.125
    rates = [bpe * n / (t * 1e-3) / 1e9 for n, t in zip(elems, per)]
    imax = max(range(len(per)), key=lambda i: per[i])
    return {"num_shards": P, "shards_with_layers": len(per), "shard_ms_mean": sum(per) / len(per),
            "shard_ms_max": per[imax], "shard_elements_max": elems[imax],
            "shard_elements_mean": sum(elems) / len(elems), "shard_alg_GBps_of_largest": rates[imax],
            "all_layers_ms": full_ms, "all_layers_alg_GBps": bpe * wl.numel / (full_ms * 1e-3) / 1e9,
            "alg_bytes_per_element": bpe}


def pack_unpack(n: int) -> dict:
    """The standalone 1-bit pack and unpack over n elements (one byte per
    predicate, a bit per element), each timed with HIP events over 5 calls
    after one untimed; algorithmic bytes n + n/8 each way."""
    import torch
    import sparse_communication_adam_amd as sc
    g = torch.Generator(device="cuda").manual_seed(7)
    pred = (torch.rand(n, device="cuda", generator=g) < 0.01).to(torch.uint8)
    bits = torch.empty((n + 63) // 64, dtype=torch.int64, device="cuda")
    back = torch.empty_like(pred)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {"elements": n, "alg_bytes": n + n / 8}
    for name, call in (("pack", lambda: sc.scape_pack(pred, bits)), ("unpack", lambda: sc.scape_unpack(bits, back))):
        call()
        ev0.record()
        for _ in range(5):
            call()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / 5
        out[f"{name}_ms"] = ms
        out[f"{name}_alg_GBps"] = (n + n / 8) / (ms * 1e-3) / 1e9
    out["round_trip_exact"] = bool(torch.equal(back, pred))
    del pred, bits, back
    torch.cuda.empty_cache()
    return out


def graph_step(name: str, steps: int = 20, warmup: int = 2) -> dict:
    """The step of a small workload replayed from HIP graphs (ScapeState.capture)
    beside the same step launched eagerly, each timed with HIP events."""
    import torch
    import synth
    import sparse_communication_adam_amd as sc
    from sparse_communication_adam_amd.state import ScapeState
    wl = synth.WORKLOADS[name]
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    out = {"workload": name, "steps": steps, "warmup": warmup}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mode in ("eager", "graph"):
        st = ScapeState(cfg)
        lay = st.layout
        synth.params_flat_gpu(wl, lay.layer_offset, st.x)
        gs = [torch.zeros(lay.n_pad, dtype=torch.int16, device="cuda") for _ in range(wl.W)]
        for i, g in enumerate(gs):
            synth.grads_flat_gpu(wl, lay.layer_offset, g, 1, i)
        if mode == "graph":
            st.capture(gs)
        run = st.step_graph if mode == "graph" else (lambda: st.step(gs, key_out=False))
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(steps):
            run()
        ev1.record()
        torch.cuda.synchronize()
        out[f"{mode}_ms_per_step"] = ev0.elapsed_time(ev1) / steps
        st.destroy()
        del st, gs
    torch.cuda.empty_cache()
    return out


def shaped_probe(state, g_il, W: int, reps: int = 5):
    """scape_stream_probe with the dense pass's traffic over the step's own
    buffers (same pages): read the W workers' residuals (4W bytes per
    element) and bf16 gradients (2W) and m (4), write the residuals back in
    place (4W) and a 2-byte key.  None where a width would pass 16 bytes
    (W > 4).  The step's state is garbage afterwards."""
    import torch
    import sparse_communication_adam_amd as sc
    if 4 * W > 16:
        return None
    n_words = state.layout.n_pad // 64
    srcs, sw = [state.r_il, g_il, state.m], [4 * W, 2 * W, 4]
    dsts, dw = [state.r_il, state.key], [4 * W, 2]
    sc.scape_stream_probe(srcs, sw, dsts, dw, n_words)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        sc.scape_stream_probe(srcs, sw, dsts, dw, n_words)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    nbytes = n_words * 64 * (sum(sw) + sum(dw))
    return {"ms": ms, "bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes_per_element": sum(sw) + sum(dw)}


def spin_up(seconds: float) -> None:
    """Plain device-to-device copies for `seconds`: an idle GPU takes a while
    to reach its steady memory and fabric clocks."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            b.copy_(a)
        torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def stream_copy_bandwidth(nbytes: int = 4 << 30) -> float:
    """Read + write bytes per second of the library's plain one-shot copy
    kernel (scape_copy_probe): the practical stream ceiling of this GPU."""
    import torch
    import sparse_communication_adam_amd as sc
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sc.scape_copy_probe(a, b)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    ev0.record()
    for _ in range(reps):
        sc.scape_copy_probe(a, b)
    ev1.record()
    torch.cuda.synchronize()
    dt = ev0.elapsed_time(ev1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


def copy_bandwidth(nbytes: int = 4 << 30) -> float:
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 10
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(CPU_SAMPLE))
    ap.add_argument("--grad-sets", type=int, default=2, help="distinct gradient batches cycled over the steps")
    ap.add_argument("--layout", choices=("interleaved", "separate"), default="interleaved",
                    help="residuals and gradients worker-interleaved (scape_step_interleaved) or one array per "
                         "worker (scape_step)")
    ap.add_argument("--no-other-layout", action="store_true",
                    help="skip timing the main workload in the other residual/gradient layout")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense AdamS comparison step")
    ap.add_argument("--no-fill-in", action="store_true", help="skip the fill-in union measurement")
    ap.add_argument("--no-offload", action="store_true", help="skip the host-residual (offload) step")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the step on the other workload shapes")
    ap.add_argument("--no-shard-build", action="store_true",
                    help="skip timing the per-worker mask build on one layer-aligned shard and the "
                         "standalone pack / unpack")
    ap.add_argument("--spinup-s", type=float, default=0.0,
                    help="seconds of plain device copies before anything else (off by default: allocating and "
                         "freeing its buffers just before the state left the state in memory where the dense "
                         "pass ran 15.3 instead of 13.5-14.2 ms)")
    ap.add_argument("--separate-update", action="store_true",
                    help="make the update a pass of its own instead of finishing it in the dense pass "
                         "(scape_set_update_in_dense_pass(0))")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              f"run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import synth
    import sparse_communication_adam_amd as sc
    from sparse_communication_adam_amd.state import ScapeState

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sc.lib()
    if args.spinup_s > 0:
        spin_up(args.spinup_s)
    wl = synth.WORKLOADS[args.workload]
    cfg = sc.ScapeConfig(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den,
                         owner_shards=wl.P, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, eps=wl.eps,
                         weight_decay=wl.weight_decay)
    il = args.layout == "interleaved"
    log(f"workload {wl.name}: {len(wl.tensors)} tensors, N={wl.numel}, W={wl.W}, keep={wl.keep_num}/{wl.keep_den}, "
        f"{'worker-interleaved' if il else 'per-worker'} residuals and gradients")
    state = ScapeState(cfg, interleaved=il)
    sc.scape_set_update_in_dense_pass(state.ctx, not args.separate_update)
    lay = state.layout
    N, W, ksum = wl.numel, wl.W, lay.k_total
    workspace = sc.scape_workspace_bytes(state.ctx)
    synth.params_flat_gpu(wl, lay.layer_offset, state.x)
    sets = [grad_set(wl, lay.layer_offset, lay.n_pad, s + 1, il) for s in range(args.grad_sets)]
    torch.cuda.synchronize()
    log(f"state and {args.grad_sets} gradient batches resident ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    for s in range(args.warmup):
        state.step(sets[s % len(sets)], key_out=False)
    torch.cuda.synchronize()
    log(f"{args.warmup} warmup steps done")

    sc.scape_profile_enable(state.ctx, True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for s in range(args.steps):
        state.step(sets[(args.warmup + s) % len(sets)], key_out=False)
        evs[s + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    phase_ms, nrec = sc.scape_profile_read(state.ctx)
    sc.scape_profile_enable(state.ctx, False)
    ms = (t1 - t0) * 1e3 / args.steps
    log(f"{args.steps} timed steps: {ms:.3f} ms/step; phases " +
        ", ".join(f"{k} {v / nrec:.3f} ms" for k, v in phase_ms.items()))

    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("calibration copy of 1 GiB done")

    fused = fused_update(lay.n_pad, ksum, not args.separate_update)
    dense_b, step_b = alg_bytes(N, W, ksum, len(wl.tensors), fused)
    ef_ms = phase_ms["ef_compact"] / nrec
    ef_gbps = dense_b / (ef_ms * 1e-3) / 1e9
    shaped = shaped_probe(state, sets[0], W) if il else None
    if shaped:
        log(f"a pass of the dense pass's shape over the same buffers: {shaped['ms']:.3f} ms, "
            f"{shaped['GBps']:.0f} GB/s (the dense pass: {ef_gbps / shaped['GBps']:.3f} of it)")
    step_gbps = step_b / (ms * 1e-3) / 1e9
    traffic = counter_traffic(wl.name, fused)
    offsets, n_pad = list(lay.layer_offset), lay.n_pad
    state.destroy()
    del state
    torch.cuda.empty_cache()
    dense = None
    if not args.no_dense:
        dense = dense_adams(wl, offsets, n_pad, sets, args.steps, args.warmup, il)
        dense["scape_step_over_dense"] = ms / dense["ms_per_step"]
        log(f"dense AdamS step: {dense['ms_per_step']:.3f} ms ({dense['alg_GBps']:.0f} GB/s algorithmic)")
    del sets
    torch.cuda.empty_cache()
    other_layout = None
    if not args.no_other_layout:
        other_layout = other_workload(wl.name, args.steps, args.warmup, interleaved=not il,
                                      update_in_dense=not args.separate_update)
        log(f"{wl.name} with {other_layout['layout']} residuals and gradients: {other_layout['ms_per_step']:.3f} ms/step, "
            f"dense pass {other_layout['dense_pass_ms']:.3f} ms ({other_layout['dense_pass_GBps']:.0f} GB/s)")
    offload = None
    if not args.no_offload:
        offload = offload_step(cfg, wl, 3, 2)
        offload["path"] = "dense pass reads and writes the pinned residuals"
        log(f"offloaded-residual step: {offload['ms_per_step']:.1f} ms ({offload['pcie_GBps']:.1f} GB/s over PCIe)")
        staged = offload_step(cfg, wl, 3, 2, staged=True)
        offload["staged"] = {k: staged[k] for k in ("ms_per_step", "params_per_s", "pcie_GBps")}
        log(f"offloaded-residual step, staged copies: {staged['ms_per_step']:.1f} ms "
            f"({staged['pcie_GBps']:.1f} GB/s over PCIe)")
    fill = None
    if not args.no_fill_in:
        fill = fill_in(wl, cfg, offsets, n_pad)
        log("fill-in union density by workers: " + ", ".join(f"{w}: {d:.4%}" for w, d in fill["union_density"].items()))
    others = {}
    if not args.no_other_workloads:
        for name in sorted(synth.WORKLOADS):
            if name == wl.name:
                continue
            others[name] = other_workload(name, 5, 2, interleaved=il, update_in_dense=not args.separate_update)
            o = others[name]
            log(f"workload {name}: {o['ms_per_step']:.3f} ms/step, {o['params_per_s'] / 1e9:.1f}G params/s, "
                f"dense pass {o['dense_pass_GBps']:.0f} GB/s")
    graphed = None
    if not args.no_other_workloads:
        graphed = graph_step("single-1024x1024")
        log(f"single-1024x1024 step: eager {graphed['eager_ms_per_step']:.3f} ms, replayed from HIP graphs "
            f"{graphed['graph_ms_per_step']:.3f} ms")
    one_worker = None
    if not args.no_other_workloads:
        one_worker = other_workload(wl.name, 5, 2, workers=1, interleaved=il,
                                    update_in_dense=not args.separate_update)
        log(f"one worker (W = 1) on {wl.name}: {one_worker['ms_per_step']:.3f} ms/step, dense pass "
            f"{one_worker['dense_pass_GBps']:.0f} GB/s")
    pu = None
    if not args.no_shard_build:
        pu = pack_unpack(N)
        log(f"pack / unpack of {N} elements: {pu['pack_ms']:.3f} / {pu['unpack_ms']:.3f} ms "
            f"({pu['pack_alg_GBps']:.0f} / {pu['unpack_alg_GBps']:.0f} GB/s)")
    shard_builds = {}
    if not args.no_shard_build:
        for name in ("gpt-345m", "llama-0.55b", "llama-1.75b"):
            shard_builds[name] = sb = shard_mask_build(name)
            log(f"shard mask build {name}: {sb['shard_ms_mean']:.3f} ms mean, {sb['shard_ms_max']:.3f} ms max over "
                f"{sb['shards_with_layers']} of {sb['num_shards']} shards; all layers {sb['all_layers_ms']:.3f} ms")
    copy_gbps = copy_bandwidth()
    stream_gbps = stream_copy_bandwidth()
    log(f"device copy: torch {copy_gbps:.0f} GB/s, one-shot stream copy {stream_gbps:.0f} GB/s")

    result = {
        "metric": METRIC, "value": N / (ms * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "params": N, "tensors": len(wl.tensors), "workers": W,
                   "keep": f"{wl.keep_num}/{wl.keep_den}", "kept_total": ksum, "grad_dtype": "bf16",
                   "gradient_batches": args.grad_sets, "update_in_dense_pass": fused,
                   "layout": "worker-interleaved residuals and gradients" if il else "one residual and gradient "
                             "array per worker"},
        "context_workspace_bytes": workspace,
        "step_ms_median": step_ms[len(step_ms) // 2], "step_ms_min": step_ms[0],
        "worker_elements_per_s": W * N / (ms * 1e-3),
        "step_alg_GBps": step_gbps, "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "phase_ms": {k: v / nrec for k, v in phase_ms.items()},
        "device_copy_GBps": copy_gbps, "stream_copy_GBps": stream_gbps,
        "roofline": {"kernel": dense_kernel_name(W, il, fused, streams_whole(lay.n_pad, ksum)), "bound": "hbm", "achieved": ef_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ef_gbps / HBM_PEAK_GBPS,
                     "alg_bytes_per_launch": dense_b, "mean_launch_ms": ef_ms, "traffic": traffic,
                     "stream_copy_GBps": stream_gbps, "frac_of_stream_copy": ef_gbps / stream_gbps,
                     "shaped_probe": shaped,
                     "frac_of_shaped_probe": ef_gbps / shaped["GBps"] if shaped else None},
    }
    if other_layout is not None:
        result["other_layout_step"] = other_layout
    if dense is not None:
        result["dense_adams"] = dense
    if fill is not None:
        result["fill_in"] = fill
    if offload is not None:
        result["offload"] = offload
    if others:
        result["workloads"] = others
    if one_worker is not None:
        result["one_worker_step"] = one_worker
    if graphed is not None:
        result["graph_step"] = graphed
    if shard_builds:
        result["shard_mask_build"] = shard_builds
    if pu is not None:
        result["pack_unpack"] = pu
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
