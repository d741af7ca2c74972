"""Device state of one SCAPE optimizer instance and its step loop.

Holds the fp32 master parameters x, moments m and v, the W residuals, the two
mask slots and the W sparse buffers as torch tensors on one GPU, and calls
``scape_step``.  The mask built at step t is used at step t+1 (Delayed Mask
Usage, gist.science Technical Summary s.2): after each step the two mask
slots swap roles.  The first step uses an all-zero mask.  With
``offload=True`` the residuals live in pinned host memory and each step calls
``scape_step_offload`` (Memory Optimization, same section).

With ``interleaved=True`` the state is in the interleaved layout of
``scape_step_interleaved``: the W residuals are one array in which each
64-element word holds the W workers' values in turn (each step takes the
gradients in the same layout, one int16 tensor of n_pad*W elements), and x
and v are one array of (x, v) pairs, ``xv``; ``x`` and ``v`` are then strided
views of it.

``capture`` records the step as HIP graphs, for small models whose step is
bound by its ~30 kernel launches: ``step_graph`` then replays it with one
launch.  scape_step never waits on the host, clears memory with kernels, and
joins its second stream back with events, so it can be captured.
"""
from __future__ import annotations

from typing import Optional, Sequence

from ._scape import (Context, Mask, ScapeConfig, alloc_mask, interleaved_view, scape_step, scape_step_interleaved,
                     scape_step_offload)


class ScapeState:
    def __init__(self, cfg: ScapeConfig, device: str = "cuda", x=None, offload: bool = False,
                 interleaved: bool = False):
        import torch
        self.cfg = cfg
        self.ctx = Context(cfg)
        self.layout = self.ctx.layout
        n, W, k = self.layout.n_pad, cfg.workers, self.layout.k_total
        f32 = dict(dtype=torch.float32, device=device)
        self.xv = None
        if interleaved:
            self.xv = torch.zeros(2 * n, **f32)
            self.x = self.xv.view(-1, 2)[:, 0]
            self.v = self.xv.view(-1, 2)[:, 1]
            if x is not None:
                self.x.copy_(x)
        else:
            self.x = torch.zeros(n, **f32) if x is None else x
            self.v = torch.zeros(n, **f32)
        self.m = torch.zeros(n, **f32)
        if offload and interleaved:
            raise ValueError("the offloaded step takes one residual array per worker")
        self.offload = offload
        self.interleaved = interleaved
        self.r_il = None
        if offload:
            self.r = [torch.zeros(n, dtype=torch.float32, pin_memory=True) for _ in range(W)]
        elif interleaved:
            self.r_il = torch.zeros(n * W, **f32)
            self.r = None
        else:
            self.r = [torch.zeros(n, **f32) for _ in range(W)]
        self.sparse = [torch.zeros(max(k, 1), **f32) for _ in range(W)]
        self.key = torch.zeros(n, dtype=torch.int32, device=device)
        self.masks = [alloc_mask(self.layout, device), alloc_mask(self.layout, device)]
        self._cur = 0
        self.t = 0

    @property
    def cur_mask(self) -> Mask:
        """The mask the next step applies (M_t)."""
        return self.masks[self._cur]

    @property
    def next_mask(self) -> Mask:
        return self.masks[1 - self._cur]

    def set_params(self, flat) -> None:
        """Copy n_pad parameters into x (whatever its layout)."""
        self.x.copy_(flat)

    def residual(self, i: int):
        """Worker i's residual as a flat n_pad tensor (a copy in the
        interleaved layout)."""
        if self.interleaved:
            return interleaved_view(self.r_il, self.cfg.workers)[:, i, :].reshape(-1)
        return self.r[i]

    def step(self, grads, stream=None, key_out: Optional[bool] = True) -> None:
        """One step with the W workers' bfloat16 gradients (int16 views): a
        list of W tensors, or in the interleaved layout one tensor of
        n_pad*W.  key_out=True also writes the full statistic keys into
        ``self.key`` (4 bytes per element more); the mask does not depend on
        it."""
        key = self.key if key_out else None
        if self.interleaved:
            scape_step_interleaved(self.ctx, self.xv, self.m, self.r_il, grads, self.cur_mask, self.next_mask,
                                   self.sparse, key, stream)
        else:
            fn = scape_step_offload if self.offload else scape_step
            fn(self.ctx, self.x, self.m, self.v, self.r, grads, self.cur_mask, self.next_mask, self.sparse, key,
               stream)
        self._cur = 1 - self._cur
        self.t += 1

    def capture(self, grads: Sequence, key_out: bool = False) -> None:
        """Capture the step as two HIP graphs, one for each assignment of the
        two mask slots (they swap roles every step).  The graphs read the
        gradients from `grads`, the W int16 tensors given here: before each
        ``step_graph`` the caller writes that step's gradients into them.
        Capturing runs nothing, so the state does not change."""
        import torch
        if self.offload:
            raise ValueError("the offloaded step copies to and from host memory and is not captured")
        self._graph_grads = grads if self.interleaved else list(grads)
        graphs = []
        for cur in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if self.interleaved:
                    scape_step_interleaved(self.ctx, self.xv, self.m, self.r_il, self._graph_grads,
                                           self.masks[cur], self.masks[1 - cur], self.sparse,
                                           self.key if key_out else None)
                else:
                    scape_step(self.ctx, self.x, self.m, self.v, self.r, self._graph_grads, self.masks[cur],
                               self.masks[1 - cur], self.sparse, self.key if key_out else None)
            graphs.append(g)
        self._graphs = graphs

    def step_graph(self) -> None:
        """One step replayed from the captured graphs on the current stream,
        with this step's gradients already in the capture buffers."""
        self._graphs[self._cur].replay()
        self._cur = 1 - self._cur
        self.t += 1

    @property
    def last_mask(self) -> Mask:
        """The mask applied by the most recent step (M_t of step t)."""
        return self.masks[1 - self._cur]

    def state_dict(self) -> dict:
        """Everything the next step depends on, as host tensors: x, m, v, the
        W residuals, the step counter, and - because the mask built at step t
        is only applied at step t+1 - the pending mask (bits, idx,
        block_prefix), plus the mask the last step applied.  The sparse
        buffers and statistic keys are outputs of a step, not state."""
        import torch
        torch.cuda.synchronize()
        cpu = lambda t: t.detach().to("cpu", copy=True).contiguous()  # noqa: E731
        lay = self.layout
        return {
            "n_pad": lay.n_pad, "k_total": lay.k_total, "workers": self.cfg.workers,
            "layer_numel": [int(n) for n in self.cfg.layer_numel], "t": self.t,
            "x": cpu(self.x), "m": cpu(self.m), "v": cpu(self.v),
            "r": [cpu(self.residual(i)) for i in range(self.cfg.workers)],
            "pending_mask": [cpu(self.cur_mask.bits), cpu(self.cur_mask.idx), cpu(self.cur_mask.block_prefix)],
            "last_mask": [cpu(self.last_mask.bits), cpu(self.last_mask.idx), cpu(self.last_mask.block_prefix)],
        }

    def load_state_dict(self, sd: dict) -> None:
        """Restore a state written by ``state_dict`` into this instance, whose
        configuration must describe the same layout and worker count."""
        lay = self.layout
        if (sd["n_pad"], sd["k_total"], sd["workers"]) != (lay.n_pad, lay.k_total, self.cfg.workers) or \
                list(sd["layer_numel"]) != [int(n) for n in self.cfg.layer_numel]:
            raise ValueError("checkpoint was written for a different layout or worker count")
        if len(sd["r"]) != self.cfg.workers:
            raise ValueError("checkpoint holds the wrong number of residuals")
        for dst, src in [(self.x, sd["x"]), (self.m, sd["m"]), (self.v, sd["v"])]:
            if dst.shape != src.shape or dst.dtype != src.dtype:
                raise ValueError("checkpoint tensor shape or dtype does not match")
        for src in sd["r"]:
            if src.shape != self.x.shape or src.dtype != self.x.dtype:
                raise ValueError("checkpoint residual shape or dtype does not match")
        for dst, src in [(self.x, sd["x"]), (self.m, sd["m"]), (self.v, sd["v"])]:
            dst.copy_(src)
        for i, src in enumerate(sd["r"]):  # residuals are stored flat, whatever the layout
            if self.interleaved:
                interleaved_view(self.r_il, self.cfg.workers)[:, i, :].copy_(src.view(-1, 64))
            else:
                self.r[i].copy_(src)
        self._cur = 0
        for mk, key in ((self.masks[0], "pending_mask"), (self.masks[1], "last_mask")):
            for dst, src in zip((mk.bits, mk.idx, mk.block_prefix), sd[key]):
                if dst.shape != src.shape or dst.dtype != src.dtype:
                    raise ValueError("checkpoint mask shape or dtype does not match")
                dst.copy_(src)
        self.t = int(sd["t"])

    def destroy(self) -> None:
        self.ctx.destroy()
