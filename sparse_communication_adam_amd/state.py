"""Device state of one SCAPE optimizer instance and its step loop.

Holds the fp32 master parameters x, moments m and v, the W residuals, the two
mask slots and the W sparse buffers as torch tensors on one GPU, and calls
``scape_step``.  The mask built at step t is used at step t+1 (Delayed Mask
Usage, gist.science Technical Summary s.2): after each step the two mask
slots swap roles.  The first step uses an all-zero mask.  With
``offload=True`` the residuals live in pinned host memory and each step calls
``scape_step_offload`` (Memory Optimization, same section).

``capture`` records the step as HIP graphs, for small models whose step is
bound by its ~30 kernel launches: ``step_graph`` then replays it with one
launch.  scape_step never waits on the host, clears memory with kernels, and
joins its second stream back with events, so it can be captured.
"""
from __future__ import annotations

from typing import Optional, Sequence

from ._scape import Context, Mask, ScapeConfig, alloc_mask, scape_step, scape_step_offload


class ScapeState:
    def __init__(self, cfg: ScapeConfig, device: str = "cuda", x=None, offload: bool = False):
        import torch
        self.cfg = cfg
        self.ctx = Context(cfg)
        self.layout = self.ctx.layout
        n, W, k = self.layout.n_pad, cfg.workers, self.layout.k_total
        f32 = dict(dtype=torch.float32, device=device)
        self.x = torch.zeros(n, **f32) if x is None else x
        self.m = torch.zeros(n, **f32)
        self.v = torch.zeros(n, **f32)
        self.offload = offload
        if offload:
            self.r = [torch.zeros(n, dtype=torch.float32, pin_memory=True) for _ in range(W)]
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

    def step(self, grads: Sequence, stream=None, key_out: Optional[bool] = True) -> None:
        """One step with the W workers' bfloat16 gradients (int16 views).
        key_out=True also writes the full statistic keys into ``self.key``
        (4 bytes per element more); the mask does not depend on it."""
        fn = scape_step_offload if self.offload else scape_step
        fn(self.ctx, self.x, self.m, self.v, self.r, grads, self.cur_mask, self.next_mask, self.sparse,
           self.key if key_out else None, stream)
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
        self._graph_grads = list(grads)
        graphs = []
        for cur in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
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

    def destroy(self) -> None:
        self.ctx.destroy()
