"""ctypes binding of libscape (include/scape.h), same names as the C ABI.

Argument marshalling only: every step of the SCAPE path runs in the HIP
kernels of libscape.so.  Device arrays are torch tensors (PyTorch supplies
device memory and streams); host arrays are Python sequences.  If the
library is not built, every call raises - there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# SCAPE_LIB selects another build of the library (the host-sanitizer build
# the CPU suite checks its host paths with).
LIB_PATH = os.environ.get("SCAPE_LIB") or os.path.join(HERE, "libscape.so")

SCAPE_OK = 0
SCAPE_ERR_INVALID_ARG = -1
SCAPE_ERR_SHAPE = -2
SCAPE_ERR_ALIGN = -3
SCAPE_ERR_OOM = -4
SCAPE_ERR_HIP = -5
SCAPE_ERR_STATE = -6
SCAPE_MAX_WORKERS = 32
PHASES = ("ef_compact", "reduce_update", "mask_select", "mask_index")

_ERR_NAMES = {-1: "INVALID_ARG", -2: "SHAPE", -3: "ALIGN", -4: "OOM", -5: "HIP", -6: "STATE"}

_lib = None


class ScapeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"SCAPE_ERR_{_ERR_NAMES.get(code, code)}: {message}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("layer_numel", ctypes.POINTER(ctypes.c_int64)),
                ("workers", ctypes.c_int32), ("owner_shards", ctypes.c_int32), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("lr", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("keep_num", ctypes.c_uint32), ("keep_den", ctypes.c_uint32)]


class _Mask(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("block_prefix", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        cfgp, maskp = ctypes.POINTER(_Config), ctypes.POINTER(_Mask)
        sig = {
            "scape_version": [vp, vp],
            "scape_layout": [cfgp, vp, vp, vp, vp, vp],
            "scape_owner_map": [cfgp, i32, vp],
            "scape_init": [cfgp, ctypes.POINTER(vp)],
            "scape_destroy": [vp],
            "scape_workspace_bytes": [vp, vp],
            "scape_selection_flags": [vp, vp],
            "scape_set_select_path": [vp, i32],
            "scape_set_update_in_dense_pass": [vp, i32],
            "scape_set_offload_path": [vp, i32],
            "scape_step": [vp, vp, vp, vp, vp, vp, maskp, maskp, vp, vp, vp],
            "scape_step_offload": [vp, vp, vp, vp, vp, vp, maskp, maskp, vp, vp, vp],
            "scape_step_interleaved": [vp, vp, vp, vp, vp, maskp, maskp, vp, vp, vp],
            "scape_dense_step": [vp, vp, vp, vp, vp, vp],
            "scape_dense_step_interleaved": [vp, vp, vp, vp, vp, vp],
            "scape_mask_union_add": [vp, vp, vp, vp],
            "scape_mask_build": [vp, vp, i32, i32, maskp, vp],
            "scape_mask_index": [vp, maskp, vp],
            "scape_mask_index_static": [vp, i64, vp, i64, vp, vp],
            "scape_pack": [vp, i64, vp, vp],
            "scape_unpack": [vp, i64, vp, vp],
            "scape_reduce_sparse": [vp, i32, i64, vp, vp],
            "scape_profile_enable": [vp, i32],
            "scape_profile_read": [vp, vp, vp],
            "scape_copy_probe": [vp, vp, ctypes.c_uint64, vp],
            "scape_stream_probe": [vp, vp, i32, vp, vp, i32, ctypes.c_uint64, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.scape_last_error.argtypes = []
        L.scape_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def scape_last_error() -> str:
    return lib().scape_last_error().decode()


def _check(rc: int) -> None:
    if rc != SCAPE_OK:
        raise ScapeError(rc, scape_last_error())


# ----------------------------------------------------------------------------
# configuration and layout


@dataclass
class ScapeConfig:
    layer_numel: Sequence[int]
    workers: int
    keep_num: int
    keep_den: int
    owner_shards: int = 0
    beta1: float = 0.9
    beta2: float = 0.95
    lr: float = 1e-3
    eps: float = 1e-8
    weight_decay: float = 0.0

    def _c(self):
        arr = (ctypes.c_int64 * max(len(self.layer_numel), 1))(*[int(n) for n in self.layer_numel])
        c = _Config(len(self.layer_numel), arr, self.workers, self.owner_shards, self.beta1, self.beta2, self.lr,
                    self.eps, self.weight_decay, self.keep_num, self.keep_den)
        c._keep = arr  # keep the array alive with the struct
        return c


@dataclass
class Layout:
    n_pad: int
    k_total: int
    layer_offset: list
    layer_k: list
    layer_owner: list

    @property
    def n_words(self) -> int:
        return self.n_pad // 64


def scape_version():
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().scape_version(ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def scape_layout(cfg: ScapeConfig) -> Layout:
    c = cfg._c()
    L = len(cfg.layer_numel)
    n_pad, k_total = ctypes.c_int64(), ctypes.c_int64()
    off = (ctypes.c_int64 * max(L, 1))()
    kk = (ctypes.c_int64 * max(L, 1))()
    own = (ctypes.c_int32 * max(L, 1))()
    _check(lib().scape_layout(ctypes.byref(c), ctypes.byref(n_pad), ctypes.byref(k_total), off, kk, own))
    return Layout(n_pad.value, k_total.value, list(off)[:L], list(kk)[:L], list(own)[:L])


def scape_owner_map(cfg: ScapeConfig, num_shards: int) -> list:
    c = cfg._c()
    L = len(cfg.layer_numel)
    own = (ctypes.c_int32 * max(L, 1))()
    _check(lib().scape_owner_map(ctypes.byref(c), num_shards, own))
    return list(own)[:L]


# ----------------------------------------------------------------------------
# device marshalling


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shape(t, dtype, numel: Optional[int], name: str) -> None:
    """Check a tensor's type, dtype, layout and length."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


def _dev(t, dtype, numel: Optional[int], name: str) -> int:
    """Device pointer of a torch tensor, after checking its type, dtype,
    layout, length and device (all before anything reaches the library)."""
    _shape(t, dtype, numel, name)
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    return t.data_ptr()


def _host(t, dtype, numel: Optional[int], name: str) -> int:
    """A pinned host tensor (the offloaded residuals)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cpu":
        raise ValueError(f"{name} must be in host memory (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_pinned():
        raise ValueError(f"{name} must be pinned host memory (pin_memory=True)")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _ptr_array(ptrs) -> ctypes.Array:
    return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)


class Mask:
    """A mask in the library layout, backed by three device tensors."""

    def __init__(self, bits, idx, block_prefix):
        self.bits, self.idx, self.block_prefix = bits, idx, block_prefix

    def _c(self, layout: "Layout", need_index: bool = True) -> _Mask:
        """The C struct, after checking each array against `layout`: bits
        needs n_pad/64 words, idx k_total entries and block_prefix
        n_pad/64 + 1 (idx and block_prefix only when the entry point uses
        them).  Every length is checked before any device check."""
        import torch
        nw = layout.n_words
        arrs = [(self.bits, (torch.int64,), nw, "mask.bits")]
        if need_index or self.idx is not None:
            arrs.append((self.idx, (torch.int32,), max(layout.k_total, 1), "mask.idx"))
        if need_index or self.block_prefix is not None:
            arrs.append((self.block_prefix, (torch.int32,), nw + 1, "mask.block_prefix"))
        for a in arrs:
            _shape(*a)
        ptrs = {name: _dev(*a[:3], name) for *a, name in arrs}
        return _Mask(ptrs["mask.bits"], ptrs.get("mask.idx"), ptrs.get("mask.block_prefix"))

    def clear(self):
        self.bits.zero_()
        self.idx.zero_()
        self.block_prefix.zero_()


def alloc_mask(layout: Layout, device="cuda") -> Mask:
    """An all-zero mask sized for `layout` (bits int64, idx/block_prefix int32)."""
    import torch
    return Mask(torch.zeros(layout.n_words, dtype=torch.int64, device=device),
                torch.zeros(max(layout.k_total, 1), dtype=torch.int32, device=device),
                torch.zeros(layout.n_words + 1, dtype=torch.int32, device=device))


# ----------------------------------------------------------------------------
# context and entry points


class Context:
    def __init__(self, cfg: ScapeConfig):
        self._h = None
        self.cfg = cfg
        self.layout = scape_layout(cfg)
        h = ctypes.c_void_p()
        c = cfg._c()
        _check(lib().scape_init(ctypes.byref(c), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ScapeError(SCAPE_ERR_STATE, "context destroyed")
        return self._h

    def destroy(self):
        if self._h is not None:
            _check(lib().scape_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def scape_init(cfg: ScapeConfig) -> Context:
    return Context(cfg)


def scape_destroy(ctx: Context) -> None:
    ctx.destroy()


def scape_workspace_bytes(ctx: Context) -> int:
    """Device memory the context's workspaces hold, in bytes."""
    b = ctypes.c_int64()
    _check(lib().scape_workspace_bytes(ctx.handle, ctypes.byref(b)))
    return b.value


SELECT_EXACT_HISTOGRAM = 1
SELECT_KEY_PASSES = 2


def scape_selection_flags(ctx: Context) -> int:
    """Fallbacks the last mask selection took (waits for the device): bit 0
    exact histogram, bit 1 passes over the keys (SELECT_* constants)."""
    f = ctypes.c_uint32()
    _check(lib().scape_selection_flags(ctx.handle, ctypes.byref(f)))
    return f.value


SELECT_PATH_AUTO = 0
SELECT_PATH_SAMPLED = 1
SELECT_PATH_COMPACT = 2


def scape_set_select_path(ctx: Context, path: int) -> None:
    """How the context selects masks from the next call on (SELECT_PATH_*):
    the sampled multi-pass path, the two-launch compact path, or AUTO (compact
    where every layer of the range has at most 2^22 elements)."""
    _check(lib().scape_set_select_path(ctx.handle, int(path)))


OFFLOAD_PATH_AUTO = 0
OFFLOAD_PATH_STAGED = 1


def scape_set_offload_path(ctx: Context, path: int) -> None:
    """From the next call on, move scape_step_offload's residuals by the
    dense pass itself over PCIe where they are pinned, mapped host memory
    (OFFLOAD_PATH_AUTO, the default), or always through the staging
    slots (OFFLOAD_PATH_STAGED)."""
    _check(lib().scape_set_offload_path(ctx.handle, int(path)))


def scape_set_update_in_dense_pass(ctx: Context, on: bool) -> None:
    """From the next call on, let the dense pass finish the reduction and the
    update at the mask's positions where the residuals are on the device (the
    default), or make the update a pass of its own (on = False)."""
    _check(lib().scape_set_update_in_dense_pass(ctx.handle, int(bool(on))))


def scape_step(ctx: Context, x, m, v, r: Sequence, g: Sequence, cur: Mask, next: Mask, sparse_bufs: Sequence,
               key_out=None, stream=None) -> None:
    import torch
    n, W, k = ctx.layout.n_pad, ctx.cfg.workers, ctx.layout.k_total
    if len(r) != W or len(g) != W or len(sparse_bufs) != W:
        raise ValueError(f"r, g and sparse_bufs need {W} entries each")
    xp = _dev(x, torch.float32, n, "x")
    mp = _dev(m, torch.float32, n, "m")
    vp = _dev(v, torch.float32, n, "v")
    rp = _ptr_array([_dev(t, torch.float32, n, f"r[{i}]") for i, t in enumerate(r)])
    gp = _ptr_array([_dev(t, (torch.int16, torch.bfloat16, torch.uint16), n, f"g[{i}]") for i, t in enumerate(g)])
    bp = _ptr_array([_dev(t, torch.float32, k, f"sparse_bufs[{i}]") for i, t in enumerate(sparse_bufs)])
    kp = _dev(key_out, torch.int32, n, "key_out") if key_out is not None else None
    c, nx = cur._c(ctx.layout), next._c(ctx.layout)
    _check(lib().scape_step(ctx.handle, xp, mp, vp, rp, gp, ctypes.byref(c), ctypes.byref(nx), bp, kp,
                            _stream(stream)))


def scape_step_interleaved(ctx: Context, xv, m, r_il, g_il, cur: Mask, next: Mask, sparse_bufs: Sequence,
                           key_out=None, stream=None) -> None:
    """scape_step in the interleaved layout: xv holds (x, v) pairs (2*n_pad
    fp32), r_il (fp32) and g_il (bf16 bits) n_pad*W elements each, word w of
    worker i at [(w*W + i)*64, (w*W + i)*64 + 64)."""
    import torch
    n, W, k = ctx.layout.n_pad, ctx.cfg.workers, ctx.layout.k_total
    if len(sparse_bufs) != W:
        raise ValueError(f"sparse_bufs needs {W} entries")
    xp = _dev(xv, torch.float32, 2 * n, "xv")
    mp = _dev(m, torch.float32, n, "m")
    rp = _dev(r_il, torch.float32, n * W, "r_il")
    gp = _dev(g_il, (torch.int16, torch.bfloat16, torch.uint16), n * W, "g_il")
    bp = _ptr_array([_dev(t, torch.float32, k, f"sparse_bufs[{i}]") for i, t in enumerate(sparse_bufs)])
    kp = _dev(key_out, torch.int32, n, "key_out") if key_out is not None else None
    c, nx = cur._c(ctx.layout), next._c(ctx.layout)
    _check(lib().scape_step_interleaved(ctx.handle, xp, mp, rp, gp, ctypes.byref(c), ctypes.byref(nx), bp, kp,
                                        _stream(stream)))


def scape_step_offload(ctx: Context, x, m, v, r_host: Sequence, g: Sequence, cur: Mask, next: Mask,
                       sparse_bufs: Sequence, key_out=None, stream=None) -> None:
    """scape_step with the residuals in pinned host tensors."""
    import torch
    n, W, k = ctx.layout.n_pad, ctx.cfg.workers, ctx.layout.k_total
    if len(r_host) != W or len(g) != W or len(sparse_bufs) != W:
        raise ValueError(f"r_host, g and sparse_bufs need {W} entries each")
    xp = _dev(x, torch.float32, n, "x")
    mp = _dev(m, torch.float32, n, "m")
    vp = _dev(v, torch.float32, n, "v")
    rp = _ptr_array([_host(t, torch.float32, n, f"r_host[{i}]") for i, t in enumerate(r_host)])
    gp = _ptr_array([_dev(t, (torch.int16, torch.bfloat16, torch.uint16), n, f"g[{i}]") for i, t in enumerate(g)])
    bp = _ptr_array([_dev(t, torch.float32, k, f"sparse_bufs[{i}]") for i, t in enumerate(sparse_bufs)])
    kp = _dev(key_out, torch.int32, n, "key_out") if key_out is not None else None
    c, nx = cur._c(ctx.layout), next._c(ctx.layout)
    _check(lib().scape_step_offload(ctx.handle, xp, mp, vp, rp, gp, ctypes.byref(c), ctypes.byref(nx), bp, kp,
                                    _stream(stream)))


def scape_dense_step(ctx: Context, x, m, v, g: Sequence, stream=None) -> None:
    import torch
    n, W = ctx.layout.n_pad, ctx.cfg.workers
    if len(g) != W:
        raise ValueError(f"g needs {W} entries")
    xp = _dev(x, torch.float32, n, "x")
    mp = _dev(m, torch.float32, n, "m")
    vp = _dev(v, torch.float32, n, "v")
    gp = _ptr_array([_dev(t, (torch.int16, torch.bfloat16, torch.uint16), n, f"g[{i}]") for i, t in enumerate(g)])
    _check(lib().scape_dense_step(ctx.handle, xp, mp, vp, gp, _stream(stream)))


def scape_dense_step_interleaved(ctx: Context, x, m, v, g_il, stream=None) -> None:
    """scape_dense_step with the gradients in the worker-interleaved layout."""
    import torch
    n, W = ctx.layout.n_pad, ctx.cfg.workers
    xp = _dev(x, torch.float32, n, "x")
    mp = _dev(m, torch.float32, n, "m")
    vp = _dev(v, torch.float32, n, "v")
    gp = _dev(g_il, (torch.int16, torch.bfloat16, torch.uint16), n * W, "g_il")
    _check(lib().scape_dense_step_interleaved(ctx.handle, xp, mp, vp, gp, _stream(stream)))


def interleaved_view(t, W: int):
    """Worker i's elements of a worker-interleaved array `t` (n_pad*W) as a
    strided (n_pad/64, 64) view; .reshape(-1) copies them out flat."""
    return t.view(-1, W, 64)


def scape_mask_build(ctx: Context, mtilde, out: Mask, num_shards: int = 0, shard: int = -1, stream=None) -> None:
    import torch
    mp = _dev(mtilde, torch.float32, ctx.layout.n_pad, "mtilde")
    o = out._c(ctx.layout, need_index=num_shards <= 0 or shard < 0)
    _check(lib().scape_mask_build(ctx.handle, mp, num_shards, shard, ctypes.byref(o), _stream(stream)))


def scape_mask_union_add(ctx: Context, mtilde, acc_bits, stream=None) -> None:
    import torch
    mp = _dev(mtilde, torch.float32, ctx.layout.n_pad, "mtilde")
    ap = _dev(acc_bits, torch.int64, ctx.layout.n_pad // 64, "acc_bits")
    _check(lib().scape_mask_union_add(ctx.handle, mp, ap, _stream(stream)))


def scape_mask_index(ctx: Context, mask: Mask, stream=None) -> None:
    c = mask._c(ctx.layout)
    _check(lib().scape_mask_index(ctx.handle, ctypes.byref(c), _stream(stream)))


def scape_mask_index_static(bits, idx, block_prefix, n_words: Optional[int] = None, k_cap: Optional[int] = None,
                            stream=None) -> None:
    """idx and block_prefix of the mask in `bits` without a context or any
    allocation (the library's static scratch)."""
    import torch
    n_words = bits.numel() if n_words is None else int(n_words)
    k_cap = (idx.numel() if idx is not None else 0) if k_cap is None else int(k_cap)
    bp = _dev(bits, torch.int64, n_words, "bits")
    ip = _dev(idx, torch.int32, k_cap, "idx") if idx is not None else None
    pp = _dev(block_prefix, torch.int32, n_words + 1, "block_prefix")
    _check(lib().scape_mask_index_static(bp, n_words, ip, k_cap, pp, _stream(stream)))


def scape_pack(pred, bits, n: Optional[int] = None, stream=None) -> None:
    import torch
    n = pred.numel() if n is None else n
    pp = _dev(pred, (torch.uint8, torch.bool), n, "pred")
    bp = _dev(bits, torch.int64, (n + 63) // 64, "bits")
    _check(lib().scape_pack(pp, n, bp, _stream(stream)))


def scape_unpack(bits, pred, n: Optional[int] = None, stream=None) -> None:
    import torch
    n = pred.numel() if n is None else n
    bp = _dev(bits, torch.int64, (n + 63) // 64, "bits")
    pp = _dev(pred, (torch.uint8, torch.bool), n, "pred")
    _check(lib().scape_unpack(bp, n, pp, _stream(stream)))


def scape_reduce_sparse(bufs: Sequence, out, k: Optional[int] = None, stream=None) -> None:
    import torch
    k = out.numel() if k is None else k
    ptrs = _ptr_array([_dev(b, torch.float32, k, f"bufs[{i}]") for i, b in enumerate(bufs)])
    op = _dev(out, torch.float32, k, "out")
    _check(lib().scape_reduce_sparse(ptrs, len(bufs), k, op, _stream(stream)))


def scape_copy_probe(src, dst, nbytes: Optional[int] = None, stream=None) -> None:
    """Copy nbytes (default: all of src) from src to dst, both device tensors
    (16-byte aligned, nbytes a multiple of 16), with the library's plain
    stream-copy kernel."""
    import torch
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name} is smaller than {nbytes} bytes")
    _check(lib().scape_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream)))


def scape_stream_probe(srcs: Sequence, src_widths: Sequence[int], dsts: Sequence, dst_widths: Sequence[int],
                       n_words: int, stream=None) -> None:
    """A pass that reads every tensor of srcs and writes every tensor of dsts
    over n_words 64-element words, width bytes per element (2, 4, 8 or 16)
    each, with no other work (scape_stream_probe in include/scape.h)."""
    import torch
    for t, w in list(zip(srcs, src_widths)) + list(zip(dsts, dst_widths)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("arrays must be contiguous device tensors")
        if t.numel() * t.element_size() < int(n_words) * 64 * int(w):
            raise ValueError(f"an array of {t.numel() * t.element_size()} bytes is smaller than "
                             f"{n_words} words of width {w}")
    sw = (ctypes.c_uint32 * max(len(srcs), 1))(*[int(w) for w in src_widths])
    dw = (ctypes.c_uint32 * max(len(dsts), 1))(*[int(w) for w in dst_widths])
    _check(lib().scape_stream_probe(_ptr_array([t.data_ptr() for t in srcs]), sw, len(srcs),
                                    _ptr_array([t.data_ptr() for t in dsts]), dw, len(dsts), int(n_words),
                                    _stream(stream)))


def scape_profile_enable(ctx: Context, enable: bool = True) -> None:
    _check(lib().scape_profile_enable(ctx.handle, 1 if enable else 0))


def scape_profile_read(ctx: Context):
    """(dict phase -> summed ms, steps recorded)."""
    ms = (ctypes.c_double * 4)()
    steps = ctypes.c_int64()
    _check(lib().scape_profile_read(ctx.handle, ms, ctypes.byref(steps)))
    return dict(zip(PHASES, list(ms))), steps.value
