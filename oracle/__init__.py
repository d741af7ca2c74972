"""Python access to the SCAPE step oracle (``scape_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of bench.py.  The product package never imports it.

Thin ctypes marshalling around the C oracle; every step of the method runs in
C.  Arrays are numpy, flat, in the layout ``layout()`` returns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SCAPE_ORACLE_LIB selects another build of the same source (the sanitizer
# build the CPU suite runs once under AddressSanitizer and UBSan).
LIB_PATH = os.environ.get("SCAPE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build_cmd(out: str, sanitize: bool = False) -> list:
    return (["gcc", "-O2", "-fPIC", "-shared", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
            + (SANITIZE_FLAGS if sanitize else []) + [os.path.join(_HERE, "scape_oracle.c"), "-o", out, "-lm"])


def build(force: bool = True, sanitize: bool = False, out: str = None) -> str:
    """Compile the oracle (gcc, OpenMP); with sanitize, an AddressSanitizer
    and UBSan build to `out` (load it with the gcc ASan runtime preloaded)."""
    out = out or LIB_PATH
    if force or not os.path.exists(out):
        subprocess.run(build_cmd(out + ".tmp", sanitize), check=True)
        os.replace(out + ".tmp", out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("off", ctypes.c_void_p), ("n", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("owner", ctypes.c_void_p), ("n_pad", ctypes.c_int64),
                ("W", ctypes.c_int32), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("lr", ctypes.c_float), ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        L.oracle_keep_count.argtypes = [i64, u32, u32]
        L.oracle_keep_count.restype = i64
        L.oracle_owner.argtypes = [i64, i64, i64, i32]
        L.oracle_owner.restype = i32
        L.oracle_layout.argtypes = [i32, vp, u32, u32, i32, vp, vp, vp, vp]
        L.oracle_layout.restype = None
        L.oracle_pack.argtypes = [vp, i64, vp]
        L.oracle_pack.restype = None
        L.oracle_unpack.argtypes = [vp, i64, vp]
        L.oracle_unpack.restype = None
        L.oracle_mask_index.argtypes = [vp, i64, vp, i64, vp]
        L.oracle_mask_index.restype = i64
        L.oracle_topk.argtypes = [vp, i64, i64, vp]
        L.oracle_topk.restype = None
        L.oracle_mask_from_keys.argtypes = [i32, vp, vp, vp, vp, i32, vp, vp]
        L.oracle_mask_from_keys.restype = None
        L.oracle_keys_of.argtypes = [vp, i64, vp]
        L.oracle_keys_of.restype = None
        L.oracle_reduce.argtypes = [vp, i32, i64, vp]
        L.oracle_reduce.restype = None
        L.oracle_step.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                  vp, vp, vp]
        L.oracle_step.restype = i64
        L.oracle_dense_step.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp]
        L.oracle_dense_step.restype = None
        L.oracle_union_mask.argtypes = [i32, vp, vp, vp, i32, vp, vp]
        L.oracle_union_mask.restype = None
        _lib = L
    return _lib


def threads() -> int:
    """Threads the oracle's parallel loops use (OMP_NUM_THREADS)."""
    return int(lib().oracle_threads())


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _ptrs(arrs: Sequence[np.ndarray]) -> np.ndarray:
    return np.array([_p(a) for a in arrs], dtype=np.uint64)


# ----------------------------------------------------------------------------
# layout


@dataclass
class Layout:
    sizes: np.ndarray   # int64 [L]
    off: np.ndarray     # int64 [L]
    k: np.ndarray       # int64 [L]
    owner: np.ndarray   # int32 [L]
    n_pad: int

    @property
    def L(self) -> int:
        return int(self.sizes.size)

    @property
    def n_words(self) -> int:
        return self.n_pad // 64

    @property
    def k_total(self) -> int:
        return int(np.minimum(self.k, self.sizes).sum())


def keep_count(n: int, num: int, den: int) -> int:
    return int(lib().oracle_keep_count(n, num, den))


def owner(off: int, n: int, n_total: int, P: int) -> int:
    return int(lib().oracle_owner(off, n, n_total, P))


def layout(sizes: Sequence[int], keep_num: int, keep_den: int, P: int) -> Layout:
    sizes = np.ascontiguousarray(sizes, dtype=np.int64)
    L = sizes.size
    off = np.zeros(L, np.int64)
    k = np.zeros(L, np.int64)
    own = np.zeros(L, np.int32)
    n_pad = np.zeros(1, np.int64)
    lib().oracle_layout(L, _p(sizes), keep_num, keep_den, P, _p(off), _p(k), _p(own), _p(n_pad))
    return Layout(sizes, off, k, own, int(n_pad[0]))


def sub_layout(full: Layout, layers: Sequence[int]) -> Layout:
    """The given layers of ``full`` packed densely, keeping their k and owner.

    Layers are independent in a step, so an oracle run on this sub-layout
    reproduces exactly what the full run computes on those layers.
    """
    layers = list(layers)
    sizes = full.sizes[layers].copy()
    off = np.zeros(len(layers), np.int64)
    cur = 0
    for i, n in enumerate(sizes):
        off[i] = cur
        cur += (int(n) + 63) // 64 * 64
    return Layout(sizes, off, full.k[layers].copy(), full.owner[layers].copy(), cur)


# ----------------------------------------------------------------------------
# masks


def pack(pred: np.ndarray) -> np.ndarray:
    pred = np.ascontiguousarray(pred, dtype=np.uint8)
    words = np.zeros((pred.size + 63) // 64, np.uint64)
    lib().oracle_pack(_p(pred), pred.size, _p(words))
    return words


def unpack(words: np.ndarray, n: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint64)
    pred = np.zeros(n, np.uint8)
    lib().oracle_unpack(_p(words), n, _p(pred))
    return pred


def mask_index(words: np.ndarray, idx_cap: Optional[int] = None):
    """(idx, prefix, count) of a packed mask."""
    words = np.ascontiguousarray(words, dtype=np.uint64)
    nw = words.size
    cnt = int(lib().oracle_mask_index(_p(words), nw, None, 0, None))
    cap = cnt if idx_cap is None else idx_cap
    idx = np.zeros(max(cap, 1), np.uint32)
    prefix = np.zeros(nw + 1, np.uint32)
    lib().oracle_mask_index(_p(words), nw, _p(idx), cap, _p(prefix))
    return idx[:min(cnt, cap)], prefix, cnt


def topk(keys: np.ndarray, k: int) -> np.ndarray:
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    sel = np.zeros(max(keys.size, 1), np.uint8)
    lib().oracle_topk(_p(keys), keys.size, k, _p(sel))
    return sel[:keys.size]


def keys_of(mtilde: np.ndarray) -> np.ndarray:
    mtilde = np.ascontiguousarray(mtilde, dtype=np.float32)
    key = np.zeros(max(mtilde.size, 1), np.uint32)
    lib().oracle_keys_of(_p(mtilde), mtilde.size, _p(key))
    return key[:mtilde.size]


def mask_from_keys(lay: Layout, keys: np.ndarray, shard: int = -1, owner_map=None,
                   words: Optional[np.ndarray] = None) -> np.ndarray:
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    assert keys.size == lay.n_pad
    own = np.ascontiguousarray(lay.owner if owner_map is None else owner_map, dtype=np.int32)
    if words is None:
        words = np.zeros(lay.n_words, np.uint64)
    lib().oracle_mask_from_keys(lay.L, _p(lay.off), _p(lay.sizes), _p(lay.k), _p(own), shard,
                                _p(keys), _p(words))
    return words


def union_mask(lay: Layout, keys: Sequence[np.ndarray]) -> np.ndarray:
    """The fill-in union: each worker's per-layer top-k of its own keys over
    every layer, OR-ed into one packed mask."""
    keys = [np.ascontiguousarray(kk, dtype=np.uint32) for kk in keys]
    for kk in keys:
        assert kk.size == lay.n_pad
    words = np.zeros(lay.n_words, np.uint64)
    kp = _ptrs(keys)
    lib().oracle_union_mask(lay.L, _p(lay.off), _p(lay.sizes), _p(lay.k), len(keys), _p(kp), _p(words))
    return words


def reduce(bufs: Sequence[np.ndarray]) -> np.ndarray:
    bufs = [np.ascontiguousarray(b, dtype=np.float32) for b in bufs]
    k = bufs[0].size
    out = np.zeros(max(k, 1), np.float32)
    ptrs = _ptrs(bufs)
    lib().oracle_reduce(_p(ptrs), len(bufs), k, _p(out))
    return out[:k]


# ----------------------------------------------------------------------------
# step


@dataclass
class Hyper:
    beta1: float = 0.9
    beta2: float = 0.95
    lr: float = 1e-3
    eps: float = 1e-8
    weight_decay: float = 0.0


@dataclass
class State:
    x: np.ndarray
    m: np.ndarray
    v: np.ndarray
    r: List[np.ndarray]

    @staticmethod
    def zeros(n_pad: int, W: int, x: Optional[np.ndarray] = None) -> "State":
        return State(np.zeros(n_pad, np.float32) if x is None else np.array(x, np.float32),
                     np.zeros(n_pad, np.float32), np.zeros(n_pad, np.float32),
                     [np.zeros(n_pad, np.float32) for _ in range(W)])

    def copy(self) -> "State":
        return State(self.x.copy(), self.m.copy(), self.v.copy(), [a.copy() for a in self.r])


@dataclass
class StepOut:
    sent: List[np.ndarray]    # per worker, candidates at M_t (ascending positions)
    bbar: np.ndarray          # reduced buffer
    key: np.ndarray           # mask statistic per element
    next_words: np.ndarray    # M_{t+1} bits
    next_idx: np.ndarray      # M_{t+1} positions
    next_prefix: np.ndarray   # M_{t+1} per-word prefix (n_words + 1)
    count: int                # |M_t|


def step(lay: Layout, hp: Hyper, st: State, grads: Sequence[np.ndarray], cur_words: np.ndarray,
         owner_map: Optional[np.ndarray] = None) -> StepOut:
    """One oracle step; updates ``st`` in place and returns the step's outputs."""
    W = len(st.r)
    assert len(grads) == W
    grads = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    for a in [st.x, st.m, st.v] + st.r:
        assert a.dtype == np.float32 and a.size == lay.n_pad and a.flags.c_contiguous
    for g in grads:
        assert g.size == lay.n_pad
    cur_words = np.ascontiguousarray(cur_words, dtype=np.uint64)
    assert cur_words.size == lay.n_words
    own = np.ascontiguousarray(lay.owner if owner_map is None else owner_map, dtype=np.int32)
    cap = max(int(np.unpackbits(cur_words.view(np.uint8)).sum()), 1)
    sent = [np.zeros(cap, np.float32) for _ in range(W)]
    bbar = np.zeros(cap, np.float32)
    key = np.zeros(lay.n_pad, np.uint32)
    nw = np.zeros(lay.n_words, np.uint64)
    nidx = np.zeros(max(lay.k_total, 1), np.uint32)
    npre = np.zeros(lay.n_words + 1, np.uint32)
    prob = _Problem(lay.L, _p(lay.off), _p(lay.sizes), _p(lay.k), _p(own), lay.n_pad, W,
                    hp.beta1, hp.beta2, hp.lr, hp.eps, hp.weight_decay)
    rp, gp, sp = _ptrs(st.r), _ptrs(grads), _ptrs(sent)
    cnt = lib().oracle_step(ctypes.byref(prob), _p(st.x), _p(st.m), _p(st.v), _p(rp), _p(gp),
                            _p(cur_words), _p(sp), _p(bbar), cap, _p(key), _p(nw), _p(nidx), _p(npre))
    assert cnt >= 0
    return StepOut([s[:cnt] for s in sent], bbar[:cnt], key, nw, nidx[:int(npre[-1])], npre, int(cnt))


def dense_step(lay: Layout, hp: Hyper, x: np.ndarray, m: np.ndarray, v: np.ndarray,
               grads: Sequence[np.ndarray]) -> None:
    """One dense AdamS step (the comparison baseline); updates x, m, v in place."""
    W = len(grads)
    grads = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    for a in (x, m, v):
        assert a.dtype == np.float32 and a.size == lay.n_pad and a.flags.c_contiguous
    for g in grads:
        assert g.size == lay.n_pad
    prob = _Problem(lay.L, _p(lay.off), _p(lay.sizes), _p(lay.k), _p(lay.owner), lay.n_pad, W,
                    hp.beta1, hp.beta2, hp.lr, hp.eps, hp.weight_decay)
    gp = _ptrs(grads)
    lib().oracle_dense_step(ctypes.byref(prob), _p(x), _p(m), _p(v), _p(gp))
