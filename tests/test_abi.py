"""The C ABI on the host: library loads, exports what include/scape.h
declares, computes the layout the oracle computes, and rejects bad arguments
before touching the GPU.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scape.h")


@pytest.fixture(scope="module")
def sc():
    import sparse_communication_adam_amd as sc
    if not os.path.exists(sc.LIB_PATH):
        sc.build()
    return sc


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(scape_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["scape_init", "scape_destroy", "scape_layout", "scape_step", "scape_step_offload", "scape_dense_step",
              "scape_mask_build",
              "scape_mask_index", "scape_mask_union_add",
              "scape_pack", "scape_unpack", "scape_reduce_sparse", "scape_last_error", "scape_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(sc):
    lib = ctypes.CDLL(sc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version(sc):
    assert sc.scape_version() == (1, 0)


def _cfg(sc, wl, **kw):
    d = dict(layer_numel=wl.layer_sizes, workers=wl.W, keep_num=wl.keep_num, keep_den=wl.keep_den)
    d.update(kw)
    return sc.ScapeConfig(**d)


@pytest.mark.parametrize("name", list(synth.WORKLOADS) + ["ragged"])
def test_layout_matches_oracle(sc, name):
    wl = synth.ragged() if name == "ragged" else synth.WORKLOADS[name]
    got = sc.scape_layout(_cfg(sc, wl))
    exp = oracle.layout(wl.layer_sizes, wl.keep_num, wl.keep_den, wl.W)
    assert got.n_pad == exp.n_pad and got.k_total == exp.k_total
    assert got.layer_offset == exp.off.tolist()
    assert got.layer_k == exp.k.tolist()
    assert got.layer_owner == exp.owner.tolist()
    for P in (1, 7, 32):
        om = sc.scape_owner_map(_cfg(sc, wl), P)
        assert om == [oracle.owner(int(o), int(n), exp.n_pad, P) for o, n in zip(exp.off, exp.sizes)]


def test_layout_edge_sizes(sc):
    cfg = sc.ScapeConfig(layer_numel=[0, 1, 63, 64, 65, 0], workers=2, keep_num=1, keep_den=3)
    got = sc.scape_layout(cfg)
    exp = oracle.layout([0, 1, 63, 64, 65, 0], 1, 3, 2)
    assert got.layer_offset == exp.off.tolist() and got.layer_k == exp.k.tolist() and got.n_pad == exp.n_pad


@pytest.mark.parametrize("kw,code", [
    (dict(layer_numel=[]), -2),
    (dict(workers=0), -1),
    (dict(workers=33), -1),
    (dict(owner_shards=5, workers=4), -1),
    (dict(keep_num=2, keep_den=1), -1),
    (dict(keep_den=0), -1),
    (dict(beta1=1.0), -1),
    (dict(beta2=-0.1), -1),
    (dict(lr=float("nan")), -1),
    (dict(layer_numel=[-5]), -2),
    (dict(layer_numel=[2 ** 31]), -2),
    (dict(layer_numel=[2 ** 30, 2 ** 30]), -2),
])
def test_invalid_config_rejected(sc, kw, code):
    d = dict(layer_numel=[1024], workers=4, keep_num=1, keep_den=10)
    d.update(kw)
    with pytest.raises(sc.ScapeError) as e:
        sc.scape_layout(sc.ScapeConfig(**d))
    assert e.value.code == code
    assert sc.scape_last_error()


def test_null_arguments_rejected_before_any_launch(sc):
    lib = sc.lib()
    assert lib.scape_step(None, None, None, None, None, None, None, None, None, None, None) == -1
    assert "ctx" in sc.scape_last_error()
    assert lib.scape_dense_step(None, None, None, None, None, None) == -1
    assert lib.scape_step_offload(None, None, None, None, None, None, None, None, None, None, None) == -1
    assert lib.scape_mask_union_add(None, None, None, None) == -1
    assert lib.scape_mask_build(None, None, 0, -1, None, None) == -1
    assert lib.scape_mask_index(None, None, None) == -1
    assert lib.scape_pack(None, -1, None, None) == -1
    assert lib.scape_pack(None, 0, None, None) == 0  # n == 0 enqueues nothing
    assert lib.scape_pack(None, 10, None, None) == -1
    assert lib.scape_unpack(None, 2 ** 37, None, None) == -2
    assert lib.scape_reduce_sparse(None, 0, 1, None, None) == -1
    assert lib.scape_reduce_sparse(None, 33, 1, None, None) == -1
    assert lib.scape_reduce_sparse(None, 4, -1, None, None) == -1
    assert lib.scape_reduce_sparse(None, 4, 0, None, None) == 0
    bufs = (ctypes.c_void_p * 2)(8, 12)
    assert lib.scape_reduce_sparse(bufs, 2, 4, ctypes.c_void_p(2), None) == -3  # misaligned out
    assert lib.scape_pack(ctypes.c_void_p(16), 64, ctypes.c_void_p(4), None) == -3  # bits not 8-aligned
    assert lib.scape_profile_enable(None, 1) == -1
    assert lib.scape_set_select_path(None, 0) == -1
    assert lib.scape_set_update_in_dense_pass(None, 1) == -1
    assert lib.scape_set_offload_path(None, 0) == -1
    assert lib.scape_copy_probe(None, None, 0, None) == 0  # nothing to copy
    assert lib.scape_copy_probe(None, None, 16, None) == -1
    assert lib.scape_copy_probe(ctypes.c_void_p(16), ctypes.c_void_p(8), 16, None) == -3  # dst misaligned
    assert lib.scape_copy_probe(ctypes.c_void_p(16), ctypes.c_void_p(32), 24, None) == -2  # not whole 16-byte units
    assert lib.scape_init(None, None) == -1
    assert lib.scape_stream_probe(None, None, 0, None, None, 0, 4, None) == -1  # no arrays
    assert lib.scape_stream_probe(None, None, 5, None, None, 0, 4, None) == -1  # too many
    w3 = (ctypes.c_uint32 * 1)(3)
    one = (ctypes.c_void_p * 1)(16)
    assert lib.scape_stream_probe(one, w3, 1, None, None, 0, 4, None) == -1  # width 3
    w8 = (ctypes.c_uint32 * 1)(8)
    odd = (ctypes.c_void_p * 1)(4)
    assert lib.scape_stream_probe(odd, w8, 1, None, None, 0, 4, None) == -3  # not aligned to its width


def test_init_without_gpu_reports_hip_error(sc):
    """Valid config, no GPU in this container: a HIP error, never a crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(sc.ScapeError) as e:
        sc.scape_init(sc.ScapeConfig(layer_numel=[4096], workers=2, keep_num=1, keep_den=10))
    assert e.value.code in (-4, -5)


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    import sparse_communication_adam_amd._scape as s
    monkeypatch.setattr(s, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(s, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        s.lib()


def test_binding_requires_pinned_host_residuals(sc):
    """The offloaded step's residuals must be pinned host memory: a device
    tensor, a pageable host tensor or a wrong dtype is refused before any
    call into the library."""
    import torch
    from sparse_communication_adam_amd._scape import _host
    with pytest.raises(ValueError, match="pinned"):
        _host(torch.zeros(16, dtype=torch.float32), torch.float32, 16, "r_host[0]")
    with pytest.raises(TypeError):
        _host(torch.zeros(16, dtype=torch.float64), torch.float32, 16, "r_host[0]")
    with pytest.raises(TypeError):
        _host(np.zeros(16, np.float32), torch.float32, 16, "r_host[0]")


def test_binding_checks_mask_lengths_against_the_layout(sc):
    """A mask array shorter than the layout needs is refused before anything
    reaches the library: bits n_pad/64 words, idx k_total, block_prefix
    n_pad/64 + 1 (length is checked before the device, so this runs on the
    host)."""
    import torch
    lay = sc.scape_layout(_cfg(sc, synth.ragged()))
    nw, k = lay.n_words, lay.k_total
    ok = dict(bits=torch.zeros(nw, dtype=torch.int64), idx=torch.zeros(k, dtype=torch.int32),
              block_prefix=torch.zeros(nw + 1, dtype=torch.int32))
    for name, short in [("bits", torch.zeros(nw - 1, dtype=torch.int64)), ("idx", torch.zeros(k - 1, dtype=torch.int32)),
                        ("block_prefix", torch.zeros(nw, dtype=torch.int32))]:
        m = sc.Mask(**{**ok, name: short})
        with pytest.raises(ValueError, match=f"mask.{name} has"):
            m._c(lay)
    # a shard build needs only the bits
    with pytest.raises(ValueError, match="mask.bits has"):
        sc.Mask(torch.zeros(nw - 1, dtype=torch.int64), None, None)._c(lay, need_index=False)
    # right lengths: the next check is the device (these are host tensors)
    with pytest.raises(ValueError, match="must be on the GPU"):
        sc.Mask(**ok)._c(lay)
