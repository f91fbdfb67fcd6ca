"""The C-ABI library on the CPU: it loads, exports every call include/pc.h
declares, compiles layouts host-only (classification, tying, outputs) and
returns the documented error codes.  No device work is done here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import log_space_sum_amd as L
from workloads import circuits as W
from workloads import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_calls():
    src = open(os.path.join(ROOT, "include", "pc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(pc_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_call():
    names = _header_calls()
    assert len(names) >= 14, names
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"libpc.so does not export {n}"
        assert n in L.EXPORTS, f"binding does not wrap {n}"


def _classes(circ):
    h = L.pc_compile_layout(circ, device=-1)
    return h, [L.pc_layer_class(h, i) for i in range(len(circ.layers))]


def test_hmm_layers_are_shared():
    c = W.hmm(16, 5, 7)
    h, cls = _classes(c)
    sums = [k for k in cls if k >= 0]
    assert sums == [L.PC_CLASS_SHARED] * 5
    info = L.pc_layout_info(h)
    assert info["device"] == -1 and info["num_sum_layers"] == 5
    assert info["num_param_blocks"] == 2          # tied transition + initial
    assert info["num_row_segments"] == 3          # transition, initial, emission
    assert info["num_outputs"] == 1


def test_dense_strided_and_lowrank_classes():
    _, cls = _classes(W.dense_layer(32, 48, groups=3))
    assert cls[1] == L.PC_CLASS_STRIDED
    _, cls = _classes(W.dense_layer(32, 48, groups=1))
    assert cls[1] == L.PC_CLASS_SHARED
    _, cls = _classes(W.hmm(8, 4, 3, lowrank_rank=4))
    assert set(k for k in cls if k >= 0) == {L.PC_CLASS_LOWRANK, L.PC_CLASS_SHARED}


def test_hclt_levels_are_strided():
    c = W.hclt(40, 8, 5, seed=1)
    _, cls = _classes(c)
    for layer, k in zip(c.layers, cls):
        if isinstance(layer, W.Sum):
            assert k == (L.PC_CLASS_STRIDED if len(layer.groups) > 1 else L.PC_CLASS_SHARED)


def test_made_up_layouts():
    """Layouts that are not evenly strided fall back to GENERAL; groups that
    share one child list are SHARED (even with different weights)."""
    ext = W.InputExternal(0, 64)
    mk = lambda gs, n: W.Circuit("t", n, 0, 10 ** 6, [ext, W.Sum(gs)])
    # uneven child stride
    gs = [W.SumGroup(64, 4, np.array([0]), 8, 0), W.SumGroup(68, 4, np.array([8]), 8, 32),
          W.SumGroup(72, 4, np.array([24]), 8, 64)]
    _, cls = _classes(mk(gs, 76))
    assert cls[1] == L.PC_CLASS_GENERAL
    # evenly strided
    gs = [W.SumGroup(64 + 4 * g, 4, np.array([8 * g]), 8, 32 * g) for g in range(3)]
    _, cls = _classes(mk(gs, 76))
    assert cls[1] == L.PC_CLASS_STRIDED
    # shared children, separate weights
    gs = [W.SumGroup(64 + 4 * g, 4, np.array([0, 16]), 8, 64 * g) for g in range(3)]
    _, cls = _classes(mk(gs, 76))
    assert cls[1] == L.PC_CLASS_SHARED
    # block sparse
    c = W.random_block_layer(3, M_blocks=6, node_block=4, ch_blocks=5, ch_block=8)
    _, cls = _classes(c)
    assert cls[1] == L.PC_CLASS_GENERAL


def _expect(code, fn, *a):
    with pytest.raises(L.PCError) as e:
        fn(*a)
    assert e.value.code == code, str(e.value)


def test_descriptor_errors():
    ext = W.InputExternal(0, 8)
    ok = W.SumGroup(8, 2, np.array([0]), 8, 0)
    base = lambda layers, n=10, npar=100, **kw: W.Circuit("t", n, 0, npar, layers, **kw)
    # child defined later than its parent
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([W.Sum([ok]), ext]), -1)
    # node defined twice
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout,
            base([ext, W.Sum([ok, W.SumGroup(9, 1, np.array([0]), 8, 16)])]), -1)
    # node never defined
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, W.Sum([ok])], n=11), -1)
    # parameters out of range
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, W.Sum([ok])], npar=15), -1)
    # tied groups of different shape
    g2 = W.SumGroup(10, 1, np.array([0]), 4, 0)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, W.Sum([ok, g2])], n=11), -1)
    # overlapping (partially tied) parameter blocks
    g3 = W.SumGroup(10, 1, np.array([0]), 8, 8)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, W.Sum([ok, g3])], n=11), -1)
    # a child listed twice in one group
    g4 = W.SumGroup(8, 2, np.array([0, 4]), 8, 0)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, W.Sum([g4])]), -1)
    # product without children
    p = W.Product(8, 2, np.array([0, 1, 1], dtype=np.int32), np.array([0], dtype=np.int32))
    _expect(L.PC_ERR_INVALID_ARG, L.pc_compile_layout, base([ext, p]), -1)
    # LowRank rank above 64 (ranks up to 64 compile)
    c = W.hmm(4, 3, 2, lowrank_rank=65)
    _expect(L.PC_ERR_UNSUPPORTED, L.pc_compile_layout, c, -1)
    L.pc_compile_layout(W.hmm(4, 3, 2, lowrank_rank=64), -1)
    L.pc_compile_layout(W.hmm(4, 3, 2, lowrank_rank=48), -1)
    # LowRank forms: exp_sum and sum_exp compile, any other value is refused
    L.pc_compile_layout(W.hmm(4, 3, 2, lowrank_rank=4, lowrank_form="sum_exp"), -1)
    c = W.hmm(4, 3, 2, lowrank_rank=4)
    L.LOWRANK_FORMS["bogus"] = 7
    try:
        c.lowrank_form = "bogus"
        _expect(L.PC_ERR_UNSUPPORTED, L.pc_compile_layout, c, -1)
    finally:
        del L.LOWRANK_FORMS["bogus"]


def test_modes_and_workspace():
    h = L.pc_compile_layout(W.hmm(64, 6, 9), device=-1)
    assert L.pc_get_precision(h) == L.PC_PREC_AUTO
    _expect(L.PC_ERR_UNSUPPORTED, L.pc_set_precision, h, "tf32")
    _expect(L.PC_ERR_INVALID_ARG, L.pc_set_precision, h, 7)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_workspace_bytes, h, 0)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_set_split, h, "auto", "fwd", 3, 1)
    a16, a64 = L.pc_workspace_bytes(h, 16), L.pc_workspace_bytes(h, 64)
    assert 0 < a16 < a64
    # batches below 16 run fp32-level: more planes than auto at 16
    assert L.pc_workspace_bytes(h, 15) > a16
    L.pc_set_precision(h, "fp32")
    assert L.pc_get_precision(h) == L.PC_PREC_FP32
    assert L.pc_workspace_bytes(h, 16) > a16
    L.pc_set_split(h, "fp32", "param", 3, 3)
    assert L.pc_workspace_bytes(h, 16) > L.pc_workspace_bytes(h, 15) - 1


def test_options():
    h = L.pc_compile_layout(W.hmm(64, 6, 9), device=-1)
    for name, good, bad in (("layer_tile", (0, 1, 2, 3, 4, 5), (6, -1)), ("param_tile", (0, 1, 2, 3), (4,)),
                            ("split_max", (1, 2, 4, 8), (0, 3, 16)), ("fuse", (0, 1), (2, -1)),
                            ("param_chunk", (-1, 0, 1, 8, 100), (-2,)), ("lr_pack", (0, 1), (2, -1)),
                            ("sumexp_fused", (0, 1), (2, -1)), ("flow_fp8", (0, 1), (2, -1))):
        for v in good:
            L.pc_set_option(h, name, v)
        for v in bad:
            _expect(L.PC_ERR_INVALID_ARG, L.pc_set_option, h, name, v)
    _expect(L.PC_ERR_INVALID_ARG, L.pc_set_option, h, 9, 0)


def test_flow_fp8_workspace():
    """The e4m3 end products keep one byte (and a scale byte per 32) per
    operand element instead of bf16 planes: a smaller workspace in auto mode,
    the same one at fp32 level, where the option does not apply."""
    h = L.pc_compile_layout(W.hmm(64, 6, 9, lowrank_rank=16, lowrank_form="sum_exp"), device=-1)
    base = L.pc_workspace_bytes(h, 32)
    L.pc_set_option(h, "flow_fp8", 1)
    assert L.pc_workspace_bytes(h, 32) < base
    L.pc_set_precision(h, "fp32")
    f8 = L.pc_workspace_bytes(h, 32)
    L.pc_set_option(h, "flow_fp8", 0)
    assert L.pc_workspace_bytes(h, 32) == f8


def test_host_only_handle_refuses_device_calls():
    h = L.pc_compile_layout(W.hmm(8, 3, 4), device=-1)
    lib = L.lib()
    rc = lib.pc_forward(h.ptr, 4, None, None, None, None, None, None, 0, None)
    assert rc == L.PC_ERR_NO_DEVICE
    rc = lib.pc_backward(h.ptr, 4, None, None, None, None, None, 0, None, None, 0, None)
    assert rc == L.PC_ERR_NO_DEVICE
    rc = lib.pc_em_step(h.ptr, None, None, 1.0, 0.0, None)
    assert rc == L.PC_ERR_NO_DEVICE
    assert "without a device" in L.pc_last_error()
    assert lib.pc_set_precision(None, 0) == L.PC_ERR_INVALID_ARG
