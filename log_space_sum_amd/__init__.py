"""Python binding of the MI355X probabilistic-circuit sum-layer library.

Thin ctypes marshalling over the C ABI declared in ``include/pc.h``: the
functions here carry the C names, check argument types and sizes, and pass
device pointers of torch tensors and the current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  The
library is ``libpc.so`` next to this file, built by ``log_space_sum_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpc.so")

PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED, PC_ERR_WORKSPACE, PC_ERR_HIP, PC_ERR_NO_DEVICE = range(6)
PC_PREC_AUTO, PC_PREC_FP32, PC_PREC_TF32 = 0, 1, 2
PC_LAYER_INPUT_CAT, PC_LAYER_INPUT_EXTERNAL, PC_LAYER_PRODUCT, PC_LAYER_SUM = 0, 1, 2, 3
PC_CLASS_SHARED, PC_CLASS_STRIDED, PC_CLASS_GENERAL, PC_CLASS_LOWRANK = 0, 1, 2, 3
PC_BWD_SEEDED = 1
PC_LOWRANK_EXP_SUM, PC_LOWRANK_SUM_EXP = 0, 1
LOWRANK_FORMS = {"exp_sum": PC_LOWRANK_EXP_SUM, "sum_exp": PC_LOWRANK_SUM_EXP}
PC_NUM_KERNEL_KINDS = 16
KERNEL_KINDS = ["sum_fwd_gemm", "elem_flow_gemm", "param_flow_gemm", "weight_split", "column_max",
                "exp_children", "scaled_flows", "input_fwd", "input_bwd", "product_fwd",
                "product_bwd", "em", "lowrank_fwd", "lowrank_bwd", "other", "lowrank_coef"]
MODES = {"auto": PC_PREC_AUTO, "fp32": PC_PREC_FP32, "tf32": PC_PREC_TF32}
GEMM_KINDS = {"fwd": 0, "elem": 1, "param": 2}

_i32p = C.POINTER(C.c_int32)


class pc_sum_group(C.Structure):
    _fields_ = [("out_start", C.c_int32), ("num_nodes", C.c_int32), ("num_ch_blocks", C.c_int32),
                ("ch_block_size", C.c_int32), ("ch_block_start", _i32p), ("param_offset", C.c_int64),
                ("lowrank_slot", C.c_int32)]


class pc_layer_desc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("node_start", C.c_int32), ("num_nodes", C.c_int32),
                ("num_cats", C.c_int32), ("num_rows", C.c_int32), ("param_offset", C.c_int64),
                ("var", _i32p), ("row", _i32p), ("ch_ptr", _i32p), ("ch_ids", _i32p),
                ("num_groups", C.c_int32), ("groups", C.POINTER(pc_sum_group))]


class pc_circuit_desc(C.Structure):
    _fields_ = [("num_nodes", C.c_int32), ("num_vars", C.c_int32), ("num_params", C.c_int64),
                ("num_layers", C.c_int32), ("layers", C.POINTER(pc_layer_desc)), ("root", C.c_int32),
                ("lowrank_rank", C.c_int32), ("lowrank_form", C.c_int32)]


class pc_lowrank_io(C.Structure):
    _fields_ = [("num_slots", C.c_int32), ("A", C.POINTER(C.c_void_p)), ("B", C.POINTER(C.c_void_p)),
                ("dA", C.POINTER(C.c_void_p)), ("dB", C.POINTER(C.c_void_p)), ("z_flows", C.c_void_p)]


class pc_layout_summary(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_sum_layers", C.c_int32), ("num_param_blocks", C.c_int32),
                ("num_row_segments", C.c_int32), ("num_params", C.c_int64), ("num_outputs", C.c_int32),
                ("device", C.c_int32)]


EXPORTS = {
    "pc_compile_layout": (C.c_int, [C.POINTER(pc_circuit_desc), C.c_int, C.POINTER(C.c_void_p)]),
    "pc_destroy": (C.c_int, [C.c_void_p]),
    "pc_set_precision": (C.c_int, [C.c_void_p, C.c_int]),
    "pc_get_precision": (C.c_int, [C.c_void_p, C.POINTER(C.c_int)]),
    "pc_set_split": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int]),
    "pc_set_option": (C.c_int, [C.c_void_p, C.c_int, C.c_int]),
    "pc_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_size_t)]),
    "pc_forward": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                             C.POINTER(pc_lowrank_io), C.c_void_p, C.c_size_t, C.c_void_p]),
    "pc_forward_static": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.POINTER(pc_lowrank_io), C.c_void_p]),
    "pc_backward": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_int, C.POINTER(pc_lowrank_io), C.c_void_p, C.c_size_t,
                              C.c_void_p]),
    "pc_em_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_float, C.c_void_p]),
    "pc_em_step_corrected": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_float,
                                       C.c_void_p]),
    "pc_last_error": (C.c_char_p, []),
    "pc_layout_info": (C.c_int, [C.c_void_p, C.POINTER(pc_layout_summary)]),
    "pc_layer_class": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int)]),
    "pc_set_timing": (C.c_int, [C.c_void_p, C.c_int]),
    "pc_kernel_times": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_double)]),
}

_lib = None


class PCError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[pc error {code}] {msg}")
        self.code = code


def load_library(path: str):
    """A build of the library at `path`, its calls typed (does not make it
    the one the binding uses; see using_library)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m log_space_sum_amd.build`")
    L = C.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def lib():
    """The loaded libpc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


class using_library:
    """Context in which the binding's calls go to another build of the
    library (loaded with load_library; handles compiled meanwhile keep it)."""

    def __init__(self, path: str):
        self.other = load_library(path)

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = self.other
        return self.other

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _check(code):
    if code != PC_OK:
        raise PCError(code, lib().pc_last_error().decode())


def pc_last_error() -> str:
    return lib().pc_last_error().decode()


# ---------------------------------------------------------------------------
# descriptor marshalling
# ---------------------------------------------------------------------------

def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_i32p)


class Handle:
    """Owns a pc_handle (destroyed with the object)."""

    def __init__(self, ptr, circuit):
        self.ptr = ptr
        self.lib = lib()             # the build that made it frees it
        self.num_nodes = circuit.num_nodes
        self.num_params = circuit.num_params
        self.num_vars = circuit.num_vars
        self.root = circuit.root

    def __del__(self):
        if getattr(self, "ptr", None) and getattr(self, "lib", None) is not None:
            self.lib.pc_destroy(self.ptr)
            self.ptr = None


def pc_compile_layout(circuit, device: int = 0) -> Handle:
    """Compile a circuit (an object with num_nodes, num_vars, num_params, root,
    lowrank_rank and a list of layers with the fields of pc_layer_desc /
    pc_sum_group) into a handle; device < 0 compiles host-only."""
    keep = []
    layers = (pc_layer_desc * len(circuit.layers))()
    for i, ly in enumerate(circuit.layers):
        d = layers[i]
        if hasattr(ly, "groups"):
            d.kind = PC_LAYER_SUM
            gs = (pc_sum_group * len(ly.groups))()
            for k, g in enumerate(ly.groups):
                arr, p = _i32(g.ch_block_start)
                keep.append(arr)
                gs[k].out_start = int(g.out_start)
                gs[k].num_nodes = int(g.num_nodes)
                gs[k].num_ch_blocks = int(len(arr))
                gs[k].ch_block_size = int(g.ch_block_size)
                gs[k].ch_block_start = p
                gs[k].param_offset = int(g.param_offset)
                gs[k].lowrank_slot = int(getattr(g, "lowrank", -1))
            keep.append(gs)
            d.num_groups = len(ly.groups)
            d.groups = gs
        elif hasattr(ly, "ch_ptr"):
            d.kind = PC_LAYER_PRODUCT
            d.node_start, d.num_nodes = int(ly.node_start), int(ly.num_nodes)
            a1, d.ch_ptr = _i32(ly.ch_ptr)
            a2, d.ch_ids = _i32(ly.ch_ids)
            keep += [a1, a2]
        elif hasattr(ly, "num_cats"):
            d.kind = PC_LAYER_INPUT_CAT
            d.node_start, d.num_nodes = int(ly.node_start), int(ly.num_nodes)
            d.num_cats, d.num_rows = int(ly.num_cats), int(ly.num_rows)
            d.param_offset = int(ly.param_offset)
            a1, d.var = _i32(ly.var)
            a2, d.row = _i32(ly.row)
            keep += [a1, a2]
        else:
            d.kind = PC_LAYER_INPUT_EXTERNAL
            d.node_start, d.num_nodes = int(ly.node_start), int(ly.num_nodes)
    desc = pc_circuit_desc(num_nodes=int(circuit.num_nodes), num_vars=int(circuit.num_vars),
                           num_params=int(circuit.num_params), num_layers=len(circuit.layers),
                           layers=layers, root=int(circuit.root),
                           lowrank_rank=int(getattr(circuit, "lowrank_rank", 0)),
                           lowrank_form=LOWRANK_FORMS[getattr(circuit, "lowrank_form", "exp_sum")])
    out = C.c_void_p()
    _check(lib().pc_compile_layout(C.byref(desc), int(device), C.byref(out)))
    return Handle(out, circuit)


def pc_destroy(h: Handle):
    if h.ptr:
        _check(lib().pc_destroy(h.ptr))
        h.ptr = None


def pc_set_precision(h: Handle, mode):
    _check(lib().pc_set_precision(h.ptr, MODES.get(mode, mode) if isinstance(mode, str) else int(mode)))


def pc_get_precision(h: Handle) -> int:
    m = C.c_int()
    _check(lib().pc_get_precision(h.ptr, C.byref(m)))
    return m.value


def pc_set_split(h: Handle, mode, gemm_kind, planes_a: int, planes_b: int):
    mode = MODES.get(mode, mode) if isinstance(mode, str) else mode
    gemm_kind = GEMM_KINDS.get(gemm_kind, gemm_kind) if isinstance(gemm_kind, str) else gemm_kind
    _check(lib().pc_set_split(h.ptr, int(mode), int(gemm_kind), int(planes_a), int(planes_b)))


OPTIONS = {"layer_tile": 0, "param_tile": 1, "split_max": 2, "fuse": 3, "param_chunk": 4, "lr_pack": 5,
           "sumexp_fused": 6, "flow_fp8": 7}


def pc_set_option(h: Handle, option, value: int):
    """Kernel tuning: layer_tile (0 auto, 1 128x128, 2 256x128, 3 128x256, 4 128x64, 5 64x128), param_tile
    (0 auto, 1 128x128, 2 256x256, 3 128x256), split_max (1, 2, 4, 8), fuse (1: product
    layers inside the adjacent sum layer's kernels, 0: separate launches),
    param_chunk (-1 automatic; 0: parameter flows in one product at the end;
    n: in chunks of n tied copies on a second stream, overlapping the element
    flows), sumexp_fused (1: LowRank "sum_exp" through the fused kernels),
    flow_fp8 (1: the "sum_exp" parameter flows and denominator statistic from
    e4m3 operands in auto mode)."""
    option = OPTIONS.get(option, option) if isinstance(option, str) else option
    _check(lib().pc_set_option(h.ptr, int(option), int(value)))


def pc_workspace_bytes(h: Handle, batch: int) -> int:
    n = C.c_size_t()
    _check(lib().pc_workspace_bytes(h.ptr, int(batch), C.byref(n)))
    return n.value


def pc_layout_info(h: Handle) -> dict:
    s = pc_layout_summary()
    _check(lib().pc_layout_info(h.ptr, C.byref(s)))
    return {f: getattr(s, f) for f, _ in pc_layout_summary._fields_}


def pc_layer_class(h: Handle, layer: int) -> int:
    c = C.c_int()
    _check(lib().pc_layer_class(h.ptr, int(layer), C.byref(c)))
    return c.value


def pc_set_timing(h: Handle, enable: bool):
    _check(lib().pc_set_timing(h.ptr, 1 if enable else 0))


def pc_kernel_times(h: Handle) -> dict:
    n = (C.c_int64 * PC_NUM_KERNEL_KINDS)()
    ms = (C.c_double * PC_NUM_KERNEL_KINDS)()
    _check(lib().pc_kernel_times(h.ptr, n, ms))
    return {KERNEL_KINDS[k]: (int(n[k]), float(ms[k])) for k in range(PC_NUM_KERNEL_KINDS)}


# ---------------------------------------------------------------------------
# passes (torch tensors: device memory and streams only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, dtype, numel=None, what="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what} has {t.numel()} elements, needs {numel}")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(int(stream))
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _lowrank_io(lowrank, grads=None, z_flows=None, num_params=None):
    """lowrank: list of (A, B) device tensors per slot; grads: list of (dA, dB);
    z_flows: the LowRank denominator statistic's accumulator ([num_params])."""
    if lowrank is None:
        return None, None
    torch = _torch()
    n = len(lowrank)
    A = (C.c_void_p * n)(*[_ptr(a, torch.float32, what="A").value for a, _ in lowrank])
    Bf = (C.c_void_p * n)(*[_ptr(b, torch.float32, what="B").value for _, b in lowrank])
    if grads is not None:
        dA = (C.c_void_p * n)(*[_ptr(a, torch.float32, what="dA").value for a, _ in grads])
        dB = (C.c_void_p * n)(*[_ptr(b, torch.float32, what="dB").value for _, b in grads])
    else:
        dA = dB = None
    z = _ptr(z_flows, torch.float32, num_params, "z_flows") if z_flows is not None else None
    io = pc_lowrank_io(num_slots=n, A=A, B=Bf, dA=dA, dB=dB, z_flows=z)
    return io, (A, Bf, dA, dB)


def pc_forward(h: Handle, batch: int, tokens, params, node_vals, ll=None, lowrank=None, ws=None,
               stream=None):
    torch = _torch()
    io, keep = _lowrank_io(lowrank)
    need = pc_workspace_bytes(h, batch)
    _check(lib().pc_forward(
        h.ptr, int(batch), _ptr(tokens, torch.int32, batch * h.num_vars, "tokens"),
        _ptr(params, torch.float32, h.num_params, "params"),
        _ptr(node_vals, torch.float32, h.num_nodes * batch, "node_vals"),
        _ptr(ll, torch.float32, batch, "ll"), C.byref(io) if io is not None else None,
        _ptr(ws, torch.uint8, need, "ws"), C.c_size_t(ws.numel() if ws is not None else 0),
        _stream(stream)))


def pc_forward_static(h: Handle, batch: int, tokens, params, node_vals, ll=None, lowrank=None, stream=None):
    """pc_forward without a workspace: the library's static device scratch
    (forward only; calls overlapping on one device race)."""
    torch = _torch()
    io, keep = _lowrank_io(lowrank)
    _check(lib().pc_forward_static(
        h.ptr, int(batch), _ptr(tokens, torch.int32, batch * h.num_vars, "tokens"),
        _ptr(params, torch.float32, h.num_params, "params"),
        _ptr(node_vals, torch.float32, h.num_nodes * batch, "node_vals"),
        _ptr(ll, torch.float32, batch, "ll"), C.byref(io) if io is not None else None, _stream(stream)))


def pc_backward(h: Handle, batch: int, tokens, params, node_vals, node_flows, param_flows, flags=0,
                lowrank=None, grads=None, ws=None, stream=None, z_flows=None):
    torch = _torch()
    io, keep = _lowrank_io(lowrank, grads, z_flows, h.num_params)
    need = pc_workspace_bytes(h, batch)
    _check(lib().pc_backward(
        h.ptr, int(batch), _ptr(tokens, torch.int32, batch * h.num_vars, "tokens"),
        _ptr(params, torch.float32, h.num_params, "params"),
        _ptr(node_vals, torch.float32, h.num_nodes * batch, "node_vals"),
        _ptr(node_flows, torch.float32, h.num_nodes * batch, "node_flows"),
        _ptr(param_flows, torch.float32, h.num_params, "param_flows"), int(flags),
        C.byref(io) if io is not None else None,
        _ptr(ws, torch.uint8, need, "ws"), C.c_size_t(ws.numel() if ws is not None else 0),
        _stream(stream)))


def pc_em_step(h: Handle, params, param_flows, step_size=1.0, pseudocount=0.0, stream=None):
    torch = _torch()
    _check(lib().pc_em_step(h.ptr, _ptr(params, torch.float32, h.num_params, "params"),
                            _ptr(param_flows, torch.float32, h.num_params, "param_flows"),
                            C.c_float(step_size), C.c_float(pseudocount), _stream(stream)))


def pc_em_step_corrected(h: Handle, params, param_flows, z_flows, step_size=1.0, pseudocount=0.0, stream=None):
    torch = _torch()
    _check(lib().pc_em_step_corrected(h.ptr, _ptr(params, torch.float32, h.num_params, "params"),
                                      _ptr(param_flows, torch.float32, h.num_params, "param_flows"),
                                      _ptr(z_flows, torch.float32, h.num_params, "z_flows"),
                                      C.c_float(step_size), C.c_float(pseudocount), _stream(stream)))


def workspace(h: Handle, batch: int, device="cuda", all_modes=False):
    """A workspace tensor (uint8) of pc_workspace_bytes(h, batch) bytes; with
    all_modes, the largest over both precision modes (so the handle's mode
    can change while the workspace stays)."""
    n = pc_workspace_bytes(h, batch)
    if all_modes:
        mode = pc_get_precision(h)
        for m in (PC_PREC_AUTO, PC_PREC_FP32):
            pc_set_precision(h, m)
            n = max(n, pc_workspace_bytes(h, batch))
        pc_set_precision(h, mode)
    return _torch().empty(max(n, 1), dtype=_torch().uint8, device=device)


class StepGraph:
    """One pass (forward, backward and, with ``em=(step_size, pseudocount)``,
    the EM update) recorded once as a HIP graph on fixed buffers and replayed
    by ``replay()``: every launch of the pass is one graph node, so a replay
    pays no per-launch host cost.  The graph is recorded again when the
    handle's precision mode changed since (the pass's kernels depend on it);
    after any other pc_set_option, make a new StepGraph.  Recording turns the
    handle's per-kernel timing off (its events cannot be graph nodes).  The
    buffers and the workspace must stay allocated, and are read and written in
    place at every replay (a workspace passed in must be large enough for every
    mode the handle will run in: ``workspace(..., all_modes=True)``); ``zero_param_flows`` clears the parameter flows at
    the start of each pass (a fill kernel, not a memset node)."""

    def __init__(self, h: Handle, batch: int, tokens, params, node_vals, node_flows, param_flows,
                 ll=None, flags=0, lowrank=None, grads=None, ws=None, em=None, zero_param_flows=True):
        self.h, self.batch = h, int(batch)
        self.args = (tokens, params, node_vals, node_flows, param_flows, ll, flags, lowrank, grads)
        self.ws = ws if ws is not None else workspace(h, batch, node_vals.device, all_modes=True)
        self.em = em
        self.zero = zero_param_flows
        self.graph = None
        self.mode = None
        # one eager forward + backward first: anything the library sets up on
        # its first call (a second stream for chunked parameter flows) exists
        # before recording; the EM update is left out so parameters do not move
        pc_set_timing(h, False)
        self._pass(None, with_em=False)
        _torch().cuda.synchronize()
        self._record()

    def _pass(self, stream, with_em=True):
        tokens, params, vals, flows, pflows, ll, flags, lowrank, grads = self.args
        s = stream.cuda_stream if stream is not None else None
        if self.zero:
            pflows.zero_()
        pc_forward(self.h, self.batch, tokens, params, vals, ll, lowrank, self.ws, s)
        pc_backward(self.h, self.batch, tokens, params, vals, flows, pflows, flags, lowrank, grads, self.ws, s)
        if with_em and self.em is not None:
            pc_em_step(self.h, params, pflows, self.em[0], self.em[1], s)

    def _record(self):
        torch = _torch()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self._pass(torch.cuda.current_stream())
        self.graph = g
        self.mode = pc_get_precision(self.h)

    def replay(self):
        if pc_get_precision(self.h) != self.mode:
            self._record()
        self.graph.replay()
