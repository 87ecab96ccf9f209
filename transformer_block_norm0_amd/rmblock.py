"""Thin ctypes binding of librmblock.so (argument marshalling only).

Every step of the block runs in the library's HIP kernels; this module only
turns torch tensors (device memory, streams) into the C ABI's pointers and
sizes.  If the library is missing it raises: there is no fallback path.

The computation is the RankMixerBlock of "Subgraph-fusion-based Mega-kernel
Generation" (page 1, "Exact computation"); shapes follow "Workload and
interfaces" and the envelope "Public checks and instructor coverage".
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librmblock.so")

RM_F32, RM_BF16, RM_F16 = 0, 1, 2
RM_WS_H1, RM_WS_Z, RM_WS_HID, RM_WS_R2, RM_WS_STATS = range(5)
STAT_NAMES = ("mu0", "rs0", "mu1", "rs1", "mux", "rsx", "mug", "rsg", "mu2", "rs2")

PARAM_NAMES = ("w1", "b1", "wout", "bout", "lnx_g", "lnx_b", "lng_g", "lng_b",
               "ln0_g", "ln0_b", "ln1_g", "ln1_b", "ln2_g", "ln2_b")

STATUS = {0: "RM_OK", 1: "RM_E_DIMS", 2: "RM_E_NULL", 3: "RM_E_ALIGN", 4: "RM_E_WORKSPACE",
          5: "RM_E_DTYPE", 6: "RM_E_HIP", 7: "RM_E_ARG", 8: "RM_E_SCRATCH"}
RM_STATIC_SCRATCH_BYTES = 256 << 20


class RmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib().rm_status_string(status).decode()})")


RM_FLAG_MAIN_KERNELS = 1
KERNEL_SETS = {"auto": 0, "main": RM_FLAG_MAIN_KERNELS}


class CDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class CParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PARAM_NAMES]


class CGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PARAM_NAMES]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m transformer_block_norm0_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        lib.rm_workspace_bytes.argtypes = [P(CDims)]
        lib.rm_workspace_bytes.restype = ctypes.c_size_t
        lib.rm_block_fwd.argtypes = [P(CDims), P(CParams), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.rm_block_fwd.restype = ctypes.c_int
        lib.rm_block_bwd.argtypes = [P(CDims), P(CParams), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, P(CGrads),
                                     ctypes.c_void_p]
        lib.rm_block_bwd.restype = ctypes.c_int
        lib.rm_block_bwd_static.argtypes = lib.rm_block_bwd.argtypes
        lib.rm_block_bwd_static.restype = ctypes.c_int
        lib.rm_token_mix.argtypes = [P(CDims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.rm_token_mix.restype = ctypes.c_int
        lib.rm_ws_region.argtypes = [P(CDims), ctypes.c_int, P(ctypes.c_size_t), P(ctypes.c_size_t)]
        lib.rm_ws_region.restype = ctypes.c_int
        lib.rm_status_string.argtypes = [ctypes.c_int]
        lib.rm_status_string.restype = ctypes.c_char_p
        lib.rm_abi_version.restype = ctypes.c_int
        lib.rm_prof_enable.argtypes = [ctypes.c_int]
        lib.rm_prof_enable.restype = ctypes.c_int
        lib.rm_prof_kernels.restype = ctypes.c_int
        lib.rm_prof_name.argtypes = [ctypes.c_int]
        lib.rm_prof_name.restype = ctypes.c_char_p
        lib.rm_prof_collect.argtypes = [P(ctypes.c_double), P(ctypes.c_int64), ctypes.c_int]
        lib.rm_prof_collect.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it has not been built)."""
    return _lib()


def dims(B: int, T: int, D: int, k: int, dtype: str, kernels: str = "auto") -> CDims:
    """rm_dims of a call.  kernels="auto" lets B <= 8, D <= 128, H <= 256 shapes take the
    small-batch kernels; "main" sends the call through the main kernel set."""
    return CDims(B, T, D, k, {"f32": RM_F32, "bf16": RM_BF16, "f16": RM_F16}[dtype], KERNEL_SETS[kernels])


def workspace_bytes(d: CDims) -> int:
    return int(_lib().rm_workspace_bytes(ctypes.byref(d)))


def ws_region(d: CDims, region: int) -> tuple[int, int]:
    off, nbytes = ctypes.c_size_t(), ctypes.c_size_t()
    st = _lib().rm_ws_region(ctypes.byref(d), region, ctypes.byref(off), ctypes.byref(nbytes))
    if st:
        raise RmError(st, "rm_ws_region")
    return off.value, nbytes.value


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _torch_dtype(d: CDims):
    import torch
    return {RM_BF16: torch.bfloat16, RM_F16: torch.float16}.get(d.dtype, torch.float32)


def _check(t, d: CDims, shape, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != _torch_dtype(d):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {_torch_dtype(d)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def param_shapes(d: CDims) -> dict:
    T, D, H = d.T, d.D, d.k * d.D
    return {"w1": (T, D, 2 * H), "b1": (T, 2 * H), "wout": (T, H, D), "bout": (T, D),
            "lnx_g": (H,), "lnx_b": (H,), "lng_g": (H,), "lng_b": (H,),
            "ln0_g": (D,), "ln0_b": (D,), "ln1_g": (D,), "ln1_b": (D,), "ln2_g": (D,), "ln2_b": (D,)}


def _cparams(d: CDims, params: dict, cls, check=True):
    shapes = param_shapes(d)
    vals = {}
    for n in PARAM_NAMES:
        t = params.get(n)
        if check:
            _check(t, d, shapes[n], n)
        vals[n] = _ptr(t)
    return cls(**vals)


def block_fwd(d: CDims, params: dict, x, y, ws, ws_bytes: int | None = None, stream=None, check=True):
    """rm_block_fwd: y = RankMixerBlock(x); saves what the backward needs in ws."""
    if check:
        _check(x, d, (d.B, d.T, d.D), "x")
        _check(y, d, (d.B, d.T, d.D), "y")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cp = _cparams(d, params, CParams, check)
    st = _lib().rm_block_fwd(ctypes.byref(d), ctypes.byref(cp), _ptr(x), _ptr(y), _ptr(ws), ws_bytes,
                             _stream(stream))
    if st:
        raise RmError(st, "rm_block_fwd")


def block_bwd(d: CDims, params: dict, x, dy, ws, dx, grads: dict, ws_bytes: int | None = None, stream=None,
              check=True):
    """rm_block_bwd: dx and every parameter gradient (overwritten) for upstream dy."""
    if check:
        for t, n in ((x, "x"), (dy, "dy"), (dx, "dx")):
            _check(t, d, (d.B, d.T, d.D), n)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cp = _cparams(d, params, CParams, check)
    cg = _cparams(d, grads, CGrads, check)
    st = _lib().rm_block_bwd(ctypes.byref(d), ctypes.byref(cp), _ptr(x), _ptr(dy), _ptr(ws), ws_bytes,
                             _ptr(dx), ctypes.byref(cg), _stream(stream))
    if st:
        raise RmError(st, "rm_block_bwd")


def block_bwd_static(d: CDims, params: dict, x, dy, ws, dx, grads: dict, ws_bytes: int | None = None, stream=None,
                     check=True):
    """rm_block_bwd_static: rm_block_bwd with the backward's scratch in the library's static
    per-GPU buffer (allocates nothing); ws needs only the forward's saved regions."""
    if check:
        for t, n in ((x, "x"), (dy, "dy"), (dx, "dx")):
            _check(t, d, (d.B, d.T, d.D), n)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    cp = _cparams(d, params, CParams, check)
    cg = _cparams(d, grads, CGrads, check)
    st = _lib().rm_block_bwd_static(ctypes.byref(d), ctypes.byref(cp), _ptr(x), _ptr(dy), _ptr(ws), ws_bytes,
                                    _ptr(dx), ctypes.byref(cg), _stream(stream))
    if st:
        raise RmError(st, "rm_block_bwd_static")


def token_mix(d: CDims, inp, out, stream=None):
    """rm_token_mix: out[b,i,j*S+s] = inp[b,j,i*S+s] (bit-exact permutation)."""
    _check(inp, d, (d.B, d.T, d.D), "in")
    _check(out, d, (d.B, d.T, d.D), "out")
    st = _lib().rm_token_mix(ctypes.byref(d), _ptr(inp), _ptr(out), _stream(stream))
    if st:
        raise RmError(st, "rm_token_mix")


def alloc_workspace(d: CDims, device="cuda"):
    import torch
    n = workspace_bytes(d)
    if n == 0:
        raise ValueError("invalid dims")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prof_enable(on: bool):
    _lib().rm_prof_enable(1 if on else 0)


def prof_collect() -> dict:
    """{kernel name: (total ms, launches)} of the launches recorded since the last collect."""
    lib = _lib()
    n = lib.rm_prof_kernels()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = lib.rm_prof_collect(ms, cnt, n)
    if st:
        raise RmError(st, "rm_prof_collect")
    return {lib.rm_prof_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}


def kernel_names() -> list[str]:
    lib = _lib()
    return [lib.rm_prof_name(i).decode() for i in range(lib.rm_prof_kernels())]
