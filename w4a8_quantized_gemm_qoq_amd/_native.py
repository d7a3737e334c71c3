"""ctypes binding of libqoq.so (argument marshalling only).

Every step of the W4A8 path runs inside the library: the host packer for the
offline weight encode, the HIP kernels for activation quantization and the
GEMM.  This module only turns NumPy arrays / torch tensors into pointers and
sizes, passes torch's current HIP stream, and maps error codes to Python
exceptions.  It never computes a result itself and has no fallback: if the
library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqoq.so")

EXPORTS = [
    "qoq_status_string",
    "qoq_last_error",
    "qoq_weight_layout_query",
    "qoq_pack_weights",
    "qoq_pack_codes",
    "qoq_unpack_weights",
    "qoq_quant_act_per_token",
    "qoq_rmsnorm_quant_per_token",
    "qoq_swiglu_quant_per_token",
    "qoq_w4a8_gemm_workspace_size",
    "qoq_w4a8_gemm",
    "qoq_w4a8_gemm_i32",
    "qoq_w4a8_gemm_noalloc",
    "qoq_w4a8_gemm_plan",
    "qoq_pack_weights_w8",
    "qoq_w8a8_gemm_workspace_size",
    "qoq_w8a8_gemm",
    "qoq_w8a8_gemm_i32",
    "qoq_w4a8_gemm_saturating",
    "qoq_w4a8_gemm_saturating_i32",
    "qoq_kv4_quant",
    "qoq_kv4_decode_attention",
    "qoq_kv4_decode_attention_workspace_size",
    "qoq_kv4_decode_attention_split",
    "qoq_kv4_decode_attention_plan",
    "qoq_hadamard_rotate",
    "qoq_smoothing_factors",
    "qoq_scale_columns",
]

GROUP = 128


class QoQError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status}: {detail}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [
        ("layout_id", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("N_pad", ctypes.c_int64),
        ("n_groups", ctypes.c_int64),
        ("qweight_bytes", ctypes.c_size_t),
        ("meta_bytes", ctypes.c_size_t),
        ("scale_bytes", ctypes.c_size_t),
    ]


_lib = None


def load_library():
    """Load libqoq.so (after torch, so that torch's HIP runtime is the one in use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m w4a8_quantized_gemm_qoq_amd.build` "
            "(there is no fallback implementation)")
    from .build import HASH_FILE, source_hash
    try:
        with open(HASH_FILE) as f:
            built_from = f.read().strip()
    except OSError:
        built_from = None
    if built_from != source_hash():
        raise RuntimeError(
            f"{LIB_PATH} was not built from the sources in this tree (its record {HASH_FILE} is "
            f"{'missing' if built_from is None else 'different'}); rebuild with "
            "`python -m w4a8_quantized_gemm_qoq_amd.build`")
    try:
        import torch  # noqa: F401  -- loads torch's libamdhip64 first
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "qoq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qoq_last_error": (ctypes.c_char_p, []),
        "qoq_weight_layout_query": (ctypes.c_int, [i64, i64, i32, ctypes.POINTER(_Layout)]),
        "qoq_pack_weights": (ctypes.c_int, [vp, i64, i64, i32, vp, vp, vp]),
        "qoq_pack_codes": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i32, vp, vp, vp]),
        "qoq_unpack_weights": (ctypes.c_int, [vp, vp, vp, i64, i64, i32, vp, vp, vp, vp]),
        "qoq_quant_act_per_token": (ctypes.c_int, [vp, i64, i64, i64, vp, vp, vp]),
        "qoq_rmsnorm_quant_per_token": (ctypes.c_int, [vp, vp, ctypes.c_float, i64, i64, i64, vp, vp, vp]),
        "qoq_swiglu_quant_per_token": (ctypes.c_int, [vp, vp, i64, i64, i64, i64, vp, vp, vp, i64, vp]),
        "qoq_w4a8_gemm_workspace_size": (sz, [i64, i64, i64, i32]),
        "qoq_w4a8_gemm": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp]),
        "qoq_w4a8_gemm_i32": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp]),
        "qoq_w4a8_gemm_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]),
        "qoq_w4a8_gemm_plan": (ctypes.c_int, [i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
        "qoq_pack_weights_w8": (ctypes.c_int, [vp, i64, i64, vp, vp]),
        "qoq_w8a8_gemm_workspace_size": (sz, [i64, i64, i64]),
        "qoq_w8a8_gemm": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]),
        "qoq_w8a8_gemm_i32": (ctypes.c_int, [vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]),
        "qoq_w4a8_gemm_saturating": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]),
        "qoq_w4a8_gemm_saturating_i32": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]),
        "qoq_kv4_quant": (ctypes.c_int, [vp, i64, i32, i64, vp, vp, vp, vp]),
        "qoq_kv4_decode_attention": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                    ctypes.c_float, vp, vp]),
        "qoq_kv4_decode_attention_workspace_size": (sz, [i32, i32, i32, i32]),
        "qoq_kv4_decode_attention_split": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                          ctypes.c_float, vp, vp, sz, vp]),
        "qoq_kv4_decode_attention_plan": (ctypes.c_int, [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32),
                                                          ctypes.POINTER(ctypes.c_int32)]),
        "qoq_hadamard_rotate": (ctypes.c_int, [vp, i64, i64, i64, vp]),
        "qoq_smoothing_factors": (ctypes.c_int, [vp, vp, i64, ctypes.c_float, vp]),
        "qoq_scale_columns": (ctypes.c_int, [vp, i64, i64, i64, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int, fn: str):
    if status != 0:
        lib = load_library()
        raise QoQError(status, fn, lib.qoq_last_error().decode() or lib.qoq_status_string(status).decode())


def _np_ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "host arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _t_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- host side

def qoq_weight_layout_query(N: int, K: int, group_size: int = GROUP) -> dict:
    lib = load_library()
    L = _Layout()
    _check(lib.qoq_weight_layout_query(N, K, group_size, ctypes.byref(L)), "qoq_weight_layout_query")
    return {f: getattr(L, f) for f, _ in _Layout._fields_}


@dataclass
class PackedWeight:
    """Packed W4 weights (host NumPy arrays or device torch tensors)."""
    qweight: object
    meta: object
    scale: object  # FP16 bit patterns (uint16) on the host, torch.float16 on the device
    N: int
    K: int
    group_size: int

    def to(self, device="cuda") -> "PackedWeight":
        import torch
        def dev(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.view(dtype)
            return t.to(device)
        return PackedWeight(dev(self.qweight), dev(self.meta), dev(self.scale, torch.float16),
                            self.N, self.K, self.group_size)


def _alloc_packed(N, K, group_size):
    L = qoq_weight_layout_query(N, K, group_size)
    return (L, np.empty(L["qweight_bytes"], np.uint8), np.empty(L["meta_bytes"], np.uint8),
            np.empty(L["N_pad"], np.uint16))


def qoq_pack_weights(W: np.ndarray, group_size: int = GROUP) -> PackedWeight:
    """Offline progressive (g128) or per-channel W4 encode + pack, on the host."""
    W = np.ascontiguousarray(W, dtype=np.float16)
    N, K = W.shape
    lib = load_library()
    _, qw, meta, scale = _alloc_packed(N, K, group_size)
    _check(lib.qoq_pack_weights(_np_ptr(W.view(np.uint16)), N, K, group_size, _np_ptr(qw), _np_ptr(meta),
                                _np_ptr(scale)), "qoq_pack_weights")
    return PackedWeight(qw, meta, scale, N, K, group_size)


def qoq_pack_codes(q4, s1, z, scale, group_size: int = GROUP) -> PackedWeight:
    q4 = np.ascontiguousarray(q4, dtype=np.uint8)
    N, K = q4.shape
    z = np.ascontiguousarray(z, dtype=np.uint8)
    s1 = None if s1 is None else np.ascontiguousarray(s1, dtype=np.uint8)
    scale = np.ascontiguousarray(np.asarray(scale, dtype=np.float16).view(np.uint16))
    lib = load_library()
    _, qw, meta, sc = _alloc_packed(N, K, group_size)
    _check(lib.qoq_pack_codes(_np_ptr(q4), _np_ptr(s1), _np_ptr(z), _np_ptr(scale), N, K, group_size, _np_ptr(qw),
                              _np_ptr(meta), _np_ptr(sc)), "qoq_pack_codes")
    return PackedWeight(qw, meta, sc, N, K, group_size)


def qoq_unpack_weights(p: PackedWeight):
    """(q4 [N,K], s1 [N,G] or None, z [N,G] or [N], scale fp16 [N]) from host-packed buffers."""
    lib = load_library()
    N, K, gs = p.N, p.K, p.group_size
    G = K // GROUP
    q4 = np.empty((N, K), np.uint8)
    s1 = np.empty((N, G), np.uint8) if gs else None
    z = np.empty((N, G), np.uint8) if gs else np.empty(N, np.uint8)
    sc = np.empty(N, np.uint16)
    scale_in = np.ascontiguousarray(np.asarray(p.scale).view(np.uint16))
    _check(lib.qoq_unpack_weights(_np_ptr(p.qweight), _np_ptr(p.meta), _np_ptr(scale_in), N, K, gs, _np_ptr(q4),
                                  _np_ptr(s1), _np_ptr(z), _np_ptr(sc)), "qoq_unpack_weights")
    return q4, s1, z, sc.view(np.float16)


# ---------------------------------------------------------------- device side

def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("device entry points take GPU tensors")


def qoq_quant_act_per_token(x, x8=None, sx=None, stream=None):
    """Per-token INT8 quantization of FP16 x [M, K] (row stride may exceed K) on the GPU."""
    import torch
    _require_cuda(x)
    if x.dtype != torch.float16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D FP16 tensor with unit column stride")
    M, K = x.shape
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float16, device=x.device)
    _require_cuda(x8, sx)
    if not (x8.is_contiguous() and x8.shape == (M, K) and x8.dtype == torch.int8):
        raise ValueError("x8 must be a contiguous int8 [M, K] tensor")
    if not (sx.is_contiguous() and sx.numel() == M and sx.dtype == torch.float16):
        raise ValueError("sx must be a contiguous float16 [M] tensor")
    lib = load_library()
    _check(lib.qoq_quant_act_per_token(_t_ptr(x), M, K, x.stride(0), _t_ptr(x8), _t_ptr(sx), _stream(stream)),
           "qoq_quant_act_per_token")
    return x8, sx


def qoq_rmsnorm_quant_per_token(x, gamma, eps: float, x8=None, sx=None, stream=None):
    """Fused RMS normalization + per-token INT8 quantization of FP16 x [M, K] on the GPU."""
    import torch
    _require_cuda(x, gamma)
    if x.dtype != torch.float16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D FP16 tensor with unit column stride")
    M, K = x.shape
    if gamma.dtype != torch.float16 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float16 [K] tensor")
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float16, device=x.device)
    _require_cuda(x8, sx)
    if not (x8.is_contiguous() and x8.shape == (M, K) and x8.dtype == torch.int8):
        raise ValueError("x8 must be a contiguous int8 [M, K] tensor")
    if not (sx.is_contiguous() and sx.numel() == M and sx.dtype == torch.float16):
        raise ValueError("sx must be a contiguous float16 [M] tensor")
    lib = load_library()
    _check(lib.qoq_rmsnorm_quant_per_token(_t_ptr(x), _t_ptr(gamma), float(eps), M, K, x.stride(0), _t_ptr(x8),
                                           _t_ptr(sx), _stream(stream)), "qoq_rmsnorm_quant_per_token")
    return x8, sx


def qoq_swiglu_quant_per_token(gate, up, x8=None, sx=None, h=None, want_h=False, stream=None):
    """Fused SiLU(gate) * up + per-token INT8 quantization on the GPU.

    gate and up: FP16 [M, K] with unit column stride (row strides may exceed
    K, e.g. the two halves of one [M, 2K] gate-up output).  Returns (x8, sx),
    or (x8, sx, h) with the FP16 activations when want_h or h is given."""
    import torch
    _require_cuda(gate, up)
    for name, t in (("gate", gate), ("up", up)):
        if t.dtype != torch.float16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D FP16 tensor with unit column stride")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    M, K = gate.shape
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.int8, device=gate.device)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float16, device=gate.device)
    if h is None and want_h:
        h = torch.empty((M, K), dtype=torch.float16, device=gate.device)
    _require_cuda(x8, sx, h)
    if not (x8.is_contiguous() and x8.shape == (M, K) and x8.dtype == torch.int8):
        raise ValueError("x8 must be a contiguous int8 [M, K] tensor")
    if not (sx.is_contiguous() and sx.numel() == M and sx.dtype == torch.float16):
        raise ValueError("sx must be a contiguous float16 [M] tensor")
    if h is not None and not (h.dtype == torch.float16 and h.shape == (M, K) and h.stride(1) == 1):
        raise ValueError("h must be a float16 [M, K] tensor with unit column stride")
    lib = load_library()
    _check(lib.qoq_swiglu_quant_per_token(_t_ptr(gate), _t_ptr(up), M, K, gate.stride(0), up.stride(0), _t_ptr(x8),
                                          _t_ptr(sx), _t_ptr(h),
                                          h.stride(0) if h is not None else 0, _stream(stream)),
           "qoq_swiglu_quant_per_token")
    return (x8, sx, h) if h is not None else (x8, sx)


def _check_gemm_inputs(x8, w: PackedWeight):
    import torch
    _require_cuda(x8, w.qweight, w.meta, w.scale)
    if x8.dtype != torch.int8 or x8.dim() != 2 or not x8.is_contiguous():
        raise ValueError("x8 must be a contiguous int8 [M, K] tensor")
    if x8.shape[1] != w.K:
        raise ValueError(f"x8 has K={x8.shape[1]}, weights have K={w.K}")


def qoq_w4a8_gemm(x8, sx, w: PackedWeight, y=None, workspace=None, stream=None):
    """y = fp16(x8 @ w8^T * s_x * scale) on the GPU; returns y [M, N] FP16."""
    import torch
    _check_gemm_inputs(x8, w)
    M = x8.shape[0]
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float16, device=x8.device)
    _require_cuda(sx, y)
    if y.dtype != torch.float16 or y.shape != (M, w.N) or y.stride(1) != 1:
        raise ValueError("y must be float16 [M, N] with unit column stride")
    if sx.dtype != torch.float16 or sx.numel() != M or not sx.is_contiguous():
        raise ValueError("sx must be contiguous float16 [M]")
    lib = load_library()
    ws_bytes = lib.qoq_w4a8_gemm_workspace_size(M, w.N, w.K, w.group_size)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x8.device)
    _check(lib.qoq_w4a8_gemm(_t_ptr(x8), _t_ptr(sx), _t_ptr(w.qweight), _t_ptr(w.meta), _t_ptr(w.scale), _t_ptr(y),
                             M, w.N, w.K, y.stride(0), w.group_size, _t_ptr(workspace) if ws_bytes else None,
                             ws_bytes, _stream(stream)), "qoq_w4a8_gemm")
    return y


GEMM_KERNELS = {0: "strip", 1: "skinny16", 2: "skinny32", 3: "skinny64", 4: "large", 5: "ring"}


def qoq_w4a8_gemm_plan(M: int, N: int, K: int, group_size: int = GROUP) -> tuple[str, int, int]:
    """(kernel family, strips per block or large-M tile, K parts or splits) of a GEMM call."""
    k, t, s = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    lib = load_library()
    _check(lib.qoq_w4a8_gemm_plan(M, N, K, group_size, ctypes.byref(k), ctypes.byref(t), ctypes.byref(s)),
           "qoq_w4a8_gemm_plan")
    return GEMM_KERNELS[k.value], int(t.value), int(s.value)


NOALLOC_SCRATCH_BYTES = 32 << 20   # QOQ_NOALLOC_SCRATCH_BYTES in qoq.h


def qoq_w4a8_gemm_noalloc(x8, sx, w: PackedWeight, y, stream=None):
    """qoq_w4a8_gemm without a workspace: the library's own per-GPU scratch
    holds any split-K partials (no device allocation in the call).  y is the
    caller's float16 [M, N] output."""
    import torch
    _check_gemm_inputs(x8, w)
    M = x8.shape[0]
    _require_cuda(sx, y)
    if y.dtype != torch.float16 or y.shape != (M, w.N) or y.stride(1) != 1:
        raise ValueError("y must be float16 [M, N] with unit column stride")
    if sx.dtype != torch.float16 or sx.numel() != M or not sx.is_contiguous():
        raise ValueError("sx must be contiguous float16 [M]")
    lib = load_library()
    _check(lib.qoq_w4a8_gemm_noalloc(_t_ptr(x8), _t_ptr(sx), _t_ptr(w.qweight), _t_ptr(w.meta), _t_ptr(w.scale),
                                     _t_ptr(y), M, w.N, w.K, y.stride(0), w.group_size, _stream(stream)),
           "qoq_w4a8_gemm_noalloc")
    return y


def qoq_w4a8_gemm_i32(x8, w: PackedWeight, acc=None, workspace=None, stream=None):
    """Exact INT32 accumulators acc = x8 @ w8^T on the GPU (debug entry point)."""
    import torch
    _check_gemm_inputs(x8, w)
    M = x8.shape[0]
    if acc is None:
        acc = torch.empty((M, w.N), dtype=torch.int32, device=x8.device)
    _require_cuda(acc)
    if acc.dtype != torch.int32 or acc.shape != (M, w.N) or acc.stride(1) != 1:
        raise ValueError("acc must be int32 [M, N] with unit column stride")
    lib = load_library()
    ws_bytes = lib.qoq_w4a8_gemm_workspace_size(M, w.N, w.K, w.group_size)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x8.device)
    _check(lib.qoq_w4a8_gemm_i32(_t_ptr(x8), _t_ptr(w.qweight), _t_ptr(w.meta), _t_ptr(acc), M, w.N, w.K,
                                 acc.stride(0), w.group_size, _t_ptr(workspace) if ws_bytes else None, ws_bytes,
                                 _stream(stream)), "qoq_w4a8_gemm_i32")
    return acc


def qoq_w4a8_forward(x, w: PackedWeight, stream=None):
    """One pass of the online path: per-token quantization then the W4A8 GEMM."""
    x8, sx = qoq_quant_act_per_token(x, stream=stream)
    return qoq_w4a8_gemm(x8, sx, w, stream=stream)


# ------------------------------------------------- comparators (same kernels)

@dataclass
class PackedWeightW8:
    """Per-channel INT8 weights of the W8A8 comparator (host or device)."""
    qweight: object
    scale: object
    N: int
    K: int

    def to(self, device="cuda") -> "PackedWeightW8":
        import torch
        qw = torch.from_numpy(np.ascontiguousarray(self.qweight)).to(device)
        sc = torch.from_numpy(np.ascontiguousarray(self.scale)).view(torch.float16).to(device)
        return PackedWeightW8(qw, sc, self.N, self.K)


def qoq_pack_weights_w8(W: np.ndarray) -> PackedWeightW8:
    """Per-channel symmetric INT8 encode + pack of W [N, K] on the host."""
    W = np.ascontiguousarray(W, dtype=np.float16)
    N, K = W.shape
    N_pad = (N + 15) // 16 * 16
    qw = np.empty(N_pad * K, np.uint8)
    scale = np.empty(N_pad, np.uint16)
    lib = load_library()
    _check(lib.qoq_pack_weights_w8(_np_ptr(W.view(np.uint16)), N, K, _np_ptr(qw), _np_ptr(scale)),
           "qoq_pack_weights_w8")
    return PackedWeightW8(qw, scale, N, K)


def _workspace(ws_bytes, workspace, device):
    import torch
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    return _t_ptr(workspace) if ws_bytes else None


def _out(x8, N, out, dtype):
    import torch
    M = x8.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=x8.device)
    _require_cuda(out)
    if out.dtype != dtype or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError(f"output must be {dtype} [M, N] with unit column stride")
    return out


def _check_x8(x8, K):
    import torch
    _require_cuda(x8)
    if x8.dtype != torch.int8 or x8.dim() != 2 or not x8.is_contiguous():
        raise ValueError("x8 must be a contiguous int8 [M, K] tensor")
    if x8.shape[1] != K:
        raise ValueError(f"x8 has K={x8.shape[1]}, weights have K={K}")


def _check_sx(sx, M):
    import torch
    _require_cuda(sx)
    if sx.dtype != torch.float16 or sx.numel() != M or not sx.is_contiguous():
        raise ValueError("sx must be contiguous float16 [M]")


def qoq_w8a8_gemm(x8, sx, w: PackedWeightW8, y=None, workspace=None, stream=None):
    """W8A8 comparator: y = fp16(x8 @ w8^T * s_x * s_w) on the GPU."""
    import torch
    _check_x8(x8, w.K)
    _require_cuda(w.qweight, w.scale)
    M = x8.shape[0]
    _check_sx(sx, M)
    y = _out(x8, w.N, y, torch.float16)
    lib = load_library()
    ws = lib.qoq_w8a8_gemm_workspace_size(M, w.N, w.K)
    _check(lib.qoq_w8a8_gemm(_t_ptr(x8), _t_ptr(sx), _t_ptr(w.qweight), _t_ptr(w.scale), _t_ptr(y), M, w.N, w.K,
                             y.stride(0), _workspace(ws, workspace, x8.device), ws, _stream(stream)), "qoq_w8a8_gemm")
    return y


def qoq_w8a8_gemm_i32(x8, w: PackedWeightW8, acc=None, workspace=None, stream=None):
    """W8A8 comparator, exact INT32 accumulators."""
    import torch
    _check_x8(x8, w.K)
    _require_cuda(w.qweight)
    M = x8.shape[0]
    acc = _out(x8, w.N, acc, torch.int32)
    lib = load_library()
    ws = lib.qoq_w8a8_gemm_workspace_size(M, w.N, w.K)
    _check(lib.qoq_w8a8_gemm_i32(_t_ptr(x8), _t_ptr(w.qweight), _t_ptr(acc), M, w.N, w.K, acc.stride(0),
                                 _workspace(ws, workspace, x8.device), ws, _stream(stream)), "qoq_w8a8_gemm_i32")
    return acc


def _check_g128(w: PackedWeight):
    if w.group_size != GROUP:
        raise ValueError("the saturating ablation takes g128 weights")
    _require_cuda(w.qweight, w.meta)


def qoq_w4a8_gemm_saturating(x8, sx, w: PackedWeight, y=None, workspace=None, stream=None):
    """Saturating-dequantization ablation of the g128 W4A8 GEMM."""
    import torch
    _check_g128(w)
    _check_x8(x8, w.K)
    _require_cuda(w.scale)
    M = x8.shape[0]
    _check_sx(sx, M)
    y = _out(x8, w.N, y, torch.float16)
    lib = load_library()
    ws = lib.qoq_w4a8_gemm_workspace_size(M, w.N, w.K, GROUP)
    _check(lib.qoq_w4a8_gemm_saturating(_t_ptr(x8), _t_ptr(sx), _t_ptr(w.qweight), _t_ptr(w.meta), _t_ptr(w.scale),
                                        _t_ptr(y), M, w.N, w.K, y.stride(0), _workspace(ws, workspace, x8.device), ws,
                                        _stream(stream)), "qoq_w4a8_gemm_saturating")
    return y


def qoq_w4a8_gemm_saturating_i32(x8, w: PackedWeight, acc=None, workspace=None, stream=None):
    """Saturating ablation, exact INT32 accumulators."""
    import torch
    _check_g128(w)
    _check_x8(x8, w.K)
    M = x8.shape[0]
    acc = _out(x8, w.N, acc, torch.int32)
    lib = load_library()
    ws = lib.qoq_w4a8_gemm_workspace_size(M, w.N, w.K, GROUP)
    _check(lib.qoq_w4a8_gemm_saturating_i32(_t_ptr(x8), _t_ptr(w.qweight), _t_ptr(w.meta), _t_ptr(acc), M, w.N, w.K,
                                            acc.stride(0), _workspace(ws, workspace, x8.device), ws,
                                            _stream(stream)), "qoq_w4a8_gemm_saturating_i32")
    return acc


# ------------------------------------------------------------------------ KV4

HEAD_DIM = 128


def qoq_kv4_quant(x, codes=None, scale=None, zero=None, stream=None):
    """Per-head asymmetric INT4 quantization of FP16 rows x [..., 128] on the GPU.

    Returns (codes uint8 [..., 64], scale float16 [...], zero uint8 [...]).
    """
    import torch
    _require_cuda(x)
    if x.dtype != torch.float16 or x.shape[-1] != HEAD_DIM or not x.is_contiguous():
        raise ValueError("x must be a contiguous float16 tensor with a last axis of 128")
    lead = tuple(x.shape[:-1])
    n = int(np.prod(lead)) if lead else 1
    codes = torch.empty(lead + (HEAD_DIM // 2,), dtype=torch.uint8, device=x.device) if codes is None else codes
    scale = torch.empty(lead, dtype=torch.float16, device=x.device) if scale is None else scale
    zero = torch.empty(lead, dtype=torch.uint8, device=x.device) if zero is None else zero
    _require_cuda(codes, scale, zero)
    if codes.numel() != n * HEAD_DIM // 2 or scale.numel() != n or zero.numel() != n:
        raise ValueError("output sizes do not match x")
    lib = load_library()
    _check(lib.qoq_kv4_quant(_t_ptr(x), n, HEAD_DIM, HEAD_DIM, _t_ptr(codes), _t_ptr(scale), _t_ptr(zero),
                             _stream(stream)), "qoq_kv4_quant")
    return codes, scale, zero


def qoq_kv4_decode_attention_workspace_size(B: int, H: int, Hkv: int, T: int) -> int:
    """Bytes of workspace the token-split attention needs (0: that shape is not split)."""
    return int(load_library().qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T))


def qoq_kv4_decode_attention_plan(B: int, H: int, Hkv: int, T: int, split: bool = False) -> tuple[int, int]:
    """(query heads per workgroup, token chunks) the attention launches for this shape."""
    r, nc = ctypes.c_int32(0), ctypes.c_int32(0)
    lib = load_library()
    _check(lib.qoq_kv4_decode_attention_plan(B, H, Hkv, T, int(split), ctypes.byref(r), ctypes.byref(nc)),
           "qoq_kv4_decode_attention_plan")
    return int(r.value), int(nc.value)


def qoq_kv4_decode_attention(q, k, v, lengths, softmax_scale, o=None, stream=None, split=False, workspace=None):
    """Decode attention of q [B, H, 128] FP16 over KV4 caches k, v = (codes
    [B, Hkv, T, 64], scale [B, Hkv, T], zero [B, Hkv, T]); lengths int32 [B].

    split=True calls the token-split entry (chunks of the cache over more
    workgroups, for small batches); its workspace is allocated here unless a
    uint8 device tensor of at least the queried size is given.
    """
    import torch
    kc, ks, kz = k
    vc, vs, vz = v
    _require_cuda(q, kc, ks, kz, vc, vs, vz, lengths)
    if q.dtype != torch.float16 or q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16 [B, H, 128] tensor")
    B, H, _ = q.shape
    if kc.dim() != 4 or kc.shape[0] != B or kc.shape[3] != HEAD_DIM // 2:
        raise ValueError("k codes must be uint8 [B, Hkv, T, 64]")
    Hkv, T = kc.shape[1], kc.shape[2]
    for t, shape in ((kc, (B, Hkv, T, 64)), (vc, (B, Hkv, T, 64)), (ks, (B, Hkv, T)), (vs, (B, Hkv, T)),
                     (kz, (B, Hkv, T)), (vz, (B, Hkv, T))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("KV cache arrays must be contiguous with matching [B, Hkv, T] shapes")
    if lengths.dtype != torch.int32 or lengths.numel() != B:
        raise ValueError("lengths must be int32 [B]")
    o = torch.empty((B, H, HEAD_DIM), dtype=torch.float16, device=q.device) if o is None else o
    lib = load_library()
    args = (_t_ptr(q), _t_ptr(kc), _t_ptr(ks), _t_ptr(kz), _t_ptr(vc), _t_ptr(vs), _t_ptr(vz), _t_ptr(lengths),
            B, H, Hkv, T, HEAD_DIM, float(softmax_scale), _t_ptr(o))
    if not split:
        _check(lib.qoq_kv4_decode_attention(*args, _stream(stream)), "qoq_kv4_decode_attention")
        return o
    if workspace is None:
        need = int(lib.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _require_cuda(workspace)
    _check(lib.qoq_kv4_decode_attention_split(*args, _t_ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)), "qoq_kv4_decode_attention_split")
    return o


# --------------------------------------------------------- offline transforms

def qoq_hadamard_rotate(X: np.ndarray) -> np.ndarray:
    """X @ H (block Walsh-Hadamard along the last axis), FP16 in and out, on the host."""
    X = np.ascontiguousarray(X, dtype=np.float16)
    K = X.shape[-1]
    rows = X.size // K
    out = np.empty_like(X)
    lib = load_library()
    _check(lib.qoq_hadamard_rotate(_np_ptr(X.view(np.uint16)), rows, K, K, _np_ptr(out.view(np.uint16))),
           "qoq_hadamard_rotate")
    return out


def qoq_smoothing_factors(act_absmax, w_absmax, alpha: float) -> np.ndarray:
    a = np.ascontiguousarray(act_absmax, dtype=np.float32)
    w = np.ascontiguousarray(w_absmax, dtype=np.float32)
    lam = np.empty_like(a)
    lib = load_library()
    _check(lib.qoq_smoothing_factors(_np_ptr(a), _np_ptr(w), a.size, float(alpha), _np_ptr(lam)),
           "qoq_smoothing_factors")
    return lam


def qoq_scale_columns(X: np.ndarray, factor, divide: bool = False) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.float16)
    K = X.shape[-1]
    f = np.ascontiguousarray(factor, dtype=np.float32)
    out = np.empty_like(X)
    lib = load_library()
    _check(lib.qoq_scale_columns(_np_ptr(X.view(np.uint16)), X.size // K, K, K, _np_ptr(f), int(divide),
                                 _np_ptr(out.view(np.uint16))), "qoq_scale_columns")
    return out
