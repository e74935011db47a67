"""Accurate float32 reductions on MI355X: compensated-tree sum and variance.

Thin Python binding over the C ABI of ``libstable_variance.so``
(``include/stable_variance.h``).  It only marshals arguments: every step of
the computation runs in the HIP kernels.  PyTorch provides device memory and
the current stream.  There is no CPU fallback: if the library is missing or
no GPU is visible, the calls raise.

    tree_sum(x)                    -> 0-d float32 tensor, compensated tree sum
    var(x, dim=-1, ddof=0, return_mean=False)
                                   -> per-slice variance (and mean) of a 2-D
                                      (or 1-D) float32 tensor

Method: Pennacchio, "Variance in float32 with a first-element shift, a local
centring and a compensated tree sum", §2 steps 1-4.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB as _LIB_PATH

__all__ = ["tree_sum", "var", "var_variant", "capi", "library_path", "SvError", "set_tuning", "VARIANTS"]

SV_OK = 0
_STATUS = {1: "SV_ERR_INVALID_ARGUMENT", 2: "SV_ERR_WORKSPACE", 3: "SV_ERR_NO_DEVICE", 4: "SV_ERR_HIP",
           5: "SV_ERR_UNSUPPORTED"}


class SvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def capi():
    """The loaded C library with argument types declared (raises if absent)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise ImportError(
                        f"libstable_variance.so is not built ({_LIB_PATH}); run __graft_entry__.build()")
                # torch first: its HIP runtime and the library's have the same
                # soname, so whichever loads first serves both, and torch's
                # allocations need its own
                import torch  # noqa: F401
                L = ctypes.CDLL(_LIB_PATH)
                i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
                L.sv_abi_version.restype = ctypes.c_int
                L.sv_abi_version.argtypes = []
                L.sv_status_string.restype = ctypes.c_char_p
                L.sv_status_string.argtypes = [ctypes.c_int]
                L.sv_last_error_message.restype = ctypes.c_char_p
                L.sv_last_error_message.argtypes = []
                L.sv_tree_sum_f32_workspace_size.restype = sz
                L.sv_tree_sum_f32_workspace_size.argtypes = [i64]
                L.sv_tree_sum_f32.restype = ctypes.c_int
                L.sv_tree_sum_f32.argtypes = [vp, i64, vp, vp, sz, vp]
                L.sv_tree_sum_f32_noalloc.restype = ctypes.c_int
                L.sv_tree_sum_f32_noalloc.argtypes = [vp, i64, vp, vp]
                L.sv_variance_f32_workspace_size.restype = sz
                L.sv_variance_f32_workspace_size.argtypes = [i64, i64, ctypes.c_int]
                L.sv_variance_f32.restype = ctypes.c_int
                L.sv_variance_f32.argtypes = [vp, i64, i64, ctypes.c_int, i64, vp, vp, vp, sz, vp]
                L.sv_set_tuning.restype = ctypes.c_int
                L.sv_set_tuning.argtypes = [ctypes.c_char_p, i64]
                L.sv_variance_c64_workspace_size.restype = sz
                L.sv_variance_c64_workspace_size.argtypes = [i64, i64, ctypes.c_int]
                L.sv_variance_c64.restype = ctypes.c_int
                L.sv_variance_c64.argtypes = [vp, i64, i64, ctypes.c_int, i64, vp, vp, vp, sz, vp]
                L.sv_variance_variant_f32.restype = ctypes.c_int
                L.sv_variance_variant_f32.argtypes = [vp, i64, i64, ctypes.c_int, i64, ctypes.c_int, vp, vp, vp]
                L.sv_variance_variant_f32_workspace_size.restype = sz
                L.sv_variance_variant_f32_workspace_size.argtypes = [i64, i64, ctypes.c_int, ctypes.c_int]
                L.sv_variance_variant_ws_f32.restype = ctypes.c_int
                L.sv_variance_variant_ws_f32.argtypes = [vp, i64, i64, ctypes.c_int, i64, ctypes.c_int, vp, vp, vp,
                                                         sz, vp]
                L.sv_tree_sum_f64_workspace_size.restype = sz
                L.sv_tree_sum_f64_workspace_size.argtypes = [i64]
                L.sv_tree_sum_f64.restype = ctypes.c_int
                L.sv_tree_sum_f64.argtypes = [vp, i64, vp, vp, sz, vp]
                L.sv_variance_f64.restype = ctypes.c_int
                L.sv_variance_f64.argtypes = [vp, i64, i64, ctypes.c_int, i64, vp, vp, vp, sz, vp]
                L.sv_variance_f64_workspace_size.restype = sz
                L.sv_variance_f64_workspace_size.argtypes = [i64, i64, ctypes.c_int]
                L.sv_tree_sum_dw_f32.restype = ctypes.c_int
                L.sv_tree_sum_dw_f32.argtypes = [vp, i64, vp, vp, sz, vp]
                L.sv_adn_sum_f32_workspace_size.restype = sz
                L.sv_adn_sum_f32_workspace_size.argtypes = [i64]
                L.sv_adn_sum_f32.restype = ctypes.c_int
                L.sv_adn_sum_f32.argtypes = [vp, i64, ctypes.c_int, vp, vp, sz, vp]
                L.sv_probe_read_bandwidth.restype = ctypes.c_int
                L.sv_probe_read_bandwidth.argtypes = [vp, i64, vp, vp]
                _lib = L
    return _lib


def _check(status: int) -> None:
    if status != SV_OK:
        msg = capi().sv_last_error_message().decode(errors="replace")
        raise SvError(status, msg)


def set_tuning(key: str, value: int) -> None:
    """Launch-geometry knob (never changes results); see the C header."""
    _check(capi().sv_set_tuning(key.encode(), int(value)))


# Workspaces, one per (kind, device, stream).  The tree sum's buffer is
# zero-filled when allocated and the library leaves its ticket counters at
# zero after every call; the variance's buffer is scratch (its axis-0 ticket
# counters are cleared inside every call).  They are never shared: scratch
# use would leave nonzero counters behind in a sum workspace.
_workspaces: dict = {}


def _workspace(kind: str, nbytes: int, device, stream_handle: int):
    import torch

    if nbytes == 0:
        return None
    key = (kind, device.index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _check_tensor(x, name="x", complex_ok=False, double_ok=False):
    import torch

    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    ok = (torch.float32,) + ((torch.complex64,) if complex_ok else ()) + ((torch.float64,) if double_ok else ())
    if x.dtype not in ok:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in ok)}, got {x.dtype}")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {x.device}")


def tree_sum(x, carry: str = "plain"):
    """Compensated pairwise tree sum of all elements of a float32 (or
    float64: every operation in double) tensor.

    ``carry="dw"`` renormalises every node's (sum, carry) pair (double-word
    carries, ``sv_tree_sum_dw_f32``)."""
    import torch

    _check_tensor(x, double_ok=True)
    if carry not in ("plain", "dw"):
        raise ValueError(f"carry must be 'plain' or 'dw', got {carry!r}")
    is_double = x.dtype == torch.float64
    if is_double and carry != "plain":
        raise ValueError("double-word carries are built for float32 input only")
    x = x.contiguous().reshape(-1)
    n = x.numel()
    L = capi()
    fn = L.sv_tree_sum_f64 if is_double else (L.sv_tree_sum_f32 if carry == "plain" else L.sv_tree_sum_dw_f32)
    wsz = L.sv_tree_sum_f64_workspace_size if is_double else L.sv_tree_sum_f32_workspace_size
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        out = torch.empty((), dtype=x.dtype, device=x.device)
        need = wsz(n)
        if need == ctypes.c_size_t(-1).value:
            raise SvError(5, f"tree_sum: n = {n} is not supported")
        ws = _workspace("sum64" if is_double else "sum", need, x.device, stream)
        _check(fn(x.data_ptr() if n else None, n, out.data_ptr(), ws.data_ptr() if ws is not None else None, need,
                  stream))
    return out


def adn_sum(x, fold: int = 3):
    """Ahrens-Demmel-Nguyen binned reproducible sum of all elements of a
    float32 tensor, with ``fold`` bins (same bits for any order)."""
    import torch

    _check_tensor(x)
    x = x.contiguous().reshape(-1)
    n = x.numel()
    L = capi()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        out = torch.empty((), dtype=torch.float32, device=x.device)
        need = L.sv_adn_sum_f32_workspace_size(n)
        if need == ctypes.c_size_t(-1).value:
            raise SvError(5, f"adn_sum: n = {n} exceeds the accumulator capacity")
        ws = _workspace("adn", need, x.device, stream)
        _check(L.sv_adn_sum_f32(x.data_ptr() if n else None, n, int(fold), out.data_ptr(),
                                ws.data_ptr() if ws is not None else None, need, stream))
    return out


def var(x, dim: int = -1, ddof: int = 0, return_mean: bool = False):
    """Variance of each slice of a 2-D (or 1-D) float32, float64 or complex64
    tensor along ``dim`` (float64: the method with every operation in double).

    Returns a tensor of the non-reduced length (a 0-d tensor for 1-D input):
    float32 for float32 and complex64 data, float64 for float64 data, and the
    mean (same dtype as the data) when ``return_mean``.  For complex64 data
    the variance is var(re) + var(im), each part as for float32.  Inputs that
    are not contiguous are copied to a contiguous tensor first.
    """
    import torch

    _check_tensor(x, complex_ok=True, double_ok=True)
    is_complex = x.dtype == torch.complex64
    is_double = x.dtype == torch.float64
    if x.dim() == 1:
        if dim not in (0, -1):
            raise ValueError(f"dim {dim} out of range for a 1-D tensor")
        x2 = x.reshape(1, -1)
        axis = 1
        squeeze = True
    elif x.dim() == 2:
        x2 = x
        if dim not in (0, 1, -1, -2):
            raise ValueError(f"dim {dim} out of range for a 2-D tensor")
        axis = dim % 2
        squeeze = False
    else:
        raise ValueError("var expects a 1-D or 2-D tensor")
    if ddof < 0:
        raise ValueError("ddof must be >= 0")
    x2 = x2.contiguous()
    rows, cols = x2.shape
    ns = rows if axis == 1 else cols
    L = capi()
    if is_double:
        with torch.cuda.device(x.device):
            stream = torch.cuda.current_stream(x.device).cuda_stream
            out = torch.empty(ns, dtype=torch.float64, device=x.device)
            mean = torch.empty(ns, dtype=torch.float64, device=x.device) if return_mean else None
            need = L.sv_variance_f64_workspace_size(rows, cols, axis)
            if need == ctypes.c_size_t(-1).value:
                raise SvError(5, f"var: shape {tuple(x2.shape)} along dim {axis} is not supported")
            ws = _workspace("var64", need, x.device, stream)
            _check(L.sv_variance_f64(x2.data_ptr() if x2.numel() else None, rows, cols, axis, int(ddof),
                                     out.data_ptr() if ns else None,
                                     mean.data_ptr() if (mean is not None and ns) else None,
                                     ws.data_ptr() if ws is not None else None, need, stream))
        if squeeze:
            out = out.reshape(())
            mean = mean.reshape(()) if mean is not None else None
        return (out, mean) if return_mean else out
    fn = L.sv_variance_c64 if is_complex else L.sv_variance_f32
    wsz = L.sv_variance_c64_workspace_size if is_complex else L.sv_variance_f32_workspace_size
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        out = torch.empty(ns, dtype=torch.float32, device=x.device)
        mean = torch.empty(ns, dtype=x.dtype, device=x.device) if return_mean else None
        need = wsz(rows, cols, axis)
        if need == ctypes.c_size_t(-1).value:
            raise SvError(5, f"var: shape {tuple(x2.shape)} along axis {axis} is not supported")
        ws = _workspace("var", need, x.device, stream)
        _check(fn(x2.data_ptr() if x2.numel() else None, rows, cols, axis, int(ddof),
                  out.data_ptr() if ns else None,
                  mean.data_ptr() if (mean is not None and ns) else None,
                  ws.data_ptr() if ws is not None else None, need, stream))
    if squeeze:
        out = out.reshape(())
        mean = mean.reshape(()) if mean is not None else None
    return (out, mean) if return_mean else out


# Ablation variants of the method page's §4 (see sv_variance_variant_f32).
VARIANTS = {
    "kernel": 0,
    "kernel_comp_y": 1,
    "reference": 2,
    "naive": 3,
    "shift_plain_no2t": 4,
    "shift_plain_2t": 5,
    "noshift_comp_2t": 6,
    "shift_comp_no2t": 7,
    "shift_kahan_no2t": 8,
}


def var_variant(x, variant, dim: int = -1, ddof: int = 0, return_mean: bool = False):
    """One of the ablation variants (a name of VARIANTS or its number) on a
    2-D float32 tensor.  The tree variants take one workgroup per slice (rows
    of up to 16384 values, columns of up to 1024) or, beyond, the long-slice
    launches with a workspace (slices of up to 2^27 values); the Kahan scan
    takes slices of up to 2^22 values."""
    import torch

    _check_tensor(x)
    code = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    axis = 1 if x.dim() == 1 else dim % 2
    x2 = x2.contiguous()
    rows, cols = x2.shape
    ns = rows if axis == 1 else cols
    L = capi()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        out = torch.empty(ns, dtype=torch.float32, device=x.device)
        mean = torch.empty(ns, dtype=torch.float32, device=x.device) if return_mean else None
        need = L.sv_variance_variant_f32_workspace_size(rows, cols, axis, code)
        need = 0 if need == ctypes.c_size_t(-1).value else need  # the call reports the error
        ws = _workspace("variant", need, x.device, stream)
        _check(L.sv_variance_variant_ws_f32(x2.data_ptr() if x2.numel() else None, rows, cols, axis, int(ddof), code,
                                            out.data_ptr() if ns else None,
                                            mean.data_ptr() if (mean is not None and ns) else None,
                                            ws.data_ptr() if ws is not None else None, need, stream))
    return (out, mean) if return_mean else out
