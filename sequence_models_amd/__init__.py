"""Python binding of libtitans_mem.so (the Titans memory scan for MI355X).

Argument marshalling only: every step of the scan runs in the HIP kernels of
the library, on torch's current stream.  torch supplies device memory and the
stream; nothing here computes.  If the library is not built this module raises
at import time -- there is no fallback.

    scan(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths) -> (y, theta_T, s_T)
    scan_backward(q, k, v, alpha, eta, beta, theta0, s0, dy, chunk, widths,
                  dtheta_T=None, ds_T=None) -> cotangents of every input
    retrieve(q, theta, widths) -> y
    mag_forward(x, w_in, b_gate, w_out, theta0, s0, chunk, window, widths, eta_scale)
                  -> (out, theta_T, s_T)    one MAG block (memory as gate)
    mac_forward(x, w_in, b_gate, w_out, theta0, s0, chunk, segment, widths, eta_scale)
                  -> (out, theta_T, s_T)    one MAC block (memory as context)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["scan_noalloc", "mac_forward", "mac_workspace_size", "MacDesc", "mag_forward", "mag_workspace_size", "MagDesc", "scan", "scan_backward", "scan_backward_workspace_size", "retrieve", "scan_workspace_size", "scan_path", "retrieve_path", "param_count", "TitansError", "LIB_PATH",
           "lib", "ScanDesc", "MlpDesc", "MAX_LAYERS"]

# TITANS_MEM_LIB loads another build of the same sources instead (the tests' host-only
# sanitizer build of the validation layer); there is no fallback either way.
LIB_PATH = os.environ.get("TITANS_MEM_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libtitans_mem.so")
MAX_LAYERS = 4
F32, BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")


class MlpDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("width", ctypes.c_int32 * (MAX_LAYERS + 1))]


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("qkv_stride", ctypes.c_int64 * 3), ("y_stride", ctypes.c_int64 * 3),
                ("gate_stride", ctypes.c_int64 * 3), ("state_stride", ctypes.c_int64 * 2),
                ("state0_stride", ctypes.c_int64 * 2), ("bias", ctypes.c_int32),
                ("bias_param", ctypes.c_float)]


class MagDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("window", ctypes.c_int32), ("eta_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class MacDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("chunk", ctypes.c_int32), ("segment", ctypes.c_int32), ("eta_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


BIASES = {"l2": 0, "huber": 1, "lp": 2}


lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
lib.titans_abi_version.restype = ctypes.c_int
lib.titans_status_string.restype = ctypes.c_char_p
lib.titans_status_string.argtypes = [ctypes.c_int]
lib.titans_last_error.restype = ctypes.c_char_p
lib.titans_mem_param_count.restype = ctypes.c_int64
lib.titans_mem_param_count.argtypes = [ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_workspace_size.restype = ctypes.c_size_t
lib.titans_mem_scan_workspace_size.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_path.restype = ctypes.c_char_p
lib.titans_mem_scan_path.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mem_retrieve_path.restype = ctypes.c_char_p
lib.titans_mem_retrieve_path.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_noalloc.restype = ctypes.c_int
lib.titans_mem_scan_noalloc.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)] + [_vp] * 12
lib.titans_mem_scan.restype = ctypes.c_int
lib.titans_mem_scan.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)] + [_vp] * 12
                                + [ctypes.c_size_t, _vp])
lib.titans_mem_scan_surprise.restype = ctypes.c_int
lib.titans_mem_scan_surprise.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
                                         + [_vp] * 13 + [ctypes.c_size_t, _vp])
lib.titans_mem_scan_surprise_path.restype = ctypes.c_char_p
lib.titans_mem_scan_surprise_path.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_surprise_workspace_size.restype = ctypes.c_size_t
lib.titans_mem_scan_surprise_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                                        ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_backward_workspace_size.restype = ctypes.c_size_t
lib.titans_mem_scan_backward_workspace_size.argtypes = [ctypes.POINTER(ScanDesc),
                                                        ctypes.POINTER(MlpDesc)]
lib.titans_mem_scan_backward.restype = ctypes.c_int
lib.titans_mem_scan_backward.argtypes = ([ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc)]
                                         + [_vp] * 20 + [ctypes.c_size_t, _vp])
lib.titans_mag_workspace_size.restype = ctypes.c_size_t
lib.titans_mag_workspace_size.argtypes = [ctypes.POINTER(MagDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mag_forward.restype = ctypes.c_int
lib.titans_mag_forward.argtypes = ([ctypes.POINTER(MagDesc), ctypes.POINTER(MlpDesc)] + [_vp] * 10
                                   + [ctypes.c_size_t, _vp])
lib.titans_mac_workspace_size.restype = ctypes.c_size_t
lib.titans_mac_workspace_size.argtypes = [ctypes.POINTER(MacDesc), ctypes.POINTER(MlpDesc)]
lib.titans_mac_forward.restype = ctypes.c_int
lib.titans_mac_forward.argtypes = ([ctypes.POINTER(MacDesc), ctypes.POINTER(MlpDesc)] + [_vp] * 10
                                   + [ctypes.c_size_t, _vp])
lib.titans_mem_retrieve.restype = ctypes.c_int
lib.titans_mem_retrieve.argtypes = [ctypes.POINTER(ScanDesc), ctypes.POINTER(MlpDesc), _vp, _vp,
                                    _vp, _vp]


class TitansError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = lib.titans_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def _check(status: int):
    if status != 0:
        raise TitansError(status, lib.titans_last_error().decode())


def mlp_desc(widths) -> MlpDesc:
    widths = [int(w) for w in widths]
    m = MlpDesc()
    m.n_layers = len(widths) - 1
    for i, w in enumerate(widths[:MAX_LAYERS + 1]):
        m.width[i] = w
    return m


def param_count(widths) -> int:
    return int(lib.titans_mem_param_count(ctypes.byref(mlp_desc(widths))))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides3(t: torch.Tensor, name: str):
    if t.numel() == 0:  # nothing is accessed; report packed strides
        return t.shape[1] * t.shape[2] * t.shape[3], t.shape[2] * t.shape[3], t.shape[3]
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t.stride(0), t.stride(1), t.stride(2)


def _state_strides(t: torch.Tensor, batch: int, name: str):
    """[H,P] (shared over the batch: b-stride 0) or [B,H,P]; P contiguous."""
    if t.numel() == 0:
        return (0, t.shape[-1]) if t.dim() == 2 else (t.shape[1] * t.shape[2], t.shape[2])
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name}: P must be contiguous")
    if t.dim() == 2:
        return 0, t.stride(0)
    if t.dim() == 3 and t.shape[0] == batch:
        return t.stride(0), t.stride(1)
    raise ValueError(f"{name}: expected [H,P] or [B,H,P], got {tuple(t.shape)}")


def make_desc(q, chunk, y, gates, theta_T, theta0) -> ScanDesc:
    B, T, H, _ = q.shape
    d = ScanDesc()
    d.batch, d.seq_len, d.heads = B, T, H
    d.chunk = int(chunk)
    d.io_dtype = _io_dtype(q)
    d.qkv_stride[:] = _strides3(q, "q")
    d.y_stride[:] = _strides3(y, "y")
    if gates is not None:
        d.gate_stride[:] = gates.stride()
    if theta_T is not None:
        d.state_stride[:] = _state_strides(theta_T, B, "theta_T")
    if theta0 is not None:
        d.state0_stride[:] = _state_strides(theta0, B, "theta0")
    return d


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def scan_workspace_size(q, chunk, widths) -> int:
    """Workspace bytes titans_mem_scan needs for q's shape (raises on invalid arguments)."""
    d = make_desc(q, chunk, q, None, None, None)
    n = lib.titans_mem_scan_workspace_size(ctypes.byref(d), ctypes.byref(mlp_desc(widths)))
    if n == ctypes.c_size_t(-1).value:
        raise TitansError(1, "invalid scan shape or MLP widths")
    return int(n)


def scan_path(q, chunk, widths) -> str:
    """Name of the kernel that serves this shape: "fused_quad", "fused_pair", "fused_mfma", "phased_mfma" /
    "phased_fp32" (layers of 128+ units; bf16 / fp32 I/O) or "generic_mfma" / "generic_fp32"."""
    d = make_desc(q, chunk, q, None, None, None)
    r = lib.titans_mem_scan_path(ctypes.byref(d), ctypes.byref(mlp_desc(widths)))
    if r is None:
        raise TitansError(1, "invalid scan shape or MLP widths")
    return r.decode()


def surprise_path(q, chunk, widths) -> str:
    """Name of the kernel the scan with per-token surprise norms runs: "phased_*" or
    "generic_*" (the fused kernels do not produce the norms)."""
    d = make_desc(q, chunk, q, None, None, None)
    r = lib.titans_mem_scan_surprise_path(ctypes.byref(d), ctypes.byref(mlp_desc(widths)))
    if r is None:
        raise TitansError(1, "invalid scan shape or MLP widths")
    return r.decode()


def scan(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths, *, y=None, theta_T=None, s_T=None,
         workspace=None, bias=None, surprise=None):
    """Chunked Titans memory scan on the current stream.

    q, k, v: [B,T,H,d] float32/bfloat16 CUDA tensors (d contiguous);
    alpha, eta, beta: [B,T,H] float32; theta0, s0: [H,P] (shared by the batch) or [B,H,P].
    bias: the attentional bias of the writes, None (squared error), ("huber", delta) or
    ("lp", p).
    surprise: None, True (allocate) or a float32 tensor with alpha's shape and strides that
    receives each token's gradient norm (titans_mem_scan_surprise: the generic kernels).
    Returns (y [B,T,H,d] like q, theta_T [B,H,P], s_T [B,H,P]) and, when surprise is asked
    for, the surprise tensor as a fourth result.  theta_T / s_T may be passed as theta0 / s0
    themselves for in-place streaming.
    """
    B, T, H, dd = q.shape
    P = param_count(widths)
    if y is None:
        y = torch.empty((B, T, H, dd), dtype=q.dtype, device=q.device)
    if theta_T is None:
        theta_T = torch.empty((B, H, P), dtype=torch.float32, device=q.device)
    if s_T is None:
        s_T = torch.empty((B, H, P), dtype=torch.float32, device=q.device)
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.stride() != q.stride() or t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's shape, strides and dtype")
    for name, g in (("eta", eta), ("beta", beta)):
        if g.shape != alpha.shape or g.stride() != alpha.stride():
            raise ValueError(f"{name} must have alpha's shape and strides")
    for name, t in (("alpha", alpha), ("eta", eta), ("beta", beta), ("theta0", theta0), ("s0", s0),
                    ("theta_T", theta_T), ("s_T", s_T)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if s0.stride() != theta0.stride() or s0.shape != theta0.shape:
        raise ValueError("s0 must have theta0's shape and strides")
    if s_T.stride() != theta_T.stride() or s_T.shape != theta_T.shape:
        raise ValueError("s_T must have theta_T's shape and strides")
    desc = make_desc(q, chunk, y, alpha, theta_T, theta0)
    _set_bias(desc, bias)
    mlp = mlp_desc(widths)
    if surprise is True:
        surprise = torch.empty_like(alpha)
    if surprise is not None:
        if surprise.shape != alpha.shape or surprise.stride() != alpha.stride() or \
                surprise.dtype != torch.float32:
            raise ValueError("surprise must be float32 with alpha's shape and strides")
    size_fn = (lib.titans_mem_scan_workspace_size if surprise is None
               else lib.titans_mem_scan_surprise_workspace_size)
    if workspace is None:
        n = size_fn(ctypes.byref(desc), ctypes.byref(mlp))
        if n == ctypes.c_size_t(-1).value:
            n = 0  # the scan call below reports the argument error
        workspace = torch.empty(max(int(n), 1), dtype=torch.uint8, device=q.device) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if surprise is not None:
        _check(lib.titans_mem_scan_surprise(
            ctypes.byref(desc), ctypes.byref(mlp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
            _ptr(eta), _ptr(beta), _ptr(theta0), _ptr(s0), _ptr(y), _ptr(theta_T), _ptr(s_T),
            _ptr(surprise), _ptr(workspace), ws_bytes, _stream()))
        return y, theta_T, s_T, surprise
    _check(lib.titans_mem_scan(ctypes.byref(desc), ctypes.byref(mlp), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(alpha), _ptr(eta), _ptr(beta), _ptr(theta0), _ptr(s0), _ptr(y),
                               _ptr(theta_T), _ptr(s_T), _ptr(workspace), ws_bytes, _stream()))
    return y, theta_T, s_T


def scan_noalloc(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths, *, y, theta_T, s_T,
                 bias=None):
    """titans_mem_scan_noalloc on the current stream: the scan with no workspace (the pair
    path's shapes only; its scratch is the library's static device array).  The outputs
    y [B,T,H,d], theta_T and s_T [B,H,P] are passed in (nothing is allocated here either);
    arguments otherwise as for scan().  Returns (y, theta_T, s_T)."""
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.stride() != q.stride() or t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's shape, strides and dtype")
    for name, g in (("eta", eta), ("beta", beta)):
        if g.shape != alpha.shape or g.stride() != alpha.stride():
            raise ValueError(f"{name} must have alpha's shape and strides")
    for name, t in (("alpha", alpha), ("eta", eta), ("beta", beta), ("theta0", theta0), ("s0", s0),
                    ("theta_T", theta_T), ("s_T", s_T)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if s0.stride() != theta0.stride() or s0.shape != theta0.shape:
        raise ValueError("s0 must have theta0's shape and strides")
    if s_T.stride() != theta_T.stride() or s_T.shape != theta_T.shape:
        raise ValueError("s_T must have theta_T's shape and strides")
    desc = make_desc(q, chunk, y, alpha, theta_T, theta0)
    _set_bias(desc, bias)
    mlp = mlp_desc(widths)
    _check(lib.titans_mem_scan_noalloc(ctypes.byref(desc), ctypes.byref(mlp), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(alpha), _ptr(eta), _ptr(beta), _ptr(theta0),
                                       _ptr(s0), _ptr(y), _ptr(theta_T), _ptr(s_T), _stream()))
    return y, theta_T, s_T


def _set_bias(desc, bias):
    if bias is not None:
        desc.bias = BIASES[bias[0]]
        desc.bias_param = float(bias[1]) if len(bias) > 1 else 0.0


def scan_backward_workspace_size(q, chunk, widths, bias=None) -> int:
    """Workspace bytes titans_mem_scan_backward needs for q's shape."""
    d = make_desc(q, chunk, q, None, None, None)
    _set_bias(d, bias)
    n = lib.titans_mem_scan_backward_workspace_size(ctypes.byref(d), ctypes.byref(mlp_desc(widths)))
    if n == ctypes.c_size_t(-1).value:
        raise TitansError(1, "invalid or unsupported shape, MLP widths or bias")
    return int(n)


BACKWARD_NAMES = ("q", "k", "v", "alpha", "eta", "beta", "theta0", "s0")


def scan_backward(q, k, v, alpha, eta, beta, theta0, s0, dy, chunk, widths, *, dtheta_T=None,
                  ds_T=None, bias=None, workspace=None, out=None):
    """Cotangents of the scan's inputs (titans_mem_scan_backward) on the current stream.

    Arguments as for scan, plus dy (y's shape, q's dtype) and dtheta_T / ds_T ([B,H,P]
    float32 or None = zero).  Returns a dict keyed by BACKWARD_NAMES: dq/dk/dv with q's
    shape, strides and dtype, gate cotangents with alpha's, state cotangents [B,H,P] (with
    dtheta_T's strides when given; the caller sums over b when theta0 is shared by the
    batch).  out may supply any of these tensors; passing dtheta_T / ds_T themselves as
    out["theta0"] / out["s0"] runs in place.
    """
    B, T, H, dd = q.shape
    P = param_count(widths)
    out = dict(out or {})
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.stride() != q.stride() or t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's shape, strides and dtype")
    if dy.shape != q.shape or dy.dtype != q.dtype:
        raise ValueError("dy must have q's shape and dtype")
    for name, g in (("eta", eta), ("beta", beta)):
        if g.shape != alpha.shape or g.stride() != alpha.stride():
            raise ValueError(f"{name} must have alpha's shape and strides")
    state_like = dtheta_T if dtheta_T is not None else ds_T
    for name in ("q", "k", "v"):
        out.setdefault(name, torch.empty_strided(q.shape, q.stride(), dtype=q.dtype,
                                                 device=q.device))
    for name in ("alpha", "eta", "beta"):
        out.setdefault(name, torch.empty_strided(alpha.shape, alpha.stride(),
                                                 dtype=torch.float32, device=q.device))
    for name in ("theta0", "s0"):
        if state_like is not None:
            out.setdefault(name, torch.empty_strided(state_like.shape, state_like.stride(),
                                                     dtype=torch.float32, device=q.device))
        else:
            out.setdefault(name, torch.empty((B, H, P), dtype=torch.float32, device=q.device))
    for name in ("dtheta_T", "ds_T"):
        t = dtheta_T if name == "dtheta_T" else ds_T
        if t is not None and (t.stride() != out["theta0"].stride() or t.dtype != torch.float32
                              or tuple(t.shape) != (B, H, P)):
            raise ValueError(f"{name} must be float32 [B,H,P] with the strides of dtheta0")
    for name in ("q", "k", "v"):
        if out[name].stride() != q.stride() or out[name].dtype != q.dtype:
            raise ValueError(f"d{name} must have q's strides and dtype")
    for name in ("alpha", "eta", "beta"):
        if out[name].stride() != alpha.stride() or out[name].dtype != torch.float32:
            raise ValueError(f"d{name} must be float32 with alpha's strides")
    if out["s0"].stride() != out["theta0"].stride():
        raise ValueError("ds0 must have dtheta0's strides")
    desc = make_desc(q, chunk, dy, alpha, out["theta0"], theta0)
    _set_bias(desc, bias)
    mlp = mlp_desc(widths)
    if workspace is None:
        n = lib.titans_mem_scan_backward_workspace_size(ctypes.byref(desc), ctypes.byref(mlp))
        if n == ctypes.c_size_t(-1).value:
            n = 0  # the call below reports the argument error
        workspace = torch.empty(int(n), dtype=torch.uint8, device=q.device) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.titans_mem_scan_backward(
        ctypes.byref(desc), ctypes.byref(mlp), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta),
        _ptr(beta), _ptr(theta0), _ptr(s0), _ptr(dy), _ptr(dtheta_T), _ptr(ds_T),
        _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["alpha"]), _ptr(out["eta"]),
        _ptr(out["beta"]), _ptr(out["theta0"]), _ptr(out["s0"]), _ptr(workspace), ws_bytes,
        _stream()))
    return out


def retrieve_path(q, widths) -> str:
    """Name of the kernel titans_mem_retrieve runs for q's shape: "fused_mfma", "wide_mfma",
    "generic_mfma" or "generic_fp32"."""
    d = make_desc(q, 1, q, None, None, None)
    r = lib.titans_mem_retrieve_path(ctypes.byref(d), ctypes.byref(mlp_desc(widths)))
    if r is None:
        raise TitansError(1, "invalid retrieve shape or MLP widths")
    return r.decode()


def retrieve(q, theta, widths, *, y=None):
    """y = M_theta(q) with fixed weights; q [B,T,H,d], theta [H,P] or [B,H,P] float32."""
    B, T, H, dd = q.shape
    if y is None:
        y = torch.empty((B, T, H, dd), dtype=q.dtype, device=q.device)
    if theta.dtype != torch.float32:
        raise TypeError("theta must be float32")
    desc = make_desc(q, 1, y, None, theta, None)
    _check(lib.titans_mem_retrieve(ctypes.byref(desc), ctypes.byref(mlp_desc(widths)), _ptr(q),
                                   _ptr(theta), _ptr(y), _stream()))
    return y


def _mag_desc(x, widths, chunk, window, eta_scale) -> MagDesc:
    B, T, D = x.shape
    d = widths[0]
    if D % d:
        raise ValueError(f"model width {D} is not a multiple of the head width {d}")
    return MagDesc(B, T, D // d, int(chunk), int(window), float(eta_scale), 0)


def mag_workspace_size(x, chunk, window, widths, eta_scale=1.0) -> int:
    """Workspace bytes of mag_forward for x [B, T, D] (raises on invalid arguments)."""
    n = lib.titans_mag_workspace_size(ctypes.byref(_mag_desc(x, widths, chunk, window, eta_scale)),
                                      ctypes.byref(mlp_desc(widths)))
    if n == ctypes.c_size_t(-1).value:
        raise TitansError(-1, lib.titans_last_error().decode())
    return int(n)


def _block(fn, size_fn, desc, x, w_in, b_gate, w_out, theta0, s0, widths, out, theta_T, s_T,
           workspace):
    B, T, D = x.shape
    d = widths[0]
    H = D // d
    P = param_count(widths)
    if out is None:
        out = torch.empty((B, T, D), dtype=torch.bfloat16, device=x.device)
    if theta_T is None:
        theta_T = torch.empty((B, H, P), dtype=torch.float32, device=x.device)
    if s_T is None:
        s_T = torch.empty((B, H, P), dtype=torch.float32, device=x.device)
    shapes = {"x": (x, torch.bfloat16, (B, T, D)), "w_in": (w_in, torch.bfloat16, (3 * D + 3 * H, D)),
              "b_gate": (b_gate, torch.float32, (3 * H,)), "w_out": (w_out, torch.bfloat16, (D, D)),
              "theta0": (theta0, torch.float32, (B, H, P)), "s0": (s0, torch.float32, (B, H, P)),
              "out": (out, torch.bfloat16, (B, T, D)), "theta_T": (theta_T, torch.float32, (B, H, P)),
              "s_T": (s_T, torch.float32, (B, H, P))}
    for name, (t, dt, shape) in shapes.items():
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape}")
    mlp = mlp_desc(widths)
    if workspace is None:
        n = size_fn(ctypes.byref(desc), ctypes.byref(mlp))
        if n == ctypes.c_size_t(-1).value:
            n = 0  # the call below reports the argument error
        workspace = torch.empty(int(n), dtype=torch.uint8, device=x.device) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(ctypes.byref(desc), ctypes.byref(mlp), _ptr(x), _ptr(w_in), _ptr(b_gate),
              _ptr(w_out), _ptr(theta0), _ptr(s0), _ptr(out), _ptr(theta_T), _ptr(s_T),
              _ptr(workspace), ws_bytes, _stream()))
    return out, theta_T, s_T


def mag_forward(x, w_in, b_gate, w_out, theta0, s0, chunk, window, widths, eta_scale, *,
                out=None, theta_T=None, s_T=None, workspace=None):
    """One MAG block on the current stream (titans_mag_forward).

    x [B, T, D] bf16; w_in [3D + 3H, D] bf16 (q, k, v rows, then alpha, eta, beta gate
    rows); b_gate [3H] float32; w_out [D, D] bf16; theta0, s0 [B, H, P] float32, with
    H = D / widths[0].  Every tensor contiguous.  Returns (out [B, T, D] bf16, theta_T,
    s_T [B, H, P])."""
    return _block(lib.titans_mag_forward, lib.titans_mag_workspace_size,
                  _mag_desc(x, widths, chunk, window, eta_scale), x, w_in, b_gate, w_out, theta0,
                  s0, widths, out, theta_T, s_T, workspace)


def _mac_desc(x, widths, chunk, segment, eta_scale) -> MacDesc:
    m = _mag_desc(x, widths, chunk, segment, eta_scale)
    return MacDesc(m.batch, m.seq_len, m.heads, m.chunk, m.window, m.eta_scale, 0)


def mac_workspace_size(x, chunk, segment, widths, eta_scale=1.0) -> int:
    """Workspace bytes of mac_forward for x [B, T, D] (raises on invalid arguments)."""
    n = lib.titans_mac_workspace_size(ctypes.byref(_mac_desc(x, widths, chunk, segment, eta_scale)),
                                      ctypes.byref(mlp_desc(widths)))
    if n == ctypes.c_size_t(-1).value:
        raise TitansError(-1, lib.titans_last_error().decode())
    return int(n)


def mac_forward(x, w_in, b_gate, w_out, theta0, s0, chunk, segment, widths, eta_scale, *,
                out=None, theta_T=None, s_T=None, workspace=None):
    """One MAC block on the current stream (titans_mac_forward): the MAG block's tensors,
    segments of `segment` tokens whose memory reads prefix the attention's keys and values."""
    return _block(lib.titans_mac_forward, lib.titans_mac_workspace_size,
                  _mac_desc(x, widths, chunk, segment, eta_scale), x, w_in, b_gate, w_out, theta0,
                  s0, widths, out, theta_T, s_T, workspace)
