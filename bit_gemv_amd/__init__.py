"""bit_gemv_amd -- Python binding of libquant, the gfx950 C-ABI library.

Argument marshalling only: every function takes torch tensors on the current
HIP device, checks dtypes and shapes, allocates missing outputs with torch,
and calls the C entry point of the same name (declared in
``include/libquant.h``) on torch's current stream. All arithmetic happens in
the HIP kernels of ``libquant.so``; there is no fallback. If the library is
not built, importing the entry points raises.

Layouts (see the header): W[n][k] row-major with groups of ``group`` along k;
INT4 codes [n][k/2] (element 2j in the low nibble of byte j, symmetric codes
stored as q + 8); INT8 codes [n][k]; fp32 scales and zeros [n][k/group].
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libquant.so")

LQ_OK, LQ_ERR_INVALID_ARG, LQ_ERR_UNSUPPORTED, LQ_ERR_HIP, LQ_ERR_NO_DEVICE = range(5)

ENTRY_POINTS = ("quantize_groupwise", "dequantize_groupwise", "w4a16_gemv", "w8a16_gemv", "w4a16_gemm",
                "smooth_scale", "quant_per_token_int8", "w8a8_gemm", "act_absmean", "awq_search",
                "mxfp4_quantize", "mxfp4_gemv", "mxfp4_gemm", "gptq_hessian_factor", "gptq_quantize")


class LibquantError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {detail} (status {status})")


_lib = None


def load_library(path: Optional[str] = None):
    """Load libquant.so (torch is imported first, so its HIP runtime is the one
    the library binds to). Raises if the library has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libquant.so not built ({p}); run `python -m bit_gemv_amd.build`")
    lib = ctypes.CDLL(p)
    P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sigs = {
        "quantize_groupwise": [P, I64, I64, I, I, I64, P, P, P, P, P],
        "dequantize_groupwise": [P, P, P, I64, I64, I, I, I64, P, P],
        "w4a16_gemv": [P, I64, P, P, P, I64, I64, I, I64, P, P],
        "w8a16_gemv": [P, I64, P, P, P, I64, I64, I, I64, P, P],
        "w4a16_gemm": [P, I64, P, P, P, I64, I64, I, I64, P, P],
        "smooth_scale": [P, I64, P, I64, I64, F, P, P],
        "quant_per_token_int8": [P, I64, I64, P, P, P, P],
        "w8a8_gemm": [P, P, I64, P, P, I64, I64, P, P, P],
        "act_absmean": [P, I64, I64, P, P],
        "mxfp4_quantize": [P, I64, I64, P, P, P],
        "mxfp4_gemv": [P, I64, P, P, I64, I64, P, P],
        "mxfp4_gemm": [P, I64, P, P, I64, I64, P, P],
        "gptq_hessian_factor": [P, I64, I64, F, P, I64, P, P],
        "gptq_quantize": [P, I64, I64, P, I, I, I64, P, I64, P, P, P, P],
        "gptq_quantize_noalloc": [P, I64, I64, P, I, I, I64, P, P, P, P],
        "awq_search": [P, I64, P, I64, I64, I, I64, I, P, P, I64, P, P, P, P, P, P, P],
    }
    for name, argtypes in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    lib.lq_last_error.restype = ctypes.c_char_p
    lib.lq_last_error.argtypes = []
    lib.lq_status_string.restype = ctypes.c_char_p
    lib.lq_status_string.argtypes = [ctypes.c_int]
    lib.lq_abi_version.restype = ctypes.c_int
    lib.awq_workspace_bytes.argtypes = [I64, I64, I64]
    lib.awq_workspace_bytes.restype = ctypes.c_int64
    lib.gptq_workspace_bytes.argtypes = [I64, I64, I64]
    lib.gptq_workspace_bytes.restype = ctypes.c_int64
    lib.gptq_quantize_noalloc_max_bytes.argtypes = []
    lib.gptq_quantize_noalloc_max_bytes.restype = ctypes.c_int64
    lib.lq_read_probe_sink_words.argtypes = []
    lib.lq_read_probe_sink_words.restype = ctypes.c_int64
    lib.lq_hbm_read_probe.argtypes = [P, I64, P, P]
    lib.lq_hbm_read_probe.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _call(name: str, *args) -> None:
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != LQ_OK:
        detail = lib.lq_last_error().decode() or lib.lq_status_string(st).decode()
        raise LibquantError(st, name, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


@dataclass
class PackedWeight:
    """Output of quantize_groupwise: codes, scales, zeros plus their settings."""
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: Optional[torch.Tensor]
    n: int
    k: int
    bits: int
    symmetric: bool
    group: int

    def nbytes(self) -> int:
        z = 0 if self.zeros is None else self.zeros.numel() * 4
        return self.codes.numel() + self.scales.numel() * 4 + z


def quantize_groupwise(w: torch.Tensor, bits: int = 4, symmetric: bool = False, group: int = 128,
                       col_scale: Optional[torch.Tensor] = None, out: Optional[PackedWeight] = None
                       ) -> PackedWeight:
    """Group-wise RTN quantization of bf16 W[n][k] (see libquant.h)."""
    n, k = w.shape
    _need(w, "w", torch.bfloat16)
    if col_scale is not None:
        _need(col_scale, "col_scale", torch.float32, (k,))
    if out is None:
        dev = w.device
        ng = k // group if group > 0 and k % group == 0 else 0
        codes = torch.empty((n, k // 2 if bits == 4 else k), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, ng), dtype=torch.float32, device=dev)
        zeros = None if symmetric else torch.empty((n, ng), dtype=torch.float32, device=dev)
        out = PackedWeight(codes, scales, zeros, n, k, bits, bool(symmetric), group)
    _call("quantize_groupwise", _ptr(w), n, k, bits, int(bool(symmetric)), group, _ptr(col_scale),
          _ptr(out.codes), _ptr(out.scales), _ptr(out.zeros), _stream())
    return out


def dequantize_groupwise(pw: PackedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x_hat = s (q - z) as fp32 [n][k]."""
    if out is None:
        out = torch.empty((pw.n, pw.k), dtype=torch.float32, device=pw.codes.device)
    _need(out, "out", torch.float32, (pw.n, pw.k))
    _call("dequantize_groupwise", _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.zeros), pw.n, pw.k, pw.bits,
          int(pw.symmetric), pw.group, _ptr(out), _stream())
    return out


def _wo(name: str, bits: int, x: torch.Tensor, pw: PackedWeight, y: Optional[torch.Tensor]) -> torch.Tensor:
    if pw.bits != bits:
        raise ValueError(f"{name} needs INT{bits} codes")
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    if k != pw.k:
        raise ValueError(f"x has {k} columns, weights have k = {pw.k}")
    if y is None:
        y = torch.empty((m, pw.n), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, pw.n))
    _call(name, _ptr(x), m, _ptr(pw.codes), _ptr(pw.scales), _ptr(pw.zeros), pw.n, pw.k, int(pw.symmetric),
          pw.group, _ptr(y), _stream())
    return y


def w4a16_gemv(x: torch.Tensor, pw: PackedWeight, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b][n] = x[b][k] W_hat^T for b <= 16 (fp32 out)."""
    return _wo("w4a16_gemv", 4, x, pw, y)


def w8a16_gemv(x: torch.Tensor, pw: PackedWeight, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b][n] = x[b][k] W_hat^T on INT8 codes for b <= 16 (fp32 out)."""
    return _wo("w8a16_gemv", 8, x, pw, y)


def w4a16_gemm(x: torch.Tensor, pw: PackedWeight, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[m][n] = x[m][k] W_hat^T for any m (fp32 out, bf16 MFMA)."""
    return _wo("w4a16_gemm", 4, x, pw, y)


def smooth_scale(x: torch.Tensor, w: torch.Tensor, alpha: float = 0.5,
                 s: Optional[torch.Tensor] = None) -> torch.Tensor:
    """s[k] = max_t|X[:,k]|^alpha / max_n|W[:,k]|^(1-alpha)."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    t, k = x.shape
    n, kw = w.shape
    if kw != k:
        raise ValueError("x and w must share k")
    if s is None:
        s = torch.empty(k, dtype=torch.float32, device=x.device)
    _need(s, "s", torch.float32, (k,))
    _call("smooth_scale", _ptr(x), t, _ptr(w), n, k, float(alpha), _ptr(s), _stream())
    return s


def quant_per_token_int8(x: torch.Tensor, smooth: Optional[torch.Tensor] = None,
                         qx: Optional[torch.Tensor] = None, sx: Optional[torch.Tensor] = None):
    """Dynamic per-token symmetric INT8 of X / smooth -> (qx int8 [t][k], sx fp32 [t])."""
    _need(x, "x", torch.bfloat16)
    t, k = x.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, (k,))
    if qx is None:
        qx = torch.empty((t, k), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty(t, dtype=torch.float32, device=x.device)
    _need(qx, "qx", torch.int8, (t, k))
    _need(sx, "sx", torch.float32, (t,))
    _call("quant_per_token_int8", _ptr(x), t, k, _ptr(smooth), _ptr(qx), _ptr(sx), _stream())
    return qx, sx


def w8a8_gemm(qx: torch.Tensor, sx: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
              y: Optional[torch.Tensor] = None, acc: Optional[torch.Tensor] = None, want_acc: bool = False):
    """INT8 GEMM: acc = qx qw^T (int32), y = acc * sx * sw (fp32). Returns (y, acc or None)."""
    _need(qx, "qx", torch.int8)
    _need(qw, "qw", torch.int8)
    m, k = qx.shape
    n, kw = qw.shape
    if kw != k:
        raise ValueError("qx and qw must share k")
    _need(sx, "sx", torch.float32, (m,))
    _need(sw, "sw", torch.float32, (n,))
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=qx.device)
    if acc is None and want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=qx.device)
    _need(y, "y", torch.float32, (m, n))
    if acc is not None:
        _need(acc, "acc", torch.int32, (m, n))
    _call("w8a8_gemm", _ptr(qx), _ptr(sx), m, _ptr(qw), _ptr(sw), n, k, _ptr(acc), _ptr(y), _stream())
    return y, acc


def abi_version() -> int:
    return load_library().lq_abi_version()


def act_absmean(x: torch.Tensor, sx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sx[k] = mean_t |X[t][k]| (fp32; fp64 sums), AWQ's channel magnitude."""
    _need(x, "x", torch.bfloat16)
    t, k = x.shape
    if sx is None:
        sx = torch.empty(k, dtype=torch.float32, device=x.device)
    _need(sx, "sx", torch.float32, (k,))
    _call("act_absmean", _ptr(x), t, k, _ptr(sx), _stream())
    return sx


@dataclass
class AwqResult:
    """Output of awq_search: the packed INT4 weights of W diag(s_best), the
    chosen scale (to fold 1/s_best into the producer of X), the loss of every
    grid point and the index of the chosen one (device tensors)."""
    packed: PackedWeight
    s_best: torch.Tensor
    losses: torch.Tensor
    best: torch.Tensor
    n_grid: int


def awq_search(x: torch.Tensor, w: torch.Tensor, sx: Optional[torch.Tensor] = None, symmetric: bool = False,
               group: int = 128, n_grid: int = 20, workspace: Optional[torch.Tensor] = None) -> AwqResult:
    """AWQ scale search over alpha = i / n_grid (see libquant.h); x [t][k] and
    w [n][k] bf16. sx defaults to act_absmean(x)."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    t, k = x.shape
    n, kw = w.shape
    if kw != k:
        raise ValueError("x and w must share k")
    if sx is None:
        sx = act_absmean(x)
    _need(sx, "sx", torch.float32, (k,))
    need = load_library().awq_workspace_bytes(t, n, k)
    if need < 0:
        raise LibquantError(LQ_ERR_INVALID_ARG, "awq_search", "sizes out of range")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    dev = x.device
    ng = k // group if group > 0 and k % group == 0 else 0
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, ng), dtype=torch.float32, device=dev)
    zeros = None if symmetric else torch.empty((n, ng), dtype=torch.float32, device=dev)
    s_best = torch.empty(k, dtype=torch.float32, device=dev)
    losses = torch.empty(n_grid + 1, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    _call("awq_search", _ptr(x), t, _ptr(w), n, k, int(bool(symmetric)), group, int(n_grid), _ptr(sx),
          _ptr(workspace), workspace.numel(), _ptr(s_best), _ptr(losses), _ptr(best), _ptr(codes), _ptr(scales),
          _ptr(zeros), _stream())
    return AwqResult(PackedWeight(codes, scales, zeros, n, k, 4, bool(symmetric), group), s_best, losses, best,
                     int(n_grid))


@dataclass
class MxWeight:
    """Output of mxfp4_quantize: E2M1 codes [n][k/2] and E8M0 block scales [n][k/32]."""
    codes: torch.Tensor
    scales: torch.Tensor
    n: int
    k: int

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel()


def mxfp4_quantize(w: torch.Tensor, out: Optional[MxWeight] = None) -> MxWeight:
    """MXFP4 of bf16 W[n][k]: blocks of 32 along k (see libquant.h)."""
    _need(w, "w", torch.bfloat16)
    n, k = w.shape
    if out is None:
        out = MxWeight(torch.empty((n, k // 2), dtype=torch.uint8, device=w.device),
                       torch.empty((n, k // 32), dtype=torch.uint8, device=w.device), n, k)
    _call("mxfp4_quantize", _ptr(w), n, k, _ptr(out.codes), _ptr(out.scales), _stream())
    return out


def mxfp4_gemv(x: torch.Tensor, mw: MxWeight, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b][n] = x[b][k] W_hat^T on MXFP4 weights, b <= 16 (fp32 out)."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    if k != mw.k:
        raise ValueError(f"x has {k} columns, weights have k = {mw.k}")
    if y is None:
        y = torch.empty((m, mw.n), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, mw.n))
    _call("mxfp4_gemv", _ptr(x), m, _ptr(mw.codes), _ptr(mw.scales), mw.n, mw.k, _ptr(y), _stream())
    return y


def mxfp4_gemm(x: torch.Tensor, mw: MxWeight, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W^T with MXFP4 weights, x bf16 [m][k], any m (prefill)."""
    _need(x, "x", torch.bfloat16)
    m, k = x.shape
    if k != mw.k:
        raise ValueError(f"x has {k} columns, weights have k = {mw.k}")
    if y is None:
        y = torch.empty((m, mw.n), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, mw.n))
    _call("mxfp4_gemm", _ptr(x), m, _ptr(mw.codes), _ptr(mw.scales), mw.n, mw.k, _ptr(y), _stream())
    return y


def _gptq_workspace(t: int, n: int, k: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    need = load_library().gptq_workspace_bytes(t, n, k)
    if need < 0:
        raise LibquantError(LQ_ERR_INVALID_ARG, "gptq", "sizes out of range")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8)
    return workspace


def gptq_hessian_factor(x: torch.Tensor, percdamp: float = 0.01, u: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """U (fp32 [k][k], upper) with U^T U = (2 X^T X + damping)^-1, X [t][k] bf16."""
    _need(x, "x", torch.bfloat16)
    t, k = x.shape
    if u is None:
        u = torch.empty((k, k), dtype=torch.float32, device=x.device)
    _need(u, "u", torch.float32, (k, k))
    ws = _gptq_workspace(t, 0, k, x.device, workspace)
    _call("gptq_hessian_factor", _ptr(x), t, k, float(percdamp), _ptr(ws), ws.numel(), _ptr(u), _stream())
    return u


def gptq_quantize(w: torch.Tensor, u: torch.Tensor, bits: int = 4, symmetric: bool = False, group: int = 128,
                  workspace: Optional[torch.Tensor] = None) -> PackedWeight:
    """GPTQ's column loop on bf16 W[n][k] with the factor U -> a PackedWeight
    laid out as quantize_groupwise's."""
    _need(w, "w", torch.bfloat16)
    n, k = w.shape
    _need(u, "u", torch.float32, (k, k))
    dev = w.device
    ng = k // group if group > 0 and k % group == 0 else 0
    codes = torch.empty((n, k // 2 if bits == 4 else k), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, ng), dtype=torch.float32, device=dev)
    zeros = None if symmetric else torch.empty((n, ng), dtype=torch.float32, device=dev)
    ws = _gptq_workspace(0, n, k, dev, workspace)
    _call("gptq_quantize", _ptr(w), n, k, _ptr(u), bits, int(bool(symmetric)), group, _ptr(ws), ws.numel(),
          _ptr(codes), _ptr(scales), _ptr(zeros), _stream())
    return PackedWeight(codes, scales, zeros, n, k, bits, bool(symmetric), group)


def hbm_read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Streaming read of the whole (contiguous, 16-byte aligned) tensor with
    the library's read-probe kernel; returns the sink it may write."""
    lib = load_library()
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(lib.lq_read_probe_sink_words(), dtype=torch.int32, device=buf.device)
    _call("lq_hbm_read_probe", _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream())
    return sink


def gptq_quantize_noalloc(w: torch.Tensor, u: torch.Tensor, bits: int = 4, symmetric: bool = False,
                          group: int = 128, out: Optional[PackedWeight] = None) -> PackedWeight:
    """gptq_quantize through the entry point without a workspace (its scratch
    is the library's static device array). Outputs are allocated here when
    not given; the C call itself allocates nothing."""
    _need(w, "w", torch.bfloat16)
    n, k = w.shape
    _need(u, "u", torch.float32, (k, k))
    if out is None:
        dev = w.device
        ng = k // group if group > 0 and k % group == 0 else 0
        codes = torch.empty((n, k // 2 if bits == 4 else k), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, ng), dtype=torch.float32, device=dev)
        zeros = None if symmetric else torch.empty((n, ng), dtype=torch.float32, device=dev)
        out = PackedWeight(codes, scales, zeros, n, k, bits, bool(symmetric), group)
    _call("gptq_quantize_noalloc", _ptr(w), n, k, _ptr(u), bits, int(bool(symmetric)), group, _ptr(out.codes),
          _ptr(out.scales), _ptr(out.zeros), _stream())
    return out
