"""CPU oracle for group-wise RTN quantization, W4A16/W8A16 matmul and SmoothQuant W8A8.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It is the
independent checker of the HIP library and shares no code with it: the
arithmetic lives in ``oracle.c`` (plain scalar C, fp32 IEEE encoding, fp64
accumulation), which this module compiles with gcc and calls through ctypes.

Every function takes and returns numpy arrays. Weights and activations are
passed as bf16 bit patterns (``uint16``) or as ``float32``.

Parity status of each function (what pins it; the tests under ``tests/``
hold the pins):

* ``quantize`` / ``dequantize``: the worked INT4 example and the INT8
  self-test of the "3.6 Quantization" page, the outlier collapse from its
  "Intuition" section, brute-force nearest-code search on tiny inputs, the
  s/2 error bound, and the constructed half-way ties.
* ``w4a16_matmul`` / ``w8a16_matmul``: the definition y = x W_hat^T,
  checked against numpy's matmul on the dequantized weights and against
  closed forms.
* ``smooth_scale``: the self-test (max|X| = 100, max|W| = 0.01 gives s = 100)
  and the equalised maxima sqrt(max|X| max|W|) of the SmoothQuant section.
* ``quant_per_token_int8`` / ``w8a8_gemm``: brute force, an int64 numpy
  matmul of the codes, the exactness of the smoothing identity and the toy
  error ratio of the code block.
* ``effective_bits`` / ``packed_bytes``: the printed effective-bit values.
* ``mx_quantize`` / ``mx_dequantize`` / ``mx_matmul``: the pages' E2M1
  magnitude table and block size, exact round trips of representable
  blocks, constructed ties, brute-force nearest-value search, the scale
  rule at its boundaries, and numpy's matmul on the dequantized weights.
* ``gptq_hessian`` / ``gptq_inverse_factor`` / ``gptq_quantize``: numpy's
  2 X^T X and inverse, the reduction to plain RTN when H is a multiple of
  the identity, an independent fp64 numpy implementation of the pages'
  update formula with explicit inverses of the remaining submatrix, and the
  pages' claim that the compensation lowers the output error versus RTN.
* ``act_absmean`` / ``awq_scale`` / ``awq_loss`` / ``awq_search``: numpy
  recomputations of the channel means and of the output error from the
  pinned quantizer, the reduction to plain RTN at alpha = 0, and the pages'
  claims (scaling a channel by s shrinks its rounding error about 1/s; the
  search beats plain RTN when activations have outlier channels).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at a deliberately broken copy of the oracle
# (a planted mistake, CPU only) to show the pins catch it.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        lib.oracle_quantize_f32.argtypes = [P, I64, I64, I, I, I64, P, P, P, P]
        lib.oracle_quantize_bf16.argtypes = [P, I64, I64, I, I, I64, P, P, P, P]
        lib.oracle_dequantize.argtypes = [P, P, P, I64, I64, I, I, I64, P]
        lib.oracle_w4a16_matmul.argtypes = [P, I64, P, P, P, I64, I64, I, I64, P]
        lib.oracle_weight_only_matmul.argtypes = [P, I64, P, P, P, I64, I64, I, I, I64, P]
        lib.oracle_act_absmean.argtypes = [P, I64, I64, P]
        lib.oracle_mx_exponent.argtypes = [F]
        lib.oracle_gptq_hessian.argtypes = [P, I64, I64, P]
        lib.oracle_gptq_inverse_factor.argtypes = [P, I64, ctypes.c_double, P]
        lib.oracle_gptq_quantize.argtypes = [P, I64, I64, P, I, I, I64, P, P, P]
        lib.oracle_mx_quantize.argtypes = [P, I64, I64, P, P]
        lib.oracle_mx_dequantize.argtypes = [P, P, I64, I64, P]
        lib.oracle_mx_matmul.argtypes = [P, I64, P, P, I64, I64, P]
        lib.oracle_awq_scale.argtypes = [P, I64, I, I, P]
        lib.oracle_awq_scale.restype = None
        lib.oracle_awq_loss.argtypes = [P, I64, P, I64, I64, I, I, I64, P, P]
        lib.oracle_awq_search.argtypes = [P, I64, P, I64, I64, I, I, I64, I, P, P, P, P]
        lib.oracle_smooth_scale_from_absmax.argtypes = [P, P, I64, F, P]
        lib.oracle_smooth_scale_from_absmax.restype = None
        lib.oracle_smooth_scale.argtypes = [P, I64, P, I64, I64, F, P]
        lib.oracle_quant_per_token_int8_f32.argtypes = [P, I64, I64, P, P, P]
        lib.oracle_quant_per_token_int8.argtypes = [P, I64, I64, P, P, P]
        lib.oracle_w8a8_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P]
        lib.oracle_effective_bits.argtypes = [I, I, I, I64]
        lib.oracle_effective_bits.restype = ctypes.c_double
        lib.oracle_packed_bytes.argtypes = [I64, I64, I, I, I64]
        lib.oracle_packed_bytes.restype = ctypes.c_int64
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def quantize(w, bits: int, symmetric: bool, group: int, col_scale=None):
    """Group-wise RTN quantization of w[n][k] along k.

    ``w`` is uint16 (bf16 bits) or float32. Returns (codes uint8 [n][k/2] for
    bits 4 or [n][k] for bits 8, scales fp32 [n][k/group], zeros fp32
    [n][k/group] or None for symmetric). INT8 symmetric codes are int8 bit
    patterns stored in uint8.
    """
    lib = _load()
    n, k = w.shape
    if group <= 0 or k % group:
        raise ValueError("k must be a multiple of group")
    codes = np.zeros((n, k // 2 if bits == 4 else k), np.uint8)
    scales = np.zeros((n, k // group), np.float32)
    zeros = None if symmetric else np.zeros((n, k // group), np.float32)
    cs = None if col_scale is None else _c(col_scale, np.float32)
    if w.dtype == np.uint16:
        fn, wc = lib.oracle_quantize_bf16, _c(w, np.uint16)
    else:
        fn, wc = lib.oracle_quantize_f32, _c(w, np.float32)
    rc = fn(_ptr(wc), n, k, bits, int(bool(symmetric)), group, _ptr(cs), _ptr(codes),
            _ptr(scales), _ptr(zeros))
    _check(rc, "quantize")
    return codes, scales, zeros


def dequantize(codes, scales, zeros, n: int, k: int, bits: int, symmetric: bool, group: int):
    """x_hat = fl((q - z) * s) in fp32, [n][k]."""
    lib = _load()
    out = np.zeros((n, k), np.float32)
    zc = None if symmetric else _c(zeros, np.float32)
    rc = lib.oracle_dequantize(_ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.float32)), _ptr(zc),
                               n, k, bits, int(bool(symmetric)), group, _ptr(out))
    _check(rc, "dequantize")
    return out


def w4a16_matmul(x_bf16, codes, scales, zeros, n: int, k: int, symmetric: bool, group: int):
    """y[m][n] = sum_k x[m][k] * x_hat[n][k] in fp64; x is uint16 bf16 bits [m][k]."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    zc = None if symmetric else _c(zeros, np.float32)
    rc = lib.oracle_w4a16_matmul(_ptr(x), m, _ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.float32)),
                                 _ptr(zc), n, k, int(bool(symmetric)), group, _ptr(y))
    _check(rc, "w4a16_matmul")
    return y


def w8a16_matmul(x_bf16, codes, scales, zeros, n: int, k: int, symmetric: bool, group: int):
    """W8A16: y[m][n] = sum_k x[m][k] * x_hat[n][k] in fp64 on INT8 codes [n][k]."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    zc = None if symmetric else _c(zeros, np.float32)
    rc = lib.oracle_weight_only_matmul(_ptr(x), m, _ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.float32)),
                                       _ptr(zc), n, k, 8, int(bool(symmetric)), group, _ptr(y))
    _check(rc, "w8a16_matmul")
    return y


def smooth_scale_from_absmax(ax, aw, alpha: float):
    lib = _load()
    ax = _c(ax, np.float32)
    aw = _c(aw, np.float32)
    s = np.zeros(ax.shape[0], np.float32)
    lib.oracle_smooth_scale_from_absmax(_ptr(ax), _ptr(aw), ax.shape[0], alpha, _ptr(s))
    return s


def smooth_scale(x_bf16, w_bf16, alpha: float):
    """s[k] from bf16 X[t][k] and W[n][k]."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    t, k = x.shape
    n = w.shape[0]
    s = np.zeros(k, np.float32)
    rc = lib.oracle_smooth_scale(_ptr(x), t, _ptr(w), n, k, alpha, _ptr(s))
    _check(rc, "smooth_scale")
    return s


def quant_per_token_int8(x, smooth=None):
    """Per-token symmetric INT8 of X / smooth. x is uint16 (bf16 bits) or float32 [t][k]."""
    lib = _load()
    t, k = x.shape
    qx = np.zeros((t, k), np.int8)
    sx = np.zeros(t, np.float32)
    sm = None if smooth is None else _c(smooth, np.float32)
    if x.dtype == np.uint16:
        rc = lib.oracle_quant_per_token_int8(_ptr(_c(x, np.uint16)), t, k, _ptr(sm), _ptr(qx), _ptr(sx))
    else:
        rc = lib.oracle_quant_per_token_int8_f32(_ptr(_c(x, np.float32)), t, k, _ptr(sm), _ptr(qx),
                                                 _ptr(sx))
    _check(rc, "quant_per_token_int8")
    return qx, sx


def w8a8_gemm(qx, sx, qw, sw):
    """acc int32 [m][n] and y fp64 [m][n] from int8 codes and fp32 scales."""
    lib = _load()
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    m, k = qx.shape
    n = qw.shape[0]
    acc = np.zeros((m, n), np.int32)
    y = np.zeros((m, n), np.float64)
    rc = lib.oracle_w8a8_gemm(_ptr(qx), _ptr(_c(sx, np.float32)), m, _ptr(qw), _ptr(_c(sw, np.float32)),
                              n, k, _ptr(acc), _ptr(y))
    _check(rc, "w8a8_gemm")
    return acc, y


def effective_bits(bits: int, scale_bits: int, zero_bits: int, group: int) -> float:
    return _load().oracle_effective_bits(bits, scale_bits, zero_bits, group)


def packed_bytes(n: int, k: int, bits: int, symmetric: bool, group: int) -> int:
    return _load().oracle_packed_bytes(n, k, bits, int(bool(symmetric)), group)


def bf16_bits_to_f32(h) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for the tests' own checks)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def act_absmean(x_bf16):
    """s_X[k] = mean_t |X[t][k]| (fp64 sum, one fp32 rounding); x: bf16 bits [t][k]."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    t, k = x.shape
    sx = np.zeros(k, np.float32)
    _check(lib.oracle_act_absmean(_ptr(x), t, k, _ptr(sx)), "act_absmean")
    return sx


def awq_scale(sx, i: int, n_grid: int):
    """Grid point i's scale: powf(max(s_X, 1e-8), i / n_grid)."""
    lib = _load()
    sx = _c(sx, np.float32)
    s = np.zeros(sx.size, np.float32)
    lib.oracle_awq_scale(_ptr(sx), sx.size, int(i), int(n_grid), _ptr(s))
    return s


def awq_loss(x_bf16, w_bf16, s, bits: int, symmetric: bool, group: int) -> float:
    """|| X W^T - bf16(X / s) quant(W diag(s))^T ||_F^2 in fp64."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    t, k = x.shape
    n = w.shape[0]
    out = np.zeros(1, np.float64)
    _check(lib.oracle_awq_loss(_ptr(x), t, _ptr(w), n, k, bits, int(bool(symmetric)), group,
                               _ptr(_c(s, np.float32)), _ptr(out)), "awq_loss")
    return float(out[0])


def awq_search(x_bf16, w_bf16, bits: int, symmetric: bool, group: int, n_grid: int):
    """AWQ grid search -> (s_X [k], losses [n_grid + 1], best index, s_best [k])."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    t, k = x.shape
    n = w.shape[0]
    sx = np.zeros(k, np.float32)
    losses = np.zeros(n_grid + 1, np.float64)
    best = np.zeros(1, np.int32)
    s_best = np.zeros(k, np.float32)
    _check(lib.oracle_awq_search(_ptr(x), t, _ptr(w), n, k, bits, int(bool(symmetric)), group, int(n_grid),
                                 _ptr(sx), _ptr(losses), _ptr(best), _ptr(s_best)), "awq_search")
    return sx, losses, int(best[0]), s_best


def mx_exponent(amax: float) -> int:
    """Shared MXFP4 exponent e of a block whose largest magnitude is amax."""
    return int(_load().oracle_mx_exponent(float(amax)))


def mx_quantize(w_bf16):
    """MXFP4 of bf16 w[n][k] -> (codes uint8 [n][k/2], scales uint8 E8M0 [n][k/32])."""
    lib = _load()
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 32), np.uint8)
    _check(lib.oracle_mx_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales)), "mx_quantize")
    return codes, scales


def mx_dequantize(codes, scales, n: int, k: int):
    lib = _load()
    out = np.zeros((n, k), np.float32)
    _check(lib.oracle_mx_dequantize(_ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.uint8)), n, k, _ptr(out)),
           "mx_dequantize")
    return out


def mx_matmul(x_bf16, codes, scales, n: int, k: int):
    """y[m][n] = sum_k x[m][k] * x_hat[n][k] in fp64 on MXFP4 weights."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    _check(lib.oracle_mx_matmul(_ptr(x), m, _ptr(_c(codes, np.uint8)), _ptr(_c(scales, np.uint8)), n, k, _ptr(y)),
           "mx_matmul")
    return y


def gptq_hessian(x_bf16):
    """H = 2 X^T X in fp64; x: bf16 bits [t][k]."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    t, k = x.shape
    h = np.zeros((k, k), np.float64)
    _check(lib.oracle_gptq_hessian(_ptr(x), t, k, _ptr(h)), "gptq_hessian")
    return h


def gptq_inverse_factor(h, percdamp: float = 0.01):
    """Damp H, then U (fp32, upper) with U^T U = H_damped^-1. Returns (H_damped, U)."""
    lib = _load()
    h = np.array(h, np.float64, copy=True, order="C")
    k = h.shape[0]
    u = np.zeros((k, k), np.float32)
    _check(lib.oracle_gptq_inverse_factor(_ptr(h), k, float(percdamp), _ptr(u)), "gptq_inverse_factor")
    return h, u


def gptq_quantize(w_bf16, u, bits: int, symmetric: bool, group: int):
    """The GPTQ column loop given U -> (codes, scales, zeros) as quantize() lays them out."""
    lib = _load()
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    ng = k // group
    codes = np.zeros((n, k // 2 if bits == 4 else k), np.uint8)
    scales = np.zeros((n, ng), np.float32)
    zeros = None if symmetric else np.zeros((n, ng), np.float32)
    _check(lib.oracle_gptq_quantize(_ptr(w), n, k, _ptr(_c(u, np.float32)), bits, int(bool(symmetric)), group,
                                    _ptr(codes), _ptr(scales), _ptr(zeros)), "gptq_quantize")
    return codes, scales, zeros
