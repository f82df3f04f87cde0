"""Plain CPU oracle for the BitNet b1.58 BitLinear (W1.58A8) path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The
product library (the HIP kernels behind the C ABI and its Python binding)
never imports, links or calls anything here, and this package imports
nothing from the product.

The arithmetic lives in ``bitlinear_oracle.c`` (plain C, one IEEE binary32
rounding per operation, exact sums where the pages leave the order open).
This module only marshals numpy arrays through ctypes.

Pins (checks against facts other than the oracle itself) live in
``tests/test_oracle_pins.py``.  Every function here is pinned; none is
"parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

EPS = np.float32(1e-5)
Q = 127


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    lib.orc_abs_sum_exact.argtypes = [P, I64]
    lib.orc_abs_sum_exact.restype = ctypes.c_double
    lib.orc_sq_sum_exact.argtypes = [P, I64]
    lib.orc_sq_sum_exact.restype = ctypes.c_double
    lib.orc_weight_scale.argtypes = [P, I64]
    lib.orc_weight_scale.restype = F
    lib.orc_ternarize.argtypes = [P, I64, F, P]
    lib.orc_binarize.argtypes = [P, I64, P]
    lib.orc_padded_k.argtypes = [I64]
    lib.orc_padded_k.restype = I64
    lib.orc_pack.argtypes = [P, I64, I64, P]
    lib.orc_unpack.argtypes = [P, I64, I64, P]
    lib.orc_unpack.restype = I64
    lib.orc_padded_k1.argtypes = [I64]
    lib.orc_padded_k1.restype = I64
    lib.orc_pack1.argtypes = [P, I64, I64, P]
    lib.orc_pack1.restype = I64
    lib.orc_unpack1.argtypes = [P, I64, I64, P]
    lib.orc_unpack1.restype = I64
    lib.orc_act_quant.argtypes = [P, I64, I64, P, P, P]
    lib.orc_act_quant_a48.argtypes = [P, I64, I64, I64, P, P, P, P, P, P, P]
    lib.orc_dequant_a48.argtypes = [P, P, P, P, F, I64, I64, P]
    lib.orc_int_linear.argtypes = [P, P, I64, I64, I64, P]
    lib.orc_dequant.argtypes = [P, P, F, I64, I64, P]
    lib.orc_rmsnorm.argtypes = [P, P, F, I64, I64, P]
    lib.orc_relu2_mul.argtypes = [P, P, I64, P]
    lib.orc_ffn.argtypes = [P, I64, I64, I64, P, F, P, F, P, F, P, F, ctypes.c_int, P, F,
                            P, P, P, P, P, P, P, P]
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def abs_sum_exact(w):
    """Exact sum of |w| rounded once to binary64."""
    w = _f32(w).reshape(-1)
    return _load().orc_abs_sum_exact(_ptr(w), w.size)


def sq_sum_exact(x):
    """Exact sum of x**2 rounded once to binary64."""
    x = _f32(x).reshape(-1)
    return _load().orc_sq_sum_exact(_ptr(x), x.size)


def weight_scale(w):
    """Absmean scale gamma_w of a whole weight tensor (binary32)."""
    w = _f32(w).reshape(-1)
    return np.float32(_load().orc_weight_scale(_ptr(w), w.size))


def ternarize(w, gamma):
    """clamp(round(w / (gamma + 1e-5)), -1, 1) as int8, same shape as w."""
    w = _f32(w)
    t = np.empty(w.shape, dtype=np.int8)
    _load().orc_ternarize(_ptr(w), w.size, float(np.float32(gamma)), _ptr(t))
    return t


def binarize(w):
    """+1 where w >= 0 else -1, as int8."""
    w = _f32(w)
    t = np.empty(w.shape, dtype=np.int8)
    _load().orc_binarize(_ptr(w), w.size, _ptr(t))
    return t


def padded_k(K):
    return int(_load().orc_padded_k(int(K)))


def pack(t):
    """Pack an int8 ternary matrix [N, K] into uint32 words [N, padded_k(K)//16]."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    out = np.empty((N, padded_k(K) // 16), dtype=np.uint32)
    _load().orc_pack(_ptr(t), N, K, _ptr(out))
    return out


def unpack(packed, K):
    """Inverse of pack.  Returns (t [N, K] int8, number of invalid fields)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    N = packed.shape[0]
    assert packed.shape[1] == padded_k(K) // 16
    t = np.zeros((N, K), dtype=np.int8)
    bad = _load().orc_unpack(_ptr(packed), N, K, _ptr(t))
    return t, int(bad)


def padded_k1(K):
    return int(_load().orc_padded_k1(int(K)))


def pack1(t):
    """Pack an int8 binary matrix [N, K] (values -1/+1) into the 1-bit layout,
    uint32 words [N, padded_k1(K)//32].  Raises on other values."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    out = np.empty((N, padded_k1(K) // 32), dtype=np.uint32)
    bad = _load().orc_pack1(_ptr(t), N, K, _ptr(out))
    if bad:
        raise ValueError(f"pack1: {bad} values other than -1/+1")
    return out


def unpack1(packed, K):
    """Inverse of pack1.  Returns (t [N, K] int8, number of set padding bits)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    N = packed.shape[0]
    assert packed.shape[1] == padded_k1(K) // 32
    t = np.zeros((N, K), dtype=np.int8)
    bad = _load().orc_unpack1(_ptr(packed), N, K, _ptr(t))
    return t, int(bad)


def quantize_weights(w, mode="ternary"):
    """Weight scale, unpacked codes and packed words of a [N, K] tensor."""
    w = _f32(w)
    g = weight_scale(w)
    t = ternarize(w, g) if mode == "ternary" else binarize(w)
    return g, t, pack(t)


def act_quant(x):
    """Per-token absmax int8 quantisation of x [M, K].

    Returns (q int8 [M, K], gamma float32 [M], rowsum int32 [M])."""
    x = _f32(x)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    g = np.empty(M, dtype=np.float32)
    rs = np.empty(M, dtype=np.int32)
    _load().orc_act_quant(_ptr(x), M, K, _ptr(q), _ptr(g), _ptr(rs))
    return q, g, rs


def act_quant_a48(x, n_out):
    """BitNet a4.8 split quantisation of x [M, K]: the n_out largest |x| per
    row (ties to the lower index) in int8, the rest in int4 ([-7, 7]).

    Returns dict q4, g4, rs4, q8, g8, rs8, outlier (uint8 mask)."""
    x = _f32(x)
    M, K = x.shape
    r = {"q4": np.empty((M, K), np.int8), "g4": np.empty(M, np.float32),
         "rs4": np.empty(M, np.int32), "q8": np.empty((M, K), np.int8),
         "g8": np.empty(M, np.float32), "rs8": np.empty(M, np.int32),
         "outlier": np.empty((M, K), np.uint8)}
    _load().orc_act_quant_a48(_ptr(x), M, K, int(n_out), _ptr(r["q4"]), _ptr(r["g4"]),
                              _ptr(r["rs4"]), _ptr(r["q8"]), _ptr(r["g8"]), _ptr(r["rs8"]),
                              _ptr(r["outlier"]))
    return r


def dequant_a48(acc4, g4, acc8, g8, gamma_w):
    acc4 = np.ascontiguousarray(acc4, dtype=np.int32)
    acc8 = np.ascontiguousarray(acc8, dtype=np.int32)
    M, N = acc4.shape
    y = np.empty((M, N), dtype=np.float32)
    _load().orc_dequant_a48(_ptr(acc4), _ptr(_f32(g4).reshape(-1)), _ptr(acc8),
                            _ptr(_f32(g8).reshape(-1)), float(np.float32(gamma_w)), M, N, _ptr(y))
    return y


def bitlinear_a48(x, t, gamma_w, n_out):
    """BitLinear with a4.8 activations: returns the quantiser's outputs, both
    accumulators and y."""
    r = act_quant_a48(x, n_out)
    r["acc4"] = int_linear(r["q4"], t)
    r["acc8"] = int_linear(r["q8"], t)
    r["y"] = dequant_a48(r["acc4"], r["g4"], r["acc8"], r["g8"], gamma_w)
    return r


def int_linear(q, t):
    """acc[m, n] = sum_k q[m, k] * t[n, k] (int32)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    t = np.ascontiguousarray(t, dtype=np.int8)
    M, K = q.shape
    N, K2 = t.shape
    assert K == K2
    acc = np.empty((M, N), dtype=np.int32)
    _load().orc_int_linear(_ptr(q), _ptr(t), M, N, K, _ptr(acc))
    return acc


def dequant(acc, gamma_x, gamma_w):
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    gx = _f32(gamma_x).reshape(-1)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float32)
    _load().orc_dequant(_ptr(acc), _ptr(gx), float(np.float32(gamma_w)), M, N, _ptr(y))
    return y


def rmsnorm(x, g=None, eps=float(np.finfo(np.float32).eps)):
    x = _f32(x)
    M, D = x.shape
    gg = _f32(g) if g is not None else None
    y = np.empty((M, D), dtype=np.float32)
    _load().orc_rmsnorm(_ptr(x), _ptr(gg), float(np.float32(eps)), M, D, _ptr(y))
    return y


def relu2_mul(g, u):
    g = _f32(g)
    u = _f32(u)
    h = np.empty(g.shape, dtype=np.float32)
    _load().orc_relu2_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def bitlinear(x, t, gamma_w):
    """Full BitLinear from float activations: returns dict of all internals."""
    q, gx, rs = act_quant(x)
    acc = int_linear(q, t)
    y = dequant(acc, gx, gamma_w)
    return {"q": q, "gamma_x": gx, "rowsum": rs, "acc": acc, "y": y}


def ffn(x, norm_w, norm_eps, tg, sg, tu, su, td, sd, subln=False, subln_w=None,
        subln_eps=float(np.finfo(np.float32).eps)):
    """RMSNorm -> quant -> gate/up -> relu(gate)^2*up -> [RMSNorm if subln] ->
    requant -> down."""
    x = _f32(x)
    M, D = x.shape
    F = tg.shape[0]
    assert tg.shape == (F, D) and tu.shape == (F, D) and td.shape == (D, F)
    nw = _f32(norm_w) if norm_w is not None else None
    sw = _f32(subln_w) if subln_w is not None else None
    out = {
        "xn": np.empty((M, D), np.float32), "qx": np.empty((M, D), np.int8),
        "gx": np.empty(M, np.float32), "h": np.empty((M, F), np.float32),
        "hn": np.empty((M, F), np.float32),
        "qh": np.empty((M, F), np.int8), "gh": np.empty(M, np.float32),
        "y": np.empty((M, D), np.float32),
    }
    c = lambda a: np.ascontiguousarray(a, dtype=np.int8)
    tg, tu, td = c(tg), c(tu), c(td)
    _load().orc_ffn(_ptr(x), M, D, F, _ptr(nw), float(np.float32(norm_eps)),
                    _ptr(tg), float(np.float32(sg)), _ptr(tu), float(np.float32(su)),
                    _ptr(td), float(np.float32(sd)),
                    1 if subln else 0, _ptr(sw), float(np.float32(subln_eps)),
                    _ptr(out["xn"]), _ptr(out["qx"]), _ptr(out["gx"]), _ptr(out["h"]),
                    _ptr(out["hn"]), _ptr(out["qh"]), _ptr(out["gh"]), _ptr(out["y"]))
    if not subln:
        del out["hn"]
    return out


def num_threads():
    return int(_load().orc_num_threads())
