"""Thin ctypes binding over libbitlinear.so (declared in include/bitlinear.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory (output tensors are allocated with
torch on the input's device) and the current stream.  There is no fallback:
if the library is missing, or a tensor is not on a GPU, a call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BL_OK, BL_EINVAL, BL_ESHAPE, BL_EALIGN, BL_EWORKSPACE, BL_EHIP = range(6)
BL_TERNARY, BL_BINARY, BL_BINARY_1BIT = 0, 1, 2
BL_F32, BL_BF16 = 0, 1
BL_KERNEL_AUTO, BL_KERNEL_GEMV, BL_KERNEL_SKINNY, BL_KERNEL_TILED = range(4)
FFN_WS_NAMES = ("XN", "QX", "GX", "RSX", "H", "HN", "GH", "QH", "RSH", "GHP")

_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m ternary_weight_linear_ternarize_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    L.bl_padded_k.argtypes = [I64]
    L.bl_padded_k.restype = I64
    L.bl_packed_bytes.argtypes = [I64, I64]
    L.bl_packed_bytes.restype = SZ
    L.bl_padded_k_1bit.argtypes = [I64]
    L.bl_padded_k_1bit.restype = I64
    L.bl_packed_bytes_1bit.argtypes = [I64, I64]
    L.bl_packed_bytes_1bit.restype = SZ
    L.bl_pack_workspace_bytes.argtypes = [I64, I64]
    L.bl_pack_workspace_bytes.restype = SZ
    L.bl_status_str.argtypes = [I]
    L.bl_status_str.restype = ctypes.c_char_p
    L.bitlinear_pack.argtypes = [P, I64, I64, I, P, P, P, SZ, P]
    L.bitlinear_pack.restype = I
    L.bitlinear_quant_act.argtypes = [P, I, I64, I64, P, P, P, P]
    L.bitlinear_quant_act.restype = I
    L.bitlinear_forward.argtypes = [P, P, P, I64, I64, P, P, I64, P, P, P]
    L.bitlinear_forward.restype = I
    L.bitlinear_forward_1bit.argtypes = [P, P, P, I64, I64, P, P, I64, P, P, P]
    L.bitlinear_forward_1bit.restype = I
    L.bitlinear_quant_act_a48.argtypes = [P, I, I64, I64, I64, P, P, P, P, P, P, P]
    L.bitlinear_quant_act_a48.restype = I
    L.bitlinear_a48_workspace_bytes.argtypes = [I64, I64]
    L.bitlinear_a48_workspace_bytes.restype = SZ
    L.bitlinear_forward_a48.argtypes = [P, P, P, P, P, P, I64, I64, P, P, I64, P, P, SZ, P]
    L.bitlinear_forward_a48.restype = I
    L.bitlinear_forward_kernel.argtypes = [P, P, P, I64, I64, P, P, I64, P, P, I, P]
    L.bitlinear_forward_kernel.restype = I
    L.bitlinear_fused_workspace_bytes.argtypes = [I64, I64]
    L.bitlinear_fused_workspace_bytes.restype = SZ
    L.bitlinear_fused_workspace_offset.argtypes = [I64, I64, I]
    L.bitlinear_fused_workspace_offset.restype = SZ
    L.bitlinear_forward_fused.argtypes = [P, I, I64, I64, P, P, I64, P, P, SZ, P]
    L.bitlinear_forward_fused.restype = I
    L.bitlinear_fused_norm_workspace_bytes.argtypes = [I64, I64]
    L.bitlinear_fused_norm_workspace_bytes.restype = SZ
    L.bitlinear_forward_fused_norm.argtypes = [P, I, I64, I64, P, F, P, P, I64, P, P, SZ, P]
    L.bitlinear_forward_fused_norm.restype = I
    L.bitnet_ffn_workspace_layout.argtypes = [I64, I64, I64, P]
    L.bitnet_ffn_workspace_layout.restype = SZ
    L.bitnet_ffn_workspace_bytes.argtypes = [I64, I64, I64]
    L.bitnet_ffn_workspace_bytes.restype = SZ
    L.bitnet_ffn_forward.argtypes = [P, I, I64, I64, I64, P, F, P, F, P, P, P, P, P, P, P, P, SZ,
                                     P]
    L.bitnet_ffn_forward.restype = I
    L.bitnet_ffn_forward_static.argtypes = [P, I, I64, I64, I64, P, F, P, F, P, P, P, P, P, P,
                                            P, P]
    L.bitnet_ffn_forward_static.restype = I
    L.bl_probe_read.argtypes = [P, SZ, I, P, P]
    L.bl_probe_read.restype = I
    L.bl_probe_empty.argtypes = [P]
    L.bl_probe_empty.restype = I
    _lib = L
    return L


def status_str(status):
    return lib().bl_status_str(int(status)).decode()


def _check(status, where):
    if status != BL_OK:
        raise BitLinearError(status, where)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_WORDS = (torch.int32, torch.uint32)


def _expect(t, name, shape=None, dtypes=None, min_bytes=None):
    """Checks a tensor's type, shape and size before its pointer reaches the
    library: the kernels trust the sizes they are given, so a mismatch here
    would read or write past an allocation."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, "
                         f"got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} must hold at least {min_bytes} bytes, "
                         f"got {t.numel() * t.element_size()}")
    return t


def _same_device(*ts):
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def padded_k(K):
    return int(lib().bl_padded_k(int(K)))


def ffn_workspace_layout(M, D, F):
    off = (ctypes.c_size_t * len(FFN_WS_NAMES))()
    total = lib().bitnet_ffn_workspace_layout(int(M), int(D), int(F), off)
    return int(total), {n: int(off[i]) for i, n in enumerate(FFN_WS_NAMES)}


def _matrix(X, name):
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return X.shape


def _check_codes(Xq, xs, rs, M, K, tag):
    """int8 codes [M, Kp], scales [M] float32, row sums [M] int32."""
    _expect(Xq, f"Xq{tag}", (M, padded_k(K)), (torch.int8,))
    _expect(xs, f"x{tag}_scale", (M,), (torch.float32,))
    _expect(rs, f"x{tag}_rowsum", (M,), (torch.int32,))


def _check_out(Y, acc, M, N):
    _expect(Y, "Y", (M, N), (torch.float32,))
    if acc is not None:
        _expect(acc, "acc_out", (M, N), (torch.int32,))


def _check_weights(Wp, w_scale, N, K, one_bit=False, name="Wp"):
    words = lib().bl_padded_k_1bit(K) // 32 if one_bit else padded_k(K) // 16
    _expect(Wp, name, (N, words), _WORDS)
    _expect(w_scale, "w_scale", None, (torch.float32,))
    if w_scale.numel() < 1:
        raise ValueError("w_scale must hold one float")


def _codes_k(Xq, K):
    if not isinstance(Xq, torch.Tensor) or Xq.dim() != 2:
        raise ValueError("Xq must be a 2-D tensor [M, Kp]")
    if int(K) < 1 or Xq.shape[1] != padded_k(K):
        raise ValueError(f"Xq has {Xq.shape[1]} columns; K = {K} needs {padded_k(K) if K > 0 else '?'}")
    return Xq.shape[0]


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)

def bitlinear_pack(W, mode=BL_TERNARY, out=None, scale=None, ws=None):
    """Quantise and pack W [N, K] float32 -> (Wp uint32 [N, Kp/16] as int32, w_scale [1]);
    with mode BL_BINARY_1BIT the words are [N, Kb/32] (1-bit layout)."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor [N, K]")
    _expect(W, "W", dtypes=(torch.float32,))
    N, K = W.shape
    dev = W.device
    words = lib().bl_padded_k_1bit(K) // 32 if mode == BL_BINARY_1BIT else padded_k(K) // 16
    Wp = out if out is not None else torch.empty((N, words), dtype=torch.int32, device=dev)
    sc = scale if scale is not None else torch.empty(1, dtype=torch.float32, device=dev)
    nws = lib().bl_pack_workspace_bytes(N, K)
    ws = ws if ws is not None else torch.empty(nws, dtype=torch.uint8, device=dev)
    _expect(Wp, "Wp", (N, words), _WORDS)
    _expect(sc, "w_scale", (1,), (torch.float32,))
    _expect(ws, "ws", min_bytes=nws)
    _same_device(W, Wp, sc, ws)
    st = lib().bitlinear_pack(_dev(W, "W"), N, K, int(mode), _dev(Wp, "Wp"), _dev(sc, "w_scale"),
                              _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "bitlinear_pack")
    return Wp, sc


def bitlinear_quant_act(X, out=None):
    """X [M, K] float32/bfloat16 -> (Xq int8 [M, Kp], x_scale [M], x_rowsum int32 [M])."""
    M, K = _matrix(X, "X")
    dt = _act_dtype(X)
    dev = X.device
    if out is None:
        out = (torch.empty((M, padded_k(K)), dtype=torch.int8, device=dev),
               torch.empty(M, dtype=torch.float32, device=dev),
               torch.empty(M, dtype=torch.int32, device=dev))
    Xq, xs, rs = out
    _check_codes(Xq, xs, rs, M, K, "")
    _same_device(X, Xq, xs, rs)
    st = lib().bitlinear_quant_act(_dev(X, "X"), dt, M, K, _dev(Xq, "Xq"), _dev(xs, "x_scale"),
                                   _dev(rs, "x_rowsum"), _stream(dev))
    _check(st, "bitlinear_quant_act")
    return Xq, xs, rs


def bitlinear_forward(Xq, x_scale, x_rowsum, K, Wp, w_scale, N, with_acc=False,
                      kernel=BL_KERNEL_AUTO, out=None, acc_out=None):
    """Y [M, N] float32 (and the int32 accumulators when with_acc)."""
    M = _codes_k(Xq, K)
    dev = Xq.device
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = acc_out
    if with_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check_codes(Xq, x_scale, x_rowsum, M, K, "")
    _check_weights(Wp, w_scale, N, K)
    _check_out(Y, acc, M, N)
    _same_device(Xq, x_scale, x_rowsum, Wp, w_scale, Y, acc)
    st = lib().bitlinear_forward_kernel(
        _dev(Xq, "Xq"), _dev(x_scale, "x_scale"), _dev(x_rowsum, "x_rowsum"), M, K,
        _dev(Wp, "Wp"), _dev(w_scale, "w_scale"), N, _dev(Y, "Y"), _opt(acc, "acc_out"),
        int(kernel), _stream(dev))
    _check(st, "bitlinear_forward")
    return (Y, acc) if with_acc else Y


def bitlinear_forward_1bit(Xq, x_scale, x_rowsum, K, Wb, w_scale, N, with_acc=False, out=None,
                           acc_out=None):
    """As bitlinear_forward for binary weights in the 1-bit layout."""
    M = _codes_k(Xq, K)
    dev = Xq.device
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = acc_out
    if with_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check_codes(Xq, x_scale, x_rowsum, M, K, "")
    _check_weights(Wb, w_scale, N, K, one_bit=True, name="Wb")
    _check_out(Y, acc, M, N)
    _same_device(Xq, x_scale, x_rowsum, Wb, w_scale, Y, acc)
    st = lib().bitlinear_forward_1bit(
        _dev(Xq, "Xq"), _dev(x_scale, "x_scale"), _dev(x_rowsum, "x_rowsum"), M, K,
        _dev(Wb, "Wb"), _dev(w_scale, "w_scale"), N, _dev(Y, "Y"), _opt(acc, "acc_out"),
        _stream(dev))
    _check(st, "bitlinear_forward_1bit")
    return (Y, acc) if with_acc else Y


def bitlinear_quant_act_a48(X, n_out, out=None):
    """a4.8 split quantisation of X [M, K] float32/bfloat16 -> dict of device
    tensors q4, g4, rs4, q8, g8, rs8 (codes int8 [M, Kp])."""
    M, K = _matrix(X, "X")
    dt = _act_dtype(X)
    dev = X.device
    kp = padded_k(K)
    if out is None:
        # stacked (int8 part right after the int4 part): the layout the
        # product runs in one pass for up to 8 tokens
        q = torch.empty((2, M, kp), dtype=torch.int8, device=dev)
        g = torch.empty((2, M), dtype=torch.float32, device=dev)
        r = torch.empty((2, M), dtype=torch.int32, device=dev)
        out = {"q4": q[0], "g4": g[0], "rs4": r[0], "q8": q[1], "g8": g[1], "rs8": r[1]}
    o = out
    _check_a48_codes(o, M, K)
    _same_device(X, *o.values())
    st = lib().bitlinear_quant_act_a48(
        _dev(X, "X"), dt, M, K, int(n_out), _dev(o["q4"], "Xq4"), _dev(o["g4"], "x4_scale"),
        _dev(o["rs4"], "x4_rowsum"), _dev(o["q8"], "Xq8"), _dev(o["g8"], "x8_scale"),
        _dev(o["rs8"], "x8_rowsum"), _stream(dev))
    _check(st, "bitlinear_quant_act_a48")
    return out


def bitlinear_forward_a48(q, K, Wp, w_scale, N, out=None, ws=None):
    """Y [M, N] float32 from a4.8 activations (dict of bitlinear_quant_act_a48)
    -> (Y, ws) where ws holds acc4 [M, N] then acc8 [M, N] int32."""
    M = _codes_k(q["q4"], K)
    dev = q["q4"].device
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    nws = lib().bitlinear_a48_workspace_bytes(M, N)
    ws = ws if ws is not None else torch.empty(nws // 4, dtype=torch.int32, device=dev)
    _check_a48_codes(q, M, K)
    _check_weights(Wp, w_scale, N, K)
    _check_out(Y, None, M, N)
    _expect(ws, "ws", min_bytes=nws)
    _same_device(Wp, w_scale, Y, ws, *q.values())
    st = lib().bitlinear_forward_a48(
        _dev(q["q4"], "Xq4"), _dev(q["g4"], "x4_scale"), _dev(q["rs4"], "x4_rowsum"),
        _dev(q["q8"], "Xq8"), _dev(q["g8"], "x8_scale"), _dev(q["rs8"], "x8_rowsum"), M, K,
        _dev(Wp, "Wp"), _dev(w_scale, "w_scale"), N, _dev(Y, "Y"), _dev(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "bitlinear_forward_a48")
    return Y, ws


def _check_a48_codes(q, M, K):
    for k in ("q4", "g4", "rs4", "q8", "g8", "rs8"):
        if k not in q:
            raise ValueError(f"a4.8 codes need the entry {k!r}")
    _check_codes(q["q4"], q["g4"], q["rs4"], M, K, "4")
    _check_codes(q["q8"], q["g8"], q["rs8"], M, K, "8")


def _act_dtype(X):
    if X.dtype == torch.float32:
        return BL_F32
    if X.dtype == torch.bfloat16:
        return BL_BF16
    raise ValueError("activations must be float32 or bfloat16")


def fused_workspace(M, K, device):
    n = lib().bitlinear_fused_workspace_bytes(int(M), int(K))
    return torch.empty(n, dtype=torch.uint8, device=device)


def bitlinear_forward_fused(X, Wp, w_scale, N, out=None, ws=None):
    """One BitLinear from float activations X [M, K] -> Y [M, N] float32.

    Returns (Y, ws); ws holds the int8 codes, scales and row sums (see
    fused_internals)."""
    M, K = _matrix(X, "X")
    _act_dtype(X)
    dev = X.device
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else fused_workspace(M, K, dev)
    _check_weights(Wp, w_scale, N, K)
    _check_out(Y, None, M, N)
    _expect(ws, "ws", min_bytes=lib().bitlinear_fused_workspace_bytes(int(M), int(K)))
    _same_device(X, Wp, w_scale, Y, ws)
    st = lib().bitlinear_forward_fused(_dev(X, "X"), _act_dtype(X), M, K, _dev(Wp, "Wp"),
                                       _dev(w_scale, "w_scale"), N, _dev(Y, "Y"), _dev(ws, "ws"),
                                       ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "bitlinear_forward_fused")
    return Y, ws


def fused_internals(ws, M, K):
    L = lib()
    kp = padded_k(K)
    o1 = L.bitlinear_fused_workspace_offset(M, K, 1)
    o2 = L.bitlinear_fused_workspace_offset(M, K, 2)
    return {"xq": ws[:M * kp].view(torch.int8).reshape(M, kp),
            "x_scale": ws[o1:o1 + 4 * M].view(torch.float32),
            "x_rowsum": ws[o2:o2 + 4 * M].view(torch.int32)}


def fused_norm_workspace(M, K, device):
    n = lib().bitlinear_fused_norm_workspace_bytes(int(M), int(K))
    return torch.empty(n, dtype=torch.uint8, device=device)


def bitlinear_forward_fused_norm(X, Wp, w_scale, N, norm_w=None, norm_eps=2.0 ** -23, out=None,
                                 ws=None):
    """y = BitLinear(RMSNorm(X)) for X [M, K] float32/bfloat16 -> Y [M, N]
    float32; norm_w a [K] float32 tensor or None (ones).  Returns (Y, ws); ws
    holds xn, the int8 codes, scales and row sums (see fused_norm_internals)."""
    M, K = _matrix(X, "X")
    dt = _act_dtype(X)
    dev = X.device
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else fused_norm_workspace(M, K, dev)
    _check_weights(Wp, w_scale, N, K)
    _check_out(Y, None, M, N)
    if norm_w is not None:
        _expect(norm_w, "norm_w", (K,), (torch.float32,))
    _expect(ws, "ws", min_bytes=lib().bitlinear_fused_norm_workspace_bytes(int(M), int(K)))
    _same_device(X, Wp, w_scale, Y, ws, norm_w)
    st = lib().bitlinear_forward_fused_norm(_dev(X, "X"), dt, M, K, _opt(norm_w, "norm_w"),
                                            float(norm_eps), _dev(Wp, "Wp"),
                                            _dev(w_scale, "w_scale"), N, _dev(Y, "Y"),
                                            _dev(ws, "ws"), ws.numel() * ws.element_size(),
                                            _stream(dev))
    _check(st, "bitlinear_forward_fused_norm")
    return Y, ws


def fused_norm_internals(ws, M, K):
    d = fused_internals(ws, M, K)
    o = lib().bitlinear_fused_workspace_bytes(M, K)
    d["xn"] = ws[o:o + 4 * M * K].view(torch.float32).reshape(M, K)
    return d


def bitnet_ffn_forward(H, norm_w, norm_eps, Wg, sg, Wu, su, Wd, sd, D, F, out=None, ws=None,
                       subln_w=None, subln_eps=2.0 ** -23):
    """FFN block; returns (Y [M, D] float32, workspace uint8 tensor).  With
    subln_w (a [F] float32 tensor) h is RMS-normalised before the down
    projection's quantiser."""
    M, Dh = _matrix(H, "H")
    if Dh != D:
        raise ValueError(f"H has {Dh} columns, D = {D}")
    dt = _act_dtype(H)
    dev = H.device
    Y = out if out is not None else torch.empty((M, D), dtype=torch.float32, device=dev)
    nws = lib().bitnet_ffn_workspace_bytes(M, D, F)
    ws = ws if ws is not None else torch.empty(nws, dtype=torch.uint8, device=dev)
    _check_weights(Wg, sg, F, D, name="Wg")
    _check_weights(Wu, su, F, D, name="Wu")
    _check_weights(Wd, sd, D, F, name="Wd")
    if norm_w is not None:
        _expect(norm_w, "norm_w", (D,), (torch.float32,))
    if subln_w is not None:
        _expect(subln_w, "subln_w", (F,), (torch.float32,))
    _expect(Y, "Y", (M, D), (torch.float32,))
    _expect(ws, "ws", min_bytes=nws)
    _same_device(H, Wg, sg, Wu, su, Wd, sd, Y, ws, norm_w, subln_w)
    st = lib().bitnet_ffn_forward(
        _dev(H, "H"), dt, M, D, F, _opt(norm_w, "norm_w"), float(norm_eps),
        _opt(subln_w, "subln_w"), float(subln_eps), _dev(Wg, "Wg"), _dev(sg, "sg"), _dev(Wu, "Wu"), _dev(su, "su"),
        _dev(Wd, "Wd"), _dev(sd, "sd"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(dev))
    _check(st, "bitnet_ffn_forward")
    return Y, ws


FFN_STATIC_SCRATCH_BYTES = 16 << 20


def bitnet_ffn_forward_static(H, norm_w, norm_eps, Wg, sg, Wu, su, Wd, sd, D, F, out=None,
                              subln_w=None, subln_eps=2.0 ** -23):
    """bitnet_ffn_forward with the library's static per-GPU scratch (no
    workspace argument, no allocation inside); returns Y [M, D] float32."""
    M, Dh = _matrix(H, "H")
    if Dh != D:
        raise ValueError(f"H has {Dh} columns, D = {D}")
    dt = _act_dtype(H)
    dev = H.device
    Y = out if out is not None else torch.empty((M, D), dtype=torch.float32, device=dev)
    _check_weights(Wg, sg, F, D, name="Wg")
    _check_weights(Wu, su, F, D, name="Wu")
    _check_weights(Wd, sd, D, F, name="Wd")
    if norm_w is not None:
        _expect(norm_w, "norm_w", (D,), (torch.float32,))
    if subln_w is not None:
        _expect(subln_w, "subln_w", (F,), (torch.float32,))
    _expect(Y, "Y", (M, D), (torch.float32,))
    _same_device(H, Wg, sg, Wu, su, Wd, sd, Y, norm_w, subln_w)
    st = lib().bitnet_ffn_forward_static(
        _dev(H, "H"), dt, M, D, F, _opt(norm_w, "norm_w"), float(norm_eps),
        _opt(subln_w, "subln_w"), float(subln_eps), _dev(Wg, "Wg"), _dev(sg, "sg"),
        _dev(Wu, "Wu"), _dev(su, "su"), _dev(Wd, "Wd"), _dev(sd, "sd"), _dev(Y, "Y"),
        _stream(dev))
    _check(st, "bitnet_ffn_forward_static")
    return Y


def ffn_internals(ws, M, D, F):
    """Views of the FFN workspace regions (see bitnet_ffn_workspace_layout)."""
    _, off = ffn_workspace_layout(M, D, F)
    dp, fp = padded_k(D), padded_k(F)

    def view(name, dtype, count, shape):
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return ws[off[name]:off[name] + nbytes].view(dtype).reshape(shape)

    return {
        "xn": view("XN", torch.float32, M * D, (M, D)),
        "qx": view("QX", torch.int8, M * dp, (M, dp)),
        "gx": view("GX", torch.float32, M, (M,)),
        "rsx": view("RSX", torch.int32, M, (M,)),
        "h": view("H", torch.float32, M * F, (M, F)),
        "hn": view("HN", torch.float32, M * F, (M, F)),
        "gh": view("GH", torch.float32, M, (M,)),
        "qh": view("QH", torch.int8, M * fp, (M, fp)),
        "rsh": view("RSH", torch.int32, M, (M,)),
    }


# --------------------------------------------------------------------------
# measurement probes (include/bitlinear_probe.h)

def probe_read(buf, per_lane=4, sink=None):
    """One kernel reading every byte of the GPU tensor `buf` once."""
    dev = buf.device
    sink = sink if sink is not None else torch.zeros(1024, dtype=torch.int32, device=dev)
    st = lib().bl_probe_read(_dev(buf, "buf"), buf.numel() * buf.element_size(), int(per_lane),
                             _dev(sink, "sink"), _stream(dev))
    _check(st, "bl_probe_read")
    return sink


def probe_empty(device):
    _check(lib().bl_probe_empty(_stream(torch.device(device))), "bl_probe_empty")
