"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/bitlinear.h declares, and rejects bad arguments on the
host before anything is enqueued.  Pointers passed here are fake non-null
addresses: validation never dereferences them, and every call below fails
validation, so no kernel is launched."""
import ctypes
import os
import re

import pytest

from ternary_weight_linear_ternarize_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

FAKE = ctypes.c_void_p(0x10000)      # 64 KiB: aligned to anything we check
ODD = ctypes.c_void_p(0x10001)       # misaligned


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = declared_functions()
    assert "bitlinear_pack" in names and "bitnet_ffn_forward" in names
    assert "bl_probe_read" in names and "bl_probe_empty" in names
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_size_helpers():
    lib = B.lib()
    assert lib.bl_padded_k(1) == 64 and lib.bl_padded_k(64) == 64 and lib.bl_padded_k(65) == 128
    assert lib.bl_padded_k(0) == 0
    assert lib.bl_packed_bytes(6912, 2560) == 4423680
    assert lib.bl_packed_bytes(28672, 8192) == 58720256
    assert lib.bl_packed_bytes(400, 512) == 51200
    assert lib.bl_pack_workspace_bytes(10, 10) >= 256 * 8
    assert lib.bl_padded_k_1bit(1) == 128 and lib.bl_padded_k_1bit(128) == 128
    assert lib.bl_padded_k_1bit(129) == 256 and lib.bl_padded_k_1bit(0) == 0
    assert lib.bl_packed_bytes_1bit(28672, 8192) == 29360128
    assert lib.bl_packed_bytes_1bit(400, 500) == 400 * 512 // 8
    total, off = B.ffn_workspace_layout(8, 2560, 6912)
    assert all(v % 256 == 0 for v in off.values())
    assert off["QX"] - off["XN"] >= 8 * 2560 * 4
    assert off["QH"] + 8 * 6912 <= total
    assert lib.bitnet_ffn_workspace_bytes(8, 2560, 6912) == total


def test_status_strings():
    for s in range(6):
        assert B.status_str(s)
    assert B.status_str(99) == "unknown status"


def test_pack_validation():
    lib = B.lib()
    ws_n = lib.bl_pack_workspace_bytes(4, 4)
    assert lib.bitlinear_pack(None, 4, 4, 0, FAKE, FAKE, FAKE, ws_n, None) == B.BL_EINVAL
    assert lib.bitlinear_pack(FAKE, 4, 4, 7, FAKE, FAKE, FAKE, ws_n, None) == B.BL_EINVAL
    assert lib.bitlinear_pack(FAKE, 0, 4, 0, FAKE, FAKE, FAKE, ws_n, None) == B.BL_ESHAPE
    assert lib.bitlinear_pack(FAKE, 4, 70000, 0, FAKE, FAKE, FAKE, ws_n, None) == B.BL_ESHAPE
    assert lib.bitlinear_pack(FAKE, 4, 4, 0, FAKE, FAKE, FAKE, ws_n - 1, None) == B.BL_EWORKSPACE
    assert lib.bitlinear_pack(FAKE, 4, 4, 0, FAKE, FAKE, None, ws_n, None) == B.BL_EWORKSPACE
    assert lib.bitlinear_pack(FAKE, 4, 4, 0, ODD, FAKE, FAKE, ws_n, None) == B.BL_EALIGN


def test_quant_validation():
    lib = B.lib()
    assert lib.bitlinear_quant_act(None, 0, 1, 8, FAKE, FAKE, FAKE, None) == B.BL_EINVAL
    assert lib.bitlinear_quant_act(FAKE, 2, 1, 8, FAKE, FAKE, FAKE, None) == B.BL_EINVAL
    # the row sums are required output (the forward takes them as input)
    assert lib.bitlinear_quant_act(FAKE, 0, 1, 8, FAKE, FAKE, None, None) == B.BL_EINVAL
    assert lib.bitlinear_quant_act(FAKE, 0, 0, 8, FAKE, FAKE, FAKE, None) == B.BL_ESHAPE
    assert lib.bitlinear_quant_act(FAKE, 0, 1, -1, FAKE, FAKE, FAKE, None) == B.BL_ESHAPE
    assert lib.bitlinear_quant_act(FAKE, 0, 1, 8, ODD, FAKE, FAKE, None) == B.BL_EALIGN
    assert lib.bitlinear_quant_act(ODD, 0, 1, 8, FAKE, FAKE, FAKE, None) == B.BL_EALIGN


def test_forward_validation():
    lib = B.lib()
    f = lib.bitlinear_forward_kernel
    args = [FAKE, FAKE, FAKE, 1, 64, FAKE, FAKE, 16, FAKE, None]
    assert f(None, *args[1:], 0, None) == B.BL_EINVAL
    a = list(args); a[2] = None  # rowsum is required
    assert f(*a, 0, None) == B.BL_EINVAL
    a = list(args); a[3] = 0
    assert f(*a, 0, None) == B.BL_ESHAPE
    a = list(args); a[7] = 0
    assert f(*a, 0, None) == B.BL_ESHAPE
    a = list(args); a[5] = ODD
    assert f(*a, 0, None) == B.BL_EALIGN
    a = list(args); a[3] = 2
    assert f(*a, B.BL_KERNEL_GEMV, None) == B.BL_ESHAPE   # GEMV needs M == 1
    a = list(args); a[3] = 65
    assert f(*a, B.BL_KERNEL_SKINNY, None) == B.BL_ESHAPE  # skinny needs M <= 64
    assert f(*args, 9, None) == B.BL_EINVAL
    assert lib.bitlinear_forward(FAKE, FAKE, FAKE, 1, 64, ODD, FAKE, 16, FAKE, None, None) == B.BL_EALIGN
    h = lib.bitlinear_quant_act_a48
    assert h(FAKE, 0, 1, 64, 3, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.BL_EINVAL
    assert h(FAKE, 0, 1, 64, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.BL_ESHAPE
    assert h(FAKE, 0, 1, 64, 3, ODD, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.BL_EALIGN
    f48 = lib.bitlinear_forward_a48
    n48 = lib.bitlinear_a48_workspace_bytes(2, 16)
    assert n48 == 2 * 16 * 8
    a48 = [FAKE] * 6 + [2, 64, FAKE, FAKE, 16, FAKE, FAKE, n48, None]
    b = list(a48); b[13] = n48 - 1
    assert f48(*b) == B.BL_EWORKSPACE
    b = list(a48); b[3] = None
    assert f48(*b) == B.BL_EINVAL
    b = list(a48); b[3] = ODD
    assert f48(*b) == B.BL_EALIGN
    g = lib.bitlinear_forward_1bit
    assert g(FAKE, FAKE, None, 1, 64, FAKE, FAKE, 16, FAKE, None, None) == B.BL_EINVAL
    assert g(FAKE, FAKE, FAKE, 0, 64, FAKE, FAKE, 16, FAKE, None, None) == B.BL_ESHAPE
    assert g(FAKE, FAKE, FAKE, 1, 64, ODD, FAKE, 16, FAKE, None, None) == B.BL_EALIGN
    assert g(FAKE, FAKE, FAKE, 1, 64, FAKE, FAKE, 16, FAKE, ODD, None) == B.BL_EALIGN


def test_ffn_validation():
    lib = B.lib()
    M, D, F = 2, 64, 128
    n = lib.bitnet_ffn_workspace_bytes(M, D, F)
    base = [FAKE, 0, M, D, F, None, 1e-6, None, 1e-6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, n, None]
    a = list(base); a[0] = None
    assert lib.bitnet_ffn_forward(*a) == B.BL_EINVAL
    a = list(base); a[1] = 5
    assert lib.bitnet_ffn_forward(*a) == B.BL_EINVAL
    a = list(base); a[4] = 0
    assert lib.bitnet_ffn_forward(*a) == B.BL_ESHAPE
    a = list(base); a[17] = n - 1
    assert lib.bitnet_ffn_forward(*a) == B.BL_EWORKSPACE
    a = list(base); a[16] = ctypes.c_void_p(0x10010)  # 16 B aligned, not 256
    assert lib.bitnet_ffn_forward(*a) == B.BL_EALIGN
    a = list(base); a[9] = ODD
    assert lib.bitnet_ffn_forward(*a) == B.BL_EALIGN
    a = list(base); a[7] = ODD  # SubLN weight
    assert lib.bitnet_ffn_forward(*a) == B.BL_EALIGN


def test_fused_norm_validation():
    lib = B.lib()
    f = lib.bitlinear_forward_fused_norm
    M, K, N = 2, 64, 16
    n = lib.bitlinear_fused_norm_workspace_bytes(M, K)
    assert n >= lib.bitlinear_fused_workspace_bytes(M, K) + M * K * 4
    assert lib.bitlinear_fused_norm_workspace_bytes(0, K) == 0
    base = [FAKE, 0, M, K, None, 1e-6, FAKE, FAKE, N, FAKE, FAKE, n, None]
    a = list(base); a[0] = None
    assert f(*a) == B.BL_EINVAL
    a = list(base); a[1] = 3
    assert f(*a) == B.BL_EINVAL
    a = list(base); a[8] = 0
    assert f(*a) == B.BL_ESHAPE
    a = list(base); a[11] = n - 1
    assert f(*a) == B.BL_EWORKSPACE
    a = list(base); a[10] = None
    assert f(*a) == B.BL_EWORKSPACE
    a = list(base); a[4] = ODD  # the norm weights
    assert f(*a) == B.BL_EALIGN
    a = list(base); a[6] = ODD
    assert f(*a) == B.BL_EALIGN


def test_product_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "ternary_weight_linear_ternarize_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "liboracle" not in text and "orc_" not in text, fn


def test_quant_act_requires_the_row_sum():
    lib = B.lib()
    assert lib.bitlinear_quant_act(FAKE, 0, 1, 8, FAKE, FAKE, None, None) == B.BL_EINVAL


# ----------------------------------------------------------------------------
# The Python binding checks shapes, dtypes and sizes before any pointer goes
# to the library (the kernels trust the sizes they are given).  These run on
# CPU tensors: a well-formed call gets as far as the device check.

def _raises(fn, *words):
    with pytest.raises(ValueError) as e:
        fn()
    msg = str(e.value)
    assert all(w in msg for w in words), msg


def test_binding_rejects_mismatched_forward_arguments():
    import torch
    M, K, N = 3, 100, 40
    kp = B.padded_k(K)
    Xq = torch.zeros((M, kp), dtype=torch.int8)
    xs = torch.zeros(M, dtype=torch.float32)
    rs = torch.zeros(M, dtype=torch.int32)
    Wp = torch.zeros((N, kp // 16), dtype=torch.int32)
    sc = torch.zeros(1, dtype=torch.float32)
    fwd = B.bitlinear_forward
    _raises(lambda: fwd(Xq, xs, rs, K, Wp, sc, N), "GPU tensor")          # well formed
    _raises(lambda: fwd(Xq, xs, rs, K + 64, Wp, sc, N), "columns")        # K does not match Xq
    _raises(lambda: fwd(Xq[:, :64].contiguous(), xs, rs, K, Wp, sc, N), "columns")
    _raises(lambda: fwd(Xq, xs[:2], rs, K, Wp, sc, N), "x_scale", "shape")
    _raises(lambda: fwd(Xq, xs, rs.float(), K, Wp, sc, N), "x_rowsum", "dtype")
    _raises(lambda: fwd(Xq, xs, rs, K, Wp, sc, N + 1), "Wp", "shape")
    _raises(lambda: fwd(Xq, xs, rs, K, Wp[:, :3].contiguous(), sc, N), "Wp", "shape")
    _raises(lambda: fwd(Xq.float(), xs, rs, K, Wp, sc, N), "Xq", "dtype")
    _raises(lambda: fwd(Xq, xs, rs, K, Wp, sc, N, out=torch.zeros((M, N + 1))), "Y", "shape")
    _raises(lambda: fwd(Xq, xs, rs, K, Wp, sc, N, acc_out=torch.zeros((M, N))), "acc_out", "dtype")
    _raises(lambda: B.bitlinear_forward_1bit(Xq, xs, rs, K, Wp, sc, N), "Wb", "shape")


def test_binding_rejects_mismatched_quant_pack_fused_and_ffn_arguments():
    import torch
    M, K, N = 2, 130, 16
    kp = B.padded_k(K)
    X = torch.zeros((M, K), dtype=torch.float32)
    good = (torch.zeros((M, kp), dtype=torch.int8), torch.zeros(M), torch.zeros(M, dtype=torch.int32))
    _raises(lambda: B.bitlinear_quant_act(X, out=good), "GPU tensor")
    _raises(lambda: B.bitlinear_quant_act(X.double()), "float32 or bfloat16")
    _raises(lambda: B.bitlinear_quant_act(X, out=(good[0][:, :64], good[1], good[2])), "Xq", "shape")
    _raises(lambda: B.bitlinear_quant_act(X, out=(good[0], good[1], good[2][:1])), "x_rowsum")
    _raises(lambda: B.bitlinear_pack(torch.zeros(N, K), out=torch.zeros((N, 2), dtype=torch.int32)),
            "Wp", "shape")
    _raises(lambda: B.bitlinear_pack(torch.zeros(N, K, dtype=torch.float64)), "W", "dtype")
    Wp = torch.zeros((N, kp // 16), dtype=torch.int32)
    sc = torch.zeros(1)
    _raises(lambda: B.bitlinear_forward_fused(X, Wp, sc, N, ws=torch.zeros(8, dtype=torch.uint8)),
            "ws", "bytes")
    _raises(lambda: B.bitlinear_forward_fused(X, Wp, sc, N + 1), "Wp", "shape")
    D, F = K, 48
    H = torch.zeros((M, D))
    Wg = torch.zeros((F, kp // 16), dtype=torch.int32)
    Wd = torch.zeros((D, B.padded_k(F) // 16), dtype=torch.int32)
    ffn = B.bitnet_ffn_forward
    _raises(lambda: ffn(H, None, 1e-6, Wg, sc, Wg, sc, Wd, sc, D, F), "GPU tensor")
    _raises(lambda: ffn(H, None, 1e-6, Wg, sc, Wg, sc, Wd, sc, D + 1, F), "H has")
    _raises(lambda: ffn(H, None, 1e-6, Wg, sc, Wg, sc, Wg, sc, D, F), "Wd", "shape")
    _raises(lambda: ffn(H, torch.zeros(D + 1), 1e-6, Wg, sc, Wg, sc, Wd, sc, D, F), "norm_w")
    _raises(lambda: ffn(H, None, 1e-6, Wg, sc, Wg, sc, Wd, sc, D, F, subln_w=torch.zeros(D)),
            "subln_w")
    q = {"q4": good[0], "g4": good[1], "rs4": good[2], "q8": good[0], "g8": good[1], "rs8": good[2]}
    _raises(lambda: B.bitlinear_forward_a48(q, K, Wp, sc, N), "GPU tensor")
    q2 = dict(q, rs8=good[2][:1])
    _raises(lambda: B.bitlinear_forward_a48(q2, K, Wp, sc, N), "x8_rowsum")
