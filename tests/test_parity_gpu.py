"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, on the
same seeded synthetic inputs.

Bar: bit-exact packed words, weight scales, int8 codes, activation scales,
row sums, int32 accumulators and FFN internals; float outputs within a
maximum relative error of 1e-5 (in practice they are bit-identical, since the
float steps follow the same binary32 operation order).  Every case is also
run twice on the GPU and must repeat bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_ternarize_amd import binding as B
from ternary_weight_linear_ternarize_amd import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-5
DEV = "cuda:0"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    _need_gpu()
    B.lib()
    yield


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_rel(y, ref, rtol=RTOL):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    err = np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)
    assert float(err.max(initial=0.0)) <= rtol, f"max rel err {err.max()}"


def gpu_pack(W, mode=B.BL_TERNARY):
    Wd = to_dev(W)
    Wp, sc = B.bitlinear_pack(Wd, mode)
    return Wp, sc


def check_pack(W, mode="ternary"):
    g, t, p = oracle.quantize_weights(W, mode)
    Wp, sc = gpu_pack(W, B.BL_TERNARY if mode == "ternary" else B.BL_BINARY)
    np.testing.assert_array_equal(host(Wp).view(np.uint32), p)
    assert host(sc)[0].view(np.uint32) == np.float32(g).view(np.uint32)
    return g, t, Wp, sc


def check_quant(X, bf16=False):
    xd = to_dev(X)
    if bf16:
        xd = xd.to(torch.bfloat16)
        X = xd.float().cpu().numpy()  # exact widening: same values for the oracle
    q, g, rs = oracle.act_quant(X)
    Xq, xs, xr = B.bitlinear_quant_act(xd)
    K = X.shape[1]
    hq = host(Xq)
    np.testing.assert_array_equal(hq[:, :K], q)
    assert not hq[:, K:].any()
    np.testing.assert_array_equal(host(xs).view(np.uint32), g.view(np.uint32))
    np.testing.assert_array_equal(host(xr), rs)
    return q, g, rs, Xq, xs, xr


def check_forward(q, gx, t, gw, Xq, xs, xr, Wp, ws, kernels):
    M, K = q.shape
    N = t.shape[0]
    acc = oracle.int_linear(q, t)
    y = oracle.dequant(acc, gx, gw)
    for kern in kernels:
        Y, A = B.bitlinear_forward(Xq, xs, xr, K, Wp, ws, N, with_acc=True, kernel=kern)
        np.testing.assert_array_equal(host(A), acc, err_msg=f"kernel {kern}")
        assert_rel(host(Y), y)
        Y2 = B.bitlinear_forward(Xq, xs, xr, K, Wp, ws, N, kernel=kern)
        np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))
    return acc, y


def kernels_for(M):
    ks = [B.BL_KERNEL_AUTO, B.BL_KERNEL_TILED]
    if M == 1:
        ks.append(B.BL_KERNEL_GEMV)
    if M <= 64:
        ks.append(B.BL_KERNEL_SKINNY)
    return ks


# ----------------------------------------------------------------------------

def test_single_layer_512_to_400_all_kernels():
    d = synth.single_layer()
    g, t, Wp, sc = check_pack(d["W"])
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    check_forward(q, gx, t, g, Xq, xs, xr, Wp, sc, kernels_for(16))
    # every single token through the GEMV and the MFMA kernels
    for m in (0, 7, 15):
        check_forward(q[m:m + 1], gx[m:m + 1], t, g, Xq[m:m + 1].contiguous(),
                      xs[m:m + 1].contiguous(), xr[m:m + 1].contiguous(), Wp, sc, kernels_for(1))


@pytest.mark.parametrize("M,K,N", [
    (1, 1, 1), (1, 15, 17), (1, 63, 257), (1, 65, 400), (1, 1040, 33), (1, 4160, 70), (1, 16448, 9),
    (2, 64, 16), (3, 16, 63), (5, 65, 64), (8, 1040, 257), (16, 512, 400), (17, 63, 15),
    (31, 1000, 100), (33, 129, 65), (64, 2560, 96), (65, 300, 130), (100, 1040, 257), (129, 64, 129),
    (300, 700, 600),
    # 17..64 tokens on the skinny tiled GEMM with 2 or 4 chunks of loads in
    # flight: partial last chunks, chunk counts not multiples of the depth
    (48, 3000, 77), (64, 4100, 50), (20, 8000, 33), (64, 7000, 40), (64, 9000, 20),
    # 17..64 tokens with long K on the kernel that splits K over the waves of a
    # block: ragged 16-token and 48-column tiles, the most pieces per wave (8)
    (17, 6912, 100), (33, 8192, 2600), (64, 4096, 2561), (40, 8100, 47),
    # 2..16 tokens with K <= 4096 and 4096..16384 columns on the same kernel,
    # 2 tokens with any K it takes; 17..64 tokens with short K; every tile
    # shape (16 x 16 .. 16 x 64, 32 x 64) and the fallback past 256 blocks
    (2, 2560, 6912), (9, 4096, 4097), (16, 1000, 16384), (5, 65, 5000),
    (2, 6912, 2560), (2, 8192, 2048), (5, 5000, 3001), (17, 2560, 6912), (64, 2560, 6912),
    (50, 1000, 9000), (33, 3000, 2048),
    # 65..384 tokens on the K-split kernel (tiles up to 64 x 64, chosen by the
    # bytes through the busiest CU) and past its range on the tiled GEMM
    (65, 2560, 6912), (128, 6912, 2560), (200, 5000, 3000), (384, 4500, 2049), (511, 4500, 2049),
    (300, 2560, 4096),
    # the tiled GEMM on 128 x 128 tiles (at most 256 of them) and on 128 x 256
    (777, 6912, 2560), (1100, 700, 2000), (520, 2560, 6912),
    # one token, packed matrix >= 16 MiB (the streaming GEMV), ragged K and odd N
    (1, 5000, 13301), (1, 4000, 17001), (1, 8192, 16385), (1, 8192, 8192), (1, 8192, 12001),
    (1, 4096, 40000),
    # the largest K, N and M the boundary accepts (65536 each), one at a time
    (1, 65536, 200), (8, 65536, 100), (40, 65536, 48), (100, 65536, 64),
    (1, 100, 65536), (8, 100, 65536), (40, 200, 65536), (100, 100, 65536),
    (65536, 100, 40),
])
def test_random_ragged_shapes(M, K, N):
    d = synth.random_case(1000 + M * 7 + N, M, K, N)
    g, t, Wp, sc = check_pack(d["W"])
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    check_forward(q, gx, t, g, Xq, xs, xr, Wp, sc, kernels_for(M))


def test_outputs_past_two_to_the_31_elements():
    """M = N = 65536 (K = 64): 2^32 outputs, so rows from 32768 on start past
    element 2^31 and byte offset 8 GiB.  Sampled rows (first, last, both sides
    of the 2^31 boundary and random ones) against the oracle, for the 2-bit
    and the 1-bit layouts."""
    M, K, N = 65536, 64, 65536
    d = synth.random_case(77, M, K, N)
    g, t, Wp, sc = check_pack(d["W"])
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, 1, 32767, 32768, 32769, M - 1],
                                     rng.integers(0, M, 40)]))
    ref = oracle.dequant(oracle.int_linear(q[rows], t), gx[rows], g)
    ridx = torch.from_numpy(rows).to(DEV)
    Y = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N)
    assert_rel(host(Y.index_select(0, ridx)), ref)
    g1, t1, Wb, sc1 = check_pack1(d["W"])
    ref1 = oracle.dequant(oracle.int_linear(q[rows], t1), gx[rows], g1)
    B.bitlinear_forward_1bit(Xq, xs, xr, K, Wb, sc1, N, out=Y)
    assert_rel(host(Y.index_select(0, ridx)), ref1)
    del Y
    torch.cuda.empty_cache()


def test_binary_mode_and_degenerate_weights():
    rng = np.random.default_rng(21)
    W = rng.standard_normal((70, 200)).astype(np.float32)
    W[3, :] = 0.0
    W[5, 7] = -0.0
    for mode in ("binary", "ternary"):
        g, t, Wp, sc = check_pack(W, mode)
        X = synth.normal(21, 1, (4, 200))
        q, gx, rs, Xq, xs, xr = check_quant(X)
        check_forward(q, gx, t, g, Xq, xs, xr, Wp, sc, kernels_for(4))
    # all-zero and identity weights
    check_pack(np.zeros((33, 100), np.float32))
    g, t, Wp, sc = check_pack(np.eye(128, dtype=np.float32))
    assert g == np.float32(1.0 / 128)


def test_weight_scale_wide_dynamic_range():
    """Weights spread over the whole binary32 range (subnormals to 2^120, zeros
    of both signs, rows of one magnitude) so the absmean sum takes every path:
    the in-window integer accumulators, the direct bins and their merge."""
    rng = np.random.default_rng(41)
    for (N, K) in ((96, 1000), (37, 301)):
        W = rng.standard_normal((N, K)).astype(np.float32)
        W *= np.ldexp(np.float32(1), rng.integers(-140, 121, size=(N, K))).astype(np.float32)
        W[0, :] = np.float32(1e-45)           # smallest subnormal
        W[1, :] = -0.0
        W[2, ::3] = 0.0
        W[3, :] = np.float32(3.0e38)
        W[4, :] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -30)
        for mode in ("ternary", "binary"):
            check_pack(W, mode)
        # the same values from a base address that is not 16-byte aligned
        flat = to_dev(np.concatenate([np.zeros(1, np.float32), W.ravel()]))
        Wd = flat[1:].view(N, K)
        Wp, sc = B.bitlinear_pack(Wd)
        g, t, pk = oracle.quantize_weights(W, "ternary")
        np.testing.assert_array_equal(host(Wp).view(np.uint32), pk)
        assert host(sc)[0].view(np.uint32) == np.float32(g).view(np.uint32)


def test_ternary_codes_at_the_rounding_threshold():
    """Weights a few ulps either side of d/2 (d = scale + 1e-5, both signs,
    d/2 itself included): the code is non-zero exactly when the correctly
    rounded quotient w / d exceeds 1/2, i.e. above d/2 and not at it.  The
    placed weights barely move the scale; they are re-placed until the scale
    is a fixed point."""
    rng = np.random.default_rng(43)
    for scale in (1.0, 1.37, 1.93, 3.1e-3):
        W = (rng.standard_normal((48, 640)) * scale).astype(np.float32)
        idx = rng.choice(W.size, 64, replace=False)
        g = oracle.weight_scale(W)
        for _ in range(20):
            d = np.float32(g) + oracle.EPS
            half = d * np.float32(0.5)
            vals, v = [], half
            for _k in range(4):
                v = np.nextafter(v, np.float32(0), dtype=np.float32)
            for _k in range(9):
                vals += [v, -v]
                v = np.nextafter(v, np.float32(np.inf), dtype=np.float32)
            Wn = W.copy()
            Wn.flat[idx[:len(vals)]] = np.asarray(vals, np.float32)
            g2 = oracle.weight_scale(Wn)
            if np.float32(g2) == np.float32(g):
                break
            g = g2
        else:
            raise AssertionError("the scale did not settle")
        t = oracle.ternarize(np.asarray(vals, np.float32), np.float32(g))
        assert (t == 0).sum() == 10 and (t != 0).sum() == 8  # the threshold is crossed
        check_pack(Wn, "ternary")


def test_quant_edge_rows_and_bf16():
    X = synth.normal(22, 1, (6, 700))
    X[1] = 0.0
    X[2] = 0.0
    X[2, 123] = -5.0
    X[3] = 1e-30
    X[4] *= np.float32(1e4)
    check_quant(X)
    check_quant(synth.normal(23, 1, (9, 2560)), bf16=True)
    x = synth.decode_100b(with_weights=False)["X"]
    check_quant(x)


def test_nonfinite_rows_leave_the_other_rows_exact():
    """NaN and Inf inputs give unspecified results, but every call completes
    and the tokens whose rows are finite come out bit for bit as the oracle
    computes them without the others (quantisation, RMSNorm and the products
    are per token), through the 8- and 40-token products and the FFN block."""
    for M, K, N in ((8, 1000, 300), (40, 700, 200)):
        d = synth.random_case(900 + M, M, K, N)
        X = d["X"].copy()
        bad = [1, 5]
        X[1, 7] = np.nan
        X[5, :3] = [np.inf, -np.inf, np.nan]
        good = np.array([m for m in range(M) if m not in bad])
        g, t, Wp, sc = check_pack(d["W"])
        Xq, xs, xr = B.bitlinear_quant_act(to_dev(X))
        for kern in kernels_for(M):
            Y, A = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N, with_acc=True, kernel=kern)
            q, gx, rs = oracle.act_quant(X[good])
            acc = oracle.int_linear(q, t)
            np.testing.assert_array_equal(host(A)[good], acc)
            assert_rel(host(Y)[good], oracle.dequant(acc, gx, g))
    M, D, F = 8, 256, 520
    x = synth.normal(950, 1, (M, D))
    x[2, 10] = np.nan
    x[6, 0] = np.inf
    good = np.array([0, 1, 3, 4, 5, 7])
    ws = [synth.normal(950, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    q = [oracle.quantize_weights(w) for w in ws]
    pk = [B.bitlinear_pack(to_dev(w)) for w in ws]
    eps = 1e-6
    ref = oracle.ffn(x[good], None, eps, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1], q[2][0])
    Y, _ = B.bitnet_ffn_forward(to_dev(x), None, eps, pk[0][0], pk[0][1], pk[1][0], pk[1][1],
                                pk[2][0], pk[2][1], D, F)
    assert_rel(host(Y)[good], ref["y"])


def test_decode_2b_gemv_up_and_down_full():
    d = synth.decode_2b()
    for Wn, xn in (("W_up", "x"), ("W_down", "x_d")):
        g, t, Wp, sc = check_pack(d[Wn])
        zero_frac = float(np.mean(t == 0))
        assert abs(zero_frac - 0.31) < 0.01
        q, gx, rs, Xq, xs, xr = check_quant(d[xn])
        check_forward(q, gx, t, g, Xq, xs, xr, Wp, sc, kernels_for(1))


def test_prefill_2b_full():
    # every accumulator and output of the 2048 x 2560 x 6912 prefill, in the
    # launch the benchmark times (no accumulator output: the LDS epilogue) and
    # with the accumulators requested (the register epilogue)
    d = synth.prefill_2b()
    g, t, Wp, sc = check_pack(d["W"])
    X = d["X"]
    q, gx, rs, Xq, xs, xr = check_quant(X)
    M, K = X.shape
    N = t.shape[0]
    acc = oracle.int_linear(q, t)
    y = oracle.dequant(acc, gx, g)
    Yb = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N)
    assert_rel(host(Yb), y)
    Y, A = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N, with_acc=True)
    np.testing.assert_array_equal(host(A), acc)
    np.testing.assert_array_equal(host(Y).view(np.uint32), host(Yb).view(np.uint32))
    Y2 = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Yb).view(np.uint32))


def test_skinny_phased_activations_ragged_k():
    # the phased staging with a K that ends inside a step (Kp = 7040: the
    # second phase stages 2944 columns and its last step reads past Kp)
    M, K, N = 16, 7000, 25600
    d = synth.random_case(1718, M, K, N)
    g, t, Wp, sc = check_pack(d["W"])
    del d["W"]
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    Y, A = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N, with_acc=True)
    acc = oracle.int_linear(q, t)
    np.testing.assert_array_equal(host(A), acc)
    assert_rel(host(Y), oracle.dequant(acc, gx, g))


def test_page_shape_example_512_to_400_on_10x1000_tokens():
    # [P2] "BitLinear層の基本実装": BitLinear(512, 400) applied to a (10, 1000, 512)
    # input gives (10, 1000, 400); here the 10 000 tokens run through the
    # tiled GEMM (78 full token tiles + a 16-row tail, a 144-column tail)
    d = synth.random_case(5120, 10 * 1000, 512, 400)
    g, t, Wp, sc = check_pack(d["W"])
    X3 = to_dev(d["X"]).view(10, 1000, 512)
    Xq, xs, xr = B.bitlinear_quant_act(X3.reshape(-1, 512))
    Y, A = B.bitlinear_forward(Xq, xs, xr, 512, Wp, sc, 400, with_acc=True)
    Y3 = Y.view(10, 1000, 400)
    assert tuple(Y3.shape) == (10, 1000, 400)
    q, gx, rs = oracle.act_quant(d["X"])
    np.testing.assert_array_equal(host(Xq)[:, :512], q)
    acc = oracle.int_linear(q, t)
    np.testing.assert_array_equal(host(A), acc)
    assert_rel(host(Y), oracle.dequant(acc, gx, g))
    Y2 = B.bitlinear_forward(Xq, xs, xr, 512, Wp, sc, 400)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


@pytest.mark.parametrize("mode", ["ternary", "binary"])
def test_decode_100b_full(mode):
    d = synth.decode_100b()
    g, t, Wp, sc = check_pack(d["W"], mode)
    del d["W"]
    for M in (1, 8):
        q, gx, rs, Xq, xs, xr = check_quant(d["X"][:M])
        check_forward(q, gx, t, g, Xq, xs, xr, Wp, sc, kernels_for(M)[:3])


def _ffn_case(M, bf16, norm, subln=False):
    d = synth.ffn_2b(norm=norm)
    D, F = synth.FFN_2B["D"], synth.FFN_2B["F"]
    pk = {}
    for name in ("W_gate", "W_up", "W_down"):
        pk[name] = check_pack(d[name])
    H = d["H"][:M]
    Hd = to_dev(H)
    if bf16:
        Hd = Hd.to(torch.bfloat16)
        H = Hd.float().cpu().numpy()
    nw = d["norm_w"]
    eps = float(np.finfo(np.float32).eps)
    sw = d["subln_w"] if subln else None
    ref = oracle.ffn(H, nw, eps, pk["W_gate"][1], pk["W_gate"][0], pk["W_up"][1], pk["W_up"][0],
                     pk["W_down"][1], pk["W_down"][0], subln=subln, subln_w=sw, subln_eps=eps)
    kw = dict(subln_w=to_dev(sw), subln_eps=eps) if subln else {}
    Y, ws = B.bitnet_ffn_forward(Hd, to_dev(nw), eps, pk["W_gate"][2], pk["W_gate"][3],
                                 pk["W_up"][2], pk["W_up"][3], pk["W_down"][2], pk["W_down"][3], D, F,
                                 **kw)
    it = {k: host(v) for k, v in B.ffn_internals(ws, M, D, F).items()}
    if subln:
        np.testing.assert_array_equal(it["hn"].view(np.uint32), ref["hn"].view(np.uint32))
    np.testing.assert_array_equal(it["xn"].view(np.uint32), ref["xn"].view(np.uint32))
    np.testing.assert_array_equal(it["qx"][:, :D], ref["qx"])
    np.testing.assert_array_equal(it["gx"].view(np.uint32), ref["gx"].view(np.uint32))
    np.testing.assert_array_equal(it["rsx"], ref["qx"].astype(np.int64).sum(1))
    np.testing.assert_array_equal(it["h"].view(np.uint32), ref["h"].view(np.uint32))
    np.testing.assert_array_equal(it["gh"].view(np.uint32), ref["gh"].view(np.uint32))
    np.testing.assert_array_equal(it["qh"][:, :F], ref["qh"])
    np.testing.assert_array_equal(it["rsh"], ref["qh"].astype(np.int64).sum(1))
    assert_rel(host(Y), ref["y"])
    Y2, _ = B.bitnet_ffn_forward(Hd, to_dev(nw), eps, pk["W_gate"][2], pk["W_gate"][3],
                                 pk["W_up"][2], pk["W_up"][3], pk["W_down"][2], pk["W_down"][3], D, F,
                                 **kw)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


@pytest.mark.parametrize("M", [1, 8, 64])
def test_ffn_2b_fp32(M):
    _ffn_case(M, False, "ones")


@pytest.mark.parametrize("M", [1, 8, 64])
def test_ffn_2b_bf16_random_norm(M):
    _ffn_case(M, True, "random")


@pytest.mark.parametrize("M", [1, 8, 64])
def test_ffn_2b_subln(M):
    _ffn_case(M, M == 8, "random", subln=True)


@pytest.mark.parametrize("M,D,F,subln", [(1, 300, 700, False), (2, 64, 128, False), (2, 17000, 100, False),
                                         (1, 17000, 100, False), (1, 300, 9000, False),
                                         (1, 17000, 100, True),
                                         (17, 512, 1000, False), (40, 1000, 3000, False),
                                         # gate/up at 17..32 tokens with K split over the
                                         # waves of a block: 1 to 5 pieces per wave
                                         (32, 2560, 6912, False), (24, 1000, 3000, True),
                                         (17, 4100, 900, False), (31, 120, 70, False),
                                         # 33..64 tokens: 64 x 32 tiles while K fits two
                                         # pieces of 256 per wave, 32 x 32 tiles above
                                         (48, 5000, 700, False), (64, 300, 4500, True),
                                         # 65..192 tokens: gate/up on the same kernel;
                                         # 200 tokens past its range
                                         (100, 2560, 6912, False), (192, 3000, 2500, True),
                                         (200, 1000, 2100, False), (300, 700, 1000, True),
                                         (513, 2560, 6912, False), (700, 300, 5000, True),
                                         (100, 256, 520, False), (256, 512, 1024, False),
                                         (1, 300, 9000, True), (5, 64, 130, True), (40, 1000, 3000, True),
                                         (100, 256, 520, True),
                                         # SubLN inside the one-token down GEMV: two chunks
                                         # per lane with 2 and 4 rows per wave, F at its limit
                                         (1, 8000, 7000, True), (1, 700, 8192, True),
                                         (1, 700, 8193, True),
                                         # the largest D and F
                                         (1, 65536, 64, False), (3, 65536, 48, True),
                                         (1, 64, 65536, False), (2, 100, 65536, True)])
def test_ffn_ragged_shapes(M, D, F, subln):
    s = 500 + M
    x = synth.normal(s, 1, (M, D))
    ws = [synth.normal(s, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    q = [oracle.quantize_weights(w) for w in ws]
    nw = (np.float32(1) + synth.normal(s, 9, (D,), 0.1)).astype(np.float32)
    sw = (np.float32(1) + synth.normal(s, 10, (F,), 0.1)).astype(np.float32) if subln else None
    eps = 1e-6
    ref = oracle.ffn(x, nw, eps, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1], q[2][0],
                     subln=subln, subln_w=sw, subln_eps=1e-5)
    pk = [B.bitlinear_pack(to_dev(w)) for w in ws]
    for i in range(3):
        np.testing.assert_array_equal(host(pk[i][0]).view(np.uint32), q[i][2])
    kw = dict(subln_w=to_dev(sw), subln_eps=1e-5) if subln else {}
    Y, wsp = B.bitnet_ffn_forward(to_dev(x), to_dev(nw), eps, pk[0][0], pk[0][1], pk[1][0],
                                  pk[1][1], pk[2][0], pk[2][1], D, F, **kw)
    it = {k: host(v) for k, v in B.ffn_internals(wsp, M, D, F).items()}
    if subln:
        np.testing.assert_array_equal(it["hn"].view(np.uint32), ref["hn"].view(np.uint32))
    np.testing.assert_array_equal(it["xn"].view(np.uint32), ref["xn"].view(np.uint32))
    np.testing.assert_array_equal(it["qx"][:, :D], ref["qx"])
    np.testing.assert_array_equal(it["h"].view(np.uint32), ref["h"].view(np.uint32))
    np.testing.assert_array_equal(it["gh"].view(np.uint32), ref["gh"].view(np.uint32))
    np.testing.assert_array_equal(it["qh"][:, :F], ref["qh"])
    assert_rel(host(Y), ref["y"])


def test_ffn_output_alignment_does_not_change_results():
    # Y only 4-byte aligned (the kernels store it in 4-byte words): the bits
    # must not depend on the output's alignment
    M, D, F = 40, 1000, 3000
    x = synth.normal(640, 1, (M, D))
    ws = [synth.normal(640, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    pk = [B.bitlinear_pack(to_dev(w)) for w in ws]
    eps = 1e-6
    args = (to_dev(x), None, eps, pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], D, F)
    Ya, _ = B.bitnet_ffn_forward(*args)
    buf = torch.zeros(M * D + 1, dtype=torch.float32, device=DEV)
    Yu = buf[1:].view(M, D)
    assert Yu.data_ptr() % 16 == 4
    B.bitnet_ffn_forward(*args, out=Yu)
    np.testing.assert_array_equal(host(Yu).view(np.uint32), host(Ya).view(np.uint32))
    q = [oracle.quantize_weights(w) for w in ws]
    ref = oracle.ffn(x, None, eps, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1], q[2][0])
    assert_rel(host(Yu), ref["y"])


@pytest.mark.parametrize("M", [1, 8, 60])
def test_rmsnorm_on_mean_squares_at_binary32_midpoints(M):
    # hidden rows whose exact mean square is a binary32 rounding midpoint (or
    # one unit of the integer sum away): the RMSNorm bits are then decided by
    # the exact sum, and one ulp of xn can flip an int8 code
    D, F = 2560, 256
    x = synth.midpoint_rows(D, M, 700 + M)
    nw = (np.float32(1) + synth.normal(700, 9, (D,), 0.1)).astype(np.float32)
    ws = [synth.normal(700, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    q = [oracle.quantize_weights(w) for w in ws]
    eps = float(np.finfo(np.float32).eps)
    ref = oracle.ffn(x, nw, eps, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1], q[2][0])
    pk = [B.bitlinear_pack(to_dev(w)) for w in ws]
    Y, wsp = B.bitnet_ffn_forward(to_dev(x), to_dev(nw), eps, pk[0][0], pk[0][1], pk[1][0],
                                  pk[1][1], pk[2][0], pk[2][1], D, F)
    it = {k: host(v) for k, v in B.ffn_internals(wsp, M, D, F).items()}
    np.testing.assert_array_equal(it["xn"].view(np.uint32), ref["xn"].view(np.uint32))
    np.testing.assert_array_equal(it["qx"][:, :D], ref["qx"])
    np.testing.assert_array_equal(it["h"].view(np.uint32), ref["h"].view(np.uint32))
    assert_rel(host(Y), ref["y"])


@pytest.mark.parametrize("M,K,N,bf16", [(1, 2560, 6912, False), (1, 6912, 2560, True),
                                        (1, 1, 5, False), (1, 16384, 33, False), (1, 16448, 40, False),
                                        (1, 8192, 300, True), (3, 700, 130, False), (80, 512, 200, True),
                                        # packed matrices of >= 16 MiB: the streaming GEMV
                                        (1, 8192, 28672, False), (1, 8192, 16400, True),
                                        # 2..5 tokens on large layers (quantiser, then the
                                        # streaming MFMA product), ragged K and N
                                        (2, 8192, 28672, False), (3, 1000, 25601, True),
                                        (4, 4096, 26000, False), (4, 8192, 25600, True),
                                        (2, 2052, 32000, False), (5, 1024, 25600, False),
                                        # the largest K and N
                                        (1, 65536, 100, False), (2, 65536, 40, True),
                                        (1, 100, 65536, True),
                                        (1, 5000, 13301, False), (1, 4000, 17001, True),
                                        (1, 4097, 16500, False), (1, 8192, 12001, False),
                                        (1, 4096, 40000, True)])
def test_forward_fused_from_float(M, K, N, bf16):
    d = synth.random_case(3000 + K + N, M, K, N)
    X = synth.with_outliers(d["X"], synth.outlier_columns(3000 + K, K)) if K > 100 else d["X"]
    g, t, Wp, sc = check_pack(d["W"])
    xd = to_dev(X)
    if bf16:
        xd = xd.to(torch.bfloat16)
        X = xd.float().cpu().numpy()
    q, gx, rs = oracle.act_quant(X)
    acc = oracle.int_linear(q, t)
    y = oracle.dequant(acc, gx, g)
    Y, ws = B.bitlinear_forward_fused(xd, Wp, sc, N)
    it = {k: host(v) for k, v in B.fused_internals(ws, M, K).items()}
    np.testing.assert_array_equal(it["xq"][:, :K], q)
    assert not it["xq"][:, K:].any()
    np.testing.assert_array_equal(it["x_scale"].view(np.uint32), gx.view(np.uint32))
    np.testing.assert_array_equal(it["x_rowsum"], rs)
    assert_rel(host(Y), y)
    Y2, _ = B.bitlinear_forward_fused(xd, Wp, sc, N)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


@pytest.mark.parametrize("M,K,N,bf16,nw,eps", [
    # one float32 token: the normalising GEMV (one and two chunks per lane)
    (1, 2560, 6912, False, True, 2.0 ** -23), (1, 6912, 2560, False, False, 2.0 ** -23),
    (1, 8192, 300, False, True, 1e-6), (1, 1, 5, False, True, 2.0 ** -23),
    (1, 4097, 1001, False, False, 1e-5), (1, 8192, 28672, False, True, 2.0 ** -23),
    # bfloat16 or K past 8192: RMSNorm + quantiser, then the GEMV
    (1, 6912, 2560, True, True, 2.0 ** -23), (1, 8200, 100, False, True, 1e-6),
    (1, 65536, 40, False, True, 2.0 ** -23),
    # several tokens: RMSNorm + quantiser, then the MFMA products
    (3, 700, 130, True, True, 1e-5), (8, 2560, 6912, False, True, 2.0 ** -23),
    (64, 2560, 6912, False, False, 2.0 ** -23), (80, 512, 200, True, True, 2.0 ** -23)])
def test_forward_fused_norm(M, K, N, bf16, nw, eps):
    d = synth.random_case(3500 + K + N, M, K, N)
    X = synth.with_outliers(d["X"], synth.outlier_columns(3500 + K, K)) if K > 100 else d["X"]
    g, t, Wp, sc = check_pack(d["W"])
    xd = to_dev(X)
    if bf16:
        xd = xd.to(torch.bfloat16)
        X = xd.float().cpu().numpy()
    w = (1.0 + 0.1 * synth.normal(3500, K, (K,))).astype(np.float32) if nw else None
    xn = oracle.rmsnorm(X, w, eps)
    q, gx, rs = oracle.act_quant(xn)
    acc = oracle.int_linear(q, t)
    y = oracle.dequant(acc, gx, g)
    wd = to_dev(w) if nw else None
    Y, ws = B.bitlinear_forward_fused_norm(xd, Wp, sc, N, wd, eps)
    it = {k: host(v) for k, v in B.fused_norm_internals(ws, M, K).items()}
    np.testing.assert_array_equal(it["xn"].view(np.uint32), xn.view(np.uint32))
    np.testing.assert_array_equal(it["xq"][:, :K], q)
    assert not it["xq"][:, K:].any()
    np.testing.assert_array_equal(it["x_scale"].view(np.uint32), gx.view(np.uint32))
    np.testing.assert_array_equal(it["x_rowsum"], rs)
    assert_rel(host(Y), y)
    Y2, _ = B.bitlinear_forward_fused_norm(xd, Wp, sc, N, wd, eps)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


def test_forward_fused_norm_rows_at_mean_square_midpoints():
    # one token and several: rows whose exact mean square is a binary32
    # rounding midpoint or next to one (the exact sum decides them)
    K, N = 2560, 700
    W = synth.normal(3600, 1, (N, K), 0.02)
    g, t, Wp, sc = check_pack(W)
    for M in (1, 6):
        X = synth.midpoint_rows(K, M, 3600 + M)
        xn = oracle.rmsnorm(X, None, 2.0 ** -23)
        q, gx, rs = oracle.act_quant(xn)
        y = oracle.dequant(oracle.int_linear(q, t), gx, g)
        Y, ws = B.bitlinear_forward_fused_norm(to_dev(X), Wp, sc, N)
        it = {k: host(v) for k, v in B.fused_norm_internals(ws, M, K).items()}
        np.testing.assert_array_equal(it["xn"].view(np.uint32), xn.view(np.uint32))
        np.testing.assert_array_equal(it["xq"][:, :K], q)
        assert_rel(host(Y), y)


# ----------------------------------------------------------------------------
# binary weights in the 1-bit layout

def check_pack1(W):
    g = oracle.weight_scale(W)
    t = oracle.binarize(W)
    p = oracle.pack1(t)
    Wb, sc = gpu_pack(W, B.BL_BINARY_1BIT)
    np.testing.assert_array_equal(host(Wb).view(np.uint32), p)
    assert host(sc)[0].view(np.uint32) == np.float32(g).view(np.uint32)
    return g, t, Wb, sc


def check_forward1(q, gx, t, gw, Xq, xs, xr, Wb, ws):
    K = q.shape[1]
    N = t.shape[0]
    acc = oracle.int_linear(q, t)
    y = oracle.dequant(acc, gx, gw)
    Y, A = B.bitlinear_forward_1bit(Xq, xs, xr, K, Wb, ws, N, with_acc=True)
    np.testing.assert_array_equal(host(A), acc)
    assert_rel(host(Y), y)
    Y2 = B.bitlinear_forward_1bit(Xq, xs, xr, K, Wb, ws, N)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))
    return Y


@pytest.mark.parametrize("M,K,N", [
    (1, 1, 1), (1, 64, 5), (1, 127, 33), (1, 129, 300), (1, 2560, 700), (1, 8192, 100),
    (1, 8320, 70), (1, 24640, 20), (1, 40000, 9), (2, 64, 16), (5, 129, 64), (8, 1040, 257),
    (16, 512, 400), (16, 8192, 70), (17, 63, 15), (33, 1000, 100), (64, 2560, 96),
    (65, 300, 130), (100, 1040, 257), (130, 128, 70),
    (1, 65536, 100), (8, 100, 65536), (100, 65536, 40),
])
def test_binary_1bit_ragged_shapes(M, K, N):
    d = synth.random_case(4000 + M * 7 + N, M, K, N)
    g, t, Wb, sc = check_pack1(d["W"])
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    Y = check_forward1(q, gx, t, g, Xq, xs, xr, Wb, sc)
    # the 2-bit layout of the same binary weights gives the same bits
    g2, t2, Wp, sc2 = check_pack(d["W"], "binary")
    Y2 = B.bitlinear_forward(Xq, xs, xr, K, Wp, sc2, N)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


def test_binary_1bit_signed_zero_and_degenerate_rows():
    W = synth.normal(31, 2, (40, 300))
    W[2, :] = 0.0
    W[3, :] = -0.0
    W[4, :] = -1.0
    g, t, Wb, sc = check_pack1(W)
    assert (t[2] == 1).all() and (t[3] == 1).all() and (t[4] == -1).all()
    X = synth.normal(31, 1, (3, 300))
    X[1] = 0.0
    q, gx, rs, Xq, xs, xr = check_quant(X)
    check_forward1(q, gx, t, g, Xq, xs, xr, Wb, sc)


def test_decode_100b_binary_1bit_full():
    d = synth.decode_100b()
    g, t, Wb, sc = check_pack1(d["W"])
    del d["W"]
    assert host(Wb).nbytes == 28672 * 8192 // 8
    for M in (1, 8):
        q, gx, rs, Xq, xs, xr = check_quant(d["X"][:M])
        check_forward1(q, gx, t, g, Xq, xs, xr, Wb, sc)


def test_skinny_phased_activations_large_layer():
    # 16 tokens, K = 8192, N = 25600 (1600 tiles of 16 rows): the activation
    # block does not fit next to 8 waves' weight patches and is staged in
    # phases; 2-bit ternary and 1-bit binary layouts, every column
    M, K, N = 16, 8192, 25600
    d = synth.random_case(1717, M, K, N)
    g, t, Wp, sc = check_pack(d["W"])
    g1, t1, Wb, sc1 = check_pack1(d["W"])
    del d["W"]
    q, gx, rs, Xq, xs, xr = check_quant(d["X"])
    runs = ((t, g, lambda **kw: B.bitlinear_forward(Xq, xs, xr, K, Wp, sc, N, **kw)),
            (t1, g1, lambda **kw: B.bitlinear_forward_1bit(Xq, xs, xr, K, Wb, sc1, N, **kw)))
    for tt, gw, fwd in runs:
        Y, A = fwd(with_acc=True)
        acc = oracle.int_linear(q, tt)
        np.testing.assert_array_equal(host(A), acc)
        assert_rel(host(Y), oracle.dequant(acc, gx, gw))
        Y2 = fwd()
        np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


# ----------------------------------------------------------------------------
# BitNet a4.8 split activations (int8 outliers + int4 rest)

def check_a48(X, n_out, t, g, Wp, sc, bf16=False):
    xd = to_dev(X)
    if bf16:
        xd = xd.to(torch.bfloat16)
        X = xd.float().cpu().numpy()
    M, K = X.shape
    N = t.shape[0]
    ref = oracle.bitlinear_a48(X, t, g, n_out)
    q = B.bitlinear_quant_act_a48(xd, n_out)
    h = {k: host(v) for k, v in q.items()}
    for part in ("q4", "q8"):
        np.testing.assert_array_equal(h[part][:, :K], ref[part], err_msg=part)
        assert not h[part][:, K:].any()
    for part in ("g4", "g8"):
        np.testing.assert_array_equal(h[part].view(np.uint32), ref[part].view(np.uint32), err_msg=part)
    np.testing.assert_array_equal(h["rs4"], ref["rs4"])
    np.testing.assert_array_equal(h["rs8"], ref["rs8"])
    Y, ws = B.bitlinear_forward_a48(q, K, Wp, sc, N)
    acc = host(ws)[:2 * M * N].reshape(2, M, N)
    np.testing.assert_array_equal(acc[0], ref["acc4"])
    np.testing.assert_array_equal(acc[1], ref["acc8"])
    assert_rel(host(Y), ref["y"])
    Y2, _ = B.bitlinear_forward_a48(q, K, Wp, sc, N)
    np.testing.assert_array_equal(host(Y2).view(np.uint32), host(Y).view(np.uint32))


@pytest.mark.parametrize("M,K,N,n_out,bf16", [
    (1, 2560, 6912, 26, False), (1, 6912, 2560, 69, True), (1, 8192, 300, 82, False),
    (1, 100, 40, 0, False), (1, 100, 40, 100, False), (1, 100, 40, 1000, False),
    (1, 16448, 33, 165, False), (3, 700, 130, 7, False), (16, 512, 400, 5, False),
    (64, 2560, 96, 26, True), (100, 1040, 257, 10, False), (1, 40000, 9, 400, False),
    (2, 20000, 17, 200, False), (1, 65536, 40, 655, False), (3, 65536, 24, 100, True),
    # one token on packed matrices of 16 MiB or more: one and two chunks per
    # lane, ragged K and N
    (1, 4000, 17001, 40, False), (1, 8192, 8192, 82, True), (1, 5000, 13301, 50, False),
])
def test_a48_quant_and_forward(M, K, N, n_out, bf16):
    d = synth.random_case(5000 + K + N + M, M, K, N)
    X = synth.with_outliers(d["X"], synth.outlier_columns(5000 + K, K)) if K > 100 else d["X"]
    if M > 1:
        X[1] = np.round(X[1] * 2) / 2  # ties in |x| across the threshold
    g, t, Wp, sc = check_pack(d["W"])
    check_a48(X, n_out, t, g, Wp, sc, bf16)


def test_a48_decode_100b_full():
    d = synth.decode_100b()
    g, t, Wp, sc = check_pack(d["W"])
    del d["W"]
    for M in (1, 8):
        check_a48(d["X"][:M], 82, t, g, Wp, sc)


@pytest.mark.parametrize("K", [3000, 5000])
def test_a48_quant_degenerate_rows(K):
    # rows made of ties: all equal, zeros, a block of equal maxima, few distinct values
    X = np.zeros((4, K), np.float32)
    X[1] = 1.5
    X[2, ::3] = -2.0
    X[3] = np.tile(np.float32([0.5, -0.5, 0.25, 3.0]), K // 4 + 1)[:K]
    d = synth.random_case(77 + K, 4, K, 40)
    g, t, Wp, sc = check_pack(d["W"])
    for n_out in (1, 30, 1000, K - 1):
        check_a48(X, n_out, t, g, Wp, sc)


def test_a48_stacked_and_separate_layouts_agree():
    # the stacked quantiser output (one product over 2M rows for M <= 8) and
    # the same codes in separate buffers (two products) give identical bits
    d = synth.random_case(909, 8, 3000, 500)
    X = synth.with_outliers(d["X"], synth.outlier_columns(909, 3000))
    g, t, Wp, sc = check_pack(d["W"])
    K, N = 3000, 500
    for M in (2, 8):
        q = B.bitlinear_quant_act_a48(to_dev(X[:M]), 30)
        assert q["q8"].data_ptr() == q["q4"].data_ptr() + q["q4"].numel()
        sep = {k: v.clone() for k, v in q.items()}
        Y1, ws1 = B.bitlinear_forward_a48(q, K, Wp, sc, N)
        Y2, ws2 = B.bitlinear_forward_a48(sep, K, Wp, sc, N)
        np.testing.assert_array_equal(host(ws1)[:2 * M * N], host(ws2)[:2 * M * N])
        np.testing.assert_array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))
        ref = oracle.bitlinear_a48(X[:M], t, g, 30)
        acc = host(ws1)[:2 * M * N].reshape(2, M, N)
        np.testing.assert_array_equal(acc[0], ref["acc4"])
        np.testing.assert_array_equal(acc[1], ref["acc8"])
