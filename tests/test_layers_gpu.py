"""GPU parity of the layer objects (ternary_weight_linear_ternarize_amd.layers)
against the CPU oracle: they only marshal, so their outputs must equal the
oracle's for every token, whatever the leading dimensions."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_ternarize_amd import binding as B
from ternary_weight_linear_ternarize_amd import layers, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _rel(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    assert y.shape == ref.shape
    return float((np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)).max(initial=0.0))


@pytest.mark.parametrize("mode", [B.BL_TERNARY, B.BL_BINARY, B.BL_BINARY_1BIT])
def test_bitlinear_layer_matches_oracle(mode):
    W = synth.normal(71, 1, (400, 520))
    X = synth.normal(71, 2, (2, 3, 520))
    layer = layers.BitLinear(_dev(W), mode)
    Y = layer(_dev(X))
    assert tuple(Y.shape) == (2, 3, 400) and Y.dtype == torch.float32
    g, t, _ = oracle.quantize_weights(W, "ternary" if mode == B.BL_TERNARY else "binary")
    q, gx, _ = oracle.act_quant(X.reshape(-1, 520))
    ref = oracle.dequant(oracle.int_linear(q, t), gx, g).reshape(2, 3, 400)
    assert _rel(_host(Y), ref) <= 1e-5
    # one token without leading dimensions, and bfloat16 input
    xb = _dev(X[0, 0]).to(torch.bfloat16)
    y1 = layer(xb)
    assert tuple(y1.shape) == (400,)
    qb, gb, _ = oracle.act_quant(xb.float().cpu().numpy()[None])
    assert _rel(_host(y1), oracle.dequant(oracle.int_linear(qb, t), gb, g)[0]) <= 1e-5
    with pytest.raises(ValueError):
        layer(_dev(X[..., :500]))


def test_bitlinear_layer_a48_matches_oracle():
    W = synth.normal(73, 1, (300, 700))
    X = synth.normal(73, 2, (2, 5, 700))
    layer = layers.BitLinear(_dev(W), a48_outliers=7)
    Y = layer(_dev(X))
    assert tuple(Y.shape) == (2, 5, 300)
    g, t, _ = oracle.quantize_weights(W, "ternary")
    ref = oracle.bitlinear_a48(X.reshape(-1, 700), t, g, 7)["y"]
    assert _rel(_host(Y).reshape(-1, 300), ref) <= 1e-5
    with pytest.raises(ValueError):
        layers.BitLinear(_dev(W), B.BL_BINARY_1BIT, a48_outliers=7)


@pytest.mark.parametrize("mode,with_w", [(B.BL_TERNARY, True), (B.BL_BINARY, False)])
def test_bitlinear_layer_with_its_norm_matches_oracle(mode, with_w):
    W = synth.normal(74, 1, (333, 640))
    X = synth.normal(74, 2, (3, 640))
    nw = (np.float32(1) + synth.normal(74, 3, (640,), 0.1)).astype(np.float32) if with_w else None
    layer = layers.BitLinear(_dev(W), mode, norm=True,
                             norm_weight=_dev(nw) if with_w else None, norm_eps=1e-6)
    g, t, _ = oracle.quantize_weights(W, "ternary" if mode == B.BL_TERNARY else "binary")
    for x in (X, X[:1]):  # several tokens, and one (the one-kernel path)
        xn = oracle.rmsnorm(x, nw, 1e-6)
        q, gx, _ = oracle.act_quant(xn)
        ref = oracle.dequant(oracle.int_linear(q, t), gx, g)
        assert _rel(_host(layer(_dev(x))), ref) <= 1e-5
    with pytest.raises(ValueError):
        layers.BitLinear(_dev(W), B.BL_BINARY_1BIT, norm=True)
    with pytest.raises(ValueError):
        layers.BitLinear(_dev(W), norm_weight=_dev(np.ones(640, np.float32)))


@pytest.mark.parametrize("subln", [False, True])
def test_ffn_layer_matches_oracle(subln):
    D, F = 256, 600
    x = synth.normal(72, 1, (2, 4, D))
    ws = [synth.normal(72, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    nw = (np.float32(1) + synth.normal(72, 9, (D,), 0.1)).astype(np.float32)
    sw = (np.float32(1) + synth.normal(72, 10, (F,), 0.1)).astype(np.float32) if subln else None
    ffn = layers.BitNetFFN(*[_dev(w) for w in ws], norm_weight=_dev(nw), norm_eps=1e-6,
                           subln_weight=_dev(sw) if subln else None, subln_eps=1e-5)
    Y = ffn(_dev(x))
    assert tuple(Y.shape) == (2, 4, D)
    q = [oracle.quantize_weights(w) for w in ws]
    ref = oracle.ffn(x.reshape(-1, D), nw, 1e-6, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1],
                     q[2][0], subln=subln, subln_w=sw, subln_eps=1e-5)
    assert _rel(_host(Y).reshape(-1, D), ref["y"]) <= 1e-5
    # a second call with another token count reuses nothing stale
    y1 = ffn(_dev(x[0, 0]))
    assert _rel(_host(y1), ref["y"][0]) <= 1e-5
