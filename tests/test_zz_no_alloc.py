"""GPU: the allocation-free FFN entry point (bitnet_ffn_forward_static, the
library's static per-GPU scratch) against bitnet_ffn_forward with a caller
workspace, bit for bit, on two calls in a row -- the second with a smaller
input, so stale scratch contents from the first call must not leak in."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_ternarize_amd import binding as B
from ternary_weight_linear_ternarize_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _layer(seed, M, D, F):
    x = synth.normal(seed, 1, (M, D))
    ws = [synth.normal(seed, 2 + i, shp, 0.02) for i, shp in enumerate(((F, D), (F, D), (D, F)))]
    nw = (np.float32(1) + synth.normal(seed, 9, (D,), 0.1)).astype(np.float32)
    return x, ws, nw


def _run_both(seed, M, D, F, subln):
    x, ws, nw = _layer(seed, M, D, F)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    pk = [B.bitlinear_pack(to(w)) for w in ws]
    eps = float(np.finfo(np.float32).eps)
    sw = to((np.float32(1) + synth.normal(seed, 10, (F,), 0.1)).astype(np.float32)) if subln else None
    args = (to(x), to(nw), eps, pk[0][0], pk[0][1], pk[1][0], pk[1][1], pk[2][0], pk[2][1], D, F)
    Y_ws, _ = B.bitnet_ffn_forward(*args, subln_w=sw, subln_eps=eps)
    Y_st = B.bitnet_ffn_forward_static(*args, subln_w=sw, subln_eps=eps)
    torch.cuda.synchronize()
    return x, ws, nw, Y_ws.cpu().numpy(), Y_st.cpu().numpy()


@pytest.mark.parametrize("first,second", [((64, 2560, 6912, False), (8, 2560, 6912, False)),
                                          ((40, 1000, 3000, True), (1, 300, 700, True)),
                                          ((8, 2560, 6912, False), (1, 2560, 6912, False))])
def test_static_scratch_matches_workspace_entry_point(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for i, (M, D, F, subln) in enumerate((first, second)):
        x, ws, nw, y_ws, y_st = _run_both(900 + 10 * i + M, M, D, F, subln)
        np.testing.assert_array_equal(y_st.view(np.uint32), y_ws.view(np.uint32))
    # the second (smaller) call also against the oracle
    q = [oracle.quantize_weights(w) for w in ws]
    eps = float(np.finfo(np.float32).eps)
    sw = (np.float32(1) + synth.normal(900 + 10 + M, 10, (F,), 0.1)).astype(np.float32) if subln else None
    ref = oracle.ffn(x, nw, eps, q[0][1], q[0][0], q[1][1], q[1][0], q[2][1], q[2][0],
                     subln=subln, subln_w=sw, subln_eps=eps)
    err = np.abs(y_st.astype(np.float64) - ref["y"]) / np.maximum(np.abs(ref["y"].astype(np.float64)), 1e-30)
    assert err.max(initial=0.0) <= 1e-5


def test_static_scratch_rejects_shapes_beyond_its_size():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, D, F = 512, 2560, 6912
    assert B.lib().bitnet_ffn_workspace_bytes(M, D, F) > B.FFN_STATIC_SCRATCH_BYTES
    H = torch.zeros((M, D), device=DEV)
    Wg = torch.zeros((F, D // 16), dtype=torch.int32, device=DEV)
    Wd = torch.zeros((D, B.padded_k(F) // 16), dtype=torch.int32, device=DEV)
    sc = torch.ones(1, device=DEV)
    with pytest.raises(B.BitLinearError) as e:
        B.bitnet_ffn_forward_static(H, None, 1e-6, Wg, sc, Wg, sc, Wd, sc, D, F)
    assert e.value.status == B.BL_ESHAPE
