"""HIP graph capture of the library's calls (GPU).

Every entry point enqueues kernels only (no allocation, no memset, no
synchronisation), so a sequence of calls can be captured once and replayed.
Each case captures the calls with caller-owned outputs and workspaces, then
replays the graph three times; before every replay the outputs are filled
with NaN and the workspaces with a byte pattern, and between replays the same
calls run eagerly.  Every replay must reproduce the eager result bit for bit
(outputs and the internal codes, scales and accumulators the workspaces hold).
"""
import numpy as np
import pytest
import torch

from ternary_weight_linear_ternarize_amd import binding as B
from ternary_weight_linear_ternarize_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def snapshot(tensors):
    torch.cuda.synchronize()
    return [t.detach().cpu().numpy().copy() for t in tensors]


def same_bits(a, b):
    assert a.dtype == b.dtype and a.shape == b.shape
    np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))


def check_replays(call, outputs, scratch, checked):
    """call() enqueues the work; outputs are filled with NaN and scratch with
    0xA5 before each replay; checked (outputs and workspaces) must match the
    eager bits after every replay."""
    call()
    ref = snapshot(checked)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        for t in outputs:
            t.fill_(float("nan"))
        for t in scratch:
            t.view(torch.uint8).fill_(0xA5)
        g.replay()
        got = snapshot(checked)
        for a, b in zip(got, ref):
            same_bits(a, b)
        call()  # eager work between replays
        for a, b in zip(snapshot(checked), ref):
            same_bits(a, b)


@pytest.mark.parametrize("M,subln", [(1, False), (8, False), (32, False), (64, False), (1, True),
                                     (8, True)])
def test_graph_ffn(M, subln):
    f = synth.ffn_2b()
    D, F = synth.FFN_2B["D"], synth.FFN_2B["F"]
    packs = [B.bitlinear_pack(to_dev(f[k])) for k in ("W_gate", "W_up", "W_down")]
    H = to_dev(f["H"][:M])
    sw = to_dev(f["subln_w"]) if subln else None
    eps = float(np.finfo(np.float32).eps)
    ws = torch.empty(B.lib().bitnet_ffn_workspace_bytes(M, D, F), dtype=torch.uint8, device=DEV)
    Y = torch.empty((M, D), dtype=torch.float32, device=DEV)
    (g, gs), (u, us), (d, ds) = packs

    def call():
        B.bitnet_ffn_forward(H, None, eps, g, gs, u, us, d, ds, D, F, out=Y, ws=ws,
                             subln_w=sw, subln_eps=eps)

    inner = B.ffn_internals(ws, M, D, F)
    keys = [k for k in sorted(inner) if subln or k != "hn"]  # hn is written by SubLN only
    checked = [Y] + [inner[k] for k in keys]
    check_replays(call, [Y], [ws], checked)


def test_graph_fused_and_plain_forward():
    d = synth.decode_2b()
    K, N = synth.DECODE_2B["K"], synth.DECODE_2B["N"]
    Wp, sc = B.bitlinear_pack(to_dev(d["W_up"]))
    x = to_dev(d["x"])
    ws = B.fused_workspace(1, K, DEV)
    Y1 = torch.empty((1, N), dtype=torch.float32, device=DEV)
    X = to_dev(synth.normal(5, 1, (40, K)))
    q = B.bitlinear_quant_act(X)
    Y2 = torch.empty((40, N), dtype=torch.float32, device=DEV)
    X8 = to_dev(synth.normal(6, 1, (8, K)))  # 8 tokens: K split over the waves of a block
    q8 = B.bitlinear_quant_act(X8)
    Y3 = torch.empty((8, N), dtype=torch.float32, device=DEV)

    def call():
        B.bitlinear_forward_fused(x, Wp, sc, N, out=Y1, ws=ws)
        B.bitlinear_quant_act(X, out=q)
        B.bitlinear_forward(q[0], q[1], q[2], K, Wp, sc, N, out=Y2)
        B.bitlinear_quant_act(X8, out=q8)
        B.bitlinear_forward(q8[0], q8[1], q8[2], K, Wp, sc, N, out=Y3)

    inner = B.fused_internals(ws, 1, K)
    checked = [Y1, Y2, Y3, q[0], q[1], q[2], q8[0]] + [inner[k] for k in sorted(inner)]
    check_replays(call, [Y1, Y2, Y3], [ws, q[0], q8[0]], checked)


@pytest.mark.parametrize("M", [1, 6])
def test_graph_fused_norm_forward(M):
    # one token: the normalising GEMV; several: RMSNorm + quantiser, product
    d = synth.decode_2b()
    K, N = synth.DECODE_2B["K"], synth.DECODE_2B["N"]
    Wp, sc = B.bitlinear_pack(to_dev(d["W_up"]))
    X = to_dev(synth.normal(6, 1, (M, K)))
    nw = to_dev((1.0 + 0.1 * synth.normal(6, 2, (K,))).astype(np.float32))
    ws = B.fused_norm_workspace(M, K, DEV)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)

    def call():
        B.bitlinear_forward_fused_norm(X, Wp, sc, N, nw, 1e-6, out=Y, ws=ws)

    inner = B.fused_norm_internals(ws, M, K)
    checked = [Y] + [inner[k] for k in sorted(inner)]
    check_replays(call, [Y], [ws], checked)


def test_graph_1bit_and_a48():
    d = synth.random_case(606, 8, 3000, 700)
    K, N = 3000, 700
    X = synth.with_outliers(d["X"], synth.outlier_columns(606, K))
    Wb, sb = B.bitlinear_pack(to_dev(d["W"]), B.BL_BINARY_1BIT)
    Wp, sc = B.bitlinear_pack(to_dev(d["W"]))
    Xd = to_dev(X)
    q = B.bitlinear_quant_act(Xd)
    Yb = torch.empty((8, N), dtype=torch.float32, device=DEV)
    qa = B.bitlinear_quant_act_a48(Xd, 30)
    Ya = torch.empty((8, N), dtype=torch.float32, device=DEV)
    wsa = torch.empty(B.lib().bitlinear_a48_workspace_bytes(8, N) // 4, dtype=torch.int32,
                      device=DEV)

    def call():
        B.bitlinear_forward_1bit(q[0], q[1], q[2], K, Wb, sb, N, out=Yb)
        B.bitlinear_quant_act_a48(Xd, 30, out=qa)
        B.bitlinear_forward_a48(qa, K, Wp, sc, N, out=Ya, ws=wsa)

    checked = [Yb, Ya, wsa[:2 * 8 * N]] + [qa[k] for k in sorted(qa)]  # acc4, acc8
    check_replays(call, [Yb, Ya], [wsa], checked)
