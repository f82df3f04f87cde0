"""Layer objects over the C ABI, for code written against the pages' PyTorch
BitLinear (ai-heartland.com "BitNet — 1-bit Transformersの実装ライブラリ",
"BitLinear層の基本実装": used where nn.Linear was) and the BitNet feed-forward
block (youngju.dev "BitNet論文分析", "BitNet b1.58"; reinforz.co.jp: ReLU²).

Marshalling only, like ``binding``: the weights are packed once by
``bitlinear_pack`` when the layer is built, and every call is one library
call on the current stream.  Inputs are device tensors; any leading
dimensions are flattened into tokens.  No bias ([P5] reinforz.co.jp).
"""
import torch

from . import binding as B


def _tokens(x, K, name):
    if not isinstance(x, torch.Tensor) or x.dim() < 1 or x.shape[-1] != K:
        raise ValueError(f"{name} must be a tensor whose last dimension is {K}")
    return x.reshape(-1, K).contiguous()


class BitLinear:
    """y = BitLinear(x) for a float32 weight [N, K] (out, in features).

    mode: B.BL_TERNARY (absmean ternary weights, BitNet b1.58), B.BL_BINARY
    (sign weights in the 2-bit layout) or B.BL_BINARY_1BIT (sign weights, one
    bit each).  x [..., K] float32 or bfloat16 -> y [..., N] float32: the
    per-token int8 quantisation, the ternary product and the dequantisation
    (one fused call for the 2-bit layouts).  a48_outliers = n (2-bit layouts
    only) takes the BitNet a4.8 activations instead (youngju.dev "BitNet
    a4.8"): per token the n largest |x| in 8 bits, the rest in 4 bits.
    norm=True (ternary and binary 2-bit layouts, int8 activations) puts the
    layer's own RMSNorm in front of the quantiser, as the BitLinear_b158 forward
    of youngju.dev "BitNet b1.58" does: norm_weight [K] float32 (None = ones)
    and norm_eps, all in the same fused call."""

    def __init__(self, weight, mode=B.BL_TERNARY, a48_outliers=None, norm=False,
                 norm_weight=None, norm_eps=2.0 ** -23):
        if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
            raise ValueError("weight must be a 2-D tensor [out_features, in_features]")
        self.out_features, self.in_features = (int(d) for d in weight.shape)
        self.mode = mode
        if a48_outliers is not None and mode == B.BL_BINARY_1BIT:
            raise ValueError("a4.8 activations run on the 2-bit layouts")
        if norm and (a48_outliers is not None or mode == B.BL_BINARY_1BIT):
            raise ValueError("the normalising layer takes int8 activations on the 2-bit layouts")
        if norm_weight is not None and not norm:
            raise ValueError("norm_weight needs norm=True")
        self.a48_outliers = a48_outliers
        self.norm, self.norm_weight, self.norm_eps = norm, norm_weight, norm_eps
        self.weight_packed, self.weight_scale = B.bitlinear_pack(weight.contiguous(), mode)
        self._ws = {}

    def _workspace(self, M, device):
        key = (M, device)
        if key not in self._ws:
            make = B.fused_norm_workspace if self.norm else B.fused_workspace
            self._ws = {key: make(M, self.in_features, device)}
        return self._ws[key]

    def __call__(self, x):
        X = _tokens(x, self.in_features, "x")
        N, K = self.out_features, self.in_features
        if self.a48_outliers is not None:
            q = B.bitlinear_quant_act_a48(X, self.a48_outliers)
            Y, _ = B.bitlinear_forward_a48(q, K, self.weight_packed, self.weight_scale, N)
        elif self.mode == B.BL_BINARY_1BIT:
            Xq, xs, xr = B.bitlinear_quant_act(X)
            Y = B.bitlinear_forward_1bit(Xq, xs, xr, K, self.weight_packed, self.weight_scale, N)
        elif self.norm:
            Y, _ = B.bitlinear_forward_fused_norm(X, self.weight_packed, self.weight_scale, N,
                                                  self.norm_weight, self.norm_eps,
                                                  ws=self._workspace(X.shape[0], X.device))
        else:
            Y, _ = B.bitlinear_forward_fused(X, self.weight_packed, self.weight_scale, N,
                                             ws=self._workspace(X.shape[0], X.device))
        return Y.reshape(*x.shape[:-1], N)


class BitNetFFN:
    """RMSNorm -> int8 quant -> gate/up BitLinears -> relu(gate)^2 * up ->
    [SubLN ->] int8 requant -> down BitLinear, from float32 weights gate and
    up [F, D] and down [D, F].  h [..., D] float32 or bfloat16 -> y [..., D]
    float32.  norm_weight (RMSNorm over D, None = ones) and subln_weight (the
    optional norm of h over F) are float32 device tensors."""

    def __init__(self, w_gate, w_up, w_down, norm_weight=None, norm_eps=2.0 ** -23,
                 subln_weight=None, subln_eps=2.0 ** -23):
        self.F, self.D = (int(d) for d in w_gate.shape)
        if tuple(w_up.shape) != (self.F, self.D) or tuple(w_down.shape) != (self.D, self.F):
            raise ValueError("expected gate and up [F, D] and down [D, F]")
        self.gate = B.bitlinear_pack(w_gate.contiguous())
        self.up = B.bitlinear_pack(w_up.contiguous())
        self.down = B.bitlinear_pack(w_down.contiguous())
        self.norm_weight, self.norm_eps = norm_weight, norm_eps
        self.subln_weight, self.subln_eps = subln_weight, subln_eps
        self._ws = {}

    def __call__(self, h):
        H = _tokens(h, self.D, "h")
        key = (H.shape[0], H.device)
        ws = self._ws.get(key)
        Y, ws = B.bitnet_ffn_forward(H, self.norm_weight, self.norm_eps, *self.gate, *self.up,
                                     *self.down, self.D, self.F, ws=ws,
                                     subln_w=self.subln_weight, subln_eps=self.subln_eps)
        self._ws = {key: ws}
        return Y.reshape(*h.shape[:-1], self.D)
