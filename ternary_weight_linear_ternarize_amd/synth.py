"""Seeded synthetic inputs for the BitLinear workloads.

This module only draws random numbers; it holds none of the method's
arithmetic (no scales, no rounding, no packing).  The same buffers feed the
HIP path and the CPU oracle.

Each tensor has its own stream: ``numpy.random.Generator(PCG64(SeedSequence(
[seed, tensor_id])))``, values from ``standard_normal(dtype=float32)`` and,
where a standard deviation other than 1 is asked for, one binary32 multiply
by that constant.  Weight tensors are drawn as ~N(0, 0.02^2), the
initialisation of the BitLinear listing on the youngju.dev page (section
"BitNet b1.58"), unless a workload says otherwise.
"""
import math

import numpy as np

# Workload shapes (M tokens, K in features, N out features).
SINGLE = dict(M=16, K=512, N=400, seed=0)            # one BitLinear(512, 400)
DECODE_2B = dict(M=1, K=2560, N=6912, seed=1)         # 2B-class decode GEMV (+ down 6912->2560)
PREFILL_2B = dict(M=2048, K=2560, N=6912, seed=2)     # prefill GEMM, weights of DECODE_2B up
FFN_2B = dict(M_list=(1, 8, 64), D=2560, F=6912, seed=3)
DECODE_100B = dict(M_list=(1, 8), K=8192, N=28672, seed=4)

# tensor ids inside a workload seed
T_W, T_X, T_W2, T_X2, T_W3, T_NORM, T_OUTLIER, T_SUBLN = range(8)


def _gen(seed, tensor_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def normal(seed, tensor_id, shape, std=1.0):
    """float32 array ~ N(0, std^2) of the given shape."""
    a = _gen(seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def outlier_columns(seed, K, frac=0.01):
    """Distinct column indices (round(frac*K) of them), sorted."""
    n = int(round(frac * K))
    cols = _gen(seed, T_OUTLIER).choice(K, size=n, replace=False)
    return np.sort(cols)


def with_outliers(x, cols, factor=20.0):
    """Copy of x with the given columns multiplied by factor (same for all tokens)."""
    y = np.array(x, dtype=np.float32, copy=True)
    y[:, cols] *= np.float32(factor)
    return y


def single_layer():
    c = SINGLE
    return {"W": normal(c["seed"], T_W, (c["N"], c["K"])),
            "X": normal(c["seed"], T_X, (c["M"], c["K"]))}


def decode_2b(with_down=True):
    c = DECODE_2B
    out = {"W_up": normal(c["seed"], T_W, (c["N"], c["K"]), 0.02),
           "x": normal(c["seed"], T_X, (1, c["K"]))}
    if with_down:
        out["W_down"] = normal(c["seed"], T_W2, (c["K"], c["N"]), 0.02)
        out["x_d"] = normal(c["seed"], T_X2, (1, c["N"]))
    return out


def prefill_2b(with_weights=True):
    c = PREFILL_2B
    out = {"X": normal(c["seed"], T_X, (c["M"], c["K"]))}
    if with_weights:
        out["W"] = decode_2b(with_down=False)["W_up"]
    return out


def ffn_2b(norm="ones"):
    c = FFN_2B
    D, F, s = c["D"], c["F"], c["seed"]
    out = {"H": normal(s, T_X, (max(c["M_list"]), D)),
           "W_gate": normal(s, T_W, (F, D), 0.02),
           "W_up": normal(s, T_W2, (F, D), 0.02),
           "W_down": normal(s, T_W3, (D, F), 0.02)}
    if norm == "ones":
        out["norm_w"] = np.ones(D, dtype=np.float32)
    else:
        out["norm_w"] = (np.float32(1.0) + normal(s, T_NORM, (D,), 0.1)).astype(np.float32)
    # SubLN weight over F (used only by the SubLN variant of the block)
    out["subln_w"] = (np.float32(1.0) + normal(s, T_SUBLN, (F,), 0.1)).astype(np.float32)
    return out


def decode_100b(with_weights=True):
    c = DECODE_100B
    K, N, s = c["K"], c["N"], c["seed"]
    x = normal(s, T_X, (max(c["M_list"]), K))
    out = {"X": with_outliers(x, outlier_columns(s, K)), "outlier_cols": outlier_columns(s, K)}
    if with_weights:
        out["W"] = normal(s, T_W, (N, K), 0.02)
    return out


def random_case(seed, M, K, N, w_std=0.02):
    """Small random layer for sweeps over ragged shapes."""
    return {"W": normal(seed, T_W, (N, K), w_std), "X": normal(seed, T_X, (M, K))}


def _sum_of_squares(target):
    """Integers a_i < 2^24 whose squares add up to target (greedy)."""
    out = []
    while target > 0:
        a = math.isqrt(target)
        out.append(a)
        target -= a * a
    assert all(a < 2 ** 24 for a in out)
    return out


def midpoint_rows(D, count, seed):
    """Rows whose exact mean square sum(x^2) / D equals a number with an odd
    25-bit significand (a binary32 rounding midpoint), or lies one unit of the
    integer sum away from it.  Each row is a few nonzero entries a * 2^e with
    integers a < 2^24 (exact in binary32) at random positions and signs: the
    integer square sum is chosen first and written as a sum of squares."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(count):
        odd = (1 << 24) + 2 * int(rng.integers(0, 1 << 23)) + 1
        target = D * odd + (0, 1, -1)[i % 3]
        a = np.array(_sum_of_squares(target), np.float64)
        row = np.zeros(D, np.float32)
        pos = rng.choice(D, size=len(a), replace=False)
        e = int(rng.integers(-40, -10))
        sign = np.where(rng.random(len(a)) < 0.5, -1.0, 1.0)
        row[pos] = (sign * np.ldexp(a, e)).astype(np.float32)
        rows.append(row)
    return np.stack(rows)
