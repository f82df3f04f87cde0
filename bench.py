"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Default workload: the 2B-class decode step, one token through a 2560 -> 6912
BitLinear and the 6912 -> 2560 down-projection (ternary weights, 2-bit
packed; fp32 activations quantised per token to int8).  One step = the up
BitLinear and the down BitLinear, each one fused launch (per-token absmax
quantisation, ternary x int8 GEMV, dequant).  Weights are packed once before
timing (the pages describe packing as a one-time conversion).  The timed
steps rotate over enough distinct copies of the packed weights (> 512 MB,
more than twice the 256 MB last-level cache, read cyclically) that every step
streams its weights from HBM.  --warmup W untimed steps, then exactly --steps
K timed steps, each set launched as one HIP graph (the replay is checked
against the eager result first; the timed graph is replayed once beforehand
as preparation, see main()).

value = packed-weight bytes of both projections per step / wall time per
step (GB/s) between synchronisations around the K steps: every kernel, the
gaps between them and the graph launch included.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-extra]
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The decode step's two kernels (template instances the fused forward
# launches for these shapes).  Their HBM traffic per launch comes from the
# rocprofv3 counter summary committed under profiles/, and is reported only
# while the kernel sources are the ones those counters were taken on.
DECODE_GEMVS = {
    "up": ("gemv_kernel<1,4,0,1,512>", "2560->6912"),
    "down": ("gemv_kernel<2,2,0,1,512>", "6912->2560"),
}
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_fused_decode_2b.md")
CSRC = os.path.join(ROOT, "ternary_weight_linear_ternarize_amd", "csrc")

METRIC = ("BitLinear W1.58A8: decode GEMV weight GB/s (% HBM peak); "
          "prefill int8 TOPS (% MFMA)")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POPS)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", choices=["decode", "prefill", "decode100b", "decode100b_1bit", "a48",
                                       "ffn", "pack", "copy", "floors"],
                    help="run one workload's kernels eagerly --steps times and exit "
                         "(for profilers); prints a short JSON line")
    ap.add_argument("--subln", action="store_true",
                    help="with --only ffn: the SubLN variant of the block")
    return ap.parse_args()


def only_workload(args):
    """Eager launches of one workload (rotating weight copies), for rocprofv3."""
    import torch
    from ternary_weight_linear_ternarize_amd import binding as B
    from ternary_weight_linear_ternarize_amd import synth
    dev = torch.device("cuda:0")
    B.lib()
    n = args.steps
    if args.only == "copy":
        a = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)  # 256 MiB
        b = torch.empty_like(a)
        for _ in range(n):
            b.copy_(a)
        torch.cuda.synchronize()
        return {"only": "copy", "bytes_per_launch": a.numel() * 4, "launches": n}
    if args.only == "floors":
        # one-shot reads of the 2B-class (4,423,680 B) and 100B-class (58,720,256 B)
        # packed matrices, rotating over copies, and an empty kernel
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)
        for nbytes in (4423680, 58720256):
            ncp = max(2, int(np.ceil(600e6 / nbytes)))
            bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(ncp)]
            for i in range(n):
                B.probe_read(bufs[i % ncp], 4, sink)
            del bufs
        for i in range(n):
            B.probe_empty(dev)
        torch.cuda.synchronize()
        return {"only": "floors", "launches_per_shape": n}
    if args.only == "decode":
        d = synth.decode_2b()
        K, N = synth.DECODE_2B["K"], synth.DECODE_2B["N"]
        Wup, sup = B.bitlinear_pack(torch.from_numpy(d["W_up"]).to(dev))
        Wdn, sdn = B.bitlinear_pack(torch.from_numpy(d["W_down"]).to(dev))
        copies = max(2, int(np.ceil(600e6 / (2 * Wup.numel() * 4))))
        ups = [Wup.clone() for _ in range(copies)]
        dns = [Wdn.clone() for _ in range(copies)]
        x = torch.from_numpy(d["x"]).to(dev)
        xd = torch.from_numpy(d["x_d"]).to(dev)
        ws1, ws2 = B.fused_workspace(1, K, dev), B.fused_workspace(1, N, dev)
        y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        y2 = torch.empty((1, K), dtype=torch.float32, device=dev)
        for i in range(n):
            B.bitlinear_forward_fused(x, ups[i % copies], sup, N, out=y1, ws=ws1)
            B.bitlinear_forward_fused(xd, dns[i % copies], sdn, K, out=y2, ws=ws2)
    elif args.only == "prefill":
        c = synth.PREFILL_2B
        M, K, N = c["M"], c["K"], c["N"]
        p = synth.prefill_2b()
        Wp, sc = B.bitlinear_pack(torch.from_numpy(p["W"]).to(dev))
        q = B.bitlinear_quant_act(torch.from_numpy(p["X"]).to(dev))
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        cps = [Wp.clone() for _ in range(4)]
        for i in range(n):
            B.bitlinear_forward(q[0], q[1], q[2], K, cps[i % 4], sc, N, out=Y)
    elif args.only == "decode100b":
        c = synth.DECODE_100B
        K, N = c["K"], c["N"]
        p = synth.decode_100b()
        Wp, sc = B.bitlinear_pack(torch.from_numpy(p["W"]).to(dev))
        del p["W"]
        ncp = max(2, int(np.ceil(600e6 / (Wp.numel() * 4))))
        cps = [Wp.clone() for _ in range(ncp)]
        for M in (1, 8):
            q = B.bitlinear_quant_act(torch.from_numpy(p["X"][:M]).to(dev))
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            for i in range(n):
                B.bitlinear_forward(q[0], q[1], q[2], K, cps[i % ncp], sc, N, out=Y)
    elif args.only == "decode100b_1bit":
        c = synth.DECODE_100B
        K, N = c["K"], c["N"]
        p = synth.decode_100b()
        Wb, sc = B.bitlinear_pack(torch.from_numpy(p["W"]).to(dev), B.BL_BINARY_1BIT)
        del p["W"]
        ncp = max(2, int(np.ceil(600e6 / (Wb.numel() * 4))))
        cps = [Wb.clone() for _ in range(ncp)]
        for M in (1, 8):
            q = B.bitlinear_quant_act(torch.from_numpy(p["X"][:M]).to(dev))
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            for i in range(n):
                B.bitlinear_forward_1bit(q[0], q[1], q[2], K, cps[i % ncp], sc, N, out=Y)
    elif args.only == "a48":
        c = synth.DECODE_100B
        K, N = c["K"], c["N"]
        p = synth.decode_100b()
        Wp, sc = B.bitlinear_pack(torch.from_numpy(p["W"]).to(dev))
        del p["W"]
        ncp = max(2, int(np.ceil(600e6 / (Wp.numel() * 4))))
        cps = [Wp.clone() for _ in range(ncp)]
        n_out = int(round(0.01 * K))
        for M in (1, 8):
            Xm = torch.from_numpy(p["X"][:M]).to(dev)
            q = B.bitlinear_quant_act_a48(Xm, n_out)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            wsa = torch.empty(B.lib().bitlinear_a48_workspace_bytes(M, N) // 4, dtype=torch.int32,
                              device=dev)
            for i in range(n):
                B.bitlinear_quant_act_a48(Xm, n_out, out=q)
                B.bitlinear_forward_a48(q, K, cps[i % ncp], sc, N, out=Y, ws=wsa)
    elif args.only == "pack":
        # weight preparation of the 100B-class matrix (absmean scale + packing), each layout
        p = synth.decode_100b()
        Wd = torch.from_numpy(p["W"]).to(dev)
        del p
        for mode in (B.BL_TERNARY, B.BL_BINARY, B.BL_BINARY_1BIT):
            for i in range(n):
                B.bitlinear_pack(Wd, mode)
    elif args.only == "ffn":
        c = synth.FFN_2B
        D, F = c["D"], c["F"]
        f = synth.ffn_2b()
        packs = [B.bitlinear_pack(torch.from_numpy(f[k]).to(dev)) for k in ("W_gate", "W_up", "W_down")]
        wbytes = sum(pk[0].numel() * 4 for pk in packs)
        ncp = max(2, int(np.ceil(600e6 / wbytes)))
        cps = [[(pk[0].clone(), pk[1]) for pk in packs] for _ in range(ncp)]
        eps = float(np.finfo(np.float32).eps)
        for M in c["M_list"]:
            H = torch.from_numpy(f["H"][:M]).to(dev)
            ws = torch.empty(B.lib().bitnet_ffn_workspace_bytes(M, D, F), dtype=torch.uint8, device=dev)
            Y = torch.empty((M, D), dtype=torch.float32, device=dev)
            sw = torch.from_numpy(f["subln_w"]).to(dev) if args.subln else None
            for i in range(n):
                g, u, dn = cps[i % ncp]
                B.bitnet_ffn_forward(H, None, eps, g[0], g[1], u[0], u[1], dn[0], dn[1], D, F,
                                     out=Y, ws=ws, subln_w=sw, subln_eps=eps)
    torch.cuda.synchronize()
    return {"only": args.only, "launches_per_shape": n}


def sources_hash():
    """sha256 (first 12 hex digits) of the HIP sources and headers."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:12]


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if
    it was taken on the current sources; (None, reason) otherwise."""
    import re
    cur = sources_hash()
    if not os.path.exists(TRAFFIC_PROFILE):
        return None, "no counter profile"
    pat = re.compile(r"^traffic: (\S+) (\d+) B/launch \(sources ([0-9a-f]{12})\)")
    seen = False
    for line in open(TRAFFIC_PROFILE):
        m = pat.match(line.strip())
        if m and m.group(1) == kernel:
            seen = True
            if m.group(3) == cur:
                return int(m.group(2)), f"{os.path.relpath(TRAFFIC_PROFILE, ROOT)} (sources {cur})"
    why = "counters taken on other sources" if seen else "kernel not in the counter profile"
    return None, f"{why}; current sources {cur}"


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def event_time_per_launch(fn, n, torch):
    """Average duration of fn()'s kernel(s), from an event pair around each
    launch on the current stream (the one the binding launches on)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return float(np.mean(ms)), float(np.median(ms))


def capture(fn, n, torch, skip_warm=False):
    """HIP graph of fn(0..n-1) launched back to back on a capture stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if not skip_warm:
        with torch.cuda.stream(s):
            for i in range(min(n, 2)):  # eager warm-up on s
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def graph_time_per_launch(fn, n, reps, torch):
    """Average time per fn() inside a replayed graph of n launches, from one
    event pair around `reps` replays on the replay stream."""
    g = capture(fn, n, torch)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (n * reps)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for {args.gpus}); splitting the "
              "layers across GPUs is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.only:
        print(json.dumps(only_workload(args)), flush=True)
        return

    import torch
    from ternary_weight_linear_ternarize_amd import binding as B
    from ternary_weight_linear_ternarize_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()

    # ---------------- setup (untimed): inputs, one-time packing, copies
    c = synth.DECODE_2B
    K, N = c["K"], c["N"]
    d = synth.decode_2b()
    Wup, sup = B.bitlinear_pack(torch.from_numpy(d["W_up"]).to(dev))
    Wdn, sdn = B.bitlinear_pack(torch.from_numpy(d["W_down"]).to(dev))
    x = torch.from_numpy(d["x"]).to(dev)
    xd = torch.from_numpy(d["x_d"]).to(dev)
    pbytes = Wup.numel() * 4
    copies = max(2, int(np.ceil(600e6 / (2 * pbytes))))
    ups = [Wup.clone() for _ in range(copies)]
    dns = [Wdn.clone() for _ in range(copies)]
    ws1 = B.fused_workspace(1, K, dev)
    ws2 = B.fused_workspace(1, N, dev)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    y2 = torch.empty((1, K), dtype=torch.float32, device=dev)

    def step(i):
        j = i % copies
        B.bitlinear_forward_fused(x, ups[j], sup, N, out=y1, ws=ws1)
        B.bitlinear_forward_fused(xd, dns[j], sdn, K, out=y2, ws=ws2)

    # eager reference of one step; the graph replay must reproduce it
    step(0)
    torch.cuda.synchronize()
    ref1, ref2 = y1.clone(), y2.clone()
    K_steps, W_steps = args.steps, args.warmup
    # steps W .. W+K-1 (copy i % copies) are timed; the copies are read
    # cyclically (> 512 MB per cycle, more than twice the last-level cache),
    # so each step's weights come from HBM
    warm = capture(lambda i: step(i), W_steps, torch, skip_warm=True) if W_steps > 0 else None
    timed = capture(lambda i: step(W_steps + i), K_steps, torch, skip_warm=True)
    check = capture(lambda i: step(i), 1, torch, skip_warm=True)
    for _ in range(2):
        y1.zero_()
        y2.zero_()
        check.replay()
        torch.cuda.synchronize()
        if not (torch.equal(y1, ref1) and torch.equal(y2, ref2)):
            raise RuntimeError("graph replay differs from the eager step")
    # The first pass over the 68 weight copies after other memory has been
    # touched runs about 1 us per step slower than every later one (the
    # address translations of 601 MB are refilled; a 512 MiB fill before the
    # warm-up made the timed replay 8.12 against 7.05 us per step, and a
    # warm-up that does not reach every copy does not remove it): the timed
    # graph is replayed once here as preparation, then the warm-up, then the
    # timed replay.  The weights still stream from HBM: 601 MB read
    # cyclically do not stay in the 256 MB last-level cache.
    timed.replay()
    torch.cuda.synchronize()
    if warm is not None:
        warm.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    timed.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K_steps
    ev_ms_step = e0.elapsed_time(e1) / K_steps
    step_bytes = 2 * pbytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    del warm, timed, check

    # eager (one launch per call from Python), for context
    for i in range(20):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ne = 2 * copies
    for i in range(ne):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / ne

    # ---------------- dominant kernel: the slower of the step's two fused
    # GEMVs, HIP events around graph replays of back-to-back launches over
    # the rotating copies
    nl = max(K_steps, copies)
    up_ms = graph_time_per_launch(
        lambda i: B.bitlinear_forward_fused(x, ups[i % copies], sup, N, out=y1, ws=ws1),
        nl, 1, torch)
    dn_ms = graph_time_per_launch(
        lambda i: B.bitlinear_forward_fused(xd, dns[i % copies], sdn, K, out=y2, ws=ws2),
        nl, 1, torch)
    alg_up = pbytes + K * 4 + 4 + N * 4      # packed W + fp32 x + w_scale + fp32 y
    alg_dn = pbytes + N * 4 + 4 + K * 4
    legs = {"up": (up_ms, alg_up), "down": (dn_ms, alg_dn)}
    dom = max(legs, key=lambda leg: legs[leg][0])
    dom_ms, dom_alg = legs[dom]
    kname, shape = DECODE_GEMVS[dom]
    achieved = dom_alg / (dom_ms * 1e-3) / 1e9
    traffic, traffic_note = traffic_from_profile(kname)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": f"{kname} (fused quant + GEMV, {shape}, M=1; the slower of the "
                          "step's two kernels)",
                "avg_us": round(dom_ms * 1e3, 3), "algorithmic_bytes": dom_alg,
                "timing": f"HIP events around one replay of a graph of {nl} back-to-back "
                          "launches on the launch stream (weight copies rotating)",
                "traffic_source": traffic_note}
    kernels = {
        "gemv_fused_up_2560x6912": {"avg_us": round(up_ms * 1e3, 3),
                                    "GBps": round(alg_up / (up_ms * 1e-3) / 1e9, 1)},
        "gemv_fused_down_6912x2560": {"avg_us": round(dn_ms * 1e3, 3),
                                      "GBps": round(alg_dn / (dn_ms * 1e-3) / 1e9, 1)},
        "decode_step_eager_us": round(eager_ms * 1e3, 3),
    }
    if not args.no_extra:
        # the same up layer with its own RMSNorm (norm weights ~1 + 0.1 N(0,1))
        # in the one kernel: bitlinear_forward_fused_norm
        nwt = (1.0 + 0.1 * torch.from_numpy(synth.normal(9, 1, (K,)))).float().to(dev)
        wsn = B.fused_norm_workspace(1, K, dev)
        upn_ms = graph_time_per_launch(
            lambda i: B.bitlinear_forward_fused_norm(x, ups[i % copies], sup, N, nwt, 2.0 ** -23,
                                                     out=y1, ws=wsn),
            nl, 1, torch)
        alg_upn = alg_up + K * 4
        kernels["gemv_fused_norm_up_2560x6912"] = {
            "avg_us": round(upn_ms * 1e3, 3), "GBps": round(alg_upn / (upn_ms * 1e-3) / 1e9, 1)}
    del ups, dns
    torch.cuda.empty_cache()

    if not args.no_extra:
        kernels.update(extra_workloads(torch, B, synth, dev))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(d, args.cpu_seconds, step_bytes)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K_steps, "warmup": W_steps, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode 2B-class: M=1, BitLinear 2560->6912 + 6912->2560 from fp32 "
                               "activations, ternary 2-bit packed weights ~N(0,0.02), x ~N(0,1), "
                               "int8 per-token quantisation fused into each GEMV",
                   "M": 1, "K": K, "N": N, "weight_copies": copies,
                   "step_weight_bytes": step_bytes,
                   "launch": "one HIP graph of the K timed steps (replayed once as "
                             "preparation before the warm-up), wall clock between "
                             "synchronisations (graph launch included)",
                   "event_ms_per_step": round(ev_ms_step, 6),
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def extra_workloads(torch, B, synth, dev):
    """Kernel timings of the other shapes (prefill GEMM, skinny 2..64-token products,
    100B-class decode, FFN),
    each from HIP events around graph replays of back-to-back launches."""
    res = {}
    # prefill GEMM: M=2048, K=2560, N=6912
    c = synth.PREFILL_2B
    M, K, N = c["M"], c["K"], c["N"]
    p = synth.prefill_2b()
    Wp, sc = B.bitlinear_pack(torch.from_numpy(p["W"]).to(dev))
    X = torch.from_numpy(p["X"]).to(dev)
    q = B.bitlinear_quant_act(X)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    copies = [Wp.clone() for _ in range(4)]
    ms = graph_time_per_launch(
        lambda i: B.bitlinear_forward(q[0], q[1], q[2], K, copies[i % 4], sc, N, out=Y), 8, 5, torch)
    ops = 2.0 * M * N * K
    res["prefill_gemm_2048x2560x6912"] = {
        "avg_us": round(ms * 1e3, 2), "TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
        "frac_int8_peak": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
    qa_ms = graph_time_per_launch(lambda i: B.bitlinear_quant_act(X, out=q), 8, 5, torch)
    res["act_quant_2048x2560"] = {"avg_us": round(qa_ms * 1e3, 2),
                                  "GBps": round(M * (K * 5 + 8) / (qa_ms * 1e-3) / 1e9, 1)}
    del copies, Y, X, q, Wp
    torch.cuda.empty_cache()

    # skinny and medium-batch products on the 2B-class shapes: 2..512 tokens
    # from int8 codes,
    # rotating weight copies (> 512 MB)
    d2 = synth.decode_2b()
    for name, K, N in (("W_up", 2560, 6912), ("W_down", 6912, 2560)):
        Wp, sc = B.bitlinear_pack(torch.from_numpy(d2[name]).to(dev))
        ncp = max(2, int(np.ceil(600e6 / (Wp.numel() * 4))))
        cps = [Wp.clone() for _ in range(ncp)]
        for M in (2, 8, 16, 32, 64, 128, 512):
            q = B.bitlinear_quant_act(torch.from_numpy(synth.normal(9, M, (M, K))).to(dev))
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ms = graph_time_per_launch(
                lambda i: B.bitlinear_forward(q[0], q[1], q[2], K, cps[i % ncp], sc, N, out=Y),
                ncp, 5, torch)
            res[f"forward_{K}x{N}_M{M}"] = {
                "avg_us": round(ms * 1e3, 2),
                "weight_GBps": round(Wp.numel() * 4 / (ms * 1e-3) / 1e9, 1),
                "TOPS": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del cps, Wp
    del d2
    torch.cuda.empty_cache()

    # 100B-class decode: K=8192, N=28672, M in {1, 8}
    c = synth.DECODE_100B
    K, N = c["K"], c["N"]
    p = synth.decode_100b()
    Wd = torch.from_numpy(p["W"]).to(dev)
    del p["W"]
    for mode, tag in ((B.BL_TERNARY, "ternary"), (B.BL_BINARY, "binary")):
        Wp, sc = B.bitlinear_pack(Wd, mode)
        pb = Wp.numel() * 4
        ncp = max(2, int(np.ceil(600e6 / pb)))
        cps = [Wp.clone() for _ in range(ncp)]
        for M in (1, 8):
            Xm = torch.from_numpy(p["X"][:M]).to(dev)
            q = B.bitlinear_quant_act(Xm)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ms = graph_time_per_launch(
                lambda i: B.bitlinear_forward(q[0], q[1], q[2], K, cps[i % ncp], sc, N, out=Y),
                ncp, 5, torch)
            alg = pb + M * (K + 8) + 4 + M * N * 4
            res[f"decode_100b_{tag}_M{M}"] = {
                "avg_us": round(ms * 1e3, 2), "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if M == 1:
                wsf = B.fused_workspace(1, K, dev)
                ms = graph_time_per_launch(
                    lambda i: B.bitlinear_forward_fused(Xm, cps[i % ncp], sc, N, out=Y, ws=wsf),
                    ncp, 5, torch)
                alg = pb + K * 4 + 4 + N * 4
                res[f"decode_100b_{tag}_M1_fused"] = {
                    "avg_us": round(ms * 1e3, 2), "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del cps, Wp
        torch.cuda.empty_cache()
    # binary weights in the 1-bit layout (half the bytes of the 2-bit codes)
    Wb, sc = B.bitlinear_pack(Wd, B.BL_BINARY_1BIT)
    pb = Wb.numel() * 4
    ncp = max(2, int(np.ceil(600e6 / pb)))
    cps = [Wb.clone() for _ in range(ncp)]
    for M in (1, 8):
        q = B.bitlinear_quant_act(torch.from_numpy(p["X"][:M]).to(dev))
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ms = graph_time_per_launch(
            lambda i: B.bitlinear_forward_1bit(q[0], q[1], q[2], K, cps[i % ncp], sc, N, out=Y),
            ncp, 5, torch)
        alg = pb + M * (K + 8) + 4 + M * N * 4
        res[f"decode_100b_binary_1bit_M{M}"] = {
            "avg_us": round(ms * 1e3, 2), "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del cps, Wb
    torch.cuda.empty_cache()
    # a4.8 split activations (1 % outliers in int8, the rest in int4): quantiser and product
    Wp, sc = B.bitlinear_pack(Wd)
    pb = Wp.numel() * 4
    ncp = max(2, int(np.ceil(600e6 / pb)))
    cps = [Wp.clone() for _ in range(ncp)]
    n_out = int(round(0.01 * K))
    for M in (1, 8):
        Xm = torch.from_numpy(p["X"][:M]).to(dev)
        q = B.bitlinear_quant_act_a48(Xm, n_out)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        wsa = torch.empty(B.lib().bitlinear_a48_workspace_bytes(M, N) // 4, dtype=torch.int32,
                          device=dev)
        ms = graph_time_per_launch(
            lambda i: B.bitlinear_forward_a48(q, K, cps[i % ncp], sc, N, out=Y, ws=wsa), ncp, 5,
            torch)
        alg = pb + 2 * M * (K + 8) + 4 + M * N * 4
        res[f"decode_100b_a48_M{M}"] = {
            "avg_us": round(ms * 1e3, 2), "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "n_out": n_out}
        qms = graph_time_per_launch(lambda i: B.bitlinear_quant_act_a48(Xm, n_out, out=q), 4, 5,
                                    torch)
        res[f"a48_quant_{M}x{K}"] = {"avg_us": round(qms * 1e3, 2)}
    del cps, Wp
    torch.cuda.empty_cache()
    del Wd
    torch.cuda.empty_cache()

    # FFN block: D=2560, F=6912, M in {1, 8, 64}
    c = synth.FFN_2B
    D, F = c["D"], c["F"]
    f = synth.ffn_2b()
    packs = [B.bitlinear_pack(torch.from_numpy(f[n]).to(dev)) for n in ("W_gate", "W_up", "W_down")]
    wbytes = sum(pk[0].numel() * 4 for pk in packs)
    ncp = max(2, int(np.ceil(600e6 / wbytes)))
    cps = [[(pk[0].clone(), pk[1]) for pk in packs] for _ in range(ncp)]
    eps = float(np.finfo(np.float32).eps)
    subln_w = torch.from_numpy(f["subln_w"]).to(dev)
    for M in c["M_list"]:
        H = torch.from_numpy(f["H"][:M]).to(dev)
        ws = torch.empty(B.lib().bitnet_ffn_workspace_bytes(M, D, F), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, D), dtype=torch.float32, device=dev)
        for tag, sw in (("", None), ("_subln", subln_w)):
            def run(i):
                g, u, dn = cps[i % ncp]
                B.bitnet_ffn_forward(H, None, eps, g[0], g[1], u[0], u[1], dn[0], dn[1], D, F,
                                     out=Y, ws=ws, subln_w=sw, subln_eps=eps)

            ms = graph_time_per_launch(run, ncp, 5, torch)
            res[f"ffn_2b{tag}_M{M}"] = {"avg_us": round(ms * 1e3, 2),
                                        "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                                        "frac_hbm": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del cps, packs
    torch.cuda.empty_cache()
    return res


def cpu_baseline(d, seconds, step_bytes):
    """The CPU oracle (as it stands) running the same decode step, on this
    host's cores, for about `seconds` of work."""
    import oracle
    gu, tu, _ = oracle.quantize_weights(d["W_up"])
    gd, td, _ = oracle.quantize_weights(d["W_down"])
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.bitlinear(d["x"], tu, gu)
        oracle.bitlinear(d["x_d"], td, gd)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(step_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "ms_per_step": round(dt * 1e3 / n, 3),
            "sample": f"{n} oracle decode steps (quant + int matmul + dequant, up and down) "
                      f"in {dt:.1f} s; same packed-weight byte count per step as the GPU"}


if __name__ == "__main__":
    main()
