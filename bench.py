"""Benchmark of the causal packed microscaled attention hot path on one MI355X.

One step = quantize Q, K, V (token-block E4M3) + forward + backward (dO
quantization, D, prescale, recomputed P/dP/dS, dK/dV/dQ, dQ finalize), the
full training call, on seeded synthetic inputs already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_doc]

Timing: each seed's step is captured once in a HIP graph and replayed; W
untimed replays, then K replays each bracketed by hipEvents on the stream;
the seed's figure is the median of the K.  Three seeds; the reported value
is the median seed's, with the seeds' range alongside.  Kernel durations
(roofline) come from a separate eager pass on the same stream, with events
that the library records just before and after each kernel's launch.

Prints one JSON line.  value = algorithmic FLOPs of attention fwd+bwd
(14 d Hq x visible pairs; a multiply-add counts 2) per second of the step.
The packed MHA and packed GQA workloads ride along as extra keys.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["bwd.hip", "device.hpp", "kernels.hpp"]
SEEDS = (0, 1, 2)


# The pages' training-call latencies for two of the packed shapes (B300,
# MXFP8): context rows only, never a vs_baseline.
PAGES_B300_MS = {"docs_16x4096": 3.17, "docs_8192_224x256": 1.67}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_file(workload):
    """rocprofv3 FETCH_SIZE / WRITE_SIZE record of the backward main kernel on
    `workload`, valid only for the sources it was measured on."""
    return os.path.join(ROOT, "profiles", "bwd_main_kernel_%s_traffic.json" % workload)


class Hip:
    """hipEvent_t and stream helpers through the HIP runtime (plumbing)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return ms.value


def kernel_sources_sha256():
    """Hash of the sources the backward main kernel is compiled from."""
    import hashlib
    hsh = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_causal_flash_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the backward main kernel on `workload`: the
    counters' KiB per dispatch, each scaled by the factor a plain copy of
    known size gives the same counter; None when no measurement exists for
    the current sources."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("sources_sha256") != kernel_sources_sha256():
        return None
    return int(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def copy_calibration(mib):
    """A plain device copy of `mib` MiB, three times: the reference the
    traffic counters are scaled by (read `mib`, write `mib` per copy)."""
    import torch
    src = torch.ones(mib * (1 << 18), dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": mib << 20, "copies": 3}), flush=True)


def cpu_baseline(w, hadamard=False, max_tokens=32768):
    """The FP64 oracle on a bounded sample of the same workload: whole kv
    groups (head 0's group first) over the first `max_tokens` tokens of the
    packed row, documents cut there, quantize + forward + backward, sized to
    about 10-30 s on a host.  FLOPs are counted on the sample's own visible
    pairs with the metric's convention."""
    import oracle
    oracle.build()
    G = w.Hq // w.Hkv
    n = min(w.T, max_tokens)
    cu = np.unique(np.minimum(w.cu, n)).astype(np.int32)
    lens = np.diff(cu.astype(np.int64))
    pairs = int(np.sum(lens * (lens + 1) // 2)) if w.causal else int(np.sum(lens * lens))
    nh = G  # one kv group
    sub = workloads.Workload("sample", n, cu, nh, 1, w.d, w.flags,
                             np.ascontiguousarray(w.q[:n, :nh]), np.ascontiguousarray(w.k[:n, :1]),
                             np.ascontiguousarray(w.v[:n, :1]), np.ascontiguousarray(w.do[:n, :nh]))
    exact = bool(w.flags & workloads.FLAG_EXACT)
    blk = 1 if exact else 32
    t0 = time.time()
    if hadamard:
        q, k = (oracle.quantize_rotated(x, sub.cu, block=blk) for x in (sub.q, sub.k))
        v = oracle.quantize(sub.v, sub.cu, block=blk)
    else:
        q, k, v = (oracle.quantize(x, sub.cu, block=blk) for x in (sub.q, sub.k, sub.v))
    scale = oracle.default_scale(w.d) / (w.d if hadamard else 1)
    views = (None, None)
    if w.flags & workloads.FLAG_FP4_SCORE:
        views = (oracle.quantize_nvfp4(sub.q, sub.cu), oracle.quantize_nvfp4(sub.k, sub.cu))
    ops = oracle.Operands.from_codes(q, k, v, *views)
    c = w.causal
    O, L = oracle.attn_fwd(sub.cu, ops, scale=scale, causal=c, mode=oracle.MODE_TILED, kblock=64)
    gc, ge, D, _ = oracle.bwd_prep(sub.cu, sub.do, oracle.to_bf16(O), k[1], v[1], 1, scale=scale,
                                   causal=c, block=blk)
    Gd = oracle.dequantize(gc, ge)
    dq = oracle.bwd_dq(sub.cu, ops, Gd, D, L, scale=scale, causal=c, per_row_ds=exact)
    dk, _ = oracle.bwd_dkdv(sub.cu, ops, Gd, D, L, scale=scale, causal=c, per_row_ds=exact)
    if hadamard:
        oracle.unrotate(dq), oracle.unrotate(dk)
    dt = time.time() - t0
    flop = 14.0 * w.d * nh * pairs
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "q heads 0..%d (one kv group) of the first %d tokens (documents cut there): "
                      "quantize + fwd + bwd in FP64, %.1f s" % (nh - 1, n, dt)}


class Step:
    """Device buffers and the three calls of one training step of workload
    `w` (one seed), plus its captured graph."""

    def __init__(self, w, args, dev):
        import torch
        from bit_causal_flash_amd import flamia as F
        self.F, self.w = F, w
        T, Hq, Hkv, d = w.T, w.Hq, w.Hkv, w.d

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

        self.cu = torch.from_numpy(w.cu.astype(np.int32)).to(dev)
        self.xq, self.xk, self.xv = up(w.q), up(w.k), up(w.v)
        self.xdo = up(w.do).view(torch.bfloat16)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.qc, self.kc, self.vc = (torch.empty((T, h, d), **u8) for h in (Hq, Hkv, Hkv))
        self.qe, self.ke, self.ve = (torch.empty((h, T), **u8) for h in (Hq, Hkv, Hkv))
        self.o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
        self.dq = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
        self.dk = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
        self.dv = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
        self.exact = bool(w.flags & workloads.FLAG_EXACT)
        self.fp4 = bool(w.flags & workloads.FLAG_FP4_SCORE)
        flags = (F.FLAMIA_CAUSAL if w.causal else 0) | (F.FLAMIA_EXACT if self.exact else 0) | \
            (F.FLAMIA_FP4_SCORE if self.fp4 else 0)
        flags |= F.FLAMIA_HADAMARD if args.hadamard else 0
        self.mode = F.FLAMIA_SCALE_PER_TOKEN if self.exact else F.FLAMIA_SCALE_TOKBLOCK32
        self.qk_mode = self.mode | (F.FLAMIA_SCALE_ROTATE if args.hadamard else 0)
        self.pq = F.make_problem(self.cu, T, Hq, Hkv, d, 0.0, flags)
        self.pf = F.make_problem(self.cu, T, Hq, Hkv, d, 0.0, flags)
        self.pb = F.make_problem(self.cu, T, Hq, Hkv, d, 0.0, flags)
        self.wsf = torch.empty(F.flamia_attn_fwd_workspace_size(self.pf), **u8)
        self.wsb = torch.empty(F.flamia_attn_bwd_workspace_size(self.pb), **u8)
        self.views = None
        self.extra_q = []
        if self.fp4:
            q4, k4 = (torch.empty((T, h, d // 2), **u8) for h in (Hq, Hkv))
            q4s, k4s = (torch.empty((T, h, d // 16), **u8) for h in (Hq, Hkv))
            self.extra_q = [(Hq, self.xq, q4, q4s), (Hkv, self.xk, k4, k4s)]
            self.views = (q4, q4s, k4, k4s)
        self.graph = None

    # Q, K and V in one launch (the E2M1 views, when asked for, in their own)
    def quant(self):
        F = self.F
        F.flamia_quantize_qkv(self.pq, self.qk_mode, self.xq, self.xk, self.xv, self.qc, self.qe,
                              self.kc, self.ke, self.vc, self.ve)
        for nh, x, c, e in self.extra_q:
            F.flamia_quantize_tokblock(self.pq, nh, F.FLAMIA_SCALE_NVFP4_16, x, c, e)

    def fwd(self):
        self.F.flamia_attn_fwd(self.pf, self.qc, self.qe, self.kc, self.ke, self.vc, self.ve,
                               self.o, self.lse, self.wsf, fp4=self.views)

    def bwd(self):
        self.F.flamia_attn_bwd(self.pb, self.qc, self.qe, self.kc, self.ke, self.vc, self.ve,
                               self.o, self.lse, self.xdo, self.dq, self.dk, self.dv, self.wsb,
                               fp4=self.views)

    def step(self):
        self.quant()
        self.fwd()
        self.bwd()

    def capture(self):
        import torch
        self.step()  # warm the kernels once outside the capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()
        torch.cuda.synchronize()


def time_replays(hip, stream, step, K, W):
    """W untimed replays, then K replays each between two events; the
    per-replay milliseconds."""
    import torch
    for _ in range(W):
        step.graph.replay()
    torch.cuda.synchronize()
    evs = [(hip.event(), hip.event()) for _ in range(K)]
    for a, b in evs:
        hip.record(a, stream)
        step.graph.replay()
        hip.record(b, stream)
    torch.cuda.synchronize()
    return [hip.elapsed_ms(a, b) for a, b in evs]


def kernel_times(hip, stream, st, K):
    """Eager pass of K steps with the library recording events around the
    forward and the backward main kernels' launches; then the quantizer
    kernels alone,
    with a forward queued ahead of each so the GPU never waits on a launch.
    Returns mean kernel milliseconds."""
    import torch
    F = st.F
    evf = [(hip.event(), hip.event()) for _ in range(K)]
    evb = [(hip.event(), hip.event()) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        F.set_events(st.pf, *evf[i])
        F.set_events(st.pb, *evb[i])
        st.step()
    torch.cuda.synchronize()
    F.set_events(st.pf, None, None)
    F.set_events(st.pb, None, None)
    ms_fwd = sum(hip.elapsed_ms(a, b) for a, b in evf) / K
    ms_bwd = sum(hip.elapsed_ms(a, b) for a, b in evb) / K
    return ms_fwd, ms_bwd


def quantizer_cold(hip, stream, steps, K):
    """The Q/K/V quantizer kernel, rotating over the seeds' input sets (more
    than the 256 MB Infinity Cache between two reads of the same set) with a
    forward of another set queued ahead of each launch.  Mean ms."""
    import torch
    F = steps[0].F
    n = len(steps)
    evq = [(hip.event(), hip.event()) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        st, ahead = steps[i % n], steps[(i + 1) % n]
        ahead.fwd()
        F.set_events(st.pq, *evq[i])
        F.flamia_quantize_qkv(st.pq, st.qk_mode, st.xq, st.xk, st.xv, st.qc, st.qe, st.kc, st.ke,
                              st.vc, st.ve)
        F.set_events(st.pq, None, None)
    torch.cuda.synchronize()
    return sum(hip.elapsed_ms(a, b) for a, b in evq) / K


def bench_workload(name, args, hip, dev, seeds, headline):
    """Every seed of one workload: graph replays (median of K per seed) and,
    for the headline workload, kernel durations and the quantizer."""
    import torch
    steps, res = [], []
    for seed in seeds:
        w = workloads.NAMED[name](seed)
        if args.noncausal:
            w.flags &= ~workloads.FLAG_CAUSAL
        log("workload %s seed %d: T=%d docs=%d Hq=%d Hkv=%d d=%d" %
            (name, seed, w.T, len(w.cu) - 1, w.Hq, w.Hkv, w.d))
        st = Step(w, args, dev)
        st.capture()
        stream = torch.cuda.current_stream().cuda_stream
        ms = time_replays(hip, stream, st, args.steps, args.warmup)
        pairs = w.visible_pairs()
        med = float(np.median(ms))
        res.append(dict(seed=seed, pairs=int(pairs), documents=int(len(w.cu) - 1), ms=med,
                        tflops=14.0 * w.d * w.Hq * pairs / (med * 1e-3) / 1e12))
        steps.append(st)
        log("  step median %.4f ms over %d graph replays (min %.4f, max %.4f)" %
            (med, len(ms), min(ms), max(ms)))
    order = sorted(range(len(res)), key=lambda i: res[i]["tflops"])
    mid = order[len(order) // 2]
    out = dict(res=res, mid=mid)
    if headline:
        stream = torch.cuda.current_stream().cuda_stream
        out["steps"] = steps
        out["ms_fwd"], out["ms_bwd"] = kernel_times(hip, stream, steps[mid], args.steps)
        out["ms_q"] = quantizer_cold(hip, stream, steps, max(args.steps, 3 * len(steps)))
    return out


def summary(name, r):
    res = r["res"]
    m = res[r["mid"]]
    return {"workload": name, "ms_per_step": round(m["ms"], 4), "tflops": round(m["tflops"], 2),
            "pct_fp8_peak": round(100.0 * m["tflops"] / FP8_PEAK_TFLOPS, 2),
            "seeds": {str(x["seed"]): {"ms": round(x["ms"], 4), "tflops": round(x["tflops"], 2),
                                       "visible_pairs": x["pairs"], "documents": x["documents"]}
                      for x in res},
            "tflops_range": [round(min(x["tflops"] for x in res), 2),
                             round(max(x["tflops"] for x in res), 2)]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed graph replays per seed")
    ap.add_argument("--warmup", type=int, default=5, help="untimed graph replays per seed")
    ap.add_argument("--workload", default="long_doc", choices=sorted(workloads.NAMED))
    ap.add_argument("--seeds", type=int, default=len(SEEDS))
    ap.add_argument("--noncausal", action="store_true",
                    help="the same workload without the causal mask (pairs counted as n^2)")
    ap.add_argument("--hadamard", action="store_true",
                    help="rotate Q and K by the Hadamard matrix (FLAMIA_HADAMARD)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the packed MHA / GQA workloads that ride along")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB (traffic counter reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from bit_causal_flash_amd import flamia as F
    F.load()
    dev = torch.device("cuda:0")
    hip = Hip()
    seeds = SEEDS[:max(1, min(args.seeds, len(SEEDS)))]

    head = bench_workload(args.workload, args, hip, dev, seeds, headline=True)
    st = head["steps"][head["mid"]]
    w = st.w
    T, Hq, Hkv, d = w.T, w.Hq, w.Hkv, w.d
    hs = summary(args.workload, head)
    pairs = head["res"][head["mid"]]["pairs"]
    flop_bwd = 10.0 * d * Hq * pairs
    flop_fwd = 4.0 * d * Hq * pairs
    bwd_tflops = flop_bwd / (head["ms_bwd"] * 1e-3) / 1e12
    qbytes = (T * (Hq + 2 * Hkv)) * (3 * d + 1)  # read bf16, write codes + exponent byte
    extras = {}
    if not args.no_extra and not args.noncausal and not args.hadamard:
        for name in ("packed_mha", "packed_gqa", "docs_16x4096", "docs_8192_224x256"):
            if name != args.workload:
                # the 65,536-token context rows on seed 0 only (their inputs
                # take seconds per seed to generate on the host)
                ss = seeds[:1] if name in PAGES_B300_MS else seeds
                extras[name] = summary(name, bench_workload(name, args, hip, dev, ss, False))
                if name in PAGES_B300_MS:
                    # context, not a target: the pages' training-call latency
                    # on another machine (B300, MXFP8) for the same shape
                    extras[name]["pages_b300_ms"] = PAGES_B300_MS[name]
    exact = st.exact
    out = {
        "metric": "causal packed attn fwd+bwd TFLOP/s at 1 MI355X; % of FP8 MFMA peak",
        "value": hs["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hs["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+e2m1" if st.fp4 else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "documents": int(len(w.cu) - 1),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "causal": bool(w.causal),
                   "visible_pairs": int(pairs), "seed": int(head["res"][head["mid"]]["seed"]),
                   "scales": ("per-token operand exponents, per-(query row, 32-key block) dS "
                              "exponents for dQ" if exact else
                              "one exponent per 32 tokens x head dim, per 32x32 block for dS"),
                   "score_view": "E2M1 + E4M3 per 16 features (FP16 MFMA)" if st.fp4 else None,
                   "rotation": "Hadamard on Q, K (scale / d; dQ, dK rotated back)" if args.hadamard else None,
                   "step": "quantize Q,K,V (one launch)%s + attn fwd + attn bwd" %
                           (" (+ E2M1 views of Q,K)" if st.fp4 else ""),
                   "timing": "HIP-graph replays of the step, median of %d per seed, median of %d seeds"
                             % (args.steps, len(seeds))},
        "seeds": hs["seeds"],
        "tflops_range": hs["tflops_range"],
        "pct_fp8_peak": hs["pct_fp8_peak"],
        "roofline": {"kernel": ("bwd_kernel<%d, true, %d>" if exact and d == 128 else
                                "bwd_wide_kernel<%d, true, %d>") % (d, (2 if st.fp4 else 1) if exact else 0),
                     "bound": "mfma", "achieved": round(bwd_tflops, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": None if args.hadamard else measured_traffic(w.name)},
        "kernels": {
            "fwd_kernel_ms": round(head["ms_fwd"], 4),
            "fwd_kernel_tflops": round(flop_fwd / (head["ms_fwd"] * 1e-3) / 1e12, 2),
            "bwd_kernel_ms": round(head["ms_bwd"], 4),
            "bwd_kernel_tflops": round(bwd_tflops, 2),
            "quantize_qkv_kernel_ms": round(head["ms_q"], 4),
            "quantize_kernel_gbps": round(qbytes / (head["ms_q"] * 1e-3) / 1e9, 1),
            "quantize_kernel_frac_hbm_peak": round(qbytes / (head["ms_q"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "quantize_inputs": "rotated over %d input sets of %d MB (cold in the 256 MB Infinity Cache)"
                               % (len(seeds), T * (Hq + 2 * Hkv) * d * 2 // 1000000),
        },
    }
    if extras:
        out["extra_workloads"] = extras
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(w, hadamard=args.hadamard)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
