"""Benchmark of the causal packed microscaled attention hot path on one MI355X.

One step = quantize Q, K, V (token-block E4M3) + forward + backward (dO
quantization, D, prescale, recomputed P/dP/dS, dK/dV/dQ, dQ finalize), the
full training call, on seeded synthetic inputs already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload packed_mha]

Prints one JSON line.  value = algorithmic FLOPs of attention fwd+bwd
(14 d Hq x visible pairs; a multiply-add counts 2) per second of the step.
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
# HBM traffic of the backward main kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs, valid only for the sources it was measured on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_kernel_packed_mha_traffic.json")
KERNEL_SOURCES = ["bwd.hip", "device.hpp", "kernels.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (plumbing for kernel timing)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


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
        with open(TRAFFIC_FILE) as f:
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


def cpu_baseline(w, flop_target=3e11, hadamard=False):
    """The FP64 oracle on a bounded sample of the same workload: the first q
    heads (whole kv groups), every document, quantize + forward + backward,
    sized to about `flop_target` algorithmic FLOPs (10-30 s on a host)."""
    import oracle
    oracle.build()
    G = w.Hq // w.Hkv
    per_head = 14.0 * w.d * w.visible_pairs()
    nh = int(round(flop_target / per_head / G)) * G
    nh = min(w.Hq, max(G, nh))
    nkv = nh // G
    sub = workloads.Workload("sample", w.T, w.cu, nh, nkv, w.d, w.flags,
                             np.ascontiguousarray(w.q[:, :nh]), np.ascontiguousarray(w.k[:, :nkv]),
                             np.ascontiguousarray(w.v[:, :nkv]), np.ascontiguousarray(w.do[:, :nh]))
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
    gc, ge, D, _ = oracle.bwd_prep(sub.cu, sub.do, oracle.to_bf16(O), k[1], v[1], nkv, scale=scale,
                                   causal=c, block=blk)
    Gd = oracle.dequantize(gc, ge)
    dq = oracle.bwd_dq(sub.cu, ops, Gd, D, L, scale=scale, causal=c, per_row_ds=exact)
    dk, _ = oracle.bwd_dkdv(sub.cu, ops, Gd, D, L, scale=scale, causal=c, per_row_ds=exact)
    if hadamard:
        oracle.unrotate(dq), oracle.unrotate(dk)
    dt = time.time() - t0
    flop = 14.0 * w.d * nh * w.visible_pairs()
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "q heads 0..%d of %d (all documents): quantize + fwd + bwd in FP64, %.1f s"
                      % (nh - 1, w.Hq, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="packed_mha", choices=sorted(workloads.NAMED))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--noncausal", action="store_true",
                    help="the same workload without the causal mask (pairs counted as n^2)")
    ap.add_argument("--hadamard", action="store_true",
                    help="rotate Q and K by the Hadamard matrix (FLAMIA_HADAMARD)")
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
    w = workloads.NAMED[args.workload](args.seed)
    if args.noncausal:
        w.flags &= ~workloads.FLAG_CAUSAL
    log("workload %s: T=%d docs=%d Hq=%d Hkv=%d d=%d" % (w.name, w.T, len(w.cu) - 1, w.Hq, w.Hkv,
                                                         w.d))
    T, Hq, Hkv, d = w.T, w.Hq, w.Hkv, w.d

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    cu = torch.from_numpy(w.cu.astype(np.int32)).to(dev)
    xq, xk, xv, xdo = up(w.q), up(w.k), up(w.v), up(w.do).view(torch.bfloat16)
    u8 = dict(dtype=torch.uint8, device=dev)
    qc, kc, vc = (torch.empty((T, h, d), **u8) for h in (Hq, Hkv, Hkv))
    qe, ke, ve = (torch.empty((h, T), **u8) for h in (Hq, Hkv, Hkv))
    o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    # the workload's options: the exact-scale path quantizes per token and,
    # with the E2M1 score view, also writes the views of Q and K
    exact = bool(w.flags & workloads.FLAG_EXACT)
    fp4 = bool(w.flags & workloads.FLAG_FP4_SCORE)
    flags = (F.FLAMIA_CAUSAL if w.causal else 0) | (F.FLAMIA_EXACT if exact else 0) | \
        (F.FLAMIA_FP4_SCORE if fp4 else 0)
    flags |= F.FLAMIA_HADAMARD if args.hadamard else 0
    mode = F.FLAMIA_SCALE_PER_TOKEN if exact else F.FLAMIA_SCALE_TOKBLOCK32
    qk_mode = mode | (F.FLAMIA_SCALE_ROTATE if args.hadamard else 0)
    pq = F.make_problem(cu, T, Hq, Hkv, d, 0.0, flags)
    pf = F.make_problem(cu, T, Hq, Hkv, d, 0.0, flags)
    pb = F.make_problem(cu, T, Hq, Hkv, d, 0.0, flags)
    wsf = torch.empty(F.flamia_attn_fwd_workspace_size(pf), **u8)
    wsb = torch.empty(F.flamia_attn_bwd_workspace_size(pb), **u8)

    qargs = [(Hq, xq, qc, qe, qk_mode), (Hkv, xk, kc, ke, qk_mode), (Hkv, xv, vc, ve, mode)]
    views = None
    if fp4:
        q4, k4 = (torch.empty((T, h, d // 2), **u8) for h in (Hq, Hkv))
        q4s, k4s = (torch.empty((T, h, d // 16), **u8) for h in (Hq, Hkv))
        qargs += [(Hq, xq, q4, q4s, F.FLAMIA_SCALE_NVFP4_16),
                  (Hkv, xk, k4, k4s, F.FLAMIA_SCALE_NVFP4_16)]
        views = (q4, q4s, k4, k4s)

    # Q, K and V in one launch (the E2M1 views, when asked for, in their own)
    def quant():
        F.flamia_quantize_qkv(pq, qk_mode, xq, xk, xv, qc, qe, kc, ke, vc, ve)
        for nh, x, c, e, m in qargs[3:]:
            F.flamia_quantize_tokblock(pq, nh, m, x, c, e)

    def fwd():
        F.flamia_attn_fwd(pf, qc, qe, kc, ke, vc, ve, o, lse, wsf, fp4=views)

    def bwd():
        F.flamia_attn_bwd(pb, qc, qe, kc, ke, vc, ve, o, lse, xdo, dq, dk, dv, wsb, fp4=views)

    def step():
        quant()
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = HipEvents()
    K = args.steps
    evf = [(hip.create(), hip.create()) for _ in range(K)]
    evb = [(hip.create(), hip.create()) for _ in range(K)]
    t_start, t_stop = hip.create(), hip.create()
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(t_start), ctypes.c_void_p(stream))
    for i in range(K):
        F.set_events(pf, *evf[i])
        F.set_events(pb, *evb[i])
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(t_stop), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    F.set_events(pf, None, None)
    F.set_events(pb, None, None)
    ms_step = hip.elapsed_ms(t_start, t_stop) / K
    ms_fwd = sum(hip.elapsed_ms(a, b) for a, b in evf) / K
    ms_bwd = sum(hip.elapsed_ms(a, b) for a, b in evb) / K

    # stage timings (same launches, separately bracketed)
    def timed(fn, reps):
        torch.cuda.synchronize()
        hip.lib.hipEventRecord(ctypes.c_void_p(t_start), ctypes.c_void_p(stream))
        for _ in range(reps):
            fn()
        hip.lib.hipEventRecord(ctypes.c_void_p(t_stop), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        return hip.elapsed_ms(t_start, t_stop) / reps

    ms_quant = timed(quant, K)

    # quantizer kernels alone: events recorded by the library around each
    # kernel, with a forward queued ahead so the GPU never waits on a launch
    evq = [[(hip.create(), hip.create()) for _ in range(len(qargs) - 2)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        fwd()
        F.set_events(pq, *evq[i][0])
        F.flamia_quantize_qkv(pq, qk_mode, xq, xk, xv, qc, qe, kc, ke, vc, ve)
        for j, (nh, x, c, e, m) in enumerate(qargs[3:]):
            F.set_events(pq, *evq[i][j + 1])
            F.flamia_quantize_tokblock(pq, nh, m, x, c, e)
    torch.cuda.synchronize()
    F.set_events(pq, None, None)
    ms_qkern = sum(hip.elapsed_ms(a, b) for ev in evq for a, b in ev) / K
    ms_attn = timed(lambda: (fwd(), bwd()), K)
    ms_bwd_det = None  # the exact-scale and rotated backwards have no deterministic variant
    if not exact and not args.hadamard:
        pdet = F.make_problem(cu, T, Hq, Hkv, d, 0.0,
                              (F.FLAMIA_CAUSAL if w.causal else 0) | F.FLAMIA_DETERMINISTIC)
        wsd = torch.empty(F.flamia_attn_bwd_workspace_size(pdet), **u8)
        ms_bwd_det = timed(lambda: F.flamia_attn_bwd(pdet, qc, qe, kc, ke, vc, ve, o, lse, xdo, dq,
                                                     dk, dv, wsd), K)

    pairs = w.visible_pairs()
    flop = 14.0 * d * Hq * pairs
    flop_bwd = 10.0 * d * Hq * pairs
    flop_fwd = 4.0 * d * Hq * pairs
    value = flop / (ms_step * 1e-3) / 1e12
    bwd_tflops = flop_bwd / (ms_bwd * 1e-3) / 1e12
    qbytes = (T * (Hq + 2 * Hkv)) * (3 * d + 1)  # read bf16, write codes + exponent byte
    if fp4:  # E2M1 views of Q and K: read bf16, write d / 2 code and d / 16 scale bytes
        qbytes += T * (Hq + Hkv) * (2 * d + d // 2 + d // 16)
    out = {
        "metric": "causal packed attn fwd+bwd TFLOP/s at 1 MI355X; % of FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+e2m1" if fp4 else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "documents": int(len(w.cu) - 1),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "causal": bool(w.causal),
                   "visible_pairs": int(pairs), "seed": args.seed,
                   "scales": ("per-token operand exponents, per-(query row, 32-key block) dS "
                              "exponents for dQ" if exact else
                              "one exponent per 32 tokens x head dim, per 32x32 block for dS"),
                   "score_view": "E2M1 + E4M3 per 16 features (FP16 MFMA)" if fp4 else None,
                   "rotation": "Hadamard on Q, K (scale / d; dQ, dK rotated back)" if args.hadamard else None,
                   "step": "quantize Q,K,V (one launch)%s + attn fwd + attn bwd" %
                           (" (+ E2M1 views of Q,K)" if fp4 else "")},
        "pct_fp8_peak": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
        "roofline": {"kernel": "bwd_kernel", "bound": "mfma", "achieved": round(bwd_tflops, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / FP8_PEAK_TFLOPS, 4), "traffic": None},
        "kernels": {
            "fwd_kernel_ms": round(ms_fwd, 4),
            "fwd_kernel_tflops": round(flop_fwd / (ms_fwd * 1e-3) / 1e12, 2),
            "bwd_kernel_ms": round(ms_bwd, 4),
            "bwd_kernel_tflops": round(bwd_tflops, 2),
            "attn_fwd_bwd_ms": round(ms_attn, 4),
            "attn_fwd_bwd_tflops": round(flop / (ms_attn * 1e-3) / 1e12, 2),
            "bwd_call_deterministic_ms": None if ms_bwd_det is None else round(ms_bwd_det, 4),
            "quantize_qkv_call_ms": round(ms_quant, 4),
            "quantize_qkv_kernel_ms": round(ms_qkern, 4),
            "quantize_kernel_gbps": round(qbytes / (ms_qkern * 1e-3) / 1e9, 1),
            "quantize_kernel_frac_hbm_peak": round(qbytes / (ms_qkern * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
    }
    # counters were taken without the rotation epilogue
    out["roofline"]["traffic"] = None if args.hadamard else measured_traffic(w.name)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(w, hadamard=args.hadamard)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
