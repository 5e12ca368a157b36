"""Benchmark of the fused LUT-dequantize + matmul on one MI355X.

Headline step: one lutq_matmul call on the Llama-3-8B MLP up-projection shape
(N = 14336, K = 4096), 4-bit uniform (INT) table, one fp16 scale per 128
weights, batch M = 1 -- the HBM-bound GEMV. Weights are "cold": every call
reads a different copy of the packed matrix, and the copies together exceed
the 256 MB Infinity Cache, so the bytes come from HBM. Also measured in the
same run (reported beside the headline):

- the same call with one warm copy (Infinity-Cache resident);
- batch 32 on the Llama-70B-shaped log table (N = 28672, K = 8192,
  tensor-wise scale): TFLOP/s against the fp16 MFMA peak;
- the CPU oracle on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
CACHE_BYTES = 256 << 20        # Infinity Cache (MALL)
COLD_SET_BYTES = 2 * CACHE_BYTES
EXTRA_REPEATS = 3  # timed replays per secondary line (median)


def algorithmic_bytes(M, N, K, bits, group):
    """Bytes the method must move: packed codes + scales + x + y + table."""
    scales = N * (K // group) * 2 if group else 2
    return N * K * bits // 8 + scales + M * K * 2 + M * N * 2 + (1 << bits) * 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Case:
    """Device-resident inputs of one workload matrix at batch M."""

    def __init__(self, lutq, torch, wname, mat, M, cold=True):
        import numpy as np

        from synth import workloads
        w = workloads.WORKLOADS[wname]
        self.w, self.M = w, M
        _, m = w.matrix(mat)
        self.N, self.K = m.N, m.K
        t0 = time.time()
        c, T, s = workloads.quantized(w, mat)
        x = workloads.activations(w, M, mat)
        log(f"[bench] {wname}/{m.name} inputs generated in {time.time() - t0:.1f}s")
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        P = lutq.repack(d(c), w.bits, w.group)
        self.packed = [P]
        if cold:
            ncopy = max(2, -(-COLD_SET_BYTES // P.nbytes))
            from weight_only_lut_amd._lib import Packed, PackedDesc
            for _ in range(ncopy - 1):
                data = P.data.clone()
                desc = PackedDesc.from_buffer_copy(P.desc)
                desc.data = data.data_ptr()
                self.packed.append(Packed(data, desc))
        self.x, self.lut, self.scales = d(x), d(T), d(s)
        self.y = torch.empty((M, self.N), dtype=torch.float16, device="cuda")
        self.bytes = algorithmic_bytes(M, self.N, self.K, w.bits, w.group)
        self.flops = 2 * M * self.N * self.K
        self.host = (c, T, s, x)
        torch.cuda.synchronize()

    def call(self, lutq, i):
        lutq.matmul(self.x, self.packed[i % len(self.packed)], self.lut, self.scales, out=self.y)


def time_case(lutq, torch, case, steps, warmup, repeats=1):
    """Average microseconds per call over exactly `steps` back-to-back calls.

    `warmup` eager calls, then the `steps` calls are captured in a HIP graph,
    replayed once untimed, and replayed once more between HIP events recorded
    on the stream the kernels run on (host-side launch cost stays outside the
    timed region), with a device synchronization on both sides. With
    `repeats` > 1 the timed replay is repeated and the median returned (the
    secondary lines: one replay of a few tens of calls varies by ~10%).
    """
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            case.call(lutq, i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            case.call(lutq, i)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            start.record()
            graph.replay()
            stop.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(stop) * 1e3 / steps)
    return sorted(times)[len(times) // 2]


def cpu_baseline(case, budget_s=15.0):
    """The oracle as it stands (unpack + dequant + fp64 matmul) on the host cores."""
    import numpy as np

    import oracle
    c, T, s, x = case.host
    w = case.w
    packed = oracle.pack_codes(c, w.bits)   # the oracle's own format; untimed
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    cores = len(os.sched_getaffinity(0))
    times = []
    t_all = time.time()
    while time.time() - t_all < budget_s or len(times) < 3:
        t0 = time.time()
        codes = oracle.unpack_codes(packed, case.N, case.K, w.bits)
        oracle.reference(x, codes, T, s, w.group)
        times.append(time.time() - t0)
        if len(times) >= 50:
            break
    med = float(np.median(times))
    return {
        "value": case.bytes / med / 1e9,
        "unit": "GB/s",
        "cores": min(cores, blas) if blas > 1 else 1,
        "host_cores": cores,
        "blas_threads": blas,
        "kind": "oracle",
        "us_per_call": med * 1e6,
        "sample": f"{w.name} N={case.N} K={case.K} M={case.M}: whole matrix, canonical unpack + "
                  f"fp32 dequant + fp64 matmul (numpy), median of {len(times)} runs",
    }


class VariantCase(Case):
    """A workload matrix launched plain, with per-group zero points
    (lutq_matmul_zp) or with four per-group data types (lutq_matmul_typed)."""

    def __init__(self, lutq, torch, wname, mat, M):
        import numpy as np

        from synth import tables
        super().__init__(lutq, torch, wname, mat, M)
        c, T, s, x = self.host
        lo, hi = float(T.astype(np.float32).min()), float(T.astype(np.float32).max())
        rng = np.random.default_rng(7)
        z = rng.uniform(lo, hi, s.shape).astype(np.float16)
        luts = np.stack([T] + [tables.make(k, self.w.bits) for k in ("nf", "lloyd_max", "log")])
        ty = rng.integers(0, 4, s.shape).astype(np.uint8)
        self.zeros, self.luts, self.types = (torch.from_numpy(a).cuda() for a in (z, luts, ty))
        self.x_bf16 = self.x.to(torch.bfloat16)
        self.y_bf16 = torch.empty_like(self.y, dtype=torch.bfloat16)
        self.base_bytes = self.bytes
        self.extra_bytes = {"plain": 0, "zeros": z.nbytes, "types": ty.nbytes + luts.nbytes, "bf16": 0}
        self.mode = "plain"

    def call(self, lutq, i):
        P = self.packed[i % len(self.packed)]
        if self.mode == "types":
            lutq.matmul(self.x, P, self.luts, self.scales, types=self.types, out=self.y)
        elif self.mode == "bf16":
            lutq.matmul(self.x_bf16, P, self.lut, self.scales, out=self.y_bf16)
        else:
            lutq.matmul(self.x, P, self.lut, self.scales,
                        zeros=self.zeros if self.mode == "zeros" else None, out=self.y)


class BcqCase:
    """Binary-coded weights (q planes, alphas per plane, row and group 128) of
    a workload matrix's shape, cold (lutq_matmul_bcq)."""

    def __init__(self, lutq, torch, wname, M, q=3):
        import numpy as np

        from synth import workloads
        w = workloads.WORKLOADS[wname]
        _, m = w.matrix(None)
        self.N, self.K, self.M = m.N, m.K, M
        rng = np.random.default_rng(5)
        c = rng.integers(0, 1 << q, (self.N, self.K)).astype(np.uint8)
        a = np.stack([rng.uniform(0.01, 0.03, (self.N, self.K // 128)) / 2 ** p
                      for p in range(q)]).astype(np.float16)
        d = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
        P = lutq.repack(d(c), q, 128)
        from weight_only_lut_amd._lib import Packed, PackedDesc
        self.packed = [P]
        for _ in range(max(2, -(-COLD_SET_BYTES // P.nbytes)) - 1):
            data = P.data.clone()
            desc = PackedDesc.from_buffer_copy(P.desc)
            desc.data = data.data_ptr()
            self.packed.append(Packed(data, desc))
        self.alphas = d(a)
        self.x = d(workloads.activations(w, M))
        self.y = torch.empty((M, self.N), dtype=torch.float16, device="cuda")
        self.bytes = (self.N * self.K * q // 8 + a.nbytes + M * self.K * 2 + M * self.N * 2)
        torch.cuda.synchronize()

    def call(self, lutq, i):
        lutq.matmul_bcq(self.x, self.packed[i % len(self.packed)], self.alphas, out=self.y)


def variant_section(lutq, torch, args):
    """bf16 activations, per-group zero points, per-group data types (four
    tables) and binary-coded weights (q = 3) on the headline matrix's shape
    at batch 1 and 16, against the plain launch (cold)."""
    out = {}
    steps = max(20, args.steps // 4)
    for M in (1, 16):
        vc = VariantCase(lutq, torch, "int4_up_proj", None, M)
        rec = {}
        for mode in ("plain", "bf16", "zeros", "types"):
            vc.mode = mode
            us = time_case(lutq, torch, vc, steps, args.warmup, repeats=EXTRA_REPEATS)
            nbytes = vc.base_bytes + vc.extra_bytes[mode]
            rec[mode] = {"us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
            log(f"[bench] variants M={M} {mode}: {us:.2f} us")
        out[f"int4_up_proj_M{M}"] = rec
        del vc
        torch.cuda.empty_cache()
        bc = BcqCase(lutq, torch, "int4_up_proj", M, q=3)
        us = time_case(lutq, torch, bc, steps, args.warmup, repeats=EXTRA_REPEATS)
        out[f"bcq3_{bc.N}x{bc.K}_M{M}"] = {"us": round(us, 3),
                                           "GBps": round(bc.bytes / (us * 1e-6) / 1e9, 1)}
        log(f"[bench] variants M={M} bcq q=3: {us:.2f} us")
        del bc
        torch.cuda.empty_cache()
    return out


class FusedCase:
    """Matrices of one layer that read the same activations (Llama-3-8B q/k/v,
    or gate and up), cold, called either as one lutq_matmul per matrix or as
    one fused lutq_matmul_multi."""

    def __init__(self, lutq, torch, wname, mats, M):
        self.parts = [Case(lutq, torch, wname, m, M) for m in mats]
        for part in self.parts[1:]:
            part.x = self.parts[0].x
        self.fused = False
        K = self.parts[0].K
        self.bytes = sum(p.bytes for p in self.parts) - (len(self.parts) - 1) * M * K * 2

    def call(self, lutq, i):
        if self.fused:
            lutq.matmul_multi(self.parts[0].x,
                              [(p.packed[i % len(p.packed)], p.lut, p.scales) for p in self.parts],
                              outs=[p.y for p in self.parts])
        else:
            for p in self.parts:
                p.call(lutq, i)


def fused_section(lutq, torch, args):
    """One fused launch against one launch per matrix, for q/k/v and gate/up
    of the Llama-3-8B layer at batch 1 and 16 (cold weights)."""
    out = {}
    steps = max(20, args.steps // 4)
    for label, mats in (("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up"))):
        for M in (1, 16):
            fc = FusedCase(lutq, torch, "nf4_layer", mats, M)
            fc.fused = False
            sep = time_case(lutq, torch, fc, steps, args.warmup, repeats=EXTRA_REPEATS)
            fc.fused = True
            fus = time_case(lutq, torch, fc, steps, args.warmup, repeats=EXTRA_REPEATS)
            out[f"{label}_M{M}"] = {
                "separate_us": round(sep, 3), "fused_us": round(fus, 3),
                "speedup": round(sep / fus, 3),
                "fused_GBps": round(fc.bytes / (fus * 1e-6) / 1e9, 1),
                "plan": lutq.plan(M, sum(-(-p.N // 16) * 16 for p in fc.parts), fc.parts[0].K, 4)}
            log(f"[bench] fused {label} M={M}: separate {sep:.2f} us, fused {fus:.2f} us")
            del fc
            torch.cuda.empty_cache()
    return out


class QuantCase:
    """The quantizer on one workload matrix: fp32 weights (cold copies) ->
    codes + scales under `rule`, with `group` (0 = tensor-wise)."""

    def __init__(self, lutq, torch, wname, group, rule, table=None):
        import numpy as np

        from synth import tables, workloads
        w = workloads.WORKLOADS[wname]
        self.w, self.group, self.rule = w, group, rule
        _, m = w.matrix(None)
        self.N, self.K = m.N, m.K
        W = workloads.weights(w)
        T = workloads.lut(w) if table is None else tables.make(table, w.bits)
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        first = d(W)
        self.ws = [first] + [first.clone() for _ in range(max(1, -(-COLD_SET_BYTES // first.nbytes)) - 1)]
        self.lut = d(T)
        self.codes = torch.empty((self.N, self.K), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((self.N, self.K // group) if group else (1,), dtype=torch.float16,
                                  device="cuda")
        nsc = self.N * (self.K // group) * 2 if group else 2
        self.bytes = 4 * self.N * self.K + self.N * self.K + nsc + (1 << w.bits) * 2
        self.host = (W, T)
        torch.cuda.synchronize()

    def call(self, lutq, i):
        from weight_only_lut_amd import _lib
        W = self.ws[i % len(self.ws)]
        rc = _lib._lib().lutq_quantize(_lib._ptr(W), _lib._ptr(self.lut), self.w.bits, self.N, self.K,
                                       self.group, _lib._RULES[self.rule], _lib._ptr(self.codes),
                                       _lib._ptr(self.scales), _lib._stream(W.device))
        if rc:
            raise _lib.LutqError(rc, "lutq_quantize")


class DenseCase:
    """The same product with dense fp16 weights through torch (the vendor GEMM
    library): the baseline that a weight-only quantized kernel is measured
    against (FLUTE abstract: speedups over existing GEMM kernels at batch
    sizes below 32). Cold: rotating copies, as the quantized cases."""

    def __init__(self, torch, N, K, M, seed):
        g = torch.Generator(device="cuda").manual_seed(seed)
        w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).half()
        self.ws = [w] + [w.clone() for _ in range(max(2, -(-COLD_SET_BYTES // w.nbytes)) - 1)]
        self.x = torch.randn(M, K, generator=g, device="cuda").half()
        self.bytes = N * K * 2 + M * K * 2 + M * N * 2
        self.flops = 2 * M * N * K
        self.linear = torch.nn.functional.linear
        torch.cuda.synchronize()

    def call(self, lutq, i):
        self.linear(self.x, self.ws[i % len(self.ws)])


def dense_section(torch, args, quantized_us):
    """Dense fp16 at the headline shapes, beside the LUT kernel's time."""
    out = {}
    for label, (N, K, M) in (("int4_up_proj_M1", (14336, 4096, 1)), ("log4_70b_M32", (28672, 8192, 32))):
        if quantized_us.get(label) is None:
            continue
        dc = DenseCase(torch, N, K, M, seed=11)
        us = time_case(None, torch, dc, max(20, args.steps // 4), args.warmup, repeats=EXTRA_REPEATS)
        q = quantized_us[label]
        out[label] = {"N": N, "K": K, "M": M, "dense_us": round(us, 3),
                      "dense_GBps": round(dc.bytes / (us * 1e-6) / 1e9, 1),
                      "dense_TFLOPs": round(dc.flops / (us * 1e-6) / 1e12, 1),
                      "lutq_us": round(q, 3), "speedup": round(us / q, 2),
                      "copies": len(dc.ws)}
        log(f"[bench] dense fp16 {label}: {us:.2f} us (lutq {q:.2f} us, {us / q:.2f}x)")
        del dc
        torch.cuda.empty_cache()
    return out


def quantizer_section(lutq, torch, args):
    """The quantizer (the step before repack) on the headline matrix: grouped
    INT (range rule) and tensor-wise NormalFloat (absmax), cold weights, with
    the oracle on a bounded row sample beside it."""
    import numpy as np

    from oracle import quantize as Q
    out = {}
    for label, group, rule, table in (("int4_g128_range", 128, "range", None),
                                      ("nf4_tensor_absmax", 0, "absmax", "nf")):
        qc = QuantCase(lutq, torch, "int4_up_proj", group, rule, table)
        us = time_case(lutq, torch, qc, max(20, args.steps // 10), args.warmup, repeats=EXTRA_REPEATS)
        gbps = qc.bytes / (us * 1e-6) / 1e9
        W, T = qc.host
        rows = 256
        t0 = time.time()
        s = Q.scales(W, T, group, rule)           # whole-matrix scales: the tensor-wise rule needs them
        Q.codes(W[:rows], T, s if group == 0 else s[:rows], group)
        cpu_s = time.time() - t0
        cpu_bytes = 4 * W.size + rows * qc.K * 1     # scales pass reads W once; codes for `rows`
        out[label] = {"N": qc.N, "K": qc.K, "group": group, "rule": rule,
                      "us_per_call": round(us, 3), "effective_GBps": round(gbps, 1),
                      "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
                      "cpu_oracle": {"seconds": round(cpu_s, 3), "GBps": round(cpu_bytes / cpu_s / 1e9, 3),
                                     "sample": f"scales over the whole matrix, codes for {rows} rows"}}
        log(f"[bench] quantizer {label}: {us:.1f} us/call, {gbps:.0f} GB/s")
        if group:
            # NormalFloat table tuning on the same weights: 5 Lloyd updates
            from synth import tables
            T0 = torch.from_numpy(tables.make("nf", qc.w.bits)).cuda()
            torch.cuda.synchronize()
            t0 = time.time()
            _, _, errs = lutq.tune_table(qc.ws[0], T0, qc.w.bits, group, "absmax", iters=5)
            dt = time.time() - t0
            out[label]["nf_tune"] = {"updates": len(errs) - 1, "seconds": round(dt, 4),
                                     "us_per_pass": round(dt * 1e6 / (len(errs) + 1), 1),
                                     "error_first_last": [errs[0], errs[-1]]}
            log(f"[bench] NF table tuning: {len(errs) - 1} updates in {dt * 1e3:.2f} ms")
        del qc
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch32", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense fp16 (torch) context timings")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the zero-point and data-type timings")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the Infinity-Cache-warm repeats (so a kernel trace holds cold calls only)")
    ap.add_argument("--sweep", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling memory counters)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("KERNEL_TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 output and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, command=args.profile_command)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only: --gpus above 1 is not supported "
                                   "(the matmul would shard along N, with no communication, but "
                                   "only the one-GPU kernel is built)"}))
        sys.exit(2)

    import torch

    import weight_only_lut_amd as lutq
    lutq.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    # ---- headline: batch-1 4-bit g128 GEMV, cold weights ------------------
    head = Case(lutq, torch, "int4_up_proj", None, 1, cold=True)
    hplan = lutq.plan(1, head.N, head.K, 4)
    log(f"[bench] headline: {len(head.packed)} rotating copies, plan={hplan}")
    region_us = time_case(lutq, torch, head, args.steps, args.warmup)
    w_region_us = None
    if not args.no_warm:
        warm = Case.__new__(Case)
        warm.__dict__.update(head.__dict__)
        warm.packed = head.packed[:1]
        w_region_us = time_case(lutq, torch, warm, args.steps, args.warmup)
    log(f"[bench] headline cold: {region_us:.2f} us/call; warm: {w_region_us} us/call")

    value = head.bytes / (region_us * 1e-6) / 1e9
    achieved = value
    traffic = load_traffic("int4_up_proj", hplan)

    extra = {
        "us_per_call": round(region_us, 3),
        "bits_read_per_weight": round(head.bytes * 8 / (head.N * head.K), 4),
        "warm": None if w_region_us is None else {
            "us_per_call": round(w_region_us, 3),
            "effective_GBps": round(head.bytes / (w_region_us * 1e-6) / 1e9, 1)},
        "plan": hplan,
    }

    # ---- batch 32: log table, Llama-70B up-projection shape ---------------
    if not args.no_batch32:
        b32 = Case(lutq, torch, "log4_70b", None, 32, cold=True)
        p32 = lutq.plan(32, b32.N, b32.K, 4)
        k_us = time_case(lutq, torch, b32, max(20, args.steps // 4), args.warmup, repeats=EXTRA_REPEATS)
        wk_us = None
        if not args.no_warm:
            warm32 = Case.__new__(Case)
            warm32.__dict__.update(b32.__dict__)
            warm32.packed = b32.packed[:1]
            wk_us = time_case(lutq, torch, warm32, max(20, args.steps // 4), args.warmup, repeats=EXTRA_REPEATS)
            del warm32
        tf = b32.flops / (k_us * 1e-6) / 1e12
        extra["batch32"] = {
            "workload": "log4_70b", "N": b32.N, "K": b32.K, "M": 32, "plan": p32,
            "us_per_call": round(k_us, 3),
            "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "effective_GBps": round(b32.bytes / (k_us * 1e-6) / 1e9, 1),
            "warm": None if wk_us is None else {
                "us_per_call": round(wk_us, 3),
                "TFLOPs": round(b32.flops / (wk_us * 1e-6) / 1e12, 1),
                "mfma_frac": round(b32.flops / (wk_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        }
        log(f"[bench] batch32 cold {k_us:.2f} us = {tf:.1f} TFLOP/s; warm {wk_us} us")
        del b32
        torch.cuda.empty_cache()

    if not args.no_quantizer:
        extra["quantizer"] = quantizer_section(lutq, torch, args)
    if not args.no_fused:
        extra["fused"] = fused_section(lutq, torch, args)
    if not args.no_variants:
        extra["variants"] = variant_section(lutq, torch, args)
    if not args.no_dense:
        extra["dense_fp16"] = dense_section(
            torch, args, {"int4_up_proj_M1": region_us,
                          "log4_70b_M32": None if args.no_batch32 else k_us})

    if args.sweep:
        extra["sweep"] = sweep(lutq, torch, args)

    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None if args.no_cpu_baseline else cpu_baseline(head)

    out = {
        "metric": "batch-1 4-bit g128 GEMV us + effective GB/s (% HBM peak); batch-32 TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(region_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "int4_up_proj", "N": head.N, "K": head.K, "M": 1, "bits": 4,
                   "group": 128, "table": "int", "weights": f"cold, {len(head.packed)} rotating copies"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def sweep(lutq, torch, args):
    """Every workload matrix at every batch size, the automatic plan and each
    kernel shape of both paths (GEMV up to 8 batch rows), cold weights; one
    JSON row per case on stderr."""
    from synth import workloads
    rows = []
    for wname, w in workloads.WORKLOADS.items():
        for m in w.matrices:
            base = Case(lutq, torch, wname, m.name, max(w.batches), cold=True)
            for M in w.batches:
                case = Case.__new__(Case)
                case.__dict__.update(base.__dict__)
                case.M = M
                case.x = base.x[:M].contiguous()
                case.y = torch.empty((M, base.N), dtype=torch.float16, device="cuda")
                case.bytes = algorithmic_bytes(M, base.N, base.K, w.bits, w.group)
                case.flops = 2 * M * base.N * base.K
                shapes = [("auto", 0)] + [("mfma", t) for t in (2, 4, 7, 8)]
                if M <= 8:
                    shapes += [("gemv", t) for t in (1, 2)]
                for path, tiles in shapes:
                    def call(lutq_, i, case=case, path=path, tiles=tiles):
                        lutq_.matmul(case.x, case.packed[i % len(case.packed)], case.lut,
                                     case.scales, out=case.y, path=path, tiles=tiles)
                    case.call = call
                    us = time_case(lutq, torch, case, max(20, args.steps // 4), args.warmup)
                    row = {"workload": wname, "matrix": m.name, "N": base.N, "K": base.K,
                           "M": M, "path": path, "tiles": tiles, "us": round(us, 3),
                           "GBps": round(case.bytes / (us * 1e-6) / 1e9, 1),
                           "TFLOPs": round(case.flops / (us * 1e-6) / 1e12, 2)}
                    if path == "auto":
                        row["plan"] = lutq.plan(M, base.N, base.K, w.bits)
                    log("[sweep] " + json.dumps(row))
                    rows.append(row)
            del base
            torch.cuda.empty_cache()
    return rows


COPY_BYTES = 256 << 20


def copy_calibration(torch):
    """A plain streaming kernel that reads COPY_BYTES and writes COPY_BYTES
    once (an elementwise negation, easy to pick out of a trace by name): the
    reference for scaling FETCH_SIZE / WRITE_SIZE."""
    a = torch.ones(COPY_BYTES // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()


# template arguments: bits, MFMA, batch rows, grouped, zero points, data types,
# binary coding, bf16, prefetch depth, tiles per wave, waves, occupancy
HEADLINE_KERNEL = "matmul_kernel<4, false, 1, true, false, false, false, false, 2, 2, 8, 4, false>"
BATCH32_KERNEL = "matmul_kernel<4, true, 32, false, false, false, false, false, 2, 7, 4, 2, false>"


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _counter_per_dispatch(dirpath, counter, name_part):
    import statistics
    per = {}
    for r in _read_csv(_find(dirpath, "counter_collection.csv")):
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return statistics.median(per.values()) if per else None, len(per)


def summarize_profile(kt_dir, fetch_dir, write_dir, command=""):
    """profiles/*: kernel durations (rocprofv3 --kernel-trace --stats) and HBM
    traffic per launch (FETCH_SIZE, WRITE_SIZE in KiB, scaled by what the same
    counters read for the COPY_BYTES copy)."""
    from weight_only_lut_amd.build import source_digest
    stats = _read_csv(_find(kt_dir, "kernel_stats.csv"))
    rows = [r for r in stats if "lutq::" in r["Name"] or "copy" in r["Name"].lower()]
    copy_name = "neg_kernel"
    f_copy, n1 = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", copy_name)
    w_copy, n2 = _counter_per_dispatch(write_dir, "WRITE_SIZE", copy_name)
    f_scale = COPY_BYTES / (f_copy * 1024) if f_copy else None
    w_scale = COPY_BYTES / (w_copy * 1024) if w_copy else None
    out = {"source_digest": source_digest(), "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    import weight_only_lut_amd as lutq
    from synth import workloads
    lutq.load_library()
    for label, part, wname, M in (("int4_up_proj", HEADLINE_KERNEL, "int4_up_proj", 1),
                                  ("log4_70b_batch32", BATCH32_KERNEL, "log4_70b", 32)):
        f, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", part)
        w, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", part)
        dur = [r for r in stats if part in r["Name"]]
        wl = workloads.WORKLOADS[wname]
        mat = wl.matrices[0]
        rec = {"kernel": part, "fetch_kib_raw": f, "write_kib_raw": w, "dispatches": [nf, nw],
               "avg_duration_us": float(dur[0]["AverageNs"]) / 1e3 if dur else None,
               "plan": lutq.plan(M, mat.N, mat.K, wl.bits)}
        if f is not None and w is not None and f_scale and w_scale:
            rec["traffic_bytes_per_launch"] = round(f * 1024 * f_scale + w * 1024 * w_scale)
        out["kernels"][label] = rec
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "matmul_kernel_counters.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    lines = ["# lutq matmul kernels: rocprofv3 summary", "",
             f"Source digest of weight_only_lut_amd/csrc: `{out['source_digest']}`", "",
             "Command:", "", "```", command or "(not recorded)", "```", "",
             "## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                     f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} |")
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"Calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE = {f_copy} KiB and "
              f"WRITE_SIZE = {w_copy} KiB per dispatch; scale factors {f_scale} (fetch) and "
              f"{w_scale} (write) turn counter KiB into bytes.", "",
              "| workload | raw FETCH KiB | raw WRITE KiB | scaled bytes / launch |", "|---|---|---|---|"]
    for label, rec in out["kernels"].items():
        lines.append(f"| {label} | {rec['fetch_kib_raw']} | {rec['write_kib_raw']} | "
                     f"{rec.get('traffic_bytes_per_launch')} |")
    with open(os.path.join(ROOT, "profiles", "matmul_kernel_int4_up_proj_log4_70b.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))
    summarize_quantizer(stats, fetch_dir, write_dir, f_copy, w_copy, f_scale, w_scale, command)


# The quantizer's kernels on the 14336 x 4096 matrix of fp32 weights, as the
# benchmark's quantizer section runs them (name part, what it does, and its
# algorithmic bytes per launch: weights read, codes and scales written).
_QN, _QK = 14336, 4096
QUANT_KERNELS = (
    ("quant_kernel<16, 8, false, false, 0, false>", "grouped g128 INT4 (range rule): extrema, scale, codes",
     4 * _QN * _QK + _QN * _QK + 2 * _QN * (_QK // 128)),
    ("tensor_extrema_kernel<0>", "tensor-wise NF4, pass 1: per-workgroup extrema", 4 * _QN * _QK),
    ("tensor_scale_kernel<16>", "tensor-wise NF4, pass 2: the scale (one workgroup)", None),
    ("quant_kernel<16, 8, false, true, 0, false>", "tensor-wise NF4, pass 3: codes",
     4 * _QN * _QK + _QN * _QK),
    ("quant_kernel<16, 8, true, false, 0, true>", "NF4 g128 table tuning, one pass: error and per-code sums",
     4 * _QN * _QK + 2 * _QN * (_QK // 128)),
    ("tune_update_kernel<16>", "NF4 table tuning: the new table (one workgroup)", None),
)


def summarize_quantizer(stats, fetch_dir, write_dir, f_copy, w_copy, f_scale, w_scale, command):
    """profiles/quant_kernel_*: the quantizer kernels' durations, HBM traffic
    per launch and achieved bandwidth against the algorithmic bytes."""
    from weight_only_lut_amd.build import QUANT_SOURCES, source_digest
    rec = {"source_digest": source_digest(QUANT_SOURCES), "kernels": {}}
    lines = ["# lutq quantizer kernels: rocprofv3 summary", "",
             f"Digest of the quantizer sources: `{rec['source_digest']}`. Matrix: {_QN} x {_QK} "
             "fp32 weights, cold (rotating copies), as the benchmark's quantizer section runs it.", "",
             "Command:", "", "```", command or "(not recorded)", "```", "",
             f"Counter calibration as the matmul summary: copy FETCH_SIZE {f_copy} KiB, "
             f"WRITE_SIZE {w_copy} KiB for {COPY_BYTES >> 20} MiB.", "",
             "| kernel | what | calls | avg us | algorithmic MB | achieved GB/s | traffic MB (fetch + write) |",
             "|---|---|---|---|---|---|---|"]
    for part, what, algo in QUANT_KERNELS:
        dur = [r for r in stats if part in r["Name"]]
        avg = float(dur[0]["AverageNs"]) / 1e3 if dur else None
        f, _ = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", part)
        w, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", part)
        traffic = (round(f * 1024 * f_scale + w * 1024 * w_scale)
                   if None not in (f, w, f_scale, w_scale) else None)
        gbps = algo / (avg * 1e-6) / 1e9 if (algo and avg) else None
        rec["kernels"][part] = {"what": what, "calls": int(dur[0]["Calls"]) if dur else 0,
                                "avg_duration_us": avg, "algorithmic_bytes": algo,
                                "achieved_GBps": gbps, "traffic_bytes_per_launch": traffic}
        lines.append(f"| `{part}` | {what} | {rec['kernels'][part]['calls']} | "
                     f"{avg if avg is None else round(avg, 3)} | "
                     f"{'-' if not algo else round(algo / 1e6, 1)} | "
                     f"{'-' if gbps is None else round(gbps)} | "
                     f"{'-' if traffic is None else round(traffic / 1e6, 1)} |")
    with open(os.path.join(ROOT, "profiles", "quant_kernel_counters.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", "quant_kernel_int4_up_proj.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def load_traffic(workload, plan):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and with the same plan; else None."""
    path = os.path.join(ROOT, "profiles", "matmul_kernel_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        from weight_only_lut_amd.build import source_digest
        if rec.get("source_digest") != source_digest():
            return None
        k = rec["kernels"][workload]
        if k.get("plan") != plan:
            return None
        return k.get("traffic_bytes_per_launch")
    except (OSError, KeyError, ValueError):
        return None


if __name__ == "__main__":
    main()
