"""Benchmark of the fused LUT-dequantize + matmul on one MI355X.

Headline step: one lutq_matmul call on the Llama-3-8B MLP up-projection shape
(N = 14336, K = 4096), 4-bit uniform (INT) table, one fp16 scale per 128
weights, batch M = 1 -- the HBM-bound GEMV. Weights are "cold": every call
reads a different copy of the packed matrix, and the copies together exceed
the 256 MB Infinity Cache, so the bytes come from HBM. Also measured in the
same run (reported under "extra"):

- the same call with one warm copy (Infinity-Cache resident);
- batch 32 on the Llama-70B-shaped log table (N = 28672, K = 8192,
  tensor-wise scale): TFLOP/s against the fp16 MFMA peak;
- the machine's measured floors (peak microbenchmarks of liblutq.so): the
  launch cost, streaming reads of several sizes, the fp16 MFMA issue rate
  and the random LDS read rate;
- every workload matrix at every batch size of its config, and the
  Llama-3-8B layer as 7 calls and as 4 (fused q/k/v and gate + up), each
  against the roofline that bounds it, at published and at measured peaks;
- the quantizer, fused launches, variants and a dense fp16 context row;
- the CPU oracle on the headline workload (all cores) and on the small
  configs with all cores and with one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep]
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
CACHE_BYTES = 256 << 20        # Infinity Cache (MALL)
COLD_SET_BYTES = 2 * CACHE_BYTES
EXTRA_REPEATS = 3    # timed replays per secondary line (median)
HEADLINE_REPEATS = 7  # timed replays of the headline (median, spread reported)
SETTLE_MS = 30.0      # untimed graph replays before the timed ones, per line


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

    def at(self, torch, M):
        """The same device inputs at batch M <= self.M (the first M rows of x)."""
        c = Case.__new__(Case)
        c.__dict__.update(self.__dict__)
        c.M = M
        c.x = self.x[:M].contiguous()
        c.y = torch.empty((M, self.N), dtype=torch.float16, device="cuda")
        c.bytes = algorithmic_bytes(M, self.N, self.K, self.w.bits, self.w.group)
        c.flops = 2 * M * self.N * self.K
        c.host = self.host[:3] + (self.host[3][:M],)
        return c


class Inputs:
    """Device inputs of every workload matrix, generated once at the largest
    batch of its workload (cold copies), shared by the sections below."""

    def __init__(self, lutq, torch):
        self.lutq, self.torch, self.cases = lutq, torch, {}

    def get(self, wname, mat, M):
        from synth import workloads
        w = workloads.WORKLOADS[wname]
        key = (wname, mat or w.matrices[0].name)
        if key not in self.cases:
            self.cases[key] = Case(self.lutq, self.torch, wname, key[1], max(max(w.batches), M))
        base = self.cases[key]
        if M > base.M:
            raise ValueError(f"{key} was generated for batch {base.M}")
        return base if M == base.M else base.at(self.torch, M)


def roof_time_us(nbytes, flops, gbps, tflops):
    """Time at the bounding roofline: the larger of the memory and the MFMA time."""
    return max(nbytes / (gbps * 1e3), flops / (tflops * 1e6))


class StreamFloor:
    """Measured time of a streaming read (with its final store) of a given
    byte count, from the peak microbenchmark at several sizes: linear
    between measured sizes, never below the launch floor."""

    def __init__(self, points, empty_us):
        self.pts = sorted(points)  # (bytes, us)
        self.empty = empty_us

    def __call__(self, nbytes):
        pts = self.pts
        if nbytes <= pts[0][0]:
            b0, t0 = pts[0]
            return max(self.empty, t0 * nbytes / b0) if nbytes < b0 else t0
        for (b0, t0), (b1, t1) in zip(pts, pts[1:]):
            if nbytes <= b1:
                return t0 + (t1 - t0) * (nbytes - b0) / (b1 - b0)
        (b0, t0), (b1, t1) = pts[-2], pts[-1]
        return t1 + (t1 - t0) * (nbytes - b1) / (b1 - b0)

    def gbps(self):
        """The asymptotic rate: the slope between the two largest sizes."""
        (b0, t0), (b1, t1) = self.pts[-2], self.pts[-1]
        return (b1 - b0) / ((t1 - t0) * 1e3)


STREAM_SIZES = (1 << 20, 4 << 20, 16 << 20, 30314528 & ~15, 64 << 20, 119799842 & ~15, 256 << 20,
                512 << 20)


def peaks_section(lutq, torch, args):
    """The measured floors (include/lutq_peaks.h), timed like the matmul."""
    out = {}
    steps, warm = 50, 5
    out["empty_launch_us"] = round(time_case(lutq, torch, Fn(lambda i: lutq.peak_empty()), 200, warm,
                                             repeats=5), 3)
    log(f"[bench] peaks: empty launch {out['empty_launch_us']} us")
    pool_bytes = 3 * (512 << 20)
    pool = torch.zeros(pool_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(lutq.peak_stream_sink_bytes(), dtype=torch.uint8, device="cuda")
    rows, floor_pts = [], []
    for nbytes in STREAM_SIZES:
        ncopy = max(2, min(pool_bytes // nbytes, -(-(3 * CACHE_BYTES) // nbytes)))
        rec = {"bytes": nbytes, "copies": ncopy}
        for store in (False, True):
            fn = Fn(lambda i, b=nbytes, st=store, n=ncopy:
                    lutq.peak_stream(pool[(i % n) * b:], b, st, sink))
            us = time_case(lutq, torch, fn, max(10, steps // (1 + nbytes // (64 << 20))), warm,
                           repeats=EXTRA_REPEATS)
            rec["with_store" if store else "read_only"] = {"us": round(us, 3),
                                                          "GBps": round(nbytes / (us * 1e3), 1)}
        floor_pts.append((nbytes, rec["with_store"]["us"]))
        rows.append(rec)
        log(f"[bench] peaks: stream {nbytes / 1e6:.1f} MB: {rec['read_only']['us']} us read, "
            f"{rec['with_store']['us']} us with store")
    del pool
    torch.cuda.empty_cache()
    floor = StreamFloor(floor_pts, out["empty_launch_us"])
    out["stream"] = rows
    out["stream_asymptotic_GBps"] = round(floor.gbps(), 1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fsink = torch.zeros(cus * 16, dtype=torch.float32, device="cuda")
    mf = {}
    for kind, name in ((lutq.PEAK_MFMA_16X16X32, "16x16x32_f16"),
                       (lutq.PEAK_MFMA_32X32X16, "32x32x16_f16")):
        for wps in (1, 2, 4):
            iters = 400
            us = time_case(lutq, torch, Fn(lambda i, k=kind, w=wps: lutq.peak_mfma(k, w, iters, fsink)),
                           20, warm, repeats=EXTRA_REPEATS)
            flops = cus * 4 * wps * iters * lutq.PEAK_MFMA_FLOPS_PER_ROUND
            mf[f"{name}_waves_per_simd{wps}"] = {"us": round(us, 3),
                                                 "TFLOPs": round(flops / (us * 1e6), 1)}
    out["mfma"] = mf
    out["mfma_best_TFLOPs"] = max(v["TFLOPs"] for v in mf.values())
    log(f"[bench] peaks: fp16 MFMA best {out['mfma_best_TFLOPs']} TFLOP/s")
    isink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lds = {}
    for wpc in (4, 8, 16):
        iters = 200
        us = time_case(lutq, torch, Fn(lambda i, w=wpc: lutq.peak_lds(w, iters, isink)), 20, warm,
                       repeats=EXTRA_REPEATS)
        instrs = cus * wpc * 16 * iters
        lds[f"waves_per_cu{wpc}"] = {"us": round(us, 3),
                                     "ds_read_b32_per_us_per_cu": round(instrs / cus / us, 1),
                                     "lane_reads_per_s": round(instrs * 64 / (us * 1e-6), 0)}
    out["lds_random_read"] = lds
    out["note"] = ("stream: 2048 workgroups of 256 threads read the buffer once (16-byte nontemporal "
                   "loads), cold (rotating copies); with_store adds one 16-byte store per wave at "
                   "the end, as a matmul writing y. Each row of extra.configs is compared with the "
                   "with_store time interpolated at its algorithmic bytes.")
    return out, floor


def row_stats(us, nbytes, flops):
    """µs, GB/s, TFLOP/s and the fraction of the bounding roofline of one case."""
    spec = roof_time_us(nbytes, flops, HBM_PEAK_GBS, MFMA_F16_PEAK_TFLOPS)
    hbm_t, mfma_t = nbytes / (HBM_PEAK_GBS * 1e3), flops / (MFMA_F16_PEAK_TFLOPS * 1e6)
    return {"us": round(us, 3), "GBps": round(nbytes / (us * 1e3), 1),
            "TFLOPs": round(flops / (us * 1e6), 2), "bytes": nbytes, "flops": flops,
            "bound": "hbm" if hbm_t >= mfma_t else "mfma",
            "frac_of_roof": round(spec / us, 4)}


def measured_roof(rec, floor, mfma_meas):
    """Adds the roofline at the measured floors to a row of row_stats: the
    streaming read with its store at the same bytes, or the measured MFMA
    rate, whichever takes longer."""
    meas = max(floor(rec["bytes"]), rec["flops"] / (mfma_meas * 1e6))
    rec["measured_roof_us"] = round(meas, 3)
    rec["frac_of_measured_roof"] = round(meas / rec["us"], 4)


def add_measured_roofs(extra, floor, mfma_meas):
    for rec in extra.get("configs", []):
        measured_roof(rec, floor, mfma_meas)
    for rec in extra.get("layer_totals", []):
        measured_roof(rec["separate"], floor, mfma_meas)
        measured_roof(rec["fused"], floor, mfma_meas)
    b = extra.get("batch32")
    if b:
        r = {"us": b["us_per_call"], "bytes": b["bytes"], "flops": b["flops"]}
        measured_roof(r, floor, mfma_meas)
        b["measured_roof_us"], b["frac_of_measured_roof"] = r["measured_roof_us"], r["frac_of_measured_roof"]


class LayerCase:
    """The seven projections of the Llama-3-8B layer at batch M, cold: either
    one call per matrix, or q/k/v and gate + up as fused launches (4 calls)."""

    def __init__(self, inputs, torch, M):
        from synth import workloads
        w = workloads.WORKLOADS["nf4_layer"]
        self.parts = {m.name: inputs.get("nf4_layer", m.name, M) for m in w.matrices}
        self.fused = False
        x_q, x_g = self.parts["q"].x, self.parts["gate"].x
        K = self.parts["q"].K
        self.bytes = sum(p.bytes for p in self.parts.values())
        # q, k, v read the same x; gate and up read the same x
        self.fused_bytes = self.bytes - 2 * M * K * 2 - M * K * 2
        self.flops = sum(p.flops for p in self.parts.values())
        self.xs = {"qkv": x_q, "gate_up": x_g}

    def call(self, lutq, i):
        P = self.parts
        if not self.fused:
            for p in P.values():
                p.call(lutq, i)
            return
        for key, names in (("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up"))):
            lutq.matmul_multi(self.xs[key], [(P[n].packed[i % len(P[n].packed)], P[n].lut, P[n].scales)
                                             for n in names], outs=[P[n].y for n in names])
        P["o"].call(lutq, i)
        P["down"].call(lutq, i)


def configs_section(lutq, torch, args, inputs):
    """Every matrix of every config at each of its batch sizes (automatic plan,
    cold weights), then the Llama-3-8B layer totals."""
    from synth import workloads
    steps = max(20, args.steps // 10)
    rows = []
    for wname, w in workloads.WORKLOADS.items():
        for m in w.matrices:
            for M in w.batches:
                case = inputs.get(wname, m.name, M)
                us = time_case(lutq, torch, case, steps, args.warmup, repeats=EXTRA_REPEATS)
                rec = {"workload": wname, "matrix": m.name, "N": m.N, "K": m.K, "M": M,
                       "bits": w.bits, "table": w.table, "group": w.group,
                       "plan": lutq.plan(M, m.N, m.K, w.bits)}
                rec.update(row_stats(us, case.bytes, case.flops))
                rec["bits_read_per_weight"] = round(case.bytes * 8 / (m.N * m.K), 4)
                rows.append(rec)
                log(f"[bench] config {wname}/{m.name} M={M}: {us:.2f} us, {rec['GBps']} GB/s, "
                    f"{rec['frac_of_roof']:.3f} of roof")
    layer = []
    for M in workloads.WORKLOADS["nf4_layer"].batches:
        lc = LayerCase(inputs, torch, M)
        rec = {"M": M, "calls_separate": 7, "calls_fused": 4}
        for fused in (False, True):
            lc.fused = fused
            us = time_case(lutq, torch, lc, max(10, steps // 2), args.warmup, repeats=EXTRA_REPEATS)
            nbytes = lc.fused_bytes if fused else lc.bytes
            rec["fused" if fused else "separate"] = row_stats(us, nbytes, lc.flops)
        rec["floor_us_at_8TBps"] = round(lc.bytes / (HBM_PEAK_GBS * 1e3), 3)
        layer.append(rec)
        log(f"[bench] layer M={M}: 7 calls {rec['separate']['us']} us, 4 calls {rec['fused']['us']} us")
    return rows, layer


class Fn:
    """A timed step that calls f(i) (i = the call's index in the graph)."""

    def __init__(self, f):
        self.f = f

    def call(self, lutq, i):
        self.f(i)


def time_replays(lutq, torch, case, steps, warmup, repeats=1):
    """Microseconds per call of every timed replay of `steps` back-to-back calls.

    `warmup` eager calls, then the `steps` calls are captured in a HIP graph,
    replayed untimed for about SETTLE_MS milliseconds (the first replays
    after an idle spell run at lower clocks), and replayed `repeats` more
    times, each between HIP events recorded on the stream the kernels run on
    (host-side launch cost stays outside the timed region), with a device
    synchronization on both sides.
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
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record()
        graph.replay()
        stop.record()
    torch.cuda.synchronize()
    settle = min(2000, int(SETTLE_MS / max(start.elapsed_time(stop), 1e-3)))
    with torch.cuda.stream(stream):
        for _ in range(settle):
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
    del graph
    return times


def time_case(lutq, torch, case, steps, warmup, repeats=1):
    """The median of time_replays (one replay of a few tens of calls varies by
    up to ~10%, hence the median for every line)."""
    times = sorted(time_replays(lutq, torch, case, steps, warmup, repeats))
    return times[len(times) // 2]


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
    tables) on the headline matrix's shape at batch 1 and 16, against the
    plain launch, and binary-coded weights (q = 3) on that shape at batch 1,
    16 and 32 (cold)."""
    out = {}
    steps = max(20, args.steps // 4)
    for M in (1, 16, 32):
        if M < 32:
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
                                           "GBps": round(bc.bytes / (us * 1e-6) / 1e9, 1),
                                           "plan": lutq.plan(M, bc.N, bc.K, 3)}
        log(f"[bench] variants M={M} bcq q=3: {us:.2f} us")
        del bc
        torch.cuda.empty_cache()
    return out


class FusedCase:
    """Matrices of one layer that read the same activations (Llama-3-8B q/k/v,
    or gate and up), cold, called either as one lutq_matmul per matrix or as
    one fused lutq_matmul_multi."""

    def __init__(self, inputs, wname, mats, M):
        self.parts = [inputs.get(wname, m, M) for m in mats]
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


def fused_section(lutq, torch, args, inputs):
    """One fused launch against one launch per matrix, for q/k/v and gate/up
    of the Llama-3-8B layer at batch 1 and 16 (cold weights)."""
    out = {}
    steps = max(20, args.steps // 4)
    for label, mats in (("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up"))):
        for M in (1, 16):
            fc = FusedCase(inputs, "nf4_layer", mats, M)
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
    return out


def cpu_oracle_section(inputs, budget_s=4.0):
    """The oracle on the small configs (batch 1), with all host cores and with
    one BLAS thread: seconds per call and GB/s of algorithmic bytes."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # threadpoolctl missing: all-cores numbers only
        threadpool_limits = None
    out = {}
    for wname, mat in (("nf4_1k", "w"), ("int4_up_proj", "up"), ("lm3", "sq"), ("lm3", "wide")):
        case = inputs.cases[(wname, mat)]
        c, T, s, x = case.host
        w = case.w
        x1 = x[:1]
        nbytes = algorithmic_bytes(1, case.N, case.K, w.bits, w.group)
        packed = oracle.pack_codes(c, w.bits)
        rec = {"N": case.N, "K": case.K, "M": 1, "bits": w.bits}

        def run():
            times, t_all = [], time.time()
            while (time.time() - t_all < budget_s and len(times) < 5) or len(times) < 1:
                t0 = time.time()
                codes = oracle.unpack_codes(packed, case.N, case.K, w.bits)
                oracle.reference(x1, codes, T, s, w.group)
                times.append(time.time() - t0)
            return float(np.median(times)), len(times)

        sec, n = run()
        rec["all_cores"] = {"seconds": round(sec, 4), "GBps": round(nbytes / sec / 1e9, 4), "runs": n,
                            "cores": len(os.sched_getaffinity(0))}
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                sec1, n1 = run()
            rec["one_core"] = {"seconds": round(sec1, 4), "GBps": round(nbytes / sec1 / 1e9, 4),
                               "runs": n1, "cores": 1}
        out[f"{wname}/{mat}"] = rec
        log(f"[bench] cpu oracle {wname}/{mat}: {rec['all_cores']['seconds']} s all cores, "
            f"{rec.get('one_core', {}).get('seconds')} s one core")
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
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak microbenchmarks")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config rows and the layer totals")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense fp16 (torch) context timings")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the zero-point and data-type timings")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the Infinity-Cache-warm repeats (so a kernel trace holds cold calls only)")
    ap.add_argument("--sweep", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--profile-set", action="store_true",
                    help="only the profiled cases (headline, batch 32, 3-bit, batch 16), cold, "
                         "plus the copy calibration: the workload of the committed rocprofv3 summaries")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling memory counters)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("KERNEL_TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 output and exit")
    ap.add_argument("--summarize-sq", metavar="SQ_DIR",
                    help="write the SQ-counter summary from a rocprofv3 --pmc run and exit")
    ap.add_argument("--summarize-mem", nargs=2, metavar=("PASS_A_DIR", "PASS_B_DIR"),
                    help="write the memory-pipeline counter summary from the two rocprofv3 --pmc "
                         "passes (MEM_COUNTERS_A, MEM_COUNTERS_B) and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, command=args.profile_command)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, command=args.profile_command)
        return
    if args.summarize_mem:
        summarize_mem(*args.summarize_mem, command=args.profile_command)
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
    if args.profile_set:
        profile_set(lutq, torch, args)
        return
    inputs = Inputs(lutq, torch)

    # ---- headline: batch-1 4-bit g128 GEMV, cold weights ------------------
    head = inputs.get("int4_up_proj", None, 1)
    hplan = lutq.plan(1, head.N, head.K, 4)
    log(f"[bench] headline: {len(head.packed)} rotating copies, plan={hplan}")
    head_times = time_replays(lutq, torch, head, args.steps, args.warmup, repeats=HEADLINE_REPEATS)
    region_us = sorted(head_times)[len(head_times) // 2]
    w_region_us = None
    if not args.no_warm:
        warm = Case.__new__(Case)
        warm.__dict__.update(head.__dict__)
        warm.packed = head.packed[:1]
        w_region_us = time_case(lutq, torch, warm, args.steps, args.warmup, repeats=EXTRA_REPEATS)
    log(f"[bench] headline cold: {region_us:.3f} us/call (replays {[round(t, 3) for t in head_times]}); "
        f"warm: {w_region_us} us/call")

    value = head.bytes / (region_us * 1e-6) / 1e9
    achieved = value
    traffic = load_traffic("int4_up_proj", hplan)

    extra = {
        "us_per_call": round(region_us, 3),
        "replays_us": [round(t, 3) for t in head_times],
        "spread_us": [round(min(head_times), 3), round(max(head_times), 3)],
        "bits_read_per_weight": round(head.bytes * 8 / (head.N * head.K), 4),
        "warm": None if w_region_us is None else {
            "us_per_call": round(w_region_us, 3),
            "effective_GBps": round(head.bytes / (w_region_us * 1e-6) / 1e9, 1)},
        "plan": hplan,
    }

    # ---- batch 32: log table, Llama-70B up-projection shape ---------------
    k_us = None
    if not args.no_batch32:
        b32 = inputs.get("log4_70b", None, 32)
        p32 = lutq.plan(32, b32.N, b32.K, 4)
        k_us = time_case(lutq, torch, b32, max(20, args.steps // 4), args.warmup, repeats=5)
        wk_us = None
        if not args.no_warm:
            warm32 = Case.__new__(Case)
            warm32.__dict__.update(b32.__dict__)
            warm32.packed = b32.packed[:1]
            wk_us = time_case(lutq, torch, warm32, max(20, args.steps // 4), args.warmup,
                              repeats=EXTRA_REPEATS)
            del warm32
        tf = b32.flops / (k_us * 1e-6) / 1e12
        gbps = b32.bytes / (k_us * 1e-6) / 1e9
        extra["batch32"] = {
            "workload": "log4_70b", "N": b32.N, "K": b32.K, "M": 32, "plan": p32,
            "us_per_call": round(k_us, 3),
            "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "effective_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
            "bytes": b32.bytes, "flops": b32.flops,
            "bound": "hbm (cold: arithmetic intensity below the machine balance)",
            "frac_of_roof": round(roof_time_us(b32.bytes, b32.flops, HBM_PEAK_GBS,
                                               MFMA_F16_PEAK_TFLOPS) / k_us, 4),
            "warm": None if wk_us is None else {
                "us_per_call": round(wk_us, 3),
                "TFLOPs": round(b32.flops / (wk_us * 1e-6) / 1e12, 1),
                "mfma_frac": round(b32.flops / (wk_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        }
        log(f"[bench] batch32 cold {k_us:.2f} us = {tf:.1f} TFLOP/s; warm {wk_us} us")

    if not args.no_configs:
        extra["configs"], extra["layer_totals"] = configs_section(lutq, torch, args, inputs)
    if not args.no_fused:
        extra["fused"] = fused_section(lutq, torch, args, inputs)
    if not args.no_quantizer:
        extra["quantizer"] = quantizer_section(lutq, torch, args)
    if not args.no_variants:
        extra["variants"] = variant_section(lutq, torch, args)
    if not args.no_dense:
        extra["dense_fp16"] = dense_section(
            torch, args, {"int4_up_proj_M1": region_us, "log4_70b_M32": k_us})

    if args.sweep:
        extra["sweep"] = sweep(lutq, torch, args)

    # The measured floors last: the MFMA microbenchmark runs the matrix pipes
    # flat out, and nothing timed above should run right after it.
    floor = None
    if not args.no_peaks:
        extra["peaks"], floor = peaks_section(lutq, torch, args)
        mfma_meas = extra["peaks"]["mfma_best_TFLOPs"]
        stream_us = floor(head.bytes)
        extra["peaks"]["headline"] = {
            "stream_with_store_us_at_headline_bytes": round(stream_us, 3),
            "frac_of_measured": round(stream_us / region_us, 4)}
        add_measured_roofs(extra, floor, mfma_meas)

    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head, budget_s=10.0)
        if not args.no_configs:
            extra["cpu_oracle"] = cpu_oracle_section(inputs)

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    if floor is not None:
        roofline["measured_peak"] = round(head.bytes / (floor(head.bytes) * 1e3), 1)
        roofline["frac_of_measured"] = round(achieved / roofline["measured_peak"], 4)
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
        "roofline": roofline,
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
                shapes = [("auto", 0)] + [("mfma", t) for t in (1, 2, 4, 7, 8)]
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


# The cases of the committed rocprofv3 summaries (label, workload, matrix, M):
# the headline GEMV, the batch-32 MFMA kernel, the 3-bit GEMV and 3-bit MFMA
# kernels (the non-evenly-divisible width), and batch-16 MFMA launches of the
# 4-tile and 1-tile shapes. Each runs a distinct kernel instantiation, so
# kernel names identify the cases.
PROFILE_CASES = (
    ("int4_up_proj", "int4_up_proj", "up", 1),
    ("log4_70b_batch32", "log4_70b", "up", 32),
    ("lm3_wide_M1", "lm3", "wide", 1),
    ("lm3_wide_M8", "lm3", "wide", 8),
    ("nf4_gate_M16", "nf4_layer", "gate", 16),
    ("nf4_q_M16", "nf4_layer", "q", 16),
)


def kernel_signature(bits, group, M, plan):
    """The matmul_kernel instantiation lutq_matmul launches for this plan (the
    launch rules of lutq_matmul.hip for plain tables and fp16 activations):
    template arguments bits, MFMA, batch rows, grouped, zero points, data
    types, binary coding, bf16, prefetch depth, tiles per wave, waves,
    occupancy, staged activations."""
    tiles, grouped = plan["tiles"], group > 0
    if plan["path"] == "gemv":
        mrows = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
        occ = 4 if mrows <= 2 else 2
        pf = 4 if (mrows == 1 and tiles == 1) else 2
        waves, xs = 8, False
        mfma = False
    else:
        mfma, pf = True, 2
        mrows = 16 if M <= 16 else 32
        if tiles in (7, 8):
            waves, occ, xs = 4, 2, False
            if grouped and mrows == 32:
                occ = 1
        elif tiles == 4:
            waves, occ, xs = (8, 2, True) if mrows == 32 else (4, 2, False)
        else:
            waves, occ, xs = (8, 2, mrows == 32 or M > 8)
    b = lambda v: "true" if v else "false"
    return (f"matmul_kernel<{bits}, {b(mfma)}, {mrows}, {b(grouped)}, false, false, false, false, "
            f"{pf}, {tiles}, {waves}, {occ}, {b(xs)}>")


def profile_set(lutq, torch, args):
    """The profiled workload: each case of PROFILE_CASES timed as in the
    benchmark (cold weights, graph replays), the quantizer section, then the
    256 MiB copy that calibrates the memory counters."""
    inputs = Inputs(lutq, torch)
    for label, wname, mat, M in PROFILE_CASES:
        case = inputs.get(wname, mat, M)
        us = time_case(lutq, torch, case, args.steps, args.warmup, repeats=EXTRA_REPEATS)
        log(f"[profile-set] {label}: {us:.3f} us per call")
        del inputs.cases[(wname, mat)], case
        torch.cuda.empty_cache()
    quantizer_section(lutq, torch, args)
    copy_calibration(torch)
    torch.cuda.synchronize()
    print(json.dumps({"profile_set": [c[0] for c in PROFILE_CASES]}), flush=True)


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


def _median_duration_us(trace, name_part):
    """Median per-dispatch duration (kernel trace) of the kernels whose name
    contains name_part, in microseconds."""
    import statistics
    d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace
         if name_part in r["Kernel_Name"]]
    return round(statistics.median(d) / 1e3, 3) if d else None


def _timed_avg_us(trace, name_part, ncalls):
    """Average duration of the last `ncalls` dispatches (by start time) of the
    kernels whose name contains name_part: the timed replays of time_replays,
    which follow the warm-up calls and the settle phase."""
    d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
               if name_part in r["Kernel_Name"])
    d = d[-ncalls:]
    return round(sum(e - b for b, e in d) / len(d) / 1e3, 3) if len(d) == ncalls else None


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
    counters read for the COPY_BYTES copy) of the PROFILE_CASES kernels, one
    summary per kernel and workload, plus the counters json."""
    from weight_only_lut_amd.build import source_digest
    stats = _read_csv(_find(kt_dir, "kernel_stats.csv"))
    trace = _read_csv(_find(kt_dir, "kernel_trace.csv"))
    copy_name = "neg_kernel"
    f_copy, _ = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", copy_name)
    w_copy, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", copy_name)
    f_scale = COPY_BYTES / (f_copy * 1024) if f_copy else None
    w_scale = COPY_BYTES / (w_copy * 1024) if w_copy else None
    out = {"source_digest": source_digest(), "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    import weight_only_lut_amd as lutq
    from synth import workloads
    lutq.load_library()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    # the timed replays of the traced run: EXTRA_REPEATS replays of --steps calls
    steps = re.search(r"--profile-set --steps (\d+)", command or "")
    ntimed = EXTRA_REPEATS * int(steps.group(1)) if steps else None
    for label, wname, mat, M in PROFILE_CASES:
        wl = workloads.WORKLOADS[wname]
        _, m = wl.matrix(mat)
        plan = lutq.plan(M, m.N, m.K, wl.bits)
        part = kernel_signature(wl.bits, wl.group, M, plan)
        f, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", part)
        w, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", part)
        dur = [r for r in stats if part in r["Name"]]
        nbytes = algorithmic_bytes(M, m.N, m.K, wl.bits, wl.group)
        flops = 2 * M * m.N * m.K
        avg = float(dur[0]["AverageNs"]) / 1e3 if dur else None
        rec = {"kernel": part, "workload": wname, "matrix": mat, "N": m.N, "K": m.K, "M": M,
               "fetch_kib_raw": f, "write_kib_raw": w, "dispatches": [nf, nw],
               "calls": int(dur[0]["Calls"]) if dur else 0, "avg_duration_us": avg,
               "min_duration_us": float(dur[0]["MinNs"]) / 1e3 if dur else None,
               "max_duration_us": float(dur[0]["MaxNs"]) / 1e3 if dur else None,
               "median_duration_us": _median_duration_us(trace, part),
               "timed_avg_duration_us": _timed_avg_us(trace, part, ntimed) if ntimed else None,
               "plan": plan, "algorithmic_bytes": nbytes, "flops": flops}
        if avg:
            rec["achieved_GBps"] = round(nbytes / (avg * 1e3), 1)
            rec["achieved_TFLOPs"] = round(flops / (avg * 1e6), 2)
            rec["frac_of_roof"] = round(roof_time_us(nbytes, flops, HBM_PEAK_GBS,
                                                     MFMA_F16_PEAK_TFLOPS) / avg, 4)
        if f is not None and w is not None and f_scale and w_scale:
            rec["traffic_bytes_per_launch"] = round(f * 1024 * f_scale + w * 1024 * w_scale)
            rec["traffic_over_algorithmic"] = round(rec["traffic_bytes_per_launch"] / nbytes, 4)
        out["kernels"][label] = rec
        lines = [f"# `{part}` on `{wname}` {mat} (N = {m.N}, K = {m.K}), batch {M}: rocprofv3 summary", "",
                 f"Source digest of the matmul kernel sources: `{out['source_digest']}`; plan {plan}.", "",
                 "Command (cold weights, rotating copies; `<repo>` is the repository root):", "", "```",
                 command or "(not recorded)", "```", "",
                 "| quantity | value |", "|---|---|",
                 f"| calls traced | {rec['calls']} |",
                 f"| average duration (kernel trace) | {avg if avg is None else round(avg, 3)} us |",
                 f"| min / median / max duration | {rec['min_duration_us']} / "
                 f"{rec['median_duration_us']} / {rec['max_duration_us']} us |",
                 f"| average of the timed replays (the last {ntimed} dispatches, after the warm-up calls "
                 f"and the settle phase, as the benchmark times them) | {rec['timed_avg_duration_us']} us |",
                 f"| algorithmic bytes per launch | {nbytes:,} |",
                 f"| achieved (algorithmic bytes / average duration) | {rec.get('achieved_GBps')} GB/s, "
                 f"{rec.get('achieved_TFLOPs')} TFLOP/s |",
                 f"| fraction of the bounding roof (8 TB/s, 2.5 PFLOP/s) | {rec.get('frac_of_roof')} |",
                 f"| FETCH_SIZE / WRITE_SIZE per dispatch (raw KiB, median) | {f} / {w} |",
                 f"| HBM traffic per launch (scaled) | {rec.get('traffic_bytes_per_launch')} bytes "
                 f"({rec.get('traffic_over_algorithmic')} of algorithmic) |", "",
                 f"Counter calibration: a {COPY_BYTES >> 20} MiB device copy reads FETCH_SIZE = {f_copy} "
                 f"KiB and WRITE_SIZE = {w_copy} KiB per dispatch; scale factors {f_scale} (fetch) and "
                 f"{w_scale} (write) turn counter KiB into bytes."]
        with open(os.path.join(ROOT, "profiles", f"matmul_kernel_{label}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "matmul_kernel_counters.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    if any("quant_kernel" in r["Name"] for r in stats):
        summarize_quantizer(stats, fetch_dir, write_dir, f_copy, w_copy, f_scale, w_scale, command)


SQ_COUNTERS = ("SQ_WAVES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES")


def summarize_sq(sq_dir, command=""):
    """profiles/matmul_kernel_sq_counters.md: the SQ counters of the
    PROFILE_CASES kernels (median per dispatch)."""
    import weight_only_lut_amd as lutq
    from synth import workloads
    from weight_only_lut_amd.build import source_digest
    lutq.load_library()
    cols = []
    for label, wname, mat, M in PROFILE_CASES:
        wl = workloads.WORKLOADS[wname]
        _, m = wl.matrix(mat)
        part = kernel_signature(wl.bits, wl.group, M, lutq.plan(M, m.N, m.K, wl.bits))
        vals = {c: _counter_per_dispatch(sq_dir, c, part) for c in SQ_COUNTERS}
        cols.append((label, part, vals))
    lines = ["# lutq matmul kernels: SQ counters (rocprofv3 --pmc)", "",
             f"Source digest of the matmul kernel sources: `{source_digest()}`. Medians per dispatch "
             "over the run; kernels as in the per-case summaries `matmul_kernel_<case>.md`.", "",
             "Command (`<repo>` is the repository root):", "", "```", command or "(not recorded)", "```", "",
             "| counter | " + " | ".join(f"`{c[0]}`" for c in cols) + " |",
             "|---|" + "---|" * len(cols)]
    for cname in SQ_COUNTERS:
        row = []
        for _, _, vals in cols:
            v, n = vals[cname]
            if v is None:
                row.append("-")
                continue
            cell = f"{v:,.0f}"
            waves, wave_cycles, busy = (vals["SQ_WAVES"][0], vals["SQ_WAVE_CYCLES"][0],
                                        vals["SQ_BUSY_CU_CYCLES"][0])
            if cname == "SQ_WAIT_INST_ANY" and wave_cycles:
                cell += f" ({v / wave_cycles:.0%} of wave cycles)"
            elif cname in ("SQ_INSTS_LDS", "SQ_INSTS_MFMA") and waves:
                cell += f" ({v / waves:,.1f} per wave)"
            elif cname == "SQ_LDS_BANK_CONFLICT" and vals["SQ_INSTS_LDS"][0]:
                cell += f" ({v / vals['SQ_INSTS_LDS'][0]:.2f} per LDS instruction)"
            elif cname == "SQ_VALU_MFMA_BUSY_CYCLES" and busy:
                cell += f" ({v / (4 * busy):.1%} of the SIMDs' busy cycles)"
            row.append(cell)
        lines.append(f"| {cname} | " + " | ".join(row) + " |")
    lines += ["", "Kernels:", ""] + [f"- `{c[0]}`: `{c[1]}`" for c in cols]
    with open(os.path.join(ROOT, "profiles", "matmul_kernel_sq_counters.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


# Memory-pipeline counters of the profiled kernels, in two rocprofv3 --pmc
# passes (each within one pass's counter limits): the address (TA) and data
# (TD) units and the vector L1 (TCP), then the L2 (TCC) and the address
# unit's stalls on it. GRBM_GUI_ACTIVE (GPU busy cycles) normalizes both.
MEM_COUNTERS_A = ("TA_TA_BUSY_sum", "TA_BUFFER_READ_WAVEFRONTS_sum", "TD_TD_BUSY_sum",
                  "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCC_READ_REQ_sum",
                  "TCP_TCP_TA_DATA_STALL_CYCLES_sum", "TCP_PENDING_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE")
MEM_COUNTERS_B = ("TCC_HIT_sum", "TCC_MISS_sum", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
                  "TA_DATA_STALLED_BY_TC_CYCLES_sum", "GRBM_GUI_ACTIVE")


def _gpu_cu_count(dirpath):
    for r in _read_csv(_find(dirpath, "agent_info.csv")):
        if r.get("Agent_Type") == "GPU":
            return int(r["Cu_Count"])
    return None


def summarize_mem(dir_a, dir_b, command=""):
    """profiles/matmul_kernel_mem_counters.md: the memory-pipeline counters of
    the PROFILE_CASES kernels (median per dispatch), with the busy fractions
    and hit rates derived from them."""
    import weight_only_lut_amd as lutq
    from synth import workloads
    from weight_only_lut_amd.build import source_digest
    lutq.load_library()
    cus = _gpu_cu_count(dir_a) or 256
    cols = []
    for label, wname, mat, M in PROFILE_CASES:
        wl = workloads.WORKLOADS[wname]
        _, m = wl.matrix(mat)
        part = kernel_signature(wl.bits, wl.group, M, lutq.plan(M, m.N, m.K, wl.bits))
        vals = {c: _counter_per_dispatch(dir_a, c, part)[0] for c in MEM_COUNTERS_A}
        vals.update({f"{c}@B": _counter_per_dispatch(dir_b, c, part)[0] for c in MEM_COUNTERS_B})
        cols.append((label, part, vals))

    def frac(a, b):
        return f"{a / b:.1%}" if a is not None and b else "-"

    derived = [
        ("address unit (TA) busy, of GPU busy cycles x CUs",
         lambda v: frac(v["TA_TA_BUSY_sum"], v["GRBM_GUI_ACTIVE"] and v["GRBM_GUI_ACTIVE"] * cus)),
        ("data unit (TD) busy, of GPU busy cycles x CUs",
         lambda v: frac(v["TD_TD_BUSY_sum"], v["GRBM_GUI_ACTIVE"] and v["GRBM_GUI_ACTIVE"] * cus)),
        ("buffer-load wave instructions per dispatch",
         lambda v: f"{v['TA_BUFFER_READ_WAVEFRONTS_sum']:,.0f}" if v["TA_BUFFER_READ_WAVEFRONTS_sum"] else "-"),
        ("L1 (TCP) tag accesses per buffer-load instruction",
         lambda v: (f"{v['TCP_TOTAL_CACHE_ACCESSES_sum'] / v['TA_BUFFER_READ_WAVEFRONTS_sum']:.1f}"
                    if v["TCP_TOTAL_CACHE_ACCESSES_sum"] and v["TA_BUFFER_READ_WAVEFRONTS_sum"] else "-")),
        ("L1 accesses that go on to the L2",
         lambda v: frac(v["TCP_TCC_READ_REQ_sum"], v["TCP_TOTAL_CACHE_ACCESSES_sum"])),
        ("L2 (TCC) hit rate",
         lambda v: frac(v["TCC_HIT_sum@B"], (v["TCC_HIT_sum@B"] or 0) + (v["TCC_MISS_sum@B"] or 0))),
        ("TA address stalled by the cache, of TA busy (second pass)",
         lambda v: frac(v["TA_ADDR_STALLED_BY_TC_CYCLES_sum@B"], v["TA_TA_BUSY_sum"])),
        ("TA data stalled by the cache, of TA busy (second pass)",
         lambda v: frac(v["TA_DATA_STALLED_BY_TC_CYCLES_sum@B"], v["TA_TA_BUSY_sum"])),
        ("L1 pending-request stall cycles, per CU and GPU busy cycle",
         lambda v: frac(v["TCP_PENDING_STALL_CYCLES_sum"], v["GRBM_GUI_ACTIVE"] and v["GRBM_GUI_ACTIVE"] * cus)),
    ]
    lines = ["# lutq matmul kernels: memory-pipeline counters (rocprofv3 --pmc)", "",
             f"Source digest of the matmul kernel sources: `{source_digest()}`. Medians per dispatch "
             f"over each run ({cus} CUs); kernels as in the per-case summaries `matmul_kernel_<case>.md`.",
             "The two passes are separate runs of the same workload, so ratios across them are "
             "approximate.", "",
             "Commands (`<repo>` is the repository root):", "", "```", command or "(not recorded)", "```", "",
             "| derived | " + " | ".join(f"`{c[0]}`" for c in cols) + " |",
             "|---|" + "---|" * len(cols)]
    for name, fn in derived:
        lines.append(f"| {name} | " + " | ".join(fn(v) for _, _, v in cols) + " |")
    lines += ["", "| counter (median per dispatch) | " + " | ".join(f"`{c[0]}`" for c in cols) + " |",
              "|---|" + "---|" * len(cols)]
    for cname in list(MEM_COUNTERS_A) + [f"{c}@B" for c in MEM_COUNTERS_B]:
        lines.append(f"| {cname.replace('@B', ' (second pass)')} | " + " | ".join(
            f"{v[cname]:,.0f}" if v[cname] is not None else "-" for _, _, v in cols) + " |")
    lines += ["", "Kernels:", ""] + [f"- `{c[0]}`: `{c[1]}`" for c in cols]
    with open(os.path.join(ROOT, "profiles", "matmul_kernel_mem_counters.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


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
