#!/usr/bin/env python3
"""Benchmark of the int4 group-64 affine linear-layer hot path on one MI355X.

One step = one pass of the whole hot path on synthetic inputs shaped like the pages'
workloads ("The inference engine -- Mojo 1.0 on Metal", "Crossing Mojo 1.0"):
  decode  -- a Qwen2.5-3B-shaped decode token at M = 1: 36 layers x (q, k, v, o, gate, up,
             down) int4 GEMVs, then the f16 LM head 2048 -> 151936 and on-device top-40;
  prefill -- a 1570-token prefill of the three MLP matrices (gate, up: 2048 -> 11008;
             down: 11008 -> 2048): each weight dequantized once into a transposed f16
             scratch (gate and up into the two halves of one 2048 x 22016 scratch, as they
             read the same activations), then f16 GEMMs with f32 accumulation.
Each phase is captured once as a HIP graph and replayed; HIP events on the replay stream
time the phases inside every timed step.

Printed (one JSON line): value = int4 GEMV GB/s of the decode phase (algorithmic bytes:
N*K/2 codes + N*K/16 scales/biases + 2*M*K x + 4*M*N y per GEMV) and, beside it, the
prefill's dequant+GEMM TFLOP/s (2*M*N*K per GEMM over the phase's wall time), each as a
fraction of MI355X's 8 TB/s HBM and 2.5 PFLOP/s dense f16.  `roofline` is the dominant
GEMV kernel's own rate from per-launch HIP events; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.  `stats` gives, per phase, the median of the timed
steps and its 95 % bootstrap interval (2000 resamples, as in "Engineering investigation: can
this MLX port become another 10x faster?", "Experimental controls and limits"); `context` a
1 GiB device copy's bandwidth and the clocks rocm-smi reports after timing (context, not
denominators).  Outputs of the timed steps are re-checked against the oracle on sampled rows
before anything is printed.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30  # distinct bytes a timed loop cycles through (4x the 256 MB last-level cache)
METRIC = "W4 GEMV GB/s (% of HBM peak); prefill dequant+GEMM TFLOP/s (% MFMA peak)"
TOPK = 40


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--eager", action="store_true", help="launch every kernel from Python instead of replaying graphs")
    p.add_argument("--unfused", action="store_true", help="run q,k,v and gate,up as separate GEMVs (7 per layer)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the parity re-check of the timed outputs")
    p.add_argument("--no-small-m", action="store_true", help="skip the side sections: batched (M = 16, 8), Gemma-shaped and symmetric group-128 GEMVs, speculative verify, the quantizer and the packer")
    p.add_argument("--counters", metavar="MANIFEST",
                   help="counter-collection pass: launch each kernel shape of the step 3 times (eagerly, between "
                        "marker kernels) plus a copy of known size, write the launch plan to MANIFEST and exit; "
                        "run under rocprofv3 --pmc")
    p.add_argument("--util-from", nargs=2, metavar=("MANIFEST", "UTIL_CSV"),
                   help="reduce a `rocprofv3 --pmc VALUBusy MfmaUtil` run of --counters into profiles/utilization.json")
    p.add_argument("--trace-from", nargs="+", metavar="FILE",
                   help="(no GPU) PROFILED_JSON TRACE_CSV [UNPROFILED_JSON]: reduce a rocprofv3 --kernel-trace run "
                        "of bench.py (its JSON line and its kernel_trace.csv) into profiles/kernel_trace.json, "
                        "rocprof durations per kernel shape beside the unprofiled run's per-launch times")
    p.add_argument("--traffic-from", nargs=3, metavar=("MANIFEST", "READ_CSV", "WRITE_CSV"),
                   help="(no GPU) turn the counter CSVs of two --counters passes (read requests by size, then "
                        "write requests) into profiles/traffic.json and print a table of them")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sha256_of(*arrays):
    """SHA-256 of host buffers' bytes, in order (C order, native little-endian)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(memoryview(a).cast("B") if a.flags.c_contiguous else a.tobytes())
    return h.hexdigest()


def gemv_bytes(m, n, k):
    return n * k // 2 + n * k // 16 + 2 * m * k + 4 * m * n


class Workload:
    """Device buffers of the decode step and the prefill, plus the host copies the oracle
    needs for the parity re-check (only of sampled layers)."""

    def __init__(self, torch, np, w4, synth, unfused=False):
        self.torch, self.np, self.w4, self.synth = torch, np, w4, synth
        dev = "cuda"
        t0 = time.time()
        self.layers = []  # per layer: list of (names, qw, s, b, x, y, (M, N, K))
        self.gemv_bytes = 0
        # SHA-256 of every input buffer as drawn on the host; a decode layer's buffers are
        # summarised by one digest over their own digests, in launch order (codes, scales,
        # biases of each GEMV, then each activation vector the first time it is read)
        self.sha = {"decode_layers": []}
        # q, k, v read one activation and gate, up another (as in the model); by default each
        # group is stored row-concatenated so it runs as one GEMV (identical outputs).
        groups = ([["q"], ["k"], ["v"], ["o"], ["gate"], ["up"], ["down"]] if unfused
                  else [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]])
        shapes = {name: (j, n, k) for j, (name, n, k) in enumerate(synth.QWEN25_3B_LAYER)}
        src_of = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}
        for l in range(synth.QWEN25_3B_LAYERS):
            xs = {}
            mats = []
            digests = []
            for grp in groups:
                qs, ss, bs = [], [], []
                for name in grp:
                    j, n, k = shapes[name]
                    q, s, b = synth.w4_weights(n, k, seed=0, workload=synth.W_DECODE, layer=l * 16 + j)
                    qs.append(q); ss.append(s); bs.append(b)
                q, s, b = np.concatenate(qs), np.concatenate(ss), np.concatenate(bs)
                digests += [sha256_of(q), sha256_of(s), sha256_of(b)]
                n, k = q.shape
                qw = w4.w4_pack(torch.from_numpy(q).to(dev))
                src = src_of[grp[0]]
                if src not in xs:
                    slot = ["attn", "o", "mlp", "down"].index(src)
                    xh = synth.activations(1, k, seed=0, workload=synth.W_DECODE, layer=l * 16 + 8 + slot)
                    digests.append(sha256_of(xh))
                    xs[src] = torch.from_numpy(xh).to(dev)
                y = torch.empty((1, n), dtype=torch.float32, device=dev)
                mats.append(("+".join(grp), qw, torch.from_numpy(s).to(dev), torch.from_numpy(b).to(dev), xs[src], y,
                             (1, n, k)))
                self.gemv_bytes += gemv_bytes(1, n, k)
            self.layers.append(mats)
            self.sha["decode_layers"].append(hashlib.sha256("".join(digests).encode()).hexdigest())
        log(f"decode weights packed on the GPU in {time.time() - t0:.1f}s ({self.gemv_bytes / 1e9:.3f} GB per step)")

        t0 = time.time()
        self.V, self.H = synth.QWEN25_3B_VOCAB, synth.QWEN25_3B_HIDDEN
        self.head_host = synth.head_f16(self.H, self.V, seed=0, workload=synth.W_DECODE, layer=999)
        self.head = torch.from_numpy(self.head_host).to(dev)
        self.x_head_host = synth.activations(1, self.H, seed=0, workload=synth.W_DECODE, layer=998)
        self.sha["head"] = sha256_of(self.head_host)
        self.sha["x_head"] = sha256_of(self.x_head_host)
        self.x_head = torch.from_numpy(self.x_head_host).to(dev)
        self.logits = torch.empty((1, self.V), dtype=torch.float32, device=dev)
        self.idx = torch.empty((1, TOPK), dtype=torch.int32, device=dev)
        self.val = torch.empty((1, TOPK), dtype=torch.float32, device=dev)
        self.topk_ws = torch.empty(max(16, w4.topk_workspace_bytes(1, self.V, TOPK)), dtype=torch.uint8, device=dev)
        self.head_bytes = 2 * self.H * self.V + 2 * self.H + 4 * self.V + 4 * self.V  # head + x + logits w/r
        log(f"f16 head [{self.H}][{self.V}] ready in {time.time() - t0:.1f}s")

        t0 = time.time()
        self.M = synth.PREFILL_TOKENS
        # gate and up read the same activations: stored row-concatenated (as in the decode
        # step), they are dequantized by one call into one [2048][22016] scratch and multiplied
        # as one GEMM.
        self.prefill_w = []  # (name, qw, s, b, scratch view, (N, K), host (q, s, b))
        self.prefill_g = []  # (name, A, scratch, C, (M, N, K), host A, [(part, column offset)])
        mats = {name: (j, n, k) for j, (name, n, k) in enumerate(synth.PREFILL_MATS)}
        a_host = {}
        for names in (["gate", "up"], ["down"]):
            k = mats[names[0]][2]
            ntot = sum(mats[nm][1] for nm in names)
            if k not in a_host:
                a_host[k] = synth.activations(self.M, k, seed=0, workload=synth.W_PREFILL, layer=100 + k)
                self.sha[f"prefill_A_{self.M}x{k}"] = sha256_of(a_host[k])
            wt = torch.empty((k, ntot), dtype=torch.float16, device=dev)
            qs, ss, bs = [], [], []
            for nm in names:
                j, n, _ = mats[nm]
                q, s, b = synth.w4_weights(n, k, seed=0, workload=synth.W_PREFILL, layer=j)
                self.sha[f"prefill_{nm}_q"], self.sha[f"prefill_{nm}_s"], self.sha[f"prefill_{nm}_b"] = (
                    sha256_of(q), sha256_of(s), sha256_of(b))
                qs.append(q), ss.append(s), bs.append(b)
            q, s, b = np.concatenate(qs), np.concatenate(ss), np.concatenate(bs)
            qw = w4.w4_pack(torch.from_numpy(q).to(dev))
            nm = "|".join(names)
            self.prefill_w.append((nm, qw, torch.from_numpy(s).to(dev), torch.from_numpy(b).to(dev), wt,
                                   (ntot, k), (q, s, b)))
            parts = [(nm, 0)]
            c = torch.empty((self.M, ntot), dtype=torch.float32, device=dev)
            self.prefill_g.append(("|".join(names), torch.from_numpy(a_host[k]).to(dev), wt, c, (self.M, ntot, k),
                                   a_host[k], parts))
        assert [w[0] for w in self.prefill_w] == [g[0] for g in self.prefill_g]  # weight i feeds GEMM i
        self.prefill_flops = sum(2 * m * n * k for _, _, _, _, (m, n, k), _, _ in self.prefill_g)
        ws = max(w4.gemm_workspace_bytes(a, wt) for _, a, wt, _, _, _, _ in self.prefill_g)
        self.gemm_ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        log(f"prefill weights ready in {time.time() - t0:.1f}s ({self.prefill_flops / 1e9:.2f} GFLOP per step)")

    # -- the three phases of a step (no allocation: every output is preallocated)
    def run_gemvs(self):
        gemv = self.w4.w4_gemv
        for mats in self.layers:
            for _, qw, s, b, x, y, _ in mats:
                gemv(qw, s, b, x, out=y)

    def run_head(self):
        self.w4.gemm_f16(self.x_head, self.head, out=self.logits)
        self.w4.logits_argmax_topk(self.logits, TOPK, idx=self.idx, val=self.val, workspace=self.topk_ws)

    def run_prefill(self):
        # each weight is dequantized once; the next weight's dequant rides in the launch of the
        # current GEMM (gemm_f16_dequant_next: in the CUs its last round of tiles leaves idle)
        _, qw, s, b, view, _, _ = self.prefill_w[0]
        self.w4.w4_dequant_f16_t(qw, s, b, out=view)
        for i, (_, a, wt, c, _, _, _) in enumerate(self.prefill_g):
            if i + 1 < len(self.prefill_w):
                _, qw, s, b, view, _, _ = self.prefill_w[i + 1]
                self.w4.gemm_f16_dequant_next(a, wt, qw, s, b, out=c, wt=view, workspace=self.gemm_ws)
            else:
                self.w4.gemm_f16(a, wt, out=c, workspace=self.gemm_ws)

    def run_prefill_sequential(self):
        # the same work as four launches: dequant, GEMM, dequant, GEMM
        for (_, qw, s, b, view, _, _), (_, a, wt, c, _, _, _) in zip(self.prefill_w, self.prefill_g):
            self.w4.w4_dequant_f16_t(qw, s, b, out=view)
            self.w4.gemm_f16(a, wt, out=c, workspace=self.gemm_ws)


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def median_ci(np, samples, reps=2000, seed=0):
    """Median of per-round samples and its 95 % bootstrap interval (reps resamples with
    replacement, percentile method, fixed seed)."""
    a = np.asarray(samples, dtype=np.float64)
    rng = np.random.default_rng(seed)
    med = np.median(rng.choice(a, size=(reps, a.size), replace=True), axis=1)
    lo, hi = np.percentile(med, [2.5, 97.5])
    return {"median": round(float(np.median(a)), 3), "ci95": [round(float(lo), 3), round(float(hi), 3)],
            "rounds": int(a.size)}


def context(torch):
    """Context for the figures (not denominators): a plain device copy's bandwidth and the
    clocks rocm-smi reports once the timed loops are done."""
    n = 1 << 29  # 1 GiB of f16
    src = torch.empty(n, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(5):
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    ctx = {"copy_1gib_read_plus_write_gbps": round(2 * 2 * n / best / 1e6, 1)}
    try:
        import subprocess
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        if r.returncode == 0:
            d = json.loads(r.stdout[r.stdout.index("{"):])
            card = d.get("card0") or next(iter(d.values()))
            ctx["clocks_after_timing"] = {k: v for k, v in card.items() if "clk" in k.lower()}
    except Exception as e:  # context only: a missing or failing tool leaves it out
        ctx["clocks_after_timing"] = f"unavailable ({type(e).__name__})"
    return ctx


def kernel_groups(wl):
    """The step's launches grouped by kernel shape: key -> algorithmic bytes and flops of one
    launch, and one closure per launch (e.g. the 36 layers' gate|up GEMVs, each on its own
    weights)."""
    groups = {}

    def add(key, nbytes, flops, fn):
        g = groups.setdefault(key, {"bytes": nbytes, "flops": flops, "fns": []})
        g["fns"].append(fn)

    for mats in wl.layers:
        for name, qw, s, b, x, y, (m, n, k) in mats:
            add(("w4_gemv", m, n, k), gemv_bytes(m, n, k), 0,
                lambda qw=qw, s=s, b=b, x=x, y=y: wl.w4.w4_gemv(qw, s, b, x, out=y))
    # the dequant shapes rotate through distinct copies of their inputs and outputs, together at
    # least ROTATE_BYTES per shape, so no launch finds its operands in the last-level cache
    torch = wl.torch
    per_shape = {}
    for w in wl.prefill_w:
        per_shape.setdefault(w[5], []).append(w)
    for (n, k), ws_ in per_shape.items():
        nb = n * k // 2 + n * k // 16 + 2 * n * k
        copies = -(-ROTATE_BYTES // nb)
        for c in range(copies):
            _, qw, s, b, _, _, _ = ws_[c % len(ws_)]
            if c >= len(ws_):
                qw, s, b = qw.clone(), s.clone(), b.clone()
            view = torch.empty((k, n), dtype=torch.float16, device="cuda")
            add(("w4_dequant_f16_t", 0, n, k), nb, 0,
                lambda qw=qw, s=s, b=b, view=view: wl.w4.w4_dequant_f16_t(qw, s, b, out=view))
    for name, a, wt, c, (m, n, k), _, _ in wl.prefill_g:
        add(("gemm_f16", m, n, k), 2 * (m * k + k * n) + 4 * m * n, 2 * m * n * k,
            lambda a=a, wt=wt, c=c: wl.w4.gemm_f16(a, wt, out=c, workspace=wl.gemm_ws))
    for i, (name, a, wt, c, (m, n, k), _, _) in enumerate(wl.prefill_g[:-1]):
        _, qw, s, b, view, (nq, kq), _ = wl.prefill_w[i + 1]
        add(("gemm_f16_dequant_next", m, n, k), 2 * (m * k + k * n) + 4 * m * n + nq * kq // 2 + nq * kq // 16 + 2 * nq * kq,
            2 * m * n * k, lambda a=a, wt=wt, c=c, qw=qw, s=s, b=b, view=view:
            wl.w4.gemm_f16_dequant_next(a, wt, qw, s, b, out=c, wt=view, workspace=wl.gemm_ws))
    add(("gemm_f16", 1, wl.V, wl.H), 2 * wl.H * wl.V + 2 * wl.H + 4 * wl.V, 2 * wl.H * wl.V,
        lambda: wl.w4.gemm_f16(wl.x_head, wl.head, out=wl.logits))
    add(("logits_argmax_topk", 1, wl.V, TOPK), 4 * wl.V, 0,
        lambda: wl.w4.logits_argmax_topk(wl.logits, TOPK, idx=wl.idx, val=wl.val, workspace=wl.topk_ws))
    return groups


def kernel_timings(torch, wl, reps=5, min_launches=36):
    """Per-launch device time of each kernel shape of the step.  The launches of one shape
    (repeated up to at least min_launches, so a shape with one launch per step is not timed
    as a one-node graph whose replay overhead would dominate) are captured in a HIP graph of
    their own and replayed between two events; time / launches is the average launch
    duration including the in-graph dispatch gap (a conservative figure)."""
    groups = kernel_groups(wl)
    stream = torch.cuda.current_stream()
    # an int16 fill before each shape's timed replays and a uint8 fill after them (kernels
    # nothing else here launches): in a kernel trace of this run the dispatches between the two
    # are exactly one shape's timed launches (see --trace-from)
    marker = torch.empty(4097, dtype=torch.int16, device="cuda")
    end_marker = torch.empty(4097, dtype=torch.uint8, device="cuda")
    out = {}
    for key, g in groups.items():
        fns = g["fns"] * ((min_launches + len(g["fns"]) - 1) // len(g["fns"]))
        graph = capture(torch, lambda fns=fns: [f() for f in fns])
        graph.replay()
        marker.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        end_marker.fill_(1)
        torch.cuda.synchronize()
        avg = e0.elapsed_time(e1) * 1e3 / (reps * len(fns))
        out[key] = {"launches": reps * len(fns), "avg_us": avg, "bytes": g["bytes"], "flops": g["flops"],
                    "gbps": g["bytes"] / avg / 1e3, "tflops": g["flops"] / avg / 1e6 if g["flops"] else 0.0}
    return out


def _short_name(kernel_name):
    return (kernel_name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            .replace("w4::", ""))


def _bench_line(path):
    with open(path) as f:
        return json.loads([l for l in f if l.lstrip().startswith("{")][-1])


def trace_from(bench_json, trace_csv, unprofiled_json=None, out_path=None):
    """profiles/kernel_trace.json from a rocprofv3 --kernel-trace run of bench.py: per kernel shape
    of the per-shape timing section (the dispatches between the start and end markers, in the
    order of the run's own `kernels` field), rocprof's kernel durations (End - Start) beside the
    HIP-event time per launch of the same command run without the profiler (unprofiled_json;
    the profiled run's own event times include the profiler's wait between dispatches)."""
    import csv
    import statistics
    ker = _bench_line(bench_json)["kernels"]
    live = _bench_line(unprofiled_json)["kernels"] if unprofiled_json else ker
    rows = sorted(csv.DictReader(open(trace_csv, newline="")), key=lambda r: int(r["Dispatch_Id"]))
    # a segment opens at an int16 fill and closes at the next uint8 fill (or, in traces taken
    # without end markers, at the next int16 fill: its timed launches are then its first ones)
    segs, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        if "FillFunctor<short>" in name or "FillFunctor<unsigned char>" in name:
            if cur is not None:
                segs.append(cur)
            cur = [] if "FillFunctor<short>" in name else None
        elif cur is not None:
            cur.append(r)
    if len(segs) != len(ker):
        raise SystemExit(f"{len(segs)} marker segments, but the run timed {len(ker)} kernel shapes")
    out = {"method": "rocprofv3 --kernel-trace --stats of bench.py; per kernel shape, the dispatches of bench.py's "
                     "per-shape timing section (between int16-fill markers); duration = End - Start per dispatch",
           "kernels": {}}
    print("| kernel shape | dispatches | kernels (grid) | rocprof mean us | median us | min us | bench us per launch | mean / bench |")
    print("|---|---|---|---|---|---|---|---|")
    for (key, k), seg in zip(ker.items(), segs):
        # one shape's launch may be several kernels (the split-K GEMM and its reduce): the launch
        # repeats once the first dispatch's kernel and grid come round again
        sig = [(r["Kernel_Name"], r["Grid_Size_X"]) for r in seg]
        per = next((i for i in range(1, len(sig)) if sig[i] == sig[0]), len(sig))
        if len(seg) < per * k["launches"]:
            raise SystemExit(f"{key}: {len(seg)} dispatches for {k['launches']} launches of {per} kernels")
        seg = seg[:per * k["launches"]]
        durs = [sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in seg[i * per:(i + 1) * per]) / 1e3
                for i in range(k["launches"])]
        names = sorted({_short_name(r["Kernel_Name"]) + f"[{int(r['Grid_Size_X']) // int(r['Workgroup_Size_X'])}]"
                        for r in seg})
        src = SOURCE_OF[key.split("/")[0]]
        ent = {"source_sha": source_hash(src), "dispatches": len(seg), "kernels_per_launch": per,
               "kernels": names, "mean_us": statistics.mean(durs), "median_us": statistics.median(durs),
               "min_us": min(durs), "bench_avg_launch_us": live[key]["avg_us"],
               "mean_over_bench": statistics.mean(durs) / live[key]["avg_us"]}
        out["kernels"][key] = ent
        print(f"| {key} | {len(seg)} | {', '.join(names)} | {ent['mean_us']:.2f} | {ent['median_us']:.2f} | "
              f"{ent['min_us']:.2f} | {live[key]['avg_us']:.2f} | {ent['mean_over_bench']:.3f} |")
    path = out_path or os.path.join(ROOT, "profiles", "kernel_trace.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")


def trace_for(key):
    """rocprof's per-dispatch duration of a kernel shape from the committed trace summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "kernel_trace.json")) as f:
            ent = json.load(f)["kernels"][key]
        if ent.get("source_sha") != source_hash(SOURCE_OF[key.split("/")[0]]):
            return None
        return ent
    except Exception:
        return None


SOURCE_OF = {"w4_gemv": "gemv.hip", "w4_dequant_f16_t": "dequant.hip", "gemm_f16": "gemm.hip",
             "gemm_f16_dequant_next": "gemm.hip", "logits_argmax_topk": "topk.hip"}
COUNTER_REPS = 3
COPY_ELEMS = 128 << 20  # f16 elements of the validation copy (256 MiB read, 256 MiB written)


def small_m_groups(torch, np, w4, synth):
    """The batched GEMV shapes of the side sections (affine format: Qwen3-1.7B classify at
    M = 16, the Gemma-12B-shaped layer at M = 8 and 1) as counter-plan groups: key -> bytes
    and COUNTER_REPS launches, each on its own copy of the weights."""
    groups = {}
    for cfg, (label, m, layer_name, wname, grps, copies, fmt) in enumerate(SMALL_M):
        if fmt != "affine64":
            continue
        m = getattr(synth, m) if isinstance(m, str) else m
        wk = getattr(synth, wname)
        shapes = {name: (j, n, k) for j, (name, n, k) in enumerate(getattr(synth, layer_name))}
        for grp in grps:
            parts = [synth.w4_weights(shapes[g][1], shapes[g][2], seed=0, workload=wk,
                                      layer=100 * cfg + shapes[g][0]) for g in grp]
            q, sc, b = (np.concatenate([p_[i] for p_ in parts]) for i in range(3))
            n, k = q.shape
            x = torch.from_numpy(synth.activations(m, k, seed=0, workload=wk,
                                                   layer=100 * cfg + 50 + shapes[grp[0]][0])).cuda()
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(16, w4.gemv_workspace_bytes(m, n, k)), dtype=torch.uint8, device="cuda")
            qw0, s0, b0 = w4.w4_pack(torch.from_numpy(q).cuda()), torch.from_numpy(sc).cuda(), torch.from_numpy(b).cuda()
            mats = [(qw0, s0, b0)] + [(qw0.clone(), s0.clone(), b0.clone()) for _ in range(COUNTER_REPS - 1)]
            groups[("w4_gemv", m, n, k)] = {"bytes": gemv_bytes(m, n, k), "flops": 0,
                                            "fns": [lambda t=t, x=x, y=y, ws=ws: w4.w4_gemv(t[0], t[1], t[2], x, out=y,
                                                                                             workspace=ws)
                                                    for t in mats]}
    return groups


# Kernels of known bytes that validate the byte counts: a plain copy (whole 128-byte lines) and
# copies that read 64 or 32 bytes of every 128 (rows of 32 or 16 f16 out of 64).  Each reads
# exactly the bytes it touches if the L2 fetches at request granularity.
VALIDATION = (("copy", 64), ("copy_64B_of_each_128B", 32), ("copy_32B_of_each_128B", 16))


def counters_pass(torch, wl, manifest_path):
    """Launch plan for the counter runs: a marker kernel (an int16 fill, a kernel nothing
    else here launches), then each validation copy COUNTER_REPS times, then for each kernel
    shape COUNTER_REPS launches on different weights, each group followed by a marker.
    The plan and the algorithmic bytes of each group go to manifest_path."""
    # every buffer (and the packing launches that build them) before the first marker
    groups = dict(kernel_groups(wl))
    groups.update(small_m_groups(torch, wl.np, wl.w4, wl.synth))
    marker = torch.empty(4097, dtype=torch.int16, device="cuda")
    src = torch.ones(COPY_ELEMS, dtype=torch.float16, device="cuda")
    views = []
    for key, cols in VALIDATION:
        sv = src.view(-1, 64)[:, :cols]
        views.append((key, sv, torch.empty(sv.shape, dtype=torch.float16, device="cuda")))
    plan = [{"key": key, "kind": "validation", "read_bytes": 2 * sv.numel(), "write_bytes": 2 * sv.numel(),
             "source": None} for key, sv, _ in views]
    torch.cuda.synchronize()
    marker.fill_(1)
    for _, sv, dv in views:
        for _ in range(COUNTER_REPS):
            torch.neg(sv, out=dv)
        marker.fill_(1)
    for key, g in groups.items():
        fns = g["fns"]
        for r in range(COUNTER_REPS):
            fns[r % len(fns)]()
        marker.fill_(1)
        plan.append({"key": "_".join(map(str, key)), "bytes": g["bytes"], "flops": g["flops"],
                     "source": SOURCE_OF[key[0]], "source_sha": source_hash(SOURCE_OF[key[0]])})
    torch.cuda.synchronize()
    with open(manifest_path, "w") as f:
        json.dump({"reps": COUNTER_REPS, "groups": plan}, f, indent=1)
    log(f"counter pass: {len(plan)} groups of {COUNTER_REPS} launches; plan in {manifest_path}")


def _counter_dispatches(csv_path, counters):
    """Per marker-delimited segment (after the first marker): each dispatch's kernel name and
    the values of the named counters (summed over the rows rocprofv3 writes per dispatch)."""
    import csv
    disp = {}
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "v": {}})
            if r["Counter_Name"] in counters:
                d["v"][r["Counter_Name"]] = d["v"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    segs, cur, started = [], None, False
    for i in sorted(disp):
        d = disp[i]
        if "FillFunctor<short>" in d["name"]:
            if started:
                segs.append(cur)
            started, cur = True, []
        elif started:
            cur.append((d["name"].replace("(anonymous namespace)::", "").split("(")[0][:80], d["v"]))
    return segs


def _segment_sums(csv_path, counters):
    """Per segment: the sum over its dispatches of each counter, and the kernel names."""
    out = []
    for seg in _counter_dispatches(csv_path, counters):
        tot = {c: sum(v.get(c, 0.0) for _, v in seg) for c in counters}
        out.append({"v": tot, "names": [n for n, _ in seg]})
    return out


UTIL_COUNTERS = ("VALUBusy", "MfmaUtil")


def util_from(manifest_path, csv_path, out_path=None):
    """profiles/utilization.json from one `rocprofv3 --pmc VALUBusy MfmaUtil` run of the
    --counters pass: per kernel shape and dispatched kernel, the mean of each metric (percent
    of the kernel's busy time) over its launches."""
    with open(manifest_path) as f:
        man = json.load(f)
    groups = man["groups"]
    segs = _counter_dispatches(csv_path, UTIL_COUNTERS)
    if len(segs) != len(groups):
        raise SystemExit(f"segments {len(segs)} do not match the plan's {len(groups)} groups")
    out = {"method": "rocprofv3 --pmc VALUBusy MfmaUtil over bench.py --counters; per dispatch, averaged "
                     "over the launches of each kernel in a shape's group", "kernels": {}}
    print("| kernel shape | dispatched kernel | launches | VALUBusy % | MfmaUtil % |")
    print("|---|---|---|---|---|")
    for g, seg in zip(groups, segs):
        if g.get("kind") == "validation":
            continue
        per = {}
        for name, v in seg:
            per.setdefault(name, []).append(v)
        out["kernels"][g["key"]] = {"source_sha": g["source_sha"], "by_kernel": {}}
        for name, vs in per.items():
            row = {c: sum(v.get(c, 0.0) for v in vs) / len(vs) for c in UTIL_COUNTERS}
            row["launches"] = len(vs)
            out["kernels"][g["key"]]["by_kernel"][name] = row
            print(f"| {g['key']} | {name} | {len(vs)} | {row['VALUBusy']:.1f} | {row['MfmaUtil']:.1f} |")
    path = out_path or os.path.join(ROOT, "profiles", "utilization.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")


# HBM traffic from the L2's requests to the memory side, by request size.  FETCH_SIZE, the
# derived counter, takes every read that is not 32 bytes as 64 unless TCC_BUBBLE fires, so it
# undercounts 128-byte reads by half; here every size has its own counter.
READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum")


def read_bytes_of(v):
    return 32 * v["TCC_EA0_RDREQ_32B_sum"] + 64 * v["TCC_EA0_RDREQ_64B_sum"] + 128 * v["TCC_EA0_RDREQ_128B_sum"]


def write_bytes_of(v):
    # write requests are 32 or 64 bytes
    return 32 * (v["TCC_EA0_WRREQ_sum"] - v["TCC_EA0_WRREQ_64B_sum"]) + 64 * v["TCC_EA0_WRREQ_64B_sum"]


def traffic_from(manifest_path, read_csv, write_csv, out_path=None):
    """profiles/traffic.json from two counter runs of the --counters pass: the read requests by
    size (READ_COUNTERS), then the write requests (WRITE_COUNTERS).  Bytes per launch are the
    requests times their sizes, with no calibration factor; the validation copies show how
    close that comes to the bytes they touch."""
    with open(manifest_path) as f:
        man = json.load(f)
    reps = man["reps"]
    rs, ws = _segment_sums(read_csv, READ_COUNTERS), _segment_sums(write_csv, WRITE_COUNTERS)
    groups = man["groups"]
    if len(rs) != len(groups) or len(ws) != len(groups):
        raise SystemExit(f"segments {len(rs)}/{len(ws)} do not match the plan's {len(groups)} groups")
    out = {"method": "rocprofv3 --pmc " + " ".join(READ_COUNTERS) + ", then --pmc " + " ".join(WRITE_COUNTERS)
                     + ", over bench.py --counters; read bytes = 32*RDREQ_32B + 64*RDREQ_64B + 128*RDREQ_128B, "
                     "write bytes = 32*(WRREQ - WRREQ_64B) + 64*WRREQ_64B, summed over each call's dispatches and "
                     "averaged over the calls",
           "validation": {}, "kernels": {}}
    rows, vrows = [], []
    for g, rseg, wseg in zip(groups, rs, ws):
        rv = {c: x / reps for c, x in rseg["v"].items()}
        wv = {c: x / reps for c, x in wseg["v"].items()}
        rd, wr = read_bytes_of(rv), write_bytes_of(wv)
        sizes_sum = rv["TCC_EA0_RDREQ_32B_sum"] + rv["TCC_EA0_RDREQ_64B_sum"] + rv["TCC_EA0_RDREQ_128B_sum"]
        ent = {"read_requests": rv, "write_requests": wv, "read_bytes": rd, "write_bytes": wr,
               "read_requests_by_size_over_all": sizes_sum / rv["TCC_EA0_RDREQ_sum"] if rv["TCC_EA0_RDREQ_sum"] else None}
        if g.get("kind") == "validation":
            ent.update(touched_read_bytes=g["read_bytes"], touched_write_bytes=g["write_bytes"],
                       read_over_touched=rd / g["read_bytes"], write_over_touched=wr / g["write_bytes"])
            out["validation"][g["key"]] = ent
            vrows.append((g["key"], g["read_bytes"], rd, g["write_bytes"], wr))
            continue
        ent.update(source_sha=g["source_sha"], dispatches=sorted(set(rseg["names"])), hbm_read_bytes=rd,
                   hbm_write_bytes=wr, hbm_bytes_per_launch=rd + wr, algorithmic_bytes=g["bytes"],
                   traffic_over_algorithmic=(rd + wr) / g["bytes"])
        out["kernels"][g["key"]] = ent
        rows.append((g["key"], g["bytes"], rd, wr, (rd + wr) / g["bytes"]))
    # the prefill GEMMs together, per launch
    pre = [k for k in out["kernels"] if k.startswith("gemm_f16_1570_")]
    if pre:
        ks = [out["kernels"][k] for k in pre]
        out["kernels"]["gemm_f16_prefill"] = {
            "source_sha": ks[0]["source_sha"], "of": pre,
            "hbm_bytes_per_launch": sum(k["hbm_bytes_per_launch"] for k in ks) / len(ks),
            "algorithmic_bytes": sum(k["algorithmic_bytes"] for k in ks) / len(ks)}
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("| validation kernel | bytes read (touched) | counted read | bytes written | counted write |")
    print("|---|---|---|---|---|")
    for key, tr, rd, tw, wr in vrows:
        print(f"| {key} | {tr} | {rd:.0f} ({rd / tr:.3f}x) | {tw} | {wr:.0f} ({wr / tw:.3f}x) |")
    print()
    print("| kernel shape | algorithmic B | HBM read B | HBM write B | traffic / algorithmic |")
    print("|---|---|---|---|---|")
    for key, b, rd, wr, ratio in rows:
        print(f"| {key} | {b} | {rd:.0f} | {wr:.0f} | {ratio:.3f} |")
    print(f"wrote {path}")


def source_hash(*names):
    """16 hex digits of the SHA-256 over kernel sources and the local headers they include
    (transitively, each once, in first-include order)."""
    csrc = os.path.join(ROOT, "int4_weight_only_group_amd", "csrc")
    h = hashlib.sha256()
    todo, seen = list(names), set()
    while todo:
        n = todo.pop(0)
        if n in seen:
            continue
        seen.add(n)
        with open(os.path.join(csrc, n), "rb") as f:
            data = f.read()
        h.update(data)
        todo += [m.decode() for m in re.findall(rb'#include "([^"/]+)"', data)]
    return h.hexdigest()[:16]


def traffic_for(kernel_src, key):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
        ent = t["kernels"][key]
        if ent.get("source_sha") != source_hash(kernel_src):
            return None
        return ent["hbm_bytes_per_launch"]
    except Exception:
        return None


def parity_check(torch, np, wl, oracle, synth):
    """Re-check the outputs of the last timed step against the oracle on sampled rows."""
    rng = np.random.default_rng(123)
    res = {}
    worst = 0.0
    # decode GEMVs of the last layer, 64 sampled output rows per GEMV
    l = synth.QWEN25_3B_LAYERS - 1
    shapes = {name: (j, n, k) for j, (name, n, k) in enumerate(synth.QWEN25_3B_LAYER)}
    for names, _, _, _, x, y, (_, n, k) in wl.layers[l]:
        parts = [synth.w4_weights(shapes[nm][1], k, seed=0, workload=synth.W_DECODE, layer=l * 16 + shapes[nm][0])
                 for nm in names.split("+")]
        q, s, b = (np.concatenate([p[i] for p in parts]) for i in range(3))
        rows = np.sort(rng.choice(n, min(n, 64), replace=False))
        y_ref, bound = oracle.gemv_ref(oracle.pack(q[rows]), s[rows], b[rows], x.cpu().numpy())
        ok, wr = oracle.check_bound(y.cpu().numpy()[:, rows], y_ref, bound)
        worst = max(worst, wr)
        if not ok:
            res["gemv_fail"] = names
    res["gemv_worst_err_over_bound"] = worst
    # f16 head on every column; top-40 against the fp64 logits (near-tie rule)
    lg = wl.logits.cpu().numpy()
    c_ref, bound = oracle.gemm_ref(wl.x_head_host, wl.head_host)
    ok_h, wr_h = oracle.check_bound(lg, c_ref, bound)
    res["head_worst_err_over_bound"] = wr_h
    idx = wl.idx.cpu().numpy()
    ok_t, loose = oracle.check_topk_vs_exact(c_ref, idx, TOPK)
    ok_t &= bool(np.array_equal(wl.val.cpu().numpy().view(np.uint32), lg[0, idx[0]][None].view(np.uint32)))
    res["topk_ok"] = ok_t
    res["topk_ranks_in_near_tie"] = loose
    del c_ref, bound
    # prefill: dequant scratch bit-exact on sampled columns; GEMM on sampled rows incl. the M tail
    worst_p = 0.0
    ok_p = True
    wt_ref = {}
    for name, qw, s, b, view, (n, k), (qh, sh, bh) in wl.prefill_w:
        wt_ref[name] = oracle.dequant_f16_t(oracle.pack(qh), sh, bh)
        cols = np.sort(rng.choice(n, 64, replace=False))
        ok_p &= bool(np.array_equal(view.cpu().numpy().view(np.uint16)[:, cols], wt_ref[name][:, cols]))
    for name, a, wt, c, (m, n, k), ah, parts in wl.prefill_g:
        full = np.concatenate([wt_ref[nm] for nm, _ in parts], axis=1)
        rows = np.unique(np.concatenate([rng.choice(m - 34, 30, replace=False), np.arange(m - 34, m)]))
        c_ref, bound = oracle.gemm_ref(ah[rows], full.view(np.float16))
        okc, wr = oracle.check_bound(c.cpu().numpy()[rows], c_ref, bound)
        ok_p &= okc
        worst_p = max(worst_p, wr)
    res["prefill_worst_err_over_bound"] = worst_p
    res["ok"] = bool("gemv_fail" not in res and ok_h and ok_t and ok_p)
    return res


# Batched-decode GEMVs at several activation rows: the batched classify decode (M = 16,
# Qwen3-1.7B shapes) and the Gemma-12B-shaped layer at M = 8 and M = 1.  Matrices that read
# the same activations run row-concatenated, as in the decode step.  Each shape is timed
# over `copies` distinct copies of its weights (together larger than the 256 MB MALL).
SMALL_M = (("qwen3-1.7b classify", "CLASSIFY_ROWS", "QWEN3_1P7B_CLASSIFY", "W_CLASSIFY",
            [["q", "k", "v"], ["gate", "up"], ["down"]], 40, "affine64"),
           ("gemma-12b layer", 8, "GEMMA12B_LAYER", "W_GEMMA", [["gate", "up"], ["down"], ["q"]], 10, "affine64"),
           ("gemma-12b layer", 1, "GEMMA12B_LAYER", "W_GEMMA", [["gate", "up"], ["down"], ["q"]], 10, "affine64"),
           # the engine's own format on the decode step's shapes (a per-layer figure: q|k|v, o,
           # gate|up, down once each, 36 copies apiece)
           ("qwen2.5-3b decode layer, symmetric group-128", 1, "QWEN25_3B_LAYER", "W_DECODE",
            [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]], 36, "sym128"))


def small_m(torch, np, w4, synth, oracle, reps=5):
    """Per-shape device time (graph of `copies` back-to-back launches on distinct weights),
    GB/s against HBM peak, and a parity re-check of the last launch on 64 sampled rows."""
    rng = np.random.default_rng(321)
    out = []
    for cfg, (label, m, layer_name, wname, groups, copies, fmt) in enumerate(SMALL_M):
        sym = fmt == "sym128"
        m = getattr(synth, m) if isinstance(m, str) else m
        wk = getattr(synth, wname)
        shapes = {name: (j, n, k) for j, (name, n, k) in enumerate(getattr(synth, layer_name))}
        rows_out = []
        tot_b = tot_us = 0.0
        worst = 0.0
        ok = True
        for grp in groups:
            if sym:
                parts = [synth.w4_sym128_weights(shapes[g][1], shapes[g][2], seed=0, workload=wk,
                                                 layer=100 * cfg + shapes[g][0]) for g in grp]
                q, s = (np.concatenate([p[i] for p in parts]) for i in range(2))
                b = None
            else:
                parts = [synth.w4_weights(shapes[g][1], shapes[g][2], seed=0, workload=wk,
                                          layer=100 * cfg + shapes[g][0]) for g in grp]
                q, s, b = (np.concatenate([p[i] for p in parts]) for i in range(3))
            n, k = q.shape
            x_host = synth.activations(m, k, seed=0, workload=wk, layer=100 * cfg + 50 + shapes[grp[0]][0])
            qw0 = w4.w4_pack(torch.from_numpy(q).cuda())
            s0 = torch.from_numpy(s).cuda()
            b0 = None if sym else torch.from_numpy(b).cuda()
            mats = [(qw0, s0, b0)] + [(qw0.clone(), s0.clone(), None if sym else b0.clone()) for _ in range(copies - 1)]
            x = torch.from_numpy(x_host).cuda()
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(16, w4.gemv_workspace_bytes(m, n, k)), dtype=torch.uint8, device="cuda")
            if sym:
                fns = [lambda t=t: w4.w4_gemv_sym128(t[0], t[1], x, out=y, workspace=ws) for t in mats]
            else:
                fns = [lambda t=t: w4.w4_gemv(t[0], t[1], t[2], x, out=y, workspace=ws) for t in mats]
            graph = capture(torch, lambda: [f() for f in fns])
            graph.replay()
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            nb = n * k // 2 + n * k // 64 + 2 * m * k + 4 * m * n if sym else gemv_bytes(m, n, k)
            sel = np.sort(rng.choice(n, min(n, 64), replace=False))
            if sym:
                y_ref, bound = oracle.gemv_ref(oracle.pack(q[sel]), s[sel], None, x_host, group=128)
            else:
                y_ref, bound = oracle.gemv_ref(oracle.pack(q[sel]), s[sel], b[sel], x_host)
            okc, wr = oracle.check_bound(y.cpu().numpy()[:, sel], y_ref, bound)
            ok &= okc
            worst = max(worst, wr)
            rows_out.append({"matrix": "|".join(grp), "M": m, "N": n, "K": k, "avg_us": round(us, 3),
                             "gbps": round(nb / us / 1e3, 1), "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)})
            tot_b += nb
            tot_us += us
            del mats, fns, graph
        out.append({"workload": f"{label} at M={m}", "format": fmt, "gemvs": rows_out, "gbps": round(tot_b / tot_us / 1e3, 1),
                    "frac_hbm": round(tot_b / tot_us / 1e3 / HBM_PEAK_GBS, 4), "parity_ok": bool(ok),
                    "worst_err_over_bound": worst, "copies": copies})
    return out


def int4_head(torch, np, w4, synth, oracle, wl, reps=10):
    """The LM head stored in the int4 format (group-64 affine, [vocab][hidden] = 151936 x 2048,
    the pages' 622 MB f16 head at 175 MB) at M = 1 with top-40: w4_gemv_topk (one call: the
    GEMV, the group maxima, the selection) and the same as two calls (w4_gemv to f32 logits, then
    logits_argmax_topk), each graph-timed over distinct copies of the head that together hold at
    least 1 GiB.  Parity: 64 sampled logits against the fp64 oracle, the selection bit-exact on
    the GPU's own logits, and the two ways' indices equal."""
    V, K = wl.V, wl.H
    q, s, b = synth.w4_weights(V, K, seed=0, workload=synth.W_DECODE, layer=990)
    qw = w4.w4_pack(torch.from_numpy(q).cuda())
    sd, bd = torch.from_numpy(s).cuda(), torch.from_numpy(b).cuda()
    nb = gemv_bytes(1, V, K) + 4 * V
    copies = -(-ROTATE_BYTES // nb)
    heads = [(qw, sd, bd)] + [(qw.clone(), sd.clone(), bd.clone()) for _ in range(copies - 1)]
    logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, TOPK), dtype=torch.int32, device="cuda")
    val = torch.empty((1, TOPK), dtype=torch.float32, device="cuda")
    flog = torch.empty(V, dtype=torch.float32, device="cuda")
    fidx = torch.empty(TOPK, dtype=torch.int32, device="cuda")
    fval = torch.empty(TOPK, dtype=torch.float32, device="cuda")
    fws = torch.empty(w4.gemv_topk_workspace_bytes(V, K, TOPK), dtype=torch.uint8, device="cuda")

    def two_calls():
        for h in heads:
            w4.w4_gemv(*h, wl.x_head, out=logits)
            w4.logits_argmax_topk(logits, TOPK, idx=idx, val=val, workspace=wl.topk_ws)

    def one_call():
        for h in heads:
            w4.w4_gemv_topk(*h, wl.x_head, TOPK, logits=flog, idx=fidx, val=fval, workspace=fws)

    stream = torch.cuda.current_stream()
    graphs = {name: capture(torch, fn) for name, fn in (("two_calls", two_calls), ("one_call", one_call))}
    times = {name: [] for name in graphs}
    for g in graphs.values():
        g.replay()
    for _ in range(5):  # the two ways alternate, so clock drift falls on both; medians
        for name, graph in graphs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) * 1e3 / (reps * copies))
    res = {name: float(np.median(t)) for name, t in times.items()}
    lg = logits.cpu().numpy()
    rows = np.sort(np.random.default_rng(11).choice(V, 64, replace=False))
    y_ref, bound = oracle.gemv_ref(oracle.pack(q[rows]), s[rows], b[rows], wl.x_head_host)
    ok = oracle.check_bound(lg[:, rows], y_ref, bound)[0]
    ok &= oracle.check_topk_selection(lg, idx.cpu().numpy(), val.cpu().numpy(), TOPK)
    fl = flog.cpu().numpy()[None]
    ok &= oracle.check_bound(fl[:, rows], y_ref, bound)[0]
    ok &= oracle.check_topk_selection(fl, fidx.cpu().numpy()[None], fval.cpu().numpy()[None], TOPK)
    ok &= bool(np.array_equal(fidx.cpu().numpy(), idx.cpu().numpy()[0]))
    us = res["one_call"]
    return {"workload": f"int4 LM head [{V}][{K}] (affine group 64) at M=1 + top-{TOPK}", "us": round(us, 3),
            "gbps": round(nb / us / 1e3, 1), "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "launch": "w4_gemv_topk (GEMV, group maxima, selection)", "two_calls_us": round(res["two_calls"], 3),
            "head_bytes": gemv_bytes(1, V, K), "copies": copies, "parity_ok": bool(ok)}


def single_gemv(torch, np, w4, synth, oracle, copies=512, reps=5):
    """The single W4A16 GEMV (M, N, K) = (1, 4864, 896), seed 0: (i) one launch between two
    events after a synchronize (latency of a lone call), (ii) steady state over `copies`
    distinct weight copies (1.27 GB, above the last-level cache) as one graph.  Parity: every
    output of the lone call against the oracle."""
    n, k = 4864, 896
    q, s, b = synth.w4_weights(n, k, seed=0, workload=synth.W_SINGLE)
    x_host = synth.activations(1, k, seed=0, workload=synth.W_SINGLE)
    qw0 = w4.w4_pack(torch.from_numpy(q).cuda())
    s0, b0 = torch.from_numpy(s).cuda(), torch.from_numpy(b).cuda()
    x = torch.from_numpy(x_host).cuda()
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        w4.w4_gemv(qw0, s0, b0, x, out=y)
    lat = []
    for _ in range(20):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        w4.w4_gemv(qw0, s0, b0, x, out=y)
        e1.record(stream)
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1) * 1e3)
    y_ref, bound = oracle.gemv_ref(oracle.pack(q), s, b, x_host)
    ok = oracle.check_bound(y.cpu().numpy(), y_ref, bound)[0]
    mats = [(qw0.clone(), s0.clone(), b0.clone()) for _ in range(copies)]
    graph = capture(torch, lambda: [w4.w4_gemv(t[0], t[1], t[2], x, out=y) for t in mats])
    graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    nb = gemv_bytes(1, n, k)
    del mats, graph
    return {"workload": f"single W4A16 GEMV (1, {n}, {k}), seed 0", "bytes": nb,
            "lone_launch_us_median": round(float(np.median(lat)), 3),
            "steady_state_us": round(us, 3), "steady_state_gbps": round(nb / us / 1e3, 1),
            "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "copies": copies, "parity_ok": bool(ok)}


def head_sections(torch, np, w4, synth, oracle, wl, reps=10):
    """The two other head steps of the workloads, each as one graph:
    * batched classify: the yes/no columns of the decode step's f16 head [2048][151936]
      (B = H + id, ldb = V) for 16 rows, then a per-row argmax over the 2 logits;
    * Gemma-12B-shaped head: f16 [3840][262144] (N(0, 0.02), drawn on the GPU from a seeded
      generator: 2 GB) at M = 1 and M = 8, then the top-64 per row.
    Parity: the classify logits against the fp64 oracle and its argmax wherever the margin
    exceeds 1e-2; for the Gemma head 64 sampled logit columns against the oracle and the top-64
    bit-exact against the host selection on the GPU's own logits."""
    out = {}
    stream = torch.cuda.current_stream()

    def timed(step):
        graph = capture(torch, step)
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    m = synth.CLASSIFY_ROWS
    ids = synth.class_ids(wl.V)
    x_host = synth.activations(m, wl.H, seed=0, workload=synth.W_CLASSIFY, layer=996)
    x = torch.from_numpy(x_host).cuda()
    lg2 = torch.empty((m, 2), dtype=torch.float32, device="cuda")
    idx = torch.empty((m, 1), dtype=torch.int32, device="cuda")
    val = torch.empty((m, 1), dtype=torch.float32, device="cuda")

    def classify():
        for j, i in enumerate(ids):
            w4.gemm_f16(x, wl.head[:, i:i + 1], out=lg2[:, j:j + 1])
        w4.logits_argmax_topk(lg2, 1, idx=idx, val=val)
    us = timed(classify)
    c_ref, bound = oracle.gemm_ref(x_host, wl.head_host[:, list(ids)])
    ok = oracle.check_bound(lg2.cpu().numpy(), c_ref, bound)[0] and oracle.check_topk_vs_exact(c_ref, idx.cpu().numpy(), 1)[0]
    out["classify"] = {"workload": f"batched classify: {m} rows x 2 columns (ids {ids[0]}, {ids[1]}) of the f16 head "
                                   f"[{wl.H}][{wl.V}] + per-row argmax over 2", "us": round(us, 3), "parity_ok": bool(ok)}

    kd, vg, topk = synth.GEMMA12B_HIDDEN, synth.GEMMA12B_VOCAB, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    head = (torch.randn((kd, vg), generator=gen, device="cuda") * 0.02).half()
    cols = np.sort(np.random.default_rng(13).choice(vg, 64, replace=False))
    head_cols = head[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    ws = torch.empty(max(16, w4.topk_workspace_bytes(8, vg, topk)), dtype=torch.uint8, device="cuda")
    for mm in (1, 8):
        xg_host = synth.activations(mm, kd, seed=0, workload=synth.W_GEMMA, layer=995 - mm)
        xg = torch.from_numpy(xg_host).cuda()
        lg = torch.empty((mm, vg), dtype=torch.float32, device="cuda")
        gws = torch.empty(max(16, w4.gemm_workspace_bytes(xg, head)), dtype=torch.uint8, device="cuda")
        gi = torch.empty((mm, topk), dtype=torch.int32, device="cuda")
        gv = torch.empty((mm, topk), dtype=torch.float32, device="cuda")

        def gemma(xg=xg, lg=lg, gws=gws, gi=gi, gv=gv):
            w4.gemm_f16(xg, head, out=lg, workspace=gws)
            w4.logits_argmax_topk(lg, topk, idx=gi, val=gv, workspace=ws)
        us = timed(gemma)
        lgh = lg.cpu().numpy()
        c_ref, bound = oracle.gemm_ref(xg_host, head_cols)
        ok = oracle.check_bound(lgh[:, cols], c_ref, bound)[0]
        ok &= oracle.check_topk_selection(lgh, gi.cpu().numpy(), gv.cpu().numpy(), topk)
        nb = 2 * kd * vg + 2 * mm * kd + 8 * mm * vg
        out[f"gemma_m{mm}"] = {"workload": f"Gemma-12B-shaped f16 head [{kd}][{vg}] at M={mm} + top-{topk}",
                               "us": round(us, 3), "gbps": round(nb / us / 1e3, 1),
                               "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "parity_ok": bool(ok)}
    del head
    return out


SPEC_ROWS = 8  # draft positions verified per step


def spec_verify(torch, np, w4, synth, oracle, wl, reps=20):
    """Speculative-verify greedy check: SPEC_ROWS draft positions through the decode step's
    f16 head (one gemm_f16 at M = 8, which streams the head once for all rows) and a per-row
    argmax (logits_argmax_topk with k = 1), as one graph.  Parity: every row's argmax against
    the fp64 logits wherever the top-2 margin exceeds 1e-2 (else within the near-tie class)."""
    m = SPEC_ROWS
    x_host = synth.activations(m, wl.H, seed=0, workload=synth.W_DECODE, layer=997)
    x = torch.from_numpy(x_host).cuda()
    logits = torch.empty((m, wl.V), dtype=torch.float32, device="cuda")
    idx = torch.empty((m, 1), dtype=torch.int32, device="cuda")
    val = torch.empty((m, 1), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, w4.topk_workspace_bytes(m, wl.V, 1)), dtype=torch.uint8, device="cuda")
    gws = torch.empty(max(16, w4.gemm_workspace_bytes(x, wl.head)), dtype=torch.uint8, device="cuda")

    def step():
        w4.gemm_f16(x, wl.head, out=logits, workspace=gws)
        w4.logits_argmax_topk(logits, 1, idx=idx, val=val, workspace=ws)
    graph = capture(torch, step)
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    c_ref, _ = oracle.gemm_ref(x_host, wl.head_host)
    ok, loose = oracle.check_topk_vs_exact(c_ref, idx.cpu().numpy(), 1)
    nb = 2 * wl.H * wl.V + 2 * m * wl.H + 8 * m * wl.V  # head + x + logits written and read
    return {"workload": f"speculative verify: {m} draft positions x f16 head [{wl.H}][{wl.V}] + per-row argmax",
            "us": round(us, 3), "gbps": round(nb / us / 1e3, 1), "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "parity_ok": bool(ok), "rows_in_near_tie": int(loose)}


def quantize_bench(torch, np, w4, synth, oracle, reps=5):
    """The load-time quantizer on the decode step's gate|up matrix ([22016][2048] f16
    weights, N(0, 0.02)): graph-timed over distinct input and output buffers that together
    hold at least 1 GiB, GB/s of 2NK bytes read + NK/2 + NK/16 written, and a bit-exact
    re-check of 64 sampled rows of the first and last copy against the oracle."""
    n = sum(nn for name, nn, _ in synth.QWEN25_3B_LAYER if name in ("gate", "up"))
    k = synth.QWEN25_3B_HIDDEN
    nb = 2 * n * k + n * k // 2 + n * k // 16
    copies = -(-ROTATE_BYTES // nb)
    w_host = synth.float_weights(n, k, seed=0, workload=synth.W_DECODE, layer=900)
    w0 = torch.from_numpy(w_host).cuda()
    ins = [w0] + [w0.clone() for _ in range(copies - 1)]
    outs = [(torch.empty((n, k // 8), dtype=torch.int32, device="cuda"),
             torch.empty((n, k // 64), dtype=torch.float16, device="cuda"),
             torch.empty((n, k // 64), dtype=torch.float16, device="cuda")) for _ in range(copies)]
    graph = capture(torch, lambda: [w4.w4_quantize(t, out=o) for t, o in zip(ins, outs)])
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    rows = np.sort(np.random.default_rng(9).choice(n, 64, replace=False))
    qw_ref, s_ref, b_ref = oracle.quantize(w_host[rows])
    ok = all(np.array_equal(out[0].cpu().numpy().view(np.uint32)[rows], qw_ref)
             and np.array_equal(out[1].cpu().numpy().view(np.uint16)[rows], s_ref.view(np.uint16))
             and np.array_equal(out[2].cpu().numpy().view(np.uint16)[rows], b_ref.view(np.uint16))
             for out in (outs[0], outs[-1]))
    return {"workload": f"w4_quantize of a [{n}][{k}] f16 matrix (gate|up), N(0, 0.02)", "avg_us": round(us, 3),
            "gbps": round(nb / us / 1e3, 1), "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": nb, "parity_ok": bool(ok), "copies": copies,
            "rotated_bytes": copies * nb}


def pack_bench(torch, np, w4, synth, oracle, reps=5):
    """The load-time packer on the decode step's gate|up codes ([22016][2048] uint8 codes):
    graph-timed over distinct input and output buffers that together hold at least 1 GiB,
    GB/s of NK bytes read + NK/2 written, and a bit-exact check of every word of the first
    and last copy against the oracle."""
    n = sum(nn for name, nn, _ in synth.QWEN25_3B_LAYER if name in ("gate", "up"))
    k = synth.QWEN25_3B_HIDDEN
    nb = n * k + n * k // 2
    copies = -(-ROTATE_BYTES // nb)
    q_host, _, _ = synth.w4_weights(n, k, seed=0, workload=synth.W_DECODE, layer=901)
    q0 = torch.from_numpy(q_host).cuda()
    ins = [q0] + [q0.clone() for _ in range(copies - 1)]
    outs = [torch.empty((n, k // 8), dtype=torch.int32, device="cuda") for _ in range(copies)]
    graph = capture(torch, lambda: [w4.w4_pack(t, out=o) for t, o in zip(ins, outs)])
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    ref = oracle.pack(q_host)
    ok = all(np.array_equal(out.cpu().numpy().view(np.uint32), ref) for out in (outs[0], outs[-1]))
    return {"workload": f"w4_pack of [{n}][{k}] uint8 codes (gate|up)", "avg_us": round(us, 3),
            "gbps": round(nb / us / 1e3, 1), "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": nb, "parity_ok": bool(ok), "copies": copies, "rotated_bytes": copies * nb}


def host_metadata(np):
    """The host the CPU figures were taken on: cores, CPU model, NumPy and its BLAS."""
    meta = {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "python": sys.version.split()[0]}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    meta["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        meta["cpu_model"] = "unknown"
    try:
        from threadpoolctl import threadpool_info
        meta["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer",
                                               "architecture")} for i in threadpool_info()]
    except Exception as e:  # metadata only
        meta["blas"] = f"unavailable ({type(e).__name__})"
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        meta[var] = os.environ.get(var)
    return meta


def _median_of(np, fn, reps=5):
    """Median wall time of reps calls after one warm-up call."""
    fn()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), [round(t, 4) for t in ts]


def cpu_baseline(np, oracle, synth):
    """The CPU oracle on this host, stage by stage, each the median of 5 timed calls after one
    warm-up:
      (a) unpack + exact dequant (NumPy elementwise, one thread) of the gate matrix;
      (b) the fp64 products through BLAS on all cores and on one thread: the decode GEMV of
          the gate matrix (with its error-bound product) and a 32-row slice of the prefill
          GEMM on the gate|up scratch;
      (c) top-40 selection over the 151936 logits;
    and, as `value`, the oracle's whole GEMV (unpack, dequant, fp64 product and bound) over
    the seven int4 matrices of one decoder layer at M = 1, on all cores, in GB/s of the
    layer's algorithmic bytes (the unit of the GPU figure)."""
    from threadpoolctl import threadpool_limits, threadpool_info
    meta = host_metadata(np)
    all_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t_start = time.perf_counter()
    stages = {}

    # (a) unpack + dequant of the 11008 x 2048 gate matrix (NumPy, no BLAS)
    n, k = 11008, 2048
    q, s, b = synth.w4_weights(n, k, seed=0, workload=synth.W_DECODE, layer=4)
    qw = oracle.pack(q)
    t, ts = _median_of(np, lambda: oracle.dequant_exact(qw, s, b))
    stages["a_unpack_dequant_1thread"] = {"shape_nk": [n, k], "median_s": t, "samples_s": ts, "threads": 1,
                                          "gweights_per_s": n * k / t / 1e9, "packed_gbps": (n * k // 2 + n * k // 16) / t / 1e9}

    # (b) fp64 products through BLAS, all cores and one thread
    w = oracle.dequant_exact(qw, s, b)
    x = synth.activations(1, k, seed=0, workload=synth.W_DECODE, layer=12).astype(np.float64)
    wabs = np.abs(w)
    a_rows = synth.activations(32, k, seed=0, workload=synth.W_PREFILL, layer=100 + k).astype(np.float64)
    wt = np.ascontiguousarray(w.T)
    for label, lim in (("all_cores", all_threads), ("1thread", 1)):
        with threadpool_limits(limits=lim, user_api="blas"):
            used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
            t, ts = _median_of(np, lambda: (x @ w.T, np.abs(x) @ wabs.T))
            stages[f"b_gemv_fp64_{label}"] = {"shape_mnk": [1, n, k], "median_s": t, "samples_s": ts, "threads": used,
                                              "gflops": 2 * 2 * n * k / t / 1e9}
            t, ts = _median_of(np, lambda: a_rows @ wt)
            stages[f"b_gemm_fp64_{label}"] = {"shape_mnk": [32, n, k], "median_s": t, "samples_s": ts,
                                              "threads": used, "gflops": 2 * 32 * n * k / t / 1e9}
    del w, wabs, wt

    # (c) top-40 of 151936 logits (f32 values of the head's output scale)
    v = synth.QWEN25_3B_VOCAB
    lg = (synth.rng(0, synth.W_DECODE, 997, synth.T_X).standard_normal((1, v)) * 0.905).astype(np.float32)
    t, ts = _median_of(np, lambda: oracle.topk_ref(lg, TOPK))
    stages["c_topk40_of_151936"] = {"median_s": t, "samples_s": ts, "threads": 1, "mlogits_per_s": v / t / 1e6}

    # the oracle's whole GEMV over one decoder layer's seven matrices, all cores
    mats = []
    nbytes = 0
    for j, (name, n_, k_) in enumerate(synth.QWEN25_3B_LAYER):
        q_, s_, b_ = synth.w4_weights(n_, k_, seed=0, workload=synth.W_DECODE, layer=j)
        x_ = synth.activations(1, k_, seed=0, workload=synth.W_DECODE, layer=8 + j)
        mats.append((oracle.pack(q_), s_, b_, x_))
        nbytes += gemv_bytes(1, n_, k_)
    with threadpool_limits(limits=all_threads, user_api="blas"):
        t, ts = _median_of(np, lambda: [oracle.gemv_ref(*m_) for m_ in mats])
    total = time.perf_counter() - t_start
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "sample": f"oracle.gemv_ref over the 7 int4 matrices of one Qwen2.5-3B decoder layer at M=1 "
                      f"({nbytes / 1e6:.1f} MB of algorithmic bytes), median of 5 after 1 warm-up, NumPy fp64 "
                      f"with BLAS on {all_threads} thread(s); stages (a)-(c) beside it",
            "median_s": t, "samples_s": ts, "stages": stages, "host": meta, "seconds": total}


def vendor_gemm(torch, wl, kt, reps=20):
    """Context only: hipBLASLt (torch.matmul, f16 in and out) on the prefill GEMM shapes, the
    best of 3 rounds of back-to-back launches, beside gemm_f16's per-launch time (which also
    writes an f32 C, twice the output bytes)."""
    res = []
    stream = torch.cuda.current_stream()
    for name, a, wt, c, (m, n, k), _, _ in wl.prefill_g:
        ref = torch.matmul(a, wt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(3):
            e0.record(stream)
            for _ in range(reps):
                torch.matmul(a, wt, out=ref)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
        ours = kt[("gemm_f16", m, n, k)]["avg_us"]
        res.append({"gemm": name, "shape_mnk": [m, n, k], "hipblaslt_f16_out_us": round(best, 2),
                    "gemm_f16_f32_out_us": round(ours, 2), "hipblaslt_over_gemm_f16": round(best / ours, 3)})
        del ref
    return res


def main():
    args = parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.trace_from:
        trace_from(*args.trace_from)
        return
    if args.util_from:
        util_from(*args.util_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import int4_weight_only_group_amd as w4
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}; library {w4.LIB_PATH}")
    wl = Workload(torch, np, w4, synth, unfused=args.unfused)
    if args.counters:
        counters_pass(torch, wl, args.counters)
        return

    phases = [wl.run_gemvs, wl.run_head, wl.run_prefill]
    if args.eager:
        runners = phases
    else:
        t0 = time.time()
        graphs = [capture(torch, f) for f in phases]
        runners = [g.replay for g in graphs]
        log(f"captured 3 HIP graphs in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        for r in runners:
            r()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, r in enumerate(runners):
            r()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)) / 1e3 for j in range(3)]
    per_step = [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(args.steps)] for j in range(3)]  # us
    stats = {"gemv_gbps": median_ci(np, [wl.gemv_bytes / t / 1e3 for t in per_step[0]]),
             "prefill_tflops": median_ci(np, [wl.prefill_flops / t / 1e6 for t in per_step[2]]),
             "gemv_us": median_ci(np, per_step[0]), "head_topk_us": median_ci(np, per_step[1]),
             "prefill_us": median_ci(np, per_step[2])}
    log(f"timed {args.steps} steps in {wall * 1e3:.1f} ms: gemv {ph[0] / args.steps * 1e6:.1f} us, "
        f"head+top-k {ph[1] / args.steps * 1e6:.1f} us, prefill {ph[2] / args.steps * 1e6:.1f} us per step")

    # Steady-state decode: the decode phases alone, back to back, as in a token loop.  In the
    # full step the GEMV phase follows the prefill, whose ~217 MB of outputs are still dirty in
    # the last-level cache and get written back while the GEMVs stream (about 65 us); the
    # headline value keeps that cost, this figure shows the decode loop without it.
    dec = None
    if not args.eager:
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            evd[i][0].record(stream)
            runners[0]()
            evd[i][1].record(stream)
            runners[1]()
            evd[i][2].record(stream)
        torch.cuda.synchronize()
        dg = sum(evd[i][0].elapsed_time(evd[i][1]) for i in range(args.steps)) / args.steps * 1e3
        dh = sum(evd[i][1].elapsed_time(evd[i][2]) for i in range(args.steps)) / args.steps * 1e3
        stats["decode_only_gemv_gbps"] = median_ci(
            np, [wl.gemv_bytes / (evd[i][0].elapsed_time(evd[i][1]) * 1e3) / 1e3 for i in range(args.steps)])
        dec = {"gemv_us": round(dg, 1), "head_topk_us": round(dh, 1),
               "gemv_gbps": round(wl.gemv_bytes / dg / 1e3, 1),
               "decode_step_gbps": round((wl.gemv_bytes + wl.head_bytes) / (dg + dh) / 1e3, 1)}
        log(f"decode-only loop: gemv {dg:.1f} us ({dec['gemv_gbps']} GB/s), head+top-k {dh:.1f} us")

    # The same step launched kernel by kernel on the stream (each launch from Python through the
    # C ABI, no graph), timed the same way: the per-launch host cost is what graphs remove.
    eager = None
    if not args.eager:
        for f in phases:
            f()
        torch.cuda.synchronize()
        eve = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        te0 = time.perf_counter()
        for i in range(args.steps):
            eve[i][0].record(stream)
            for j, f in enumerate(phases):
                f()
                eve[i][j + 1].record(stream)
        torch.cuda.synchronize()
        ewall = time.perf_counter() - te0
        eph = [sum(eve[i][j].elapsed_time(eve[i][j + 1]) for i in range(args.steps)) / args.steps * 1e3
               for j in range(3)]
        eager = {"launch": "stream (eager, one ctypes call per kernel)", "ms_per_step": round(ewall / args.steps * 1e3, 4),
                 "gemv_us": round(eph[0], 1), "head_topk_us": round(eph[1], 1), "prefill_us": round(eph[2], 1),
                 "gemv_gbps": round(wl.gemv_bytes / eph[0] / 1e3, 1),
                 "prefill_tflops": round(wl.prefill_flops / eph[2] / 1e6, 1)}
        log(f"stream-launched step: {eager['ms_per_step']} ms per step; gemv {eph[0]:.1f} us "
            f"({eager['gemv_gbps']} GB/s), head+top-k {eph[1]:.1f} us, prefill {eph[2]:.1f} us")

    check = None
    if not args.no_check:
        import oracle
        t0 = time.time()
        check = parity_check(torch, np, wl, oracle, synth)
        log(f"parity re-check {'ok' if check['ok'] else 'FAILED'} in {time.time() - t0:.1f}s: {check}")

    # The prefill as four launches (each dequant on its own, before its GEMM) in place of the
    # step's prefill graph, timed inside the same step: what riding the next dequant in the
    # GEMM's launch saves.
    seq = None
    if not args.eager:
        gseq = capture(torch, wl.run_prefill_sequential)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            runners[0]()
            runners[1]()
            evs[i][0].record(stream)
            gseq.replay()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ps = [evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(args.steps)]
        seq = {"prefill_us": median_ci(np, ps), "prefill_tflops": round(wl.prefill_flops / float(np.median(ps)) / 1e6, 1),
               "launches": "dequant, GEMM, dequant, GEMM (hipgraph)"}
        del gseq
        log(f"prefill as four launches: {seq['prefill_us']['median']} us "
            f"(step's prefill {stats['prefill_us']['median']} us)")

    kt = kernel_timings(torch, wl)
    # dominant decode kernel: the GEMV shape with the largest total time per step
    per_step = {}
    for mats in wl.layers[:1]:
        for _, _, _, _, _, _, (m, n, k) in mats:
            key = ("w4_gemv", m, n, k)
            per_step[key] = per_step.get(key, 0.0) + kt[key]["avg_us"] * synth.QWEN25_3B_LAYERS
    dom = max(per_step, key=per_step.get)
    d = kt[dom]
    roofline = {"bound": "hbm", "kernel": f"w4_gemv (M,N,K)=({dom[1]},{dom[2]},{dom[3]})",
                "achieved": d["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": d["gbps"] / HBM_PEAK_GBS,
                "traffic": traffic_for("gemv.hip", f"w4_gemv_{dom[1]}_{dom[2]}_{dom[3]}"),
                "bytes_per_launch": d["bytes"], "avg_launch_us": d["avg_us"], "launches_timed": d["launches"]}
    tr = trace_for("/".join(map(str, dom)))
    if tr is not None:  # the committed rocprof trace of this kernel shape, beside the live figure
        roofline["rocprof"] = {"mean_us": round(tr["mean_us"], 3), "median_us": round(tr["median_us"], 3),
                               "frac_from_mean": d["bytes"] / tr["mean_us"] / 1e3 / HBM_PEAK_GBS,
                               "live_over_rocprof_mean": round(tr["mean_us"] / d["avg_us"], 3),
                               "source": "profiles/kernel_trace.json"}
    gk = [v for k_, v in kt.items() if k_[0] == "gemm_f16" and k_[1] == synth.PREFILL_TOKENS]
    g_us = sum(v["avg_us"] for v in gk)
    g_fl = sum(v["flops"] for v in gk)
    roofline_prefill = {"bound": "mfma", "kernel": "gemm_f16 prefill GEMMs (1570x22016x2048 gate|up, 1570x2048x11008 down)",
                        "achieved": g_fl / g_us / 1e6, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": g_fl / g_us / 1e6 / MFMA_F16_PEAK_TFLOPS,
                        "traffic": traffic_for("gemm.hip", "gemm_f16_prefill"), "avg_launch_us": g_us / len(gk)}

    sm = None
    if not args.no_small_m:
        import oracle
        t0 = time.time()
        sm = small_m(torch, np, w4, synth, oracle)
        log(f"small-M GEMVs in {time.time() - t0:.1f}s: " + "; ".join(f"{c['workload']} {c['gbps']} GB/s" for c in sm))

    qz = pk = sv = ih = hs = sg = vg = None
    if not args.no_small_m:
        vg = vendor_gemm(torch, wl, kt)
        log("hipBLASLt on the prefill shapes: " + "; ".join(
            f"{v_['shape_mnk']} {v_['hipblaslt_f16_out_us']} us vs gemm_f16 {v_['gemm_f16_f32_out_us']} us" for v_ in vg))
        import oracle
        sv = spec_verify(torch, np, w4, synth, oracle, wl)
        ih = int4_head(torch, np, w4, synth, oracle, wl)
        hs = head_sections(torch, np, w4, synth, oracle, wl)
        sg = single_gemv(torch, np, w4, synth, oracle)
        log(f"single GEMV: lone launch {sg['lone_launch_us_median']} us, steady state {sg['steady_state_us']} us "
            f"({sg['steady_state_gbps']} GB/s)")
        log("heads: " + "; ".join(f"{k_} {v_['us']} us" for k_, v_ in hs.items()))
        log(f"int4 head + top-{TOPK}: one call {ih['us']} us ({ih['gbps']} GB/s), two calls {ih['two_calls_us']} us, "
            f"parity {'ok' if ih['parity_ok'] else 'FAILED'}")
        log(f"speculative verify: {sv['us']} us, parity {'ok' if sv['parity_ok'] else 'FAILED'}")
        qz = quantize_bench(torch, np, w4, synth, oracle)
        log(f"quantizer: {qz['avg_us']} us, {qz['gbps']} GB/s, parity {'ok' if qz['parity_ok'] else 'FAILED'}")
        pk = pack_bench(torch, np, w4, synth, oracle)
        log(f"packer: {pk['avg_us']} us, {pk['gbps']} GB/s, parity {'ok' if pk['parity_ok'] else 'FAILED'}")

    ctx = context(torch)
    log(f"context: device copy {ctx['copy_1gib_read_plus_write_gbps']} GB/s; clocks {ctx.get('clocks_after_timing')}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(np, oracle, synth)
        log(f"cpu baseline {cpu['value']:.4f} GB/s ({cpu['cores']} BLAS threads) in {cpu['seconds']:.1f}s; "
            + "; ".join(f"{k_} {v_['median_s'] * 1e3:.1f} ms" for k_, v_ in cpu["stages"].items()))

    gemv_gbps = wl.gemv_bytes * args.steps / ph[0] / 1e9
    prefill_tflops = wl.prefill_flops * args.steps / ph[2] / 1e12
    decode_bytes = wl.gemv_bytes + wl.head_bytes
    out = {
        "metric": METRIC,
        "value": round(gemv_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen2.5-3B-shaped int4 decode step at M=1 (36 layers x q,k,v,o,gate,up,down W4 GEMVs, "
                        "f16 head 2048->151936, top-40) + 1570-token prefill of gate/up/down (dequant once + f16 GEMM, "
                        "gate|up as one 2048x22016 scratch and GEMM)",
            "group": 64, "launch": "eager" if args.eager else "hipgraph",
            "gemv_launches_per_step": sum(len(m) for m in wl.layers),
            "qkv_gateup": "separate" if args.unfused else "row-concatenated",
            "gemv_bytes_per_step": wl.gemv_bytes, "prefill_flops_per_step": wl.prefill_flops,
        },
        "frac_hbm": round(gemv_gbps / HBM_PEAK_GBS, 4),
        "prefill_tflops": round(prefill_tflops, 2),
        "prefill_frac_mfma": round(prefill_tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "phase_us_per_step": {"gemv": ph[0] / args.steps * 1e6, "head_topk": ph[1] / args.steps * 1e6,
                              "prefill": ph[2] / args.steps * 1e6},
        "decode_step_gbps": decode_bytes * args.steps / (ph[0] + ph[1]) / 1e9,
        "decode_only_loop": dec,
        "stream_launched_step": eager,
        "prefill_sequential": seq,
        "stats": stats,
        "context": ctx,
        "roofline": roofline,
        "roofline_prefill": roofline_prefill,
        "kernels": {"/".join(map(str, k)): {kk: round(vv, 3) if isinstance(vv, float) else vv for kk, vv in v.items()}
                    for k, v in kt.items()},
        "cpu_baseline": cpu,
        "inputs_sha256": dict(wl.sha, method="SHA-256 of each host buffer's bytes as drawn (uint8 codes before "
                                              "packing, f16 scales/biases/activations/head); each decode layer is one "
                                              "SHA-256 over the hex digests of its buffers in launch order"),
        "host": (cpu or {}).get("host") or host_metadata(np),
        "parity": check,
        "small_m": sm,
        "quantize": qz,
        "pack": pk,
        "spec_verify": sv,
        "int4_head": ih,
        "heads": hs,
        "single_gemv": sg,
        "vendor_gemm_context": vg,
    }
    if ((sm is not None and not all(c["parity_ok"] for c in sm)) or (qz is not None and not qz["parity_ok"]) or (pk is not None and not pk["parity_ok"])
            or (sv is not None and not sv["parity_ok"]) or (ih is not None and not ih["parity_ok"])
            or (hs is not None and not all(v_["parity_ok"] for v_ in hs.values()))
            or (sg is not None and not sg["parity_ok"])):
        check = dict(check or {}, ok=False, side_section_fail=True)
        out["parity"] = check
    if check is not None and not check["ok"]:
        out["value"] = None
        out["error"] = "parity re-check failed"
    print(json.dumps(out), flush=True)
    if check is not None and not check["ok"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
