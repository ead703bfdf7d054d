#!/usr/bin/env python
"""Benchmark of the gfx950 W4A16 group-quantized linear (INT4 weights, group 128, bf16 X).

Default run (one GPU): the decode workload -- M = 1, the gate/up projection
(K 2560 -> N 9728) and the down projection (K 9728 -> N 2560) of a 4B-class MLP;
one step = both projections.  Prints ONE JSON line with:
  value          algorithmic HBM GB/s of the whole step (inputs resident in HBM,
                 weight copies rotated over > 768 MB so the 256 MB Infinity Cache
                 cannot serve them), steps replayed from a HIP graph
  roofline       the dominant kernel (gemv_kernel) against 8 TB/s: algorithmic
                 bytes per launch / average launch time, from HIP events recorded on
                 the launch stream around the timed region (every launch in it is a
                 gemv_kernel); traffic = HBM bytes per launch from the committed
                 rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain
                 copy of known size), or null if the kernel sources changed since
  cpu_baseline   the fp64 CPU oracle timed on this host on a bounded sample
  workloads      the same measurements for the other shapes: a single 512x512
                 linear, one decoder layer's seven projections at M = 16 (a draft
                 block), the fused lm_head verify over a 151936 vocabulary,
                 prefill at M = 8192 (TFLOP/s against the bf16 MFMA peak), and the
                 further calls: the layer in four batched launches, re-quantization,
                 an act-order projection, sliding-window attention and the gated
                 gate/up pair (silu(gate) * up in one launch); and, as context only, a
                 dense bf16 library GEMM (hipBLASLt) of the prefill shapes
Options: --only WORKLOAD times one workload (for profiling runs), --calib runs a
plain copy of known size (HBM counter calibration), --pmc-summary writes the
traffic summary from the counter CSVs of those runs (no GPU needed).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
CACHE_ROTATE_BYTES = 768 << 20
METRIC = "W4A16 linear µs and HBM GB/s (% of peak) at M=1/16; TFLOP/s at M=8192"
HEADLINE = "decode_gemv_m1"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def algo_bytes(M, N, K, out_bytes=2, lmhead=False):
    """Bytes a call must move: the packed grid, X, and Y (out_bytes per output).  The
    lm_head call as timed here writes no logits, only the argmax ids and the accepted
    length (and reads the draft ids)."""
    G = K // 128
    if lmhead:
        out_bytes = 0
    b = N * K // 2 + 2 * N * G + N * G // 2 + 2 * M * K + out_bytes * M * N
    if lmhead:
        b += 4 * M + 4 * M + 4  # draft ids in, argmax ids + accept length out
    return b


# the kernel each small-M workload's launches run, and the sources that decide what it
# reads and writes (their hash stamps a counter summary)
KERNEL_OF = {"decode_gemv_m1": "gemv_kernel", "single_512": "gemv_kernel", "verify_block_m16": "block_kernel",
             "verify_block_m16+batch": "block_kernel", "lmhead_verify_m16": "skinny_kernel",
             "prefill_m8192": "tiled_kernel"}
KERNEL_SOURCES = {"gemv_kernel": ("common.h", "kernels.h", "gemv.hip", "api.hip"),
                  "block_kernel": ("common.h", "kernels.h", "block.hip", "api.hip"),
                  "skinny_kernel": ("common.h", "kernels.h", "skinny.hip", "api.hip"),
                  "tiled_kernel": ("common.h", "kernels.h", "tiled.hip", "api.hip")}
CALIB_BYTES = 1 << 30


def kernel_source_sha(kernel="gemv_kernel"):
    """Hash of the code (comments and blank lines removed) of the sources that decide
    what the kernel reads and writes."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "int4_weight_only_02_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def pmc_path(workload):
    return os.path.join(PROFILE_DIR, "%s__%s__pmc.txt" % (KERNEL_OF[workload], workload.replace("+", "_")))


def load_traffic(workload):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernels."""
    path = pmc_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha(KERNEL_OF[workload]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ReadProbe:
    """A plain streaming read (libw4a16_bench.so) of a launch's byte count, over
    rotating slices of a 1 GiB buffer: the ceiling of a kernel that only reads them."""

    def __init__(self, dev):
        import ctypes
        import torch
        self.lib = ctypes.CDLL(os.path.join(ROOT, "int4_weight_only_02_amd", "libw4a16_bench.so"))
        self.lib.w4a16_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        self.lib.w4a16_bench_read.restype = ctypes.c_int
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4, dtype=torch.uint8, device=dev)

    def us(self, nbytes, reps=200):
        import ctypes
        import torch
        nb = (nbytes + 255) // 256 * 256
        R = max(2, min(256, (1 << 30) // nb))
        base = self.buf.data_ptr()

        def one(r, s):
            st = self.lib.w4a16_bench_read(ctypes.c_void_p(base + r * nb), nb, ctypes.c_void_p(self.sink.data_ptr()),
                                           ctypes.c_void_p(s.cuda_stream))
            assert st == 0

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            one(0, s)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for r in range(R):
                    one(r, s)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        n = max(1, reps // R)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (n * R)


# Projections of one step that read the same activations, so that nothing in the
# group waits for another's output: they may share one launch.  In a decoder layer q,
# k and v read the layer input and gate and up the MLP input, while o reads the
# attention output and down the gated MLP activation; a decode step's MLP (gate/up,
# then down) is a chain.
BATCH_GROUPS = {
    "verify_block_m16": [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]],
}


class Workload:
    """Device tensors for one workload: R rotating copies of every projection."""

    def __init__(self, name, dev, lmhead=False, max_copies=64, batched=False):
        import torch
        import int4_weight_only_02_amd as w4
        self.name = name
        self.lmhead = lmhead
        self.batched = batched
        self.shapes = synth.WORKLOADS[name]
        self.projs = []
        per_copy = 0
        for j, (label, M, K, N) in enumerate(self.shapes):
            per_copy += algo_bytes(M, N, K)
        self.R = int(min(max_copies, max(1, -(-CACHE_ROTATE_BYTES // per_copy))))
        ws_need = 0
        for j, (label, M, K, N) in enumerate(self.shapes):
            d = synth.workload_inputs(name, j)
            codes = torch.from_numpy(d["codes"]).to(dev)
            zeros = torch.from_numpy(d["zeros"]).to(dev)
            qw, qz = w4.w4a16_pack(codes, zeros)
            del codes, zeros
            X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
            S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
            copies = [(X, qw, S, qz)] + [(X.clone(), qw.clone(), S.clone(), qz.clone()) for _ in range(self.R - 1)]
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            p = {"label": label, "M": M, "K": K, "N": N, "copies": copies, "Y": Y, "host": d}
            if lmhead:
                # the draft block: seeded ids, the first L0 forced to the oracle's greedy
                # choice (the pages' verifier accepts exactly that prefix); the oracle's
                # logits are kept for the check of the benchmarked call
                import oracle
                draft, L0, rng = synth.draft_block(synth.seed_for(name, j), M, N)
                oqw, oqz = oracle.pack(d["codes"], d["zeros"])
                p["Yo"] = oracle.linear_matmul(d["X"], oqw, d["scales"], oqz)
                del oqw, oqz
                am_o = oracle.argmax_accept(p["Yo"], np.zeros(M, np.int32))[0]
                draft = synth.force_prefix(draft, L0, am_o, rng, N)
                p["L0"] = L0
                p["draft"] = torch.from_numpy(draft).to(dev)
                p["argmax"] = torch.empty((M,), dtype=torch.int32, device=dev)
                p["accept"] = torch.empty((1,), dtype=torch.int32, device=dev)
                ws_need = max(ws_need, w4.w4a16_workspace_bytes(w4.OP_LMHEAD, M, N, K))
            else:
                ws_need = max(ws_need, w4.w4a16_workspace_bytes(w4.OP_LINEAR, M, N, K))
            self.projs.append(p)
        self.groups = None
        if batched:
            idx = {p["label"]: q for q, p in enumerate(self.projs)}
            self.groups = [[idx[l] for l in g] for g in BATCH_GROUPS[name]]
            ws_need = max(ws_need, max(sum(w4.w4a16_workspace_bytes(w4.OP_LINEAR, self.projs[q]["M"],
                                                                   self.projs[q]["N"], self.projs[q]["K"])
                                           for q in g) for g in self.groups))
        self.ws = w4.Workspace(dev)
        self.ws.get(ws_need)
        self.bytes_per_step = sum(algo_bytes(p["M"], p["N"], p["K"], lmhead=lmhead) for p in self.projs)
        self.flops_per_step = sum(2 * p["M"] * p["N"] * p["K"] for p in self.projs)

    def launch(self, p, r):
        import int4_weight_only_02_amd as w4
        X, qw, S, qz = p["copies"][r]
        if self.lmhead:
            w4.w4a16_lmhead_verify(X, qw, S, qz, p["draft"], workspace=self.ws,
                                   argmax_out=p["argmax"], accept_out=p["accept"])
        else:
            w4.w4a16_linear(X, qw, S, qz, out=p["Y"], workspace=self.ws)

    def launch_group(self, g, r):
        """One launch for the projections g (w4a16_linear_batch), or the plain call."""
        import int4_weight_only_02_amd as w4
        if len(g) == 1:
            self.launch(self.projs[g[0]], r)
            return
        w4.w4a16_linear_batch([self.projs[q]["copies"][r] for q in g], workspace=self.ws,
                              outs=[self.projs[q]["Y"] for q in g])

    def step(self, r):
        if self.batched:
            for g in self.groups:
                self.launch_group(g, r % self.R)
            return
        for p in self.projs:
            self.launch(p, r % self.R)

    def check(self):
        """Sanity check of one step against the oracle on sampled outputs: f32 Y, so the
        figure is the arithmetic error alone (no bf16 output rounding).  The lm_head
        call is checked by its own rules instead (check_lmhead)."""
        import torch
        import oracle
        import int4_weight_only_02_amd as w4
        if self.lmhead:
            return None
        worst = 0.0
        ys = None
        if self.batched:
            ys = [None] * len(self.projs)
            for g in self.groups:
                out = w4.w4a16_linear_batch([self.projs[q]["copies"][0] for q in g], out_dtype=torch.float32,
                                            workspace=self.ws)
                for q, y in zip(g, out):
                    ys[q] = y
        for q, p in enumerate(self.projs):
            X, qw, S, qz = p["copies"][0]
            Y = ys[q] if ys is not None else w4.w4a16_linear(X, qw, S, qz, out_dtype=torch.float32,
                                                              workspace=self.ws)
            torch.cuda.synchronize()
            d = p["host"]
            oqw, oqz = oracle.pack(d["codes"], d["zeros"])
            rng = np.random.default_rng(0)
            rows = rng.integers(0, p["M"], 256)
            cols = rng.integers(0, p["N"], 256)
            ref = oracle.linear_at(d["X"], oqw, d["scales"], oqz, rows, cols)
            got = Y.cpu().numpy()[rows, cols]
            rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
            worst = max(worst, float(np.abs(got - ref).max()) / rms)
            del Y
        return worst

    def check_lmhead(self):
        """The benchmarked lm_head call against the oracle's logits on the same inputs:
        argmax equal wherever the oracle's top-2 gap exceeds 1e-2 * rms(logits), the
        chosen logit within that tolerance of the maximum elsewhere, the accepted length
        equal to the first mismatch of the GPU's argmax with the draft, and equal to the
        forced prefix L0 when the rows up to it are clear."""
        import torch
        import oracle
        import int4_weight_only_02_amd as w4
        p = self.projs[0]
        X, qw, S, qz = p["copies"][0]
        w4.w4a16_lmhead_verify(X, qw, S, qz, p["draft"], workspace=self.ws, argmax_out=p["argmax"],
                               accept_out=p["accept"])
        torch.cuda.synchronize()
        am = p["argmax"].cpu().numpy()
        L = int(p["accept"].cpu()[0])
        Yo = p["Yo"]
        tol = 1e-2 * float(np.sqrt(np.mean(Yo * Yo)))
        am_o, gap, _ = oracle.argmax_accept(Yo, np.zeros(p["M"], np.int32))
        draft = p["draft"].cpu().numpy()
        clear = gap > tol
        agree = bool((am[clear] == am_o[clear]).all())
        near = bool(all(Yo[i, am[i]] >= Yo[i].max() - tol for i in np.nonzero(~clear)[0]))
        expect_L = next((i for i in range(p["M"]) if am[i] != draft[i]), p["M"])
        L0 = p["L0"]
        l0_ok = L == L0 if bool(clear[: min(L0 + 1, p["M"])].all()) else None
        return {"rows": int(p["M"]), "clear_rows": int(clear.sum()), "argmax_agree_on_clear_rows": agree,
                "ambiguous_rows_within_tol": near, "accept_len": L, "accept_len_matches_argmax": L == expect_L,
                "forced_prefix_L0": int(L0), "accept_len_equals_L0": l0_ok}


def time_events(wl, reps):
    """Eager per-launch time (us, median) from HIP events around every launch, per
    projection (or per batch launch): back-to-back calls from the host, launch
    overhead included."""
    import torch
    out = {}
    if wl.batched:
        for g in wl.groups:
            evs = []
            for i in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                wl.launch_group(g, i % wl.R)
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
            out["+".join(wl.projs[q]["label"] for q in g)] = float(np.median([a.elapsed_time(b) * 1e3
                                                                              for a, b in evs]))
        return out
    for p in wl.projs:
        evs = []
        for i in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            wl.launch(p, i % wl.R)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) * 1e3 for a, b in evs]
        out[p["label"]] = float(np.median(t))
    return out


def capture(wl, steps, start):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(2):  # warm the lazy initialisation outside the capture
            wl.step(start + i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                wl.step(start + i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_steps(wl, steps, warmup):
    """Exactly `steps` steps replayed from HIP graphs (a cycle over the R copies plus
    a remainder), bracketed by device synchronization.  Returns seconds per step."""
    import torch
    cyc = capture(wl, wl.R, 0)
    rem_n = steps % wl.R
    rem = capture(wl, rem_n, 0) if rem_n else None
    for _ in range(max(1, -(-warmup // wl.R))):
        cyc.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps // wl.R):
        cyc.replay()
    if rem is not None:
        rem.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, e0.elapsed_time(e1) * 1e-3 / steps


def cpu_baseline(name, budget_s=10.0):
    """The fp64 oracle (as it stands) on this host, on the headline step: repeat whole
    steps (both projections at full size) until about budget_s seconds have passed."""
    import oracle
    data = []
    for j, (label, M, K, N) in enumerate(synth.WORKLOADS[name]):
        d = synth.workload_inputs(name, j)
        qw, qz = oracle.pack(d["codes"], d["zeros"])
        data.append((d["X"], qw, d["scales"], qz, algo_bytes(M, N, K)))
    n = 0
    t0 = time.perf_counter()
    while True:
        for X, qw, S, qz, _ in data:
            oracle.linear(X, qw, S, qz)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    gbs = sum(b for *_, b in data) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "%d full decode steps (M=1, K2560xN9728 and K9728xN2560), fp64 naive loops, %.1f s"
                      % (n, dt * n),
            "ms_per_step": round(dt * 1e3, 3)}


def _graph_of(fn, count):
    """A HIP graph of fn(0) .. fn(count - 1) captured on a side stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for r in range(count):
                fn(r)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_median_steps(wl, calls=200):
    """Median over `calls` back-to-back steps, each step one graph replay (a graph per
    weight copy, in rotation) bracketed by its own HIP events: the median of >= 200
    calls, queued behind a GPU-side wait so that the host's launch rate does not enter
    the figure.  Returns microseconds."""
    import torch
    graphs = [_graph_of(lambda i, r=r: wl.step(r), 1) for r in range(wl.R)]
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    # hold the GPU (about 20 ms) while the host queues every call, so that the calls
    # then run back to back and each pair of events brackets GPU time only
    torch.cuda._sleep(50_000_000)
    evs = []
    for i in range(calls):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graphs[i % wl.R].replay()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))


def time_launch_graph(wl, p, calls=200):
    """One projection alone: graph replays of the rotating copies back to back; the
    median of five runs of about `calls` launches each.  Microseconds per launch."""
    import torch
    g = _graph_of(lambda r: wl.launch(p, r % wl.R), wl.R)
    g.replay()
    torch.cuda.synchronize()
    n = max(1, calls // wl.R)
    runs = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / (n * wl.R))
    return float(np.median(runs))


READ_PROBE = None


def measure(name, dev, steps, warmup, lmhead=False, ev_reps=200, batched=False):
    wl = Workload(name, dev, lmhead=lmhead, batched=batched)
    err = wl.check()
    lm = wl.check_lmhead() if lmhead else None
    ev = time_events(wl, ev_reps)
    wall, gpu = time_steps(wl, steps, warmup)
    med = time_median_steps(wl)
    res = {"copies": wl.R, "bytes_per_step": wl.bytes_per_step, "flops_per_step": wl.flops_per_step,
           "us_per_step": round(wall * 1e6, 3), "us_per_step_gpu_events": round(gpu * 1e6, 3),
           "us_per_step_median200": round(med, 3),
           "GBps": round(wl.bytes_per_step / wall / 1e9, 2),
           "hbm_frac": round(wl.bytes_per_step / wall / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(wl.flops_per_step / wall / 1e12, 3),
           "launches_per_step": len(wl.groups) if batched else len(wl.projs),
           "batched": batched, "kernel": KERNEL_OF.get(name + ("+batch" if batched else "")),
           "kernel_us_eager_median": {k: round(v, 3) for k, v in ev.items()},
           "sampled_max_err_over_rms": err}
    if lm is not None:
        res["lmhead_check"] = lm
    per = {}
    for p in wl.projs:
        if batched:
            continue
        t = ev[p["label"]] * 1e-6
        b = algo_bytes(p["M"], p["N"], p["K"], lmhead=lmhead)
        f = 2 * p["M"] * p["N"] * p["K"]
        entry = {"M": p["M"], "K": p["K"], "N": p["N"], "eager_us": round(t * 1e6, 3),
                 "GBps": round(b / t / 1e9, 1), "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                 "TFLOPs": round(f / t / 1e12, 2), "mfma_frac": round(f / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
        if p["M"] <= 64:
            tg = time_launch_graph(wl, p)
            entry.update({"graph_us": round(tg, 3), "graph_GBps": round(b / tg / 1e3, 1),
                          "graph_hbm_frac": round(b / tg / 1e3 / HBM_PEAK_GBS, 4)})
            if READ_PROBE is not None:
                tr = READ_PROBE.us(b)
                entry.update({"plain_read_us": round(tr, 3), "plain_read_GBps": round(b / tr / 1e3, 1),
                              "kernel_over_plain_read": round(tg / tr, 3)})
        per[p["label"]] = entry
    res["per_launch"] = per
    del wl
    import torch
    torch.cuda.empty_cache()
    return res


def measure_requant(dev, steps, warmup, N=9728, K=2560):
    """w4a16_quantize on one gate/up-shaped matrix: rounding weights near the grid back
    onto it (frozen scales and zeros), bf16 in, packed words out.  HBM-bound; bytes per
    launch = 2NK (W) + NK/2 (codes) + 2NG + NG/2 (scales, zeros)."""
    import torch
    import int4_weight_only_02_amd as w4
    import oracle
    G = K // 128
    d = synth.requant_inputs(4242, N, K)
    W = torch.from_numpy(d["W"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    qz = w4.w4a16_pack(torch.zeros((N, K), dtype=torch.uint8, device=dev), torch.from_numpy(d["zeros"]).to(dev))[1]
    nbytes = 2 * N * K + N * K // 2 + 2 * N * G + N * G // 2
    R = int(max(1, min(32, -(-CACHE_ROTATE_BYTES // nbytes))))
    copies = [W] + [W.clone() for _ in range(R - 1)]
    out = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    # check: a sample of rows bit-exact against the oracle
    w4.w4a16_quantize(W, S, qz, out=out)
    torch.cuda.synchronize()
    rows = np.arange(0, N, max(1, N // 64))
    codes = oracle.quantize(d["W"][rows], d["scales"][rows], d["zeros"][rows])
    want = np.zeros((len(rows), K // 8), np.uint32)
    for j in range(8):
        want |= codes[:, j::8].astype(np.uint32) << (4 * j)
    exact = bool((out.cpu().numpy().view(np.uint32)[rows] == want).all())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        w4.w4a16_quantize(copies[0], S, qz, out=out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for r in range(R):
                w4.w4a16_quantize(copies[r], S, qz, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(max(1, warmup // R)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // R)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * R)
    return {"N": N, "K": K, "copies": R, "launches": reps * R, "bytes_per_launch": nbytes,
            "us_per_launch": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
            "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bit_exact_sample": exact}


def measure_actorder(dev, steps, warmup, M=16, N=9728, K=2560):
    """One gate/up-shaped projection at M = 16 with GPTQ act-order groups
    (w4a16_linear_actorder: gather X by the column permutation, then the ordinary
    kernels), next to the same call on the plain grid; graph replay over rotating
    weight copies.  The difference is the cost of act-order."""
    import torch
    import int4_weight_only_02_amd as w4
    import oracle
    rng = np.random.default_rng(4343)
    d = synth.linear_inputs(4343, M, N, K)
    order = rng.permutation(K)
    g_idx = np.empty(K, np.int32)
    g_idx[order] = np.arange(K) // 128
    perm = torch.from_numpy(w4.w4a16_actorder_perm(g_idx)).to(dev)
    codes = torch.from_numpy(d["codes"]).to(dev)
    zeros = torch.from_numpy(d["zeros"]).to(dev)
    qw, qz = w4.w4a16_pack_actorder(codes, zeros, perm)
    X = torch.from_numpy(d["X"].view(np.int16)).to(dev).view(torch.bfloat16)
    S = torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16)
    nbytes = algo_bytes(M, N, K)
    R = int(max(1, min(32, -(-CACHE_ROTATE_BYTES // nbytes))))
    copies = [(qw, S, qz)] + [(qw.clone(), S.clone(), qz.clone()) for _ in range(R - 1)]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = w4.Workspace(dev)
    ws.get(w4.w4a16_workspace_bytes(w4.OP_LINEAR_ACTORDER, M, N, K))
    # check: sampled outputs against the oracle's act-order definition
    Yf = w4.w4a16_linear_actorder(X, perm, qw, S, qz, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    oqw, oqz = oracle.pack(d["codes"], d["zeros"])
    cols = np.arange(0, N, max(1, N // 256))
    sub = oracle.linear_gidx(d["X"], oqw[cols], d["scales"][cols], oracle.pack(d["codes"][cols], d["zeros"][cols])[1],
                             g_idx) if len(cols) % 8 == 0 else None
    err = None
    if sub is not None:
        got = Yf.cpu().numpy()[:, cols].astype(np.float64)
        err = float(np.abs(got - sub).max() / np.sqrt((sub ** 2).mean()))

    def timed(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            fn(0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for r in range(R):
                    fn(r)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // R)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // R)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * R)

    t_act = timed(lambda r: w4.w4a16_linear_actorder(X, perm, *copies[r], out=Y, workspace=ws))
    t_plain = timed(lambda r: w4.w4a16_linear(X, *copies[r], out=Y, workspace=ws))
    return {"M": M, "N": N, "K": K, "copies": R, "bytes_per_call": nbytes,
            "us_per_call_actorder": round(t_act, 3), "us_per_call_plain": round(t_plain, 3),
            "GBps_actorder": round(nbytes / t_act / 1e3, 1), "sampled_max_err_over_rms": err}


def measure_gated(dev, steps, warmup, N=9728, K=2560):
    """The MLP's gate and up projections (K 2560 -> N 9728 each) on the same rows, at
    M = 16 (a draft block) and M = 1: w4a16_linear_gated (both projections and
    silu(gate) * up in one launch, one bf16 output) next to w4a16_linear_batch of the
    two projections (one launch, two outputs, no activation); at M = 8192 (prefill) the
    gated tile kernel next to the two w4a16_linear calls alone (two bf16 outputs, no
    activation).  Graph replay over rotating weight copies.  Algorithmic bytes: both
    packed grids, X once, Y once; flops 2 * 2MNK."""
    import torch
    import int4_weight_only_02_amd as w4
    import oracle
    G = K // 128
    out = {"N": N, "K": K}
    for M in (16, 1, 8192):
        dg = synth.linear_inputs(5151 + M, M, N, K)
        du = synth.linear_inputs(5152 + M, M, N, K)
        X = torch.from_numpy(dg["X"].view(np.int16)).to(dev).view(torch.bfloat16)

        def grid(d):
            qw, qz = w4.w4a16_pack(torch.from_numpy(d["codes"]).to(dev), torch.from_numpy(d["zeros"]).to(dev))
            return qw, torch.from_numpy(d["scales"].view(np.int16)).to(dev).view(torch.float16), qz

        gate, up = grid(dg), grid(du)
        nbytes = 2 * (N * K // 2 + 2 * N * G + N * G // 2) + 2 * M * K + 2 * M * N
        R = int(max(1, min(32, -(-CACHE_ROTATE_BYTES // nbytes))))
        copies = [(gate, up)] + [(tuple(t.clone() for t in gate), tuple(t.clone() for t in up))
                                 for _ in range(R - 1)]
        ws = w4.Workspace(dev)
        ws.get(max(w4.w4a16_workspace_bytes(w4.OP_LINEAR_GATED, M, N, K),
                   2 * w4.w4a16_workspace_bytes(w4.OP_LINEAR, M, N, K), 1 << 20))
        # check: sampled outputs against the oracle (both projections one by one)
        Yf = w4.w4a16_linear_gated(X, gate, up, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        rng = np.random.default_rng(M)
        rows = rng.integers(0, M, 256).astype(np.int32)
        cols = rng.integers(0, N, 256).astype(np.int32)
        og = oracle.pack(dg["codes"], dg["zeros"])
        ou = oracle.pack(du["codes"], du["zeros"])
        go = oracle.linear_at(dg["X"], og[0], dg["scales"], og[1], rows, cols)
        uo = oracle.linear_at(dg["X"], ou[0], du["scales"], ou[1], rows, cols)
        yo = oracle.silu_mul(go, uo)
        dy = np.abs(Yf.cpu().numpy()[rows, cols] - yo)
        err = float(dy.max() / np.sqrt((yo ** 2).mean()))
        # the gated bound: each projection's 1e-2 rms carried through silu(g) * u
        eg, eu = 1e-2 * np.sqrt((go ** 2).mean()), 1e-2 * np.sqrt((uo ** 2).mean())
        bound = 1.1 * np.abs(uo) * eg + np.abs(go / (1.0 + np.exp(-go))) * eu + 1.1 * eg * eu
        err_b = float((dy / bound).max())
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        Yg = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        Yu = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def timed(fn):
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                fn(0)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for r in range(R):
                        fn(r)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            for _ in range(max(1, warmup // R)):
                g.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // R)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * R)

        t_gated = timed(lambda r: w4.w4a16_linear_gated(X, *copies[r], out=Y, workspace=ws))
        if M <= 16:
            t_batch = timed(lambda r: w4.w4a16_linear_batch([(X,) + copies[r][0], (X,) + copies[r][1]],
                                                            outs=[Yg, Yu], workspace=ws))
            out["m%d" % M] = {"copies": R, "bytes_per_call": nbytes, "us_per_call_gated": round(t_gated, 3),
                              "GBps_gated": round(nbytes / t_gated / 1e3, 1),
                              "hbm_frac_gated": round(nbytes / t_gated / 1e3 / HBM_PEAK_GBS, 4),
                              "us_per_call_batch_two_outputs": round(t_batch, 3),
                              "sampled_max_err_over_rms": err, "sampled_max_err_over_bound": err_b}
        else:
            t_two = timed(lambda r: (w4.w4a16_linear(X, *copies[r][0], out=Yg, workspace=ws),
                                     w4.w4a16_linear(X, *copies[r][1], out=Yu, workspace=ws)))
            flops = 2 * 2 * M * N * K
            out["m%d" % M] = {"copies": R, "flops_per_call": flops, "us_per_call_gated": round(t_gated, 3),
                              "TFLOPs_gated": round(flops / t_gated / 1e6, 1),
                              "mfma_frac_gated": round(flops / t_gated / 1e6 / BF16_PEAK_TFLOPS, 4),
                              "us_per_call_two_linear_calls": round(t_two, 3),
                              "sampled_max_err_over_bound": err_b}
    return out


def measure_gemm_ceiling(dev, steps, warmup):
    """Context for the prefill figure, not part of the layer: a plain dense bf16 GEMM of
    the prefill shapes through the vendor library (torch.mm -> hipBLASLt), fp32
    accumulation, no quantization -- what a tuned library reaches on these shapes with
    no dequantization work at all.  Back-to-back eager calls over two weight copies,
    HIP events on the current stream (each call runs hundreds of microseconds)."""
    import torch
    out = {}
    M = 8192
    for label, K, N in (("gate_up", 2560, 9728), ("down", 9728, 2560)):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + K)
        X = torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16)
        Ws = [(torch.randn((N, K), device=dev, generator=g) * 0.02).to(torch.bfloat16).t().contiguous()
              for _ in range(2)]  # [K, N], contiguous (no transposed views)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for r in range(4):
            torch.mm(X, Ws[r % 2], out=Y)
        torch.cuda.synchronize()
        reps = max(4, min(steps, 40))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            torch.mm(X, Ws[r % 2], out=Y)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        tf = 2.0 * M * N * K / t / 1e12
        out[label] = {"M": M, "K": K, "N": N, "us_per_call": round(t * 1e6, 2), "TFLOPs": round(tf, 1),
                      "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        del X, Ws, Y
        torch.cuda.empty_cache()
    out["note"] = "dense bf16 torch.mm (hipBLASLt), unquantized weights: an achievable-ceiling reference only"
    return out


def measure_swa(dev, steps, warmup, M=16, T=8192, Hq=32, Hkv=8, window=1024):
    """The drafter's sliding-window attention for one verify block: M = 16 queries at
    the end of an 8192-token context, 32 query heads over 8 key/value heads of 128,
    window 1024 (the pages' leaderboard setting) and 2048; causal, and bidirectional
    within the block (block_window_*).  Algorithmic bytes: the keys
    and values of the union of the windows, Q and O (bf16)."""
    import torch
    import int4_weight_only_02_amd as w4
    import oracle
    D = 128
    rng = np.random.default_rng(5151)
    bits = lambda a: synth.f32_to_bf16_bits(np.asarray(a, np.float32))
    Q = bits(rng.normal(0, 1, (M, Hq, D)))
    K = bits(rng.normal(0, 1, (T, Hkv, D)))
    Vt = bits(rng.normal(0, 1, (Hkv, D, T)))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    out = {}
    for block, W in ((False, window), (False, 2 * window), (True, window), (True, 2 * window)):
        nkeys = min(T, W + M - 1)
        nbytes = 2 * nkeys * Hkv * D * 2 + 2 * M * Hq * D * 2
        R = int(max(1, min(32, -(-CACHE_ROTATE_BYTES // (2 * T * Hkv * D * 2)))))
        caches = [(t(K), t(Vt)) for _ in range(R)]
        Qd = t(Q)
        O = torch.empty((M, Hq, D), dtype=torch.bfloat16, device=dev)
        ws = w4.Workspace(dev)
        Of = w4.w4a16_swa_attention(Qd, *caches[0], T, W, out_dtype=torch.float32, workspace=ws, block=block)
        torch.cuda.synchronize()
        Oo = (oracle.swa_block if block else oracle.swa)(Q, K, Vt, W)
        err = float(np.abs(Of.cpu().numpy() - Oo).max() / np.sqrt((Oo ** 2).mean()))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            w4.w4a16_swa_attention(Qd, *caches[0], T, W, out=O, workspace=ws, block=block)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for r in range(R):
                    w4.w4a16_swa_attention(Qd, *caches[r], T, W, out=O, workspace=ws, block=block)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // R)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // R)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * R)
        out[("block_window_%d" if block else "window_%d") % W] = {"us_per_call": round(us, 3), "bytes_per_call": nbytes,
                                "GBps": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                "max_err_over_rms": err, "copies": R}
    out.update({"M": M, "T": T, "Hq": Hq, "Hkv": Hkv, "D": D})
    return out


def calib_copy(dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "reps": reps}))


def _pmc_mean(path, counter, name_filter):
    """Mean value of one counter per dispatch of the kernels whose name contains
    name_filter, from a rocprofv3 counter_collection.csv."""
    import csv
    vals = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter and name_filter in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no %s rows for kernels matching %r in %s" % (counter, name_filter, path))
    return float(np.mean(vals)), len(vals)


def pmc_summary(workload, fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, commands):
    """HBM traffic per launch of the workload's kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a plain copy of CALIB_BYTES."""
    kernel = KERNEL_OF[workload]
    fk, fn = _pmc_mean(fetch_csv, "FETCH_SIZE", kernel)
    wk, wn = _pmc_mean(write_csv, "WRITE_SIZE", kernel)
    cf, _ = _pmc_mean(calib_fetch_csv, "FETCH_SIZE", "copy")
    cw, _ = _pmc_mean(calib_write_csv, "WRITE_SIZE", "copy")
    f_scale = CALIB_BYTES / (cf * 1024.0)
    w_scale = CALIB_BYTES / (cw * 1024.0)
    fetch_b = fk * 1024.0 * f_scale
    write_b = wk * 1024.0 * w_scale
    base = workload.split("+")[0]
    launches = synth.WORKLOADS[base]
    lm = base == "lmhead_verify_m16"
    if workload.endswith("+batch"):
        groups = BATCH_GROUPS[base]
        idx = {l[0]: l for l in launches}
        per = [sum(algo_bytes(idx[x][1], idx[x][3], idx[x][2]) for x in g) for g in groups]
        algo = float(np.mean(per))
    else:
        algo = float(np.mean([algo_bytes(M, N, K, lmhead=lm) for _, M, K, N in launches]))
    lines = ["# %s HBM traffic per launch, workload %s" % (kernel, workload),
             "# shapes (label, M, K, N): %s" % (launches,),
             "# commands (each counter in its own run):"] + ["#   %s" % c for c in commands] + [
             "# calibration: a plain device copy of %d bytes (torch copy_) reads FETCH_SIZE %.1f KiB and"
             " WRITE_SIZE %.1f KiB per dispatch -> scale fetch x%.4f, write x%.4f" % (CALIB_BYTES, cf, cw, f_scale, w_scale),
             "fetch_kib_per_dispatch: %.1f" % fk, "fetch_dispatches: %d" % fn,
             "write_kib_per_dispatch: %.1f" % wk, "write_dispatches: %d" % wn,
             "hbm_fetch_bytes_per_launch: %.0f" % fetch_b, "hbm_write_bytes_per_launch: %.0f" % write_b,
             "hbm_bytes_per_launch: %.0f" % (fetch_b + write_b),
             "algorithmic_bytes_per_launch: %.0f" % algo,
             "traffic_over_algorithmic: %.4f" % ((fetch_b + write_b) / algo),
             "kernel_source_sha: %s" % kernel_source_sha(kernel)]
    os.makedirs(PROFILE_DIR, exist_ok=True)
    out = pmc_path(workload)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--only", default=None, help="time one workload only (profiling runs)")
    ap.add_argument("--proj", default=None, help="with --only: keep only the projection of this label "
                    "(e.g. gate_up or down of prefill_m8192), for per-shape counter runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the plain-read ceiling beside each launch")
    ap.add_argument("--calib", action="store_true")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_FETCH_CSV", "CALIB_WRITE_CSV"),
                    help="write the traffic summary of --only WORKLOAD (default the headline) from counter CSVs")
    ap.add_argument("--pmc-command", action="append", default=[], help="command line recorded in the summary")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.only or HEADLINE, *args.pmc_summary, commands=args.pmc_command)
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the layer runs on one GPU's share; "
              "multi-GPU sharding is described, not run); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_only_02_amd as w4
    w4.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    if args.calib:
        calib_copy(dev)
        return
    global READ_PROBE
    if not args.no_read_probe:
        READ_PROBE = ReadProbe(dev)

    if args.proj:
        if not args.only or args.only not in synth.WORKLOADS:
            raise SystemExit("--proj needs --only with a linear workload")
        keep = [p for p in synth.WORKLOADS[args.only] if p[0] == args.proj]
        if not keep:
            raise SystemExit("no projection %r in %s" % (args.proj, args.only))
        synth.WORKLOADS[args.only] = keep
    names = [HEADLINE, "single_512", "verify_block_m16", "lmhead_verify_m16", "prefill_m8192",
             "verify_block_m16+batch", "requantize_9728x2560", "actorder_gate_m16", "swa_verify_m16_t8192",
             "mlp_gate_up_gated", "prefill_bf16_gemm_library"]
    if args.only:
        names = [args.only]
    results = {}
    for key in names:
        if key in ("requantize_9728x2560", "actorder_gate_m16", "swa_verify_m16_t8192", "mlp_gate_up_gated",
                   "prefill_bf16_gemm_library"):
            fn = {"requantize_9728x2560": measure_requant, "actorder_gate_m16": measure_actorder,
                  "swa_verify_m16_t8192": measure_swa, "mlp_gate_up_gated": measure_gated,
                  "prefill_bf16_gemm_library": measure_gemm_ceiling}[key]
            results[key] = fn(dev, max(64, min(args.steps, 1000)), 32)
            print("[bench] %s: %s" % (key, json.dumps(results[key])), file=sys.stderr, flush=True)
            continue
        name, batched = key.split("+")[0], key.endswith("+batch")
        steps = args.steps if name != "prefill_m8192" else max(4, min(args.steps, 40))
        warm = args.warmup if name != "prefill_m8192" else 4
        if name == "lmhead_verify_m16":
            steps = max(10, min(args.steps, 400))
        results[key] = measure(name, dev, steps, warm, lmhead=(name == "lmhead_verify_m16"), batched=batched)
        print("[bench] %s: %s" % (key, json.dumps(results[key])), file=sys.stderr, flush=True)

    head = results.get(HEADLINE) or results[names[0]]
    if "per_launch" not in head:  # --only requantize_9728x2560 / actorder_gate_m16
        print(json.dumps({"workloads": results}))
        return
    head_name = HEADLINE if HEADLINE in results else names[0]
    per = head["per_launch"]
    kernel = KERNEL_OF.get(head_name, "gemv_kernel")
    # every launch in the timed region is one `kernel` launch (one per projection)
    b_launch = head["bytes_per_step"] / head["launches_per_step"]
    t_launch = head["us_per_step_gpu_events"] * 1e-6 / head["launches_per_step"]
    achieved = b_launch / t_launch / 1e9
    traffic = load_traffic(head_name)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel, "algorithmic_bytes_per_launch": int(b_launch),
            "avg_launch_us": round(t_launch * 1e6, 3),
            "timing": "HIP events on the launch stream around the timed graph replays / launches"}
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(HEADLINE)
    steps_head = args.steps
    line = {"metric": METRIC, "value": head["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": steps_head,
            "warmup": args.warmup, "ms_per_step": round(head["us_per_step"] / 1e3, 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": head_name, "M": 1, "group": 128,
                       "shapes": [[v["M"], v["K"], v["N"]] for v in per.values()],
                       "cache": "cold: %d rotating weight copies (> 768 MB)" % head["copies"],
                       "timing": "HIP graph replay of exactly `steps` steps, wall clock between device syncs"},
            "roofline": roof, "cpu_baseline": cpu,
            "workloads": results}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
