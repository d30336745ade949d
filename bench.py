"""Benchmark: Q4_K decode GEMV sweep over 36 Qwen3-4B-shaped layers on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A step is one batch-1 decode token: for each of 36 layers and each projection
q, k, v, o, gate, up, down (distinct seeded Q4_K matrices, 2.04 GB in total, so
nothing stays in the 256 MB last-level cache) the activation of that product (a
fresh N(0,1) fp32 row) is quantized to Q8 and multiplied by the matrix.  The
products that share an input width go out together: per layer one
q4k_quantize_gemv_batch launch for {q, k, v}, one for {o}, one for {gate, up}
and one for {down} (144 launches per step, each quantizing inside the GEMV,
codes bit-identical to q4k_quantize_act).  All inputs are resident in HBM
before timing.  Each step is replayed from a HIP graph (the host cost of the
small launches would otherwise be measured instead of the GPU).  One pair of
HIP events on the launch stream brackets every timed step, which is exactly the
block of back-to-back GEMV dispatches; that gives the mean launch duration for
the roofline (an event pair around each kernel would add a marker dispatch of
several microseconds).  The same sweep as one q4k_quantize_gemv launch per
product (252 per step), and as two launches per product (q4k_quantize_act, then
q4k_gemv), are timed after the timed region and reported beside it, and so
is the step with o and down adding into a residual stream inside their GEMVs
(q4k_quantize_gemv_residual, in place).

Printed: one JSON line with the whole-job rate (algorithmic bytes / wall time),
the per-step distribution (median, p10, p90 over the timed steps), the GEMV
roofline (algorithmic bytes per launch / mean launch duration, against
8 TB/s), and the CPU oracle timed on this host on a bounded sample of the same
sweep, single-threaded and on all cores (OpenMP over output rows).  Beside
them, outside the timed region: the practical decode ceilings (a plain
16-byte stream read of each launch group's bytes and an empty kernel), the
same sweep at one GPU's share of an 8-way row shard, the
prefill GEMM (M = 512, 20 steps, with the shader clock sampled during the
steps for a measured-clock peak, and how far fp16 matrix-core ops and fp32
vector fmas of one SIMD overlap), the small-batch GEMV (M = 2, 4, 8), the
routed-expert layer (T = 1, 16) and the Q6_K decode GEMV over the same
projection shapes -- each checked against the oracle before it is timed --
and the oracle's own rate on each of those workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix peak
FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak (the prefill GEMM's matrix-core dtype)
LAYERS = 36
PREFILL_M = 512
METRIC = "Q4_K decode GEMV GB/s (% HBM peak); prefill Q4_K×Q8 GEMM TOPS (% MFMA)"


def dist(seconds):
    """median / p10 / p90 / mean of per-pass times, in the unit given."""
    a = np.asarray(seconds, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "passes": int(a.size)}


def dist_ms(seconds):
    return {k: (round(v * 1e3, 4) if k != "passes" else v) for k, v in dist(seconds).items()}


class ClockSampler:
    """Samples the GPU's shader clock (MHz) from sysfs while running, in a
    background thread; mean() is None where the clock cannot be read."""

    def __init__(self, period=0.02):
        import glob
        import threading
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period, self.samples, self.stop = period, [], threading.Event()
        self.thread = threading.Thread(target=self.run, daemon=True)

    def read(self):
        for f in self.files:
            try:
                for line in open(f):
                    if "*" in line:
                        return float(line.split(":")[1].strip().lower().rstrip("*").strip()
                                     .replace("mhz", "").strip())
            except (OSError, ValueError, IndexError):
                continue
        return None

    def run(self):
        while not self.stop.is_set():
            v = self.read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()

    def mean(self):
        return float(np.mean(self.samples)) if self.samples else None


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def gemv_bytes(N, K, M=1):
    """Algorithmic bytes of one GEMV: Q4_K weights once, the Q8 activation
    (codes + fp32 scale + int32 sum per 32 values), the fp32 output."""
    return N * K // 256 * 144 + M * K + M * (K // 32) * 8 + 4 * M * N


def fused_bytes(N, K, M=1):
    """Algorithmic bytes of one fused quantize+GEMV call: Q4_K weights once,
    the fp32 activation, the fp32 output (the Q8 codes never leave the CU)."""
    return N * K // 256 * 144 + 4 * M * K + 4 * M * N


def quant_bytes(K, M=1):
    """fp32 input read, Q8 codes + scales + sums written."""
    return 4 * M * K + M * K + M * (K // 32) * 8


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stream_gemv_decode_qwen3-4b_traffic.json")


def measured_traffic():
    """HBM bytes per launch of the decode GEMV, as the profiler counters
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size) read them for
    the kernel sources recorded beside them; None once those sources change."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_sources_sha256"):
        return None
    return rec["hbm_bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the secondary prefill-GEMM measurement")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the prefill GEMM measurement (with its parity check) and "
                         "print it")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the small-batch and routed-expert measurements")
    ap.add_argument("--prefill-group", choices=sorted(PREFILL_GROUPS),
                    help="only run 3 launches of one prefill launch group (for profiler "
                         "counter passes) and exit")
    ap.add_argument("--gemm-int8", action="store_true",
                    help="with --prefill-group: the GEMM's int8 contraction")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 10 times (known bytes, "
                         "to scale the HBM traffic counters of a profiler run) and exit")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration(torch):
    """A plain copy of known size: COPY_BYTES read and COPY_BYTES written per
    dispatch.  Profiler counters of this run give the scale of the same
    counters read on the GEMV kernels."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_dispatch": COPY_BYTES,
                                           "bytes_written_per_dispatch": COPY_BYTES,
                                           "dispatches": 10}}))


PREFILL_GROUPS = {"qkv": (0, 1, 2), "o": (3,), "gate_up": (4, 5), "down": (6,)}


def prefill_group(torch, q4k, qi, name, launches=3, int8=False):
    """Only `launches` launches of one prefill launch group (layer 0's weights,
    M = 512), for profiler counter passes; prints one line and exits.  int8:
    the GEMM's int8 contraction (libq4k_gemm_int8.so)."""
    L = q4k.lib_gemm_int8() if int8 else None
    dev = torch.device("cuda:0")
    idx = PREFILL_GROUPS[name]
    K = qi.QWEN3_4B_LAYER[idx[0]][1]
    probs = [(torch.from_numpy(qi.make_q4k_bytes(qi.QWEN3_4B_LAYER[p][2], K,
                                                 qi.weight_seed(2, 0, p))).to(dev),
              qi.QWEN3_4B_LAYER[p][2]) for p in idx]
    x = torch.from_numpy(qi.make_act(PREFILL_M, K, qi.act_seed(20000 + idx[0]))).to(dev)
    c, sc, su = q4k.q4k_quantize_act(x)
    for _ in range(launches):
        if len(probs) > 1:
            q4k.q4k_gemm_batch(probs, K, c, sc, su, library=L)
        else:
            q4k.q4k_gemm(probs[0][0], probs[0][1], K, c, sc, su, library=L)
    torch.cuda.synchronize()
    print(json.dumps({"prefill_group": {"name": name, "N": [N for _, N in probs], "K": K,
                                        "M": PREFILL_M, "launches": launches,
                                        "contraction": "int8" if int8 else "fp16"}}))


class Decode:
    """Inputs and graphs of the 36-layer decode sweep."""

    def __init__(self, torch, q4k, qi):
        self.torch, self.q4k, self.qi = torch, q4k, qi
        self.L = q4k.lib()
        dev = torch.device("cuda:0")
        self.shapes = qi.QWEN3_4B_LAYER
        self.weights, self.acts, self.host_w = [], [], {}
        call = 0
        for layer in range(LAYERS):
            for p, (name, K, N) in enumerate(self.shapes):
                w = qi.make_q4k_bytes(N, K, qi.weight_seed(1, layer, p))
                if layer == 0:
                    self.host_w[p] = w
                self.weights.append((torch.from_numpy(w).to(dev), N, K))
                self.acts.append(torch.from_numpy(qi.make_act(1, K, qi.act_seed(call))).to(dev))
                call += 1
        self.qbufs = [(torch.empty((1, K), dtype=torch.int8, device=dev),
                       torch.empty((1, K // 32), dtype=torch.float32, device=dev),
                       torch.empty((1, K // 32), dtype=torch.int32, device=dev))
                      for (_, N, K) in self.weights]
        self.ys = {N: torch.empty((1, N), dtype=torch.float32, device=dev)
                   for _, _, N in self.shapes}
        # one output per projection for the batched launches (products of one
        # launch must not share an output)
        self.yp = [torch.empty((1, N), dtype=torch.float32, device=dev)
                   for _, _, N in self.shapes]
        # per layer: {q, k, v}, {o}, {gate, up}, {down} -- same input width
        self.groups = [[l * len(self.shapes) + p for p in grp]
                       for l in range(LAYERS) for grp in ((0, 1, 2), (3,), (4, 5), (6,))]
        self.batches = []
        for grp in self.groups:
            arr = (q4k._lib.GemvProblem * len(grp))()
            for j, i in enumerate(grp):
                wt, N, K = self.weights[i]
                arr[j] = q4k._lib.GemvProblem(wt.data_ptr(), self.acts[i].data_ptr(),
                                              self.yp[i % len(self.shapes)].data_ptr(), N)
            self.batches.append((arr, len(grp), self.weights[grp[0]][2]))
        # residual stream of the decode step (the o and down outputs add into it)
        self.resid = torch.zeros((1, self.shapes[3][2]), dtype=torch.float32, device=dev)
        self.n_gemv = len(self.weights)
        self.n_batch = len(self.groups)
        self.bytes_gemv = sum(gemv_bytes(N, K) for _, N, K in self.weights)
        self.bytes_quant = sum(quant_bytes(K) for _, N, K in self.weights)
        self.bytes_fused = sum(fused_bytes(N, K) for _, N, K in self.weights)
        torch.cuda.synchronize()

    def quantize(self, i, s):
        _, N, K = self.weights[i]
        c, sc, su = self.qbufs[i]
        if self.L.q4k_quantize_act(self.acts[i].data_ptr(), 1, K, None, c.data_ptr(),
                                   sc.data_ptr(), su.data_ptr(), s):
            raise RuntimeError("q4k_quantize_act launch failed")

    def gemv(self, i, s):
        wt, N, K = self.weights[i]
        c, sc, su = self.qbufs[i]
        if self.L.q4k_gemv(wt.data_ptr(), N, K, c.data_ptr(), sc.data_ptr(), su.data_ptr(),
                           1, self.ys[N].data_ptr(), s):
            raise RuntimeError("q4k_gemv launch failed")

    def fused(self, i, s):
        wt, N, K = self.weights[i]
        if self.L.q4k_quantize_gemv(wt.data_ptr(), N, K, self.acts[i].data_ptr(), 1,
                                    self.ys[N].data_ptr(), s):
            raise RuntimeError("q4k_quantize_gemv launch failed")

    def batch(self, g, s):
        arr, n, K = self.batches[g]
        if self.L.q4k_quantize_gemv_batch(arr, n, K, 1, s):
            raise RuntimeError("q4k_quantize_gemv_batch launch failed")

    def batch_residual(self, g, s):
        """As batch(), with the single-product groups {o} and {down} adding
        into the residual stream in place (q4k_quantize_gemv_residual)."""
        arr, n, K = self.batches[g]
        if n != 1:
            return self.batch(g, s)
        wt, N, _ = self.weights[self.groups[g][0]]
        if self.L.q4k_quantize_gemv_residual(wt.data_ptr(), N, K,
                                             self.acts[self.groups[g][0]].data_ptr(), 1,
                                             self.resid.data_ptr(), self.resid.data_ptr(), s):
            raise RuntimeError("q4k_quantize_gemv_residual launch failed")

    def graph(self, fn, indices, stream):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            s = torch.cuda.current_stream().cuda_stream
            for i in indices:
                fn(i, s)
        return g

    def parity(self, oracle):
        """Layer 0's seven projections: Q8 codes bit-exact with the oracle, the
        batched launches and the fused call bit-identical to quantize + GEMV, and
        34 sampled outputs per projection within tolerance of the oracle."""
        torch, q4k = self.torch, self.q4k
        max_rel, checked = 0.0, 0
        s = torch.cuda.current_stream().cuda_stream
        for g in range(4):
            self.batch(g, s)
        torch.cuda.synchronize()
        for p, (name, K, N) in enumerate(self.shapes):
            wt = self.weights[p][0]
            c, sc, su = q4k.q4k_quantize_act(self.acts[p])
            y2 = q4k.q4k_gemv(wt, N, K, c, sc, su)
            y = q4k.q4k_quantize_gemv(wt, N, K, self.acts[p])
            torch.cuda.synchronize()
            if not torch.equal(y, y2):
                raise SystemExit("parity: fused and two-launch GEMV differ for %s" % name)
            if not torch.equal(y, self.yp[p]):
                raise SystemExit("parity: batched and single fused GEMV differ for %s" % name)
            if name in ("o", "down"):
                r = torch.from_numpy(self.qi.make_act(1, N, 77 + p)).to(y.device)
                yr = q4k.q4k_quantize_gemv_residual(wt, N, K, self.acts[p], r)
                if not torch.equal(yr, y + r):
                    raise SystemExit("parity: residual GEMV is not GEMV + residual for %s" % name)
            rc, rs, _ = oracle.quantize_act(self.acts[p].cpu().numpy())
            if not (c.cpu().numpy() == rc).all():
                raise SystemExit("parity: Q8 codes differ from the oracle for %s" % name)
            rows = np.unique(np.r_[0, N - 1, np.random.default_rng(p).integers(0, N, 32)])
            ref = oracle.matvec(self.host_w[p], N, K, rc, rs, rows=rows)[0]
            got = y.cpu().numpy()[0, rows].astype(np.float64)
            err = np.abs(got - ref)
            if (err > np.maximum(2e-3 * np.abs(ref), 1e-4)).any():
                raise SystemExit("parity: GEMV %s outside tolerance" % name)
            max_rel = max(max_rel, float((err / np.maximum(np.abs(ref), 0.05)).max()))
            checked += rows.size
        return {"rows_checked": checked, "max_rel_err": max_rel}


class Prefill:
    """Inputs of the prefill GEMM workload: M = 512 prompt tokens through the
    same seven projection shapes over 36 layers (distinct seeded weights)."""

    def __init__(self, torch, q4k, qi):
        self.torch, self.q4k = torch, q4k
        self.L = q4k.lib()
        dev = torch.device("cuda:0")
        self.shapes = qi.QWEN3_4B_LAYER
        self.weights, self.acts, self.host_w = [], [], {}
        M = PREFILL_M
        for layer in range(LAYERS):
            for p, (name, K, N) in enumerate(self.shapes):
                w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, layer, p))
                if layer == 0:
                    self.host_w[p] = w
                self.weights.append((torch.from_numpy(w).to(dev), N, K))
        # one N(0,1) 512 x K fp32 activation per projection shape, quantized
        # again by every call (the data does not change the work)
        self.act_of = {}
        for p, (name, K, N) in enumerate(self.shapes):
            self.act_of[p] = torch.from_numpy(qi.make_act(M, K, qi.act_seed(20000 + p))).to(dev)
        self.qbufs = {p: (torch.empty((M, K), dtype=torch.int8, device=dev),
                          torch.empty((M, K // 32), dtype=torch.float32, device=dev),
                          torch.empty((M, K // 32), dtype=torch.int32, device=dev))
                      for p, (_, K, N) in enumerate(self.shapes)}
        self.ys = {p: torch.empty((M, N), dtype=torch.float32, device=dev)
                   for p, (_, _, N) in enumerate(self.shapes)}
        self.n = len(self.weights)
        self.ops = sum(2 * M * N * K for _, N, K in self.weights)
        # the headline path: per layer one q4k_gemm_batch for {q,k,v} and for
        # {gate,up} (products sharing an activation), one q4k_gemm for o and down
        self.groups = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
        P = q4k._lib.GemmProblem
        self.batch_arr = {}
        for layer in range(LAYERS):
            for gi, (_, idx) in enumerate(self.groups):
                if len(idx) > 1:
                    base = layer * len(self.shapes)
                    self.batch_arr[(layer, gi)] = (P * len(idx))(*[
                        P(self.weights[base + p][0].data_ptr(), self.ys[p].data_ptr(),
                          self.weights[base + p][1]) for p in idx])
        self.units = LAYERS * len(self.groups)
        # split-tile workspace (counters zero once; every call leaves them zero)
        self.ws = q4k.gemm_workspace(dev)
        self.ws_args = (self.ws.data_ptr(), self.ws.numel())
        torch.cuda.synchronize()

    def quantize(self, i, s):
        p = i % len(self.shapes)
        _, N, K = self.weights[i]
        c, sc, su = self.qbufs[p]
        if self.L.q4k_quantize_act(self.act_of[p].data_ptr(), PREFILL_M, K, None, c.data_ptr(),
                                   sc.data_ptr(), su.data_ptr(), s):
            raise RuntimeError("q4k_quantize_act launch failed")

    def gemm(self, i, s):
        p = i % len(self.shapes)
        wt, N, K = self.weights[i]
        c, sc, su = self.qbufs[p]
        if self.L.q4k_gemm(wt.data_ptr(), N, K, c.data_ptr(), sc.data_ptr(), su.data_ptr(),
                           PREFILL_M, self.ys[p].data_ptr(), *self.ws_args, s):
            raise RuntimeError("q4k_gemm launch failed")

    def gemm_unit(self, u, s):
        """Launch unit u of the headline path: layer u // 4, group u % 4."""
        layer, gi = divmod(u, len(self.groups))
        idx = self.groups[gi][1]
        if len(idx) == 1:
            return self.gemm(layer * len(self.shapes) + idx[0], s)
        _, _, K = self.weights[layer * len(self.shapes) + idx[0]]
        c, sc, su = self.qbufs[idx[0]]
        if self.L.q4k_gemm_batch(self.batch_arr[(layer, gi)], len(idx), K, c.data_ptr(),
                                 sc.data_ptr(), su.data_ptr(), PREFILL_M, *self.ws_args, s):
            raise RuntimeError("q4k_gemm_batch launch failed")

    def parity(self, oracle, library=None):
        """Layer 0: every projection through q4k_gemm and through the batched
        launches of the headline path, 8 sampled weight rows x all 512
        activation rows each, against the oracle (library: the GEMM's int8
        contraction instead of the default)."""
        torch, q4k = self.torch, self.q4k
        max_rel, checked = 0.0, 0
        batched = {}
        for _, idx in self.groups:
            K = self.shapes[idx[0]][1]
            c, sc, su = q4k.q4k_quantize_act(self.act_of[idx[0]])
            ys = q4k.q4k_gemm_batch([(self.weights[p][0], self.shapes[p][2]) for p in idx],
                                    K, c, sc, su, library=library)
            batched.update(zip(idx, ys))
        for p, (name, K, N) in enumerate(self.shapes):
            wt = self.weights[p][0]
            src = self.act_of[p] if p not in (1, 2, 5) else self.act_of[{1: 0, 2: 0, 5: 4}[p]]
            c, sc, su = q4k.q4k_quantize_act(src)
            y = q4k.q4k_gemm(wt, N, K, c, sc, su, library=library)
            torch.cuda.synchronize()
            rc, rs, _ = oracle.quantize_act(src.cpu().numpy())
            rows = np.unique(np.r_[0, N - 1, np.random.default_rng(p).integers(0, N, 6)])
            ref = oracle.matvec(self.host_w[p], N, K, rc, rs, rows=rows)
            for out in (y, batched[p]):
                got = out.cpu().numpy()[:, rows].astype(np.float64)
                err = np.abs(got - ref)
                if (err > np.maximum(2e-3 * np.abs(ref), 1e-4)).any():
                    raise SystemExit("parity: GEMM %s outside tolerance" % name)
                max_rel = max(max_rel, float((err / np.maximum(np.abs(ref), 0.05)).max()))
                checked += ref.size
        return {"outputs_checked": checked, "max_rel_err": max_rel}


def prefill_int8(torch, q4k, pre, oracle, g_q, cap, steps):
    """The same 36-layer prefill step with the GEMM's int8 contraction
    (libq4k_gemm_int8.so: v_mfma_i32_32x32x32_i8, exact int32 sub-block dots,
    three fp32 vector ops per output and sub-block), checked against the oracle
    first, timed as the default."""
    pre.L = q4k.lib_gemm_int8()
    try:
        parity = pre.parity(oracle, library=pre.L)
        g8 = Decode.graph(pre, pre.gemm_unit, range(pre.units), cap)
        g_q.replay()
        g8.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g8.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
    finally:
        pre.L = q4k.lib()
    t = float(np.median(times))
    tops = pre.ops / t / 1e12
    return {"gemm_ms_per_step": round(t * 1e3, 3), "gemm_ms_per_step_dist": dist_ms(times),
            "TOPS": round(tops, 1), "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
            "parity": parity}


def measure_prefill(torch, q4k, qi, oracle, steps):
    pre = Prefill(torch, q4k, qi)
    parity = pre.parity(oracle)
    cap = torch.cuda.Stream()
    g_q = Decode.graph(pre, pre.quantize, range(pre.n), cap)
    g_g = Decode.graph(pre, pre.gemm_unit, range(pre.units), cap)
    g_q.replay(); g_g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for k in range(steps):
            g_q.replay()
            ev[k][0].record()
            g_g.replay()
            ev[k][1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_s = [a.elapsed_time(b) * 1e-3 for a, b in ev]
    gemm_s = float(np.median(step_s))
    per_group = {}
    for gi, (gname, idx) in enumerate(pre.groups):
        g = Decode.graph(pre, pre.gemm_unit, range(gi, pre.units, len(pre.groups)), cap)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        d = a.elapsed_time(b) * 1e-3 / LAYERS
        ops = sum(2 * PREFILL_M * pre.shapes[p][2] * pre.shapes[p][1] for p in idx)
        per_group[gname] = {"N": [pre.shapes[p][2] for p in idx], "K": pre.shapes[idx[0]][1],
                            "us": round(d * 1e6, 2), "TOPS": round(ops / d / 1e12, 1)}
    per_shape = {}
    for p, (name, K, N) in enumerate(pre.shapes):
        g = Decode.graph(pre, pre.gemm, range(p, pre.n, len(pre.shapes)), cap)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        d = a.elapsed_time(b) * 1e-3 / LAYERS
        per_shape[name] = {"N": N, "K": K, "us": round(d * 1e6, 2),
                           "TOPS": round(2 * PREFILL_M * N * K / d / 1e12, 1)}
    tops = pre.ops / gemm_s / 1e12
    sclk = clk.mean()
    # the matrix-core peak at the clock measured during the run (peaks scale
    # with the clock; the published figures are at 2400 MHz)
    clock_peak = None if sclk is None else {
        "sclk_mhz_mean": round(sclk, 1), "samples": len(clk.samples),
        "fp16_peak_TFLOPS": round(FP16_PEAK_TFLOPS * sclk / 2400.0, 1),
        "int8_peak_TOPS": round(INT8_PEAK_TOPS * sclk / 2400.0, 1),
        "frac_of_fp16_peak_at_clock": round(tops / (FP16_PEAK_TFLOPS * sclk / 2400.0), 4),
        "frac_of_int8_peak_at_clock": round(tops / (INT8_PEAK_TOPS * sclk / 2400.0), 4)}
    out = {"workload": "prefill GEMM, M=512 tokens x the seven Qwen3-4B projection shapes x "
                       "36 layers (3.72 T int ops per step); q4k_gemm_batch launches {q,k,v} "
                       "and {gate,up}, q4k_gemm o and down (4 launches per layer)",
           "steps": steps, "ms_per_step": round(elapsed / steps * 1e3, 3),
           "tok_per_s": round(PREFILL_M * steps / elapsed, 0),
           "gemm_ms_per_step": round(gemm_s * 1e3, 3),
           "gemm_ms_per_step_dist": dist_ms(step_s),
           "measured_clock_peak": clock_peak,
           # achieved: algorithmic Q4_K x Q8 ops (2*M*N*K) per second; the kernel
           # issues one fp16 matrix op per algorithmic one on integer-valued
           # operands, plus 3/16 as many bf16 ones for the min term
           "roofline": {"bound": "mfma", "kernel": "q4k gemm_kernel (fp16 matrix cores on "
                                                   "integer operands sc*q and codes, "
                                                   "deterministic split tiles)",
                        "achieved": round(tops, 1), "peak": FP16_PEAK_TFLOPS, "unit": "TOPS",
                        "frac": round(tops / FP16_PEAK_TFLOPS, 4),
                        "matrix_core_busy": round(tops * (1 + 3 / 16) / FP16_PEAK_TFLOPS, 4),
                        "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                        "mean_launch_us": round(gemm_s / pre.units * 1e6, 2),
                        "timing": "median over %d steps of HIP events around the %d GEMM "
                                  "launches of a step" % (steps, pre.units)},
           "per_group": per_group, "single_call_per_shape": per_shape, "parity": parity,
           "int8_contraction": prefill_int8(torch, q4k, pre, oracle, g_q, cap, steps),
           "matrix_vector_coissue": measure_coissue(torch, q4k)}
    del pre
    torch.cuda.empty_cache()
    return out


def measure_coissue(torch, q4k, iters=16384, reps=5):
    """Whether fp16 matrix-core ops and fp32 vector fmas from two waves of one
    SIMD overlap (q4k_ceiling_mfma_valu, one workgroup per CU): the time of
    the matrix-core waves alone, the vector waves alone (vrep rounds of 32
    fmas per 4 matrix ops) and both together; overlap = (alone sum - both) /
    the shorter alone time (1: fully concurrent, 0: one after the other)."""
    L = q4k.lib()
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def timed(vrep, what):
        if L.q4k_ceiling_mfma_valu(grid, iters, vrep, what, sink.data_ptr(), s):
            raise RuntimeError("q4k_ceiling_mfma_valu failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            L.q4k_ceiling_mfma_valu(grid, iters, vrep, what, sink.data_ptr(), s)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    mfma_ops = grid * 4 * iters * 4 * 32 * 32 * 16 * 2
    out = {"grid": grid, "matrix_op": "v_mfma_f32_32x32x16_f16", "iters": iters}
    t_m = timed(1, 1)
    out["matrix_alone_us"] = round(t_m * 1e6, 1)
    out["matrix_alone_TFLOPS"] = round(mfma_ops / t_m / 1e12, 1)
    for vrep in (1, 2):
        t_v = timed(vrep, 2)
        t_b = timed(vrep, 3)
        out["vrep_%d" % vrep] = {"vector_alone_us": round(t_v * 1e6, 1),
                                 "both_us": round(t_b * 1e6, 1),
                                 "overlap": round((t_m + t_v - t_b) / min(t_m, t_v), 3)}
    return out


ATTN_HEADS, ATTN_KV_HEADS, HEAD_DIM = 32, 8, 128


def attn_bytes(n_ctx, M=1):
    """Algorithmic bytes of one attention launch: the codes and scales of K and
    V over the context, the queries read and the outputs written."""
    return ATTN_KV_HEADS * n_ctx * (2 * HEAD_DIM + 8) + 2 * 4 * M * ATTN_HEADS * HEAD_DIM


def measure_attention(torch, q4k, qi, oracle, dec, ctxs=(1024, 16384), reps=5):
    """INT8-KV decode attention (q4k_kv_store + q4k_attn_decode), Qwen3-4B heads.

    For each context: one layer's cache written by q4k_kv_store from seeded fp32
    K/V and checked against the oracle (all 32 heads, fresh seeded query), then
    copied to as many layer caches as fill 600 MB (more than the 256 MB
    Infinity Cache), and a graph of one attention launch per layer cache timed
    between two events.  Then the decode token with attention at 1024
    positions: per layer the q|k|v GEMV, the cache store of the new k, v at
    position 1023, attention over 1024 positions into the o GEMV (with the
    residual add), gate|up and down."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    scale = HEAD_DIM ** -0.5
    out = {"heads": ATTN_HEADS, "kv_heads": ATTN_KV_HEADS, "head_dim": HEAD_DIM,
           "kv_format": "int8 codes + fp32 absmax scale per (layer, position, kv head)"}
    ws = q4k.attn_workspace(dev, q4k.q4k_attn_workspace_bytes(1, ATTN_HEADS, ATTN_KV_HEADS))
    wsb = ws.numel()
    cap_stream = torch.cuda.Stream()

    def caches(nl, n_ctx):
        return (torch.empty((nl, ATTN_KV_HEADS, n_ctx, HEAD_DIM), dtype=torch.int8, device=dev),
                torch.empty((nl, ATTN_KV_HEADS, n_ctx), dtype=torch.float32, device=dev),
                torch.empty((nl, ATTN_KV_HEADS, n_ctx, HEAD_DIM), dtype=torch.int8, device=dev),
                torch.empty((nl, ATTN_KV_HEADS, n_ctx), dtype=torch.float32, device=dev))

    def fill(c, n_ctx, seed):
        kc, ks, vc, vs = c
        k, v = qi.make_kv(n_ctx, ATTN_KV_HEADS, HEAD_DIM, seed)
        dk, dv = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
        for p0 in range(0, n_ctx, 4096):
            m = min(4096, n_ctx - p0)
            q4k.q4k_kv_store(dk[p0:p0 + m], dv[p0:p0 + m], p0, kc[0], ks[0], vc[0], vs[0])
        for l in range(1, kc.shape[0]):
            kc[l].copy_(kc[0]); ks[l].copy_(ks[0]); vc[l].copy_(vc[0]); vs[l].copy_(vs[0])
        torch.cuda.synchronize()
        return k, v

    def attn_call(c, l, n_ctx, q, o, s):
        kc, ks, vc, vs = c
        if L.q4k_attn_decode(q.data_ptr(), 1, ATTN_HEADS, ATTN_KV_HEADS, HEAD_DIM,
                             kc[l].data_ptr(), ks[l].data_ptr(), vc[l].data_ptr(),
                             vs[l].data_ptr(), n_ctx, n_ctx, scale, o.data_ptr(),
                             ws.data_ptr(), wsb, s):
            raise RuntimeError("q4k_attn_decode launch failed")

    legs = {}
    for n_ctx in ctxs:
        per = attn_bytes(n_ctx)
        nl = max(LAYERS, int(np.ceil(600e6 / per)))
        c = caches(nl, n_ctx)
        k, v = fill(c, n_ctx, qi.kv_seed(0))
        q = qi.make_query(1, ATTN_HEADS, HEAD_DIM, qi.query_seed(0))
        dq = torch.from_numpy(q).to(dev)
        got = q4k.q4k_attn_decode(dq, c[0][0], c[1][0], c[2][0], c[3][0], n_ctx, scale)
        torch.cuda.synchronize()
        kq, ksq = oracle.kv_quantize(k)
        vq, vsq = oracle.kv_quantize(v)
        ref = oracle.attn_int8kv(q, kq.transpose(1, 0, 2), ksq.T, vq.transpose(1, 0, 2), vsq.T,
                                 n_ctx, scale, parallel=True)
        g64 = got.cpu().numpy().astype(np.float64)
        err = np.abs(g64 - ref)
        if (err > np.maximum(2e-3 * np.abs(ref), 1e-4)).any():
            raise SystemExit("parity: attention at %d positions outside tolerance" % n_ctx)
        qs = torch.from_numpy(qi.make_query(nl, ATTN_HEADS, HEAD_DIM, qi.query_seed(1))).to(dev)
        os_ = torch.empty_like(qs)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            s = torch.cuda.current_stream().cuda_stream
            for l in range(nl):
                attn_call(c, l, n_ctx, qs[l], os_[l], s)
        torch.cuda.synchronize()
        g.replay()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / nl)
        t = float(np.median(times))
        legs[str(n_ctx)] = {
            "n_ctx": n_ctx, "layer_caches": nl, "bytes_per_launch": per,
            "us_per_launch": round(t * 1e6, 3), "us_dist": dist(np.array(times) * 1e6),
            "GBps": round(per / t / 1e9, 1), "hbm_frac": round(per / t / 1e9 / HBM_PEAK_GBS, 4),
            "us_per_token_36_layers": round(36 * t * 1e6, 2),
            "spot_check": {"outputs": int(ref.size),
                           "max_rel_err": float((err / np.maximum(np.abs(ref), 0.05)).max())}}
        del c, qs, os_, g
        torch.cuda.empty_cache()
    out["attention_only"] = legs

    # Decode token with attention over 1024 positions.
    n_ctx = 1024
    c = caches(LAYERS, n_ctx)
    fill(c, n_ctx, qi.kv_seed(0))
    att = torch.empty((1, ATTN_HEADS * HEAD_DIM), dtype=torch.float32, device=dev)
    q_, k_, v_ = dec.yp[0], dec.yp[1], dec.yp[2]
    nproj = len(dec.shapes)

    def token(l, s):
        dec.batch(4 * l, s)                                   # q | k | v
        kc, ks, vc, vs = c
        if L.q4k_kv_store(k_.data_ptr(), v_.data_ptr(), 1, ATTN_KV_HEADS, HEAD_DIM, n_ctx - 1,
                          n_ctx, kc[l].data_ptr(), ks[l].data_ptr(), vc[l].data_ptr(),
                          vs[l].data_ptr(), s):
            raise RuntimeError("q4k_kv_store launch failed")
        attn_call(c, l, n_ctx, q_, att, s)
        wt, N, K = dec.weights[l * nproj + 3]                 # o, from the attention output
        if L.q4k_quantize_gemv_residual(wt.data_ptr(), N, K, att.data_ptr(), 1,
                                        dec.resid.data_ptr(), dec.resid.data_ptr(), s):
            raise RuntimeError("q4k_quantize_gemv_residual launch failed")
        dec.batch(4 * l + 2, s)                               # gate | up
        dec.batch_residual(4 * l + 3, s)                      # down (+ residual)

    g = dec.graph(token, range(LAYERS), cap_stream)
    torch.cuda.synchronize()
    g.replay()
    times = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.median(times))
    tok_bytes = dec.bytes_fused + LAYERS * attn_bytes(n_ctx)
    out["decode_token_with_attention"] = {
        "n_ctx": n_ctx, "launches_per_token": 6 * LAYERS,
        "ms_per_token": round(t * 1e3, 4), "ms_dist": dist_ms(np.array(times)),
        "tok_per_s": round(1.0 / t, 1), "bytes_per_token": int(tok_bytes),
        "GBps": round(tok_bytes / t / 1e9, 1),
        "note": "per layer: q|k|v GEMV, kv store of the new k and v, attention over 1024 "
                "positions, o GEMV on the attention output with the residual add, gate|up, "
                "down with the residual add (norms and rotary embedding are not in scope)"}
    del c, g
    torch.cuda.empty_cache()
    return out


def measure_small_batch(torch, dec, oracle, steps=5):
    """Small-batch verification GEMV: M = 2, 4, 8 seeded N(0,1) activation rows
    against the 36-layer sweep's weights, through q4k_gemv (one launch per
    product, 252) and through q4k_gemm_batch per launch group ({q,k,v}, {o},
    {gate,up}, {down}: 144 launches; up to 8 rows it runs one of q4k_gemv's
    kernels over the whole group -- streaming at M = 2, the matrix-core GEMV
    from M = 3 where the group's rows favour it).  Only the products are timed (the Q8 rows are prepared
    once).  Before timing, layer 0's seven products through both paths are
    checked against the oracle on sampled weight rows (all M rows)."""
    import gemm_q4_super_amd as q4k
    L = dec.L
    dev = torch.device("cuda:0")
    out = {}
    cap = torch.cuda.Stream()
    for M in (2, 4, 8):
        host = {K: dec.qi.make_act(M, K, dec.qi.act_seed(30000 + 100 * M + K // 256))
                for K in sorted({K for _, _, K in dec.weights})}
        xs = {K: q4k.q4k_quantize_act(torch.from_numpy(x).to(dev)) for K, x in host.items()}
        ys = {N: torch.empty((M, N), dtype=torch.float32, device=dev)
              for N in {N for _, N, _ in dec.weights}}
        gws = q4k.gemm_workspace(dev)
        # spot check: layer 0, both paths, against the oracle
        worst, checked = 0.0, 0
        for p, (name, K, N) in enumerate(dec.shapes):
            wt = dec.weights[p][0]
            c, sc, su = xs[K]
            rc, rs, _ = oracle.quantize_act(host[K])
            if not (c.cpu().numpy() == rc).all():
                raise SystemExit("small batch: Q8 codes differ from the oracle (M=%d)" % M)
            rows = np.unique(np.r_[0, N - 1, np.random.default_rng(M * 7 + p).integers(0, N, 12)])
            ref = oracle.matvec(dec.host_w[p], N, K, rc, rs, rows=rows, parallel=True)
            for y in (q4k.q4k_gemv(wt, N, K, c, sc, su),
                      q4k.q4k_gemm_batch([(wt, N)], K, c, sc, su)[0]):
                got = y.cpu().numpy()[:, rows].astype(np.float64)
                err = np.abs(got - ref)
                if (err > np.maximum(2e-3 * np.abs(ref), 1e-4)).any():
                    raise SystemExit("small batch: %s M=%d outside tolerance" % (name, M))
                worst = max(worst, float((err / np.maximum(np.abs(ref), 0.05)).max()))
                checked += ref.size
        res = {"parity": {"outputs_checked": checked, "max_rel_err": worst}}
        # batched launches: products of one group write their own outputs
        yp = [torch.empty((M, N), dtype=torch.float32, device=dev) for _, _, N in dec.shapes]
        groups = []
        for grp in dec.groups:
            arr = (q4k._lib.GemmProblem * len(grp))()
            for j, i in enumerate(grp):
                wt, N, K = dec.weights[i]
                arr[j] = q4k._lib.GemmProblem(wt.data_ptr(), yp[i % len(dec.shapes)].data_ptr(), N)
            groups.append((arr, len(grp), dec.weights[grp[0]][2]))
        for path in ("gemv", "batched"):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                s = torch.cuda.current_stream().cuda_stream
                if path == "gemv":
                    for wt, N, K in dec.weights:
                        c, sc, su = xs[K]
                        if L.q4k_gemv(wt.data_ptr(), N, K, c.data_ptr(), sc.data_ptr(),
                                      su.data_ptr(), M, ys[N].data_ptr(), s):
                            raise RuntimeError("launch failed")
                else:
                    for arr, n, K in groups:
                        c, sc, su = xs[K]
                        if L.q4k_gemm_batch(arr, n, K, c.data_ptr(), sc.data_ptr(), su.data_ptr(),
                                            M, gws.data_ptr(), gws.numel(), s):
                            raise RuntimeError("launch failed")
            g.replay()
            ts = []
            for _ in range(steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                ts.append((a, b))
            torch.cuda.synchronize()
            ts = [a.elapsed_time(b) * 1e-3 for a, b in ts]
            t = float(np.median(ts))
            nbytes = sum(gemv_bytes(N, K, M) for _, N, K in dec.weights)
            ops = sum(2 * M * N * K for _, N, K in dec.weights)
            res[path] = {"us_per_sweep": round(t * 1e6, 1), "GBps": round(nbytes / t / 1e9, 1),
                         "TOPS": round(ops / t / 1e12, 2),
                         "calls": len(dec.weights) if path == "gemv" else len(groups),
                         "us_dist": {k: (round(v * 1e6, 1) if k != "passes" else v)
                                     for k, v in dist(ts).items()}}
        res["faster"] = min(("gemv", "batched"), key=lambda k: res[k]["us_per_sweep"])
        out["M=%d" % M] = res
    return out


def measure_ceilings(torch, q4k, dec, reps=5):
    """Practical per-launch ceilings of the decode step: a plain 16-byte stream
    read of each launch group's bytes (the fused GEMV's algorithmic bytes), 36
    launches on distinct regions of one 2.1 GB buffer per group (as the
    weights, nothing stays in the last-level cache), best of several grids;
    and an empty kernel's duration per launch (graph of 144)."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    groups = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    gbytes = {n: sum(fused_bytes(dec.shapes[p][2], dec.shapes[p][1]) for p in idx)
              for n, idx in groups}
    stride = max((b + 4095) // 4096 * 4096 for b in gbytes.values())
    buf = torch.ones(LAYERS * stride // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    cap = torch.cuda.Stream()

    def timed(fn, n_launch):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            s = torch.cuda.current_stream().cuda_stream
            for i in range(n_launch):
                if fn(i, s):
                    raise RuntimeError("ceiling launch failed")
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / (reps * n_launch)

    out = {}
    for name, _ in groups:
        nb = gbytes[name] // 16 * 16
        best = None
        for grid in (256, 512, 1024, 2048):
            t = timed(lambda i, s, grid=grid: L.q4k_ceiling_stream_read(
                buf.data_ptr() + i * stride, nb, grid, sink.data_ptr(), s), LAYERS)
            if best is None or t < best[0]:
                best = (t, grid)
        out[name] = {"bytes": nb, "us": round(best[0] * 1e6, 3),
                     "GBps": round(nb / best[0] / 1e9, 1), "grid": best[1]}
    empty = {}
    for grid in (1, 256, 1024):
        empty["grid_%d" % grid] = round(timed(lambda i, s, grid=grid: L.q4k_ceiling_empty(grid, s),
                                              4 * LAYERS) * 1e6, 3)
    del buf
    torch.cuda.empty_cache()
    return {"stream_read_per_launch_group": out, "empty_kernel_us_per_launch": empty}


def measure_shard(torch, q4k, dec, G=8, steps=20):
    """The decode sweep at one GPU's share of a G-way row shard (each GPU owns
    N/G complete Q4_K rows of every projection: q 2560->512, k and v ->128,
    o 4096->320, gate and up ->1216, down 9728->320 at G = 8): the first N/G
    rows of each of the sweep's 252 matrices (a prefix of its row-major
    bytes), the same activations and the same four batched launches per
    layer.  Checked first: every shard output equals the full launch's output
    for that row, bit for bit (a row's sum does not depend on the launch
    shape).  The shard's 36 layers (255 MB) about fill the 256 MB last-level
    cache, as they would on each of G GPUs."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    ys = [torch.empty((1, N // G), dtype=torch.float32, device=dev) for _, _, N in dec.shapes]
    batches, nbytes = [], 0
    for grp in dec.groups:
        arr = (q4k._lib.GemvProblem * len(grp))()
        for j, i in enumerate(grp):
            wt, N, K = dec.weights[i]
            arr[j] = q4k._lib.GemvProblem(wt.data_ptr(), dec.acts[i].data_ptr(),
                                          ys[i % len(dec.shapes)].data_ptr(), N // G)
            nbytes += fused_bytes(N // G, K)
        batches.append((arr, len(grp), dec.weights[grp[0]][2]))

    def launch(g, s):
        arr, n, K = batches[g]
        if L.q4k_quantize_gemv_batch(arr, n, K, 1, s):
            raise RuntimeError("q4k_quantize_gemv_batch launch failed")

    # layer 0: shard outputs against the full launches' first N/G outputs
    s = torch.cuda.current_stream().cuda_stream
    for g in range(4):
        dec.batch(g, s)
        launch(g, s)
    torch.cuda.synchronize()
    for p, (name, K, N) in enumerate(dec.shapes):
        if not torch.equal(ys[p], dec.yp[p][:, :N // G]):
            raise SystemExit("shard: %s differs from the full launch's rows" % name)
    cap = torch.cuda.Stream()
    g_all = dec.graph(launch, range(len(batches)), cap)
    g_all.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g_all.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.median(times))
    per_group = {}
    for gi, (gname, members) in enumerate((("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)),
                                           ("down", (6,)))):
        g = dec.graph(launch, range(gi, len(batches), 4), cap)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per_group[gname] = {"N": [dec.shapes[m][2] // G for m in members],
                            "us": round(a.elapsed_time(b) * 1e-3 / LAYERS * 1e6, 3)}
    return {"shards": G, "workload": "first N/%d rows of every projection of the 36-layer decode "
                                     "sweep, batch 1, fused Q8, 4 batched launches per layer" % G,
            "bytes_per_token": nbytes, "us_per_token": round(t * 1e6, 1),
            "us_dist": dist(np.array(times) * 1e6), "GBps": round(nbytes / t / 1e9, 1),
            "launches_per_token": len(batches), "per_group": per_group,
            "check": "every shard output bit-identical to the full launch's (layer 0)"}


def q6k_bytes(N, K, M=1):
    """Algorithmic bytes of one Q6_K GEMV: weights once (210 B per 256), the
    Q8 codes and scales it reads, the fp32 output."""
    return N * K // 256 * 210 + M * K + M * (K // 32) * 4 + 4 * M * N


def measure_large_launch(torch, q4k, qi, steps=5):
    """The decode GEMV kernel on one large launch, where the per-launch floor no
    longer dominates: a Q4_K matrix of an output head's shape (151936 x 2560,
    150 MB; three distinct copies rotated past the 256 MB last-level cache),
    q4k_quantize_gemv at batch 1 from an HIP graph."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    N, K = 151936, 2560
    ws = [torch.from_numpy(qi.make_q4k_bytes(N, K, qi.weight_seed(7, 0, i))).to(dev)
          for i in range(3)]
    x = torch.from_numpy(qi.make_act(1, K, qi.act_seed(70000))).to(dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        s = torch.cuda.current_stream().cuda_stream
        for i in range(3):
            if L.q4k_quantize_gemv(ws[i].data_ptr(), N, K, x.data_ptr(), 1, y.data_ptr(), s):
                raise RuntimeError("q4k_quantize_gemv launch failed")
    g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / steps / 3
    nb = fused_bytes(N, K)
    del ws
    torch.cuda.empty_cache()
    return {"workload": "one q4k_quantize_gemv launch, Q4_K 151936 x 2560 (150 MB), batch 1",
            "us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1),
            "hbm_frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)}


def measure_q6k(torch, q4k, qi, oracle, steps=5):
    """Q6_K decode GEMV (q6k_gemv, prepared Q8 rows, M = 1) over the 36-layer
    sweep's projection shapes with distinct seeded Q6_K matrices (2.98 GB):
    one graph of the 252 launches, replayed once untimed and `steps` times
    timed, plus a per-shape breakdown and a sampled check against the oracle;
    beside it the sweep with the quantizer inside, per product (252 launches)
    and batched per launch group (144, q6k_quantize_gemv_batch)."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    shapes = qi.QWEN3_4B_LAYER
    ws = [[torch.from_numpy(qi.make_q6k_bytes(N, K, qi.weight_seed(5, l, p))).to(dev)
           for l in range(LAYERS)] for p, (_, K, N) in enumerate(shapes)]
    acts = {}
    for K in sorted({K for _, K, _ in shapes}):
        x = qi.make_act(1, K, qi.act_seed(50000 + K))
        c, sc, _ = oracle.quantize_act(x)
        acts[K] = (torch.from_numpy(c).to(dev), torch.from_numpy(sc).to(dev), c, sc)
    ys = {N: torch.empty((1, N), dtype=torch.float32, device=dev) for _, _, N in shapes}
    cap = torch.cuda.Stream()

    def graph(ps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            s = torch.cuda.current_stream().cuda_stream
            for l in range(LAYERS):
                for p in ps:
                    _, K, N = shapes[p]
                    c, sc = acts[K][0], acts[K][1]
                    if L.q6k_gemv(ws[p][l].data_ptr(), N, K, c.data_ptr(), sc.data_ptr(), 1,
                                  ys[N].data_ptr(), s):
                        raise RuntimeError("q6k_gemv launch failed")
        return g

    def timed(g, reps):
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    t = timed(graph(range(len(shapes))), steps)
    nbytes = LAYERS * sum(q6k_bytes(N, K) for _, K, N in shapes)
    # the same sweep with the quantizer inside (q6k_quantize_gemv, fp32 rows)
    xs = {K: torch.from_numpy(qi.make_act(1, K, qi.act_seed(51000 + K))).to(dev)
          for K in sorted({K for _, K, _ in shapes})}
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf, stream=cap):
        s = torch.cuda.current_stream().cuda_stream
        for l in range(LAYERS):
            for p, (_, K, N) in enumerate(shapes):
                if L.q6k_quantize_gemv(ws[p][l].data_ptr(), N, K, xs[K].data_ptr(), 1,
                                       ys[N].data_ptr(), s):
                    raise RuntimeError("q6k_quantize_gemv launch failed")
    tf = timed(gf, steps)
    fbytes = LAYERS * sum(N * K // 256 * 210 + 4 * K + 4 * N for _, K, N in shapes)
    # ... and batched per launch group like the Q4_K headline ({q,k,v}, {o},
    # {gate,up}, {down}: 144 launches, q6k_quantize_gemv_batch), checked bit for
    # bit against q6k_quantize_gemv on layer 0 first
    P = q4k._lib.GemvProblem
    groups = ((0, 1, 2), (3,), (4, 5), (6,))
    yb = [torch.empty((1, N), dtype=torch.float32, device=dev) for _, _, N in shapes]
    def group_array(l, grp):
        return (P * len(grp))(*[P(ws[p][l].data_ptr(), xs[shapes[p][1]].data_ptr(),
                                  yb[p].data_ptr(), shapes[p][2]) for p in grp])
    barrs = [[(group_array(l, grp), len(grp), shapes[grp[0]][1]) for grp in groups]
             for l in range(LAYERS)]
    s0 = torch.cuda.current_stream().cuda_stream
    for arr, n, K in barrs[0]:
        if L.q6k_quantize_gemv_batch(arr, n, K, 1, s0):
            raise RuntimeError("q6k_quantize_gemv_batch launch failed")
    for p, (name, K, N) in enumerate(shapes):
        y1 = q4k.q6k_quantize_gemv(ws[p][0], N, K, xs[K])
        torch.cuda.synchronize()
        if not torch.equal(y1, yb[p]):
            raise RuntimeError("q6k_quantize_gemv_batch differs from q6k_quantize_gemv on %s" % name)
    gb = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gb, stream=cap):
        s = torch.cuda.current_stream().cuda_stream
        for l in range(LAYERS):
            for arr, n, K in barrs[l]:
                if L.q6k_quantize_gemv_batch(arr, n, K, 1, s):
                    raise RuntimeError("q6k_quantize_gemv_batch launch failed")
    tb = timed(gb, steps)
    per = {}
    for p, (name, K, N) in enumerate(shapes):
        d = timed(graph([p]), steps) / LAYERS
        per[name] = {"N": N, "K": K, "us": round(d * 1e6, 3),
                     "GBps": round(q6k_bytes(N, K) / d / 1e9, 1)}
    # sampled parity: layer 0 of each shape, 24 rows, against the oracle
    worst = 0.0
    for p, (name, K, N) in enumerate(shapes):
        c, sc = acts[K][0], acts[K][1]
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        if L.q6k_gemv(ws[p][0].data_ptr(), N, K, c.data_ptr(), sc.data_ptr(), 1, y.data_ptr(),
                      torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("q6k_gemv launch failed")
        torch.cuda.synchronize()
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(p).integers(0, N, 22)])
        ref = oracle.q6k_matvec(ws[p][0].cpu().numpy(), N, K, acts[K][2], acts[K][3], rows=rows)[0]
        got = y.cpu().numpy()[0, rows].astype(np.float64)
        err = np.abs(got - ref) / np.maximum(np.abs(ref), 0.05)
        if not (np.abs(got - ref) <= np.maximum(2e-3 * np.abs(ref), 1e-4)).all():
            raise RuntimeError("q6k_gemv parity failure on %s" % name)
        worst = max(worst, float(err.max()))
    del ws
    torch.cuda.empty_cache()
    # one large launch: a Q6_K output head (vocabulary 151936 x hidden 2560, 218 MB),
    # three distinct copies rotated so the 256 MB last-level cache cannot hold them
    NH, KH = 151936, 2560
    heads = [torch.from_numpy(qi.make_q6k_bytes(NH, KH, qi.weight_seed(6, 0, i))).to(dev)
             for i in range(3)]
    yh = torch.empty((1, NH), dtype=torch.float32, device=dev)
    gh = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gh, stream=cap):
        s = torch.cuda.current_stream().cuda_stream
        for i in range(3):
            if L.q6k_gemv(heads[i].data_ptr(), NH, KH, acts[KH][0].data_ptr(),
                          acts[KH][1].data_ptr(), 1, yh.data_ptr(), s):
                raise RuntimeError("q6k_gemv launch failed")
    th = timed(gh, steps) / 3
    hb = q6k_bytes(NH, KH)
    del heads
    torch.cuda.empty_cache()
    return {"workload": "Q6_K decode GEMV, batch 1, prepared Q8 rows: 36 layers x the seven "
                        "Qwen3-4B projection shapes in Q6_K (2.98 GB), one q6k_gemv per "
                        "product (252 launches)",
            "us_per_sweep": round(t * 1e6, 1), "GBps": round(nbytes / t / 1e9, 1),
            "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "mean_launch_us": round(t / (LAYERS * len(shapes)) * 1e6, 3),
            "fused_quantizer_sweep": {"us_per_sweep": round(tf * 1e6, 1),
                                      "GBps": round(fbytes / tf / 1e9, 1)},
            "fused_batched_sweep": {"launches": LAYERS * len(groups),
                                    "us_per_sweep": round(tb * 1e6, 1),
                                    "GBps": round(fbytes / tb / 1e9, 1),
                                    "hbm_frac": round(fbytes / tb / 1e9 / HBM_PEAK_GBS, 4),
                                    "bit_identical_to_single_calls": True},
            "per_shape": per,
            "output_head_151936x2560": {"us": round(th * 1e6, 2), "GBps": round(hb / th / 1e9, 1),
                                        "hbm_frac": round(hb / th / 1e9 / HBM_PEAK_GBS, 4)},
            "parity": {"rows_checked_per_shape": "24 sampled", "max_rel_err": worst}}


def measure_q6k_gemm(torch, q4k, qi, oracle, M=512, reps=20):
    """Q6_K prefill GEMM (q6k_gemm) on the seven Qwen3-4B projection shapes at
    M = 512, each launch timed in a graph of `reps` launches (median of 5),
    beside q4k_gemm on the same shapes and activations; every shape is first
    spot-checked against the oracle on sampled rows."""
    dev = torch.device("cuda:0")
    L = q4k.lib()
    ws = q4k.gemm_workspace(dev)
    cap = torch.cuda.Stream()
    out, tot = {}, {"q6k_us": 0.0, "q4k_us": 0.0, "flop": 0.0}
    for p, (name, K, N) in enumerate(qi.QWEN3_4B_LAYER):
        w6 = qi.make_q6k_bytes(N, K, qi.weight_seed(6, 0, p))
        w4 = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 0, p))
        x = qi.make_act(M, K, qi.act_seed(60000 + p))
        codes, scales, sums = oracle.quantize_act(x)
        d6, d4 = torch.from_numpy(w6).to(dev), torch.from_numpy(w4).to(dev)
        dc, dsc, dsu = (torch.from_numpy(a).to(dev) for a in (codes, scales, sums))
        y = q4k.q6k_gemm(d6, N, K, dc, dsc)
        torch.cuda.synchronize()
        rows = np.unique(np.r_[0, N - 1, np.random.default_rng(p).integers(0, N, 14)])
        ref = oracle.q6k_matvec(w6, N, K, codes, scales, rows=rows, parallel=True)
        got = y.cpu().numpy()[:, rows].astype(np.float64)
        if (np.abs(got - ref) > np.maximum(2e-3 * np.abs(ref), 1e-4)).any():
            raise SystemExit("parity: q6k_gemm %s outside tolerance" % name)
        yb = torch.empty((M, N), dtype=torch.float32, device=dev)

        def timed(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                s = torch.cuda.current_stream().cuda_stream
                for _ in range(reps):
                    fn(s)
            g.replay()
            per = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) * 1e-3 / reps)
            return float(np.median(per))

        def run6(s):
            if L.q6k_gemm(d6.data_ptr(), N, K, dc.data_ptr(), dsc.data_ptr(), M, yb.data_ptr(),
                          ws.data_ptr(), ws.numel(), s):
                raise RuntimeError("q6k_gemm launch failed")

        def run4(s):
            if L.q4k_gemm(d4.data_ptr(), N, K, dc.data_ptr(), dsc.data_ptr(), dsu.data_ptr(), M,
                          yb.data_ptr(), ws.data_ptr(), ws.numel(), s):
                raise RuntimeError("q4k_gemm launch failed")

        t6, t4 = timed(run6), timed(run4)
        flop = 2.0 * M * N * K
        out[name] = {"N": N, "K": K, "q6k_us": round(t6 * 1e6, 2),
                     "q6k_TOPS": round(flop / t6 / 1e12, 1), "q4k_us": round(t4 * 1e6, 2),
                     "q4k_TOPS": round(flop / t4 / 1e12, 1)}
        tot["q6k_us"] += t6 * 1e6
        tot["q4k_us"] += t4 * 1e6
        tot["flop"] += flop
    out["one_layer"] = {"q6k_us": round(tot["q6k_us"], 1),
                        "q6k_TOPS": round(tot["flop"] / tot["q6k_us"] / 1e6, 1),
                        "q4k_us": round(tot["q4k_us"], 1),
                        "q4k_TOPS": round(tot["flop"] / tot["q4k_us"] / 1e6, 1)}
    out["M"] = M
    out["note"] = ("Q6_K: 4 fp16 matrix-core ops per 32-element block (two exact weight parts) "
                   "and no min term, against Q4_K's 2 plus the 3-part min term per super-block")
    return out


def measure_moe(torch, q4k, qi, oracle, steps=5, layers=8, Ts=(1, 16)):
    """Routed-expert FFN layer (64 experts, hidden 2048, FFN 1024, top-8) over
    `layers` distinct seeded layers per pass (1.81 GB, past the last-level
    cache), for each T in Ts: q4k_moe_ffn (the reported time), and the six-call
    chain quantize -> grouped gate GEMV -> grouped up GEMV -> SwiGLU + Q8 ->
    grouped down GEMV with the routing-weighted sum, whose output the fused
    layer must equal bit for bit."""
    L = q4k.lib()
    dev = torch.device("cuda:0")
    E, H, F, TOPK = qi.MOE_EXPERTS, qi.MOE_HIDDEN, qi.MOE_FFN, qi.MOE_TOPK
    sgu, sdn = F * (H // 256) * 144, H * (F // 256) * 144
    W, W_host = [], []
    for l in range(layers):
        host = tuple(np.concatenate(
            [qi.make_q4k_bytes(*((F, H) if k < 2 else (H, F)), qi.expert_seed(l, e, k))
             for e in range(E)]) for k in range(3))
        if l == 0:
            W_host.append(host)
        W.append(tuple(torch.from_numpy(h).to(dev) for h in host))
    out = {}
    cap = torch.cuda.Stream()
    for T in Ts:
        P = T * TOPK
        routes = [qi.make_routing(T, E, TOPK, qi.routing_seed(100 * T + l)) for l in range(layers)]
        ids = [torch.from_numpy(r[0]).to(dev) for r in routes]
        rws = [torch.from_numpy(r[1]).to(dev) for r in routes]
        x = torch.from_numpy(qi.make_act(T, H, qi.act_seed(70000 + T))).to(dev)
        xq = q4k.q4k_quantize_act(x)
        g = torch.empty((P, F), dtype=torch.float32, device=dev)
        u = torch.empty((P, F), dtype=torch.float32, device=dev)
        hq = (torch.empty((P, F), dtype=torch.int8, device=dev),
              torch.empty((P, F // 32), dtype=torch.float32, device=dev),
              torch.empty((P, F // 32), dtype=torch.int32, device=dev))
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws_gu = torch.zeros(q4k.q4k_moe_workspace_bytes(T, TOPK, E, F), dtype=torch.uint8,
                            device=dev)
        ws_dn = torch.zeros(q4k.q4k_moe_workspace_bytes(T, TOPK, E, H), dtype=torch.uint8,
                            device=dev)

        def layer(l, s):
            wg, wu, wd = W[l]
            c, sc, su = xq
            st = L.q4k_quantize_act(x.data_ptr(), T, H, None, c.data_ptr(), sc.data_ptr(),
                                    su.data_ptr(), s)
            for wt, dst in ((wg, g), (wu, u)):
                st |= L.q4k_moe_gemv(wt.data_ptr(), E, sgu, F, H, ids[l].data_ptr(), None, T,
                                     TOPK, c.data_ptr(), sc.data_ptr(), su.data_ptr(), 0,
                                     dst.data_ptr(), ws_gu.data_ptr(), ws_gu.numel(), s)
            st |= L.q4k_quantize_act(u.data_ptr(), P, F, g.data_ptr(), hq[0].data_ptr(),
                                     hq[1].data_ptr(), hq[2].data_ptr(), s)
            st |= L.q4k_moe_gemv(wd.data_ptr(), E, sdn, H, F, ids[l].data_ptr(),
                                 rws[l].data_ptr(), T, TOPK, hq[0].data_ptr(), hq[1].data_ptr(),
                                 hq[2].data_ptr(), 1, y.data_ptr(), ws_dn.data_ptr(),
                                 ws_dn.numel(), s)
            if st:
                raise RuntimeError("launch failed")

        ws_ffn = torch.zeros(q4k.q4k_moe_ffn_workspace_bytes(T, TOPK, E, H, F),
                             dtype=torch.uint8, device=dev)
        y2 = torch.empty_like(y)

        def fused(l, s):
            wg, wu, wd = W[l]
            if L.q4k_moe_ffn(wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), E, sgu, sdn, H, F,
                             ids[l].data_ptr(), rws[l].data_ptr(), T, TOPK, x.data_ptr(),
                             y2.data_ptr(), ws_ffn.data_ptr(), ws_ffn.numel(), s):
                raise RuntimeError("launch failed")

        def timed(fn):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                s = torch.cuda.current_stream().cuda_stream
                for l in range(layers):
                    fn(l, s)
            gr.replay()
            per = []
            for _ in range(5):   # median of 5 timings of `steps` replays
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(steps):
                    gr.replay()
                b.record()
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) * 1e-3 / (steps * layers))
            return float(np.median(per))

        # spot check before timing: layer 0 through q4k_moe_ffn against the
        # oracle layer (codes of h may differ by one next to a rounding
        # boundary, so a few outputs may exceed the bar by what such a flip
        # moves them; the exact flip-aware bound is checked by the tests)
        fused(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(W_host[0][0], W_host[0][1], W_host[0][2], E, H, F, routes[0][0],
                               routes[0][1], x.cpu().numpy(), parallel=True)["y"]
        got = y2.cpu().numpy().astype(np.float64)
        bar = np.maximum(2e-3 * np.abs(ref), 1e-4)
        over = np.abs(got - ref) / bar
        if (over > 1).mean() > 0.01 or over.max() > 20:
            raise SystemExit("moe: T=%d layer outside the spot-check bound" % T)
        spot = {"outputs_checked": int(ref.size), "outputs_over_bar": int((over > 1).sum()),
                "max_err_over_bar": round(float(over.max()), 3),
                "max_rel_err": float((np.abs(got - ref) / np.maximum(np.abs(ref), 0.05)).max())}
        t_chain = timed(layer)
        t = timed(fused)
        same = bool(torch.equal(y.view(torch.int32), y2.view(torch.int32)))
        distinct = np.mean([len(np.unique(r[0])) for r in routes])
        nbytes = distinct * 3 * F * H // 256 * 144
        out["T=%d" % T] = {"us_per_layer": round(t * 1e6, 2),
                           "distinct_experts": float(distinct),
                           "expert_MB_per_layer": round(nbytes / 1e6, 2),
                           "GBps": round(nbytes / t / 1e9, 1),
                           "path": "q4k_moe_ffn (%d launches)" % (2 if T <= 2 else 4),
                           "six_call_chain_us_per_layer": round(t_chain * 1e6, 2),
                           "fused_equals_chain_bitwise": same, "oracle_spot_check": spot}
    del W
    torch.cuda.empty_cache()
    return out


def cpu_baselines(qi, oracle, seconds):
    """The oracle as it stands (plain C, fp64 products), timed on this host:
    single-threaded and with OpenMP over output rows on all cores (the same
    arithmetic), each on a bounded sample of a workload.  Returns the decode
    figure (the headline's unit, all cores) and one entry per workload."""
    shapes = qi.QWEN3_4B_LAYER
    threads = oracle.threads(True)
    info = dict(cpu_info(), omp_threads=threads)

    def decode(parallel, budget):
        t_cpu, nbytes, done = 0.0, 0, 0
        for layer in range(LAYERS):
            for p, (name, K, N) in enumerate(shapes):
                w = qi.make_q4k_bytes(N, K, qi.weight_seed(1, layer, p))
                x = qi.make_act(1, K, qi.act_seed(layer * len(shapes) + p))
                ta = time.perf_counter()
                rc, rs, _ = oracle.quantize_act(x)
                oracle.matvec(w, N, K, rc, rs, parallel=parallel)
                t_cpu += time.perf_counter() - ta
                nbytes += gemv_bytes(N, K) + quant_bytes(K)
            done += 1
            if t_cpu >= budget:
                break
        return {"GBps": round(nbytes / t_cpu / 1e9, 4), "seconds": round(t_cpu, 2),
                "sample": "layers 0..%d of the 36-layer decode sweep (%d quantize+GEMV calls, "
                          "%.2f GB)" % (done - 1, done * len(shapes), nbytes / 1e9)}

    def prefill(parallel, rows_per_proj):
        t_cpu = 0.0
        step_est = 0.0
        for p, (name, K, N) in enumerate(shapes):
            w = qi.make_q4k_bytes(N, K, qi.weight_seed(2, 0, p))
            x = qi.make_act(PREFILL_M, K, qi.act_seed(20000 + p))
            rows = np.arange(min(rows_per_proj, N))
            ta = time.perf_counter()
            rc, rs, _ = oracle.quantize_act(x)
            oracle.matvec(w, N, K, rc, rs, rows=rows, parallel=parallel)
            dt = time.perf_counter() - ta
            t_cpu += dt
            step_est += dt * N / rows.size
        step_est *= LAYERS
        ops = sum(2 * PREFILL_M * N * K for _, K, N in shapes) * LAYERS
        return {"TOPS": round(ops / step_est / 1e12, 6), "ms_per_step_extrapolated":
                round(step_est * 1e3, 1), "seconds": round(t_cpu, 2),
                "sample": "%d weight rows of each of layer 0's seven projections x 512 "
                          "activation rows; scaled to all rows and 36 layers (extrapolated)"
                          % rows_per_proj}

    def small(M, parallel, rows_per_proj):
        t_cpu, nbytes, est = 0.0, 0, 0.0
        for p, (name, K, N) in enumerate(shapes):
            w = qi.make_q4k_bytes(N, K, qi.weight_seed(1, 0, p))
            x = qi.make_act(M, K, qi.act_seed(30000 + 100 * M + K // 256))
            rows = np.arange(min(rows_per_proj, N))
            ta = time.perf_counter()
            rc, rs, _ = oracle.quantize_act(x)
            oracle.matvec(w, N, K, rc, rs, rows=rows, parallel=parallel)
            dt = time.perf_counter() - ta
            t_cpu += dt
            est += dt * N / rows.size
            nbytes += gemv_bytes(N, K, M)
        return {"GBps": round(nbytes / est / 1e9, 4), "seconds": round(t_cpu, 2),
                "sample": "%s weight rows of each of layer 0's seven projections, M = %d"
                          % ("all" if rows_per_proj >= 9728 else str(rows_per_proj), M)}

    def moe(T, parallel):
        E, H, F, TOPK = qi.MOE_EXPERTS, qi.MOE_HIDDEN, qi.MOE_FFN, qi.MOE_TOPK
        ids, rw = qi.make_routing(T, E, TOPK, qi.routing_seed(100 * T))
        touched = np.unique(ids)
        # only the touched experts' matrices are needed; untouched ones stay zero
        wg = np.zeros(E * F * (H // 256) * 144, np.uint8)
        wu, wd = np.zeros_like(wg), np.zeros(E * H * (F // 256) * 144, np.uint8)
        sgu, sdn = F * (H // 256) * 144, H * (F // 256) * 144
        for e in touched:
            wg[e * sgu:(e + 1) * sgu] = qi.make_q4k_bytes(F, H, qi.expert_seed(0, e, 0)).ravel()
            wu[e * sgu:(e + 1) * sgu] = qi.make_q4k_bytes(F, H, qi.expert_seed(0, e, 1)).ravel()
            wd[e * sdn:(e + 1) * sdn] = qi.make_q4k_bytes(H, F, qi.expert_seed(0, e, 2)).ravel()
        x = qi.make_act(T, H, qi.act_seed(70000 + T))
        ta = time.perf_counter()
        oracle.moe_layer(wg, wu, wd, E, H, F, ids, rw, x, parallel=parallel)
        dt = time.perf_counter() - ta
        nbytes = len(touched) * (sgu * 2 + sdn)
        return {"us_per_layer": round(dt * 1e6, 1), "GBps": round(nbytes / dt / 1e9, 4),
                "distinct_experts": int(len(touched))}

    budget = max(seconds / 3.0, 1.0)
    dec1, decN = decode(False, budget), decode(True, budget / 2)
    out = {
        "host": info,
        "decode": {"1_thread": dec1, "all_cores": decN},
        "prefill": {"1_thread": prefill(False, 48), "all_cores": prefill(True, 96 * threads)},
        "small_batch": {"M=%d" % M: {"1_thread": small(M, False, 768),
                                     "all_cores": small(M, True, 9728)}
                        for M in (2, 4, 8)},
        "moe_layer": {"T=1": {"1_thread": moe(1, False), "all_cores": moe(1, True)},
                      "T=16": {"all_cores": moe(16, True)}},
    }
    headline = {"value": decN["GBps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": decN["sample"] + ", OpenMP over output rows on all host cores",
                "single_thread": {"value": dec1["GBps"], "cores": 1, "sample": dec1["sample"]},
                "cpu_model": info["cpu_model"]}
    return headline, out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import gemm_q4_super_amd as q4k
    import q4k_inputs as qi
    if args.prefill_group:
        prefill_group(torch, q4k, qi, args.prefill_group, int8=args.gemm_int8)
        return
    import oracle

    oracle.build(force=False)
    if args.prefill_only:
        print(json.dumps({"prefill_gemm": measure_prefill(torch, q4k, qi, oracle,
                                                          args.prefill_steps)}))
        return
    dec = Decode(torch, q4k, qi)
    parity = dec.parity(oracle)

    steps, warmup = args.steps, args.warmup
    cap = torch.cuda.Stream()
    idx = range(dec.n_gemv)
    g_batch = dec.graph(dec.batch, range(dec.n_batch), cap)
    torch.cuda.synchronize()
    for _ in range(warmup):
        g_batch.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]

    # ------------------------------------------------------------ timed
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record()
        g_batch.replay()
        ev[k][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # ------------------------------------------------------------------

    block_s = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    mean_launch_s = float(block_s.mean()) / dec.n_batch

    def timed(g, reps=5):
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    # The same sweep as one fused launch per product, and as two launches per
    # product (quantize, then GEMV).
    t_single = timed(dec.graph(dec.fused, idx, cap))
    single = {"ms_per_step": round(t_single * 1e3, 4),
              "GBps": round(dec.bytes_fused / t_single / 1e9, 1),
              "launches": dec.n_gemv,
              "mean_launch_us": round(t_single / dec.n_gemv * 1e6, 3)}
    t_q2 = timed(dec.graph(dec.quantize, idx, cap))
    t_g2 = timed(dec.graph(dec.gemv, idx, cap))
    two_step = {"ms_per_step": round((t_q2 + t_g2) * 1e3, 4),
                "quantize_ms": round(t_q2 * 1e3, 4), "gemv_ms": round(t_g2 * 1e3, 4),
                "GBps": round((dec.bytes_gemv + dec.bytes_quant) / (t_q2 + t_g2) / 1e9, 1),
                "gemv_mean_launch_us": round(t_g2 / dec.n_gemv * 1e6, 3)}

    # Per-launch-group breakdown, outside the timed region: a graph of the 36
    # launches of one group, replayed 5 times between two events.
    per_group = {}
    for gi, gname in enumerate(("qkv", "o", "gate_up", "down")):
        d = timed(dec.graph(dec.batch, range(gi, dec.n_batch, 4), cap)) / LAYERS
        members = dec.groups[gi]
        nb = sum(fused_bytes(dec.weights[i][1], dec.weights[i][2]) for i in members)
        per_group[gname] = {"N": [dec.weights[i][1] for i in members],
                            "K": dec.weights[members[0]][2], "us": round(d * 1e6, 3),
                            "GBps": round(nb / d / 1e9, 1)}

    # The same step with the residual add of o and down inside their GEMVs
    # (4 launches per layer as above; N more fp32 reads per o / down launch).
    residual = None
    if not args.no_extra:
        t_res = timed(dec.graph(dec.batch_residual, range(dec.n_batch), cap))
        t_plain = timed(dec.graph(dec.batch, range(dec.n_batch), cap))
        residual = {"ms_per_step": round(t_res * 1e3, 4),
                    "same_graph_without_residual_ms": round(t_plain * 1e3, 4),
                    "launches": dec.n_batch,
                    "residual_launches": 2 * LAYERS}

    value = dec.bytes_fused * steps / elapsed / 1e9
    bytes_per_launch = dec.bytes_fused / dec.n_batch
    achieved = bytes_per_launch / mean_launch_s / 1e9
    n_launch = dec.n_batch
    small = None if args.no_extra else measure_small_batch(torch, dec, oracle)
    ceilings = None if args.no_extra else measure_ceilings(torch, q4k, dec)
    shard = None if args.no_extra else measure_shard(torch, q4k, dec)
    attention = None if args.no_extra else measure_attention(torch, q4k, qi, oracle, dec)
    del g_batch, dec
    torch.cuda.empty_cache()
    prefill = None if args.no_prefill else measure_prefill(torch, q4k, qi, oracle,
                                                           args.prefill_steps)
    moe = None if args.no_extra else measure_moe(torch, q4k, qi, oracle)
    q6k = None if args.no_extra else measure_q6k(torch, q4k, qi, oracle)
    q6k_gemm = None if args.no_extra else measure_q6k_gemm(torch, q4k, qi, oracle)
    large = None if args.no_extra else measure_large_launch(torch, q4k, qi)
    cpu, cpu_all = (None, None) if args.no_cpu else cpu_baselines(qi, oracle, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "step_ms_dist": dist_ms(block_s),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k x q8 (int8 dot4, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "decode GEMV sweep, batch 1: 36 Qwen3-4B-shaped layers x "
                               "(q 2560->4096, k 2560->1024, v 2560->1024, o 4096->2560, "
                               "gate 2560->9728, up 2560->9728, down 9728->2560), 2.04 GB of "
                               "Q4_K weights, Q8 quantization of a fresh N(0,1) row per "
                               "product inside the GEMV; q4k_quantize_gemv_batch launches "
                               "{q,k,v}, {o}, {gate,up}, {down} per layer",
                   "layers": LAYERS, "batch": 1,
                   "tok_per_s": round(steps / elapsed, 1),
                   "hbm_frac_whole_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "q4k stream_gemv_kernel (M=1, fused Q8, batched)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch (profiler counters)",
                     "mean_launch_us": round(mean_launch_s * 1e6, 3),
                     "bytes_per_launch": round(bytes_per_launch),
                     "launches_per_step": n_launch,
                     "timing": "HIP events on the launch stream around the %d back-to-back "
                               "dispatches of each timed step (dispatch gaps included)"
                               % n_launch,
                     "per_group": per_group},
        "single_call_path": single,
        "residual_epilogue_path": residual,
        "two_launch_path": two_step,
        "cpu_baseline": cpu,
        "cpu_baselines": cpu_all,
        "decode_ceilings": ceilings,
        "decode_one_gpu_share_of_8": shard,
        "parity": parity,
        "prefill_gemm": prefill,
        "small_batch_gemv": small,
        "int8_kv_attention": attention,
        "moe_layer": moe,
        "q6k_decode_gemv": q6k,
        "q6k_prefill_gemm": q6k_gemm,
        "decode_gemv_one_large_launch": large,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
