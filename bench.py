"""Benchmark of the quantized prefill GEMM path on one MI355X.

One step = one launch of the hot path over the measured workload, with inputs
already resident in HBM.  The headline workload is the 1B-shape MLP
up-projection prefill (Q4_0 weights [8192, 2048], X fp16 [2048, 2048]); the
line reports TFLOP/s (2*M*N*K per second) with its fraction of the fp16 dense
MFMA peak.  The other workloads (MLX4 fused SwiGLU and GeGLU, the Q2_0, Q8_0,
Q4_K, MLX4-G32 and ternary GEMMs, the direct-head projection, the M=1 / M=64
GEMVs and the Q8_0-KV attention) are timed the same way under "secondary",
each with its own roofline.

Cold caches: every timed launch uses one of R rotated copies of weights, X and
Y (R copies together exceed the 256 MB Infinity Cache), in the spirit of the
pages' cache flush before every measured run.  Timing: torch.cuda.Event on the
stream the kernels are launched on, bracketing all K launches, after W warmup
launches; ms_per_step is the mean launch duration.

read_ceiling (decode lines): the library's plain streaming-read kernel timed the
same way over the same number of bytes -- what one read-only kernel sustains
at that size on this device, beside the GEMV's fraction of 8 TB/s.

parity: every line's output (the last timed launch) is compared with the fp64
oracle on sampled rows x columns, first and last included; the headline is
also compared on every row the CPU baseline computes.

cpu_baseline: the fp64 oracle (tests' reference implementation) timed on a
bounded sample of the same workload -- exact decode of all of W, then the
first rows of X against it -- on the host's cores, decode and matmul timed
apart; the GPU output is checked against it on the same rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu] [--no-secondary] [--rotate R]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
MALL_BYTES = 256 << 20
HEADLINE = "q4_0_prefill_2048x2048x8192"
SECONDARY = ["q4_0_tiny_16x256x256", "mlx4_swiglu_2048x4096x14336", "q2_0_prefill_2048x4096x4096",
             "q4_0_gemv_1x4096x14336", "q4_0_gemv_64x4096x14336", "q8_0_prefill_2048x2048x8192",
             "mlx4_geglu_2048x4096x14336", "q4_0_qproj_heads_2048x4096x4096", "mlx4_g32_prefill_2048x2048x8192",
             "q4_k_prefill_2048x2048x8192", "q4_k_gemv_1x4096x14336",
             "ternary_prefill_2048x2048x8192", "ternary_gemv_1x4096x14336",
             "ternary_q2_prefill_2048x2048x8192", "ternary_q2_gemv_1x4096x14336"]
# sources whose change invalidates counter-derived traffic figures: the kernels
# and everything that decides which kernel runs with which launch shape
KERNEL_SOURCES = ["gemm.hip", "gemv.hip", "api.hip", "launch.h", "dispatch.h", "kutil.h", "unpack.h", "planar.h",
                  "lds_dma.h"]
ATTN_SOURCES = ["attention.hip", "api.hip", "launch.h", "unpack.h"]


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    """Hash of the kernel sources' code: comments and blank lines are left out,
    so a counter summary stays valid across edits of comments only."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_prefill_gemm_codec_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def bound_of(wl) -> str:
    return "hbm" if wl.op == "gemv" else "mfma"


class Prepared:
    """R rotated device copies of one workload's packed weights, X and Y."""

    def __init__(self, torch, qg, wl, rotate=None):
        self.wl = wl
        x = wl.x()
        self.x_host = x
        self.canon = wl.weights()
        planes = [qg.qg_pack_host(wl.codec, wl.n, wl.k, c) for c in self.canon]
        per_set = sum(qs.size + sc.size for qs, sc in planes) + x.nbytes + 2 * wl.m * wl.n
        if rotate is None:
            rotate = max(2, min(16, -(-(MALL_BYTES + (32 << 20)) // per_set) + 1))
        self.rotate = rotate
        self.sets = []
        for _ in range(rotate):
            ws = [qg.QWeight(wl.codec, wl.n, wl.k, torch.from_numpy(qs).cuda(), torch.from_numpy(sc).cuda())
                  for qs, sc in planes]
            xd = torch.from_numpy(x).cuda()
            ldy = 8 * ((wl.n + 7) // 8)
            y = torch.empty((wl.m, ldy), dtype=torch.float16, device="cuda")
            self.sets.append((ws, xd, y, ldy))
        self.qg = qg
        # The timed loop calls the C-ABI entry points with argument tuples built
        # once (same functions the binding wraps), so launches outpace the GPU.
        L = qg.lib()
        stream = qg._stream(None)
        self.calls = []
        for ws, xd, y, ldy in self.sets:
            if wl.op in synth.GATED:
                fn = L.qgemm_swiglu if wl.op == "swiglu" else L.qgemm_geglu
                self.calls.append((fn, (ws[0].desc, ws[1].desc, xd.data_ptr(), wl.m, wl.k,
                                                    y.data_ptr(), ldy, stream)))
            elif wl.op == "heads":
                self.calls.append((L.qgemm_prefill_heads, (ws[0].desc, xd.data_ptr(), wl.m, wl.k, y.data_ptr(),
                                                           wl.head_dim, stream)))
            elif wl.op == "gemv":
                self.calls.append((L.qgemv_decode, (ws[0].desc, xd.data_ptr(), wl.m, wl.k, y.data_ptr(), ldy, stream)))
            else:
                self.calls.append((L.qgemm_prefill, (ws[0].desc, xd.data_ptr(), wl.m, wl.k, y.data_ptr(), ldy, stream)))

    def launch(self, i):
        fn, args = self.calls[i % self.rotate]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{fn.__name__} returned status {st}")
        self.last = i % self.rotate
        return self.sets[self.last][2][:, :self.wl.n]

    def last_out(self):
        """Output buffer of the most recent launch ([M, N] rows; head-major data for 'heads')."""
        y = self.sets[getattr(self, "last", 0)][2]
        return y if self.wl.op == "heads" else y[:, :self.wl.n]


class ReadPrepared:
    """R rotated device buffers of `nbytes` (rounded up to 16) for the library's
    streaming-read calibration kernel: the best a single plain read of the
    same byte count achieves on this device, measured like the GEMV beside it."""

    def __init__(self, torch, qg, nbytes, rotate):
        nbytes = -(-nbytes // 16) * 16
        self.nbytes = nbytes
        self.rotate = rotate
        self.bufs = [torch.full((nbytes // 4,), r + 1, dtype=torch.int32, device="cuda") for r in range(rotate)]
        self.acc = torch.zeros(qg.QG_STREAM_READ_SLOTS, dtype=torch.int32, device="cuda")
        L = qg.lib()
        stream = qg._stream(None)
        self.calls = [(L.qg_stream_read, (b.data_ptr(), nbytes, self.acc.data_ptr(), stream)) for b in self.bufs]

    def launch(self, i):
        fn, args = self.calls[i % self.rotate]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"qg_stream_read returned status {st}")


def read_ceiling(torch, qg, wl, rotate, steps, warmup, settle_ms, gemv_ms):
    """Streaming-read rate for the GEMV's algorithmic bytes, and the GEMV's
    share of it (context for the HBM roofline fraction: at a few tens of MB a
    single kernel's launch ramp and drain keep any read well below 8 TB/s)."""
    rp = ReadPrepared(torch, qg, wl.algorithmic_bytes(), rotate)
    ms, _ = time_launches(torch, rp, steps, warmup, settle_ms)
    gbs = rp.nbytes / (ms * 1e-3) / 1e9
    del rp
    torch.cuda.empty_cache()
    return {"kernel": "qg_stream_read", "bytes": -(-wl.algorithmic_bytes() // 16) * 16,
            "us_per_launch": round(ms * 1e3, 2), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "gemv_frac_of_ceiling": round(ms / gemv_ms, 4)}


SETTLE_MS = 40.0


def settle(torch, prep, settle_ms=SETTLE_MS):
    """Launch the kernel back to back for settle_ms of wall time before the
    warmup steps.  After idle the chip's power management takes roughly
    15 ms of sustained load to reach its steady clock; launches inside that
    transient run 5-20% slower than the sustained rate a prefill sees.
    Returns the number of launches spent."""
    n = 0
    stream = torch.cuda.current_stream()
    marks = []
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            prep.launch(n)
            n += 1
        ev = torch.cuda.Event()
        ev.record(stream)
        marks.append(ev)
        if len(marks) > 2:  # keep at most two chunks queued, so the GPU never idles
            marks.pop(0).synchronize()
    torch.cuda.synchronize()
    return n


class AttnPrepared:
    """R rotated device copies of an attention workload's queries, Q8_0 KV
    cache and output; launch(i) calls the C-ABI entry point on copy i mod R."""

    def __init__(self, torch, qg, wl, rotate=None):
        self.wl = wl
        q = wl.q()
        kc, vc = wl.kv()
        per_set = 2 * q.nbytes + kc.size + vc.size
        if rotate is None:
            rotate = max(2, min(16, -(-(MALL_BYTES + (32 << 20)) // per_set) + 1))
        self.rotate = rotate
        self.sets = []
        for _ in range(rotate):
            cache = qg.Q8KVCache.from_canonical(wl.kv_heads, wl.s, wl.head_dim, kc, vc)
            qd = torch.from_numpy(q).cuda()
            self.sets.append((qd, cache, torch.empty_like(qd)))
        L = qg.lib()
        stream = qg._stream(None)
        scale = 1.0 / float(np.sqrt(wl.head_dim))
        self.calls = [(L.qattn_prefill_q8kv, (qd.data_ptr(), o.data_ptr(), wl.heads, wl.m, wl.head_dim,
                                              c.k_codes.data_ptr(), c.k_scales.data_ptr(), c.v_codes.data_ptr(),
                                              c.v_scales.data_ptr(), wl.kv_heads, wl.s, 1 if wl.causal else 0,
                                              scale, stream))
                      for qd, c, o in self.sets]

    def launch(self, i):
        fn, args = self.calls[i % self.rotate]
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"{fn.__name__} returned status {st}")
        self.last = i % self.rotate

    def last_out(self):
        return self.sets[getattr(self, "last", 0)][2]


def time_launches(torch, prep, steps, warmup, settle_ms=SETTLE_MS):
    settled = settle(torch, prep, settle_ms) if settle_ms > 0 else 0
    for i in range(warmup):
        prep.launch(settled + i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        prep.launch(settled + warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, settled


def roofline(wl, ms, traffic=None):
    if bound_of(wl) == "hbm":
        achieved = wl.algorithmic_bytes() / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    achieved = wl.flops() / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "traffic": traffic}


def load_traffic(name):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the
    committed rocprofv3 summary; None if absent or taken with other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = kernel_source_hash(ATTN_SOURCES if name in synth.ATTN_WORKLOADS else KERNEL_SOURCES)
    with open(path) as f:
        for line in f:
            if line.startswith("#") or "workload=" not in line:
                continue
            kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok and not tok.startswith('kernel="'))
            if kv.get("workload") == name and kv.get("kernel_sha") == sha:
                return int(kv["bytes_per_launch"])
    return None


def _sample(rng, size, count):
    """count sorted indices out of range(size), always with the first and the last."""
    if size <= count:
        return np.arange(size)
    mid = rng.choice(np.arange(1, size - 1), count - 2, replace=False)
    return np.sort(np.concatenate([[0, size - 1], mid]))


def _rel_err(y, ref):
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def gemm_parity(torch, prep, y, rows=8, cols=256):
    """The last timed launch's output against the oracle on sampled rows x
    columns (first and last of each included), element by element."""
    import oracle
    wl = prep.wl
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed)
    rm, rn = _sample(rng, wl.m, rows), _sample(rng, wl.n, cols)
    if wl.op == "heads":
        full = y.reshape(-1)[:wl.m * wl.n].reshape(wl.n // wl.head_dim, wl.m, wl.head_dim)
        ys = full.permute(1, 0, 2).reshape(wl.m, wl.n)[rm][:, rn]
    else:
        ys = y[rm][:, rn]
    ys = ys.float().cpu().numpy().astype(np.float64)
    finite = bool(np.all(np.isfinite(ys)))
    x = prep.x_host[rm]
    out = {"rows": len(rm), "cols": len(rn), "tol": 1e-2, "finite": finite}
    if wl.op in synth.GATED:
        fn = oracle.swiglu_ref if wl.op == "swiglu" else oracle.geglu_ref
        ref = fn(wl.codec, prep.canon[0], prep.canon[1], wl.n, wl.k, x, rows_n=rn)
        raw = _rel_err(ys, ref) if finite else float("inf")
        beyond = float(np.max(np.maximum(np.abs(ys - ref) - 2.0 ** -11 * np.abs(ref), 0.0)) /
                       np.sqrt(np.mean(ref ** 2))) if finite else float("inf")
        out.update({"max_abs_err_over_rms": round(raw, 6), "beyond_fp16_output_rounding": round(beyond, 6),
                    "ok": bool(finite and beyond <= 1e-2)})
    else:
        ref = oracle.gemm_ref(wl.codec, prep.canon[0], wl.n, wl.k, x, rows_n=rn)
        err = _rel_err(ys, ref) if finite else float("inf")
        out.update({"max_abs_err_over_rms": round(err, 6), "ok": bool(finite and err <= 1e-2)})
    return out


def attn_parity(torch, prep, rows=6):
    """The last timed launch's output against the oracle on sampled query rows of every head."""
    from oracle.attention import q8kv_attention_ref
    aw = prep.wl
    torch.cuda.synchronize()
    q = aw.q()
    kc, vc = aw.kv()
    rm = _sample(np.random.default_rng(aw.seed), aw.m, rows)
    got = prep.last_out()[:, rm].float().cpu().numpy().astype(np.float64)
    scale = np.float32(1.0 / np.sqrt(aw.head_dim)).item()
    ref = q8kv_attention_ref(q, kc, vc, aw.kv_heads, aw.s, aw.causal, scale, rows=rm)
    finite = bool(np.all(np.isfinite(got)))
    err = _rel_err(got, ref) if finite else float("inf")
    return {"rows": len(rm), "heads": aw.heads, "max_abs_err_over_rms": round(err, 6), "tol": 1e-2, "finite": finite,
            "ok": bool(finite and err <= 1e-2)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, prep, target_s=12.0):
    """The oracle timed on the host on a bounded sample of the workload: exact
    fp64 decode of all of W (each matrix), then the naive fp64 triple loop over
    the first rows of X; the GPU output is checked against it on those rows."""
    import oracle
    wl = prep.wl
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
    mats = len(prep.canon)
    per_row_flops = 2 * wl.n * wl.k * mats

    t0 = time.perf_counter()
    ws = [oracle.decode(wl.codec, c, wl.n, wl.k) for c in prep.canon]
    decode_s = time.perf_counter() - t0

    def matmul(rows):
        t = time.perf_counter()
        refs = [oracle.matmul_xwt(prep.x_host[:rows], w, threads) for w in ws]
        return refs, time.perf_counter() - t

    probe = min(wl.m, max(threads, 16))
    _, dt = matmul(probe)
    rows = max(1, int(min(wl.m, max(probe, probe * target_s / max(dt, 1e-3)))))
    refs, matmul_s = matmul(rows)
    reps = 1
    while rows == wl.m and reps * matmul_s < target_s * 0.8:   # whole workload is short: repeat for a stable figure
        _, more = matmul(rows)
        matmul_s = (matmul_s * reps + more) / (reps + 1)
        reps += 1
    if wl.op in synth.GATED:
        ref = (oracle.swiglu if wl.op == "swiglu" else oracle.geglu)(refs[0], refs[1])
    else:
        ref = refs[0]
    y = prep.launch(0)
    torch.cuda.synchronize()
    yh = y[:rows].cpu().numpy().astype(np.float64)
    finite = bool(np.all(np.isfinite(yh)))
    err = _rel_err(yh, ref) if finite else float("inf")
    total_s = decode_s + matmul_s
    base = {"value": round(per_row_flops * rows / total_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "decode_s": round(decode_s, 3), "matmul_s": round(matmul_s, 3),
            "matmul_gflops": round(per_row_flops * rows / matmul_s / 1e9, 2),
            "sample": f"{rows} of {wl.m} rows of X against all {wl.n} rows of W (K={wl.k}); exact fp64 decode of "
                      f"all of W ({decode_s:.2f} s), then the naive k-ascending fp64 triple loop ({matmul_s:.2f} s"
                      f"{f', mean of {reps} passes' if reps > 1 else ''}); value = sampled flops / (decode + matmul)"}
    parity = {"sample_rows": rows, "max_abs_err_over_rms": err, "tol": 1e-2, "finite": finite,
              "ok": bool(finite and err <= 1e-2)}
    return base, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(synth.WORKLOADS))
    ap.add_argument("--rotate", type=int, default=None)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="back-to-back launches for this long before the warmup steps (0: none)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU layout of this path is a design note, not a run", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_prefill_gemm_codec_amd as qg
    if not os.path.exists(qg.LIB_PATH):
        from quantized_prefill_gemm_codec_amd import build as qbuild
        qbuild.build()
    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calib:
        nbytes = args.copy_calib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy_calibration", "bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": args.steps}), flush=True)
        return

    wl = synth.WORKLOADS[args.workload]
    prep = Prepared(torch, qg, wl, args.rotate)
    print(f"# prepared {wl.name}: rotate={prep.rotate}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    ms, settled = time_launches(torch, prep, args.steps, args.warmup, args.settle_ms)
    print(f"# timed {wl.name}: {ms * 1e3:.1f} us/launch", file=sys.stderr, flush=True)

    unit = "TFLOP/s" if bound_of(wl) == "mfma" else "GB/s"
    value = wl.flops() / (ms * 1e-3) / 1e12 if unit == "TFLOP/s" else wl.algorithmic_bytes() / (ms * 1e-3) / 1e9
    rec = {
        "metric": "quant GEMM TFLOPS at M=2048 (% fp16 MFMA peak); M=1 GEMV HBM GB/s",
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": wl.name, "codec": synth.CODEC_NAMES[wl.codec], "m": wl.m, "n": wl.n, "k": wl.k,
                   "op": wl.op, "rotate": prep.rotate},
        "roofline": roofline(wl, ms, load_traffic(wl.name)),
        "kernel": qg.qg_kernel_for(wl.op, wl.codec, wl.m, wl.n, wl.k),
        "settle": {"ms": args.settle_ms, "launches": settled},
        "parity": gemm_parity(torch, prep, prep.last_out()),
    }
    if wl.op == "gemv":
        rec["read_ceiling"] = read_ceiling(torch, qg, wl, prep.rotate, args.steps, args.warmup, args.settle_ms, ms)
    if not args.no_secondary:
        sec = {}
        for name in SECONDARY:
            if name == wl.name:
                continue
            w2 = synth.WORKLOADS[name]
            p2 = Prepared(torch, qg, w2)
            ms2, settled2 = time_launches(torch, p2, max(10, args.steps), args.warmup, args.settle_ms)
            r2 = roofline(w2, ms2, load_traffic(name))
            sec[name] = {"us_per_launch": round(ms2 * 1e3, 2), "tflops": round(w2.flops() / (ms2 * 1e-3) / 1e12, 2),
                         "gbs": round(w2.algorithmic_bytes() / (ms2 * 1e-3) / 1e9, 1), "roofline": r2,
                         "kernel": qg.qg_kernel_for(w2.op, w2.codec, w2.m, w2.n, w2.k),
                         "rotate": p2.rotate, "settle_launches": settled2}
            sec[name]["parity"] = gemm_parity(torch, p2, p2.last_out())
            if w2.op == "gemv":
                sec[name]["read_ceiling"] = read_ceiling(torch, qg, w2, p2.rotate, max(10, args.steps), args.warmup,
                                                         args.settle_ms, ms2)
            print(f"# timed {name}: {ms2 * 1e3:.1f} us/launch, parity ok={sec[name]['parity']['ok']}",
                  file=sys.stderr, flush=True)
            del p2
            torch.cuda.empty_cache()
        for name, aw in synth.ATTN_WORKLOADS.items():
            p2 = AttnPrepared(torch, qg, aw)
            ms2, settled2 = time_launches(torch, p2, max(10, args.steps), args.warmup, args.settle_ms)
            achieved = aw.flops() / (ms2 * 1e-3) / 1e12
            sec[name] = {"us_per_launch": round(ms2 * 1e3, 2), "tflops": round(achieved, 2),
                         "gbs": round(aw.algorithmic_bytes() / (ms2 * 1e-3) / 1e9, 1),
                         "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                                      "traffic": load_traffic(name)},
                         "kernel": f"attn_q8kv_kernel<{aw.head_dim}>",
                         "rotate": p2.rotate, "settle_launches": settled2}
            sec[name]["parity"] = attn_parity(torch, p2)
            print(f"# timed {name}: {ms2 * 1e3:.1f} us/launch, parity ok={sec[name]['parity']['ok']}",
                  file=sys.stderr, flush=True)
            del p2
            torch.cuda.empty_cache()
        rec["secondary"] = sec
    if not args.no_cpu:
        base, parity = cpu_baseline(torch, prep)
        rec["cpu_baseline"] = base
        rec["parity_oracle_rows"] = parity
        rec["parity"]["ok"] = bool(rec["parity"]["ok"] and parity["ok"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
