"""Benchmark of the FP8 E4M3 block-scaled GEMM hot path on one MI355X.

Default workload (--config dense): the dense LLM projection GEMMs
(M, N, K) in {(4096, 7168, 2048), (4096, 4096, 7168), (8192, 8192, 8192)},
A ~ N(0, 1), B ~ N(0, 0.02^2), both quantised with 128x128 block scales,
BF16 output.  One step = for every shape: quantise A (FP32 -> E4M3 + scales),
quantise B, and the block-scaled GEMM -- every stage of the path.  Inputs are
resident in HBM before timing starts.

value = total GEMM FLOP of a step (2*M*N*K summed) / step time, TFLOP/s.

Timing: HIP events on the stream the kernels are launched on.  A few
consecutive steps (4 or 5, or the decode workload's weight rotation) are
captured once into a HIP graph and replayed until exactly --steps steps have
run (every replay of the verification pass is checked bit for bit against
the eager outputs), so neither the host-side launch overhead of the Python
binding nor the runtime's per-graph launch and completion (about 45 us a
replay) counts as a step's GPU time; --no-graph times eager launches
instead.

Other workloads print their own JSON line: --config decode (M in {1,16,64} x
(N,K) in {(24576,1536),(7168,16384),(4096,4096)}, 1x128 activation scales,
weights rotated over > 768 MB of copies so the 256 MB Infinity Cache cannot
hold them), --config moe (8 experts, 1024 tokens top-2, up and down
projections), --config small (128x256x512), --config outlier (8192^3 with
heavy-tailed, hot-channel activations and 1x128 activation scales),
--config ue8m0 (the dense shapes with power-of-two block scales applied by the
scaled matrix instruction), --config epilogue (SwiGLU and in-place residual
fused into the write-back of MLP-shaped GEMMs, against the unfused pair),
--config wgrad (MoE weight gradient: token-major operands transposed, then
the K-grouped GEMM), --config masked (decode-time MoE on the masked grouped
layout: 8 experts with a capacity of 32 rows, 64 tokens top-2), --config
copy (a plain device copy of known size, used to calibrate the
FETCH_SIZE/WRITE_SIZE counters), --config peak (the FP8 MFMA-loop probe: the
matrix-core rate and shader clock this GPU sustains; the dense line also
carries it as roofline.measured_peak).

Measurement helpers: --roofline-only launches, after the warm-up, only the
roofline kernel (what rocprofv3 counter passes profile); --record-traffic DIR
(no GPU) turns the FETCH_SIZE/WRITE_SIZE passes under DIR into the calibrated
HBM-traffic record in profiles/traffic.json that roofline.traffic reports.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import datagen  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
CSRC = os.path.join(ROOT, "fp8_block_scaled_dg_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

GEMM_TILED_SOURCES = ("gemm_tiled.hip", "dg_device.hpp", "dg_internal.hpp")
GEMM_SKINNY_SOURCES = ("gemm_skinny.hip", "dg_device.hpp", "dg_internal.hpp")

# Roofline kernels whose HBM traffic is recorded in profiles/traffic.json:
# config -> (record key, sources hashed into the record, part of the kernel's
# symbol that the counter rows must carry).
TRAFFIC_KERNELS = {
    "dense": ("gemm_tiled_kernel<256,128,false> 8192x8192x8192", GEMM_TILED_SOURCES,
              "gemm_tiled_kernel<256, 128, false, false, false>"),
    "decode": ("gemm_skinny_kernel<64,1,codes,false,4> 64x7168x16384", GEMM_SKINNY_SOURCES,
               "gemm_skinny_kernel<64, 1, 0, false, 4, false>"),
    "moe": ("gemm_ring_kernel<1,true> grouped up projection 8x11008x4096", GEMM_TILED_SOURCES,
            "gemm_ring_kernel<1, true>"),
}
COPY_BYTES = 1 << 30       # the calibration copy of --config copy

DENSE = [(4096, 7168, 2048), (4096, 4096, 7168), (8192, 8192, 8192)]
DECODE = [(m, n, k) for (n, k) in [(24576, 1536), (7168, 16384), (4096, 4096)] for m in (1, 16, 64)]


def cdiv(a, b):
    return (a + b - 1) // b


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_key: str, sources):
    """HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE
    (calibrated against a plain copy) and recorded in profiles/traffic.json,
    valid only while the kernel sources still have the recorded hash."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(sources):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP events on the launch stream; optionally over HIP-graph replays."""

    def __init__(self, use_graph: bool):
        self.stream = torch.cuda.current_stream()
        self.use_graph = use_graph
        self.graphs = {}

    def graph(self, key, fn):
        if key not in self.graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            torch.cuda.synchronize()
            self.graphs[key] = g
        return self.graphs[key]

    def stats(self, fn, reps: int, key, calls: int = 4, warmup: int = 3) -> dict:
        """Per-launch microseconds over `reps` replays of a graph of `calls`
        back-to-back launches (events around each replay): mean, median, min."""
        def body():
            for _ in range(calls):
                fn()
        g = self.graph((key, calls), body)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for s, e in ev:
            s.record(self.stream)
            g.replay()
            e.record(self.stream)
        torch.cuda.synchronize()
        us = sorted(s.elapsed_time(e) * 1e3 / calls for s, e in ev)
        return {"mean": sum(us) / len(us), "median": us[len(us) // 2], "min": us[0],
                "launches": reps * calls, "warmup_launches": warmup * calls}

    def time(self, fn, reps: int, key=None, calls: int = 1) -> float:
        """Milliseconds per call of fn (fn may enqueue several kernels).

        With graphs, one graph holds `calls` back-to-back calls of fn, so that
        the host cost of a replay is spread over enough GPU work to stay hidden
        behind it (a single short kernel per replay would time the host)."""
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        if self.use_graph and key is not None:
            def body():
                for _ in range(calls):
                    fn()
            g = self.graph((key, calls), body)
            g.replay()
            torch.cuda.synchronize()
            s.record(self.stream)
            for _ in range(reps):
                g.replay()
            n = reps * calls
        else:
            fn()
            torch.cuda.synchronize()
            s.record(self.stream)
            for _ in range(reps):
                fn()
            n = reps
        e.record(self.stream)
        e.synchronize()
        return s.elapsed_time(e) / n


# ---------------------------------------------------------------------------
# workloads.  Each has: rot (rotation states per graph), step(i), outputs(),
# flops (per step), config(), breakdown(timer, reps), roofline(timer, reps),
# cpu_baseline().
# ---------------------------------------------------------------------------

class Dense:
    rot = 1

    def __init__(self, dg, shapes, seed=0, outlier=False, ue8m0=False):
        """outlier: A = heavy-tailed rows with 1% hot channels x100, quantised
        with 1x128 (per-row) scales; otherwise A ~ N(0,1) with 128x128 scales.
        ue8m0: power-of-two scales packed four K blocks per int32, applied by
        the scaled MFMA."""
        self.dg = dg
        self.outlier = outlier
        self.ue8m0 = ue8m0
        self.a_br = 1 if outlier else 128
        self.items = []
        for (M, N, K) in shapes:
            if outlier:
                a_np, _ = datagen.student_t_outliers(M, K, seed=seed, stream=5)
            else:
                a_np = datagen.normal((M, K), 1.0, seed=seed, stream=0)
            a = torch.from_numpy(a_np).cuda()
            b = torch.from_numpy(datagen.normal((N, K), 0.02, seed=seed, stream=1)).cuda()
            if ue8m0:
                sa = torch.empty((cdiv(K // 128, 4), cdiv(M, self.a_br)), dtype=torch.int32,
                                 device="cuda")
                sb = torch.empty((cdiv(K // 128, 4), cdiv(N, 128)), dtype=torch.int32, device="cuda")
            else:
                sa = torch.empty((K // 128, cdiv(M, self.a_br)), dtype=torch.float32, device="cuda")
                sb = torch.empty((K // 128, cdiv(N, 128)), dtype=torch.float32, device="cuda")
            self.items.append(dict(
                M=M, N=N, K=K, a=a, b=b, sa=sa, sb=sb,
                qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                qb=torch.empty((N, K), dtype=torch.uint8, device="cuda"),
                c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        self.flops = sum(2.0 * it["M"] * it["N"] * it["K"] for it in self.items)

    def quant_a(self, it):
        if self.ue8m0:
            self.dg.dg_quantize_fp8_block_ue8m0(it["qa"], it["sa"], it["a"], self.a_br)
        else:
            self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], self.a_br)

    def quant_b(self, it):
        if self.ue8m0:
            self.dg.dg_quantize_fp8_block_ue8m0(it["qb"], it["sb"], it["b"], 128)
        else:
            self.dg.dg_quantize_fp8_block(it["qb"], it["sb"], it["b"], 128)

    def gemm(self, it):
        if self.ue8m0:
            self.dg.dg_fp8_gemm_nt_ue8m0(it["c"], it["qa"], it["qb"], it["sa"], it["sb"],
                                         self.a_br)
        else:
            self.dg.dg_fp8_gemm_nt(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], self.a_br)

    def step(self, i=0):
        for it in self.items:
            self.quant_a(it)
            self.quant_b(it)
            self.gemm(it)

    def outputs(self):
        return [t for it in self.items for t in (it["qa"], it["sa"], it["qb"], it["sb"], it["c"])]

    def config(self):
        if self.outlier:
            return {"workload": "outlier activations: 8192^3 GEMM, A heavy-tailed (Student-t, "
                                "nu=3) with 1% hot channels x100, 1x128 A scales",
                    "shapes_mnk": [[it["M"], it["N"], it["K"]] for it in self.items],
                    "a_scales": "1x128", "b_scales": "128x128",
                    "step": "quantise A + quantise B + GEMM",
                    "inputs": "B ~ N(0,0.02^2), float32, seed 0"}
        if self.ue8m0:
            return {"workload": "dense LLM projection GEMMs, E4M3 128x128 blocks with "
                                "power-of-two (UE8M0) scales packed 4 per int32, BF16 out",
                    "shapes_mnk": [[it["M"], it["N"], it["K"]] for it in self.items],
                    "a_scales": "128x128 UE8M0", "b_scales": "128x128 UE8M0",
                    "step": "quantise A + quantise B + GEMM, per shape",
                    "inputs": "A ~ N(0,1), B ~ N(0,0.02^2), float32, seed 0"}
        return {"workload": "dense LLM projection GEMMs, E4M3 128x128 block scales, BF16 out",
                "shapes_mnk": [[it["M"], it["N"], it["K"]] for it in self.items],
                "a_scales": "128x128", "b_scales": "128x128",
                "step": "quantise A + quantise B + GEMM, per shape",
                "inputs": "A ~ N(0,1), B ~ N(0,0.02^2), float32, seed 0"}

    def breakdown(self, timer, reps):
        out = []
        for n, it in enumerate(self.items):
            M, N, K = it["M"], it["N"], it["K"]
            tq_a = timer.time(lambda: self.quant_a(it), reps, key=("qa", n), calls=10)
            tq_b = timer.time(lambda: self.quant_b(it), reps, key=("qb", n), calls=10)
            tg = timer.time(lambda: self.gemm(it), reps, key=("g", n), calls=4)
            sbytes = 1 if self.ue8m0 else 4
            qbytes_a = M * K * 5 + sbytes * (K // 128) * cdiv(M, self.a_br)
            qbytes_b = N * K * 5 + sbytes * (K // 128) * cdiv(N, 128)
            out.append({"mnk": [M, N, K],
                        "gemm_us": tg * 1e3, "gemm_tflops": 2.0 * M * N * K / (tg * 1e-3) / 1e12,
                        "quant_a_us": tq_a * 1e3, "quant_a_gbs": qbytes_a / (tq_a * 1e-3) / 1e9,
                        "quant_b_us": tq_b * 1e3, "quant_b_gbs": qbytes_b / (tq_b * 1e-3) / 1e9})
        return out

    def roofline(self, timer, reps):
        """Dominant kernel: the GEMM launch on the largest shape (8192^3)."""
        n, it = max(enumerate(self.items), key=lambda t: t[1]["M"] * t[1]["N"] * t[1]["K"])
        if timer.use_graph:
            st = timer.stats(lambda: self.gemm(it), max(reps, 25), ("g", n), calls=4)
            t = st["mean"] * 1e-3
        else:
            st = None
            t = timer.time(lambda: self.gemm(it), reps, key=("g", n), calls=4)
        flop = 2.0 * it["M"] * it["N"] * it["K"]
        ach = flop / (t * 1e-3) / 1e12
        key = "gemm_tiled_kernel<256,%d,false%s> %dx%dx%d" % (
            self.a_br, ",true" if self.ue8m0 else "", it["M"], it["N"], it["K"])
        return {"kernel": key, "bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_FP8_TFLOPS,
                "traffic": recorded_traffic(key, GEMM_TILED_SOURCES),
                "algorithmic_bytes": it["M"] * it["K"] + it["N"] * it["K"] + 2 * it["M"] * it["N"]
                + 4 * (it["K"] // 128) * (cdiv(it["M"], self.a_br) + cdiv(it["N"], 128)),
                "avg_launch_us": t * 1e3, "launch_us_stats": st}

    def cpu_baseline(self):
        """The oracle (plain C, one call per thread over disjoint rows) on a
        bounded sample, timed on the host's cores: per shape, quantise all of
        B (split at 128-row block boundaries, one slice per thread) and one
        128-row block of A, and compute 8 full output rows per thread.
        Extrapolated to the whole step on the same threads (B quantised once,
        A in M/128 blocks, M output rows)."""
        if self.ue8m0:
            return None
        import concurrent.futures as cf
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        rows_per_thread = 8
        oracle.e4m3_decode(np.zeros(1, np.uint8))      # load the library before threading
        total = 0.0
        spent = 0.0
        quant_s = gemm_s = 0.0
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            for it in self.items:
                M, N, K = it["M"], it["N"], it["K"]
                a = it["a"][:128].cpu().numpy()
                b = it["b"].cpu().numpy()
                nblk = cdiv(N, 128)
                cuts = [min(N, 128 * (nblk * t // threads)) for t in range(threads + 1)]
                t0 = time.perf_counter()
                parts = list(ex.map(lambda t: oracle.quantize(b[cuts[t]:cuts[t + 1]], 128)
                                    if cuts[t + 1] > cuts[t] else None, range(threads)))
                t1 = time.perf_counter()
                qb = np.concatenate([p[0] for p in parts if p is not None])
                sb = np.concatenate([p[1] for p in parts if p is not None], axis=1)
                t1b = time.perf_counter()
                qa, sa = oracle.quantize(a, self.a_br)
                t2 = time.perf_counter()
                rows = np.linspace(0, 127, threads * rows_per_thread).astype(np.int64)

                def gemm_rows(t):
                    r = rows[t * rows_per_thread:(t + 1) * rows_per_thread]
                    return oracle.gemm_nt_points(qa, sa, qb, sb, np.repeat(r, N),
                                                 np.tile(np.arange(N, dtype=np.int64), r.size),
                                                 a_block_rows=self.a_br)
                t2b = time.perf_counter()
                list(ex.map(gemm_rows, range(threads)))
                t3 = time.perf_counter()
                spent += (t1 - t0) + (t2 - t1b) + (t3 - t2b)
                quant = (t1 - t0) + (M / 128) * (t2 - t1b) / threads
                gemm = (M / (threads * rows_per_thread)) * (t3 - t2b)
                total += quant + gemm
                quant_s += quant
                gemm_s += gemm
        single = oracle_single_thread_cases()
        return {"value": self.flops / total / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle", "cpu_model": cpu_model(),
                "quantise_s": quant_s, "gemm_s": gemm_s, "single_thread": single,
                "sample": "per shape: oracle quantise of all of B (%d threads, one slice of "
                          "128-row blocks each) and of one 128-row block of A, then %d full "
                          "output rows of the FP64 dequantised GEMM per thread (%.1f s wall); "
                          "extrapolated to the full step on the same threads (%.0f s: "
                          "quantise %.1f s, GEMM %.0f s); single_thread: two whole small "
                          "cases timed on one thread"
                          % (threads, rows_per_thread, spent, total, quant_s, gemm_s)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_single_thread_cases() -> dict:
    """The oracle on one thread, whole cases, wall seconds split into
    quantisation and GEMM: the small single GEMM (128 x 256 x 512, both
    operands with 128x128 blocks) and one decode GEMM (1 x 24576 x 1536, A
    with 1x128 blocks, B with 128x128 blocks), seeded normals as in the
    workloads."""
    import oracle
    out = {}
    for name, (M, N, K, br) in (("small_128x256x512", (128, 256, 512, 128)),
                                ("decode_1x24576x1536", (1, 24576, 1536, 1))):
        a = datagen.normal((M, K), 1.0, seed=0, stream=0)
        b = datagen.normal((N, K), 0.02, seed=0, stream=1)
        t0 = time.perf_counter()
        qa, sa = oracle.quantize(a, br)
        qb, sb = oracle.quantize(b, 128)
        t1 = time.perf_counter()
        oracle.gemm_nt(qa, sa, qb, sb, a_block_rows=br)
        t2 = time.perf_counter()
        out[name] = {"quantise_s": t1 - t0, "gemm_s": t2 - t1,
                     "tflops": 2.0 * M * N * K / (t2 - t0) / 1e12}
    return out


class Decode:
    def __init__(self, dg, rotate_bytes=768 << 20, seed=0):
        self.dg = dg
        self.items = []
        for (M, N, K) in DECODE:
            copies = max(2, cdiv(rotate_bytes, N * K))
            g = torch.Generator(device="cuda")
            g.manual_seed(seed + M * 7 + N)
            qb = torch.randint(0, 0x7E, (copies, N, K), dtype=torch.uint8, device="cuda",
                               generator=g)
            sb = torch.rand((copies, K // 128, N // 128), device="cuda", generator=g) * 1e-3
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=M)).cuda()
            ws_bytes = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
            a16 = a.to(torch.bfloat16)
            # power-of-two (UE8M0) exponent bytes 120..127, four K blocks per int32
            w = cdiv(K // 128, 4)
            sfa = (torch.randint(120, 128, (w, M, 4), device="cuda", generator=g)
                   .to(torch.uint8).view(torch.int32).reshape(w, M))
            sfb = (torch.randint(120, 128, (w, cdiv(N, 128), 4), device="cuda", generator=g)
                   .to(torch.uint8).view(torch.int32).reshape(w, cdiv(N, 128)))
            self.items.append(dict(sfa=sfa, sfb=sfb,
                M=M, N=N, K=K, qb=qb, sb=sb, a=a, a16=a16, copies=copies,
                qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                sa=torch.empty((K // 128, M), dtype=torch.float32, device="cuda"),
                ws=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda"),
                c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        self.rot = max(it["copies"] for it in self.items)
        self.flops = sum(2.0 * it["M"] * it["N"] * it["K"] for it in self.items)

    @staticmethod
    def bytes_of(it):
        M, N, K = it["M"], it["N"], it["K"]
        return N * K + M * K + 4 * (K // 128) * (M + N // 128) + 2 * M * N

    def gemm(self, it, i):
        j = i % it["copies"]
        self.dg.dg_fp8_gemm_nt(it["c"], it["qa"], it["qb"][j], it["sa"], it["sb"][j], 1,
                               workspace=it["ws"])

    # rows up to which the step quantises A inside the GEMM: measured faster
    # than quantiser + GEMM there, slower above (every workgroup then stages
    # M rows of FP32 A per K block: 4 bytes per value instead of 1)
    FUSED_STEP_MAX_M = 16

    def step(self, i=0):
        # M <= 16: one call quantises A inside the GEMM (same codes and scales);
        # larger M: quantiser, then GEMM
        for it in self.items:
            if it["M"] <= self.FUSED_STEP_MAX_M:
                self.fused(it, i)
            else:
                self.quantise_and_gemm(it, i)

    def outputs(self):
        out = []
        for it in self.items:
            out += [it["c"]] if it["M"] <= self.FUSED_STEP_MAX_M else [it["qa"], it["sa"], it["c"]]
        return out

    def config(self):
        return {"workload": "decode-shaped GEMMs, M in {1,16,64} x (N,K) in {(24576,1536),"
                            "(7168,16384),(4096,4096)}, A 1x128 scales, B 128x128 scales",
                "step": "quantise A + GEMM per shape (M <= 16: one call that quantises FP32 A "
                        "inside the GEMM, measured faster there; M = 64: quantiser, then GEMM, "
                        "measured faster than the fused call); weights rotated over >768 MB "
                        "of copies"}

    def _time_gemm(self, timer, n, it, reps):
        rot = it["copies"]
        return timer.time(lambda: [self.gemm(it, i) for i in range(rot)], reps,
                          key=("dec", n)) / rot

    def gemm_e8(self, it, i):
        j = i % it["copies"]
        self.dg.dg_fp8_gemm_nt_ue8m0(it["c"], it["qa"], it["qb"][j], it["sfa"], it["sfb"], 1,
                                     workspace=it["ws"])

    def quantise_and_gemm(self, it, i):
        self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 1)
        self.gemm(it, i)

    def fused(self, it, i, bf16=False):
        j = i % it["copies"]
        self.dg.dg_fp8_gemm_nt_fused_a(it["c"], it["a16"] if bf16 else it["a"], it["qb"][j],
                                       it["sb"][j], workspace=it["ws"])

    def read_probe(self, timer, it, reps):
        """The weight read alone: the probe kernel reads the same rotated
        copies of B with 128 bytes per row per K block, 8 KB per wave in
        flight (no A, no arithmetic); best time over its split counts."""
        lib = probe_lib()
        if lib is None:
            return None
        N, K = it["N"], it["K"]
        best = None
        for splits in (1, 2, 4, 8):
            if K % (512 * splits):
                continue
            out = torch.empty(N // 64 * splits * 256, dtype=torch.int32, device="cuda")

            def one(i, splits=splits, out=out):
                rc = lib.dgp_hbm_read(it["qb"][i % it["copies"]].data_ptr(), N, K, splits,
                                      out.data_ptr(),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc != 0:
                    raise RuntimeError("read probe launch failed (%d)" % rc)
            rot = it["copies"]
            t = timer.time(lambda: [one(i) for i in range(rot)], reps,
                           key=("rdp", N, K, splits)) / rot
            if best is None or t < best[0]:
                best = (t, splits)
        return {"us": best[0] * 1e3, "splits": best[1], "workgroups": N // 64 * best[1],
                "tbs": N * K / (best[0] * 1e-3) / 1e12}

    def breakdown(self, timer, reps):
        out = []
        probes = {}
        for n, it in enumerate(self.items):
            t = self._time_gemm(timer, n, it, reps)
            b = self.bytes_of(it)
            row = {"mnk": [it["M"], it["N"], it["K"]], "gemm_us": t * 1e3,
                   "hbm_gbs": b / (t * 1e-3) / 1e9,
                   "hbm_frac": b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
            key = (it["N"], it["K"])
            if key not in probes:
                probes[key] = self.read_probe(timer, it, reps)
            if probes[key] is not None:
                row["weight_read_probe"] = probes[key]
            rot = it["copies"]
            row["quantise_gemm_us"] = timer.time(
                lambda: [self.quantise_and_gemm(it, i) for i in range(rot)], reps,
                key=("decq", n)) / rot * 1e3
            if it["M"] <= self.dg.FUSED_A_MAX_M:
                row["fused_us"] = timer.time(lambda: [self.fused(it, i) for i in range(rot)],
                                             reps, key=("decf", n)) / rot * 1e3
                row["fused_bf16_us"] = timer.time(
                    lambda: [self.fused(it, i, True) for i in range(rot)], reps,
                    key=("decb", n)) / rot * 1e3
            # the same GEMM with power-of-two (UE8M0) scales on the scaled MFMA
            row["ue8m0_gemm_us"] = timer.time(lambda: [self.gemm_e8(it, i) for i in range(rot)],
                                              reps, key=("dece", n)) / rot * 1e3
            out.append(row)
        return out

    def roofline(self, timer, reps):
        n, it = max(enumerate(self.items), key=lambda t: t[1]["N"] * t[1]["K"] * 1000 + t[1]["M"])
        t = self._time_gemm(timer, n, it, reps)
        b = self.bytes_of(it)
        ach = b / (t * 1e-3) / 1e9
        key, src, _ = TRAFFIC_KERNELS["decode"]
        shape = "%dx%dx%d" % (it["M"], it["N"], it["K"])
        return {"kernel": "decode GEMM %s" % [it["M"], it["N"], it["K"]], "bound": "hbm",
                "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": recorded_traffic(key, src) if key.endswith(shape) else None,
                "algorithmic_bytes": b, "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        return None


class Epilogue:
    """Fused epilogues on LLM-MLP-shaped GEMMs (2048 tokens): the up
    projection with gate and up interleaved and SwiGLU applied on write-back
    (N = 2 x 11008, K = 4096, C has 11008 columns), and the down projection
    with a BF16 residual added on write-back (N = 4096, K = 11008).  A step =
    quantise A (1x128 scales) + the fused GEMM, per shape; B is quantised
    once.  The breakdown also times the unfused pair (plain GEMM, then the
    same element-wise step as a separate PyTorch operation) for comparison."""
    rot = 1

    def __init__(self, dg, seed=0):
        self.dg = dg
        self.items = []
        for (M, N, K, act) in [(2048, 22016, 4096, "swiglu"), (2048, 4096, 11008, "none")]:
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=0)).cuda()
            b = torch.from_numpy(datagen.normal((N, K), 0.02, seed=seed, stream=1)).cuda()
            qb, sb = dg.to_fp8(b, 128)
            n_out = N // 2 if act == "swiglu" else N
            res = None
            if act == "none":
                res = torch.from_numpy(datagen.normal((M, N), 1.0, seed=seed, stream=2)).cuda()
                res = res.to(torch.bfloat16)
            self.items.append(dict(
                M=M, N=N, K=K, act=act, a=a, qb=qb, sb=sb, res=res,
                qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                sa=torch.empty((K // 128, M), dtype=torch.float32, device="cuda"),
                c=torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda"),
                c_full=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        self.flops = sum(2.0 * it["M"] * it["N"] * it["K"] for it in self.items)

    def fused(self, it):
        # the residual is read from its own buffer here (the same bytes as in
        # place, without re-seeding C before every call)
        self.dg.dg_fp8_gemm_nt_epilogue(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], 1,
                                        act=it["act"], residual=it["res"])

    def unfused(self, it):
        self.dg.dg_fp8_gemm_nt(it["c_full"], it["qa"], it["qb"], it["sa"], it["sb"], 1)
        if it["act"] == "swiglu":
            g = it["c_full"][:, 0::2].float()
            u = it["c_full"][:, 1::2].float()
            it["c"].copy_(torch.nn.functional.silu(g) * u)
        else:
            torch.add(it["c_full"], it["res"], out=it["c"])

    def step(self, i=0):
        for it in self.items:
            self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 1)
            self.fused(it)

    def outputs(self):
        return [t for it in self.items for t in (it["qa"], it["sa"], it["c"])]

    def config(self):
        return {"workload": "fused GEMM epilogues at 2048 tokens: up projection 4096 -> 2 x 11008 "
                            "with interleaved gate/up and SwiGLU on write-back; down projection "
                            "11008 -> 4096 with a BF16 residual added on write-back",
                "shapes_mnk": [[it["M"], it["N"], it["K"]] for it in self.items],
                "a_scales": "1x128", "b_scales": "128x128",
                "step": "quantise A + fused GEMM per shape (B quantised once)",
                "inputs": "A ~ N(0,1), B ~ N(0,0.02^2), residual ~ N(0,1) in BF16, seed 0"}

    def breakdown(self, timer, reps):
        out = []
        for n, it in enumerate(self.items):
            tf = timer.time(lambda: self.fused(it), reps, key=("ef", n), calls=4)
            tu = timer.time(lambda: self.unfused(it), reps, key=("eu", n), calls=4)
            out.append({"mnk": [it["M"], it["N"], it["K"]], "epilogue": it["act"] if it["res"] is None
                        else "residual", "fused_us": tf * 1e3, "unfused_us": tu * 1e3,
                        "fused_tflops": 2.0 * it["M"] * it["N"] * it["K"] / (tf * 1e-3) / 1e12})
        return out

    def roofline(self, timer, reps):
        it = self.items[0]
        st = timer.stats(lambda: self.fused(it), max(reps, 25), ("ef", 0), calls=4)
        t = st["mean"] * 1e-3
        flop = 2.0 * it["M"] * it["N"] * it["K"]
        ach = flop / (t * 1e-3) / 1e12
        return {"kernel": "gemm_tiled_kernel<256,1,false> %dx%dx%d + SwiGLU epilogue"
                          % (it["M"], it["N"], it["K"]),
                "bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_FP8_TFLOPS, "traffic": None, "avg_launch_us": t * 1e3,
                "launch_us_stats": st}

    def cpu_baseline(self):
        return None


class WeightGrad:
    """MoE weight gradient of the down projection (8 experts, 1024 tokens
    top-2, hidden 4096, intermediate 11008): per expert g,
    dW_g[4096][11008] = dY_g^T . H_g over that expert's tokens, i.e. a
    K-grouped GEMM with K = the expert's token rows (padded to 128, the
    routing of the MoE workload).  The operands arrive token-major (dY
    [T][4096], H [T][11008], already quantised: 1x128 blocks along the token
    axis for dY^T, 128x128 for H^T), so a step = transpose both code matrices
    + the K-grouped GEMM."""
    rot = 1

    def __init__(self, dg, seed=0):
        self.dg = dg
        E, tokens, H, I = 8, 1024, 4096, 11008
        r = datagen.moe_routing(tokens, E, 2, align=128, seed=seed)
        padded = r["padded"]
        ko = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
        T = int(ko[-1])
        self.M, self.N, self.K, self.G = H, I, T, E
        a = datagen.normal((H, T), 1.0, seed=seed, stream=3)        # dY^T (logical [M][K])
        b = datagen.normal((I, T), 1.0, seed=seed, stream=4)        # H^T  (logical [N][K])
        qa, sa = dg.to_fp8(torch.from_numpy(a).cuda(), 1)
        qb, sb = dg.to_fp8(torch.from_numpy(b).cuda(), 128)
        # stored token-major, as a backward pass produces them
        self.a_tok = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        self.b_tok = torch.empty((T, I), dtype=torch.uint8, device="cuda")
        dg.dg_transpose_fp8(self.a_tok, qa)
        dg.dg_transpose_fp8(self.b_tok, qb)
        self.sa, self.sb = sa, sb
        self.qa = torch.empty((H, T), dtype=torch.uint8, device="cuda")
        self.qb = torch.empty((I, T), dtype=torch.uint8, device="cuda")
        self.ko = torch.from_numpy(ko).cuda()
        self.c = torch.empty((E, H, I), dtype=torch.bfloat16, device="cuda")
        self.flops = 2.0 * H * I * T
        self.padded = [int(x) for x in padded]

    def transposes(self):
        self.dg.dg_transpose_fp8(self.qa, self.a_tok)
        self.dg.dg_transpose_fp8(self.qb, self.b_tok)

    def gemm(self):
        self.dg.dg_fp8_grouped_gemm_k(self.c, self.qa, self.qb, self.sa, self.sb, 1, self.ko)

    def step(self, i=0):
        self.transposes()
        self.gemm()

    def outputs(self):
        return [self.qa, self.qb, self.c]

    def config(self):
        return {"workload": "MoE weight gradient, K-grouped: 8 experts x dW[4096][11008] over each "
                            "expert's token rows (1024 tokens top-2, padded to 128)",
                "groups_k": self.padded, "mnk_total": [self.M, self.N, self.K],
                "a_scales": "1x128 (along tokens)", "b_scales": "128x128",
                "step": "transpose the token-major dY and H codes + K-grouped GEMM",
                "inputs": "synthetic N(0,1) operands, uniform top-2 routing, seed 0"}

    def breakdown(self, timer, reps):
        tt = timer.time(self.transposes, reps, key=("wt",), calls=4)
        tg = timer.time(self.gemm, reps, key=("wg",), calls=2)
        tbytes = 2 * (self.M + self.N) * self.K
        return [{"transposes_us": tt * 1e3, "transpose_gbs": tbytes / (tt * 1e-3) / 1e9,
                 "gemm_us": tg * 1e3, "gemm_tflops": self.flops / (tg * 1e-3) / 1e12}]

    def algorithmic_bytes(self):
        """One launch: the G x M x N BF16 outputs written, the two code
        matrices and their scales read once."""
        scales = 4 * (self.K // 128) * (self.M + cdiv(self.N, 128))
        return 2 * self.G * self.M * self.N + (self.M + self.N) * self.K + scales

    def roofline(self, timer, reps):
        """HBM-bound: with 256-384 tokens per expert the launch does about
        290 FLOP per byte of output written, below the chip's FP8 balance
        (5.0 PFLOP/s over 8 TB/s = 625 FLOP/B)."""
        st = timer.stats(self.gemm, max(reps, 25), ("wg",), calls=2)
        t = st["mean"] * 1e-3
        b = self.algorithmic_bytes()
        ach = b / (t * 1e-3) / 1e9
        return {"kernel": "gemm_tiled_kernel<256,1,false,false,true> K-grouped %dx%dx%d, 8 groups"
                          % (self.M, self.N, self.K),
                "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": None, "algorithmic_bytes": b,
                "flop_per_byte": self.flops / b,
                "tflops": self.flops / (t * 1e-3) / 1e12, "avg_launch_us": t * 1e3,
                "launch_us_stats": st}

    def cpu_baseline(self):
        return None


class Moe:
    rot = 1

    def __init__(self, dg, seed=0):
        self.dg = dg
        G, tokens, H, I = 8, 1024, 4096, 11008
        r = datagen.moe_routing(tokens, G, 2, align=128, seed=seed)
        mi = torch.from_numpy(r["m_indices"]).cuda()
        M = mi.shape[0]
        self.real_rows = int((r["m_indices"] >= 0).sum())
        self.items = []
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        for (N, K) in ((I, H), (H, I)):
            qb = torch.randint(0, 0x7E, (G, N, K), dtype=torch.uint8, device="cuda", generator=gen)
            sb = torch.rand((G, K // 128, N // 128), device="cuda", generator=gen) * 1e-3
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=K)).cuda()
            a[mi < 0] = 0
            self.items.append(dict(
                M=M, N=N, K=K, qb=qb, sb=sb, a=a, mi=mi,
                qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                sa=torch.empty((K // 128, M), dtype=torch.float32, device="cuda"),
                c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        self.flops = sum(2.0 * self.real_rows * it["N"] * it["K"] for it in self.items)
        # breakdown only: the balanced grouped call (work shared out by K block
        # over one workgroup per CU), slower on these weight-streaming shapes
        self.ws = dg.alloc_workspace(max(dg.dg_fp8_grouped_gemm_contig_workspace_bytes(
            it["M"], it["N"], it["K"]) for it in self.items))
        # breakdown only: the up projection with gate and up interleaved
        # (2 x 11008 rows per expert) and SwiGLU fused on the write-back
        up = self.items[0]
        self.glu = dict(
            qb=torch.randint(0, 0x7E, (G, 2 * I, H), dtype=torch.uint8, device="cuda", generator=gen),
            sb=torch.rand((G, H // 128, 2 * I // 128), device="cuda", generator=gen) * 1e-3,
            c=torch.empty((M, I), dtype=torch.bfloat16, device="cuda"),
            c_full=torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda"), up=up)

    def gemm(self, it, workspace=None):
        self.dg.dg_fp8_grouped_gemm_contig(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], 1,
                                           it["mi"], workspace=workspace)

    def glu_fused(self):
        g, up = self.glu, self.glu["up"]
        self.dg.dg_fp8_grouped_gemm_contig(g["c"], up["qa"], g["qb"], up["sa"], g["sb"], 1,
                                           up["mi"], act="swiglu")

    def glu_unfused(self):
        g, up = self.glu, self.glu["up"]
        self.dg.dg_fp8_grouped_gemm_contig(g["c_full"], up["qa"], g["qb"], up["sa"], g["sb"], 1,
                                           up["mi"])
        gate = g["c_full"][:, 0::2].float()
        u = g["c_full"][:, 1::2].float()
        g["c"].copy_(torch.nn.functional.silu(gate) * u)

    def step(self, i=0):
        for it in self.items:
            self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 1)
            self.gemm(it)

    def outputs(self):
        return [t for it in self.items for t in (it["qa"], it["sa"], it["c"])]

    def config(self):
        return {"workload": "grouped MoE GEMM, M-contiguous, 8 experts, 1024 tokens top-2, "
                            "hidden 4096, intermediate 11008, up and down projections",
                "m_total": self.items[0]["M"], "real_rows": self.real_rows}

    def breakdown(self, timer, reps):
        out = []
        for n, it in enumerate(self.items):
            t = timer.time(lambda: self.gemm(it), reps, key=("moe", n), calls=4)
            tb = timer.time(lambda: self.gemm(it, self.ws), reps, key=("moebal", n), calls=4)
            byts = 8 * it["N"] * it["K"] + it["M"] * it["K"] + 2 * it["M"] * it["N"]
            out.append({"nk": [it["N"], it["K"]], "gemm_us": t * 1e3,
                        "tflops_real_rows": 2.0 * self.real_rows * it["N"] * it["K"]
                        / (t * 1e-3) / 1e12,
                        "hbm_gbs": byts / (t * 1e-3) / 1e9, "balanced_gemm_us": tb * 1e3})
        up = self.items[0]
        tf = timer.time(self.glu_fused, reps, key=("moeglu", 0), calls=4)
        tu = timer.time(self.glu_unfused, reps, key=("moeglu", 1), calls=4)
        out.append({"nk": [2 * up["N"], up["K"]], "epilogue": "swiglu (gate/up interleaved)",
                    "fused_us": tf * 1e3, "unfused_us": tu * 1e3,
                    "tflops_real_rows": 2.0 * self.real_rows * 2 * up["N"] * up["K"]
                    / (tf * 1e-3) / 1e12})
        return out

    def roofline(self, timer, reps):
        it = self.items[0]
        t = timer.time(lambda: self.gemm(it), reps, key=("moe", 0), calls=4)
        byts = 8 * it["N"] * it["K"] + it["M"] * it["K"] + 2 * it["M"] * it["N"]
        ach = byts / (t * 1e-3) / 1e9
        key, src, _ = TRAFFIC_KERNELS["moe"]
        return {"kernel": "grouped GEMM up-projection", "bound": "hbm", "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": recorded_traffic(key, src), "algorithmic_bytes": byts,
                "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        return None


class Masked:
    """Decode-time MoE on the masked grouped layout: 8 experts, 64 tokens
    routed top-2 (uniform, distinct experts), a capacity of 32 rows per
    expert with masked_m = the routed count; up (N 11008, K 4096) and down
    (N 4096, K 11008) projections.  Activations arrive quantised per expert
    (1x128 scales); the step is the two masked GEMMs."""
    rot = 1

    def __init__(self, dg, seed=0):
        self.dg = dg
        G, tokens, H, I, cap = 8, 64, 4096, 11008, 32
        r = datagen.moe_routing(tokens, G, 2, align=1, seed=seed)
        counts = np.minimum(r["counts"], cap).astype(np.int32)
        self.counts = counts
        self.real_rows = int(counts.sum())
        mm = torch.from_numpy(counts).cuda()
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        self.items = []
        for (N, K) in ((I, H), (H, I)):
            qb = torch.randint(0, 0x7E, (G, N, K), dtype=torch.uint8, device="cuda", generator=gen)
            sb = torch.rand((G, K // 128, N // 128), device="cuda", generator=gen) * 1e-3
            qa = torch.randint(0, 0x7E, (G, cap, K), dtype=torch.uint8, device="cuda",
                               generator=gen)
            sa = torch.rand((G, K // 128, cap), device="cuda", generator=gen) * 1e-2
            ws_bytes = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, cap, N, K)
            self.items.append(dict(
                G=G, cap=cap, N=N, K=K, qb=qb, sb=sb, qa=qa, sa=sa, mm=mm,
                ws=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda"),
                c=torch.zeros((G, cap, N), dtype=torch.bfloat16, device="cuda")))
        self.flops = sum(2.0 * self.real_rows * it["N"] * it["K"] for it in self.items)

    def gemm(self, it):
        self.dg.dg_fp8_grouped_gemm_masked(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], 1,
                                           it["mm"], workspace=it["ws"])

    def step(self, i=0):
        for it in self.items:
            self.gemm(it)

    def outputs(self):
        return [it["c"] for it in self.items]

    def config(self):
        return {"workload": "masked grouped MoE GEMM (decode), 8 experts x capacity 32, 64 "
                            "tokens top-2, hidden 4096, intermediate 11008, up and down "
                            "projections, A pre-quantised 1x128",
                "masked_m": self.counts.tolist(), "real_rows": self.real_rows}

    def bytes_of(self, it):
        # weights + the valid rows of A and C + scales
        return (it["G"] * it["N"] * it["K"] + self.real_rows * (it["K"] + 2 * it["N"])
                + 4 * it["G"] * (it["K"] // 128) * (it["cap"] + it["N"] // 128))

    def breakdown(self, timer, reps):
        out = []
        for n, it in enumerate(self.items):
            t = timer.time(lambda: self.gemm(it), reps, key=("masked", n), calls=4)
            b = self.bytes_of(it)
            out.append({"nk": [it["N"], it["K"]], "gemm_us": t * 1e3,
                        "hbm_gbs": b / (t * 1e-3) / 1e9,
                        "hbm_frac": b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS})
        return out

    def roofline(self, timer, reps):
        it = self.items[0]
        t = timer.time(lambda: self.gemm(it), reps, key=("masked", 0), calls=4)
        ach = self.bytes_of(it) / (t * 1e-3) / 1e9
        return {"kernel": "masked grouped GEMM up-projection", "bound": "hbm", "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": None, "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        return None


def dpm_clocks():
    """Current shader and memory clock levels (MHz) from the amdgpu sysfs DPM
    tables of the card torch uses, or None where they are not readable."""
    import glob
    try:
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
    except Exception:
        bus = None
    cards = sorted(glob.glob("/sys/class/drm/card[0-9]*/device"))
    if bus is not None:
        cards = [c for c in cards if os.path.realpath(c).split("/")[-1].split(":")[-2:-1] ==
                 ["%02x" % bus]] or cards
    for c in cards:
        out = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(c, name)) as f:
                    cur = [ln for ln in f.read().splitlines() if ln.strip().endswith("*")]
            except OSError:
                cur = []
            if cur:
                out[name[-4:]] = cur[0].split(":", 1)[1].strip(" *")
        if out:
            out["card"] = os.path.basename(os.path.dirname(c))
            return out
    return None


def probe_lib():
    """The measurement probes' own library (not the GEMM library), or None."""
    path = os.path.join(ROOT, "fp8_block_scaled_dg_amd", "lib", "libdg_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dgp_hbm_read.restype = ctypes.c_int
    lib.dgp_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_long, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    return lib


def measured_mfma_peak(blocks=1024, iters=10000, reps=3):
    """Dense FP8 matrix-core rate this GPU sustains on a pure MFMA loop
    (4 waves per SIMD, 8 independent 16x16x128 chains per wave, pseudo-random
    E4M3 operands), and the shader clock it ran at (s_memtime cycles over the
    100 MHz s_memrealtime interval of one wave).  None without the probe."""
    import ctypes
    path = os.path.join(ROOT, "fp8_block_scaled_dg_amd", "lib", "libdg_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dgp_mfma_fp8_loop.restype = ctypes.c_int
    lib.dgp_mfma_fp8_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.dgp_mfma_fp8_loop(out.data_ptr(), clk.data_ptr(), blocks, iters,
                                   ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("MFMA probe launch failed (%d)" % rc)

    launch()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        launch()
        e.record(stream)
        e.synchronize()
        ms = s.elapsed_time(e)
        best = ms if best is None else min(best, ms)
    cycles, ticks = (int(v) for v in clk.cpu().tolist())
    flop = float(blocks) * 4 * iters * 8 * 65536
    return {"tflops": flop / (best * 1e-3) / 1e12,
            "sclk_ghz": cycles / (ticks / 100e6) / 1e9 if ticks > 0 else None,
            "what": "FP8 16x16x128 MFMA loop, %d workgroups x 4 waves, %d x 8 MFMAs per wave, "
                    "best of %d" % (blocks, iters, reps)}


def run_copy(args):
    """A plain device-to-device copy of known size (for counter calibration)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"metric": "device copy bandwidth (read+write)", "bytes_read": n,
                      "bytes_written": n, "value": 2 * n / (ms * 1e-3) / 1e9, "unit": "GB/s",
                      "ms_per_copy": ms, "n_gpus": 1, "steps": args.steps}), flush=True)


def pmc_rows(path, counter):
    """Rows of one counter from a rocprofv3 --pmc CSV (a file, or a directory
    searched for *counter_collection.csv), in dispatch order."""
    import csv
    import glob
    if os.path.isdir(path):
        found = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                 recursive=True))
        if len(found) != 1:
            raise SystemExit("expected one counter CSV under %s, found %d" % (path, len(found)))
        path = found[0]
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def last_run(rows, symbol):
    """Counter values of the last run of back-to-back launches of one library
    kernel (same symbol and grid, no other library kernel in between): under
    --roofline-only these are exactly the roofline kernel's launches, which
    come after a separating library launch.  The run's symbol must contain
    `symbol`."""
    lib = [r for r in rows if "dg::" in r["Kernel_Name"]]
    if not lib:
        raise SystemExit("no library kernel in the counter rows")
    last = (lib[-1]["Kernel_Name"], lib[-1]["Grid_Size"])
    if symbol not in last[0]:
        raise SystemExit("last library kernel is %s, expected %s" % (last[0], symbol))
    run = []
    for r in reversed(lib):
        if (r["Kernel_Name"], r["Grid_Size"]) != last:
            break
        run.append(float(r["Counter_Value"]))
    return last[0], int(last[1]) // int(lib[-1]["Workgroup_Size"]), run


def record_traffic(config, pmc_dir):
    """Write the HBM bytes per launch of `config`'s roofline kernel into
    profiles/traffic.json, from four rocprofv3 --pmc runs under pmc_dir:
    <config>_FETCH_SIZE and <config>_WRITE_SIZE of
    `bench.py --config <config> --roofline-only --kernel-reps 2`, and
    copy_FETCH_SIZE and copy_WRITE_SIZE of `bench.py --config copy`.  The
    counters of the copy (COPY_BYTES read, COPY_BYTES written) give the bytes
    each counter unit stands for; the record carries the hash of the kernel
    sources, so the bench reports it only while they are unchanged."""
    key, sources, symbol = TRAFFIC_KERNELS[config]
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        v = [float(r["Counter_Value"])
             for r in pmc_rows(os.path.join(pmc_dir, "copy_" + counter), counter)
             if "copyBuffer" in r["Kernel_Name"]]
        if not v or (max(v) - min(v)) > 0.02 * max(v):
            raise SystemExit("copy calibration for %s: values %s" % (counter, v))
        cal[counter] = COPY_BYTES / (sum(v) / len(v) * 1024.0)
    rec = {"source_sha256_16": source_hash(sources)}
    for counter, what in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        name, wgs, run = last_run(pmc_rows(os.path.join(pmc_dir, "%s_%s" % (config, counter)),
                                           counter), symbol)
        if (max(run) - min(run)) > 0.05 * max(run):
            log("note: %s per dispatch spreads %.1f .. %.1f KiB" % (counter, min(run), max(run)))
        kib = sum(run) / len(run)
        rec.update({"kernel": name, "workgroups": wgs,
                    what + "_dispatches": len(run),
                    what + "_size_kib_per_dispatch": kib,
                    what + "_calibration": cal[counter],
                    what + "_bytes": int(round(kib * 1024.0 * cal[counter]))})
    rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[key] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(json.dumps({key: rec}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="dense",
                    choices=["dense", "decode", "moe", "small", "outlier", "ue8m0", "epilogue",
                             "wgrad", "masked", "copy", "peak"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--roofline-only", action="store_true",
                    help="after the warm-up steps, launch only the roofline kernel (eager, "
                         "--kernel-reps + 1 times, after one separating library launch) and "
                         "print its figures: the run that counter passes profile")
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="no GPU: write the roofline kernel's HBM traffic for --config "
                         "(dense, decode or moe) into profiles/traffic.json from the "
                         "rocprofv3 --pmc runs under PMC_DIR")
    args = ap.parse_args()
    if args.record_traffic:
        if args.config not in TRAFFIC_KERNELS:
            raise SystemExit("--record-traffic covers %s" % sorted(TRAFFIC_KERNELS))
        record_traffic(args.config, args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.config == "copy":
        run_copy(args)
        return
    if args.config == "peak":
        mp = measured_mfma_peak()
        print(json.dumps({"metric": "measured FP8 MFMA peak", "value": mp and mp["tflops"],
                          "unit": "TFLOP/s", "published_peak": PEAK_FP8_TFLOPS,
                          "sclk_ghz": mp and mp["sclk_ghz"], "what": mp and mp["what"],
                          "n_gpus": 1}), flush=True)
        return

    import fp8_block_scaled_dg_amd as dg
    log("building inputs for", args.config)
    if args.config == "dense":
        w = Dense(dg, DENSE)
    elif args.config == "small":
        w = Dense(dg, [(128, 256, 512)])
    elif args.config == "outlier":
        w = Dense(dg, [(8192, 8192, 8192)], outlier=True)
    elif args.config == "ue8m0":
        w = Dense(dg, DENSE, ue8m0=True)
    elif args.config == "epilogue":
        w = Epilogue(dg)
    elif args.config == "wgrad":
        w = WeightGrad(dg)
    elif args.config == "decode":
        w = Decode(dg)
    elif args.config == "masked":
        w = Masked(dg)
    else:
        w = Moe(dg)
    torch.cuda.synchronize()

    log("warmup", args.warmup)
    for i in range(args.warmup):
        w.step(i)
    torch.cuda.synchronize()

    if args.roofline_only:
        # a launch of another library kernel separates the warm-up's launches
        # from the roofline kernel's
        sep = torch.zeros((16, 16), dtype=torch.uint8, device="cuda")
        dg.dg_transpose_fp8(torch.empty_like(sep), sep)
        roof = w.roofline(Timer(False), args.kernel_reps)
        torch.cuda.synchronize()
        print(json.dumps({"metric": "roofline kernel alone (eager launches)",
                          "config": w.config(), "roofline": roof}), flush=True)
        return

    use_graph = not args.no_graph
    timer = Timer(use_graph)
    rounds = args.steps
    per = 1
    if use_graph:
        # one graph = per x w.rot consecutive steps (w.rot rotation states),
        # per chosen to divide the step count: each replay also pays the
        # runtime's graph launch and end-of-graph synchronisation (about
        # 45 us on MI355X), which a single step per graph would charge to
        # every step.  Replays are verified against eager execution.
        rounds = cdiv(args.steps, w.rot)
        per = next(p for p in (4, 5, 2, 3, 1) if rounds % p == 0)
        eager = []
        for i in range(w.rot):
            w.step(i)
        torch.cuda.synchronize()
        eager = [t.clone() for t in w.outputs()]
        g = timer.graph("step", lambda: [w.step(i % w.rot) for i in range(per * w.rot)])
        for _ in range(3):
            for t in w.outputs():
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(x, y) for x, y in zip(w.outputs(), eager)):
                log("graph replay differs from eager execution: timing eager launches")
                use_graph = False
                timer = Timer(False)
                break
    steps = rounds * w.rot if use_graph else args.steps
    clocks_before = dpm_clocks()
    log("timing", steps, "steps", "(graph of %d steps)" % (per * w.rot) if use_graph else "(eager)")
    t0 = time.perf_counter()
    if use_graph:
        ms = timer.time(lambda: [w.step(i % w.rot) for i in range(per * w.rot)], rounds // per,
                        key="step") / (per * w.rot)
    else:
        ms = timer.time(w.step, steps)
    wall = time.perf_counter() - t0
    clocks_after = dpm_clocks()
    log("step %.4f ms (wall %.2f s)" % (ms, wall))

    breakdown = w.breakdown(timer, args.kernel_reps)
    roof = w.roofline(timer, args.kernel_reps)
    if roof["bound"] == "mfma":
        mp = measured_mfma_peak()
        if mp is not None:
            roof["measured_peak"] = mp["tflops"]
            roof["frac_of_measured_peak"] = roof["achieved"] / mp["tflops"]
            roof["measured_peak_sclk_ghz"] = mp["sclk_ghz"]
            roof["measured_peak_what"] = mp["what"]
    log("roofline", roof)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        cpu = w.cpu_baseline()

    rec = {"metric": "FP8 block-scaled GEMM TFLOPS", "value": w.flops / (ms * 1e-3) / 1e12,
           "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
           "config": dict(w.config(), timing=("hip graph replay, %d steps per graph" % (per * w.rot))
                          if use_graph else "eager"),
           "roofline": roof, "cpu_baseline": cpu, "breakdown": breakdown,
           "clocks": {"before": clocks_before, "after": clocks_after}}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
