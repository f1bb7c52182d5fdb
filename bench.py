"""Benchmark of the FP8 E4M3 block-scaled GEMM hot path on one MI355X.

Default workload (--config dense): the dense LLM projection GEMMs
(M, N, K) in {(4096, 7168, 2048), (4096, 4096, 7168), (8192, 8192, 8192)},
A ~ N(0, 1), B ~ N(0, 0.02^2), both quantised with 128x128 block scales,
BF16 output.  One step = for every shape: quantise A (FP32 -> E4M3 + scales),
quantise B, and the block-scaled GEMM, i.e. every stage of the path.  The
inputs are resident in HBM before timing starts.

value = total GEMM FLOP of a step (2*M*N*K summed) / step time, in TFLOP/s.

Other workloads, each printing its own JSON line: --config decode (M in
{1,16,64} x (N,K) in {(24576,1536),(7168,16384),(4096,4096)}, 1x128
activation scales, weights rotated through buffers larger than the caches),
--config moe (8 experts, 1024 tokens top-2, up and down projections),
--config small (128x256x512).

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
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

DENSE = [(4096, 7168, 2048), (4096, 4096, 7168), (8192, 8192, 8192)]
DECODE = [(m, n, k) for (n, k) in [(24576, 1536), (7168, 16384), (4096, 4096)] for m in (1, 16, 64)]


def cdiv(a, b):
    return (a + b - 1) // b


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class EventTimer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self):
        self.stream = torch.cuda.current_stream()

    def time(self, fn, reps: int) -> float:
        """Average milliseconds per call over `reps` back-to-back calls."""
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(self.stream)
        for _ in range(reps):
            fn()
        e.record(self.stream)
        e.synchronize()
        return s.elapsed_time(e) / reps


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class Dense:
    name = "dense"

    def __init__(self, dg, shapes, seed=0):
        self.dg = dg
        self.items = []
        for (M, N, K) in shapes:
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=0)).cuda()
            b = torch.from_numpy(datagen.normal((N, K), 0.02, seed=seed, stream=1)).cuda()
            it = dict(M=M, N=N, K=K, a=a, b=b,
                      qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                      qb=torch.empty((N, K), dtype=torch.uint8, device="cuda"),
                      sa=torch.empty((K // 128, cdiv(M, 128)), dtype=torch.float32, device="cuda"),
                      sb=torch.empty((K // 128, cdiv(N, 128)), dtype=torch.float32, device="cuda"),
                      c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
            self.items.append(it)
        self.flops = sum(2.0 * it["M"] * it["N"] * it["K"] for it in self.items)

    def quant_a(self, it):
        self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 128)

    def quant_b(self, it):
        self.dg.dg_quantize_fp8_block(it["qb"], it["sb"], it["b"], 128)

    def gemm(self, it):
        self.dg.dg_fp8_gemm_nt(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], 128)

    def step(self):
        for it in self.items:
            self.quant_a(it)
            self.quant_b(it)
            self.gemm(it)

    def config(self):
        return {"workload": "dense LLM projection GEMMs, E4M3 128x128 block scales, BF16 out",
                "shapes_mnk": [[it["M"], it["N"], it["K"]] for it in self.items],
                "a_scales": "128x128", "b_scales": "128x128",
                "step": "quantise A + quantise B + GEMM, per shape",
                "inputs": "A ~ N(0,1), B ~ N(0,0.02^2), float32, seed 0"}

    def breakdown(self, timer, reps):
        out = []
        for it in self.items:
            M, N, K = it["M"], it["N"], it["K"]
            tq_a = timer.time(lambda: self.quant_a(it), reps)
            tq_b = timer.time(lambda: self.quant_b(it), reps)
            tg = timer.time(lambda: self.gemm(it), reps)
            qbytes_a = M * K * 5 + 4 * (K // 128) * cdiv(M, 128)
            qbytes_b = N * K * 5 + 4 * (K // 128) * cdiv(N, 128)
            out.append({"mnk": [M, N, K],
                        "gemm_us": tg * 1e3, "gemm_tflops": 2.0 * M * N * K / (tg * 1e-3) / 1e12,
                        "quant_a_us": tq_a * 1e3,
                        "quant_a_gbs": qbytes_a / (tq_a * 1e-3) / 1e9,
                        "quant_b_us": tq_b * 1e3,
                        "quant_b_gbs": qbytes_b / (tq_b * 1e-3) / 1e9})
        return out

    def roofline(self, timer, reps):
        """Dominant kernel: the GEMM launch on the largest shape."""
        it = max(self.items, key=lambda t: t["M"] * t["N"] * t["K"])
        t = timer.time(lambda: self.gemm(it), reps)
        flop = 2.0 * it["M"] * it["N"] * it["K"]
        ach = flop / (t * 1e-3) / 1e12
        return {"kernel": "gemm_tiled_kernel<256,128,false> M=N=K=8192" if it["M"] == 8192 else
                "gemm_tiled_kernel %s" % [it["M"], it["N"], it["K"]],
                "bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_FP8_TFLOPS, "traffic": None, "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        """The oracle (single thread, plain C) on a bounded sample: per shape,
        quantise all of B and one 128-row block of A, and compute one full
        output row; extrapolate to the whole step (B quantised once, A in
        M/128 blocks, M output rows)."""
        import oracle
        total = 0.0
        for it in self.items:
            M, N, K = it["M"], it["N"], it["K"]
            a = datagen.normal((128, K), 1.0, seed=0, stream=0)
            b = it["b"].cpu().numpy()
            t0 = time.perf_counter()
            qb, sb = oracle.quantize(b, 128)
            t1 = time.perf_counter()
            qa, sa = oracle.quantize(a, 128)
            t2 = time.perf_counter()
            oracle.gemm_nt_points(qa, sa, qb, sb, np.zeros(N, np.int64), np.arange(N),
                                  a_block_rows=128)
            t3 = time.perf_counter()
            total += (t1 - t0) + (M / 128) * (t2 - t1) + M * (t3 - t2)
        return {"value": self.flops / total / 1e12, "unit": "TFLOP/s", "cores": 1,
                "kind": "oracle",
                "sample": "per shape: oracle quantise of all of B and one 128-row block of A, "
                          "one full output row of the FP64 dequantised GEMM; extrapolated to "
                          "the full step (%.1f s extrapolated)" % total}


class Decode:
    name = "decode"

    def __init__(self, dg, rotate_bytes=768 << 20, seed=0):
        self.dg = dg
        self.items = []
        for (M, N, K) in DECODE:
            wbytes = N * K
            copies = max(2, cdiv(rotate_bytes, wbytes))
            qb = torch.randint(0, 0x7E, (copies, N, K), dtype=torch.uint8, device="cuda")
            sb = torch.rand((copies, K // 128, N // 128), device="cuda") * 1e-3
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=M)).cuda()
            qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
            sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
            ws_bytes = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
            c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            self.items.append(dict(M=M, N=N, K=K, qb=qb, sb=sb, a=a, qa=qa, sa=sa, c=c, ws=ws,
                                   copies=copies, i=0))
        self.flops = sum(2.0 * it["M"] * it["N"] * it["K"] for it in self.items)

    def gemm(self, it):
        i = it["i"]
        it["i"] = (i + 1) % it["copies"]
        self.dg.dg_fp8_gemm_nt(it["c"], it["qa"], it["qb"][i], it["sa"], it["sb"][i], 1,
                               workspace=it["ws"])

    def quant(self, it):
        self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 1)

    def step(self):
        for it in self.items:
            self.quant(it)
            self.gemm(it)

    def config(self):
        return {"workload": "decode-shaped GEMMs, M in {1,16,64} x (N,K) in {(24576,1536),"
                            "(7168,16384),(4096,4096)}, A 1x128 scales, B 128x128 scales",
                "step": "quantise A + GEMM per shape; weights rotated over >768 MB of copies"}

    def breakdown(self, timer, reps):
        out = []
        for it in self.items:
            M, N, K = it["M"], it["N"], it["K"]
            t = timer.time(lambda: self.gemm(it), reps)
            byts = N * K + M * K + 4 * (K // 128) * (M + N // 128) + 2 * M * N
            out.append({"mnk": [M, N, K], "gemm_us": t * 1e3, "hbm_gbs": byts / (t * 1e-3) / 1e9,
                        "hbm_frac": byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS})
        return out

    def roofline(self, timer, reps):
        it = max(self.items, key=lambda t: t["N"] * t["K"] * 1000 + t["M"])
        t = timer.time(lambda: self.gemm(it), reps)
        M, N, K = it["M"], it["N"], it["K"]
        byts = N * K + M * K + 4 * (K // 128) * (M + N // 128) + 2 * M * N
        ach = byts / (t * 1e-3) / 1e9
        return {"kernel": "decode GEMM %s" % [M, N, K], "bound": "hbm", "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": None, "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        return None


class Moe:
    name = "moe"

    def __init__(self, dg, seed=0):
        self.dg = dg
        G, tokens, H, I = 8, 1024, 4096, 11008
        r = datagen.moe_routing(tokens, G, 2, align=128, seed=seed)
        mi = torch.from_numpy(r["m_indices"]).cuda()
        M = mi.shape[0]
        self.real_rows = int((r["m_indices"] >= 0).sum())
        self.items = []
        for (N, K) in ((I, H), (H, I)):
            qb = torch.randint(0, 0x7E, (G, N, K), dtype=torch.uint8, device="cuda")
            sb = torch.rand((G, K // 128, N // 128), device="cuda") * 1e-3
            a = torch.from_numpy(datagen.normal((M, K), 1.0, seed=seed, stream=K)).cuda()
            a[mi < 0] = 0
            self.items.append(dict(M=M, N=N, K=K, qb=qb, sb=sb, a=a, mi=mi,
                                   qa=torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                                   sa=torch.empty((K // 128, M), dtype=torch.float32, device="cuda"),
                                   c=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        self.flops = sum(2.0 * self.real_rows * it["N"] * it["K"] for it in self.items)

    def gemm(self, it):
        self.dg.dg_fp8_grouped_gemm_contig(it["c"], it["qa"], it["qb"], it["sa"], it["sb"], 1,
                                           it["mi"])

    def step(self):
        for it in self.items:
            self.dg.dg_quantize_fp8_block(it["qa"], it["sa"], it["a"], 1)
            self.gemm(it)

    def config(self):
        return {"workload": "grouped MoE GEMM, M-contiguous, 8 experts, 1024 tokens top-2, "
                            "hidden 4096, intermediate 11008, up and down projections",
                "m_total": self.items[0]["M"], "real_rows": self.real_rows}

    def breakdown(self, timer, reps):
        out = []
        for it in self.items:
            t = timer.time(lambda: self.gemm(it), reps)
            byts = 8 * it["N"] * it["K"] + it["M"] * it["K"] + 2 * it["M"] * it["N"]
            out.append({"nk": [it["N"], it["K"]], "gemm_us": t * 1e3,
                        "tflops_real_rows": 2.0 * self.real_rows * it["N"] * it["K"] / (t * 1e-3) / 1e12,
                        "hbm_gbs": byts / (t * 1e-3) / 1e9})
        return out

    def roofline(self, timer, reps):
        it = self.items[0]
        t = timer.time(lambda: self.gemm(it), reps)
        byts = 8 * it["N"] * it["K"] + it["M"] * it["K"] + 2 * it["M"] * it["N"]
        ach = byts / (t * 1e-3) / 1e9
        return {"kernel": "grouped GEMM up-projection", "bound": "hbm", "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": None, "avg_launch_us": t * 1e3}

    def cpu_baseline(self):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="dense", choices=["dense", "decode", "moe", "small"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import fp8_block_scaled_dg_amd as dg
    torch.cuda.set_device(0)
    log("building inputs for", args.config)
    if args.config == "dense":
        w = Dense(dg, DENSE)
    elif args.config == "small":
        w = Dense(dg, [(128, 256, 512)])
    elif args.config == "decode":
        w = Decode(dg)
    else:
        w = Moe(dg)
    torch.cuda.synchronize()

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    log("timing", args.steps, "steps")
    timer = EventTimer()
    t0 = time.perf_counter()
    ms = timer.time(w.step, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("step %.3f ms (wall %.2f s)" % (ms, wall))

    breakdown = w.breakdown(timer, args.kernel_reps)
    roof = w.roofline(timer, args.kernel_reps)
    log("roofline", roof)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        cpu = w.cpu_baseline()

    rec = {"metric": "FP8 block-scaled GEMM TFLOPS", "value": w.flops / (ms * 1e-3) / 1e12,
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
           "config": w.config(), "roofline": roof, "cpu_baseline": cpu,
           "breakdown": breakdown}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
