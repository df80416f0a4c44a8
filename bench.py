#!/usr/bin/env python3
"""Benchmark of liblinattn on one MI355X.

Default workload (the causal D=128 streaming case): B=256 H=32 Dk=Dv=128 bf16,
elu+1, normalized; one step = reset the fp32 state, four chained 1024-token
causal prefill calls (state updated in place), then 512 T=1 decode steps on the
same state.  Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line:
  value            prefill tokens/s (B*4096 tokens / prefill time of a step)
  prefill          prefill kernel duration, HBM GB/s, MFMA utilisation
  decode           decode kernel duration and state-streaming HBM GB/s
  roofline         the dominant kernel by time in a step (the decode kernel),
                   algorithmic bytes per launch / average launch duration
  roofline_prefill the same for the prefill kernel
  cpu_baseline     the fp64 oracle on a bounded sample of the same prefill
Kernel durations come from HIP events recorded on the stream the library
launches on (torch's current stream) at the boundaries of each phase of every
timed step: mean launch duration = phase time / launches in the phase.

--workload selects one of the other workloads for an extra measurement line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
MFMA_16x16x32_FLOPS = 2 * 16 * 16 * 32

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kernelized_linear_attention_chunked_amd", "csrc")


def _src_sha(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel, src, launches_per_record=1):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    when the summary is missing or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, kernel + "_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != _src_sha(src):
        return None
    return rec.get("traffic_bytes_per_launch")


def prefill_mfma_per_chunk(D=128, norm=True):
    """MFMA instructions one workgroup issues per 64-token chunk in the causal
    prefill kernel (bf16, v_mfma_f32_16x16x32_bf16), from its tiling.  Query
    block qr (16 rows) forms A^T over key pairs of 32 up to its diagonal, 2
    tiles per pair x D/32 steps, once per value half (two halves at D=128).
    Each value half's waves hold their D/32 value tiles plus the normaliser
    tile (both halves form the denominator they divide by): intra V^T A^T,
    pairs x tiles x 2 (hi/lo of A); inter S^T phiQ^T, tiles x D/32 per query
    block.  State update: (D/16)(D/16 + norm) tiles x 2 token steps.  At D=128
    this gives 520 per chunk, which rocprofv3's SQ_INSTS_VALU_MFMA_MOPS_BF16
    reproduces exactly (profiles/causal_prefill_kernel_mfma.md)."""
    halves = 2 if D >= 128 else 1
    tiles = D // 16 // halves + (1 if norm else 0)   # a wave's value tiles (+ normaliser)
    nq = D // 32
    pairs = [(16 * qr + 15) // 32 + 1 for qr in range(4)]
    a_t = halves * sum(2 * p for p in pairs) * nq
    intra = halves * sum(pairs) * tiles * 2
    inter = halves * 4 * tiles * nq
    upd = (D // 16) * (D // 16 + (1 if norm else 0)) * 2
    return a_t + intra + inter + upd


def _profile_record(name, src):
    """A committed rocprofv3 summary (profiles/<name>.json) if the kernel source
    is unchanged since it was taken, else None."""
    path = os.path.join(PROFILES, name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("kernel_src_sha") == _src_sha(src) else None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _elapsed_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def cpu_baseline_streaming(d, target_s, log):
    """fp64 oracle (as it stands) on a bounded sample of the prefill: the first
    n (batch, head) units, 4096 tokens each; n sized for ~target_s seconds."""
    import numpy as np
    import torch

    import oracle

    H = d.H
    q, k, v = d.qc, d.kc, d.vc

    def units(nb):
        # nb whole batch rows (all H heads), all 4096 tokens, as float64 on the host
        cat = lambda parts: torch.cat([p[:nb] for p in parts], 1).to("cpu", torch.float64).numpy()
        return cat(q), cat(k), cat(v)

    qs, ks, vs = units(1)
    t0 = time.perf_counter()
    oracle.causal(qs, ks, vs)
    t1 = time.perf_counter() - t0
    nb = int(max(1, min(d.B, round(target_s / max(t1, 1e-3)))))
    log("cpu_baseline: 1 batch row (%d units) took %.2f s; timing %d rows" % (H, t1, nb))
    if nb > 1:
        qs, ks, vs = units(nb)
        t0 = time.perf_counter()
        oracle.causal(qs, ks, vs)
        t1 = time.perf_counter() - t0
    tokens = nb * H * d.T
    return {"value": tokens / t1, "unit": "tokens/s", "cores": oracle.max_threads(),
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "kind": "oracle", "seconds": round(t1, 3),
            "sample": "%d of %d (batch, head) units x %d prefill tokens (batch rows 0..%d), "
                      "fp64 per-token recurrence" % (nb * H, d.B * H, d.T, nb - 1)}


def bench_streaming(args, log):
    import torch

    from kernelized_linear_attention_chunked_amd import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    d = workloads.StreamingD128(dev)
    B, H, D, T, Td, C = d.B, d.H, d.D, d.T, d.Td, d.chunk
    n_chunks = T // C
    log("streaming_d128: B=%d H=%d D=%d, %d x %d prefill + %d decode" % (B, H, D, n_chunks, C, Td))
    for _ in range(args.warmup):
        d.step()
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)
    # events only at phase boundaries: a marker between every launch would add
    # its own few microseconds to each short decode launch
    steps = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        s0, r1, mid, s1 = E(), E(), E(), E()
        s0.record()
        d.reset_state()
        r1.record()
        for i in range(n_chunks):
            d.prefill_call(i)
        mid.record()
        for t in range(Td):
            d.decode_call(t)
        s1.record()
        steps.append((s0, r1, mid, s1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    mean = lambda xs: sum(xs) / len(xs)
    prefill_step_ms = mean([s0.elapsed_time(mid) for s0, _, mid, _ in steps])
    pf_kernel_ms = mean([r1.elapsed_time(mid) for _, r1, mid, _ in steps]) / n_chunks
    decode_ms = [mid.elapsed_time(s1) for _, _, mid, s1 in steps]
    dc_kernel_ms = mean(decode_ms) / Td

    # algorithmic bytes / flops per launch
    units = B * H
    pf_bytes = units * C * D * 2 * 4 + units * (D * D + D) * 4 * 2      # q,k,v,out + state in/out
    dc_bytes = units * (D * D + D) * 4 * 2 + units * D * 2 * 4          # state in/out + q,k,v,out
    pf_exec_flops = units * (C // 64) * prefill_mfma_per_chunk(D) * MFMA_16x16x32_FLOPS
    pf_alg_flops = units * C * (2 * 64 * (D + D) + 4 * D * D)           # dense 64x64 tiles + 4 Dk Dv
    pf_gbs = pf_bytes / (pf_kernel_ms * 1e-3) / 1e9
    dc_gbs = dc_bytes / (dc_kernel_ms * 1e-3) / 1e9
    prefill_tps = B * T / (prefill_step_ms * 1e-3)

    dc_traffic = _traffic("decode_kernel", "la_decode.hip")
    pf_traffic = _traffic("causal_prefill_kernel", "la_chunk.hip")
    mfma_prof = _profile_record("causal_prefill_kernel_mfma", "la_chunk.hip")
    rec = {
        "metric": "prefill tokens/s + MFMA util (causal, D=128); decode state HBM GB/s",
        "value": prefill_tps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "streaming causal elu+1 normalized linear attention: "
                               "4 x 1024-token prefill calls + 512 T=1 decode steps, fp32 state",
                   "B": B, "H": H, "Dk": D, "Dv": D, "prefill_tokens": T, "prefill_call_tokens": C,
                   "decode_steps": Td, "feature_map": "elu_plus_one", "eps": 1e-6},
        "prefill": {"tokens_per_s": prefill_tps, "ms_per_step": prefill_step_ms,
                    "kernel_ms": pf_kernel_ms, "hbm_GBps": pf_gbs, "hbm_frac": pf_gbs / HBM_PEAK_GBS,
                    "mfma_util_executed": pf_exec_flops / (pf_kernel_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                    "mfma_util_algorithmic": pf_alg_flops / (pf_kernel_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                    "executed_mfma_TFLOPs": pf_exec_flops / (pf_kernel_ms * 1e-3) / 1e12,
                    "executed_mfma_per_chunk": prefill_mfma_per_chunk(D),
                    # SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs, from the committed
                    # rocprofv3 pass of this kernel source (null if it changed since)
                    "mfma_busy_rocprof": None if mfma_prof is None else mfma_prof["mfma_busy"],
                    # the most MFMA-busy this 64-token-chunk kernel can honestly be
                    # while moving its bytes at the 8 TB/s HBM bound: executed bf16
                    # MFMA time at peak / HBM time for the algorithmic bytes
                    "mfma_busy_ceiling_at_hbm_bound": (pf_exec_flops / (BF16_PEAK_TFLOPS * 1e12))
                                                      / (pf_bytes / (HBM_PEAK_GBS * 1e9)),
                    "mfma_target_note": "a 50% MFMA target is above this chunk size's HBM-bound ceiling; "
                                        "MFMA utilisation is reported as measured"},
        "decode": {"kernel_us": dc_kernel_ms * 1e3, "ms_per_step": mean(decode_ms),
                   "state_GBps": units * (D * D + D) * 8 / (dc_kernel_ms * 1e-3) / 1e9,
                   "hbm_GBps": dc_gbs, "hbm_frac": dc_gbs / HBM_PEAK_GBS,
                   "tokens_per_s": B * Td / (mean(decode_ms) * 1e-3)},
        "roofline": {"kernel": "decode_kernel<bf16,128,elu+1,norm>", "bound": "hbm",
                     "achieved": dc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dc_gbs / HBM_PEAK_GBS, "traffic": dc_traffic,
                     "algorithmic_bytes_per_launch": dc_bytes},
        "roofline_prefill": {"kernel": "chunk_kernel<bf16,128,elu+1,norm,causal>", "bound": "hbm",
                             "achieved": pf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": pf_gbs / HBM_PEAK_GBS, "traffic": pf_traffic,
                             "algorithmic_bytes_per_launch": pf_bytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_streaming(d, args.cpu_baseline_seconds, log)
    return rec


def cpu_baseline_workload(d, name, target_s, log):
    """The fp64 oracle (as it stands) on a bounded sample of a workload's own
    inputs: whole batch rows (all heads), as many as fit about target_s
    seconds, scaled to tokens/s of the same kind as the GPU figure."""
    import numpy as np
    import torch

    import oracle

    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()

    def run(nb):
        """Oracle time for batch rows 0..nb-1, and the tokens they cover."""
        if name in ("causal_bf16_d64", "causal_fp32_small"):
            q, k, v = (f64(t[:nb]) for t in (d.q, d.k, d.v))
            t0 = time.perf_counter()
            oracle.causal(q, k, v)
            return time.perf_counter() - t0, nb * d.T
        if name == "noncausal_relu_d128":
            q, k, v = (f64(t[:nb]) for t in (d.q, d.k, d.v))
            m = d.mask[:nb].cpu().numpy()
            t0 = time.perf_counter()
            oracle.noncausal(q, k, v, m, "relu", True, 1e-6)
            return time.perf_counter() - t0, nb * d.T
        if name == "backward_bf16_d64":
            q, k, v, dy = (f64(t[:nb]) for t in (d.q, d.k, d.v, d.dy))
            t0 = time.perf_counter()
            oracle.causal_backward(q, k, v, dy)
            return time.perf_counter() - t0, nb * d.T
        if name in ("gated_step_d128", "delta_step_d128"):
            # step-major inputs (T, B, ...): the oracle runs the same tokens per row
            tb = lambda t: f64(t[:, :nb].transpose(0, 1))
            beta = tb(d.beta) if name == "delta_step_d128" else None
            rule = "gated_delta" if name == "delta_step_d128" else "gated"
            past = f64(d.state[:nb])
            args_ = (tb(d.q), tb(d.k), tb(d.v), d.Hq, d.Hkv, rule)
            t0 = time.perf_counter()
            oracle.la_op(*args_, decay=tb(d.g), beta=beta, past_state=past, scale=d.scale)
            return time.perf_counter() - t0, nb * d.T
        # gated, per-dim, gated delta: packed (B, T, ...) inputs
        rule = "gated_delta" if name == "gated_delta_d128" else "gated"
        beta = f64(d.beta[:nb]) if name == "gated_delta_d128" else None
        q, k, v, g = (f64(t[:nb]) for t in (d.q, d.k, d.v, d.g))
        t0 = time.perf_counter()
        oracle.la_op(q, k, v, d.Hq, d.Hkv, rule, decay=g, beta=beta, scale=d.scale)
        return time.perf_counter() - t0, nb * d.T

    # the row is the unit of the sample; long rows are cut to a token prefix
    t1, tok1 = run(1)
    nb = int(max(1, min(d.B, round(target_s / max(t1, 1e-3)))))
    log("cpu_baseline %s: 1 batch row took %.2f s; timing %d rows" % (name, t1, nb))
    if nb > 1:
        t1, tok1 = run(nb)
    return {"value": tok1 / t1, "unit": "tokens/s", "cores": oracle.max_threads(), "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(), "kind": "oracle", "seconds": round(t1, 3),
            "sample": "batch rows 0..%d of %d (all heads), every token of the workload's step" % (nb - 1, d.B)}


def bench_other(args, log):
    """One extra line for a non-default workload: median step time over at least 20
    timed steps after at least 3 warm-up steps and 0.3 s of warm-up, tokens/s, algorithmic GB/s and the
    dense-tile MFMA flops as a fraction of the bf16 peak.  The causal D=64
    workload fits the 256 MB Infinity Cache, so it is also timed cold, rotating
    over 8 input sets (about 0.54 GB)."""
    import torch

    from kernelized_linear_attention_chunked_amd import workloads

    torch.cuda.set_device(0)
    d = workloads.DRIVERS[args.workload]("cuda:0")
    reps, warm = max(args.steps, 20), max(args.warmup, 3)
    E = lambda: torch.cuda.Event(enable_timing=True)

    def median_ms(drivers):
        # warm up for at least 0.3 s: the first few dozen steps of these short
        # workloads run measurably slower than the steady state
        t_w, i = time.perf_counter(), 0
        while i < warm or time.perf_counter() - t_w < 0.3:
            drivers[i % len(drivers)].step()
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = []
        for i in range(reps):
            a, b = E(), E()
            a.record()
            drivers[i % len(drivers)].step()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        return sorted(_elapsed_ms(ev))[reps // 2]

    t0 = time.perf_counter()
    ms = median_ms([d])
    wall = time.perf_counter() - t0
    D, Tt = d.D, d.B * d.T
    extra = {}
    if args.workload == "gated_step_d128":
        # per token step: the fp32 state read and written once, plus q, k, v, decay, out
        U = d.B * d.Hkv
        nbytes = d.T * (U * D * D * 4 * 2 + d.B * (d.Hq * D * 2 * 2 + d.Hkv * D * 2 * 2 + d.Hkv * 2))
        flops = d.T * (U * D * D * 3 + d.B * d.Hq * D * D * 2)  # update (3/elem), readout
    elif args.workload == "delta_step_d128":
        # the gated step's bytes plus beta; per state element: decay, S'^T k, the
        # rank-1 update (1 + 2 + 2 flops), plus the readout
        U = d.B * d.Hkv
        nbytes = d.T * (U * D * D * 4 * 2 + d.B * (d.Hq * D * 2 * 2 + d.Hkv * D * 2 * 2 + d.Hkv * 2 * 2))
        flops = d.T * (U * D * D * 5 + d.B * d.Hq * D * D * 2)
    elif args.workload == "gated_delta_d128":
        # q, k, v, out, decay and beta once; the final state written
        nbytes = Tt * (d.Hq * D * 2 * 2 + d.Hkv * D * 2 * 2 + d.Hkv * 2 * 2) + d.B * d.Hkv * D * D * 4
        # per token and q head: intra (64-wide A tile and A U) and inter; per kv head:
        # R (Kbar S), the key tiles (64 wide), the update, and the solve's products
        flops = Tt * d.Hq * (2 * 64 * 2 * D + 2 * D * D) + Tt * d.Hkv * (2 * D * D * 2 + 2 * 64 * D * 2)
    elif args.workload == "backward_bf16_d64":
        # q, k, v, dy read and dq, dk, dv written once (bf16); the state gradient
        nbytes = Tt * d.H * D * 2 * 7 + d.B * d.H * (D * D + D) * 4
        # three linear-rule recurrences: per token a 64-wide intra tile, A V and
        # the inter and state products (2 D D each)
        flops = 3 * Tt * d.H * (2 * 64 * D * 2 + 4 * D * D)
    elif args.workload in ("gated_gqa_d128", "gated_perdim_d128", "gated_perdim_f32_d128"):
        per_dim = args.workload != "gated_gqa_d128"
        esz = d.q.element_size()
        nbytes = (Tt * (d.Hq * D * esz * 2 + d.Hkv * D * esz * 2 + d.Hkv * (D if per_dim else 1) * esz)
                  + d.B * d.Hkv * D * D * 4)
        # dense 64x64 intra tiles per q head plus inter and state update (2 Dk Dv each)
        flops = Tt * d.Hq * (2 * 64 * 2 * D + 2 * D * D) + Tt * d.Hkv * 2 * D * D
    elif args.workload == "noncausal_relu_d128":
        # the kernels skip masked tokens' reads (whole 64-token chunks of k and v,
        # 16-row blocks of q): q, k, v read for the valid tokens, every output
        # row written (zeros where masked), the mask read
        valid = int(d.lengths.sum())
        nbytes = valid * d.H * D * 2 * 3 + Tt * d.H * D * 2 + Tt
        flops = valid * d.H * (2 * D * (D + 1) * 2)  # reduce (phiK^T V, Z) and readout
        extra = {"valid_tokens": valid, "valid_fraction": valid / Tt,
                 "bytes_note": "bytes count q, k, v of valid tokens only (what the kernels read)"}
    else:
        nbytes = Tt * d.H * D * 2 * 4 + d.B * d.H * (D * D + D) * 4
        flops = Tt * d.H * (2 * 64 * (D + D) + 4 * D * D)
    rec = {"metric": "tokens/s", "value": d.prefill_tokens / (ms * 1e-3), "unit": "tokens/s",
           "n_gpus": 1, "steps": reps, "warmup": warm,
           "ms_per_step": wall * 1e3 / (reps + warm), "step_kernel_ms": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": args.workload},
           "algorithmic_GBps": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "mfma_util_algorithmic": flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), **extra}
    if d.q.dtype.itemsize == 4:
        rec["dtype"] = "f32"
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_workload(d, args.workload, args.cpu_baseline_seconds, log)
    if args.workload == "causal_bf16_d64":
        cold = [d] + [workloads.DRIVERS[args.workload]("cuda:0") for _ in range(7)]
        ms_cold = median_ms(cold)
        rec["warm_step_kernel_ms"] = ms
        rec["cold_step_kernel_ms"] = ms_cold
        rec["cold_tokens_per_s"] = d.prefill_tokens / (ms_cold * 1e-3)
        rec["cold_algorithmic_GBps"] = nbytes / (ms_cold * 1e-3) / 1e9
        rec["cold"] = "8 rotating input sets, about 0.54 GB, beyond the 256 MB Infinity Cache"
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="streaming_d128",
                    choices=["streaming_d128", "causal_bf16_d64", "noncausal_relu_d128",
                             "gated_gqa_d128", "gated_perdim_d128", "gated_perdim_f32_d128",
                             "gated_delta_d128", "backward_bf16_d64", "gated_step_d128",
                             "delta_step_d128"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times) and "
                         "exit: the reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU only (--gpus 1): this library has no multi-GPU path; "
                 "the per-GPU kernel is the same at any GPU count")
    log = lambda m: print("[bench] " + m, file=sys.stderr, flush=True)
    if args.workload == "streaming_d128":
        rec = bench_streaming(args, log)
    else:
        rec = bench_other(args, log)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
