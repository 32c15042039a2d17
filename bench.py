#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 top-k MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode16]

One step = one moe_fp4_forward call (routing, FC1 + SwiGLU, FC2, router-
weighted combine) over one batch of synthetic input already resident in HBM.
The default workload is the W4A16 NVFP4 group16 decode layer (T=64 tokens,
E=256 experts, top-8, H=6144, I=2048).  Prints ONE JSON line with tokens/s,
the HBM roofline of the dominant kernel (HIP events recorded by the library
on the launch stream around each stage), the whole-forward roofline, the
FP64 oracle timed on the host cores on a bounded sample (cpu_baseline, and
its group16 -> group32 requantisation as cpu_baseline_requant), and
secondary figures for the other workloads of the hot path (FP8xFP4 decode,
prefill, group16 -> group32 requantisation of the whole layer).
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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 MoE fwd tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill) vs peak"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
WORKLOAD_TEXT = {
    "tiny": "tiny MoE: T=32 E=8 top-2 H=512 I=256, bf16 x, E2M1 + E4M3 k16, global scale 1 (latency only)",
    "decode16": "W4A16 NVFP4 decode: T=64 E=256 top-8 H=6144 I=2048, bf16 x, E2M1 + E4M3 k16 + fp32 global",
    "decode32": "FP8xFP4 decode: T=256 E=256 top-8 H=6144 I=2048, E4M3+UE8M0 k32 x, E2M1 + UE8M0 k32",
    "decode32_a4": "A4 decode: T=256 E=256 top-8 H=6144 I=2048, bf16 x quantised by the library to MXFP4 "
                   "(E2M1+UE8M0 k32), h MXFP4, E2M1 + UE8M0 k32 weights",
    "decode16_fused": "W4A16 NVFP4 decode as decode16, FC1 and FC2 in one persistent launch "
                      "(moe_fp4_forward_fused)",
    "decode32_fused": "FP8xFP4 decode as decode32, FC1 and FC2 in one persistent launch (moe_fp4_forward_fused)",
    "prefill32": "prefill: T=8192 E=256 top-8 Zipf(1.1) H=6144 I=2048, E4M3+UE8M0 k32 x, E2M1 + UE8M0 k32",
    "prefill32_bf16q": "prefill: T=8192 E=256 top-8 Zipf(1.1) H=6144 I=2048, bf16 x quantised by the "
                       "library to E4M3+UE8M0 k32, E2M1 + UE8M0 k32",
    "prefill32_a4": "A4 prefill: T=8192 E=256 top-8 Zipf(1.1) H=6144 I=2048, bf16 x quantised by the "
                    "library to MXFP4 (E2M1+UE8M0 k32), h MXFP4, E2M1 + UE8M0 k32 weights",
    "prefill32_prep": "prefill: T=8192 E=256 top-8 Zipf(1.1) H=6144 I=2048, E4M3+UE8M0 k32 x, E2M1 + UE8M0 "
                      "k32 weights in the GEMM layout (moe_fp4_prepare_gemm_weights, not timed)",
    "prefill32_a4_prep": "A4 prefill: T=8192 E=256 top-8 Zipf(1.1) H=6144 I=2048, bf16 x quantised by the "
                         "library to MXFP4, h MXFP4, E2M1 + UE8M0 k32 weights in the GEMM layout",
}
DTYPE = {"decode16": "f16", "decode32": "fp8xfp4", "decode32_a4": "fp4xfp4", "prefill32": "fp8xfp4", "prefill32_bf16q": "fp8xfp4",
         "prefill32_a4": "fp4xfp4", "prefill32_prep": "fp8xfp4", "prefill32_a4_prep": "fp4xfp4"}
STAGES = ["route", "act_prep", "fc1_swiglu", "fc2", "combine"]


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its launch stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            if self.hip.hipEventCreate(ctypes.byref(self.arr, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")

    def record(self, i, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(self.arr[i]), ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def sub(self, i0, n):
        return ctypes.cast(ctypes.byref(self.arr, i0 * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def ms(self, i, j):
        f = ctypes.c_float(0)
        if self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.arr[i]),
                                        ctypes.c_void_p(self.arr[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


def prepare_weights(moe, torch, d):
    """Weights of a *_prep workload in the GEMM layout (prepared once, not
    timed)."""
    d["w13"], d["w13_sf"] = moe.prepare_gemm_weights(d["w13"], d["w13_sf"], "w13")
    d["w2"], d["w2_sf"] = moe.prepare_gemm_weights(d["w2"], d["w2_sf"], "w2")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def to_dev(torch, inp):
    d = {}
    if inp.x_sf is None:
        d["x"] = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
        d["x_sf"] = None
    else:
        d["x"] = torch.from_numpy(inp.x).cuda()
        d["x_sf"] = torch.from_numpy(inp.x_sf).cuda()
    d["topk_ids"] = torch.from_numpy(inp.topk_ids).cuda()
    d["topk_w"] = torch.from_numpy(inp.topk_w).cuda()
    for n in ("w13", "w13_sf", "w2", "w2_sf"):
        d[n] = torch.from_numpy(getattr(inp, n)).cuda()
    for n in ("w13_gs", "w2_gs"):
        v = getattr(inp, n)
        d[n] = None if v is None else torch.from_numpy(v).cuda()
    return d


def alloc_forward(moe, torch, inp):
    """The workspace and output of a forward on this workload (no launch)."""
    c = inp.cfg
    p = moe.make_problem(c.T, c.E, c.k, c.H, c.I, c.gran,
                         {"fp8": moe.ACT_FP8_UE8M0_K32,
                          "bf16q": moe.ACT_BF16_QUANT_FP8_K32,
                          "bf16q4": moe.ACT_BF16_QUANT_FP4_K32}.get(c.act, moe.ACT_BF16),
                         w_layout="gemm" if c.name.endswith("_prep") else "raw")
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device="cuda")
    return ws, out


def gpu_forward_into(moe, torch, inp, d, ws, out):
    """One forward into the given workspace and output."""
    moe.forward(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["w13_sf"], d["w13_gs"], d["w2"],
                d["w2_sf"], d["w2_gs"], inp.cfg.gran, x_sf=d["x_sf"], out=out, workspace=ws,
                quantize_x={"bf16q": "fp8", "bf16q4": "fp4"}.get(inp.cfg.act, False),
                w_layout="gemm" if inp.cfg.name.endswith("_prep") else "raw",
                fused=inp.cfg.name.endswith("_fused"))


def stage_kernel(cfg, ids, stage):
    """Symbol of the kernel the library launches for an FC stage at this
    shape (the dispatch rule of moe_fp4_forward: 16-row expert tiles when an
    active expert averages at most 16 assignments, else 128-row tiles for the
    FP8 x FP4 GEMM or 64-row tiles)."""
    A = ids.size
    active = len(np.unique(ids[ids >= 0]))
    a4 = cfg.act == "bf16q4"
    mode = 3 if a4 else 2 if cfg.act in ("fp8", "bf16q") else (0 if cfg.gran == 16 else 1)
    gemm_ok = (mode >= 2 and cfg.I % 512 == 0 and cfg.H % 512 == 0 and cfg.T * cfg.H < 2**31
               and A * cfg.I < 2**31 and cfg.I * cfg.H < 2**31)
    nt = (8 if gemm_ok else 4) if active and A / active > 16 else 1
    if nt == 8:
        return (f"fc_gemm_a8_kernel<{'true' if stage == 'fc1_swiglu' else 'false'}, "
                f"{'true' if a4 else 'false'}, {'true' if cfg.name.endswith('_prep') else 'false'}>")
    if nt == 1:
        return f"fc_decode_kernel<{mode}, {'true' if stage == 'fc1_swiglu' else 'false'}>"
    fc1 = "true" if stage == "fc1_swiglu" else "false"
    return f"fc_a8_kernel<{nt}, {fc1}>" if mode == 2 else f"fc_a16_kernel<{cfg.gran}, {nt}, {fc1}>"


def workload_cfg(synth, name):
    """Synthetic configuration of a named workload (the prefill variants
    take bfloat16 x that the library quantises)."""
    if name in synth.CONFIGS:
        return synth.CONFIGS[name]
    base, _, form = name.partition("_")
    if form in ("prep", "fused"):
        return synth.variant(synth.CONFIGS[base], name=name)
    return synth.variant(synth.CONFIGS[base], name=name,
                         act="bf16q4" if form in ("a4", "a4_prep") else "bf16q")


def kernel_file_key(symbol):
    """File-name form of a kernel symbol: fc_decode_kernel<0, true> -> fc_decode_0_true."""
    return symbol.replace("_kernel<", "_").replace(", ", "_").replace(">", "")


def algorithmic_bytes(cfg, ids):
    """Compulsory HBM bytes: the weights (codes, block scales, global scales)
    of every expert that receives at least one token, the activations read
    once, the output written once, ids and router weights; and the FC1 /
    FC2 kernel shares (FC1: w13 + x + h written; FC2: w2 + h read + rows of
    f32 partial outputs written)."""
    E, H, I, T, k, g = cfg.E, cfg.H, cfg.I, cfg.T, cfg.k, cfg.gran
    active = int(np.unique(ids[(ids >= 0) & (ids < E)]).size)
    A = T * k
    gs = 0 if cfg.global_scale == "none" else 4
    w13 = 2 * I * H // 2 + 2 * I * H // g + gs
    w2 = H * I // 2 + H * I // g + gs
    if cfg.act == "bf16":
        x_bytes, h_bytes = T * H * 2, A * I * 2
    elif cfg.act == "bf16q":
        x_bytes, h_bytes = T * H * 2, A * I + A * I // 32
    elif cfg.act == "bf16q4":
        x_bytes, h_bytes = T * H * 2, A * I // 2 + A * I // 32
    else:
        x_bytes, h_bytes = T * H + T * H // 32, A * I + A * I // 32
    whole = active * (w13 + w2) + x_bytes + T * H * 2 + T * k * 8
    fc1 = active * w13 + x_bytes + h_bytes
    fc2 = active * w2 + h_bytes + A * H * 4
    return dict(active=active, whole=whole, fc1=fc1, fc2=fc2)


def flops(cfg):
    return 2.0 * cfg.T * cfg.k * 3 * cfg.I * cfg.H


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "block_scaled_fp4_topk_amd", "csrc"))):
        with open(os.path.join(ROOT, "block_scaled_fp4_topk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_key, workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    --pmc summary, if it was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel_key}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def run_forward_timed(moe, torch, inp, d, steps, warmup):
    """Exactly `warmup` untimed forwards, then `steps` forwards timed by the
    wall clock with no instrumentation (synchronised on both sides: the
    headline); then `steps` forwards with one HIP event at each step boundary
    on the launch stream (per-step durations: median and mean); then `steps`
    with per-stage events recorded by the library (an event record between
    two kernels adds a few microseconds of its own)."""
    ws, out = alloc_forward(moe, torch, inp)
    for _ in range(warmup):
        gpu_forward_into(moe, torch, inp, d, ws, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        gpu_forward_into(moe, torch, inp, d, ws, out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stream = torch.cuda.current_stream()
    be = HipEvents(steps + 1)
    for i in range(steps):
        be.record(i, stream)
        gpu_forward_into(moe, torch, inp, d, ws, out)
    be.record(steps, stream)
    torch.cuda.synchronize()
    per_step = np.array([be.ms(i, i + 1) for i in range(steps)])
    ev = HipEvents(6 * steps)
    for i in range(steps):
        moe.set_stage_events(ev.sub(6 * i, 6), 6)
        gpu_forward_into(moe, torch, inp, d, ws, out)
    torch.cuda.synchronize()
    moe.set_stage_events(None, 0)
    stage_ms = {name: float(np.mean([ev.ms(6 * i + s, 6 * i + s + 1) for i in range(steps)]))
                for s, name in enumerate(STAGES)}
    return {"wall_ms": (t1 - t0) * 1e3 / steps, "event_median_ms": float(np.median(per_step)),
            "event_mean_ms": float(np.mean(per_step)), "stage_ms": stage_ms}


_CPU_INP = None  # the workload the oracle workers read (inherited through fork)


def _oracle_token(t):
    inp = _CPU_INP
    import oracle
    oracle.moe_forward(inp.x, inp.topk_ids, inp.topk_w, inp.w13, inp.w13_sf, inp.w13_gs,
                       inp.w2, inp.w2_sf, inp.w2_gs, inp.cfg.gran, x_sf=inp.x_sf, tokens=[t])
    return t


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def cpu_baseline(inp, budget_s=15.0):
    """The FP64 oracle as it stands, on this host's cores, on a bounded sample
    of the same workload: a process pool over tokens (each token's k experts
    and all H outputs; N = the CPUs this process may run on, at most 16, the
    host share of one GPU; one BLAS thread per worker) until about budget_s
    seconds or every token; tokens/s = tokens done / wall time.  Runs before
    the GPU is initialised (the workers are forked)."""
    import multiprocessing as mp
    global _CPU_INP
    _CPU_INP = inp
    n = max(1, min(len(os.sched_getaffinity(0)), 16))
    finished, failed = [], []
    with mp.get_context("fork").Pool(n, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        for t in range(inp.cfg.T):
            pool.apply_async(_oracle_token, (t,), callback=lambda _: finished.append(time.perf_counter()),
                             error_callback=failed.append)
        # until the budget is spent (and at least one token per worker, or
        # every token, has finished); a worker's error ends the wait, and so
        # does a hard limit of ten budgets
        while (not failed and len(finished) < inp.cfg.T and time.perf_counter() - t0 < 10 * budget_s
               and (time.perf_counter() - t0 < budget_s or len(finished) < min(n, inp.cfg.T))):
            time.sleep(0.05)
        ends = sorted(finished)
        pool.terminate()
    if failed:
        raise RuntimeError(f"the oracle baseline failed in a worker: {failed[0]!r}")
    if not ends:
        raise RuntimeError(f"the oracle baseline finished no token in {10 * budget_s:.0f} s")
    done, dt = len(ends), ends[-1] - t0
    _CPU_INP = None
    return {"value": done / dt, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{done} of the {inp.cfg.T} tokens of the {inp.cfg.name} workload (each with its "
                      f"{inp.cfg.k} experts and all {inp.cfg.H} outputs) in {dt:.1f} s; numpy FP64, a pool of "
                      f"{n} processes over tokens, one BLAS thread each"}


_RQ_ROWS = 256  # rows of one expert's w13 per oracle requantisation task


def _oracle_requant_slice(task):
    e, r0 = task
    inp = _CPU_INP
    import oracle
    oracle.requant_g16_to_g32(inp.w13[e:e + 1, r0:r0 + _RQ_ROWS], inp.w13_sf[e:e + 1, r0:r0 + _RQ_ROWS],
                              None if inp.w13_gs is None else inp.w13_gs[e:e + 1])
    return task


def cpu_baseline_requant(inp, budget_s=5.0):
    """The FP64 oracle's group16 -> group32 requantisation on this host's
    cores, on a bounded sample of the layer: a process pool over slices of
    256 rows of w13 (expert after expert, the same pool shape as
    cpu_baseline) until about budget_s seconds; GB/s = the slices'
    algorithmic bytes (codes and scales in, codes and scales out) / wall
    time.  Runs before the GPU is initialised."""
    import multiprocessing as mp
    global _CPU_INP
    _CPU_INP = inp
    n = max(1, min(len(os.sched_getaffinity(0)), 16))
    E, N, kh = inp.w13.shape
    K = 2 * kh
    tasks = [(e, r0) for e in range(E) for r0 in range(0, N - _RQ_ROWS + 1, _RQ_ROWS)]
    finished, failed = [], []
    with mp.get_context("fork").Pool(n, initializer=_one_blas_thread) as pool:
        t0 = time.perf_counter()
        for t in tasks[: 64 * n]:
            pool.apply_async(_oracle_requant_slice, (t,), callback=lambda _: finished.append(time.perf_counter()),
                             error_callback=failed.append)
        while (not failed and len(finished) < min(len(tasks), 64 * n) and time.perf_counter() - t0 < 10 * budget_s
               and (time.perf_counter() - t0 < budget_s or len(finished) < n)):
            time.sleep(0.05)
        ends = sorted(finished)
        pool.terminate()
    _CPU_INP = None
    if failed:
        raise RuntimeError(f"the oracle requantisation baseline failed in a worker: {failed[0]!r}")
    if not ends:
        raise RuntimeError(f"the oracle requantisation baseline finished no slice in {10 * budget_s:.0f} s")
    done, dt = len(ends), ends[-1] - t0
    per_slice = _RQ_ROWS * (K // 2 + K // 16 + K // 2 + K // 32)
    return {"value": done * per_slice / dt / 1e9, "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"{done} slices of {_RQ_ROWS} rows x K={K} of the decode16 layer's w13 "
                      f"({done * per_slice / 1e6:.0f} MB algorithmic) in {dt:.1f} s; numpy FP64, a pool of {n} "
                      f"processes over the slices, one BLAS thread each"}


def measured_peaks(moe, torch):
    """What this GPU delivers, beside the published peaks: a 1 GiB device
    copy (read + write bytes / time) and the register-only loop of the
    block-scaled MFMA with FP4 x FP8 and FP4 x FP4 operands (best of 3
    HIP-event timings each)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 1e30
    for _ in range(5):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    copy_gbs = 2 * (1 << 30) / (best * 1e-3) / 1e9
    del a, b
    blocks = torch.cuda.get_device_properties(0).multi_processor_count  # one workgroup per CU
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda")
    res = {"copy_GBps": copy_gbs}
    for name, a4 in (("mfma_fp4xfp8_TFLOPs", False), ("mfma_fp4xfp4_TFLOPs", True)):
        moe.mfma_peak_probe(a4, 200, blocks, sink)
        best, fl = 1e30, 0.0
        for _ in range(3):
            e0.record()
            fl = moe.mfma_peak_probe(a4, 4000, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name] = fl / (best * 1e-3) / 1e12
    del sink
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first ~30 forwards after the GPU has been idle (even 0.5 s) run up
    # to 20% slower (decode16 on MI355X: 0.99, 0.92, 0.86, 0.83 ms per step
    # over the first four groups of 10, then 0.82), so the default warmup
    # covers ~80 ms
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode16", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the primary workload (for rocprofv3 runs)")
    ap.add_argument("--requant-only", action="store_true",
                    help="only the group16 -> group32 requantisation of the decode16 layer "
                         "(for rocprofv3 runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp4_topk_amd as moe
    import synth
    # (device_count does not initialise the GPU: the CPU baseline's workers
    # are forked before anything touches it)
    if torch.cuda.device_count() < 1:
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.requant_only:
        moe.lib()  # fails loudly if the HIP library is not built
        print("[bench] generating decode16 weights", file=sys.stderr, flush=True)
        inp16 = synth.make_moe_inputs(workload_cfg(synth, "decode16"))
        print("[bench] timing requant", file=sys.stderr, flush=True)
        res = {"requant_layer": requant_layer(moe, torch, inp16)}
        res["copy_calibration_bytes"] = copy_calibration(torch)
        print(json.dumps(res), flush=True)
        return

    cfg = workload_cfg(synth, args.workload)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    inp = synth.make_moe_inputs(cfg)
    cpu = cpu_rq = None
    if not args.no_cpu_baseline and not args.profile:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        # (a failure of the CPU baseline is reported in its place; the GPU
        # measurement goes on)
        try:
            cpu = cpu_baseline(inp)
        except Exception as e:  # noqa: BLE001
            cpu = {"error": repr(e), "kind": "oracle"}
        if inp.cfg.gran == 16:
            try:
                cpu_rq = cpu_baseline_requant(inp)
            except Exception as e:  # noqa: BLE001
                cpu_rq = {"error": repr(e), "kind": "oracle"}
    moe.lib()  # fails loudly if the HIP library is not built
    d = to_dev(torch, inp)
    if cfg.name.endswith("_prep"):
        prepare_weights(moe, torch, d)
    print("[bench] timing", file=sys.stderr, flush=True)
    tm = run_forward_timed(moe, torch, inp, d, args.steps, args.warmup)
    ms_step, stage_ms = tm["wall_ms"], tm["stage_ms"]
    ab = algorithmic_bytes(cfg, inp.topk_ids)
    dom = max(("fc1_swiglu", "fc2"), key=lambda s: stage_ms[s])
    dom_bytes = ab["fc1"] if dom == "fc1_swiglu" else ab["fc2"]
    achieved = dom_bytes / (stage_ms[dom] * 1e-3) / 1e9
    kernel = stage_kernel(cfg, inp.topk_ids, dom)
    kernel_key = kernel_file_key(kernel)
    res = {
        "metric": METRIC,
        "value": cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[cfg.name],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[cfg.name], "T": cfg.T, "E": cfg.E, "top_k": cfg.k,
                   "H": cfg.H, "I": cfg.I, "gran_k": cfg.gran, "act": cfg.act,
                   "active_experts": ab["active"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": pmc_traffic(kernel_key, cfg.name),
                     "algorithmic_bytes_per_launch": dom_bytes, "launch_ms": stage_ms[dom]},
        # ms: the uninstrumented timed steps (wall clock, the headline);
        # event_median_ms / event_mean_ms: per-step HIP events at the step
        # boundaries over as many further steps; stage_ms: per-stage events
        "forward": {"ms": ms_step, "event_median_ms": tm["event_median_ms"],
                    "event_mean_ms": tm["event_mean_ms"], "stage_ms": stage_ms,
                    "algorithmic_bytes": ab["whole"],
                    "achieved_GBps": ab["whole"] / (ms_step * 1e-3) / 1e9,
                    "hbm_frac": ab["whole"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "hbm_frac_event_median": ab["whole"] / (tm["event_median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "tflops": flops(cfg) / (ms_step * 1e-3) / 1e12},
    }
    if args.profile:
        res["copy_calibration_bytes"] = copy_calibration(torch)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    if cpu_rq is not None:
        res["cpu_baseline_requant"] = cpu_rq
    if not args.no_secondary and not args.profile:
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        pk = measured_peaks(moe, torch)
        res["measured_peaks"] = dict(pk, copy_frac_of_8TBps=pk["copy_GBps"] / HBM_PEAK_GBS,
                                     mfma_fp4xfp8_frac_of_5PF=pk["mfma_fp4xfp8_TFLOPs"] / PEAK_TFLOPS["fp8"],
                                     mfma_fp4xfp4_frac_of_10_1PF=pk["mfma_fp4xfp4_TFLOPs"] / PEAK_TFLOPS["fp4"])
        res["roofline"]["frac_of_measured_copy"] = achieved / pk["copy_GBps"]
        res["secondary"] = secondary(moe, torch, synth, args, inp, d, pk)
    print(json.dumps(res), flush=True)


def copy_calibration(torch):
    """A plain device copy of 1 GiB, for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) of profiled kernels; returns its size."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return 1 << 30


def requant_layer(moe, torch, inp16):
    """group16 -> group32 requantisation of the whole decode16 layer (its
    w13 and w2), timed with HIP events over 5 passes after 2 untimed ones."""
    src13 = torch.from_numpy(inp16.w13).cuda()
    sf13 = torch.from_numpy(inp16.w13_sf).cuda()
    gs13 = torch.from_numpy(inp16.w13_gs).cuda()
    src2 = torch.from_numpy(inp16.w2).cuda()
    sf2 = torch.from_numpy(inp16.w2_sf).cuda()
    gs2 = torch.from_numpy(inp16.w2_gs).cuda()
    d13, s13 = torch.empty_like(src13), torch.empty(src13.shape[:2] + (src13.shape[2] * 2 // 32,),
                                                    dtype=torch.uint8, device="cuda")
    d2, s2 = torch.empty_like(src2), torch.empty(src2.shape[:2] + (src2.shape[2] * 2 // 32,),
                                                 dtype=torch.uint8, device="cuda")

    def rq():
        moe.requant_gran_k(src13, sf13, gs13, dst=d13, dst_sf=s13)
        moe.requant_gran_k(src2, sf2, gs2, dst=d2, dst_sf=s2)

    for _ in range(2):
        rq()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    e0.record()
    for _ in range(n):
        rq()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = sum(int(t.numel()) for t in (src13, sf13, d13, s13, src2, sf2, d2, s2)) + 2 * 256 * 4
    res = {"workload": "requant w13 [256,4096,6144] + w2 [256,6144,2048] g16 -> g32",
           "ms": ms, "algorithmic_bytes": nbytes,
           "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del src13, sf13, gs13, src2, sf2, gs2, d13, s13, d2, s2
    torch.cuda.empty_cache()
    return res


def gemm_counters(kernel_key, workload):
    """MFMA busy and issued / algorithmic MFMA counts of a prefill GEMM
    kernel from the committed rocprofv3 --pmc summary, if it was taken on the
    current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel_key}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return {k: d[k] for k in ("mfma_busy", "mfmas_issued", "mfmas_algorithmic", "fetch_over_algorithmic")
            if k in d}


def tiny_latency(moe, torch, synth):
    """The tiny MoE's forward: a latency, in microseconds (its few hundred
    kilobytes and 50 MFLOP put no roofline in reach)."""
    name = "tiny"
    inp = synth.make_moe_inputs(workload_cfg(synth, name))
    d = to_dev(torch, inp)
    print(f"[bench] secondary {name}", file=sys.stderr, flush=True)
    tm = run_forward_timed(moe, torch, inp, d, 50, 100)
    del d
    return {"workload": WORKLOAD_TEXT[name], "us_per_step": tm["wall_ms"] * 1e3,
            "event_median_us": tm["event_median_ms"] * 1e3,
            "stage_us": {k: v * 1e3 for k, v in tm["stage_ms"].items()}}


def secondary(moe, torch, synth, args, inp16, d16, peaks):
    """The other workloads of the hot path, each timed the same way; the
    prefill ones with the MFMA roofline of their FC1 GEMM."""
    out = {}
    del d16
    torch.cuda.empty_cache()
    out["requant_layer"] = requant_layer(moe, torch, inp16)
    out["tiny"] = tiny_latency(moe, torch, synth)
    for name in ("decode32", "decode32_a4", "decode16_fused", "decode32_fused", "prefill32", "prefill32_bf16q",
                 "prefill32_a4", "prefill32_prep", "prefill32_a4_prep"):
        cfg = workload_cfg(synth, name)
        print(f"[bench] secondary {name}", file=sys.stderr, flush=True)
        inp = synth.make_moe_inputs(cfg)
        d = to_dev(torch, inp)
        if name.endswith("_prep"):
            prepare_weights(moe, torch, d)
        steps, warm = (10, 10) if name.startswith("prefill") else (50, 100)
        tm = run_forward_timed(moe, torch, inp, d, steps, warm)
        ms_step, stage_ms = tm["wall_ms"], tm["stage_ms"]
        ab = algorithmic_bytes(cfg, inp.topk_ids)
        r = {"workload": WORKLOAD_TEXT[name], "ms_per_step": ms_step, "tokens_per_s": cfg.T / (ms_step * 1e-3),
             "event_median_ms": tm["event_median_ms"],
             "stage_ms": stage_ms, "algorithmic_bytes": ab["whole"],
             "hbm_frac": ab["whole"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "tflops": flops(cfg) / (ms_step * 1e-3) / 1e12}
        a4 = cfg.act == "bf16q4"
        peak = PEAK_TFLOPS["fp4" if a4 else "fp8"]
        r["mfma_frac_fp4_peak" if a4 else "mfma_frac_fp8_peak"] = r["tflops"] / peak
        if name.startswith("prefill"):
            kern = stage_kernel(cfg, inp.topk_ids, "fc1_swiglu")
            fl1 = 2.0 * cfg.T * cfg.k * 2 * cfg.I * cfg.H
            ach = fl1 / (stage_ms["fc1_swiglu"] * 1e-3) / 1e12
            meas = peaks["mfma_fp4xfp4_TFLOPs" if a4 else "mfma_fp4xfp8_TFLOPs"]
            r["roofline"] = {"bound": "mfma", "kernel": kern, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                             "frac": ach / peak, "measured_peak": meas, "frac_of_measured_peak": ach / meas,
                             "algorithmic_flops_per_launch": fl1, "launch_ms": stage_ms["fc1_swiglu"],
                             "counters": gemm_counters(kernel_file_key(kern), name)}
        out[name] = r
        del d
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
