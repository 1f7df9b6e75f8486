"""Decode benchmark: the routed FP8 MoE layer at batch 1 on one MI355X.

One step = one ``moe_decode_layer`` launch over the full layer: 256 resident
experts (hidden 6144, intermediate 2048, E4M3 weights with fp32 block-128
scales, ~10 GB in HBM), fresh N(0,1) router logits per step (64 pre-drawn
sets, so consecutive steps touch mostly different experts and the 256 MB
Infinity Cache cannot serve them), top-8 routing, live FP8 activation
quantisation, gate_up + SiLU*up, h re-quantisation, down and the weighted
combine.  Inputs are resident in HBM before timing starts.

Reported (one JSON line):
  value        algorithmic bytes moved per second over the timed steps (GB/s)
  ms_per_step  wall time per layer call (K back-to-back calls, no other work in the timed region)
  roofline     the layer kernel against HBM peak: algorithmic bytes per launch
               divided by its mean launch duration (HIP events around each
               launch on the launch stream, in a second pass over the same
               draws); traffic = FETCH_SIZE + WRITE_SIZE
               of the kernel from the committed rocprofv3 counter summary,
               scaled by a plain copy kernel of known size (null when the
               kernel source changed since the counters were taken)
               (+ launch-duration p10/p50/p90, and the traffic over the mean
               launch duration when the counters are current)
  measured_read_peak
               the HBM read bandwidth the library's streaming-read probe
               reaches on this device (the practical ceiling of this load
               path), and the layer kernel's fraction of it
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--m M]
       python bench.py --workload moe_tp8 [--m M]    (the layer's per-rank share under 8-way TP, I = 256)
       python bench.py --workload moe_full [--m M]   (the layer with the router GEMV and a shared expert in the launch)
       python bench.py --workload prefill [--tokens T]   (prefill FP8 GEMM on the matrix cores, MFMA roofline)
       python bench.py --workload gemv_small|gate_up|lm_head|q4_stack [--m M] [--steps K]   (dense GEMVs)
       python bench.py --ingest-pmc FETCH.csv WRITE.csv   (writes the counter summary)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_NAME = "moe_barrier_kernel"   # the layer kernel of the batch-1 workload (the counters are its)
MOE_SRC = os.path.join(ROOT, "quantized_moe_weight_amd", "csrc", "pq_moe.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "moe_barrier_kernel_e256_h6144_i2048_m1.pmc.txt")
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written per dispatch
COPY_REPS = 3                 # calibration copies at the end of a profile pass
METRIC = "achieved HBM GB/s (% of 8 TB/s) + µs/layer, batch-1 top-8 FP8 MoE GEMV"


def layer_kernel_name(M: int) -> str:
    """The kernel the library runs for an M-token call (one token: the barrier
    kernel; more: the stream kernel; PQ_MOE_PATH overrides)."""
    p = os.environ.get("PQ_MOE_PATH", "")
    if p in ("barrier", "stream"):
        return f"moe_{p}_kernel"
    return "moe_barrier_kernel" if M <= 1 else "moe_stream_kernel"


# the source files each kernel family is compiled from (its .hip and the
# device headers it includes), keyed by a substring of the kernel's name
KERNEL_SOURCES = (
    ("moe_", ("pq_moe.hip", "pq_common.h", "pq_quant_dev.h")),
    ("gemv_q4", ("pq_gemv_q4.hip", "pq_common.h")),
    ("gemv_fp8", ("pq_gemv_fp8.hip", "pq_common.h", "pq_quant_dev.h")),
    ("gemm_fp8", ("pq_gemm_fp8.hip", "pq_common.h")),
)


def kernel_source_sha(kernel: str = "moe_") -> str:
    """Hash of the sources of the kernel family whose name contains one of
    KERNEL_SOURCES' keys (the layer kernels by default), recorded with every
    counter summary: a summary whose hash differs no longer describes the
    built kernel."""
    files = next((fs for key, fs in KERNEL_SOURCES if key in kernel), None)
    if files is None:
        raise KeyError(f"no source list for kernel {kernel!r}")
    h = hashlib.sha1()
    for f in files:
        h.update(open(os.path.join(ROOT, "quantized_moe_weight_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def build_bank(pq, shp, seed=0):
    """Resident expert bank: master weights drawn per expert on the device,
    quantised by the library (E4M3 + fp32 block-128 scales)."""
    import torch
    import workloads
    E, H, I = shp.E, shp.H, shp.I
    w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((E, 2 * I, H // 128), dtype=torch.float32, device="cuda")
    w2 = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E, H, I // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        m13 = workloads.master_weights_torch(2 * I, H, workload=workloads.MOE_LAYER, tensor=workloads.T_W13,
                                             expert=e, seed=seed)
        q, s = pq.quantize_fp8(m13)
        w13[e].copy_(q); s13[e].copy_(s)
        m2 = workloads.master_weights_torch(H, I, workload=workloads.MOE_LAYER, tensor=workloads.T_W2,
                                            expert=e, seed=seed)
        q, s = pq.quantize_fp8(m2)
        w2[e].copy_(q); s2[e].copy_(s)
    torch.cuda.synchronize()
    return w13, s13, w2, s2


def read_traffic(bytes_alg):
    """HBM bytes per launch from the committed counter summary, or None."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    try:
        d = json.loads(open(PMC_SUMMARY, encoding="utf-8").read().split("\n---\n")[0])
    except Exception:
        return None
    if d.get("source_sha") != kernel_source_sha():
        return None
    return d["fetch_kib"] * 1024 * d["fetch_scale"] + d["write_kib"] * 1024 * d["write_scale"]


def cpu_experts(shp, lg):
    """The oracle's own coding of the experts one layer call routes to (untimed)."""
    import oracle
    import workloads
    ids, _ = oracle.route_topk(lg, shp.top_k)
    experts = {}
    for e in oracle.union_of_experts(ids):
        m13 = workloads.master_weights_torch(2 * shp.I, shp.H, workload=workloads.MOE_LAYER,
                                             tensor=workloads.T_W13, expert=int(e)).cpu().numpy()
        m2 = workloads.master_weights_torch(shp.H, shp.I, workload=workloads.MOE_LAYER,
                                            tensor=workloads.T_W2, expert=int(e)).cpu().numpy()
        experts[int(e)] = oracle.block_quant_fp8(m13) + oracle.block_quant_fp8(m2)
    return experts


def cpu_baseline(shp, x_bits, lg, experts, budget_s=12.0, threads=None):
    """Time the CPU oracle on one routed layer call (repeated until ~budget_s;
    at least once).  threads: limit the BLAS thread pools to that many threads
    for the timing (None: as configured, i.e. all cores)."""
    import oracle
    import contextlib
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:
        threadpool_info = threadpool_limits = None
    limit = (threadpool_limits(limits=threads) if (threads and threadpool_limits)
             else contextlib.nullcontext())
    with limit:
        if threadpool_info is not None:
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        else:
            cores = threads or len(os.sched_getaffinity(0))
        reps, t0 = 0, time.perf_counter()
        res = None
        while True:
            res = oracle.moe_layer(x_bits, lambda e: experts[e], logits=lg, top_k=shp.top_k)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
    return dt, reps, cores, res, len(experts)


def measure_read_peak(pq, nbytes=4 << 30, reps=10):
    """Achievable HBM read bandwidth (GB/s, median of reps) of the weight-stream
    load path, from the library's streaming-read probe over nbytes."""
    import numpy as np
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pq.stream_probe(src, sink)
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        pq.stream_probe(src, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del src
    return nbytes / float(np.median(ts)) / 1e9


def run(args):
    import numpy as np
    import torch

    import quantized_moe_weight_amd as pq
    import workloads

    torch.cuda.set_device(0)
    tp8 = args.workload == "moe_tp8"
    full = args.workload == "moe_full"         # router GEMV + shared expert in the launch
    shp = workloads.MOE_TP8_SHAPE if tp8 else workloads.MOE_SHAPE
    M = args.m
    t_setup = time.perf_counter()
    w13, s13, w2, s2 = build_bank(pq, shp)
    wl = workloads.MOE_LAYER if M == 1 else workloads.MOE_VERIFY
    x_bits = workloads.activation_bf16(M, shp.H, workload=wl)
    to_t = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    x = to_t(x_bits)
    n_draws = 64
    if full:
        # routing follows the activations: one x draw per step, logits computed in the launch
        xs = [to_t(workloads.activation_bf16(M, shp.H, workload=wl, seed=d)) for d in range(n_draws)]
        wr = to_t(workloads.router_weights_bf16(shp.E, shp.H))
        sh = []
        for t, (rows, cols) in ((workloads.T_SH13, (2 * shp.I, shp.H)), (workloads.T_SH2, (shp.H, shp.I))):
            q, sc = pq.quantize_fp8(workloads.master_weights_torch(rows, cols, workload=workloads.MOE_LAYER, tensor=t))
            sh += [q, sc]
        call = pq.MoeLayerCall(w13, s13, w2, s2, M=M, top_k=shp.top_k, router_w=wr, shared=tuple(sh))
        step = lambda i: call(xs[i % n_draws])
        pool_np = None
    else:
        if M == 1:
            pool_np = [workloads.router_logits(1, shp.E, workload=wl, draw=d) for d in range(n_draws)]
        else:
            pool_np = [workloads.verify_logits(M, shp.E, draw=d) for d in range(n_draws)]
        pool = [torch.from_numpy(p).cuda() for p in pool_np]
        call = pq.MoeLayerCall(w13, s13, w2, s2, M=M, top_k=shp.top_k)
        step = lambda i: call(x, pool[i % n_draws])
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # distinct experts per draw -> algorithmic bytes of each step
    expert_bytes = 2 * shp.I * shp.H + 4 * 2 * shp.I * (shp.H // 128) + shp.H * shp.I + 4 * shp.H * (shp.I // 128)
    io_bytes = M * (2 * shp.H + 2 * shp.H + 4 * shp.E)
    extra_bytes = expert_bytes + 2 * shp.E * shp.H if full else 0   # the shared expert and the router weights
    uni = []
    for d in range(n_draws):
        step(d)
        uni.append(len(np.unique(call.topk_ids.cpu().numpy())))
    step_bytes = [u * expert_bytes + io_bytes + extra_bytes for u in uni]
    assert call.check() == 0

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K back-to-back layer calls, nothing else on the stream
    K = args.steps
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for i in range(K):
        step(i)
    t_all1.record()
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    # a second pass over the same draws, with an event pair around each launch
    # (on the launch stream), gives the per-launch kernel durations
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    status = call.check()
    if status != 0:
        raise RuntimeError(f"kernel reported status {status}")

    bytes_timed = sum(step_bytes[i % n_draws] for i in range(K))
    value = bytes_timed / (total_ms * 1e-3) / 1e9
    # the kernel's average launch duration: HIP events around the timed region
    # of K back-to-back launches (one launch per layer call, nothing else on
    # the stream); the per-launch event pairs of the second pass keep the
    # spread, but each pair also holds the dispatch gap it forces
    mean_launch_s = total_ms / K * 1e-3
    isolated_launch_s = float(np.mean(per_launch_ms)) * 1e-3
    bytes_per_launch = bytes_timed / K
    achieved = bytes_per_launch / mean_launch_s / 1e9
    traffic = read_traffic(bytes_per_launch) if M == 1 and not tp8 and not full else None

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": (f"routed FP8 MoE decode layer, M={M}: 256 experts resident in HBM, hidden 6144, "
                         f"expert intermediate {shp.I} (gate||up 6144->2x{shp.I}, SiLU*up, down {shp.I}->6144), "
                         "E4M3 weights with fp32 scale per 128-wide K block, top-8 of N(0,1) logits, "
                         "live FP8 activation quantisation, bf16 in/out"
                         + ("; one rank's share of the 2048-wide layer under 8-way tensor parallelism" if tp8 else "")
                         + ("; the router GEMV (bf16 6144->256) and a shared expert in the same launch, "
                            "routing from the activations" if full else "")),
            "M": M, "experts": shp.E, "hidden": shp.H, "intermediate": shp.I, "top_k": shp.top_k,
            "mean_experts_streamed": float(np.mean(uni)),
            "bytes_per_step": int(round(bytes_per_launch)),
            "launches_per_layer": pq.launches_per_call("moe_decode_layer_ex"),
            "parallelism": "single GPU",
        },
        "us_per_layer": round(total_ms / K * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic),
            "kernel": layer_kernel_name(M),
            "mean_launch_us": round(mean_launch_s * 1e6, 2),
        },
        "setup_s": round(setup_s, 1),
    }
    q10, q50, q90 = np.percentile(per_launch_ms, [10, 50, 90]) * 1e3
    out["roofline"]["isolated_launch_us_mean"] = round(isolated_launch_s * 1e6, 2)
    out["roofline"]["isolated_launch_us_p10_p50_p90"] = [round(float(q10), 2), round(float(q50), 2), round(float(q90), 2)]
    if traffic is not None:
        out["roofline"]["achieved_hbm_traffic_gbs"] = round(traffic / mean_launch_s / 1e9, 1)
    peak_meas = measure_read_peak(pq)
    out["measured_read_peak"] = {
        "value": round(peak_meas, 1), "unit": "GB/s",
        "how": "pq_stream_probe over 4 GiB (128-bit non-temporal loads, one 512-thread block per CU, 3 loads in flight per lane: the fastest shape of a sweep), median of 10",
        "frac_achieved": round(achieved / peak_meas, 4),
    }
    if M > 1:
        out["config"]["bytes_per_token"] = int(bytes_per_launch / M)
        out["config"]["bytes_per_accepted_token_L3.5"] = int(bytes_per_launch / 3.5)

    if args.cpu_baseline and pool_np is not None:
        experts = cpu_experts(shp, pool_np[0])
        dt, reps, cores, ref, nexp = cpu_baseline(shp, x_bits, pool_np[0], experts)
        b0 = step_bytes[0]
        call(x, pool[0])
        torch.cuda.synchronize()
        y = call.out.float().cpu().numpy().astype(np.float64)
        rel = float(np.max(np.abs(y - ref["out"]) / ref["S"]))
        out["cpu_baseline"] = {
            "value": round(b0 / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": int(cores),
            "kind": "oracle",
            "sample": (f"one layer call (routing draw 0, {nexp} experts, {b0} bytes) of the same workload, "
                       f"float64 dequantise-then-matmul oracle repeated {reps}x, {dt:.2f} s per call; "
                       "weights pre-quantised by the oracle, untimed"),
            "seconds_per_call": round(dt, 3),
        }
        dt1, reps1, cores1, _, _ = cpu_baseline(shp, x_bits, pool_np[0], experts, budget_s=6.0, threads=1)
        out["cpu_baseline"]["single_thread"] = {
            "value": round(b0 / dt1 / 1e9, 3), "unit": "GB/s", "cores": int(cores1),
            "seconds_per_call": round(dt1, 3), "reps": reps1,
            "how": "the same oracle call with the BLAS thread pools limited to one thread",
        }
        out["parity_check"] = {"max_err_over_S": rel, "bound": 2e-3, "ok": rel <= 2e-3}
    print(json.dumps(out), flush=True)


def run_dense(args):
    """The dense configurations: FP8 GEMV 512->256 (launch bound), one expert's
    gate_up 6144->2x2048 with SiLU*up, and the int4 g32 stack of 64 blocks x 3
    linears (5120->5120, 5120->2x17408 SiLU*up, 17408->5120).  Weights rotate
    over distinct copies (>= 2 GB) or form a 10.57 GB stack so no cache serves
    them; every launch is timed with HIP events on the launch stream, and the
    FP8 calls (one launch each, short) are also replayed from one HIP graph,
    whose time per launch is the roofline's."""
    import ctypes

    import numpy as np
    import torch

    import quantized_moe_weight_amd as pq
    import workloads
    torch.cuda.set_device(0)
    lib = pq.lib()
    M = args.m
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)

    def xbits(K, wl, seed=0):
        xb = workloads.activation_bf16(M, K, workload=wl, seed=seed, outliers=0 if wl == workloads.Q4_STACK else 2)
        return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()

    launches = []      # (callable, bytes)
    on_stream = []     # the same calls taking the stream handle (HIP-graph timing)
    if args.workload in ("gemv_small", "gate_up", "lm_head"):
        if args.workload == "gemv_small":
            K, N, epi, wl, desc = 512, 256, 0, workloads.FP8_GEMV_SMALL, "FP8 GEMV 512->256"
        elif args.workload == "lm_head":
            K, N, epi, wl, desc = 6144, workloads.LM_HEAD_V, 0, workloads.LM_HEAD, \
                f"FP8 LM-head GEMV 6144->{workloads.LM_HEAD_V}"
        else:
            K, N, epi, wl, desc = 6144, 4096, 1, workloads.FP8_GATE_UP, "FP8 expert gate_up 6144->2x2048 + SiLU*up"
        m = workloads.master_weights_torch(N, K, workload=wl)
        q, sc = pq.quantize_fp8(m)
        per = q.numel() + sc.numel() * 4
        copies = max(80, int(np.ceil((2 << 30) / per))) if args.workload != "lm_head" else 3
        W = q.unsqueeze(0).expand(copies, -1, -1).contiguous()
        S = sc.unsqueeze(0).expand(copies, -1, -1).contiguous()
        del m
        x = xbits(K, wl)
        n_out = N // 2 if epi else N
        y = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")
        nb = int(lib.pq_gemv_fp8_workspace(M, K, N, epi))
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        lib.pq_workspace_init(P(ws), ws.numel(), st)
        io = 2 * M * K + 2 * M * n_out
        for c in range(copies):
            wp, sp = P(W[c]), P(S[c])
            launches.append((lambda wp=wp, sp=sp: lib.pq_gemv_fp8(P(x), M, K, wp, sp, N, epi, P(y), None, None,
                                                                   P(ws), ws.numel(), st), per + io))
            on_stream.append(lambda sh, wp=wp, sp=sp: lib.pq_gemv_fp8(P(x), M, K, wp, sp, N, epi, P(y), None, None,
                                                                      P(ws), ws.numel(), sh))
        fp8_path = os.environ.get("PQ_FP8_PATH", "")
        big = M >= 3 and N * K >= (128 << 20)           # the library's default rule
        kernel = ("gemv_fp8_mfma_kernel" if fp8_path == "mfma" or (big and fp8_path != "valu")
                  else "gemv_fp8_kernel")
        unit = "call"
        config = {"workload": f"{desc}, M={M}, E4M3 weights + fp32 block-128 scales, live FP8 act quant, "
                              f"{copies} weight copies rotated", "M": M, "K": K, "N": N, "epilogue": "silu_mul" if epi else "none"}
    elif args.workload == "q4_stack":
        layers = []
        for blk in range(64):
            for j, (K, N, silu) in enumerate(workloads.Q4_SHAPES):
                m = workloads.master_weights_torch(N, K, workload=workloads.Q4_STACK, tensor=workloads.T_W,
                                                   expert=blk * 3 + j)
                q, sc = pq.quantize_q4(m)
                del m
                layers.append((K, N, 1 if silu else 0, q, sc))
        torch.cuda.synchronize()
        xs = {K: xbits(K, workloads.Q4_STACK) for K in (5120, 17408)}
        ys = {}
        nb = max(int(lib.pq_gemv_q4_workspace(M, K, N, e)) for K, N, e, _, _ in layers[:3])
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        lib.pq_workspace_init(P(ws), ws.numel(), st)
        group = args.q4_mode == "group"
        arr = (pq._lib.Q4Linear * len(layers))()
        pass_bytes = 0
        for i, (K, N, e, q, sc) in enumerate(layers):
            n_out = N // 2 if e else N
            y = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")   # its own output: independent linears
            ys[i] = y
            b = q.numel() + sc.numel() * 2 + 2 * M * K + 2 * M * n_out
            pass_bytes += b
            arr[i] = pq._lib.Q4Linear(xs[K].data_ptr(), q.data_ptr(), sc.data_ptr(), y.data_ptr(), K, N, e)
            if not group:
                launches.append((lambda K=K, N=N, e=e, q=q, sc=sc, y=y: lib.pq_gemv_q4(
                    P(xs[K]), M, K, P(q), P(sc), N, e, P(y), P(ws), ws.numel(), st), b))
        n_launch = ctypes.c_int(0)
        if group:
            # the whole stack in one library call: the linears are packed into as few
            # launches as LDS allows (one persistent grid streams each pack)
            launches.append((lambda: lib.pq_gemv_q4_group(arr, len(layers), M, ctypes.byref(n_launch), st),
                             pass_bytes))
        kernel = "gemv_q4_kernel (grouped)" if group else "gemv_q4 kernels"
        unit = "stack pass (192 linears)"
        config = {"workload": f"int4 g32 W4A16 decode stack, M={M}: 64 blocks x (5120->5120, 5120->2x17408 SiLU*up, "
                              "17408->5120), fp16 group scales, 10.57 GB, fresh activation per linear",
                  "M": M, "linears": len(layers),
                  "issue": ("one pq_gemv_q4_group call per pass" if group else "one pq_gemv_q4 call per linear")}
    else:
        raise SystemExit(f"unknown workload {args.workload}")

    n = len(launches)
    for i in range(max(min(n, 2 * args.warmup + n // 4), args.warmup)):
        launches[i % n][0]()
    torch.cuda.synchronize()
    K_steps = args.steps
    total = K_steps if args.workload != "q4_stack" else K_steps * n
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(total)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    byts = 0
    stride = 1 if args.workload == "q4_stack" else max(1, n // total) | 1   # spread the steps over every copy
    for i in range(total):
        fn, b = launches[(i * stride) % n]
        ev[i][0].record()
        rc = fn()
        ev[i][1].record()
        if rc != 0:
            raise RuntimeError(f"launch returned {rc}")
        byts += b
    t1.record()
    torch.cuda.synchronize()
    # these kernels are short enough (5-25 us) that Python's launch rate could
    # leave gaps between back-to-back launches, so each launch carries its own
    # event pair on the launch stream and the kernel time is their sum
    per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    wall = t0.elapsed_time(t1) * 1e-3
    # Short kernels: an event pair around each launch adds a dispatch gap of
    # its own, so the same launches are also captured into one HIP graph
    # (no host gaps, no per-launch events) and replayed between one event
    # pair; its time per launch is the kernel time the roofline uses.
    graph = None
    if on_stream:
        try:
            s_g = torch.cuda.Stream()
            sh = ctypes.c_void_p(s_g.cuda_stream)
            with torch.cuda.stream(s_g):
                for i in range(min(n, 8)):
                    if on_stream[i % n](sh) != 0:
                        raise RuntimeError("launch failed")
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s_g):
                for i in range(total):
                    if on_stream[(i * stride) % n](sh) != 0:
                        raise RuntimeError("launch failed while capturing")
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s_g):
                g.replay()                                 # one untimed replay
                g0.record()
                g.replay()
                g1.record()
            torch.cuda.synchronize()
            graph = g0.elapsed_time(g1) * 1e-3 / total
            del g
        except Exception as ex:                            # the per-launch event timing stands
            graph = None
            print(f"HIP-graph timing unavailable ({ex}); using per-launch events", file=sys.stderr, flush=True)
    passes = K_steps
    kern_s = per.sum() / passes
    event_pair_s = kern_s
    if graph is not None:                     # dense FP8 calls: one launch per step
        kern_s = graph
    bytes_per_pass = byts / passes
    achieved = bytes_per_pass / kern_s / 1e9
    q10, q50, q90 = np.percentile(per, [10, 50, 90]) * 1e6
    out = {
        "metric": "achieved HBM GB/s (% of 8 TB/s) + µs per " + unit,
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": passes, "warmup": args.warmup,
        "ms_per_step": round(kern_s * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3" if args.workload != "q4_stack" else "int4g32xbf16", "data": "synthetic",
        "config": config,
        "us_per_" + ("call" if unit == "call" else "pass"): round(kern_s * 1e6, 2),
        "wall_us_per_step_with_host_gaps": round(wall / passes * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel,
                     "launch_us_p10_p50_p90": [round(float(q10), 2), round(float(q50), 2), round(float(q90), 2)],
                     "bytes_per_step": int(bytes_per_pass)},
    }
    if graph is not None:
        out["roofline"]["timing"] = (f"{total} launches replayed from one HIP graph between one event pair; "
                                     "launch_us_p10_p50_p90 are event pairs around single launches")
        out["roofline"]["event_pair_us_mean"] = round(event_pair_s * 1e6, 2)
    if args.workload == "q4_stack" and n > 1:
        per_shape = per.reshape(passes, n)
        out["per_linear_median_us"] = {f"{K}->{N}{' silu' if e else ''}": round(float(np.median(per_shape[:, j::3])) * 1e6, 2)
                                       for j, (K, N, e, _, _) in enumerate(layers[:3])}
    if args.workload == "q4_stack":
        out["config"]["launches_per_pass"] = n_launch.value if n == 1 else n
    print(json.dumps(out), flush=True)


MFMA_FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 matrix peak


def run_prefill(args):
    """Prefill (large-M) block-scaled FP8 GEMM: one expert's gate_up (K=6144,
    N=2x2048, SiLU*up) over args.tokens tokens.  A step is one pq_gemm_fp8
    call (live activation quant + GEMM); the roofline is the matrix cores'
    fp8 peak, with the GEMM launch timed alone (pq_gemm_fp8_prequant on the
    same quantised activation, events on the launch stream)."""
    import ctypes
    import numpy as np
    import torch

    import quantized_moe_weight_amd as pq
    import workloads

    torch.cuda.set_device(0)
    lib = pq.lib()
    T, K, N, epi = args.tokens, 6144, 4096, 1
    m = workloads.master_weights_torch(N, K, workload=workloads.FP8_GATE_UP)
    q, sc = pq.quantize_fp8(m)
    del m
    g = torch.Generator(device="cuda")
    g.manual_seed(workloads.torch_seed(workloads.FP8_GATE_UP, workloads.T_X))
    x = torch.randn((T, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty((T, N // 2), dtype=torch.bfloat16, device="cuda")
    nb = int(lib.pq_gemm_fp8_workspace(T, K, N, epi))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    xq, xs = pq.quantize_fp8(x)

    def full():
        rc = lib.pq_gemm_fp8(P(x), T, K, P(q), P(sc), N, epi, P(y), P(ws), nb, st)
        if rc != 0:
            raise RuntimeError(f"pq_gemm_fp8 returned {rc}")

    def gemm_only():
        rc = lib.pq_gemm_fp8_prequant(P(xq), P(xs), T, K, P(q), P(sc), N, epi, P(y), st)
        if rc != 0:
            raise RuntimeError(f"pq_gemm_fp8_prequant returned {rc}")

    for _ in range(args.warmup):
        full()
    torch.cuda.synchronize()
    Ks = args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(Ks):
        full()
    t1.record()
    torch.cuda.synchronize()
    step_s = t0.elapsed_time(t1) * 1e-3 / Ks
    # the GEMM kernel alone: K back-to-back launches on the same quantised
    # activation between one pair of events (its average launch duration),
    # then a pass with an event pair per launch for the spread
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(Ks):
        gemm_only()
    g1.record()
    torch.cuda.synchronize()
    gemm_s = g0.elapsed_time(g1) * 1e-3 / Ks
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(Ks)]
    for a_, b_ in ev:
        a_.record()
        gemm_only()
        b_.record()
    torch.cuda.synchronize()
    per = np.array([a_.elapsed_time(b_) for a_, b_ in ev]) * 1e-3
    flops = 2.0 * T * N * K
    achieved = flops / gemm_s / 1e12
    q10, q50, q90 = np.percentile(per, [10, 50, 90]) * 1e6
    out = {
        "metric": "prefill FP8 GEMM TFLOP/s (fraction of the 5.0 PFLOP/s dense fp8 matrix peak)",
        "value": round(flops / step_s / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": Ks,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
        "config": {"workload": (f"prefill block-scaled FP8 GEMM: {T} tokens through one expert's gate_up "
                                f"(K={K}, N=2x{N // 2}, SiLU*up), E4M3 weights + fp32 block-128 scales, "
                                "activation quantised live per token and 128-block (a second launch), bf16 out"),
                   "tokens": T, "K": K, "N": N, "epilogue": "silu_mul", "launches_per_call": pq.launches_per_call("pq_gemm_fp8")},
        "us_per_call": round(step_s * 1e6, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": ("gemm_fp8_kernel_t256" if (T + 255) // 256 * ((N // 2 + 127) // 128)
                                >= torch.cuda.get_device_properties(0).multi_processor_count else "gemm_fp8_kernel_t128"),
                     "mean_launch_us": round(gemm_s * 1e6, 2),
                     "isolated_launch_us_mean": round(float(np.mean(per)) * 1e6, 2),
                     "isolated_launch_us_p10_p50_p90": [round(float(q10), 2), round(float(q50), 2), round(float(q90), 2)],
                     "flops_per_launch": int(flops)},
    }
    print(json.dumps(out), flush=True)


def ingest_pmc(fetch_csv, write_csv, copy_bytes=COPY_BYTES, kernel=KERNEL_NAME, summary=None, made_by=None):
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE run, WRITE_SIZE run) into
    a summary: mean KiB per dispatch of the kernel whose name contains
    ``kernel`` and of the calibration copy kernel, and the copy-derived scale
    factors.  By default the headline layer kernel, into the summary the bench
    line's traffic figure is read from."""
    import csv
    headline = summary is None
    summary = PMC_SUMMARY if headline else summary

    def per_kernel(path, counter):
        rows = list(csv.DictReader(open(path, encoding="utf-8")))
        acc = {}
        for i, r in enumerate(rows):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            order = int(r.get("Dispatch_Id") or i)
            acc.setdefault(name, []).append((order, float(r["Counter_Value"])))
        return acc

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, key, calibration=False):
        vals, name = [], None
        for n, v in d.items():
            if key in n:
                vals += v
                name = n
        if not vals:
            raise KeyError(key)
        if calibration:          # the pass ends with the calibration copies: its last COPY_REPS copies
            vals = sorted(vals)[-COPY_REPS:]
        vals = [v for _, v in vals]
        return sum(vals) / len(vals), len(vals), name

    mf, nf, kname = pick(f, kernel)
    mw, nw, _ = pick(w, kernel)
    cf, ncf, cname = pick(f, "copy", calibration=True)
    cw, ncw, _ = pick(w, "copy", calibration=True)
    d = {
        "kernel": kernel if headline else kname, "source_sha": kernel_source_sha(kname),
        "fetch_kib": mf, "write_kib": mw, "dispatches": [nf, nw],
        "copy_kernel": cname, "copy_bytes": copy_bytes, "copy_dispatches": [ncf, ncw],
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": copy_bytes / (cf * 1024), "write_scale": copy_bytes / (cw * 1024),
    }
    txt = json.dumps(d, indent=1)
    pass_args = made_by or "--profile-pass --steps 20"
    os.makedirs(os.path.dirname(summary), exist_ok=True)
    with open(summary, "w", encoding="utf-8") as fh:
        fh.write(txt + "\n---\n" + f"source: {fetch_csv}, {write_csv}\n"
                 "made by (from the repository root on the MI355X box, $REPO = that root):\n"
                 "  cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d "
                 f"$REPO/<dir>/fetch -o f -- python3 $REPO/bench.py {pass_args}\n"
                 "  cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d "
                 f"$REPO/<dir>/write -o w -- python3 $REPO/bench.py {pass_args}\n"
                 "  python3 bench.py --ingest-pmc <dir>/fetch/f_counter_collection.csv "
                 "<dir>/write/w_counter_collection.csv"
                 + ("" if headline else f" --kernel '{kernel}' --summary {os.path.relpath(summary, ROOT)}"
                    + (f" --pass-args '{made_by}'" if made_by else "")) + "\n"
                 "fetch_kib / write_kib: mean KiB per dispatch of the kernel; the scales are the copy "
                 "kernel's known bytes over what the same counters read for it.\n")
    print(txt)


def ingest_sq(csv_path, kernel, summary, made_by):
    """Mean per dispatch of every counter of one rocprofv3 --pmc CSV for the
    kernel whose name contains ``kernel`` (instruction and cycle counters)."""
    import csv
    acc = {}
    name = None
    for r in csv.DictReader(open(csv_path, encoding="utf-8")):
        if kernel not in r.get("Kernel_Name", ""):
            continue
        name = r["Kernel_Name"]
        acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not acc:
        raise KeyError(kernel)
    d = {"kernel": name, "source_sha": kernel_source_sha(name),
         "dispatches": len(next(iter(acc.values()))),
         "mean_per_dispatch": {c: sum(v) / len(v) for c, v in sorted(acc.items())}}
    txt = json.dumps(d, indent=1)
    counters = " ".join(sorted(acc))
    with open(summary, "w", encoding="utf-8") as fh:
        fh.write(txt + "\n---\n" + f"source: {csv_path}\n"
                 "made by (from the repository root on the MI355X box, $REPO = that root):\n"
                 f"  cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {counters} --output-format csv -d "
                 f"$REPO/<dir>/sq -o s -- python3 $REPO/bench.py {made_by}\n"
                 f"  python3 bench.py --ingest-sq <dir>/sq/s_counter_collection.csv --kernel '{kernel}' "
                 f"--summary {os.path.relpath(summary, ROOT)} --pass-args '{made_by}'\n"
                 "SQ counters are summed over the device's shader engines; GRBM_GUI_ACTIVE counts GPU-busy "
                 "cycles.\n")
    print(txt)


def profile_pass(args):
    """Short run for rocprofv3 counter collection: a few launches of the
    workload plus a 1 GiB device copy (the calibration kernel of known size).
    The default (batch-1 layer) runs only the layer calls; another workload
    runs its bench pass with --steps as given."""
    import numpy as np
    import torch

    import quantized_moe_weight_amd as pq
    import workloads
    torch.cuda.set_device(0)
    if args.workload != "moe" or args.m != 1:
        args.cpu_baseline = False
        args.warmup = min(args.warmup, 5)
        if args.workload == "prefill":
            run_prefill(args)
        elif args.workload in ("moe", "moe_tp8", "moe_full"):
            run(args)
        else:
            run_dense(args)
    else:
        shp = workloads.MOE_SHAPE
        w13, s13, w2, s2 = build_bank(pq, shp)
        x_bits = workloads.activation_bf16(1, shp.H, workload=workloads.MOE_LAYER)
        x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
        call = pq.MoeLayerCall(w13, s13, w2, s2, M=1, top_k=shp.top_k)
        pool = [torch.from_numpy(workloads.router_logits(1, shp.E, workload=workloads.MOE_LAYER, draw=d)).cuda()
                for d in range(64)]
        for i in range(args.steps):
            call(x, pool[i % 64])
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):   # the last copies of the pass (a workload may copy buffers of its own before)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile pass: {args.workload} M={args.m}, {args.steps} steps, {COPY_REPS} copies of {COPY_BYTES} bytes",
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--m", type=int, default=1, choices=range(1, 9), metavar="M")
    ap.add_argument("--workload", default="moe",
                    choices=["moe", "moe_tp8", "moe_full", "gemv_small", "gate_up", "lm_head", "q4_stack", "prefill"],
                    help="moe (default: the routed layer) or one of the dense configurations")
    ap.add_argument("--tokens", type=int, default=4096, help="prefill workload: tokens per call")
    ap.add_argument("--q4-mode", default="group", choices=["group", "single"],
                    help="q4_stack: one grouped call per pass (default) or one pq_gemv_q4 call per linear")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--ingest-sq", metavar="SQ_CSV")
    ap.add_argument("--kernel", default=KERNEL_NAME, help="ingest: substring of the kernel's name")
    ap.add_argument("--summary", help="ingest: summary file to write (default: the headline layer's)")
    ap.add_argument("--pass-args", help="ingest: the bench.py arguments of the profiled run (for the record)")
    args = ap.parse_args()
    if args.ingest_pmc:
        summ = os.path.join(ROOT, args.summary) if args.summary else None
        ingest_pmc(*args.ingest_pmc, kernel=args.kernel, summary=summ, made_by=args.pass_args)
        return
    if args.ingest_sq:
        ingest_sq(args.ingest_sq, args.kernel, os.path.join(ROOT, args.summary), args.pass_args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("RANK", "0")) != 0:
        return
    if args.profile_pass:
        profile_pass(args)
        return
    if args.workload == "prefill":
        run_prefill(args)
        return
    if args.workload not in ("moe", "moe_tp8", "moe_full"):
        run_dense(args)
        return
    run(args)


if __name__ == "__main__":
    main()
