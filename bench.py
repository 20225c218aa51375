"""Benchmark: useful TFLOP/s of the banded sparse attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --decode swa512_decode_32k [--steps K] [--warmup W]
    python bench.py --backward [--workload NAME] [--steps K] [--warmup W]
    python bench.py --tglobal tglobal_16k [--steps K] [--warmup W]
    python bench.py --gates [--workload NAME] [--steps K] [--warmup W]

One step is one full forward pass (global-row partials, main sparse kernel, global-row combine)
over the workload's seeded synthetic inputs, already resident in device memory.  K steps are
timed back to back between two device synchronisations.  Useful work is 4*d*E floating-point
operations, E being the number of allowed (query, key) score entries counted by the library on
the GPU.  Prints one JSON line.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful TFLOP/s + % bf16 MFMA peak, window attn fwd at n=4096/16384 (1 GPU)"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
DEFAULT_WORKLOAD = "dilated_16k"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU takes a few hundred microseconds of back-to-back work to reach its steady clock:
    # the defaults time 500 steps after 100 warm-up steps (about 50 ms at dilated_16k)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="forward bench: untimed passes for about this long before the warm-up "
                         "steps, so that the GPU runs at its steady clock when the timed region "
                         "starts also with a short --warmup (reported as `settle`; 0 = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-passes", type=int, default=50,
                    help="forward (or decode) calls timed one by one after a read of a 512 MiB "
                         "buffer that flushes L2 and the MALL (0 = skip)")
    ap.add_argument("--cpu-budget-gflop", type=float, default=640.0,
                    help="fp64 work of the oracle sample: whole heads (at least one); a workload "
                         "smaller than the budget is run repeatedly")
    ap.add_argument("--decode", default=None, metavar="NAME",
                    help="instead of the forward bench: time decode steps of the named decode "
                         "workload (swa512_decode_32k), an HBM-bound path, reported in GB/s")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward bench: time the backward pass (dQ, dK, dV from "
                         "the saved out and lse) of the workload")
    ap.add_argument("--tglobal", default=None, metavar="NAME",
                    help="instead of the forward bench: time LongT5 Transient-Global attention "
                         "(global-token pass + attention) on the named workload (tglobal_16k)")
    ap.add_argument("--gates", action="store_true",
                    help="instead of the forward bench: time the forward pass with the fused "
                         "elementwise output gate against the plain one (workload given by "
                         "--workload), and the low-rank gate (r = 128) on that workload's output")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the attention bench: time K device-to-device copies of this "
                         "many MiB (a kernel of known HBM traffic, used to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def _copy_calibration(args):
    import torch

    nbytes = args.copy_calibration_mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": args.steps,
                      "ms_per_copy": round(dt * 1e3, 5),
                      "GB_per_s": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def _decode_bench(args):
    """Decode steps over a rolling or linear key/value cache: whole-step throughput in GB/s of
    algorithmic bytes (each reachable K and V row read once, Q read, out and lse written)."""
    import numpy as np
    import torch

    import sparse_long_sequence_banded_amd as la
    from workloads.decode import DECODE_WORKLOADS, decode_to_torch, decode_workload_inputs

    wl = DECODE_WORKLOADS[args.decode]
    inp = decode_workload_inputs(wl)
    dev = torch.device("cuda:0")
    t = decode_to_torch(inp, dev)
    q = t["q"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    desc = la.make_decode_desc(q, t["k_cache"], t["positions"], window=inp.window,
                               scale=inp.scale, ring=inp.ring)
    _, ws_bytes = la.longattn_decode_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ptrs = (q.data_ptr(), t["k_cache"].data_ptr(), t["v_cache"].data_ptr(), out.data_ptr(),
            lse.data_ptr(), ws.data_ptr(), ws_bytes, stream.cuda_stream)

    def step():
        st = la.longattn_decode(desc, *ptrs)
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, "longattn_decode")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # cold steps: reading a 512 MiB buffer before each evicts L2 and the MALL (the step's 134 MB
    # of window rows would otherwise stay in the 256 MB MALL between back-to-back steps)
    cold_ms = _cold_times(step, stream, args.cold_passes) if args.cold_passes > 0 else None

    elem = 2 if inp.dtype == "bf16" else 4
    last = inp.positions.astype(np.int64) + inp.m - 1
    first = np.maximum(0, inp.positions.astype(np.int64) - inp.window + 1)
    rows_kv = int((last - first + 1).sum()) * inp.heads  # distinct K (and V) rows read
    alg_bytes = (2 * rows_kv * inp.d * elem                           # K and V
                 + 2 * inp.batch * inp.heads * inp.m * inp.d * elem  # q in, out
                 + 4 * inp.batch * inp.heads * inp.m)                # lse
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": "decode step HBM throughput (K/V window rows read once + q, out, lse)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": inp.batch, "heads": inp.heads, "head_dim": inp.d,
                   "window": inp.window, "new_rows": inp.m, "cache_len": inp.cache_len,
                   "ring": inp.ring, "algorithmic_bytes": alg_bytes, "description": wl.note},
        "cold_l2_mall_flushed": None if cold_ms is None else {
            "passes": args.cold_passes, "flush_read_bytes": 512 << 20,
            "ms_median": round(float(np.median(cold_ms)), 5),
            "ms_p10": round(float(np.percentile(cold_ms, 10)), 5),
            "ms_p90": round(float(np.percentile(cold_ms, 90)), 5),
            "GB_per_s_median": round(alg_bytes / (float(np.median(cold_ms)) * 1e-3) / 1e9, 1)},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_window_kernel (whole step: one launch for this shape)",
            "achieved": round(value, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": _traffic_of("pmc_decode_swa512_decode_32k.json", "attn_decode.hip")
            if wl.name == "swa512_decode_32k" else None,
        },
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        # whole decode steps (every sample) repeated for about 10 s
        reps = 0
        t0 = time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            oracle.decode_inputs(inp, nthreads=threads)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        rec["cpu_baseline"] = {
            "value": round(alg_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole step ({inp.batch} samples, oracle forward on each gathered "
                      f"window), {dt:.2f} s per step, mean of {reps}"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def _backward_bench(args):
    """Backward steps: useful TFLOP/s = 10*d*E / step time (per allowed entry: the score, dP, dQ,
    dK and dV products, 2d flops each; the kernels recompute the score and dP once more)."""
    import numpy as np
    import torch

    import sparse_long_sequence_banded_amd as la
    from workloads import draw_dout, make_inputs, workload
    from workloads.torch_io import to_torch

    w = workload(args.workload)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    t = to_torch(inp, dev)
    q, k, v = t["q"], t["k"], t["v"]
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=t["global_idx"], key_pad=t["key_pad"],
              block_layout=t["layout"], block=inp.block)
    E, _ = la.count_entries(q, **{k2: kw[k2] for k2 in kw if k2 != "scale"})
    out, lse = la.forward(q, k, v, **kw)
    g = draw_dout(inp, 1)
    dout = (torch.from_numpy(g.view(np.int16)).view(torch.bfloat16) if inp.dtype == "bf16"
            else torch.from_numpy(g)).to(dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    desc, keep = la.make_desc(q, **kw)
    _, ws_bytes = la.longattn_backward_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
            ws_bytes, stream.cuda_stream)

    def step(marks=None):
        st = (la.longattn_backward(desc, *ptrs) if marks is None
              else la.longattn_backward_marked(desc, *ptrs, marks))
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, "longattn_backward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(la.LONGATTN_BWD_N_MARKS)]
             for _ in range(args.steps)]
    for row in marks:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        step([e.cuda_event for e in marks[s_]])
    torch.cuda.synchronize()
    spans = np.array([[marks[s_][2 * i].elapsed_time(marks[s_][2 * i + 1]) for i in range(3)]
                      for s_ in range(args.steps)]).mean(axis=0)
    dq_ms, dkv_ms, comb_ms = (float(x) for x in spans)
    useful = 10.0 * inp.d * E
    value = useful / (ms_per_step * 1e-3) / 1e12
    # per-kernel useful work: the dQ kernel does the score, dP and dQ products (6d per entry),
    # the dK/dV kernel the score, dP, dK and dV products (8d per entry)
    dq_tf = 6.0 * inp.d * E / (dq_ms * 1e-3) / 1e12
    dkv_tf = 8.0 * inp.d * E / (dkv_ms * 1e-3) / 1e12
    rec = {
        "metric": "useful TFLOP/s of the backward pass (10*d*E per step), window attn at "
                  "n=4096/16384 (1 GPU)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": inp.batch, "heads": inp.heads, "seq_len": inp.n,
                   "head_dim": inp.d, "useful_entries": E, "description": w.note},
        "pct_bf16_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "kernels_ms": {"dq": round(dq_ms, 5), "dkdv": round(dkv_ms, 5),
                       "global_combine": round(comb_ms, 5)},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bwd_kernel dK/dV step (useful score, dP, dK, dV products: 8*d*E; one "
                      "fused launch, or dK and dV passes at head dim 128)",
            "achieved": round(dkv_tf, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dkv_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
        },
        "roofline_dq": {"achieved": round(dq_tf, 3), "frac": round(dq_tf / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle
        from workloads import widen

        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        sub = inp.select_heads([0])
        t0 = time.perf_counter()
        oracle.backward_inputs(sub, widen(np.ascontiguousarray(g[:, :1]), inp.dtype),
                               nthreads=threads)
        dt = time.perf_counter() - t0
        E1 = oracle.count_inputs(sub)
        rec["cpu_baseline"] = {
            "value": round(10.0 * inp.d * E1 / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(threads, inp.batch), "kind": "oracle",
            "sample": f"head 0 of {inp.heads} (all rows; the oracle runs one thread per (b, h)), "
                      f"{E1} entries, {dt:.2f} s"}
    else:
        rec["cpu_baseline"] = None
    del keep
    print(json.dumps(rec), flush=True)


def _tglobal_bench(args):
    """Transient-Global steps: the global-token pass (block sums, RMS norm, key and value
    projections) and the attention (local window plus every global token, bucketed biases).
    Useful work: 4*d per attended (query, key) pair plus 2*d_model*H*d per global token and
    projection."""
    import numpy as np
    import torch

    import sparse_long_sequence_banded_amd as la
    from workloads.tglobal import TG_WORKLOADS, tglobal_to_torch, tglobal_workload_inputs

    wl = TG_WORKLOADS[args.tglobal]
    inp = tglobal_workload_inputs(wl)
    t = tglobal_to_torch(inp, "cuda:0")
    B, H, n, d = inp.batch, inp.heads, inp.n, inp.d
    G = max(1, n // inp.block)
    desc = la.make_tglobal_desc(t["q"], d_model=inp.d_model, radius=inp.radius, block=inp.block,
                                scale=inp.scale, num_buckets=inp.num_buckets,
                                max_distance=inp.max_distance, eps=inp.eps, key_pad=t["key_pad"])
    _, wsb = la.longattn_tglobal_workspace_size(desc)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda:0")
    sk = torch.empty((B, H, G, d), dtype=torch.bfloat16, device="cuda:0")
    sv = torch.empty_like(sk)
    valid = torch.empty((B, G), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def side():
        st = la.longattn_tglobal_side(desc, t["x"].data_ptr(), t["gamma"].data_ptr(),
                                      t["wk"].data_ptr(), t["wv"].data_ptr(), sk.data_ptr(),
                                      sv.data_ptr(), valid.data_ptr(), ws.data_ptr(), wsb, sh)
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, "longattn_tglobal_side")

    def attn():
        st = la.longattn_tglobal_forward(desc, t["q"].data_ptr(), t["k"].data_ptr(),
                                         t["v"].data_ptr(), sk.data_ptr(), sv.data_ptr(),
                                         valid.data_ptr(), t["bias_local"].data_ptr(),
                                         t["bias_side"].data_ptr(), out.data_ptr(),
                                         lse.data_ptr(), ws.data_ptr(), wsb, sh)
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, "longattn_tglobal_forward")

    for _ in range(args.warmup):
        side()
        attn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        side()
        attn()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        side()
        ev[s_][1].record(stream)
        attn()
        ev[s_][2].record(stream)
    torch.cuda.synchronize()
    side_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    if inp.key_pad is None:
        r = min(inp.radius, n - 1)
        E = B * H * (n * (2 * r + 1) - r * (r + 1) + n * G)
    else:
        raise SystemExit("padded Transient-Global workloads are parity cases, not bench lines")
    side_flop = 2.0 * 2 * B * G * inp.d_model * H * d
    useful = 4.0 * d * E + side_flop
    value = useful / (ms_per_step * 1e-3) / 1e12
    attn_tf = 4.0 * d * E / (attn_ms * 1e-3) / 1e12
    rec = {
        "metric": "useful TFLOP/s of LongT5 Transient-Global attention (global-token pass + "
                  "attention, 1 GPU)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": H, "seq_len": n, "head_dim": d,
                   "d_model": inp.d_model, "radius": inp.radius, "global_block": inp.block,
                   "global_tokens": G, "useful_entries": E, "description": wl.note},
        "kernels_ms": {"global_tokens": round(side_ms, 5), "attention": round(attn_ms, 5)},
        "roofline": {
            "bound": "mfma",
            "kernel": "tg_attn_kernel (events around the attention call: bias vectors + kernel)",
            "achieved": round(attn_tf, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        hs = [0]
        t0 = time.perf_counter()
        sk64, sv64, val64 = oracle.tglobal_side(inp.f64("x"), inp.gamma, inp.f64("wk"),
                                                inp.f64("wv"), heads=H, d=d, block=inp.block,
                                                eps=inp.eps)
        oracle.tglobal_forward(inp.f64("q")[:, hs], inp.f64("k")[:, hs], inp.f64("v")[:, hs],
                               sk64[:, hs], sv64[:, hs], val64, radius=inp.radius,
                               block=inp.block, num_buckets=inp.num_buckets,
                               max_distance=inp.max_distance, scale=inp.scale,
                               bias_local=inp.bias_local[:, hs], bias_side=inp.bias_side[:, hs],
                               nthreads=threads)
        dt = time.perf_counter() - t0
        work = side_flop + 4.0 * d * E / H
        rec["cpu_baseline"] = {
            "value": round(work / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the global-token pass of all {H} heads + attention of head 0, "
                      f"{work / 1e9:.1f} GFLOP fp64, {dt:.2f} s"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def _gates_bench(args):
    """Gated attention's output gates.  The elementwise gate is fused into the forward pass: the
    line gives the gated step time and its overhead over the plain step.  The low-rank gate
    (bottleneck 128) needs every output read and written once plus the two weight matrices;
    value = those algorithmic bytes per second."""
    import numpy as np
    import torch

    import sparse_long_sequence_banded_amd as la
    from workloads import make_inputs, workload
    from workloads.gates import gate_logits, lowrank_inputs
    from workloads.torch_io import to_torch

    w = workload(args.workload)
    inp = make_inputs(w)
    t = to_torch(inp, "cuda:0")
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=t["global_idx"], key_pad=t["key_pad"],
              block_layout=t["layout"], block=inp.block)
    g = torch.from_numpy(gate_logits(inp.q.shape, 500).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda:0")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    # raw C calls with the descriptor and pointers resolved once (as in the forward bench), so
    # the host enqueues ahead of the GPU and the times are the GPU's
    desc, keep = la.make_desc(t["q"], **kw)
    _, ws_bytes = la.longattn_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    qkv = (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr())
    tail = (out.data_ptr(), lse.data_ptr(), ws.data_ptr() if ws_bytes else None, ws_bytes, sh)

    def call(st, name):
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, name)

    plain_ms = timed(lambda: call(la.longattn_forward(desc, *qkv, *tail), "longattn_forward"))
    gated_ms = timed(lambda: call(la.longattn_forward_gated(desc, *qkv, g.data_ptr(), *tail),
                                  "longattn_forward_gated"))
    B, H, n, d = inp.q.shape
    r = 128
    o, wd, wu = lowrank_inputs(7, batch=B, heads=H, n=n, d=d, rank=r)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    ob, wdb, wub = dev(o), dev(wd), dev(wu)
    gdesc = la.longattn_gate_desc(batch=B, heads=H, n=n, d=d, rank=r)
    lr_ms = timed(lambda: call(la.longattn_gate_lowrank(gdesc, ob.data_ptr(), wdb.data_ptr(),
                                                        wub.data_ptr(), sh),
                               "longattn_gate_lowrank"))
    del keep
    nbytes = 2 * ob.numel() * 2 + 2 * wdb.numel() * 2  # outputs read and written once, weights
    value = nbytes / (lr_ms * 1e-3) / 1e9
    rec = {
        "metric": "output gates of gated attention: low-rank gate HBM throughput; fused "
                  "elementwise gate overhead on the forward step",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(lr_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "lowrank_rank": r, "tokens": B * n, "hd": H * d,
                   "lowrank_flop": 4.0 * B * n * H * d * r},
        "forward_ms": {"plain": round(plain_ms, 5), "gated": round(gated_ms, 5),
                       "overhead_pct": round(100.0 * (gated_ms - plain_ms) / plain_ms, 2)},
        "roofline": {"bound": "hbm", "kernel": "gate_lowrank_kernel (whole call)",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def _cold_times(step, stream, passes):
    """Per-call times (ms) of `passes` calls, each after a read of a 512 MiB buffer (a
    reduction, so the caches are left holding clean lines of that buffer)."""
    import numpy as np
    import torch

    flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(passes)]
    for e0, e1 in ev:
        sink += flush.sum()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    times = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    del flush, sink
    return times


def _environment():
    """The GPU, its clock and the software stack the numbers were taken with."""
    import subprocess

    import torch

    props = torch.cuda.get_device_properties(0)
    env = {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "hbm_bytes": props.total_memory, "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None)}
    env["max_sclk_mhz"] = None
    try:  # the GPU agent's maximum engine clock, as rocminfo reports it
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30)
        for agent in r.stdout.split("Agent ")[1:]:
            if "Device Type:             GPU" in agent or "gfx9" in agent:
                for ln in agent.splitlines():
                    if "Max Clock Freq. (MHz)" in ln:
                        env["max_sclk_mhz"] = int(ln.split(":")[1].split()[0])
                        break
                break
    except (OSError, subprocess.SubprocessError, ValueError, IndexError):
        pass
    return env


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _traffic_of(profile, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a copy kernel's readings), if it was taken on the current kernel
    sources (the summary lists them, `source` first; their joint hash must match), else None."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sources = rec.get("sources") or [source]
    if sources[0] != source:
        return None
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "sparse_long_sequence_banded_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if rec.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    return rec.get("hbm_bytes_per_launch")


def _traffic(workload):
    """HBM bytes per launch of the main forward kernel (see _traffic_of)."""
    return _traffic_of(f"pmc_main_kernel_{workload}.json", "attn_mfma.hip")


def _cpu_baseline(inp, budget_gflop):
    import oracle

    E_head = []
    for h in range(inp.heads):
        E_head.append(oracle.count_inputs(inp.select_heads([h])))
    flop_head = [4.0 * inp.d * e for e in E_head]
    heads = []
    tot = 0.0
    for h in range(inp.heads):
        if heads and tot + flop_head[h] > budget_gflop * 1e9:
            break
        heads.append(h)
        tot += flop_head[h]
    sub = inp.select_heads(heads)
    reps = max(1, int(budget_gflop * 1e9 // tot)) if len(heads) == inp.heads else 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    for _ in range(reps):
        _, _, E = oracle.forward_inputs(sub, nthreads=threads)
    dt = (time.perf_counter() - t0) / reps
    return {
        "value": 4.0 * inp.d * E / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu": _cpu_model(),
        "kind": "oracle",
        "sample": f"heads {heads[0]}-{heads[-1]} of {inp.heads} (all rows), {E} entries, "
                  f"{4.0 * inp.d * E / 1e9:.1f} GFLOP fp64, {dt:.2f} s per pass, mean of {reps}",
    }


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the sparse attention path here has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        _copy_calibration(args)
        return
    if args.decode:
        _decode_bench(args)
        return
    if args.backward:
        _backward_bench(args)
        return
    if args.tglobal:
        _tglobal_bench(args)
        return
    if args.gates:
        _gates_bench(args)
        return

    import numpy as np
    import torch

    import sparse_long_sequence_banded_amd as la
    from workloads import make_inputs, workload
    from workloads.torch_io import to_torch

    w = workload(args.workload)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    t = to_torch(inp, dev)
    q, k, v = t["q"], t["k"], t["v"]
    kw = dict(scale=inp.scale, win_left=inp.win_left, win_right=inp.win_right,
              dilation=inp.dilation, global_idx=t["global_idx"], key_pad=t["key_pad"],
              block_layout=t["layout"], block=inp.block)
    E, E_global_rows = la.count_entries(q, **{k2: kw[k2] for k2 in kw if k2 != "scale"})
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    desc, keep = la.make_desc(q, **kw)
    _, ws_bytes = la.longattn_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # the raw C call with everything resolved once, so the host enqueues far ahead of the GPU
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            ws.data_ptr() if ws_bytes else None, ws_bytes, stream.cuda_stream)

    def step(marks=None):
        st = (la.longattn_forward(desc, *ptrs) if marks is None
              else la.longattn_forward_marked(desc, *ptrs, marks))
        if st != la.LONGATTN_OK:
            raise la.LongAttnError(st, "longattn_forward")

    # clock settle: untimed passes for about --settle-ms (the GPU takes a few ms of back-to-back
    # work to leave its idle clock; a short warm-up alone then overstates the step time by 10-15%)
    settle_passes = 0
    t_settle = time.perf_counter()
    while args.settle_ms > 0 and (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        settle_passes += 50
    settle = {"passes": settle_passes, "ms": round((time.perf_counter() - t_settle) * 1e3, 1)}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole forward passes back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel durations: a second pass of K steps with HIP events that the library attaches to
    # the attention kernel's and the combine kernel's own dispatches (start and end of each)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(la.LONGATTN_N_MARKS)]
             for _ in range(args.steps)]
    for row in marks:  # create the underlying events before their handles are used
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in marks]
    for s in range(args.steps):
        step(handles[s])
    torch.cuda.synchronize()
    spans = np.array([[marks[s][0].elapsed_time(marks[s][1]), marks[s][2].elapsed_time(marks[s][3])]
                      for s in range(args.steps)])  # ms
    attn_ms, comb_ms = (float(x) for x in spans.mean(axis=0))
    ms_per_step = elapsed * 1e3 / args.steps

    # cold passes: before each, reading a 512 MiB buffer evicts the inputs from L2 and the MALL
    # (the 256 MB last-level cache would otherwise hold a 134 MB working set); a read leaves
    # clean lines, so no write-back of the flush competes with the pass.  Events bracket the
    # forward alone on the launch stream.
    cold = None
    if args.cold_passes > 0:
        cms = _cold_times(step, stream, args.cold_passes)
        cold = {"passes": args.cold_passes, "flush_read_bytes": 512 << 20,
                "ms_median": round(float(np.median(cms)), 5),
                "ms_p10": round(float(np.percentile(cms, 10)), 5),
                "ms_p90": round(float(np.percentile(cms, 90)), 5),
                "tflops_median": round(4.0 * inp.d * E / (float(np.median(cms)) * 1e-3) / 1e12, 3)}
    useful_flop = 4.0 * inp.d * E
    value = useful_flop / (ms_per_step * 1e-3) / 1e12

    # attention kernel (one launch: every non-global row, plus the global rows' per-chunk
    # partials): all useful score entries go through it; the combine only merges the partials.
    # Algorithmic bytes = Q, K, V read once + O written once (+ lse).
    elem = 2 if inp.dtype == "bf16" else 4
    attn_tflops = useful_flop / (attn_ms * 1e-3) / 1e12
    alg_bytes = 4.0 * inp.batch * inp.heads * inp.n * inp.d * elem + 4.0 * inp.batch * inp.heads * inp.n
    traffic = _traffic(args.workload)

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "settle": settle,
        "config": {
            "workload": w.name,
            "batch": inp.batch, "heads": inp.heads, "seq_len": inp.n, "head_dim": inp.d,
            "win_left": inp.win_left, "win_right": inp.win_right,
            "dilation": None if inp.dilation is None else inp.dilation.tolist(),
            "n_global": inp.n_global, "block": inp.block,
            "useful_entries": E, "useful_entries_global_rows": E_global_rows,
            "description": w.note,
        },
        "pct_bf16_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        # which timing `value` is, and the flushed one beside it
        "value_timing": "warm: wall clock over the K timed passes issued back to back, the device "
                        "synchronized before and after; value_flushed is the median of single "
                        "passes each timed after the L2 and MALL were flushed",
        "value_flushed": cold["tflops_median"] if cold else None,
        "cold_l2_mall_flushed": cold,
        "kernels_ms": {"attention": round(attn_ms, 5),
                       "global_combine": round(comb_ms, 5) if inp.n_global else 0.0},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel (band/layout rows + global-row partials, one launch)",
            "achieved": round(attn_tflops, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "roofline_hbm": {
            "achieved": round(alg_bytes / (attn_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(alg_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": alg_bytes,
        },
    }
    rec["cpu_baseline"] = None if args.no_cpu_baseline else _cpu_baseline(inp, args.cpu_budget_gflop)
    rec["environment"] = _environment()
    del keep
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
