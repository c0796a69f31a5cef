"""Benchmark of the fused dequantize-and-multiply GEMM on one MI355X.

One step = the dense W4A16 layer (int4 symmetric weights, group 128, fp16
scales, bf16 activations, bf16 output) at its two projection shapes
(K=4096 -> N=14336 and K=14336 -> N=4096) for every M of the sweep
{1, 16, 128, 1024, 8192}: ten GEMM launches on one stream, inputs resident in
HBM. Small-M cases rotate over enough packed weight copies to defeat the
256 MB last-level cache, so their weights really stream from HBM.

Prints one compact JSON line last on stdout: `value` is the step's
algorithmic TFLOP/s; `roofline` describes the kernel that dominates the
step's time, `roofline_m16` the HBM-bound M=16 cases (also as a fraction of
`hbm_copy_gbs`, the box's measured device-to-device copy rate), and
`cpu_baseline` the fp64 CPU oracle timed on a bounded sample of the same
workload. The full record (`cases`: every launch of the step; `autotuned`:
each case again with a plan tuned per M range next to the heuristic plan;
`jit`: the hipRTC compile time of one instance of each W4A16 family; `rows`: the
other hot-path rows at their own shapes) goes to the JSON file named by
--detail (default gpurun_out/bench_detail.json), and one progress line per
measurement goes to stderr.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-rows] [--no-autotune] [--no-jit]
                    [--detail PATH]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16/W4A8 GEMM TFLOP/s + %HBM roofline (M=16), %MFMA peak (M=4096)"
SHAPES = [(4096, 14336), (14336, 4096)]  # (K, N): up and down projection
M_SWEEP = [1, 16, 128, 1024, 8192]
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
CACHE_BYTES = 256 << 20
COPY_CAL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_w4a16_dense.md")


def alg_bytes(m, n, k):
    # packed int4 weights + fp16 group scales + bf16 A + bf16 Y, each once
    return n * k // 2 + n * (k // 128) * 2 + m * k * 2 + m * n * 2


def alg_flops(m, n, k):
    return 2 * m * n * k


def kernel_source_sha(name):
    import hashlib
    with open(os.path.join(ROOT, "quantized_dequant_gemm_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(case, source):
    """HBM bytes per launch of `case` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy calibration), or None
    when there is none or the kernel source has changed since it was taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    sha = next((l.split(":", 1)[1].strip() for l in lines if l.startswith(f"source sha256 {source}:")), None)
    if sha != kernel_source_sha(source):
        return None
    for l in lines:
        cells = [c.strip() for c in l.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == case:
            try:
                return int(float(cells[3]))
            except ValueError:
                return None
    return None


def gpu_leg(args):
    import torch
    import quantized_dequant_gemm_amd as q
    import synth

    q.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # the box's own device-to-device copy rate (read + write bytes), the
    # practical HBM reference next to the published 8 TB/s; with
    # --copy-calibration the first copy is the counters' known-size reference
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_CAL_BYTES * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    layers = {}
    for (k, n) in SHAPES:
        layer = q.layer_w4a16(n, k)
        nbytes = q.qdg_preprocess_query(layer)
        qw = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((n, k // 128), dtype=torch.int16, device=dev)
        w = synth.device_normal_f32((n, k), 0.02, seed=synth.seed_for(1, synth.TID_W))
        q.qdg_quantize_weights(layer, w.data_ptr(), qw.data_ptr(), sc.data_ptr(), None, sh)
        del w
        copies = max(2, -(-2 * CACHE_BYTES // nbytes))  # >= 2x the cache
        bufs = []
        for _ in range(copies):
            b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), None), b.data_ptr(), nbytes, sh)
            bufs.append(b)
        layers[(k, n)] = (layer, q.qdg_plan_create(layer, q.dense()), bufs)

    # launch order within a step: largest M first, so that while its
    # millisecond-scale GEMMs run the host has queued every small-M launch;
    # the small cases then run back to back and their events time the
    # kernels, not the host's launch latency
    cases = []
    for m in sorted(M_SWEEP, reverse=True):
        for (k, n) in SHAPES:
            layer, plan, bufs = layers[(k, n)]
            a = synth.device_activations_bf16(m, k, seed=synth.seed_for(1, synth.TID_A, m))
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsb = q.qdg_plan_workspace(plan, m)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            cases.append(dict(k=k, n=n, m=m, plan=plan, bufs=bufs, a=a, y=y, ws=ws, wsb=wsb,
                              desc=q.qdg_plan_describe(plan, m), times=[]))
    torch.cuda.synchronize()

    it = [0]

    def step(record):
        for c in cases:
            buf = c["bufs"][it[0] % len(c["bufs"])]
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            q.qdg_gemm(c["plan"], c["a"].data_ptr(), None, buf.data_ptr(), c["y"].data_ptr(), c["m"],
                       c["ws"].data_ptr(), c["wsb"], sh)
            if record:
                e1.record(stream)
                c["times"].append((e0, e1))
        it[0] += 1

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    flops_step = 0
    out_cases = []
    for c in cases:
        us = sum(e0.elapsed_time(e1) for e0, e1 in c["times"]) * 1e3 / len(c["times"])
        fl = alg_flops(c["m"], c["n"], c["k"])
        by = alg_bytes(c["m"], c["n"], c["k"])
        flops_step += fl
        out_cases.append(dict(M=c["m"], K=c["k"], N=c["n"], us=round(us, 3),
                              tflops=round(fl / us / 1e6, 2), gbs=round(by / us / 1e3, 1),
                              hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                              mfma_frac=round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4),
                              instance=c["desc"].split(": ", 1)[1]))
    dom = max(out_cases, key=lambda d: d["us"])
    big = dom["M"] >= 128
    case_name = f"M={dom['M']} K={dom['K']} N={dom['N']}"
    traffic = measured_traffic(case_name, "tile_gemm.hip" if big else "wstream_gemm.hip")
    if big:
        roof = dict(bound="mfma", achieved=dom["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(dom["tflops"] / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                    kernel=f"w4a16 M={dom['M']} K={dom['K']} N={dom['N']}",
                    per_launch=alg_flops(dom["M"], dom["N"], dom["K"]))
    else:
        roof = dict(bound="hbm", achieved=dom["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(dom["gbs"] / PEAK_HBM_GBS, 4), traffic=traffic,
                    kernel=f"w4a16 M={dom['M']} K={dom['K']} N={dom['N']}",
                    per_launch=alg_bytes(dom["M"], dom["N"], dom["K"]))
    # the small-M cases once more as a stream of back-to-back launches (one
    # event pair over all of them): per-launch markers add about 2 us to a
    # 10 us kernel, back-to-back launches agree with the profiler's kernel
    # durations
    for c, d in zip(cases, out_cases):
        if c["m"] > 16:
            continue

        def launch(i, c=c):
            q.qdg_gemm(c["plan"], c["a"].data_ptr(), None, c["bufs"][i % len(c["bufs"])].data_ptr(),
                       c["y"].data_ptr(), c["m"], c["ws"].data_ptr(), c["wsb"], sh)
        us = _time_launches(launch, 60, stream)
        by = alg_bytes(c["m"], c["n"], c["k"])
        d.update(us_stream=round(us, 3), gbs_stream=round(by / us / 1e3, 1),
                 hbm_frac_stream=round(by / us / 1e3 / PEAK_HBM_GBS, 4))
    # per-M-range autotuning: a fresh plan per shape, tuned at each M of the
    # sweep (the library rotates its own weight copies while it times), then
    # timed like the heuristic plan (rotating copies, back-to-back launches);
    # not part of `value`
    autotuned = []
    if args.autotune:
        for (k, n) in SHAPES:
            layer, plan_h, bufs = layers[(k, n)]
            plan_a = q.qdg_plan_create(layer, q.dense())
            for c in cases:
                if (c["k"], c["n"]) != (k, n):
                    continue
                m = c["m"]
                ws_a = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
                _, best = q.qdg_plan_autotune(plan_a, c["a"].data_ptr(), None, bufs[0].data_ptr(), c["y"].data_ptr(),
                                              m, ws_a.data_ptr(), ws_a.numel(), 5 if m >= 1024 else 10, sh)
                reps = 5 if m >= 1024 else 60

                def run(i, plan=plan_h, c=c, ws=c["ws"], wsb=c["wsb"]):
                    q.qdg_gemm(plan, c["a"].data_ptr(), None, c["bufs"][i % len(c["bufs"])].data_ptr(),
                               c["y"].data_ptr(), c["m"], ws.data_ptr(), wsb, sh)
                # interleaved rounds, best of three each: at M = 8192 a single
                # back-to-back pair measures the clock drifting under load
                # (the same instance timed twice differs by up to 4 %)
                us_h = us_a = float("inf")
                for _ in range(3):
                    us_h = min(us_h, _time_launches(run, reps, stream))
                    us_a = min(us_a, _time_launches(lambda i: run(i, plan=plan_a, ws=ws_a, wsb=ws_a.numel()), reps,
                                                    stream))
                same = (q.qdg_plan_describe(plan_a, m).split("tuning=")[0] ==
                        q.qdg_plan_describe(plan_h, m).split("tuning=")[0])
                autotuned.append(dict(M=m, K=k, N=n, heuristic_us=round(us_h, 3), autotuned_us=round(us_a, 3),
                                      speedup=round(us_h / us_a, 3), autotune_best_us=round(best, 3),
                                      same_instance_as_heuristic=same,
                                      instance=q.qdg_plan_describe(plan_a, m).split(": ", 1)[1]))
                print(f"autotune M={m} K={k} N={n}: heuristic {us_h:.2f} us, autotuned {us_a:.2f} us",
                      file=sys.stderr, flush=True)
                del ws_a
    # run-time compilation: one streaming-family instance (M = 32 of the up
    # projection) compiled with hipRTC into a fresh cache directory, then
    # timed against the ahead-of-time instance (rotating weight copies)
    jit = None
    if args.jit:
        # one instance of each W4A16 family compiled at run time (hipRTC):
        # streaming (M = 32), weight streaming (M = 16), LDS-tiled (M = 1024);
        # compile time, and the run-time compiled instance timed beside the
        # ahead-of-time one
        import tempfile
        k, n = SHAPES[0]
        layer, plan_h, bufs = layers[(k, n)]
        jit = []
        for m in (32, 16, 1024):
            plan_j = q.qdg_plan_create(layer, q.dense())
            with tempfile.TemporaryDirectory() as cache:
                info = q.qdg_plan_jit(plan_j, m, 0, cache)
            a = synth.device_activations_bf16(m, k, seed=synth.seed_for(1, synth.TID_A, m))
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsb = q.qdg_plan_workspace(plan_h, m)
            wsj = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)

            def run_j(i, plan, m=m, a=a, y=y, wsj=wsj, wsb=wsb):
                q.qdg_gemm(plan, a.data_ptr(), None, bufs[i % len(bufs)].data_ptr(), y.data_ptr(), m,
                           wsj.data_ptr(), wsb, sh)
            run_j(0, plan_h)
            run_j(0, plan_j)
            reps = 60 if m <= 32 else 20
            us_aot = _time_launches(lambda i: run_j(i, plan_h), reps, stream)
            us_jit = _time_launches(lambda i: run_j(i, plan_j), reps, stream)
            jit.append(dict(M=m, K=k, N=n, compile_ms=round(info.compile_ms, 1), load_ms=round(info.load_ms, 2),
                            code_bytes=info.code_bytes, us_aot=round(us_aot, 3), us_jit=round(us_jit, 3),
                            instance=q.qdg_plan_describe(plan_j, m).split(": ", 1)[1]))
            print(f"jit M={m} K={k} N={n}: compile {info.compile_ms:.0f} ms, aot {us_aot:.2f} us, "
                  f"jit {us_jit:.2f} us", file=sys.stderr, flush=True)
            del a, y, wsj
        jit.append(dict(note="the pages' figure for compiling one W4A16 kernel: 1.82 s with NVCC (H200 host); "
                             "context only"))
    m16 = [d for d in out_cases if d["M"] == 16]
    roof16 = [dict(bound="hbm", achieved=d["gbs_stream"], peak=PEAK_HBM_GBS, unit="GB/s", frac=d["hbm_frac_stream"],
                   frac_of_copy=round(d["gbs_stream"] / copy_gbs, 4), kernel=f"w4a16 M=16 K={d['K']} N={d['N']}",
                   us=d["us_stream"], us_with_markers=d["us"],
                   traffic=measured_traffic(f"M=16 K={d['K']} N={d['N']}", "wstream_gemm.hip"))
              for d in m16]
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    return dict(value=value, ms_per_step=ms_per_step, roofline=roof, roofline_m16=roof16, cases=out_cases,
                hbm_copy_gbs=round(copy_gbs, 1), autotuned=autotuned, jit=jit)


PEAK_INT8_TOPS = 5000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0


def _time_launches(launch, reps, stream):
    """Average GPU time per launch (us) over `reps` back-to-back launches:
    the host queues them behind a short spin kernel and one event pair
    brackets them all, so the figure is the kernels' duration plus the
    launch gaps between them (the rate a stream of such calls sustains),
    without the host's launch latency or per-launch event markers."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(3e6))
    e0.record(stream)
    for i in range(reps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def rows_leg(reps=30):
    """The other rows of the hot path, each timed at its own shapes (not part
    of `value`): W8A8, W4A8-INT8, W8A16, W4A16-NVFP4 and W2A16 (K=4096, N in
    {4096, 14336}, M in {16, 256, 4096}), W4A8-MXFP4 ((K,N) in {(7168,2048), (2048,7168)}, M in
    {16, 512, 4096}), W4A4-MXFP4 and MXFP4 x INT8 at the same shapes, the activation
    quantizers, and the grouped MoE W4A16
    GEMMs (E=256, top-8, hidden 7168, intermediate 2048, T in {64, 512,
    4096}) with their expert sort, the gate+up GEMM with the SiLU*mul
    epilogue and the top-k combine, and the grouped MoE W4A8-INT8 GEMMs of
    the same experts at T in {64, 512, 4096}. Every figure is the average over
    back-to-back launches."""
    import torch
    import quantized_dequant_gemm_amd as q
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    out = []

    def dense_row(name, layer, k, n, ms, qa_dtype, act_group, peak, w_bytes, a_bits=8, as_bytes=4):
        nbytes = q.qdg_preprocess_query(layer)
        w = synth.device_normal_f32((n, k), 0.02, seed=synth.seed_for(2, synth.TID_W, n + k))
        if layer.wtype == q.QDG_W_INT8:
            qw = torch.empty((n, k), dtype=torch.int8, device=dev)
            sc = torch.empty(n, dtype=torch.float32, device=dev)
        elif layer.wtype == q.QDG_W_MXFP4:
            qw = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((n, k // 32), dtype=torch.uint8, device=dev)
        elif layer.wtype == q.QDG_W_NVFP4:
            qw = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        elif layer.wtype == q.QDG_W_UINT2:
            qw = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
            sc = torch.empty((n, k // 128), dtype=torch.int16, device=dev)
        else:
            qw = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((n, k // 128), dtype=torch.int16, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev)  # NVFP4 tensor scale
        zp = torch.empty((n, k // 128), dtype=torch.uint8, device=dev) if layer.has_zeros else None
        q.qdg_quantize_weights(layer, w.data_ptr(), qw.data_ptr(), sc.data_ptr(),
                               ts.data_ptr() if layer.wtype == q.QDG_W_NVFP4 else
                               zp.data_ptr() if zp is not None else None, sh)
        del w
        copies = max(2, -(-2 * CACHE_BYTES // nbytes))
        bufs = []
        for _ in range(copies):
            b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), zp.data_ptr() if zp is not None else None,
                                                 ts.data_ptr()), b.data_ptr(), nbytes, sh)
            bufs.append(b)
        plan = q.qdg_plan_create(layer, q.dense())
        for m in ms:
            a = synth.device_activations_bf16(m, k, seed=synth.seed_for(2, synth.TID_A, m))
            qa = torch.empty((m, k), dtype=qa_dtype, device=dev)
            sa = torch.empty((m, k // act_group) if act_group else m, dtype=torch.float32, device=dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsb = q.qdg_plan_workspace(plan, m)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

            bf16_a = layer.atype == q.QDG_A_BF16  # W8A16: A goes in as it is

            def quant(i):
                q.qdg_quantize_act(layer, a.data_ptr(), m, qa.data_ptr(), sa.data_ptr(), sh)

            def gemm(i):
                q.qdg_gemm(plan, (a if bf16_a else qa).data_ptr(), None if bf16_a else sa.data_ptr(),
                           bufs[i % len(bufs)].data_ptr(), y.data_ptr(), m, ws.data_ptr(), wsb, sh)
            if not bf16_a:
                quant(0)
            for i in range(3):
                gemm(i)
            us_q = 0.0 if bf16_a else _time_launches(quant, reps, stream)
            us = _time_launches(gemm, reps, stream)
            fl = 2 * m * n * k
            if bf16_a:
                by = w_bytes + m * k * 2 + m * n * 2
            else:
                by = (w_bytes + m * k * a_bits // 8 + (m * (k // act_group) * as_bytes if act_group else m * 4)
                      + m * n * 2)
            print(f"row {name} M={m} K={k} N={n}: {us:.2f} us", file=sys.stderr, flush=True)
            out.append(dict(row=name, M=m, K=k, N=n, us=round(us, 3), tflops=round(fl / us / 1e6, 2),
                            gbs=round(by / us / 1e3, 1), hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                            mfma_frac=round(fl / us / 1e6 / peak, 4), act_quant_us=round(us_q, 3),
                            instance=q.qdg_plan_describe(plan, m).split(": ", 1)[1]))
        del bufs

    for n in (4096, 14336):
        k = 4096
        dense_row("w8a8", q.layer_w8a8(n, k), k, n, (16, 256, 4096), torch.int8, 0, PEAK_INT8_TOPS,
                  n * k + n * 4)
        dense_row("w4a8-int8", q.layer_w4a8(n, k), k, n, (16, 256, 4096), torch.int8, 0, PEAK_INT8_TOPS,
                  n * k // 2 + n * (k // 128) * 2)
        dense_row("w8a16", q.layer_w8a16(n, k), k, n, (16, 256, 4096), torch.int8, 0, PEAK_BF16_TFLOPS,
                  n * k + n * 4)
        dense_row("w4a16-nvfp4", q.layer_nvfp4(n, k), k, n, (16, 256, 4096), torch.int8, 0, PEAK_BF16_TFLOPS,
                  n * k // 2 + n * (k // 16) + 4)
        dense_row("w2a16-uint2", q.layer_w2a16(n, k), k, n, (16, 256, 4096), torch.int8, 0, PEAK_BF16_TFLOPS,
                  n * k // 4 + n * (k // 128) * 3)
    for (k, n) in ((7168, 2048), (2048, 7168)):
        dense_row("w4a8-mxfp4", q.layer_mxfp4(n, k), k, n, (16, 512, 4096), torch.uint8, 128, PEAK_FP8_TFLOPS,
                  n * k // 2 + n * (k // 32))
        dense_row("w4a4-mxfp4", q.layer_w4a4(n, k), k, n, (16, 512, 4096), torch.uint8, 32, PEAK_FP4_TFLOPS,
                  n * k // 2 + n * (k // 32), a_bits=4, as_bytes=1)
        dense_row("w4a8-mxfp4-int8", q.layer_mxfp4_int8(n, k), k, n, (16, 512, 4096), torch.int8, 0, PEAK_FP8_TFLOPS,
                  n * k // 2 + n * (k // 32))

    # ---- grouped MoE W4A16
    E, top_k, hid, inter = 256, 8, 7168, 2048
    layers = {}
    for name, (n, k) in (("moe-gate-up", (2 * inter, hid)), ("moe-down", (hid, inter))):
        layer = q.layer_w4a16(n, k, num_experts=E)
        qw = torch.empty((E, n, k // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((E, n, k // 128), dtype=torch.int16, device=dev)
        one = q.layer_w4a16(n, k)
        for e in range(E):
            w = synth.device_normal_f32((n, k), 0.02, seed=synth.seed_for(4, synth.TID_W, e + (E if k == inter else 0)))
            q.qdg_quantize_weights(one, w.data_ptr(), qw[e].data_ptr(), sc[e].data_ptr(), None, sh)
        nbytes = q.qdg_preprocess_query(layer)
        pk = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), None), pk.data_ptr(), nbytes, sh)
        del qw, sc
        layers[name] = (layer, pk, n, k, q.qdg_plan_create(layer, q.moe(top_k)))
        print(f"row {name}: {E} experts packed", file=sys.stderr, flush=True)
    silu_plan = q.qdg_plan_create(layers["moe-gate-up"][0], q.moe(top_k, epilogue=q.QDG_EPI_SILU_MUL))
    for t in (64, 512, 4096):
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed_for(4, synth.TID_LOGITS, t))
        logits = torch.randn((t, E), generator=g, device=dev, dtype=torch.float32)
        ids = torch.topk(logits, top_k, dim=1).indices.to(torch.int32).contiguous()
        touched = int(torch.unique(ids).numel())
        # expert block size (the caller's choice in the API; measured on
        # MI355X): 16-row streaming blocks while experts hold a few rows
        # (T = 64), 32-row tiled blocks around 16 rows per expert (T = 512),
        # 64-row tiled blocks around 128 (T = 4096: less padding than 128-row
        # blocks)
        blk_m = 16 if t * top_k <= 4 * E else 32 if t * top_k <= 32 * E else 64
        aligned = {}
        for bm in (blk_m,):
            cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
            sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
            block_expert = torch.empty(cap // bm, dtype=torch.int32, device=dev)
            npad = torch.empty(1, dtype=torch.int32, device=dev)

            def align(i, bm=bm, sorted_ids=sorted_ids, block_expert=block_expert, npad=npad):
                q.qdg_moe_align(ids.data_ptr(), t, top_k, E, bm, sorted_ids.data_ptr(), block_expert.data_ptr(),
                                npad.data_ptr(), sh)
            align(0)
            aligned[bm] = (sorted_ids, block_expert, npad, _time_launches(align, reps, stream))
        for name, (layer, pk, n, k, plan) in layers.items():
            per_pair = name == "moe-down"
            bm = blk_m
            sorted_ids, block_expert, npad, us_align = aligned[bm]
            rows_in = t * top_k if per_pair else t
            a = synth.device_activations_bf16(rows_in, k, seed=synth.seed_for(4, synth.TID_H, t + k))
            y = torch.empty((t * top_k, n), dtype=torch.bfloat16, device=dev)
            wsb = q.qdg_plan_workspace(plan, t)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

            def gemm(i):
                q.qdg_moe_gemm(plan, a.data_ptr(), None, pk.data_ptr(), sorted_ids.data_ptr(),
                               block_expert.data_ptr(), npad.data_ptr(), t, bm, 1 if per_pair else 0,
                               y.data_ptr(), ws.data_ptr(), wsb, sh)
            gemm(0)
            us = _time_launches(gemm, max(5, reps // 3), stream)
            fl = 2 * t * top_k * n * k
            by = touched * (n * k // 2 + n * (k // 128) * 2) + rows_in * k * 2 + t * top_k * n * 2
            print(f"row {name} T={t}: {us:.2f} us", file=sys.stderr, flush=True)
            out.append(dict(row=name, T=t, K=k, N=n, block_m=bm, experts_touched=touched, us=round(us, 3),
                            tflops=round(fl / us / 1e6, 2), gbs=round(by / us / 1e3, 1),
                            hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                            mfma_frac=round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4), align_us=round(us_align, 3),
                            instance=q.qdg_moe_describe(plan, t, bm).split(": ", 1)[1]))
            if not per_pair:
                # the same gate+up GEMM with the SiLU*mul epilogue: [T*top_k][n/2] out
                yh = torch.empty((t * top_k, n // 2), dtype=torch.bfloat16, device=dev)
                wsb_h = q.qdg_plan_workspace(silu_plan, t)
                ws_h = torch.zeros(max(wsb_h, 1), dtype=torch.uint8, device=dev)

                def gemm_h(i):
                    q.qdg_moe_gemm(silu_plan, a.data_ptr(), None, pk.data_ptr(), sorted_ids.data_ptr(),
                                   block_expert.data_ptr(), npad.data_ptr(), t, bm, 0, yh.data_ptr(),
                                   ws_h.data_ptr(), wsb_h, sh)
                gemm_h(0)
                us = _time_launches(gemm_h, max(5, reps // 3), stream)
                by = touched * (n * k // 2 + n * (k // 128) * 2) + rows_in * k * 2 + t * top_k * (n // 2) * 2
                print(f"row moe-gate-up-silu T={t}: {us:.2f} us", file=sys.stderr, flush=True)
                out.append(dict(row="moe-gate-up-silu", T=t, K=k, N=n, block_m=bm, experts_touched=touched,
                                us=round(us, 3), tflops=round(fl / us / 1e6, 2), gbs=round(by / us / 1e3, 1),
                                hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                                mfma_frac=round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4),
                                instance=q.qdg_moe_describe(silu_plan, t, bm).split(": ", 1)[1]))
                del yh, ws_h
            else:
                # top-k weighted combine of the down projection's pair rows
                y32 = torch.empty((t * top_k, n), dtype=torch.float32, device=dev)
                rw = torch.rand(t * top_k, dtype=torch.float32, device=dev)
                yo = torch.empty((t, n), dtype=torch.bfloat16, device=dev)

                def comb(i):
                    q.qdg_moe_combine(y32.data_ptr(), rw.data_ptr(), t, top_k, n, yo.data_ptr(), q.QDG_O_BF16, sh)
                comb(0)
                us = _time_launches(comb, reps, stream)
                by = t * top_k * (n * 4 + 4) + t * n * 2
                print(f"row moe-combine T={t}: {us:.2f} us", file=sys.stderr, flush=True)
                out.append(dict(row="moe-combine", T=t, N=n, top_k=top_k, us=round(us, 3),
                                gbs=round(by / us / 1e3, 1), hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4)))

                # the same combine straight from the down projection's bf16 rows
                def comb_b(i):
                    q.qdg_moe_combine_bf16(y.data_ptr(), rw.data_ptr(), t, top_k, n, yo.data_ptr(), q.QDG_O_BF16,
                                           sh)
                comb_b(0)
                us = _time_launches(comb_b, reps, stream)
                by = t * top_k * (n * 2 + 4) + t * n * 2
                print(f"row moe-combine-bf16 T={t}: {us:.2f} us", file=sys.stderr, flush=True)
                out.append(dict(row="moe-combine-bf16", T=t, N=n, top_k=top_k, us=round(us, 3),
                                gbs=round(by / us / 1e3, 1), hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4)))
                del y32, rw, yo

    # ---- grouped MoE W4A8-INT8 (the same experts; int8 activations per token
    # for gate+up and per pair for down)
    del layers
    torch.cuda.empty_cache()
    layers8 = {}
    for name, (n, k) in (("moe-w4a8-gate-up", (2 * inter, hid)), ("moe-w4a8-down", (hid, inter))):
        layer = q.layer_w4a8(n, k, num_experts=E)
        qw = torch.empty((E, n, k // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((E, n, k // 128), dtype=torch.int16, device=dev)
        one = q.layer_w4a8(n, k)
        for e in range(E):
            w = synth.device_normal_f32((n, k), 0.02, seed=synth.seed_for(4, synth.TID_W, e + (E if k == inter else 0)))
            q.qdg_quantize_weights(one, w.data_ptr(), qw[e].data_ptr(), sc[e].data_ptr(), None, sh)
        nbytes = q.qdg_preprocess_query(layer)
        pk = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), None), pk.data_ptr(), nbytes, sh)
        del qw, sc
        layers8[name] = (layer, pk, n, k, q.qdg_plan_create(layer, q.moe(top_k)))
        print(f"row {name}: {E} experts packed", file=sys.stderr, flush=True)
    for t in (64, 512, 4096):
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed_for(4, synth.TID_LOGITS, t))
        logits = torch.randn((t, E), generator=g, device=dev, dtype=torch.float32)
        ids = torch.topk(logits, top_k, dim=1).indices.to(torch.int32).contiguous()
        touched = int(torch.unique(ids).numel())
        # 16-row blocks in the streaming family while experts hold a few
        # rows (T = 64), 64-row blocks in the 8-bit LDS-tiled family from
        # about 16 rows per expert (measured on MI355X, gate+up / down: T = 512
        # 802 / 486 us against 898 / 548 us with 32-row streaming blocks;
        # T = 4096 1959 / 1228 us against 2164 / 1384 us with 128-row blocks)
        bm = 16 if t * top_k <= 4 * E else 64
        cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
        sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
        block_expert = torch.empty(cap // bm, dtype=torch.int32, device=dev)
        npad = torch.empty(1, dtype=torch.int32, device=dev)
        q.qdg_moe_align(ids.data_ptr(), t, top_k, E, bm, sorted_ids.data_ptr(), block_expert.data_ptr(),
                        npad.data_ptr(), sh)
        for name, (layer, pk, n, k, plan) in layers8.items():
            per_pair = name.endswith("down")
            rows_in = t * top_k if per_pair else t
            a = synth.device_activations_bf16(rows_in, k, seed=synth.seed_for(4, synth.TID_H, t + k))
            qa = torch.empty((rows_in, k), dtype=torch.int8, device=dev)
            sa = torch.empty(rows_in, dtype=torch.float32, device=dev)

            def quant(i):
                q.qdg_quantize_act(layer, a.data_ptr(), rows_in, qa.data_ptr(), sa.data_ptr(), sh)
            quant(0)
            us_q = _time_launches(quant, reps, stream)
            y = torch.empty((t * top_k, n), dtype=torch.bfloat16, device=dev)
            wsb = q.qdg_plan_workspace(plan, t)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

            def gemm(i):
                q.qdg_moe_gemm(plan, qa.data_ptr(), sa.data_ptr(), pk.data_ptr(), sorted_ids.data_ptr(),
                               block_expert.data_ptr(), npad.data_ptr(), t, bm, 1 if per_pair else 0,
                               y.data_ptr(), ws.data_ptr(), wsb, sh)
            gemm(0)
            us = _time_launches(gemm, max(5, reps // 3), stream)
            fl = 2 * t * top_k * n * k
            by = touched * (n * k // 2 + n * (k // 128) * 2) + rows_in * (k + 4) + t * top_k * n * 2
            print(f"row {name} T={t}: {us:.2f} us", file=sys.stderr, flush=True)
            out.append(dict(row=name, T=t, K=k, N=n, block_m=bm, experts_touched=touched, us=round(us, 3),
                            tflops=round(fl / us / 1e6, 2), gbs=round(by / us / 1e3, 1),
                            hbm_frac=round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                            mfma_frac=round(fl / us / 1e6 / PEAK_INT8_TOPS, 4), act_quant_us=round(us_q, 3),
                            instance=q.qdg_moe_describe(plan, t, bm).split(": ", 1)[1]))
    return out


def _blas_info():
    """The BLAS numpy calls, as the BLAS itself reports it (vendor, version,
    thread count)."""
    try:
        import threadpoolctl
        for d in threadpoolctl.threadpool_info():
            if d.get("user_api") == "blas":
                return dict(vendor=d.get("internal_api"), version=d.get("version"), threads=d.get("num_threads"),
                            threading_layer=d.get("threading_layer"))
    except Exception as e:  # the BLAS still runs; only its report is missing
        return dict(vendor="unknown", error=str(e))
    return dict(vendor="unknown")


def _oracle_pass(cases):
    """One untuned pass of the fp64 oracle over `cases` (each: dequantize the
    layer, then the GEMM). Returns (seconds, flops, dequant seconds)."""
    from oracle import ref
    t_all = t_deq = 0.0
    fl = 0
    for (qv, s, a, m, n, k) in cases:
        t0 = time.perf_counter()
        w64 = ref.dequant_int4_sym(qv, s)
        t1 = time.perf_counter()
        ref.gemm_w4a16(a, w64)
        t2 = time.perf_counter()
        t_all += t2 - t0
        t_deq += t1 - t0
        fl += alg_flops(m, n, k)
    return t_all, fl, t_deq


def cpu_leg():
    """The fp64 oracle, untuned, on the host cores: the whole step (both
    projection shapes, M in the sweep; dequantize the layer, then the GEMM)
    three times, the median reported, about 10-20 s of host work; then the
    tiny W4A16 workload and the M=16 cases on one BLAS thread."""
    import statistics
    import numpy as np
    import synth
    from oracle import quant, ref

    cores = len(os.sched_getaffinity(0))
    blas = _blas_info()
    cases = []
    for (k, n) in SHAPES:
        w = synth.weights_f32(n, k, workload_id=1)
        qv, s = quant.quantize_int4_sym(w)
        del w
        for m in M_SWEEP:
            cases.append((qv, s, synth.activations_bf16_bits(m, k, workload_id=1, salt=m), m, n, k))
    runs = [_oracle_pass(cases) for _ in range(3)]
    secs = [r[0] for r in runs]
    med = statistics.median(secs)
    flops = runs[0][1]
    out = dict(value=round(flops / med / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
               sample="fp64 dequantize + BLAS GEMM of the dense W4A16 layer, both shapes, "
                      "M in {1,16,128,1024,8192}: the whole step, median of 3 runs",
               seconds_median=round(med, 3), seconds_runs=[round(x, 3) for x in secs],
               dequant_seconds_median=round(statistics.median(r[2] for r in runs), 3),
               blas=blas)
    # one BLAS thread: the tiny asymmetric uint4 workload and the M=16 cases
    one = {}
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits(limits=1, user_api="blas")
    except Exception:
        limiter = None
    try:
        m, k, n = 16, 1024, 512
        a = synth.activations_bf16_bits(m, k, workload_id=0)
        qv, s, z = quant.quantize_uint4_asym(synth.weights_f32(n, k, workload_id=0))
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            ref.gemm_w4a16(a, ref.dequant_uint4_asym(qv, s, z))
            ts.append(time.perf_counter() - t0)
        t = statistics.median(ts)
        one["tiny_M16_K1024_N512"] = dict(seconds=round(t, 5), gflops=round(alg_flops(m, n, k) / t / 1e9, 3))
        for (qv, s, a, m, n, k) in cases:
            if m != 16:
                continue
            rs = [_oracle_pass([(qv, s, a, m, n, k)]) for _ in range(3)]
            t = statistics.median(r[0] for r in rs)
            one[f"M16_K{k}_N{n}"] = dict(seconds=round(t, 4),
                                         dequant_seconds=round(statistics.median(r[2] for r in rs), 4),
                                         gflops=round(alg_flops(m, n, k) / t / 1e9, 3))
        one["blas_threads"] = _blas_info().get("threads")
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    out["one_thread"] = one
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rows", action="store_true", help="skip the W8A8 / W4A8 / MXFP4 / MoE rows")
    ap.add_argument("--no-jit", dest="jit", action="store_false",
                    help="skip the run-time compilation measurement")
    ap.add_argument("--no-autotune", dest="autotune", action="store_false",
                    help="skip the autotuned-plan comparison of the dense sweep")
    ap.add_argument("--detail", default=os.path.join(ROOT, "gpurun_out", "bench_detail.json"),
                    help="file for the full record (every case, autotuned, jit, rows); '' for none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 256 MiB device to device once (the known-size reference that scales "
                         "HBM byte counters in a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    g = gpu_leg(args)
    detail = dict(cases=g["cases"], hbm_copy_gbs=g["hbm_copy_gbs"])
    if g["autotuned"]:
        detail["autotuned"] = g["autotuned"]
    if g["jit"]:
        detail["jit"] = g["jit"]
    if not args.no_rows:
        detail["rows"] = rows_leg()
    line = {
        "metric": METRIC, "value": round(g["value"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights N(0,0.02) quantized on device, activations N(0,1))",
        "config": {"workload": "dense W4A16 layer: int4 sym g128 fp16 scales, bf16 act/out; "
                               "(K,N) in {(4096,14336),(14336,4096)}, M in {1,16,128,1024,8192}",
                   "launches_per_step": len(g["cases"])},
        "roofline": g["roofline"], "roofline_m16": g["roofline_m16"], "hbm_copy_gbs": g["hbm_copy_gbs"],
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_leg()
    line["detail"] = os.path.relpath(args.detail, ROOT) if args.detail else None
    if args.detail:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as f:
            json.dump(dict(line, **detail), f, indent=1)
    print(json.dumps(line, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
