#!/usr/bin/env python3
"""Benchmark of the lossless BF16 MLP-weight hot path on one MI355X.

Default workload (the metric's configuration): 80 Llama-70B MLP layers
(gate and up 28672 x 8192 stored [N][K], down 8192 x 28672 stored transposed
[K][N]), bf16 N(0, 0.02), compressed-resident in HBM with both the Huffman
stream and the 4-bit palette indices of every matrix.  The autotuner chooses
pipeline, GEMM variant, K split and CU split per projection and batch on the
first --tune-layers layers; its choices go into the library's tuning table
and every job then runs with UW_PIPE_AUTO and cfg NULL.

One step = one sweep over the batch sizes 1, 2, 4, ..., 1024: for each, one
pass over all 240 matrices through uw_run_sequence (x ~ N(0,1) bf16
[B][8192] for gate and up, h ~ N(0,1) bf16 [B][28672] for down).  Inputs
are resident in HBM before the timed region.

value = decoded-weight GB/s of the step: the bf16 bytes of weights delivered
to the GEMMs (11 passes x 2 x 56.37 G weights) over the step's wall time.
Per-batch rows report decoded GB/s, TFLOP/s and the roofline fraction; the
roofline object reports the kernel launch configuration with the largest
share of the sweep.  Prints one JSON line.

--workload gate8b runs the single-matrix step of the Llama-3.1-8B gate
projection (the four pipelines at batch 1) on its own.
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

METRIC = "decoded weight GB/s + fused MLP GEMM TFLOP/s (batch 1..1024), % roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PIPE_NAMES = ("full", "exponent", "transcode", "direct")
# kernel symbol (as rocprofv3 prints it, prefix) for each timed stage
STAGE_KERNELS = {
    "decode_full": "k_decode_staged<2,", "gemv_full": "k_gemv_nk_pipe<0, 1, 4>",
    "decode_exponent": "k_decode_staged<1,", "gemv_exponent": "k_gemv_nk_pipe<1, 1, 4>",
    "transcode": "k_decode_staged<0,", "gemv_transcode": "k_gemv_nk_pipe<2, 1, 4>",
    "gemv_direct": "k_gemv_nk_pipe<2, 1, 4>",
}
STAGE_SOURCES = {"decode": ["decode.hip", "rebuild.h", "uw_internal.h"],
                 "gemv": ["gemm.hip", "rebuild.h", "uw_internal.h"]}


def source_sha(stage_or_files) -> str:
    """Hash of the kernel sources a stage runs (a list of csrc files, or a
    gate8b stage name)."""
    if isinstance(stage_or_files, (list, tuple)):
        files = stage_or_files
    else:
        files = STAGE_SOURCES["decode" if stage_or_files.startswith(("decode", "transcode")) else "gemv"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "decode_gemm_exp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(info, stage: str, batch: int = 1) -> float:
    """Compulsory HBM bytes of one launch of a stage (compressed inputs +
    outputs; not the dense work avoided)."""
    M = info.numel
    Z = 4 * (info.stream_words + 2)
    O = 4 * (info.segments + 1)
    Aux = 8 * ((info.groups + 31) // 32)
    Vb = 64 * info.verbatim_groups
    X = 2 * batch * info.k
    Y = 4 * batch * info.n
    return {
        "decode_full": Z + O + Aux + Vb + M + 2 * M,
        "decode_exponent": Z + O + Aux + Vb + M,
        "transcode": Z + O + Aux + M / 2,
        "gemv_full": 2 * M + X + Y,
        "gemv_exponent": 2 * M + X + Y,
        "gemv_transcode": 1.5 * M + Aux + Vb + X + Y,
        "gemv_direct": 1.5 * M + Aux + Vb + X + Y,
    }[stage]


def load_traffic(stage: str, workload: str = "gate8b"):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(stage)
    if not k or k.get("source_sha") != source_sha(k.get("sources", stage)):
        return None
    return k.get("hbm_bytes_per_launch")


def load_valu_floor(stage: str):
    """The decoder's VALU floor (its VALU instruction count from committed
    rocprofv3 counters at one 64-lane instruction per SIMD every 4 cycles on
    1024 SIMDs at 2.4 GHz), if the counters were taken on the current source."""
    path = os.path.join(ROOT, "profiles", "decode_counters_gate8b.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        k = json.load(f).get("kernels", {}).get(stage)
    if not k or k.get("source_sha") != source_sha(stage):
        return None
    return k


def cpu_baseline_gate8b(w_np, x_np, min_seconds: float = 10.0):
    """The oracle, as it stands, on the same matrix: 3 decodes + 4 fp64 GEMVs
    per step, repeated whole steps until min_seconds have passed."""
    import threadpoolctl

    from oracle import oracle
    om = oracle.compress(w_np, seg_groups=4)
    steps = 0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        while True:
            st1, full = om.decode_full()
            st2, e = om.decode_exponent()
            st3, idx = om.transcode()
            assert st1 == st2 == st3 == 0
            for _ in range(4):
                oracle.gemm_ref(x_np, full.reshape(w_np.shape), 0)
            steps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = time.perf_counter() - t0
    return {"value": round(4 * 2 * w_np.size * steps / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"full {w_np.shape[0]}x{w_np.shape[1]} matrix, {steps} whole steps "
                      f"(decode_full + decode_exponent + transcode + 4 fp64 GEMVs, single thread), "
                      f"{dt:.1f} s"}


def hold_gpu(torch, launches: int) -> None:
    """Keep the GPU busy (a spin kernel, about 40 us per launch to come) while
    the host queues a timed burst, so the burst measures the kernels and not
    the host's call rate."""
    torch.cuda._sleep(int(launches * 1e5))


def extras(uw, synth, torch, dev, iters: int = 12, copies: int = 4):
    """Short measurements of the larger-batch rows: fused gate+up (2 x
    14336x4096) and the transposed down projection (stored [14336][4096]).
    Each row cycles through `copies` compressed copies, so the working set is
    larger than the 256 MB last-level cache."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    wl = synth.WORKLOADS["gateup8b"]
    sets = [[] for _ in range(copies)]
    for i in range(2):
        _, n, k, layout = wl.mats[i]
        w = synth.workload_weights(wl, i, device=dev)
        for c in range(copies):
            m = uw.uw_compress(w, n, k, layout)
            uw.uw_transcode_palette(m, None)
            sets[c].append(m)
        del w
    N = sum(m.info().n for m in sets[0])
    for b in wl.batches:
        x = synth.activations(b, 4096, seed=wl.seed, device=dev)
        y = torch.empty((b, N), dtype=torch.float32, device=dev)
        for p in (2, 3):
            ws = torch.empty(max(16, uw.uw_workspace_size_grouped(sets[0], p, b)), dtype=torch.uint8, device=dev)
            for c in range(copies):
                uw.uw_matmul_reconstruct_grouped(sets[c], p, x, y, ws)
            s, e = ev(), ev()
            hold_gpu(torch, iters)
            s.record()
            for it in range(iters):
                uw.uw_matmul_reconstruct_grouped(sets[it % copies], p, x, y, ws)
            e.record()
            torch.cuda.synchronize()
            t = s.elapsed_time(e) / iters / 1e3
            flops = 2.0 * b * N * 4096
            out[f"gateup8b_b{b}_{PIPE_NAMES[p]}"] = {"us": round(t * 1e6, 2),
                                                   "tflops": round(flops / t / 1e12, 3),
                                                   "decoded_gbs": round(2 * 2 * 14336 * 4096 / t / 1e9, 1)}
    del sets
    wl = synth.WORKLOADS["down8b"]
    _, n, k, layout = wl.mats[0]
    w = synth.workload_weights(wl, 0, device=dev)
    # compression (a1..a5) of the 58.7 M-weight down matrix: wall time of the
    # whole call, including its three small host round trips
    times = []
    for r in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mc = uw.uw_compress(w, n, k, layout)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        del mc
    tc = sorted(times)[1]
    out["compress_down8b"] = {"ms": round(tc * 1e3, 3), "bf16_input_gbs": round(2 * n * k / tc / 1e9, 1)}
    ms = []
    for c in range(copies):
        m = uw.uw_compress(w, n, k, layout)
        uw.uw_transcode_palette(m, None)
        ms.append(m)
    del w
    for b in wl.batches:
        x = synth.activations(b, k, seed=wl.seed, device=dev)
        y = torch.empty((b, n), dtype=torch.float32, device=dev)
        for p in (1, 2, 3):
            ws = torch.empty(max(16, uw.uw_workspace_size(ms[0], p, b)), dtype=torch.uint8, device=dev)
            for c in range(copies):
                uw.uw_matmul_reconstruct(ms[c], p, x, y, ws)
            s, e = ev(), ev()
            hold_gpu(torch, iters)
            s.record()
            for it in range(iters):
                uw.uw_matmul_reconstruct(ms[it % copies], p, x, y, ws)
            e.record()
            torch.cuda.synchronize()
            t = s.elapsed_time(e) / iters / 1e3
            flops = 2.0 * b * n * k
            out[f"down8b_b{b}_{PIPE_NAMES[p]}"] = {"us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 2),
                                                 "mfma_frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del ms
    out.update(attention_rows(uw, synth, torch, dev, iters, copies))
    out.update(fp8_rows(uw, synth, torch, dev, iters, copies))
    return out


def attention_rows(uw, synth, torch, dev, iters: int, copies: int):
    """The attention projections of Llama-3.1-8B and Llama-70B with the
    palette-direct pipeline: q, k and v fused into one call (they share x)
    and o on its own, at each workload's batches.  `roofline` is the larger
    of the HBM time of the algorithmic bytes and the MFMA time of the flops,
    over the measured time."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for name in ("attn8b", "attn70b"):
        wl = synth.WORKLOADS[name]
        sets = [[] for _ in range(copies)]
        for i, (_, n, k, layout) in enumerate(wl.mats):
            w = synth.workload_weights(wl, i, device=dev)
            for c in range(copies):
                m = uw.uw_compress(w, n, k, layout)
                uw.uw_transcode_palette(m, None)
                sets[c].append(m)
            del w
        infos = [m.info() for m in sets[0]]
        k = infos[0].k
        for b in wl.batches:
            x = synth.activations(b, k, seed=wl.seed, device=dev)
            for part, idx in (("qkv", (0, 1, 2)), ("o", (3,))):
                N = sum(infos[i].n for i in idx)
                y = torch.empty((b, N), dtype=torch.float32, device=dev)
                ws = torch.empty(max(16, uw.uw_workspace_size_grouped([sets[0][i] for i in idx], 3, b)),
                                 dtype=torch.uint8, device=dev)
                run = lambda c: uw.uw_matmul_reconstruct_grouped([sets[c][i] for i in idx], 3, x, y, ws)  # noqa: E731
                for c in range(copies):
                    run(c)
                s, e = ev(), ev()
                hold_gpu(torch, iters)
                s.record()
                for it in range(iters):
                    run(it % copies)
                e.record()
                torch.cuda.synchronize()
                t = s.elapsed_time(e) / iters / 1e3
                flops = 2.0 * b * N * k
                nbytes = sum(algorithmic_bytes(infos[i], "gemv_direct", b) for i in idx)
                out[f"{name}_{part}_b{b}_direct"] = {
                    "us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 3),
                    "decoded_gbs": round(2 * sum(infos[i].numel for i in idx) / t / 1e9, 1),
                    "roofline": round(max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)) / t, 4)}
        del sets
    return out


def fp8_rows(uw, synth, torch, dev, iters: int, copies: int):
    """Lossless coding over FP8 E4M3 weights at the 8B gate shape (14336 x
    4096, N(0, 0.02) scaled per tensor to the E4M3 maximum): the three decode
    outputs (E4M3 bytes, exponent fields, palette slots), each over `copies`
    compressed copies.  Algorithmic bytes: stream, offsets and flag words
    read, plus the sign+mantissa nibbles for the full decode, plus the output
    written."""
    n, k = 14336, 4096
    w = synth.fp8_weights(n, k, device=dev)
    ms = [uw.uw_compress_fp8(w, n, k, 0) for _ in range(copies)]
    del w
    info = ms[0].info()
    M = info.numel
    base = 4 * (info.stream_words + 2) + 4 * (info.segments + 1) + 8 * ((info.groups + 31) // 32)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out8 = torch.empty(M, dtype=torch.uint8, device=dev)
    outp = torch.empty(M // 2, dtype=torch.uint8, device=dev)
    rows = {}
    for name, call, nbytes in (("decode_fp8", lambda c: uw.uw_decode_fp8(ms[c], out8), base + M // 2 + M),
                               ("decode_exponent", lambda c: uw.uw_decode_exponent(ms[c], out8), base + M),
                               ("transcode", lambda c: uw.uw_transcode_palette(ms[c], outp), base + M // 2)):
        for c in range(copies):
            call(c)
        s, e = ev(), ev()
        hold_gpu(torch, iters)
        s.record()
        for it in range(iters):
            call(it % copies)
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / iters / 1e3
        rows[f"fp8_gate8b_{name}"] = {"us": round(t * 1e6, 2), "gbs": round(nbytes / t / 1e9, 1),
                                      "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                                      "bits_per_weight": round(info.bits_per_weight, 3)}
    del ms
    return rows


def job_bytes(info, pipeline: int, batch: int) -> float:
    """Compulsory HBM bytes of one projection under a pipeline (preprocessing
    writes and re-reads included)."""
    M = info.numel
    Z = 4 * (info.stream_words + 2)
    O = 4 * (info.segments + 1)
    Aux = 8 * ((info.groups + 31) // 32)
    Vb = 64 * info.verbatim_groups
    X, Y = 2 * batch * info.k, 4 * batch * info.n
    return {0: (Z + O + Aux + Vb + M + 2 * M) + (2 * M + X + Y),
            1: (Z + O + Aux + Vb + M) + (2 * M + X + Y),
            2: (Z + O + Aux + M / 2) + (1.5 * M + Aux + Vb + X + Y),
            3: 1.5 * M + Aux + Vb + X + Y}[pipeline]


def resident_bytes(info) -> int:
    """HBM bytes a matrix keeps: the UWF1 sections that are still resident
    (the Huffman stream and its offsets may have been dropped) plus the
    4-bit palette indices when resident."""
    b = info.compressed_bytes
    if not info.has_stream:
        b -= 4 * (info.segments + 1) + 4 * (info.stream_words + 2)
    if info.has_palette_idx:
        b += info.numel // 2
    return b


def yardsticks(uw, torch, dev, copy_mib: int = 1024, reps: int = 5):
    """Achievable rates on this machine, measured by the library's own kernels: a
    device copy and a streaming read of `copy_mib` MiB, and an MFMA-only loop
    (v_mfma_f32_32x32x16_bf16 on register operands, two waves per SIMD)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    nbytes = copy_mib << 20
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    sink = torch.empty(uw.YARDSTICK_SINK_BYTES, dtype=torch.uint8, device=dev)
    out = {}
    for kind, name, dst in ((0, "copy", b), (1, "read", sink)):
        for _ in range(2):
            uw.uw_yardstick(kind, a, dst, nbytes)
        ts = []
        for _ in range(reps):
            s, e = ev(), ev()
            s.record()
            work = uw.uw_yardstick(kind, a, dst, nbytes)
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e) / 1e3)
        t = sorted(ts)[len(ts) // 2]
        out[f"{name}_gbs"] = round(work / t / 1e9, 1)
    del a, b
    iters = 20000
    uw.uw_yardstick(2, None, sink, 0, iters)
    ts = []
    for _ in range(reps):
        s, e = ev(), ev()
        s.record()
        work = uw.uw_yardstick(2, None, sink, 0, iters)
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) / 1e3)
    t = sorted(ts)[len(ts) // 2]
    out["mfma_bf16_tflops"] = round(work / t / 1e12, 1)
    out["copy_frac_of_spec"] = round(out["copy_gbs"] / HBM_PEAK_GBS, 4)
    out["read_frac_of_spec"] = round(out["read_gbs"] / HBM_PEAK_GBS, 4)
    out["mfma_frac_of_spec"] = round(out["mfma_bf16_tflops"] / BF16_PEAK_TFLOPS, 4)
    out["how"] = (f"uw_yardstick: copy and read of {copy_mib} MiB (each block a contiguous span, 16-byte "
                  f"non-temporal accesses, 8 blocks per CU), MFMA loop of {iters} x 4 "
                  f"v_mfma_f32_32x32x16_bf16 per wave; median of {reps}")
    return out


def gemm_stage_bytes(info, pipeline: int, batch: int) -> float:
    """Compulsory HBM bytes of one GEMM-stage launch: the weights in the form
    the stage reads, x and y."""
    M = info.numel
    Aux = 8 * ((info.groups + 31) // 32)
    Vb = 64 * info.verbatim_groups
    X, Y = 2 * batch * info.k, 4 * batch * info.n
    return 2 * M + X + Y if pipeline in (0, 1) else 1.5 * M + Aux + Vb + X + Y


def prep_stage_bytes(info, pipeline: int) -> float:
    """Compulsory HBM bytes of one preprocessing launch (decode / transcode)."""
    M = info.numel
    Z = 4 * (info.stream_words + 2)
    O = 4 * (info.segments + 1)
    Aux = 8 * ((info.groups + 31) // 32)
    Vb = 64 * info.verbatim_groups
    return {0: Z + O + Aux + Vb + M + 2 * M, 1: Z + O + Aux + Vb + M, 2: Z + O + Aux + M / 2}[pipeline]


def build_c5(uw, synth, torch, dev, layers: int, seg_groups: int, alternate: bool):
    """The resident 70B model: every layer's gate, up and down compressed, with
    resident palette indices (and, with `alternate`, even layers keep only the
    indices and odd layers only the Huffman stream)."""
    wl = synth.WORKLOADS["mlp70b"]
    mats, proj = [], []
    t0 = time.perf_counter()
    for layer in range(layers):
        easy = not alternate or layer % 2 == 0
        for i, (label, n, k, layout) in enumerate(wl.mats):
            w = synth.workload_weights(wl, i, layer=layer, device=dev)
            m = uw.uw_compress(w, n, k, layout, seg_groups=seg_groups)
            if easy:
                uw.uw_transcode_palette(m, None)
                if alternate:
                    uw.uw_drop_stream(m)
            mats.append(m)
            proj.append((layer % 2) * 3 + i if alternate else i)
            del w
        if layer % 20 == 19:
            print(f"bench: {layer + 1}/{layers} layers resident ({time.perf_counter() - t0:.0f} s)", file=sys.stderr,
                  flush=True)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return wl, mats, proj


def c5_jobs(uw, synth, torch, dev, wl, mats, b: int):
    """One pass over every matrix at batch b: gate and up read x [b][8192],
    down reads h [b][28672]; outputs alternate between two buffers per
    projection.  Every job runs UW_PIPE_AUTO with the tuned choice."""
    K_in = wl.mats[0][2]
    H = wl.mats[2][2]
    x = synth.activations(b, K_in, seed=wl.seed + b, device=dev)
    h = synth.activations(b, H, seed=wl.seed + 7 + b, device=dev)
    ys = {(i, par): torch.empty((b, wl.mats[i][1]), dtype=torch.float32, device=dev)
          for i in range(3) for par in range(2)}
    jobs = []
    for j, m in enumerate(mats):
        layer, i = divmod(j, 3)
        jobs.append(uw.Job(m, uw.PIPE_AUTO, h if i == 2 else x, ys[(i, layer % 2)], None))
    return jobs, (x, h, ys)


def c5_step(uw, plan, ws):
    for b, (jobs, arr, _) in plan.items():
        uw.uw_run_sequence(jobs, 0, ws, _arr=arr)


def c5_breakdown(uw, torch, dev, wl, mats, proj, infos, batches, plan, alternate: bool, launches: int = 8):
    """Per (batch, projection): the stages the tuned choice runs, each timed
    over `launches` back-to-back launches rotating over four layers, and its
    share of one sweep (x 80 layers).  The largest share is the roofline's
    kernel."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    nproj = 6 if alternate else 3
    L = len(mats) // 3
    rot_layers = [l for l in range(0, L, max(1, L // 4))][:4]
    rows = []
    stream = torch.cuda.current_stream()
    for b in batches:
        jobs, _, (x, h, ys) = plan[b]
        for pj in range(nproj):
            idx = [j for j in range(len(mats)) if proj[j] == pj and (j // 3) in rot_layers] or \
                  [j for j in range(len(mats)) if proj[j] == pj][:4]
            if not idx:
                continue
            m0 = mats[idx[0]]
            info = infos[idx[0]]
            gp = uw.uw_plan_gemm(m0, uw.PIPE_AUTO, b)
            p = gp["pipeline"]
            xin = h if pj % 3 == 2 else x
            y = ys[(pj % 3, 0)]
            preps = []
            if p != 3:
                nb = {0: 2 * info.numel, 1: info.numel, 2: info.numel // 2}[p]
                preps = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in idx]
                call = {0: uw.uw_decode_full, 1: uw.uw_decode_exponent, 2: uw.uw_transcode_palette}[p]
                for m, buf in zip((mats[j] for j in idx), preps):
                    call(m, buf, stream)
            part = torch.empty(max(16, uw.uw_workspace_size(m0, p, b)), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()

            def burst(fn):
                for i in range(2):
                    fn(i)
                d0, d1 = ev(), ev()
                hold_gpu(torch, launches)
                d0.record(stream)
                for i in range(launches):
                    fn(i)
                d1.record(stream)
                torch.cuda.synchronize()
                return 1e3 * d0.elapsed_time(d1) / launches

            def kernel_burst(fn):
                # the same launches, each call's main kernel alone between two
                # events the library records around its launch
                # (uw_set_kernel_events); the events are recorded once first
                # so that they exist
                pairs = [(ev(), ev()) for _ in range(launches)]
                for a, b_ in pairs:
                    a.record(stream)
                    b_.record(stream)
                for i in range(2):
                    fn(i)
                hold_gpu(torch, launches)
                try:
                    for i in range(launches):
                        uw.uw_set_kernel_events(pairs[i][0], pairs[i][1])
                        fn(i)
                finally:
                    uw.uw_set_kernel_events(None, None)
                torch.cuda.synchronize()
                return 1e3 * sum(a.elapsed_time(b_) for a, b_ in pairs) / launches

            stages = []
            if p != 3:
                t = burst(lambda i: call(mats[idx[i % len(idx)]], preps[i % len(idx)], stream))
                stages.append(("prep", {0: "decode_full", 1: "decode_exponent", 2: "transcode"}[p],
                               {0: "k_decode_staged<2,", 1: "k_decode_staged<1,", 2: "k_decode_staged<0,"}[p],
                               t, prep_stage_bytes(info, p), 0.0, t))
            def gemm_call(i):
                uw.uw_matmul_stage(mats[idx[i % len(idx)]], p, preps[i % len(idx)] if preps else None,
                                   xin, y, part, stream=stream)
            t = burst(gemm_call)
            tk = kernel_burst(gemm_call) if gp["kernel"].startswith("k_mfma") else None
            stages.append(("gemm", f"gemm_{PIPE_NAMES[p]}", gp["kernel"], t, gemm_stage_bytes(info, p, b),
                           2.0 * b * info.n * info.k, tk))
            count = sum(1 for q in proj if q == pj)
            label = ("easy_" if pj < 3 else "hard_") + wl.mats[pj % 3][0] if alternate else wl.mats[pj][0]
            for kind, stage, kernel, t, nbytes, flops, tk in stages:
                rows.append({"batch": b, "projection": label, "stage": stage, "kernel": kernel,
                             "variant": gp["variant"], "tile": [gp["tile_m"], gp["tile_n"], gp["waves"]],
                             "k_slices": gp["k_slices"], "us": round(t, 2),
                             "kernel_us": round(tk, 2) if tk is not None else None, "launches_per_sweep": count,
                             "share_us": round(t * count, 1), "alg_bytes": int(nbytes), "flops": flops,
                             "launches_timed": launches})
            del preps, part
    rows.sort(key=lambda r: -r["share_us"])
    return rows


def roofline_of(row, peaks):
    # the kernel alone where it was timed so (MFMA stages), else the stage
    t = (row.get("kernel_us") or row["us"]) * 1e-6
    t_hbm = row["alg_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = row["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        ach = row["flops"] / t / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
        if peaks:
            r["peak_measured"] = peaks["mfma_bf16_tflops"]
            r["frac_of_measured"] = round(ach / peaks["mfma_bf16_tflops"], 4)
    else:
        ach = row["alg_bytes"] / t / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
        if peaks:
            r["peak_measured"] = peaks["read_gbs"]
            r["frac_of_measured"] = round(ach / peaks["read_gbs"], 4)
    return r


def cpu_baseline_c5(synth, wl, batches, min_rows: int = 128):
    """The oracle, as it stands, on a bounded sample of the same workload: for
    each projection a slice of `min_rows` output features (gate and up: rows
    of the stored [N][K]; down: columns of the stored [K][N]) drawn from the
    same distribution, split into sub-matrices that the oracle compresses on
    its own; then, per batch of the sweep, decode_full of every sub-matrix and
    the fp64 reference GEMM at that batch.  Run with one thread and with one
    thread per core (independent sub-matrices and output columns), and scaled
    to the metric's unit: bf16 weight bytes delivered per second."""
    import concurrent.futures as cf

    import numpy as np

    from oracle import oracle
    threads = oracle.default_threads()
    subs = []
    for i, (label, n, k, layout) in enumerate(wl.mats):
        if layout == 0:
            per = max(1, min_rows // threads)
            for t in range(threads):
                w = synth.weights(per, k, wl.sigma, seed=wl.seed + 900, stream=100 * i + t)
                subs.append((synth.bits_numpy(w), layout, k))
        else:
            ncol = 64
            for t in range(max(1, min_rows // ncol)):
                w = synth.weights(k, ncol, wl.sigma, seed=wl.seed + 900, stream=100 * i + t)
                subs.append((synth.bits_numpy(w), layout, k))
    xs = {}
    for b in batches:
        for K in {s[2] for s in subs}:
            xs[(b, K)] = synth.bits_numpy(synth.activations(b, K, seed=wl.seed + 901 + b))
    t0 = time.perf_counter()
    comp = [oracle.compress(w, seg_groups=4, layout=layout) for w, layout, _ in subs]
    t_compress = time.perf_counter() - t0
    M = sum(w.size for w, _, _ in subs)

    split = [0.0, 0.0]   # single-thread sweep: seconds in decode_full, in the fp64 GEMM

    def work(i: int, b: int, tally: bool = False) -> None:
        w, layout, K = subs[i]
        t0 = time.perf_counter()
        st, full = comp[i].decode_full()
        assert st == 0
        t1 = time.perf_counter()
        oracle.gemm_ref(xs[(b, K)], full.reshape(w.shape), layout, threads=1)
        if tally:
            split[0] += t1 - t0
            split[1] += time.perf_counter() - t1

    def sweep(nthreads: int) -> float:
        t0 = time.perf_counter()
        if nthreads == 1:
            for b in batches:
                for i in range(len(subs)):
                    work(i, b, True)
        else:
            with cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(lambda a: work(*a), [(i, b) for b in batches for i in range(len(subs))]))
        return time.perf_counter() - t0

    t_multi = sweep(threads)
    t_one = sweep(1)
    rate = lambda t: len(batches) * 2 * M / t / 1e9  # noqa: E731

    # single-thread time of each phase over the whole sample: compress (timed
    # above), one pass of each decode mode, and the fp64 GEMM at every batch
    # (its share of the single-thread sweep)
    def timed(fn) -> float:
        t0 = time.perf_counter()
        for c in comp:
            st, _ = fn(c)
            assert st == 0
        return time.perf_counter() - t0

    t_full = timed(lambda c: c.decode_full())
    t_exp = timed(lambda c: c.decode_exponent())
    t_tc = timed(lambda c: c.transcode())
    t_gemm = split[1]
    layer = sum(n * k for _, n, k, _ in wl.mats)   # weights of one full layer
    scale = layer / M
    phases = {"compress_s": round(t_compress, 3), "decode_full_s": round(t_full, 3),
              "decode_exponent_s": round(t_exp, 3), "transcode_s": round(t_tc, 3),
              "gemm_fp64_all_batches_s": round(t_gemm, 3),
              "weights_per_s": {k: round(M / t, 1) for k, t in (("compress", t_compress), ("decode_full", t_full),
                                                               ("decode_exponent", t_exp), ("transcode", t_tc))},
              "extrapolated": (f"x{scale:.1f} per full layer, x80 layers (extrapolated, not run): "
                               f"compress {t_compress * scale * 80 / 3600:.2f} h, one sweep (decode_full + fp64 GEMM "
                               f"per batch) {t_one * scale * 80 / 3600:.2f} h on 1 thread, "
                               f"{t_multi * scale * 80 / 3600:.2f} h on {threads}")}
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(rate(t_multi), 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(rate(t_one), 4), "cpu_model": model, "nproc": os.cpu_count(),
            "phases_single_thread": phases,
            "sample": (f"{M} weights of one 70B MLP layer ({min_rows} output features of each of gate, up, down, "
                       f"N(0,0.02), in {len(subs)} oracle-compressed sub-matrices); per batch of the sweep "
                       f"{list(batches)}: decode_full of each + fp64 reference GEMM; {t_one:.1f} s on 1 thread, "
                       f"{t_multi:.1f} s on {threads}; value = sweep batches x 2 x sample weights / time")}


def run_c5(args) -> int:
    import torch

    from decode_gemm_exp_amd import synth, uw
    dev = "cuda:0"
    torch.cuda.set_device(0)
    alternate = args.residency == "alternate"
    wl = synth.WORKLOADS["mlp70b"]
    L = args.layers
    batches = [int(b) for b in args.batches.split(",")] if args.batches else list(wl.batches)
    print("bench: building the resident 70B model", file=sys.stderr, flush=True)
    wl, mats, proj = build_c5(uw, synth, torch, dev, L, args.seg_groups, alternate)
    infos = [m.info() for m in mats]
    resident = sum(resident_bytes(i) for i in infos)
    nt = min(args.tune_layers, L) * 3
    if alternate and nt < 6:
        nt = 6
    t_tune = time.perf_counter()
    uw.uw_clear_tuning()
    if args.fixed_pipeline >= 0:   # the library's default kernels, no tuning
        tuned = [{"batch": b, "projection": pj, "pipeline": args.fixed_pipeline, "variant": 0, "split_k": 0,
                  "decode_cus": 0, "layout": infos[pj].layout, "residency": 3, "n": infos[pj].n,
                  "k": infos[pj].k, "sequence_us": 0.0} for b in batches for pj in range(3)]
        nt = 0
    else:
        print(f"bench: autotune on {nt // 3} layers, batches {batches}", file=sys.stderr, flush=True)
        tuned = uw.uw_autotune(mats[:nt], proj[:nt], batches, max_passes=2, json_path=args.tuning_json or None)
    uw.uw_set_tuning(tuned)
    t_tune = time.perf_counter() - t_tune

    plan = {}
    ws_need = 16
    for b in batches:
        jobs, keep = c5_jobs(uw, synth, torch, dev, wl, mats, b)
        plan[b] = (jobs, uw._jobs(jobs), keep)
        ws_need = max(ws_need, uw.uw_sequence_workspace_size(jobs))
    ws = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        c5_step(uw, plan, ws)
    torch.cuda.synchronize()
    print("bench: timing", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        c5_step(uw, plan, ws)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    for m in mats:
        assert uw.uw_sync_status(m) == 0, "decoder reported corrupt data"

    # per-batch pass times: events around each batch's pass, median of 3 sweeps
    per_b = {b: [] for b in batches}
    for _ in range(3):
        evs = []
        for b, (jobs, arr, _) in plan.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            uw.uw_run_sequence(jobs, 0, ws, _arr=arr)
            e1.record()
            evs.append((b, e0, e1))
        torch.cuda.synchronize()
        for b, e0, e1 in evs:
            per_b[b].append(e0.elapsed_time(e1) * 1e3)
    M_total = sum(i.numel for i in infos)
    rows = []
    flops_step = 0.0
    for b in batches:
        t = sorted(per_b[b])[1]
        flops = sum(2.0 * b * i.n * i.k for i in infos)
        flops_step += flops
        choice = {}
        nbytes = 0.0
        for j, (m, i) in enumerate(zip(mats, infos)):
            gp = uw.uw_plan_gemm(m, uw.PIPE_AUTO, b)
            nbytes += job_bytes(i, gp["pipeline"], b)
            pj = proj[j]
            lab = (("easy_" if pj < 3 else "hard_") + wl.mats[pj % 3][0]) if alternate else wl.mats[pj][0]
            if lab not in choice:
                e = uw.uw_lookup_tuning(i.n, i.k, i.layout, (1 if i.has_stream else 0) | (2 if i.has_palette_idx else 0), b)
                choice[lab] = {"pipeline": PIPE_NAMES[gp["pipeline"]], "kernel": gp["kernel"],
                               "variant": gp["variant"], "k_slices": gp["k_slices"],
                               "decode_cus": e["decode_cus"] if e else 0}
        rows.append({"batch": b, "us_per_pass": round(t, 1), "decoded_gbs": round(2 * M_total / t / 1e3, 1),
                     "tflops": round(flops / t / 1e6, 2), "hbm_frac": round(nbytes / t / 1e3 / HBM_PEAK_GBS, 4),
                     "mfma_frac": round(flops / t / 1e6 / BF16_PEAK_TFLOPS, 4),
                     "roofline_frac": round(max(nbytes / 8e12, flops / 2.5e15) / (t * 1e-6), 4), "choice": choice})
        print(f"bench: batch {b}: {t / 1e3:.2f} ms per pass", file=sys.stderr, flush=True)

    print("bench: per-kernel breakdown", file=sys.stderr, flush=True)
    peaks = yardsticks(uw, torch, dev)
    breakdown = c5_breakdown(uw, torch, dev, wl, mats, proj, infos, batches, plan, alternate,
                             launches=max(8, min(args.steps, 20)))
    dom = breakdown[0]
    roof = roofline_of(dom, peaks)
    roof.update({"traffic": load_traffic(f"{dom['stage']}_{dom['projection']}_b{dom['batch']}", "mlp70b"),
                 "kernel": dom["kernel"], "stage": dom["stage"], "projection": dom["projection"],
                 "batch": dom["batch"], "alg_bytes_per_launch": dom["alg_bytes"],
                 "flops_per_launch": dom["flops"], "avg_launch_us": dom.get("kernel_us") or dom["us"],
                 "stage_us": dom["us"], "launches_timed": dom["launches_timed"],
                 "share_of_step": round(dom["share_us"] / (ms_per_step * 1e3), 4),
                 "timing": f"avg_launch_us: the kernel alone, between HIP events the library records on the launch "
                           f"stream immediately around its launch (uw_set_kernel_events), over "
                           f"{dom['launches_timed']} launches rotating over 4 layers after the timed steps; "
                           f"stage_us: HIP events around the whole stage call over the same launches back to back "
                           f"(with x packing and any split-K reduction); the dominant stage is the one with the "
                           f"largest share of the step"})
    value = len(batches) * 2 * M_total / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"mlp70b: {L} layers of Llama-70B MLP (gate/up 28672x8192 stored [N][K], down "
                               f"8192x28672 stored [K][N]) bf16 N(0,0.02), compressed-resident, autotuned, one "
                               f"80-layer pass per batch of the sweep {batches}",
                   "batches": batches, "layers": L, "tune_layers": nt // 3,
                   "residency": "even layers palette indices only, odd layers Huffman stream only" if alternate
                                else "palette indices and Huffman stream in every layer",
                   "resident_gb": round(resident / 1e9, 2), "dense_bf16_gb": round(2 * M_total / 1e9, 2),
                   "bits_per_weight": round(8 * sum(i.compressed_bytes for i in infos) / M_total, 3),
                   "seg_groups": args.seg_groups, "parallelism": "single GPU"},
        "value_definition": "sum over the sweep's batches of the bf16 weight bytes delivered to the GEMMs "
                            "(2 x 56.37 G weights per pass) / step wall time",
        "tflops_step": round(flops_step / (ms_per_step * 1e-3) / 1e12, 1),
        "tune_seconds": round(t_tune, 1), "rows": rows, "roofline": roof, "measured_peaks": peaks,
        "breakdown_top": breakdown[:12],
    }
    if not args.no_extras:
        print("bench: single-matrix and larger-batch rows", file=sys.stderr, flush=True)
        res["gate8b"] = gate8b_section(uw, synth, torch, dev, args, with_cpu=False)
        res["extras"] = extras(uw, synth, torch, dev)
    if not args.no_cpu:
        print("bench: oracle cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_c5(synth, wl, batches)
    uw.uw_clear_tuning()
    uw.uw_release_resources()
    print(json.dumps(res), flush=True)
    return 0


def gate8b_section(uw, synth, torch, dev, args, with_cpu: bool):
    """The four pipelines of the method on the Llama-3.1-8B gate projection
    (14336 x 4096 bf16, N(0,0.02), 0.05 % outliers x 2^10) at batch 1, over
    `rotate` compressed copies: per-stage kernel times, per-pipeline rates,
    and the roofline of its longest stage.  Returns a dict; `value` is the
    step's decoded-weight GB/s (4 x 2 x numel per step)."""
    stream = torch.cuda.current_stream()
    wl = synth.WORKLOADS["gate8b"]
    _, n, k, layout = wl.mats[0]
    w = synth.workload_weights(wl, 0, device=dev)
    x = synth.activations(1, k, seed=wl.seed, device=dev)
    mats = []
    for _ in range(args.rotate):
        m = uw.uw_compress(w, n, k, layout, seg_groups=args.seg_groups)
        uw.uw_transcode_palette(m, None)
        mats.append(m)
    torch.cuda.synchronize()
    info = mats[0].info()
    w_np = synth.bits_numpy(w) if with_cpu else None
    x_np = synth.bits_numpy(x) if with_cpu else None
    del w
    numel = info.numel
    ws_bf16 = torch.empty(numel, dtype=torch.int16, device=dev)
    ws_e = torch.empty(numel, dtype=torch.uint8, device=dev)
    ws_p = torch.empty(numel // 2, dtype=torch.uint8, device=dev)
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for _ in range(4)]
    part = torch.empty(max(16, max(uw.uw_workspace_size(mats[0], p, 1) for p in range(4))), dtype=torch.uint8,
                       device=dev)
    stages = ["decode_full", "gemv_full", "decode_exponent", "gemv_exponent", "transcode", "gemv_transcode",
              "gemv_direct"]

    def run_stage(st, m):
        if st == "decode_full":
            uw.uw_decode_full(m, ws_bf16, stream)
        elif st == "gemv_full":
            uw.uw_matmul_stage(m, 0, ws_bf16, x, ys[0], part, stream=stream)
        elif st == "decode_exponent":
            uw.uw_decode_exponent(m, ws_e, stream)
        elif st == "gemv_exponent":
            uw.uw_matmul_stage(m, 1, ws_e, x, ys[1], part, stream=stream)
        elif st == "transcode":
            uw.uw_transcode_palette(m, ws_p, stream)
        elif st == "gemv_transcode":
            uw.uw_matmul_stage(m, 2, ws_p, x, ys[2], part, stream=stream)
        else:
            uw.uw_matmul_stage(m, 3, None, x, ys[3], part, stream=stream)

    def step(i):
        m = mats[i % len(mats)]
        for st in stages:
            run_stage(st, m)

    def burst_us(st, nl, i0):
        """Average launch of one stage: one pair of events around nl
        back-to-back launches over the rotated inputs.  A timing marker between
        two kernels holds the next dispatch back by about 5 us, so events
        around single launches would overstate these short kernels."""
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_gpu(torch, nl)
        d0.record(stream)
        for i in range(nl):
            run_stage(st, mats[(i0 + i) % len(mats)])
        d1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * d0.elapsed_time(d1) / nl

    steps = args.gate8b_steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nb = max(5, steps // 4)
    stage_us = {st: burst_us(st, nb, args.warmup) for st in stages}
    dom = max(stages, key=lambda st: stage_us[st])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    dom_us = burst_us(dom, steps, args.warmup)
    for m in mats:
        assert uw.uw_sync_status(m) == 0, "decoder reported corrupt data"
    kernels = {}
    for st in stages:
        t = stage_us[st] * 1e-6
        ab = algorithmic_bytes(info, st)
        kernels[st] = {"kernel": STAGE_KERNELS[st], "us": round(stage_us[st], 2), "alg_bytes": int(ab),
                       "gbs": round(ab / t / 1e9, 1), "hbm_frac": round(ab / t / 1e9 / HBM_PEAK_GBS, 4),
                       "traffic": load_traffic(st)}
        vf = load_valu_floor(st) if st.startswith(("decode", "transcode")) else None
        if vf:   # the decoders against the vector ALU as well as HBM
            kernels[st]["alu"] = {"valu_instr": int(vf["valu_instr"]), "floor_us": vf["valu_floor_us"],
                                  "frac": round(vf["valu_floor_us"] / stage_us[st], 4)}
    pipes = {}
    for p, (pre, gem) in zip(PIPE_NAMES, [("decode_full", "gemv_full"), ("decode_exponent", "gemv_exponent"),
                                          ("transcode", "gemv_transcode"), (None, "gemv_direct")]):
        t = (stage_us[pre] if pre else 0.0) + stage_us[gem]
        pb = (algorithmic_bytes(info, pre) if pre else 0.0) + algorithmic_bytes(info, gem)
        pipes[p] = {"us": round(t, 2), "decoded_gbs": round(2 * numel / (t * 1e-6) / 1e9, 1),
                    "hbm_frac": round(pb / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    dom_t = dom_us * 1e-6
    dom_b = algorithmic_bytes(info, dom)
    roofline = {"bound": "hbm", "achieved": round(dom_b / dom_t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_b / dom_t / 1e9 / HBM_PEAK_GBS, 4), "traffic": load_traffic(dom),
                "kernel": STAGE_KERNELS[dom], "stage": dom, "alg_bytes_per_launch": int(dom_b),
                "avg_launch_us": round(dom_us, 2), "launches_timed": steps,
                "timing": f"HIP events around {steps} back-to-back launches after the timed steps"}
    out = {"value": round(4 * 2 * numel / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s",
           "ms_per_step": round(ms_per_step, 4), "steps": steps,
           "workload": "gate8b: Llama-3.1-8B gate projection 14336x4096 bf16 N(0,0.02), 0.05% outliers x2^10, "
                       "batch 1, pipelines full/exponent/transcode/direct",
           "rotated_copies": args.rotate, "bits_per_weight": round(info.bits_per_weight, 3),
           "verbatim_groups": int(info.verbatim_groups), "pipelines": pipes, "kernels": kernels,
           "roofline": roofline}
    del mats
    torch.cuda.empty_cache()
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline_gate8b(w_np, x_np)
    return out


def run_gate8b(args) -> int:
    import torch

    from decode_gemm_exp_amd import synth, uw
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        uw.uw_yardstick(0, a, b, nb)
        torch.cuda.synchronize()
        del a, b
    args.gate8b_steps = args.steps
    g = gate8b_section(uw, synth, torch, dev, args, with_cpu=not args.no_cpu)
    res = {"metric": METRIC, "value": g["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": g["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": g["workload"], "batch": 1, "rotated_copies": args.rotate,
                      "seg_groups": args.seg_groups, "parallelism": "single GPU"}}
    res.update({k: v for k, v in g.items() if k not in res and k != "workload"})
    uw.uw_release_resources()
    print(json.dumps(res), flush=True)
    return 0


def run_probe(args) -> int:
    """A short run for counter collection (rocprofv3 --pmc): a plain device
    copy of 256 MiB by the library's copy kernel (the counters' calibration),
    then `launches` launches of one stage of the resident 70B model, given as
    stage,projection,batch,pipeline,variant,split (stage 'gemm' or 'prep')."""
    import torch

    from decode_gemm_exp_amd import synth, uw
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stage, pname, b, p, v, sk = args.probe.split(",")
    b, p, v, sk = int(b), int(p), int(v), int(sk)
    wl, mats, proj = build_c5(uw, synth, torch, dev, 4, args.seg_groups, False)
    pj = [lab for lab, _, _, _ in wl.mats].index(pname)
    idx = [j for j in range(len(mats)) if proj[j] == pj]
    info = mats[idx[0]].info()
    nb = 256 << 20
    a = torch.empty(nb, dtype=torch.uint8, device=dev)
    c = torch.empty_like(a)
    uw.uw_yardstick(0, a, c, nb)
    torch.cuda.synchronize()
    del a, c
    xin = synth.activations(b, info.k, seed=wl.seed + b, device=dev)
    y = torch.empty((b, info.n), dtype=torch.float32, device=dev)
    preps = []
    if p != 3:
        sz = {0: 2 * info.numel, 1: info.numel, 2: info.numel // 2}[p]
        preps = [torch.empty(sz, dtype=torch.uint8, device=dev) for _ in idx]
        call = {0: uw.uw_decode_full, 1: uw.uw_decode_exponent, 2: uw.uw_transcode_palette}[p]
    cfg = {"variant": v, "split_k": sk}
    part = torch.empty(max(16, uw.uw_workspace_size_cfg(mats[idx[0]], p, b, cfg)), dtype=torch.uint8, device=dev)
    for i in range(args.steps):
        j = i % len(idx)
        if p != 3 and (stage == "prep" or i < len(idx)):
            call(mats[idx[j]], preps[j])
        if stage == "gemm":
            uw.uw_matmul_stage(mats[idx[j]], p, preps[j] if preps else None, xin, y, part, cfg=cfg)
    torch.cuda.synchronize()
    uw.uw_release_resources()
    print(json.dumps({"probe": args.probe, "launches": args.steps}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed sweeps (mlp70b) or steps (gate8b)")
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--rotate", type=int, default=10, help="gate8b: compressed copies cycled through")
    ap.add_argument("--gate8b-steps", type=int, default=20, help="gate8b rows inside the mlp70b run")
    ap.add_argument("--seg-groups", type=int, default=4, help="groups per bitstream segment")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the single-matrix and larger-batch rows")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="gate8b: run the library's device copy of this size first (HBM counter calibration)")
    ap.add_argument("--workload", default="mlp70b", choices=["gate8b", "mlp70b"])
    ap.add_argument("--layers", type=int, default=80, help="mlp70b: resident layers")
    ap.add_argument("--tune-layers", type=int, default=4, help="mlp70b: layers the autotuner times")
    ap.add_argument("--batches", default="", help="mlp70b: comma-separated batch sizes")
    ap.add_argument("--fixed-pipeline", type=int, default=-1, choices=[-1, 0, 1, 2, 3],
                    help="mlp70b: skip the autotuner; every projection runs this pipeline with the default kernels")
    ap.add_argument("--residency", default="both", choices=["both", "alternate"],
                    help="mlp70b: both forms in every layer, or alternating easy (palette indices) and hard "
                         "(Huffman stream) layers")
    ap.add_argument("--probe", default="", help="counter run: stage,projection,batch,pipeline,variant,split")
    ap.add_argument("--tuning-json", default="", help="mlp70b: also write the autotuner's choices to this file")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; the path shards per matrix "
                                   "(see the design notes) but no multi-GPU run is made", "n_gpus": args.gpus}))
        return 2
    if args.probe:
        return run_probe(args)
    if args.workload == "gate8b":
        return run_gate8b(args)
    return run_c5(args)


if __name__ == "__main__":
    sys.exit(main())
