"""Parity on the 80-layer Llama-70B MLP workload as the benchmark runs it.

* Codec: for every 8th layer and the last (33 matrices of 235 M weights), the
  GPU's UWF1 blob equals the oracle's byte for byte, the GPU full decode gives
  back the original weights, the exponent decode their exponent bytes, and the
  GPU transcode equals the oracle's.
* Sequence: all 80 layers resident with both forms, the autotuner's choices
  loaded into the tuning table, one uw_run_sequence pass over the 240 matrices
  with UW_PIPE_AUTO jobs at 1, 8, 64, 256, 512 and 1024 rows (the GEMVs, the
  register-fed kernel, the LDS tiles and the single-rebuild tile), every job
  with its own output; each output checked on 64 sampled columns against the
  oracle's fp64 GEMM on the original weights (|y - y_ref| <= 2^-10 sum|x w|).
"""
import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WORKERS = max(1, min(8, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def uw():
    from decode_gemm_exp_amd import uw as _uw
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return _uw


@pytest.fixture(scope="module")
def synth():
    from decode_gemm_exp_amd import synth as _s
    return _s


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_check(oracle, w_np, layout, blob, tc, what):
    """Runs on a worker thread: the oracle's blob and transcode for one matrix
    against the GPU's."""
    om = oracle.compress(w_np, seg_groups=4, layout=layout)
    oblob = om.export()
    if blob != oblob:
        a = np.frombuffer(blob, np.uint8)
        b = np.frombuffer(oblob, np.uint8)
        if a.size != b.size:
            return f"{what}: blob sizes {a.size} vs {b.size}"
        bad = np.nonzero(a != b)[0]
        return f"{what}: blob differs at {bad.size} bytes, first {bad[:6]}"
    st, otc = om.transcode()
    if st != 0 or not np.array_equal(otc, tc):
        return f"{what}: transcode differs"
    return None


@pytest.mark.timeout(900)
def test_c5_codec_every_8th_layer(uw, synth, oracle):
    wl = synth.WORKLOADS["mlp70b"]
    layers = list(range(0, wl.layers, 8)) + [wl.layers - 1]
    futures = []
    with cf.ThreadPoolExecutor(max_workers=WORKERS) as ex:
        for layer in layers:
            for i, (label, n, k, layout) in enumerate(wl.mats):
                what = f"layer {layer} {label}"
                say(f"c5 codec: {what}")
                w = synth.workload_weights(wl, i, layer=layer, device=DEV)
                m = uw.uw_compress(w, n, k, layout)
                numel = n * k
                out = torch.empty(numel, dtype=torch.int16, device=DEV)
                uw.uw_decode_full(m, out)
                e = torch.empty(numel, dtype=torch.uint8, device=DEV)
                uw.uw_decode_exponent(m, e)
                tc = torch.empty(numel // 2, dtype=torch.uint8, device=DEV)
                uw.uw_transcode_palette(m, tc)
                assert uw.uw_sync_status(m) == 0, what
                wi = w.view(torch.int16).reshape(-1)
                assert torch.equal(out, wi), f"{what}: full decode not bit-exact"
                assert torch.equal(e, ((wi.to(torch.int32) >> 7) & 0xFF).to(torch.uint8)), \
                    f"{what}: exponent decode differs"
                blob = uw.uw_export(m)
                futures.append(ex.submit(_oracle_check, oracle, bits(w), layout, blob, tc.cpu().numpy(), what))
                del w, out, e, tc, wi, m
                torch.cuda.empty_cache()
                while len(futures) >= 2 * WORKERS or any(f.done() for f in futures):   # bounded host memory
                    f = next((f for f in futures if f.done()), futures[0])
                    assert f.result() is None, f.result()
                    futures.remove(f)
        for f in futures:
            assert f.result() is None, f.result()


@pytest.mark.timeout(900)
def test_c5_tuned_sequence_all_layers(uw, synth, oracle):
    wl = synth.WORKLOADS["mlp70b"]
    L = wl.layers
    mats, proj = [], []
    for layer in range(L):
        for i, (label, n, k, layout) in enumerate(wl.mats):
            w = synth.workload_weights(wl, i, layer=layer, device=DEV)
            m = uw.uw_compress(w, n, k, layout)
            uw.uw_transcode_palette(m, None)
            mats.append(m)
            proj.append(i)
            del w
    torch.cuda.synchronize()
    say("c5 sequence: 80 layers resident; tuning on 4 layers")
    batches = [1, 8, 64, 256, 512, 1024]
    tuned = uw.uw_autotune(mats[:12], proj[:12], batches, max_passes=1)
    uw.uw_clear_tuning()
    uw.uw_set_tuning(tuned)
    rng = np.random.default_rng(5)
    cols = {i: np.sort(rng.choice(wl.mats[i][1], 64, replace=False)) for i in range(3)}
    try:
        for b in batches:
            K_in, H = wl.mats[0][2], wl.mats[2][2]
            x = synth.activations(b, K_in, seed=wl.seed + b, device=DEV)
            h = synth.activations(b, H, seed=wl.seed + 7 + b, device=DEV)
            ys = [torch.full((b, wl.mats[j % 3][1]), float("nan"), dtype=torch.float32, device=DEV)
                  for j in range(len(mats))]
            jobs = [uw.Job(m, uw.PIPE_AUTO, h if j % 3 == 2 else x, ys[j], None) for j, m in enumerate(mats)]
            ws = torch.empty(max(16, uw.uw_sequence_workspace_size(jobs)), dtype=torch.uint8, device=DEV)
            choice = {wl.mats[i][0]: uw.uw_plan_gemm(mats[i], uw.PIPE_AUTO, b) for i in range(3)}
            say(f"c5 sequence: batch {b}, " + ", ".join(f"{k}: pipeline {v['pipeline']} {v['kernel']}"
                                                      for k, v in choice.items()))
            uw.uw_run_sequence(jobs, 0, ws)
            torch.cuda.synchronize()
            for m in mats[:3]:
                assert uw.uw_sync_status(m) == 0
            del ws
            x_np, h_np = bits(x), bits(h)
            pending = []
            with cf.ThreadPoolExecutor(max_workers=2) as ex:
                for j in range(len(mats)):
                    layer, i = divmod(j, 3)
                    label, n, k, layout = wl.mats[i]
                    c = cols[i]
                    w = synth.workload_weights(wl, i, layer=layer, device=DEV)
                    ci = torch.from_numpy(c).to(DEV)
                    w_sel = (w.index_select(0, ci) if layout == 0 else w.index_select(1, ci)).contiguous()
                    y_sel = ys[j].index_select(1, ci).cpu().numpy()
                    del w
                    pending.append(ex.submit(_gemm_check, oracle, y_sel, h_np if i == 2 else x_np, bits(w_sel),
                                             layout, f"batch {b} layer {layer} {label}"))
                    if len(pending) >= 8:
                        for f in pending:
                            assert f.result() is None, f.result()
                        pending = []
                for f in pending:
                    assert f.result() is None, f.result()
            del ys, jobs
            torch.cuda.empty_cache()
    finally:
        uw.uw_clear_tuning()
        uw.uw_release_resources()


def _gemm_check(oracle, y_sel, x_np, w_sel, layout, what):
    if not np.all(np.isfinite(y_sel)):
        return f"{what}: unwritten or non-finite outputs"
    y_ref, A = oracle.gemm_ref(x_np, w_sel, layout)
    ok, worst = oracle.gemm_check(y_sel, y_ref, A)
    return None if ok else f"{what}: worst err/bound {worst:.3g}"
