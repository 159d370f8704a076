"""GPU checks of the boundary's run-time choices: UW_PIPE_AUTO and cfg == NULL
against the tuning table (the autotuner's per-projection, per-batch
configuration, looked up at run time), the allocator hooks, and the release
of the library's HIP objects.  Every GEMM output is also checked against the
fp64 oracle with the 2^-10 * sum|x w| bound."""
import os
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def uw():
    from decode_gemm_exp_amd import uw as _uw
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return _uw


@pytest.fixture(scope="module")
def synth():
    from decode_gemm_exp_amd import synth as _s
    return _s


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def matmul(uw, m, pipeline, x, cfg=None, ws_bytes=None):
    info = m.info()
    y = torch.full((x.shape[0], info.n), float("nan"), dtype=torch.float32, device=DEV)
    nb = ws_bytes if ws_bytes is not None else uw.uw_workspace_size_cfg(m, pipeline, x.shape[0], cfg)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    uw.uw_matmul_reconstruct(m, pipeline, x, y, ws, cfg=cfg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def within(oracle, y, x, w_np, layout):
    y_ref, A = oracle.gemm_ref(bits(x), w_np, layout)
    ok, worst = oracle.gemm_check(y, y_ref, A)
    assert ok, f"worst err/bound {worst:.3g}"


@pytest.fixture()
def clean_table(uw):
    uw.uw_clear_tuning()
    yield
    uw.uw_clear_tuning()


def test_auto_equals_tuned_choice(uw, synth, oracle, clean_table, tmp_path):
    """uw_autotune's JSON loaded into the table: AUTO runs exactly the tuned
    pipeline and kernel (bit-identical output), within the fp64 bound."""
    say("boundary: autotune 2 matrices, AUTO vs tuned choice")
    n, k = 1024, 2048
    ws_ = [synth.weights(n, k, 0.02, 0.001, 10, seed=71 + i).to(DEV) for i in range(2)]
    ms = [uw.uw_compress(w, n, k, 0) for w in ws_]
    for m in ms:
        uw.uw_transcode_palette(m, None)
    batches = [1, 24, 160]
    path = str(tmp_path / "tuned.json")
    tuned = uw.uw_autotune(ms, [0, 0], batches, max_passes=1, json_path=path)
    assert len(tuned) == len(batches)
    for e in tuned:
        assert (e["n"], e["k"], e["layout"], e["residency"]) == (n, k, 0, 3)
    uw.uw_load_tuning(path)
    w_np = bits(ws_[0])
    for b, e in zip(batches, tuned):
        x = synth.activations(b, k, seed=5 + b).to(DEV)
        got = uw.uw_lookup_tuning(n, k, 0, 3, b)
        assert (got["pipeline"], got["variant"], got["split_k"]) == (e["pipeline"], e["variant"], e["split_k"])
        cfg = {"variant": e["variant"], "split_k": e["split_k"], "decode_cus": e["decode_cus"]}
        y_auto = matmul(uw, ms[0], uw.PIPE_AUTO, x)
        y_tuned = matmul(uw, ms[0], e["pipeline"], x, cfg)
        y_null = matmul(uw, ms[0], e["pipeline"], x)          # cfg NULL: the tuned kernel
        assert np.array_equal(y_auto, y_tuned), f"batch {b}"
        assert np.array_equal(y_null, y_tuned), f"batch {b}"
        within(oracle, y_auto, x, w_np, 0)


def test_null_cfg_takes_tuned_kernel_and_split(uw, synth, oracle, clean_table):
    """A table entry forcing a K split: cfg == NULL runs it, and the plain
    uw_workspace_size covers it."""
    n, k, b = 768, 4096, 96
    say(f"boundary: tuned split on {n}x{k} at {b} rows")
    w = synth.weights(n, k, 0.02, 0.001, 10, seed=91).to(DEV)
    m = uw.uw_compress(w, n, k, 0)
    uw.uw_transcode_palette(m, None)
    x = synth.activations(b, k, seed=92).to(DEV)
    cfg = {"variant": 3, "split_k": 4, "decode_cus": 0}    # 128x128 LDS tile, K in 4 slices
    uw.uw_set_tuning([{"batch": 64, "projection": 0, "pipeline": 3, "variant": 3, "split_k": 4, "decode_cus": 0,
                       "layout": 0, "residency": 3, "n": n, "k": k, "sequence_us": 0.0}])
    need_null = uw.uw_workspace_size(m, 3, b)
    assert need_null >= uw.uw_workspace_size_cfg(m, 3, b, cfg)
    y_null = matmul(uw, m, 3, x, None, ws_bytes=need_null)
    y_cfg = matmul(uw, m, 3, x, cfg)
    assert np.array_equal(y_null, y_cfg)
    # another pipeline at the same shape keeps the library default
    y_exp = matmul(uw, m, 1, x)
    within(oracle, y_null, x, bits(w), 0)
    within(oracle, y_exp, x, bits(w), 0)
    # AUTO with the table: the tuned pipeline (3); without: direct palette
    # (indices resident), and exponent once they are dropped
    assert np.array_equal(matmul(uw, m, uw.PIPE_AUTO, x), y_cfg)
    uw.uw_clear_tuning()
    assert np.array_equal(matmul(uw, m, uw.PIPE_AUTO, x), matmul(uw, m, 3, x))
    uw.uw_drop_palette(m)
    assert np.array_equal(matmul(uw, m, uw.PIPE_AUTO, x), matmul(uw, m, 1, x))


def test_sequence_auto_jobs_and_release(uw, synth, oracle, clean_table):
    """uw_run_sequence with AUTO jobs equals the explicit jobs; the split
    streams and events are destroyed by uw_release_resources and made again."""
    n, k = 640, 1024
    say("boundary: AUTO sequence + release")
    w0 = synth.weights(n, k, 0.02, 0.0, 0, seed=101).to(DEV)
    w1 = synth.weights(k, n, 0.02, 0.0, 0, seed=102).to(DEV)     # a second projection: N = 1024, K = 640
    m0 = uw.uw_compress(w0, n, k, 0)
    m1 = uw.uw_compress(w1, k, n, 0)
    b = 48
    x0 = synth.activations(b, k, seed=103).to(DEV)
    x1 = synth.activations(b, n, seed=104).to(DEV)
    uw.uw_set_tuning([
        {"batch": b, "projection": 0, "pipeline": 2, "variant": 2, "split_k": 0, "decode_cus": 64,
         "layout": 0, "residency": 1, "n": n, "k": k, "sequence_us": 0.0},
        {"batch": b, "projection": 1, "pipeline": 1, "variant": 0, "split_k": 0, "decode_cus": 256,
         "layout": 0, "residency": 1, "n": k, "k": n, "sequence_us": 0.0}])

    def run(jobs_spec):
        ys = [torch.full((b, m.info().n), float("nan"), dtype=torch.float32, device=DEV) for m, _, _, _ in jobs_spec]
        jobs = [uw.Job(m, p, x, y, cfg) for (m, p, x, cfg), y in zip(jobs_spec, ys)]
        ws = torch.empty(max(16, uw.uw_sequence_workspace_size(jobs)), dtype=torch.uint8, device=DEV)
        uw.uw_run_sequence(jobs, 0, ws)
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys]

    auto = run([(m0, uw.PIPE_AUTO, x0, None), (m1, uw.PIPE_AUTO, x1, None)])
    explicit = run([(m0, 2, x0, {"variant": 2, "decode_cus": 64}), (m1, 1, x1, {"decode_cus": 256})])
    for a, e in zip(auto, explicit):
        assert np.array_equal(a, e)
    within(oracle, auto[0], x0, bits(w0), 0)
    within(oracle, auto[1], x1, bits(w1), 0)
    uw.uw_release_resources()
    again = run([(m0, uw.PIPE_AUTO, x0, None), (m1, uw.PIPE_AUTO, x1, None)])
    for a, e in zip(again, explicit):
        assert np.array_equal(a, e)
    uw.uw_release_resources()


def grouped(uw, ms, pipeline, x, cfg=None):
    n = sum(m.info().n for m in ms)
    y = torch.full((x.shape[0], n), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, uw.uw_workspace_size_grouped(ms, pipeline, x.shape[0], cfg)), dtype=torch.uint8,
                     device=DEV)
    uw.uw_matmul_reconstruct_grouped(ms, pipeline, x, y, ws, cfg=cfg)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("shape", ["qkv", "gate_up"])
def test_grouped_auto_equals_tuned_choice(uw, synth, oracle, clean_table, tmp_path, shape):
    """uw_autotune_grouped on two layers of the 8B q+k+v (4096, 1024, 1024 x
    4096) or gate+up (2 x 14336 x 4096) calls, its JSON loaded: a grouped
    AUTO call and a grouped call with cfg == NULL run exactly the tuned
    pipeline and kernel (bit-identical to the explicit choice), each
    matrix's columns within the fp64 bound on 48 sampled columns."""
    k = 4096
    ns = [4096, 1024, 1024] if shape == "qkv" else [14336, 14336]
    say(f"boundary: grouped autotune {shape}")
    ws_ = [[synth.weights(n, k, 0.02, 0.001, 10, seed=400 + 10 * g + i).to(DEV) for i, n in enumerate(ns)]
           for g in range(2)]
    ms = [[uw.uw_compress(w, n, k, 0) for w, n in zip(gw, ns)] for gw in ws_]
    for g in ms:
        for m in g:
            uw.uw_transcode_palette(m, None)
    batches = [1, 24, 300]
    path = str(tmp_path / "grouped.json")
    tuned = uw.uw_autotune_grouped(ms, batches, json_path=path)
    assert len(tuned) == len(batches)
    for b, e in zip(batches, tuned):
        assert (e["batch"], e["n"], e["k"], e["layout"], e["residency"], e["group"]) == (b, sum(ns), k, 0, 3, len(ns))
        say(f"  batch {b}: pipeline {e['pipeline']} variant {e['variant']} split {e['split_k']} "
            f"{e['sequence_us']:.1f} us")
    uw.uw_load_tuning(path)
    rng = np.random.default_rng(17)
    for b, e in zip(batches, tuned):
        got = uw.uw_lookup_tuning_grouped(sum(ns), k, 0, 3, len(ns), b)
        assert (got["pipeline"], got["variant"], got["split_k"]) == (e["pipeline"], e["variant"], e["split_k"])
        x = synth.activations(b, k, seed=31 + b).to(DEV)
        cfg = {"variant": e["variant"], "split_k": e["split_k"], "decode_cus": 0}
        y_auto = grouped(uw, ms[1], uw.PIPE_AUTO, x)
        y_tuned = grouped(uw, ms[1], e["pipeline"], x, cfg)
        y_null = grouped(uw, ms[1], e["pipeline"], x)
        assert np.array_equal(y_auto, y_tuned), f"batch {b}"
        assert np.array_equal(y_null, y_tuned), f"batch {b}"
        x_np = bits(x)
        col = 0
        for i, n in enumerate(ns):
            c = np.sort(rng.choice(n, 48, replace=False))
            w_sel = bits(ws_[1][i].index_select(0, torch.from_numpy(c).to(DEV)))
            y_ref, A = oracle.gemm_ref(x_np, w_sel, 0)
            ok, worst = oracle.gemm_check(y_auto[:, col + c], y_ref, A)
            assert ok, f"batch {b} matrix {i}: worst err/bound {worst:.3g}"
            col += n
    uw.uw_release_resources()


@pytest.mark.parametrize("batch,cfg", [(512, None), (16, {"variant": 13}), (100, {"variant": 11}), (48, {"variant": 3, "split_k": 3})])
def test_kernel_events_bracket_the_kernel(uw, synth, batch, cfg):
    """uw_set_kernel_events: the output is unchanged, and the events bracket
    the main kernel alone (a positive time no longer than the whole call's);
    the 512-row call packs x first, the 100-row register-fed call launches
    its kernel twice (64 + 36 rows), the 48-row one reduces three K slices."""
    n, k = 1024, 2048
    say(f"boundary: kernel events, batch {batch}, cfg {cfg}")
    w = synth.weights(n, k, 0.02, 0.001, 10, seed=131).to(DEV)
    m = uw.uw_compress(w, n, k, 0)
    uw.uw_transcode_palette(m, None)
    x = synth.activations(batch, k, seed=132).to(DEV)
    y_ref = matmul(uw, m, 3, x, cfg)
    stream = torch.cuda.current_stream()
    y = torch.full((batch, n), float("nan"), dtype=torch.float32, device=DEV)
    nb = uw.uw_workspace_size_cfg(m, 3, batch, cfg) if cfg else uw.uw_workspace_size(m, 3, batch)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    ka, kb, ca, cb = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (ka, kb):
        e.record(stream)
    torch.cuda.synchronize()
    try:
        uw.uw_set_kernel_events(ka, kb)
        ca.record(stream)
        uw.uw_matmul_reconstruct(m, 3, x, y, ws, cfg=cfg, stream=stream)
        cb.record(stream)
    finally:
        uw.uw_set_kernel_events(None, None)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_ref)
    t_kernel, t_call = ka.elapsed_time(kb), ca.elapsed_time(cb)
    assert 0.0 < t_kernel <= t_call, (t_kernel, t_call)


def test_allocator_hooks(uw, synth, oracle):
    """Sections, scratch and resident indices come from the hooks and go back
    through them; a NULL from the hook is UW_ERR_NOMEM."""
    say("boundary: allocator hooks")
    alloc = uw.TorchAllocator(DEV)
    n, k = 512, 1024
    w = synth.weights(n, k, 0.02, 0.002, 12, seed=111).to(DEV)
    try:
        uw.uw_set_allocator(alloc.alloc, alloc.free)
        m = uw.uw_compress(w, n, k, 0)
        made = alloc.allocs
        assert made >= 6                     # sm, flags, ranks, offsets, stream, table, flag; scratch
        uw.uw_transcode_palette(m, None)
        assert alloc.allocs == made + 1      # the resident indices
        out = torch.empty(n * k, dtype=torch.int16, device=DEV)
        uw.uw_decode_full(m, out)
        assert uw.uw_sync_status(m) == 0
        assert np.array_equal(out.cpu().numpy().view(np.uint16), bits(w).ravel())
        x = synth.activations(4, k, seed=112).to(DEV)
        within(oracle, matmul(uw, m, 3, x), x, bits(w), 0)
        # a handle frees through the hooks it was made with, even after a reset
        uw.uw_set_allocator(None, None)
        m.free()
        torch.cuda.synchronize()
        assert alloc.frees == alloc.allocs and not alloc.live
        uw.uw_set_allocator(lambda nbytes: 0, lambda p: None)
        with pytest.raises(uw.UwError) as ei:
            uw.uw_compress(w, n, k, 0)
        assert ei.value.status == -3
    finally:
        uw.uw_set_allocator(None, None)
    m2 = uw.uw_compress(w, n, k, 0)          # back on hipMalloc
    assert m2.info().numel == n * k
