"""Parity at the full sizes of the workloads, in the launch configuration
the benchmark times.

  w256x512 : 256x512, 0.2% outliers x2^12 -- compress, full decode, B=1 GEMM
  gate8b   : 14336x4096, 0.05% outliers x2^10 -- full + exponent decode, B=1
  gateup8b : 2 x 14336x4096 -- transcode + direct palette, fused, B=1,8,64
  down8b   : 4096x14336 stored transposed [14336][4096] -- B=256,1024
  mlp70b   : Llama-70B MLP layer shapes (gate/up 28672x8192, down 8192x28672
             stored [28672][8192]); streams of one full layer against the
             oracle, GEMMs on sampled output columns at B=1,64,1024
  attn8b, attn70b : attention q/k/v/o of the same models (q, o hidden x
             hidden; k, v 1024 x hidden); fused q+k+v and o

Streams and decoded weights are compared whole; GEMMs whole where the fp64
reference takes seconds, else on sampled output columns.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def uw():
    from decode_gemm_exp_amd import uw as _uw
    return _uw


@pytest.fixture(scope="module")
def synth():
    from decode_gemm_exp_amd import synth as _s
    return _s


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def codec_parity(uw, oracle, w, n, k, layout, sg=4):
    w_np = bits(w)
    m = uw.uw_compress(w, n, k, layout, seg_groups=sg)
    om = oracle.compress(w_np, seg_groups=sg, layout=layout)
    assert uw.uw_export(m) == om.export(), "UWF1 blob differs from the oracle"
    numel = w_np.size
    out = torch.empty(numel, dtype=torch.int16, device=DEV)
    uw.uw_decode_full(m, out)
    assert uw.uw_sync_status(m) == 0
    assert torch.equal(out, w.view(torch.int16).reshape(-1)), "decode_full not bit-exact"
    del out
    e = torch.empty(numel, dtype=torch.uint8, device=DEV)
    uw.uw_decode_exponent(m, e)
    assert torch.equal(e, ((w.view(torch.int16).reshape(-1).to(torch.int32) >> 7) & 0xFF).to(torch.uint8))
    del e
    p = torch.empty(numel // 2, dtype=torch.uint8, device=DEV)
    uw.uw_transcode_palette(m, p)
    st, op = om.transcode()
    assert st == 0 and np.array_equal(p.cpu().numpy(), op), "transcode differs from the oracle"
    del p
    uw.uw_transcode_palette(m, None)
    return m, w_np, om


def gemm_parity(uw, oracle, m, w_np, layout, x, pipelines, cols=None, grouped=None, what=""):
    x_np = bits(x)
    batch = x.shape[0]
    ms = grouped or [m]
    N = sum(mm.info().n for mm in ms)
    for p in pipelines:
        y = torch.full((batch, N), float("nan"), dtype=torch.float32, device=DEV)
        nbytes = uw.uw_workspace_size_grouped(ms, p, batch) if grouped else uw.uw_workspace_size(m, p, batch)
        ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=DEV)
        if grouped:
            uw.uw_matmul_reconstruct_grouped(ms, p, x, y, ws)
        else:
            uw.uw_matmul_reconstruct(m, p, x, y, ws)
        torch.cuda.synchronize()
        yn = y.cpu().numpy()
        assert np.all(np.isfinite(yn)), f"{what} pipeline {p}: unwritten outputs"
        if grouped:
            col0 = 0
            for mm, wnp in zip(ms, w_np):
                n = mm.info().n
                y_ref, A = oracle.gemm_ref(x_np, wnp, layout, cols=cols)
                sub = yn[:, col0:col0 + n]
                ok, worst = oracle.gemm_check(sub if cols is None else sub[:, cols], y_ref, A)
                assert ok, f"{what} pipeline {p}: worst {worst}"
                col0 += n
        else:
            y_ref, A = oracle.gemm_ref(x_np, w_np, layout, cols=cols)
            ok, worst = oracle.gemm_check(yn if cols is None else yn[:, cols], y_ref, A)
            assert ok, f"{what} pipeline {p}: worst {worst}"
        say(f"  {what} pipeline {p} batch {batch}: ok")


def test_w256x512(uw, synth, oracle):
    wl = synth.WORKLOADS["w256x512"]
    _, n, k, layout = wl.mats[0]
    w = synth.workload_weights(wl, 0, device=DEV)
    m, w_np, _ = codec_parity(uw, oracle, w, n, k, layout)
    assert 0.02 < m.info().verbatim_groups / m.info().groups < 0.15
    x = synth.activations(1, k, seed=wl.seed, device=DEV)
    gemm_parity(uw, oracle, m, w_np, layout, x, range(4), what="w256x512")


def test_gate8b(uw, synth, oracle):
    wl = synth.WORKLOADS["gate8b"]
    _, n, k, layout = wl.mats[0]
    say("gate8b: codec")
    w = synth.workload_weights(wl, 0, device=DEV)
    m, w_np, _ = codec_parity(uw, oracle, w, n, k, layout)
    info = m.info()
    assert 10.0 < info.bits_per_weight < 11.5
    x = synth.activations(1, k, seed=wl.seed, device=DEV)
    gemm_parity(uw, oracle, m, w_np, layout, x, range(4), what="gate8b")


def test_gateup8b_fused(uw, synth, oracle):
    wl = synth.WORKLOADS["gateup8b"]
    ms, wnps = [], []
    for i in range(2):
        _, n, k, layout = wl.mats[i]
        say(f"gateup8b: codec {i}")
        w = synth.workload_weights(wl, i, device=DEV)
        m, w_np, _ = codec_parity(uw, oracle, w, n, k, layout)
        ms.append(m)
        wnps.append(w_np)
        del w
    for b in wl.batches:
        x = synth.activations(b, 4096, seed=wl.seed + b, device=DEV)
        gemm_parity(uw, oracle, None, wnps, 0, x, (2, 3), grouped=ms, what="gateup8b")


def test_down8b_transposed(uw, synth, oracle):
    wl = synth.WORKLOADS["down8b"]
    _, n, k, layout = wl.mats[0]
    say("down8b: codec")
    w = synth.workload_weights(wl, 0, device=DEV)
    m, w_np, _ = codec_parity(uw, oracle, w, n, k, layout)
    rng = np.random.default_rng(0)
    cols = np.sort(rng.choice(n, 256, replace=False))
    for b in wl.batches:
        x = synth.activations(b, k, seed=wl.seed + b, device=DEV)
        gemm_parity(uw, oracle, m, w_np, layout, x, (1, 2, 3), cols=cols, what="down8b")


@pytest.mark.timeout(900)
def test_mlp70b_one_layer(uw, synth, oracle):
    wl = synth.WORKLOADS["mlp70b"]
    rng = np.random.default_rng(1)
    for i, (label, n, k, layout) in enumerate(wl.mats):
        say(f"mlp70b layer 0 {label}: codec")
        w = synth.workload_weights(wl, i, layer=0, device=DEV)
        m, w_np, om = codec_parity(uw, oracle, w, n, k, layout)
        del w, om
        cols = np.sort(rng.choice(n, 64, replace=False))
        # all four pipelines at 1, 192 and 512 rows (the 256-row tiles with
        # the one-round K cap and the palette tail split act from 65 to 512
        # rows); exponent and direct palette at 64 and 1024
        for b in (1, 64, 192, 512, 1024):
            x = synth.activations(b, k, seed=wl.seed + b, device=DEV)
            gemm_parity(uw, oracle, m, w_np, layout, x, (1, 3) if b in (64, 1024) else range(4), cols=cols,
                        what=f"mlp70b {label} b{b}")
        del m, w_np
        torch.cuda.empty_cache()


def _attention(uw, synth, oracle, name, cols_for):
    """q/k/v/o of one attention layer: codec parity per matrix (blob equals
    the oracle's, decodes bit-exact), the fused q+k+v GEMM (one x, N = q+k+v)
    and o on their own, every pipeline at one row, the palette pipelines at
    the larger batches; output columns sampled where the fp64 reference
    would take long."""
    wl = synth.WORKLOADS[name]
    ms, wnps = [], []
    for i, (label, n, k, layout) in enumerate(wl.mats):
        say(f"{name} {label}: codec")
        w = synth.workload_weights(wl, i, device=DEV)
        m, w_np, _ = codec_parity(uw, oracle, w, n, k, layout)
        ms.append(m)
        wnps.append(w_np)
        del w
    k = wl.mats[0][2]
    rng = np.random.default_rng(3)
    for b in wl.batches:
        x = synth.activations(b, k, seed=wl.seed + b, device=DEV)
        pipes = range(4) if b == 1 else (2, 3)
        gemm_parity(uw, oracle, None, wnps[:3], 0, x, pipes, grouped=ms[:3], what=f"{name} qkv b{b}")
        n_o = wl.mats[3][1]
        cols = cols_for(b, n_o, rng)
        gemm_parity(uw, oracle, ms[3], wnps[3], 0, x, pipes, cols=cols, what=f"{name} o b{b}")
    del ms, wnps
    torch.cuda.empty_cache()


def test_attn8b_qkv_fused_and_o(uw, synth, oracle):
    _attention(uw, synth, oracle, "attn8b", lambda b, n, rng: None)


@pytest.mark.timeout(600)
def test_attn70b_qkv_fused_and_o(uw, synth, oracle):
    _attention(uw, synth, oracle, "attn70b",
               lambda b, n, rng: None if b == 1 else np.sort(rng.choice(n, 64, replace=False)))

